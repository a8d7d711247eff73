// Gather of a paged latent cache into contiguous rows ("cpu_mla_prefill.cpp",
// GatherMlaCache): output row t of sequence b = token_to_seq[t] is skipped when t
// lies past the sequence's end cu_seq_lens[b + 1]; otherwise its position in the
// sequence is t - cu_seq_lens[b] (+ seq_starts[b]) and it receives the cache row at
// slot position % block_size of block block_table[b][position / block_size],
// converted to the output dtype.
//
// Mapping onto gfx950: the copy is a stream of (row, unit) pairs, one per thread,
// so consecutive lanes read and write consecutive 16-byte chunks of a row (same
// dtype, aligned rows) or consecutive elements (conversions, other layouts).  The
// row's source offset comes from four dependent index loads that all lanes of the
// row share (broadcast from the caches).  With a status word, one workgroup checks
// every row first and the copy kernel exits before writing when it fails.
#include "pa_common.h"
#include "pa_internal.h"

namespace pa {

constexpr int kGatherCopy = 0, kGatherSkip = 1, kGatherBad = 2;

// What happens to output row t: copied from element offset *src of the cache,
// skipped (past its sequence's end), or refused (an index outside its range).
__device__ __forceinline__ int gather_row(const GatherArgs& a, int64_t t, int64_t* src) {
  const int64_t b = a.token_to_seq[t];
  if (b < 0 || b >= a.num_seqs) return kGatherBad;
  if (t >= a.cu_seq_lens[b + 1]) return kGatherSkip;
  const int64_t pos = t - a.cu_seq_lens[b] + (a.seq_starts != nullptr ? a.seq_starts[b] : 0);
  if (pos < 0) return kGatherBad;
  const int64_t idx = pos / a.block_size;
  if (idx >= a.max_blocks) return kGatherBad;
  const int64_t blk = a.block_table[b * a.max_blocks + idx];
  if (blk < 0 || blk >= a.num_blocks) return kGatherBad;
  *src = blk * a.block_stride + (pos % a.block_size) * a.slot_stride;
  return kGatherCopy;
}

__global__ __launch_bounds__(1024) void gather_validate_kernel(const GatherArgs a) {
  __shared__ int bad;
  if (threadIdx.x == 0) bad = 0;
  __syncthreads();
  int found = 0;
  for (int64_t t = threadIdx.x; t < a.num_tokens; t += blockDim.x) {
    int64_t src;
    found |= gather_row(a, t, &src) == kGatherBad;
  }
  if (found) atomicOr(&bad, 1);
  __syncthreads();
  if (threadIdx.x == 0) *a.status = bad ? PA_EINVAL : PA_OK;
}

template <typename S, typename D>
__device__ __forceinline__ void copy_elem(const GatherArgs& a, int64_t from, int64_t to) {
  float x;
  if constexpr (S::bytes == 4)
    x = static_cast<const float*>(a.cache)[from];
  else
    x = widen<S>((uint32_t) static_cast<const uint16_t*>(a.cache)[from], 0);
  if constexpr (D::bytes == 4)
    static_cast<float*>(a.dst)[to] = x;
  else
    static_cast<uint16_t*>(a.dst)[to] = (uint16_t)narrow<D>(x);
}

template <typename S, typename D>
__global__ __launch_bounds__(256) void gather_cache_kernel(const GatherArgs a) {
  if (status_failed(a.status)) return;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = i / a.units_per_row;
  const int u = (int)(i - row * a.units_per_row);
  if (row >= a.num_tokens) return;
  int64_t src;
  if (gather_row(a, row, &src) != kGatherCopy) return;  // skipped, or refused without a status word
  if (a.vec16) {
    constexpr int EB = S::bytes;
    const u32x4* from = reinterpret_cast<const u32x4*>(static_cast<const char*>(a.cache) + src * EB) + u;
    u32x4* to = reinterpret_cast<u32x4*>(static_cast<char*>(a.dst) + row * a.dst_stride * EB) + u;
    *to = *from;
  } else {
    copy_elem<S, D>(a, src + u, row * a.dst_stride + u);
  }
}

template <typename S>
hipError_t launch_gather_from(const GatherArgs& a, dim3 grid, hipStream_t stream) {
  if (a.dst_dtype == PA_F32)
    hipLaunchKernelGGL((gather_cache_kernel<S, F32>), grid, dim3(256), 0, stream, a);
  else if (a.dst_dtype == PA_F16)
    hipLaunchKernelGGL((gather_cache_kernel<S, F16>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((gather_cache_kernel<S, BF16>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_gather(const GatherArgs& a, hipStream_t stream) {
  if (a.status != nullptr) {
    hipLaunchKernelGGL(gather_validate_kernel, dim3(1), dim3(1024), 0, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t threads = a.num_tokens * a.units_per_row;
  if (threads == 0) return hipSuccess;
  const int64_t wgs = (threads + 255) / 256;
  if (wgs > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 grid((unsigned)wgs);
  if (a.cache_dtype == PA_F32) return launch_gather_from<F32>(a, grid, stream);
  if (a.cache_dtype == PA_F16) return launch_gather_from<F16>(a, grid, stream);
  return launch_gather_from<BF16>(a, grid, stream);
}

}  // namespace pa
