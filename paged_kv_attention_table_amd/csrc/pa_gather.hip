// Gather of a paged latent cache into contiguous rows ("cpu_mla_prefill.cpp",
// GatherMlaCache): output row t of sequence b = token_to_seq[t] is skipped when t
// lies past the sequence's end cu_seq_lens[b + 1]; otherwise its position in the
// sequence is t - cu_seq_lens[b] (+ seq_starts[b]) and it receives the cache row at
// slot position % block_size of block block_table[b][position / block_size],
// converted to the output dtype.
//
// Mapping onto gfx950: same dtype and 16-byte aligned rows -- a wave looks up the
// sources of 8 rows at once (one lane each) and its 64 lanes stream the rows'
// 16-byte chunks, consecutive lanes on consecutive chunks.  Conversions and other
// layouts: one thread per (row, element), consecutive lanes on consecutive elements.
// With a status word, every row is checked first (over the whole grid) and the copy
// kernels exit before writing when one is refused.
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

// Rows are checked over the whole grid; a wave that finds a refused row ORs
// PA_EINVAL (1) into the status word, which a one-thread kernel cleared first.
__global__ __launch_bounds__(256) void gather_validate_kernel(const GatherArgs a) {
  bool found = false;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < a.num_tokens;
       t += (int64_t)gridDim.x * blockDim.x) {
    int64_t src;
    found |= gather_row(a, t, &src) == kGatherBad;
  }
  if (__any(found) && lane_id() == 0) atomicOr(a.status, PA_EINVAL);
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
  copy_elem<S, D>(a, src + u, row * a.dst_stride + u);
}

// Same dtype, 16-byte aligned rows: a wave copies kGatherRows rows.  Lanes 0 ..
// kGatherRows - 1 look up one row's source each; every lane then takes the wave's
// 16-byte chunks lane, lane + 64, ... (consecutive lanes, consecutive chunks) with
// its row's source offset fetched from the lane that looked it up.
constexpr int kGatherRows = 8;

__global__ __launch_bounds__(256) void gather_rows16_kernel(const GatherArgs a) {
  if (status_failed(a.status)) return;
  const int lane = lane_id();
  const int64_t row0 = ((int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave) * kGatherRows;
  if (row0 >= a.num_tokens) return;
  int64_t src = -1;
  if (lane < kGatherRows && row0 + lane < a.num_tokens) {
    int64_t s;
    if (gather_row(a, row0 + lane, &s) == kGatherCopy) src = s;
  }
  const int cpr = a.units_per_row;
  const int total = kGatherRows * cpr;
  const char* cache = static_cast<const char*>(a.cache);
  char* dst = static_cast<char*>(a.dst);
  const int64_t eb = a.cache_dtype == PA_F32 ? 4 : 2;
  for (int k = lane; k < total; k += kWave) {
    const int r = k / cpr, c = k - r * cpr;
    const int64_t s = __shfl(src, r);
    if (s < 0) continue;  // past the last row, skipped, or refused
    const u32x4 x = *reinterpret_cast<const u32x4*>(cache + s * eb + 16 * c);
    *reinterpret_cast<u32x4*>(dst + (row0 + r) * a.dst_stride * eb + 16 * c) = x;
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
    hipError_t e = launch_status_clear(a.status, stream);
    if (e != hipSuccess) return e;
    if (a.num_tokens > 0) {
      int64_t blocks = (a.num_tokens + 255) / 256;
      if (blocks > 2048) blocks = 2048;
      hipLaunchKernelGGL(gather_validate_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  if (a.num_tokens == 0) return hipSuccess;
  if (a.vec16) {
    const int64_t rows_per_wg = 4 * kGatherRows;
    const int64_t wgs = (a.num_tokens + rows_per_wg - 1) / rows_per_wg;
    if (wgs > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(gather_rows16_kernel, dim3((unsigned)wgs), dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  const int64_t threads = a.num_tokens * a.units_per_row;
  const int64_t wgs = (threads + 255) / 256;
  if (wgs > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 grid((unsigned)wgs);
  if (a.cache_dtype == PA_F32) return launch_gather_from<F32>(a, grid, stream);
  if (a.cache_dtype == PA_F16) return launch_gather_from<F16>(a, grid, stream);
  return launch_gather_from<BF16>(a, grid, stream);
}

}  // namespace pa
