// pa_decode_noalloc: split-KV decode for callers that cannot allocate device memory.
// The partition states (max_logits, exp_sums, tmp_out) that pa_decode takes from the
// caller live here in one static device array, `scratch`, which every GPU the
// library runs on holds (kScratchBytes) until the process ends.  The call resolves
// the array's device address once per device, then runs pa_decode's kernels on that
// memory.  It issues kernel launches only: no allocation, free, memset or copy.
#include <mutex>

#include "pa_common.h"
#include "pa_internal.h"

namespace {

constexpr int64_t kScratchBytes = int64_t(96) << 20;
constexpr int64_t kScratchAlign = 256;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, once resolved

// The device address of `scratch` on the current device.  In host code the array's
// name is only a stand-in for the symbol; hipGetSymbolAddress, with the device
// current, gives the address kernels may use.
int scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return PA_EDEVICE;
  if (dev < 0 || dev >= kMaxDevices) return PA_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return PA_EDEVICE;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PA_OK;
}

int64_t round_up(int64_t x) { return (x + kScratchAlign - 1) / kScratchAlign * kScratchAlign; }

}  // namespace

extern "C" int pa_decode_noalloc(const pa_kv_pool* pool, const void* q, int32_t q_dtype, void* out,
                                 int32_t out_dtype, const int32_t* block_tables, int32_t max_blocks,
                                 const int32_t* seq_lens, int32_t num_seqs, int32_t num_heads, float scale,
                                 int32_t sliding_window, int32_t partition_size, const float* sinks,
                                 const float* alibi_slopes, int32_t* status, void* stream) {
  if (pool == nullptr) return PA_EINVAL;
  if (partition_size == 0)  // unsplit: pa_decode needs no workspace
    return pa_decode(pool, q, q_dtype, out, out_dtype, block_tables, max_blocks, seq_lens, num_seqs, num_heads,
                     scale, sliding_window, 0, 0, nullptr, nullptr, nullptr, sinks, alibi_slopes, status, stream);
  if (partition_size < 0 || pool->block_size < 1 || max_blocks < 1 || num_seqs < 0 || num_heads < 1 ||
      pool->head_dim_v < 1)
    return PA_EINVAL;
  if (partition_size % pool->block_size != 0) return PA_EINVAL;
  // partitions per (sequence, head): enough for the longest context the tables allow
  const int64_t max_len = (int64_t)max_blocks * pool->block_size;
  const int64_t max_partitions = (max_len + partition_size - 1) / partition_size;
  if (max_partitions > 8192) return PA_EUNSUPPORTED;  // as pa_decode
  const int64_t states = (int64_t)num_seqs * num_heads * max_partitions;
  if (states > kScratchBytes / 4) return PA_ESCRATCH;
  const int64_t scalars = round_up(states * 4);
  const int64_t need = 2 * scalars + round_up(states * pool->head_dim_v * 4);
  if (need > kScratchBytes) return PA_ESCRATCH;

  void* base = nullptr;
  const int st = scratch_on_current_device(&base);
  if (st != PA_OK) return st;
  char* p = static_cast<char*>(base);
  float* max_logits = reinterpret_cast<float*>(p);
  float* exp_sums = reinterpret_cast<float*>(p + scalars);
  float* tmp_out = reinterpret_cast<float*>(p + 2 * scalars);
  return pa_decode(pool, q, q_dtype, out, out_dtype, block_tables, max_blocks, seq_lens, num_seqs, num_heads, scale,
                   sliding_window, partition_size, (int32_t)max_partitions, max_logits, exp_sums, tmp_out, sinks,
                   alibi_slopes, status, stream);
}
