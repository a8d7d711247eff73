// The C entry points declared in include/pa.h: synchronous argument checks, then
// kernel launches on the caller's stream.  The library allocates nothing.
#include <math.h>

#include "pa_common.h"
#include "pa_internal.h"
#include "pa_prefill.h"

namespace pa {
hipError_t launch_rows_f32(const RowsArgs& a, int dk, int dv, dim3 grid, hipStream_t stream);
hipError_t launch_rows_f16(const RowsArgs& a, int dk, int dv, dim3 grid, hipStream_t stream);
hipError_t launch_rows_bf16(const RowsArgs& a, int dk, int dv, dim3 grid, hipStream_t stream);

hipError_t launch_rows(const RowsArgs& a, int dtype, int dk, int dv, dim3 grid, hipStream_t stream) {
  if (dtype == PA_F32) return launch_rows_f32(a, dk, dv, grid, stream);
  if (dtype == PA_F16) return launch_rows_f16(a, dk, dv, grid, stream);
  if (dtype == PA_BF16) return launch_rows_bf16(a, dk, dv, grid, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_prefill_bf16(const PrefillArgs& a, int dk, int dv, dim3 grid, hipStream_t stream);
hipError_t launch_prefill_f16(const PrefillArgs& a, int dk, int dv, dim3 grid, hipStream_t stream);
hipError_t launch_prefill_fp8_bf16(const PrefillArgs& a, int dk, int dv, dim3 grid, hipStream_t stream);
hipError_t launch_prefill_fp8_f16(const PrefillArgs& a, int dk, int dv, dim3 grid, hipStream_t stream);

// Tile kernel launch for a pool of kv_dtype and queries of q_dtype.
hipError_t launch_prefill(const PrefillArgs& a, int kv_dtype, int q_dtype, int dk, int dv, dim3 grid,
                          hipStream_t stream) {
  if (kv_dtype == PA_FP8_E4M3) {
    if (q_dtype == PA_BF16) return launch_prefill_fp8_bf16(a, dk, dv, grid, stream);
    if (q_dtype == PA_F16) return launch_prefill_fp8_f16(a, dk, dv, grid, stream);
    return hipErrorInvalidValue;
  }
  if (q_dtype != kv_dtype) return hipErrorInvalidValue;
  if (kv_dtype == PA_BF16) return launch_prefill_bf16(a, dk, dv, grid, stream);
  if (kv_dtype == PA_F16) return launch_prefill_f16(a, dk, dv, grid, stream);
  return hipErrorInvalidValue;
}

// The tiled prefill kernel: f16 / bf16 pools with queries of the same type, or fp8
// pools with f16 / bf16 queries; these head dims (fp8: 128 / 128 and 192 / 128), a
// power-of-two block size of at least 16 (a 32-key tile then spans at most two
// blocks, one per half), and a pool of fewer than 2^32 rows (the kernel forms row
// indices in 32 bits).
bool prefill_supported(int kv_dtype, int q_dtype, int dk, int dv, int group, int block_size, int64_t num_blocks) {
  bool dims;
  if (kv_dtype == PA_FP8_E4M3) {
    if (q_dtype != PA_BF16 && q_dtype != PA_F16) return false;
    dims = (dk == 128 || dk == 192) && dv == 128;
  } else {
    if ((kv_dtype != PA_BF16 && kv_dtype != PA_F16) || q_dtype != kv_dtype) return false;
    dims = (dk == 128 && dv == 128) || (dk == 192 && dv == 128) || (dk == 64 && dv == 64);
  }
  const bool pow2 = block_size >= 16 && (block_size & (block_size - 1)) == 0;
  const bool rows32 = num_blocks * (int64_t)block_size <= 0xffffffffLL;
  return dims && pow2 && rows32 && group >= 1 && group <= kPrefillRows;
}

hipError_t launch_varlen_fused_f16(const PrefillArgs& p, const RowsArgs& r, int block_shift, uint32_t prefill_wgs,
                                  hipStream_t stream);
hipError_t launch_varlen_fused_bf16(const PrefillArgs& p, const RowsArgs& r, int block_shift, uint32_t prefill_wgs,
                                   hipStream_t stream);
hipError_t launch_varlen_fused_fp8_f16(const PrefillArgs& p, const RowsArgs& r, int block_shift,
                                      uint32_t prefill_wgs, hipStream_t stream);
hipError_t launch_varlen_fused_fp8_bf16(const PrefillArgs& p, const RowsArgs& r, int block_shift,
                                       uint32_t prefill_wgs, hipStream_t stream);

// The fused varlen kernel (tiles and single-token rows in one launch) for a pool of
// kv_dtype and queries of q_dtype.
hipError_t launch_varlen_fused(const PrefillArgs& p, const RowsArgs& r, int kv_dtype, int q_dtype, int block_shift,
                               uint32_t prefill_wgs, hipStream_t stream) {
  const bool bf16 = q_dtype == PA_BF16;
  if (kv_dtype == PA_FP8_E4M3)
    return bf16 ? launch_varlen_fused_fp8_bf16(p, r, block_shift, prefill_wgs, stream)
                : launch_varlen_fused_fp8_f16(p, r, block_shift, prefill_wgs, stream);
  return bf16 ? launch_varlen_fused_bf16(p, r, block_shift, prefill_wgs, stream)
              : launch_varlen_fused_f16(p, r, block_shift, prefill_wgs, stream);
}

hipError_t launch_decode_bf16(const RowsArgs& a, int block_shift, int dk, int dv, dim3 grid, hipStream_t stream);
hipError_t launch_decode_f16(const RowsArgs& a, int block_shift, int dk, int dv, dim3 grid, hipStream_t stream);
hipError_t launch_decode_fp8_bf16(const RowsArgs& a, int block_shift, int dk, int dv, dim3 grid, hipStream_t stream);
hipError_t launch_decode_fp8_f16(const RowsArgs& a, int block_shift, int dk, int dv, dim3 grid, hipStream_t stream);

// The MFMA decode kernel: f16 / bf16, a power-of-two block size that is a multiple
// of 16, up to 16 q heads per kv head.
bool decode_mfma_supported(int dtype, int dk, int dv, int group, int block_size) {
  if (dtype != PA_BF16 && dtype != PA_F16) return false;
  const bool dims = dk == 128 && dv == 128;
  const bool pow2 = block_size >= 16 && (block_size & (block_size - 1)) == 0;
  return dims && pow2 && group >= 1 && group <= 16;
}

// Row kernel launch: the MFMA decode kernel when it supports the shape, else the
// general per-row kernel.  `dtype` is the queries' (f16 / bf16 for an fp8 pool).
hipError_t launch_row_kernel(const RowsArgs& a, int kv_dtype, int dtype, int dk, int dv, dim3 grid,
                             hipStream_t stream) {
  int shift = 0;
  while ((1 << shift) < a.block_size) ++shift;
  if (kv_dtype == PA_FP8_E4M3) {
    if (!decode_mfma_supported(dtype, dk, dv, a.group, a.block_size)) return hipErrorInvalidValue;
    return dtype == PA_BF16 ? launch_decode_fp8_bf16(a, shift, dk, dv, grid, stream)
                            : launch_decode_fp8_f16(a, shift, dk, dv, grid, stream);
  }
  if (decode_mfma_supported(dtype, dk, dv, a.group, a.block_size))
    return dtype == PA_BF16 ? launch_decode_bf16(a, shift, dk, dv, grid, stream)
                            : launch_decode_f16(a, shift, dk, dv, grid, stream);
  return launch_rows(a, dtype, dk, dv, grid, stream);
}

bool rows_supported(int dtype, int dk, int dv, int group) {
  if (dtype != PA_F32 && dtype != PA_F16 && dtype != PA_BF16) return false;
  const bool dims = (dk == dv && (dk == 32 || dk == 64 || dk == 128 || dk == 256)) || (dk == 192 && dv == 128);
  if (!dims || group < 1 || group > 16) return false;
  if (group > 8 && dv > 128) return false;
  return true;
}
}  // namespace pa

using namespace pa;

namespace {

// Bytes of a value type (queries, outputs, merged states, latent rows).
int element_bytes(int dtype) {
  switch (dtype) {
    case PA_F32: return 4;
    case PA_F16:
    case PA_BF16: return 2;
    default: return 0;
  }
}

// Bytes of a pool element: the value types, or one byte of fp8.
int pool_element_bytes(int dtype) { return dtype == PA_FP8_E4M3 ? 1 : element_bytes(dtype); }

int check_pool(const pa_kv_pool* pool) {
  if (pool == nullptr || pool->k == nullptr || pool->v == nullptr) return PA_EINVAL;
  if (pool->num_blocks < 1 || pool->block_size < 1 || pool->num_kv_heads < 1 || pool->head_dim_k < 1 ||
      pool->head_dim_v < 1)
    return PA_EINVAL;
  if (pool_element_bytes(pool->dtype) == 0) return PA_EUNSUPPORTED;
  if (!isfinite(pool->k_scale) || !(pool->k_scale > 0.f) || !isfinite(pool->v_scale) || !(pool->v_scale > 0.f))
    return PA_EINVAL;
  return PA_OK;
}

// The queries' type must be the pool's, or f16 / bf16 over an fp8 pool.
bool query_type_ok(const pa_kv_pool* pool, int q_dtype) {
  if (pool->dtype == PA_FP8_E4M3) return q_dtype == PA_F16 || q_dtype == PA_BF16;
  return q_dtype == pool->dtype;
}

// The softmax scale with k_scale folded in (a score is scale * k_scale * <q, stored
// k>); false when the product is not a finite positive binary32.
bool folded_scale(const pa_kv_pool* pool, float scale, float& scale_log2) {
  if (!isfinite(scale) || !(scale > 0.f)) return false;
  const float s = scale * pool->k_scale;
  if (!isfinite(s) || !(s > 0.f) || !isfinite(s * kLog2e) || !(s * kLog2e > 0.f)) return false;
  scale_log2 = s * kLog2e;
  return true;
}

int from_hip(hipError_t e) { return e == hipSuccess ? PA_OK : PA_EDEVICE; }

// log2(x) when x is a power of two, else -1.
int pow2_shift(int x) {
  if (x <= 0 || (x & (x - 1)) != 0) return -1;
  int s = 0;
  while ((1 << s) < x) ++s;
  return s;
}

}  // namespace

extern "C" {

const char* pa_strerror(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_EINVAL: return "invalid argument or device content (block table, length, position or slot)";
    case PA_ESHAPE: return "shape mismatch (num_heads not a multiple of num_kv_heads, or dims disagree)";
    case PA_EUNSUPPORTED: return "unsupported element type, head dim or head-group size";
    case PA_EDEVICE: return "HIP launch failure";
    case PA_ESCRATCH: return "the call needs more split-KV workspace than the library's static buffer holds";
    default: return "unknown status";
  }
}

int pa_write_kv(const pa_kv_pool* pool, const void* k_new, const void* v_new, const int32_t* slot_mapping,
                int64_t num_tokens, int32_t* status, void* stream) {
  int st = check_pool(pool);
  if (st != PA_OK) return st;
  if (num_tokens < 0) return PA_EINVAL;
  if (num_tokens > 0 && (k_new == nullptr || v_new == nullptr || slot_mapping == nullptr)) return PA_EINVAL;
  const int eb = pool_element_bytes(pool->dtype);
  WriteArgs a;
  a.k_pool = pool->k;
  a.v_pool = pool->v;
  a.num_slots = pool->num_blocks * pool->block_size;
  a.k_row_bytes = (int64_t)pool->num_kv_heads * pool->head_dim_k * eb;
  a.v_row_bytes = (int64_t)pool->num_kv_heads * pool->head_dim_v * eb;
  if (a.k_row_bytes % 4 != 0 || a.v_row_bytes % 4 != 0) return PA_EUNSUPPORTED;
  a.k_new = k_new;
  a.v_new = v_new;
  a.slot_mapping = slot_mapping;
  a.num_tokens = num_tokens;
  a.status = status;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (status != nullptr) {
    ValidateArgs v = {};
    v.mode = kValidateWrite;
    v.num_blocks = pool->num_blocks;
    v.block_size = pool->block_size;
    v.slot_mapping = slot_mapping;
    v.num_new_tokens = num_tokens;
    v.status = status;
    st = from_hip(launch_validate(v, s));
    if (st != PA_OK) return st;
  }
  if (num_tokens == 0) return PA_OK;
  return from_hip(launch_write(a, s));
}

int pa_decode(const pa_kv_pool* pool, const void* q, int32_t q_dtype, void* out, int32_t out_dtype,
              const int32_t* block_tables, int32_t max_blocks, const int32_t* seq_lens, int32_t num_seqs,
              int32_t num_heads, float scale, int32_t sliding_window, int32_t partition_size,
              int32_t max_partitions, float* max_logits, float* exp_sums, float* tmp_out, const float* sinks,
              const float* alibi_slopes, int32_t* status, void* stream) {
  int st = check_pool(pool);
  if (st != PA_OK) return st;
  if (num_seqs < 0 || num_heads < 1 || max_blocks < 1 || partition_size < 0) return PA_EINVAL;
  if (num_seqs > 0 && (q == nullptr || out == nullptr || block_tables == nullptr || seq_lens == nullptr))
    return PA_EINVAL;
  if (num_heads % pool->num_kv_heads != 0) return PA_ESHAPE;
  if (pool->head_dim_k != pool->head_dim_v) return PA_EUNSUPPORTED;
  if (!query_type_ok(pool, q_dtype)) return PA_EUNSUPPORTED;
  if (out_dtype != PA_F32 && out_dtype != q_dtype) return PA_EUNSUPPORTED;
  const int group = num_heads / pool->num_kv_heads;
  const bool fp8 = pool->dtype == PA_FP8_E4M3;
  if (fp8 ? !decode_mfma_supported(q_dtype, pool->head_dim_k, pool->head_dim_v, group, pool->block_size)
          : !rows_supported(pool->dtype, pool->head_dim_k, pool->head_dim_v, group))
    return PA_EUNSUPPORTED;
  float scale_log2;
  if (!folded_scale(pool, scale, scale_log2)) return PA_EINVAL;
  if (partition_size > 0) {
    if (partition_size % pool->block_size != 0) return PA_EINVAL;
    if (max_partitions < 1 || max_logits == nullptr || exp_sums == nullptr || tmp_out == nullptr)
      return PA_EINVAL;
    if (max_partitions > 8192) return PA_EUNSUPPORTED;
  }
  if (num_seqs > 65535 * 1024) return PA_EUNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (status != nullptr) {
    ValidateArgs v = {};
    v.mode = kValidateDecode;
    v.num_blocks = pool->num_blocks;
    v.block_size = pool->block_size;
    v.block_tables = block_tables;
    v.max_blocks = max_blocks;
    v.seq_lens = seq_lens;
    v.num_seqs = num_seqs;
    v.partition_size = partition_size;
    v.max_partitions = max_partitions;
    v.status = status;
    st = from_hip(launch_validate(v, s));
    if (st != PA_OK) return st;
  }
  if (num_seqs == 0) return PA_OK;

  RowsArgs a = {};
  a.k_pool = pool->k;
  a.v_pool = pool->v;
  a.num_blocks = pool->num_blocks;
  a.block_size = pool->block_size;
  a.num_kv_heads = pool->num_kv_heads;
  a.q = q;
  a.out = out;
  a.out_dtype = out_dtype;
  a.lse = nullptr;
  a.block_tables = block_tables;
  a.max_blocks = max_blocks;
  a.seq_lens = seq_lens;
  a.query_start_loc = nullptr;
  a.positions = nullptr;
  a.num_seqs = num_seqs;
  a.num_rows = num_seqs;
  a.num_heads = num_heads;
  a.group = group;
  a.scale_log2 = scale_log2;
  a.v_scale = pool->v_scale;
  a.causal = 1;
  a.window = sliding_window;
  a.partition_size = partition_size;
  a.max_partitions = partition_size > 0 ? max_partitions : 1;
  a.max_logits = max_logits;
  a.exp_sums = exp_sums;
  a.tmp_out = tmp_out;
  a.sinks = sinks;
  a.alibi = alibi_slopes;
  a.status = status;
  const dim3 grid((unsigned)num_seqs, (unsigned)pool->num_kv_heads, (unsigned)(partition_size > 0 ? max_partitions : 1));
  st = from_hip(launch_row_kernel(a, pool->dtype, q_dtype, pool->head_dim_k, pool->head_dim_v, grid, s));
  if (st != PA_OK || partition_size == 0) return st;

  ReduceArgs r = {};
  r.max_logits = max_logits;
  r.exp_sums = exp_sums;
  r.tmp_out = tmp_out;
  r.seq_lens = seq_lens;
  r.max_blocks = max_blocks;
  r.block_size = pool->block_size;
  r.num_seqs = num_seqs;
  r.num_heads = num_heads;
  r.head_dim = pool->head_dim_v;
  r.partition_size = partition_size;
  r.max_partitions = max_partitions;
  r.out = out;
  r.out_dtype = out_dtype;
  r.sinks = sinks;
  r.status = status;
  return from_hip(launch_reduce(r, s));
}

// pa_varlen and pa_varlen_merge (merge != 0: out, float32, and lse hold a state that
// this call's attention is merged into).
static int varlen_impl(const pa_kv_pool* pool, const void* q, int32_t q_dtype, void* out, int32_t out_dtype,
                       float* lse, const int32_t* query_start_loc, const int32_t* seq_lens, const int32_t* positions,
                       const int32_t* block_tables, int32_t max_blocks, int32_t num_seqs, int64_t num_tokens,
                       int32_t max_query_len, int32_t num_heads, float scale, int32_t causal, int32_t sliding_window,
                       int32_t partition_size, int32_t max_partitions, float* max_logits, float* exp_sums,
                       float* tmp_out, const float* sinks, const float* alibi_slopes, int32_t* status, void* stream,
                       int merge) {
  int st = check_pool(pool);
  if (st != PA_OK) return st;
  if (merge) {
    if (lse == nullptr) return PA_EINVAL;
    if (out_dtype != PA_F32 || partition_size != 0) return PA_EUNSUPPORTED;
  }
  if (num_seqs < 0 || num_tokens < 0 || num_heads < 1 || max_blocks < 1 || max_query_len < 0) return PA_EINVAL;
  if (query_start_loc == nullptr) return PA_EINVAL;
  if (num_seqs > 0 && (seq_lens == nullptr || block_tables == nullptr)) return PA_EINVAL;
  if (num_tokens > 0 && (q == nullptr || out == nullptr || num_seqs == 0)) return PA_EINVAL;
  if (causal && num_tokens > 0 && positions == nullptr) return PA_EINVAL;
  if (num_heads % pool->num_kv_heads != 0) return PA_ESHAPE;
  if (!query_type_ok(pool, q_dtype)) return PA_EUNSUPPORTED;
  if (out_dtype != PA_F32 && out_dtype != q_dtype) return PA_EUNSUPPORTED;
  const int group = num_heads / pool->num_kv_heads;
  const bool fp8 = pool->dtype == PA_FP8_E4M3;
  // The row kernels: every shape for 16-bit pools' single tokens and longer queries;
  // for fp8 pools the MFMA decode kernel, single tokens only.  The tile kernel:
  // queries of several tokens (and single tokens the row kernels cannot take).
  const bool rows_ok = fp8 ? decode_mfma_supported(q_dtype, pool->head_dim_k, pool->head_dim_v, group,
                                                   pool->block_size)
                           : rows_supported(pool->dtype, pool->head_dim_k, pool->head_dim_v, group);
  const bool tiles_ok = prefill_supported(pool->dtype, q_dtype, pool->head_dim_k, pool->head_dim_v, group,
                                          pool->block_size, pool->num_blocks);
  if (!rows_ok && !tiles_ok) return PA_EUNSUPPORTED;
  if (fp8 && max_query_len > 1 && !tiles_ok) return PA_EUNSUPPORTED;
  float scale_log2;
  if (!folded_scale(pool, scale, scale_log2)) return PA_EINVAL;
  if (num_tokens > 0x7fffffffLL || num_seqs > 65535) return PA_EUNSUPPORTED;
  if (partition_size < 0) return PA_EINVAL;
  if (partition_size > 0) {
    if (partition_size % pool->block_size != 0) return PA_EINVAL;
    if (max_partitions < 1 || max_logits == nullptr || exp_sums == nullptr || tmp_out == nullptr)
      return PA_EINVAL;
    if (max_partitions > 8192) return PA_EUNSUPPORTED;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (status != nullptr) {
    ValidateArgs v = {};
    v.mode = kValidateVarlen;
    v.partition_size = partition_size;
    v.max_partitions = max_partitions;
    v.num_blocks = pool->num_blocks;
    v.block_size = pool->block_size;
    v.block_tables = block_tables;
    v.max_blocks = max_blocks;
    v.seq_lens = seq_lens;
    v.num_seqs = num_seqs;
    v.query_start_loc = query_start_loc;
    v.num_tokens = num_tokens;
    v.max_query_len = max_query_len;
    v.positions = positions;
    v.causal = causal;
    v.status = status;
    st = from_hip(launch_validate(v, s));
    if (st != PA_OK) return st;
  }
  if (num_tokens == 0) return PA_OK;

  RowsArgs a = {};
  a.k_pool = pool->k;
  a.v_pool = pool->v;
  a.num_blocks = pool->num_blocks;
  a.block_size = pool->block_size;
  a.num_kv_heads = pool->num_kv_heads;
  a.q = q;
  a.out = out;
  a.out_dtype = out_dtype;
  a.lse = lse;
  a.block_tables = block_tables;
  a.max_blocks = max_blocks;
  a.seq_lens = seq_lens;
  a.query_start_loc = query_start_loc;
  a.positions = causal ? positions : nullptr;
  a.num_seqs = num_seqs;
  a.num_rows = num_tokens;
  a.num_heads = num_heads;
  a.group = group;
  a.scale_log2 = scale_log2;
  a.v_scale = pool->v_scale;
  a.causal = causal ? 1 : 0;
  a.window = sliding_window;
  a.partition_size = 0;
  a.max_partitions = 1;
  a.sinks = sinks;
  a.alibi = alibi_slopes;
  a.merge = merge;
  a.status = status;

  // Sequences of exactly one query token can run split-KV: partitions on the row
  // kernels (one row per sequence), then the log-sum-exp reduce, which writes their
  // outputs and lse.
  const bool rows_take_singles = rows_ok;
  const bool split = partition_size > 0 && rows_take_singles;
  auto split_singles = [&]() -> int {
    RowsArgs b = a;
    b.single_token_seqs = 1;
    b.skip_single_token_seqs = 0;
    b.partition_size = partition_size;
    b.max_partitions = max_partitions;
    b.max_logits = max_logits;
    b.exp_sums = exp_sums;
    b.tmp_out = tmp_out;
    const dim3 grid((unsigned)num_seqs, (unsigned)pool->num_kv_heads, (unsigned)max_partitions);
    int rc = from_hip(launch_row_kernel(b, pool->dtype, q_dtype, pool->head_dim_k, pool->head_dim_v, grid, s));
    if (rc != PA_OK) return rc;
    ReduceArgs r = {};
    r.max_logits = max_logits;
    r.exp_sums = exp_sums;
    r.tmp_out = tmp_out;
    r.seq_lens = seq_lens;
    r.max_blocks = max_blocks;
    r.block_size = pool->block_size;
    r.num_seqs = num_seqs;
    r.num_heads = num_heads;
    r.head_dim = pool->head_dim_v;
    r.partition_size = partition_size;
    r.max_partitions = max_partitions;
    r.out = out;
    r.out_dtype = out_dtype;
    r.sinks = sinks;
    r.query_start_loc = query_start_loc;
    r.lse = lse;
    r.num_rows = num_tokens;
    r.status = status;
    return from_hip(launch_reduce(r, s));
  };

  if (!tiles_ok || (max_query_len <= 1 && rows_ok)) {
    // every token through the per-row kernel (single-token sequences split, if asked)
    if (split && max_query_len <= 1) return split_singles();
    a.single_token_seqs = 0;
    a.skip_single_token_seqs = split ? 1 : 0;
    const dim3 grid((unsigned)num_tokens, (unsigned)pool->num_kv_heads, 1);
    st = from_hip(launch_row_kernel(a, pool->dtype, q_dtype, pool->head_dim_k, pool->head_dim_v, grid, s));
    if (st != PA_OK || !split) return st;
    return split_singles();
  }
  // sequences with several tokens: tiled MFMA kernel; single tokens: per-row kernel
  PrefillArgs p = {};
  p.k_pool = pool->k;
  p.v_pool = pool->v;
  p.num_blocks = pool->num_blocks;
  p.block_size = pool->block_size;
  p.num_kv_heads = pool->num_kv_heads;
  p.q = q;
  p.out = out;
  p.out_dtype = out_dtype;
  p.lse = lse;
  p.block_tables = block_tables;
  p.max_blocks = max_blocks;
  p.seq_lens = seq_lens;
  p.query_start_loc = query_start_loc;
  p.positions = causal ? positions : nullptr;
  p.num_seqs = num_seqs;
  p.num_tokens = num_tokens;
  p.num_heads = num_heads;
  p.group = group;
  p.block_shift = pow2_shift(pool->block_size);
  p.tokens_per_tile = kPrefillRows / group;
  p.min_q_len = rows_take_singles ? 2 : 1;
  p.scale_log2 = scale_log2;
  p.v_scale = pool->v_scale;
  p.causal = causal ? 1 : 0;
  p.window = sliding_window;
  p.sinks = sinks;
  p.alibi = alibi_slopes;
  p.merge = merge;
  p.status = status;
  p.tiles_per_seq = (max_query_len + p.tokens_per_tile - 1) / p.tokens_per_tile;
  const int64_t groups8 = ((int64_t)num_seqs * pool->num_kv_heads + 7) / 8 * 8;
  const int64_t wgs = groups8 * p.tiles_per_seq;
  if (wgs > 0x7fffffffLL) return PA_EUNSUPPORTED;
  if (wgs == 0) return PA_OK;
  // Single-token sequences on the MFMA decode kernel's shapes share the tile launch
  // (the fused kernel); otherwise they follow it on a launch of their own.
  const bool fuse = rows_take_singles && !split &&
                    decode_mfma_supported(q_dtype, pool->head_dim_k, pool->head_dim_v, group, pool->block_size);
  if (fuse) {
    a.single_token_seqs = 1;
    const int shift = pow2_shift(pool->block_size);
    return from_hip(launch_varlen_fused(p, a, pool->dtype, q_dtype, shift, (uint32_t)wgs, s));
  }
  st = from_hip(launch_prefill(p, pool->dtype, q_dtype, pool->head_dim_k, pool->head_dim_v, dim3((unsigned)wgs), s));
  if (st != PA_OK || !rows_take_singles) return st;
  if (split) return split_singles();
  a.single_token_seqs = 1;
  const dim3 grid((unsigned)num_seqs, (unsigned)pool->num_kv_heads, 1);
  return from_hip(launch_row_kernel(a, pool->dtype, q_dtype, pool->head_dim_k, pool->head_dim_v, grid, s));
}

int pa_varlen(const pa_kv_pool* pool, const void* q, int32_t q_dtype, void* out, int32_t out_dtype, float* lse,
              const int32_t* query_start_loc, const int32_t* seq_lens, const int32_t* positions,
              const int32_t* block_tables, int32_t max_blocks, int32_t num_seqs, int64_t num_tokens,
              int32_t max_query_len, int32_t num_heads, float scale, int32_t causal, int32_t sliding_window,
              int32_t partition_size, int32_t max_partitions, float* max_logits, float* exp_sums, float* tmp_out,
              const float* sinks, const float* alibi_slopes, int32_t* status, void* stream) {
  return varlen_impl(pool, q, q_dtype, out, out_dtype, lse, query_start_loc, seq_lens, positions, block_tables,
                     max_blocks, num_seqs, num_tokens, max_query_len, num_heads, scale, causal, sliding_window,
                     partition_size, max_partitions, max_logits, exp_sums, tmp_out, sinks, alibi_slopes, status, stream,
                     0);
}

int pa_varlen_merge(const pa_kv_pool* pool, const void* q, int32_t q_dtype, float* out, float* lse,
                    const int32_t* query_start_loc, const int32_t* seq_lens, const int32_t* positions,
                    const int32_t* block_tables, int32_t max_blocks, int32_t num_seqs, int64_t num_tokens,
                    int32_t max_query_len, int32_t num_heads, float scale, int32_t causal, int32_t sliding_window,
                    const float* sinks, const float* alibi_slopes, int32_t* status, void* stream) {
  return varlen_impl(pool, q, q_dtype, out, PA_F32, lse, query_start_loc, seq_lens, positions, block_tables,
                     max_blocks, num_seqs, num_tokens, max_query_len, num_heads, scale, causal, sliding_window, 0, 0,
                     nullptr, nullptr, nullptr, sinks, alibi_slopes, status, stream, 1);
}

int pa_varlen_ctx_new(const pa_kv_pool* pool, const void* q, int32_t q_dtype, float* out, float* lse, int32_t merge,
                      const int32_t* query_start_loc, const int32_t* ctx_lens, const int32_t* ctx_tables,
                      int32_t ctx_max_blocks, const int32_t* new_lens, const int32_t* new_positions,
                      const int32_t* new_tables, int32_t new_max_blocks, int32_t num_seqs, int64_t num_tokens,
                      int32_t max_query_len, int32_t num_heads, float scale, const float* sinks, int32_t* status,
                      void* stream) {
  int st = check_pool(pool);
  if (st != PA_OK) return st;
  if (num_seqs < 0 || num_tokens < 0 || num_heads < 1 || ctx_max_blocks < 1 || new_max_blocks < 1 ||
      max_query_len < 0 || query_start_loc == nullptr)
    return PA_EINVAL;
  if (num_seqs > 0 && (ctx_lens == nullptr || ctx_tables == nullptr || new_lens == nullptr || new_tables == nullptr))
    return PA_EINVAL;
  if (num_tokens > 0 && (q == nullptr || out == nullptr || lse == nullptr || new_positions == nullptr || num_seqs == 0))
    return PA_EINVAL;
  if (num_heads % pool->num_kv_heads != 0) return PA_ESHAPE;
  if (!query_type_ok(pool, q_dtype)) return PA_EUNSUPPORTED;
  const int group = num_heads / pool->num_kv_heads;
  if (!prefill_supported(pool->dtype, q_dtype, pool->head_dim_k, pool->head_dim_v, group, pool->block_size,
                         pool->num_blocks))
    return PA_EUNSUPPORTED;
  float scale_log2;
  if (!folded_scale(pool, scale, scale_log2)) return PA_EINVAL;
  if (num_tokens > 0x7fffffffLL || num_seqs > 65535) return PA_EUNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (status != nullptr) {
    // the context segment as a non-causal varlen call, then the new tokens' segment
    // (positions checked where it is not empty), ORed into the same word
    ValidateArgs v = {};
    v.mode = kValidateVarlen;
    v.num_blocks = pool->num_blocks;
    v.block_size = pool->block_size;
    v.block_tables = ctx_tables;
    v.max_blocks = ctx_max_blocks;
    v.seq_lens = ctx_lens;
    v.num_seqs = num_seqs;
    v.query_start_loc = query_start_loc;
    v.num_tokens = num_tokens;
    v.max_query_len = max_query_len;
    v.status = status;
    st = from_hip(launch_validate(v, s));
    if (st != PA_OK) return st;
    v.block_tables = new_tables;
    v.max_blocks = new_max_blocks;
    v.seq_lens = new_lens;
    v.positions = new_positions;
    v.causal = 1;
    v.positions_if_nonempty = 1;
    v.accumulate = 1;
    st = from_hip(launch_validate(v, s));
    if (st != PA_OK) return st;
  }
  if (num_tokens == 0) return PA_OK;
  PrefillArgs p = {};
  p.k_pool = pool->k;
  p.v_pool = pool->v;
  p.num_blocks = pool->num_blocks;
  p.block_size = pool->block_size;
  p.num_kv_heads = pool->num_kv_heads;
  p.q = q;
  p.out = out;
  p.out_dtype = PA_F32;
  p.lse = lse;
  p.block_tables = ctx_tables;
  p.max_blocks = ctx_max_blocks;
  p.seq_lens = ctx_lens;
  p.query_start_loc = query_start_loc;
  p.positions = new_positions;
  p.num_seqs = num_seqs;
  p.num_tokens = num_tokens;
  p.num_heads = num_heads;
  p.group = group;
  p.block_shift = pow2_shift(pool->block_size);
  p.tokens_per_tile = kPrefillRows / group;
  p.min_q_len = 1;
  p.scale_log2 = scale_log2;
  p.v_scale = pool->v_scale;
  p.causal = 0;
  p.window = 0;
  p.sinks = sinks;
  p.alibi = nullptr;
  p.merge = merge ? 1 : 0;
  p.new_lens = new_lens;
  p.new_tables = new_tables;
  p.new_max_blocks = new_max_blocks;
  p.status = status;
  p.tiles_per_seq = (max_query_len + p.tokens_per_tile - 1) / p.tokens_per_tile;
  const int64_t groups8 = ((int64_t)num_seqs * pool->num_kv_heads + 7) / 8 * 8;
  const int64_t wgs = groups8 * p.tiles_per_seq;
  if (wgs > 0x7fffffffLL) return PA_EUNSUPPORTED;
  if (wgs == 0) return PA_OK;
  return from_hip(launch_prefill(p, pool->dtype, q_dtype, pool->head_dim_k, pool->head_dim_v, dim3((unsigned)wgs), s));
}

int pa_merge_states(void* out, float* out_lse, const void* prefix_out, const float* prefix_lse,
                    const void* suffix_out, const float* suffix_lse, int64_t num_tokens, int32_t num_heads,
                    int32_t head_dim, int64_t prefill_tokens_with_context, int32_t dtype, void* stream) {
  if (num_tokens < 0 || num_heads < 1 || head_dim < 1) return PA_EINVAL;
  if (element_bytes(dtype) == 0) return PA_EUNSUPPORTED;
  if (num_tokens == 0) return PA_OK;
  if (out == nullptr || prefix_out == nullptr || prefix_lse == nullptr || suffix_out == nullptr ||
      suffix_lse == nullptr)
    return PA_EINVAL;
  MergeArgs a;
  a.out = out;
  a.out_lse = out_lse;
  a.prefix_out = prefix_out;
  a.prefix_lse = prefix_lse;
  a.suffix_out = suffix_out;
  a.suffix_lse = suffix_lse;
  a.num_tokens = num_tokens;
  a.num_heads = num_heads;
  a.head_dim = head_dim;
  a.with_prefix = prefill_tokens_with_context < 0 ? num_tokens : prefill_tokens_with_context;
  a.dtype = dtype;
  return from_hip(launch_merge(a, static_cast<hipStream_t>(stream)));
}

int pa_gather_cache(const void* cache, int32_t cache_dtype, int64_t num_blocks, int32_t block_size, int32_t head_dim,
                    int64_t cache_block_stride, int64_t cache_slot_stride, void* dst, int32_t dst_dtype,
                    int64_t dst_row_stride, const int32_t* block_table, int32_t max_blocks, const int32_t* cu_seq_lens,
                    const int32_t* token_to_seq, const int32_t* seq_starts, int32_t num_seqs, int64_t num_tokens,
                    int32_t* status, void* stream) {
  const int cb = element_bytes(cache_dtype), db = element_bytes(dst_dtype);
  if (cb == 0 || db == 0) return PA_EUNSUPPORTED;
  if (num_tokens < 0 || num_blocks < 1 || block_size < 1 || head_dim < 1 || max_blocks < 1 || num_seqs < 0)
    return PA_EINVAL;
  if (cache_slot_stride < head_dim || cache_block_stride < 1 || dst_row_stride < head_dim) return PA_EINVAL;
  if (num_tokens > 0 && (cache == nullptr || dst == nullptr || block_table == nullptr || cu_seq_lens == nullptr ||
                         token_to_seq == nullptr || num_seqs < 1))
    return PA_EINVAL;
  if (num_tokens > 0x7fffffffLL) return PA_EUNSUPPORTED;
  GatherArgs g = {};
  g.cache = cache;
  g.cache_dtype = cache_dtype;
  g.num_blocks = num_blocks;
  g.block_size = block_size;
  g.head_dim = head_dim;
  g.block_stride = cache_block_stride;
  g.slot_stride = cache_slot_stride;
  g.dst = dst;
  g.dst_dtype = dst_dtype;
  g.dst_stride = dst_row_stride;
  g.block_table = block_table;
  g.max_blocks = max_blocks;
  g.cu_seq_lens = cu_seq_lens;
  g.token_to_seq = token_to_seq;
  g.seq_starts = seq_starts;
  g.num_seqs = num_seqs;
  g.num_tokens = num_tokens;
  g.status = status;
  // 16-byte copies when nothing is converted and every row starts 16-byte aligned
  const bool aligned = ((uintptr_t)cache % 16 == 0) && ((uintptr_t)dst % 16 == 0) &&
                       ((int64_t)head_dim * cb) % 16 == 0 && (cache_block_stride * cb) % 16 == 0 &&
                       (cache_slot_stride * cb) % 16 == 0 && (dst_row_stride * db) % 16 == 0;
  g.vec16 = cache_dtype == dst_dtype && aligned;
  g.units_per_row = g.vec16 ? head_dim * cb / 16 : head_dim;
  return from_hip(launch_gather(g, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
