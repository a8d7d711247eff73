// Kernel argument blocks and launcher declarations shared by the host entry points
// (pa_api.hip) and the kernel translation units.  Internal to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// One workgroup answers one query row for one kv head (all q heads of its group),
// optionally restricted to one context partition.
struct RowsArgs {
  const void* k_pool;
  const void* v_pool;
  int64_t num_blocks;
  int block_size;
  int num_kv_heads;
  const void* q;
  void* out;
  int out_dtype;
  float* lse;  // [H, rows], nullable
  const int32_t* block_tables;
  int max_blocks;
  const int32_t* seq_lens;
  const int32_t* query_start_loc;  // nullptr: decode (row = sequence, query at n - 1)
  const int32_t* positions;        // varlen causal positions, nullable
  int single_token_seqs;           // varlen: row = sequence, only sequences of one token
  int skip_single_token_seqs;      // varlen, row = token: leave sequences of one token out
  int num_seqs;
  int64_t num_rows;  // decode: sequences; varlen: tokens
  int num_heads;
  int group;  // q heads per kv head
  float scale_log2;  // softmax scale (with the pool's k_scale folded in) times log2(e)
  float v_scale;     // the pool's v_scale: multiplies every output (and partition output)
  int causal;
  int window;
  int partition_size;  // 0: whole visible range
  int max_partitions;
  float* max_logits;
  float* exp_sums;
  float* tmp_out;
  const float* sinks;  // [num_heads] sink logits, nullable; unsplit outputs only
  const float* alibi;  // [num_heads] ALiBi slopes, nullable
  int merge;           // out (float32) and lse hold a state: merge this call's into it
  const int32_t* status;
};

struct ValidateArgs {
  int mode;  // kValidateWrite / kValidateDecode / kValidateVarlen
  int64_t num_blocks;
  int block_size;
  const int32_t* slot_mapping;
  int64_t num_new_tokens;
  const int32_t* block_tables;
  int max_blocks;
  const int32_t* seq_lens;
  int num_seqs;
  int partition_size;
  int max_partitions;
  const int32_t* query_start_loc;
  int64_t num_tokens;
  int max_query_len;
  const int32_t* positions;
  int causal;
  int positions_if_nonempty;  // causal positions checked only for sequences of length > 0
  int accumulate;             // OR into the status word left by an earlier check (no clear)
  int32_t* status;
};
// Latent-cache gather ("cpu_mla_prefill.cpp", GatherMlaCache).
struct GatherArgs {
  const void* cache;
  int cache_dtype;
  int64_t num_blocks;
  int block_size;
  int head_dim;
  int64_t block_stride;  // elements
  int64_t slot_stride;   // elements
  void* dst;
  int dst_dtype;
  int64_t dst_stride;  // elements per output row
  const int32_t* block_table;
  int max_blocks;
  const int32_t* cu_seq_lens;
  const int32_t* token_to_seq;
  const int32_t* seq_starts;  // nullable
  int num_seqs;
  int64_t num_tokens;
  int vec16;           // same dtype, rows and bases 16-byte aligned: 16-byte copies
  int units_per_row;   // 16-byte chunks (vec16) or elements per row
  int32_t* status;     // nullable
};
hipError_t launch_gather(const GatherArgs& a, hipStream_t stream);

constexpr int kValidateWrite = 0;
constexpr int kValidateDecode = 1;
constexpr int kValidateVarlen = 2;

struct WriteArgs {
  void* k_pool;
  void* v_pool;
  int64_t num_slots;
  int64_t k_row_bytes;  // num_kv_heads * head_dim_k * element bytes
  int64_t v_row_bytes;
  const void* k_new;
  const void* v_new;
  const int32_t* slot_mapping;
  int64_t num_tokens;
  const int32_t* status;
};

struct ReduceArgs {
  const float* max_logits;
  const float* exp_sums;
  const float* tmp_out;
  const int32_t* seq_lens;
  int max_blocks;
  int block_size;
  int num_seqs;
  int num_heads;
  int head_dim;
  int partition_size;
  int max_partitions;
  void* out;
  int out_dtype;
  const float* sinks;  // [num_heads] sink logits, nullable
  // varlen (nullable for decode): only sequences of exactly one query token were
  // split; their output row is query_start_loc[s], and lse [num_heads, num_rows]
  // (nullable) receives M + ln(sum of weights)
  const int32_t* query_start_loc;
  float* lse;
  int64_t num_rows;
  const int32_t* status;
};

struct MergeArgs {
  void* out;
  float* out_lse;
  const void* prefix_out;
  const float* prefix_lse;
  const void* suffix_out;
  const float* suffix_lse;
  int64_t num_tokens;
  int num_heads;
  int head_dim;
  int64_t with_prefix;  // tokens at or past this index copy the suffix
  int dtype;
};

// Returns hipErrorInvalidValue (without launching) for a combination not built.
hipError_t launch_rows(const RowsArgs& a, int dtype, int dk, int dv, dim3 grid, hipStream_t stream);
struct PrefillArgs;
hipError_t launch_prefill(const PrefillArgs& a, int kv_dtype, int q_dtype, int dk, int dv, dim3 grid,
                          hipStream_t stream);
bool prefill_supported(int kv_dtype, int q_dtype, int dk, int dv, int group, int block_size, int64_t num_blocks);
hipError_t launch_validate(const ValidateArgs& a, hipStream_t stream);
// Stores PA_OK in *status (the first kernel of a validated call).
hipError_t launch_status_clear(int32_t* status, hipStream_t stream);
hipError_t launch_write(const WriteArgs& a, hipStream_t stream);
hipError_t launch_reduce(const ReduceArgs& a, hipStream_t stream);
hipError_t launch_merge(const MergeArgs& a, hipStream_t stream);
bool rows_supported(int dtype, int dk, int dv, int group);
// Compute units of the current device (queried once per device), or 0 if the query
// fails.
int device_cu_count();

}  // namespace pa
