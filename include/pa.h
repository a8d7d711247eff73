/*
 * pa.h -- batched paged attention over a block-pooled KV cache, for AMD Instinct
 * MI355X (gfx950).  C ABI: plain pointers and sizes, no framework types.
 *
 * Data model (TensorSharp "ManagedPagedAttention.cs", class summary; "Paged attention
 * for decode in C", section 2.1):
 *   - A pool holds K and V in blocks of `block_size` token slots:
 *       K [num_blocks, block_size, num_kv_heads, head_dim_k]
 *       V [num_blocks, block_size, num_kv_heads, head_dim_v]
 *     row-major, all in the pool's element type.  Slot = block_id * block_size +
 *     offset is the flat index of a [num_kv_heads, head_dim] row.
 *   - Sequence s owns row s of `block_tables` ([num_seqs, max_blocks], int32): its
 *     position j lives at offset j % block_size of block block_tables[s][j / block_size].
 *     Ids are arbitrary; several tables may name one block (shared prefixes).
 *   - q and out are [tokens, num_heads, head_dim].  q head h reads kv head
 *     h / (num_heads / num_kv_heads) (grouped-query attention).
 *   - A query at position pos of a sequence of seq_len tokens sees positions
 *     [start, end): end = pos + 1 when causal, else seq_len; start = max(0, end -
 *     sliding_window) when sliding_window > 0, else 0.  Scores are
 *     scale * <q, k_j> (plus an ALiBi term when slopes are given, see pa_decode),
 *     normalised by softmax over the visible positions; scale must be finite and
 *     > 0 (else PA_EINVAL).
 *   - lse arrays are float32 [num_heads, tokens] in natural log; a row that sees no
 *     position has output 0 and lse -inf ("cpu_mla_prefill.cpp", MlaPrefillAttention).
 *   - Every stored K element counts as its value times the pool's k_scale, every V
 *     element as its value times v_scale ("paged_attention_v2_pytorch.py", phase 1,
 *     the KV gather); 1.0 leaves a cache as stored.  A pool of PA_FP8_E4M3 holds
 *     the OCP 8-bit E4M3 format (4 exponent bits, bias 7, 3 fraction bits, largest
 *     finite 448, no infinities) -- the fp8 KV caches of "Paged attention for decode
 *     in C" (table of extensions); its queries are f16 or bf16 (outputs float32 or
 *     the queries' type).
 *
 * Ownership and streams: the caller owns every buffer.  The library allocates no
 * memory and keeps no state between calls (pa_decode_noalloc's static device buffer
 * aside, see there), and enqueues all work on `stream` (a
 * hipStream_t; NULL is the default stream) without synchronising.  Device pointers
 * must stay valid until the work completes.  The pool descriptor is host memory and
 * is read during the call only.
 *
 * Errors: every entry point returns a pa_status synchronously.  Argument errors
 * (null pointers, sizes, unsupported combinations) are found on the host, and then
 * nothing is enqueued, so outputs are untouched.  Errors in device-resident content
 * (block ids, lengths, positions, slots, query_start_loc) can only be found on the
 * device: when `status` (a device int32) is non-NULL, a validation kernel runs first
 * on the same stream and stores PA_OK or PA_EINVAL there, and every later kernel of
 * the call exits before writing anything if it holds an error.  Read it after the
 * stream synchronises.  With status == NULL no validation runs; kernels still never
 * read or write outside the pool, the tables or the outputs (bad ids are clamped),
 * but results for invalid content are unspecified.
 *
 * Element offsets are computed in 64 bits, so pools may exceed 2^31 elements.
 */
#ifndef PA_H_
#define PA_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
  PA_OK = 0,
  PA_EINVAL = 1,       /* bad argument or bad device content */
  PA_ESHAPE = 2,       /* num_heads % num_kv_heads != 0, or dims that disagree */
  PA_EUNSUPPORTED = 3, /* an element type / head-dim / group combination not built */
  PA_EDEVICE = 4,      /* a HIP launch failed */
  PA_ESCRATCH = 5      /* pa_decode_noalloc: the call needs more than its static workspace */
} pa_status;

typedef enum pa_dtype { PA_F32 = 0, PA_F16 = 1, PA_BF16 = 2, PA_FP8_E4M3 = 3 } pa_dtype;

typedef struct pa_kv_pool {
  void* k;              /* device, [num_blocks, block_size, num_kv_heads, head_dim_k] */
  void* v;              /* device, [num_blocks, block_size, num_kv_heads, head_dim_v] */
  int64_t num_blocks;   /* >= 1 */
  int32_t block_size;   /* tokens per block, >= 1 */
  int32_t num_kv_heads; /* >= 1 */
  int32_t head_dim_k;   /* QK head dim */
  int32_t head_dim_v;   /* V head dim */
  int32_t dtype;        /* pa_dtype of both pools */
  float k_scale;        /* finite, > 0: K element = stored value * k_scale (1.0: none) */
  float v_scale;        /* finite, > 0: V element = stored value * v_scale (1.0: none) */
} pa_kv_pool;

/* Static text for a status code: the status codes of "Paged attention for decode in
 * C" (section 4, the interface and its error returns), plus PA_ESCRATCH. */
const char* pa_strerror(int status);

/* Write new tokens' K and V into their pool slots (TensorSharp page,
 * WriteKvToPagedPool).  k_new [num_tokens, num_kv_heads, head_dim_k] and v_new
 * [num_tokens, num_kv_heads, head_dim_v] are device arrays in the pool dtype (already
 * quantized, for an fp8 pool); token t goes to slot slot_mapping[t] (device int32).
 * Bytes are copied unchanged; a row must be a multiple of 4 bytes.
 * Device check (with status): every slot in [0, num_blocks * block_size).  A slot
 * repeated within one call is written by one of its tokens, unspecified which.
 * num_tokens == 0 enqueues nothing. */
int pa_write_kv(const pa_kv_pool* pool, const void* k_new, const void* v_new,
                const int32_t* slot_mapping, int64_t num_tokens, int32_t* status, void* stream);

/* One decode step ("Paged attention for decode in C", sections 2.2-2.6): for each
 * sequence s and head h, the query q[s, h, :] sits at position seq_lens[s] - 1
 * (causal) and attends over its visible positions.
 *   q [num_seqs, num_heads, head_dim_k] in q_dtype (the pool dtype; F16 or BF16 for
 *     an fp8 pool);
 *   out [num_seqs, num_heads, head_dim_v] in out_dtype (PA_F32 or q_dtype);
 *   block_tables [num_seqs, max_blocks]; seq_lens [num_seqs] (device int32).
 * partition_size == 0: one pass per (sequence, kv head).
 * partition_size > 0 (a multiple of block_size): split-KV, after
 * "paged_attention_v2_pytorch.py".  Partition p covers positions
 * [p * partition_size, (p + 1) * partition_size); for p < ceil(seq_len /
 * partition_size) the call stores, in caller-owned float32 workspaces,
 *   max_logits [num_seqs, num_heads, max_partitions]  max score over the partition,
 *   exp_sums   [num_seqs, num_heads, max_partitions]  sum of exp(score - max),
 *   tmp_out    [num_seqs, num_heads, max_partitions, head_dim_v]  the partition's
 *              softmax-normalised output,
 * with (-inf, 0, 0) for a partition outside the window; entries at larger p are
 * not touched.  A second kernel then combines the partitions into out with
 * log-sum-exp weights exp_sums * exp(max_logits - max).  The workspaces may be NULL
 * when partition_size == 0.
 * Device checks (with status): seq_len >= 1, ceil(seq_len / block_size) <=
 * max_blocks, the first ceil(seq_len / block_size) ids in [0, num_blocks), and
 * ceil(seq_len / partition_size) <= max_partitions.
 * sinks [num_heads] float32 (device, nullable): per-head attention-sink logits
 * (TensorSharp page, ForwardWithSinks): head h's softmax gains one more position of
 * score sinks[h] and value zero, which takes probability mass and adds nothing to
 * the output; -inf means no sink.  With partitions the workspaces stay sink-free and
 * the sink joins in the combining step.
 * alibi_slopes [num_heads] float32 (device, nullable): ALiBi ("paged_attention_v2_pytorch.py",
 * phase 1): head h's score for position j gains slopes[h] * (j - (end - 1)), end - 1
 * being the query's position.  Per row this differs from the page's slopes[h] * j by
 * a constant, so outputs are the page's; max_logits (and lse, in pa_varlen) are the
 * page's minus slopes[h] * (end - 1), which keeps them exact at long contexts.
 * Slopes must be finite.  A sink logit competes with these biased scores.
 * Supported: head_dim_k == head_dim_v in {32, 64, 128, 256}; num_heads /
 * num_kv_heads <= 16 (<= 8 at head dim 256); any block_size.  PA_FP8_E4M3 pools: q_dtype PA_F16 or PA_BF16,
 * head dims 128, block_size a power of two >= 16. */
int pa_decode(const pa_kv_pool* pool, const void* q, int32_t q_dtype, void* out, int32_t out_dtype,
              const int32_t* block_tables, int32_t max_blocks, const int32_t* seq_lens,
              int32_t num_seqs, int32_t num_heads, float scale, int32_t sliding_window,
              int32_t partition_size, int32_t max_partitions, float* max_logits, float* exp_sums,
              float* tmp_out, const float* sinks, const float* alibi_slopes, int32_t* status,
              void* stream);

/* pa_decode for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same arguments and
 * results as pa_decode, except that split-KV (partition_size > 0) keeps its
 * partition states in a static device buffer of the library instead of caller
 * workspaces: 96 MiB per GPU, held from the first call on that GPU until the process
 * ends.  The states need num_seqs * num_heads * max_partitions * (head_dim_v + 2) * 4
 * bytes (each of the three arrays rounded up to 256), max_partitions =
 * ceil(max_blocks * block_size / partition_size); a call that needs more returns
 * PA_ESCRATCH and enqueues nothing.  partition_size == 0 is pa_decode unsplit.
 * The buffer of the current device is used (the stream must belong to it); every
 * call on one GPU shares it, so calls whose work overlaps on one GPU (other streams,
 * other threads) race on it.  Nothing in it needs clearing: each call writes every
 * state it reads.  The first call on each device resolves the buffer's address
 * (hipGetSymbolAddress); make it outside graph capture.  The call itself allocates,
 * frees and copies nothing. */
int pa_decode_noalloc(const pa_kv_pool* pool, const void* q, int32_t q_dtype, void* out, int32_t out_dtype,
                      const int32_t* block_tables, int32_t max_blocks, const int32_t* seq_lens,
                      int32_t num_seqs, int32_t num_heads, float scale, int32_t sliding_window,
                      int32_t partition_size, const float* sinks, const float* alibi_slopes, int32_t* status,
                      void* stream);

/* Variable-length attention over many sequences in one call (TensorSharp page,
 * Forward; "cpu_mla_prefill.cpp", MlaPrefillAttention): prefill chunks and single
 * decode tokens mixed.  Sequence s owns query tokens [query_start_loc[s],
 * query_start_loc[s + 1]) of q [num_tokens, num_heads, head_dim_k] and holds
 * seq_lens[s] >= 0 cached positions.  positions [num_tokens] give each token's
 * absolute position (used for the causal bound only; may be NULL when causal == 0).
 * out [num_tokens, num_heads, head_dim_v] in out_dtype (PA_F32 or q_dtype);
 * lse [num_heads, num_tokens] float32, nullable.  max_query_len is an upper bound on
 * any sequence's token count (sizes the grid).  A row that sees nothing gets
 * out = 0 and lse = -inf; sequences with no tokens are skipped.
 * Device checks (with status): query_start_loc[0] == 0, non-decreasing, last entry
 * == num_tokens; every token count <= max_query_len; seq_len >= 0;
 * ceil(seq_len / block_size) <= max_blocks with those ids in [0, num_blocks); when
 * causal, every position in [0, seq_len).
 * sinks [num_heads] float32 (device, nullable): per-head attention-sink logits, as
 * for pa_decode (TensorSharp page, ForwardWithSinks).  The lse then includes the
 * sink's mass (a row that sees nothing gets out = 0 and lse = sinks[h]); when
 * states of several calls are merged, give the sinks to one of them only.
 * alibi_slopes [num_heads] float32 (device, nullable): ALiBi as for pa_decode, the
 * bias counted from each row's last visible position end - 1 (the token's position
 * when causal, seq_len - 1 otherwise).
 * partition_size > 0 (a multiple of block_size): sequences holding exactly one query
 * token are computed split-KV, as pa_decode does ("paged_attention_v2_pytorch.py",
 * phases 1 and 2), so that a few long single-token rows spread over the whole GPU.
 * max_logits / exp_sums [num_seqs, num_heads, max_partitions] and tmp_out [num_seqs,
 * num_heads, max_partitions, head_dim_v] are caller-owned float32 scratch, indexed by
 * sequence; their contents after the call are unspecified.  Device check (with
 * status): ceil(seq_len / partition_size) <= max_partitions for those sequences.
 * partition_size == 0: no split, workspaces may be NULL.  Ignored for shapes whose
 * single-token rows run on the tiled kernel (the row kernels do not take them).
 * Supported: (head_dim_k, head_dim_v) in {(32,32), (64,64), (128,128), (256,256),
 * (192,128)}; num_heads / num_kv_heads <= 16 (<= 8 at (256,256)); any block_size.
 * Beyond that, the tiled kernel's shapes (below) with num_heads / num_kv_heads up
 * to 128.
 * PA_FP8_E4M3 pools: q_dtype PA_F16 or PA_BF16, block_size a power of two >= 16,
 * num_blocks * block_size < 2^32, and (head_dim_k, head_dim_v) = (128,128) with
 * num_heads / num_kv_heads <= 16 (single-token sequences on the fp8 decode kernel,
 * longer ones on the tiled kernel), or any call on the tiled kernel's fp8 shapes:
 * (128,128) or (192,128), num_heads / num_kv_heads <= 128.
 * Which kernel runs: sequences of two or more query tokens run on the tiled MFMA
 * prefill kernel when the pool is F16 or BF16 with (head_dim_k, head_dim_v) in
 * {(64,64), (128,128), (192,128)}, or FP8_E4M3 with (128,128) or (192,128), and
 * block_size is a power of two >= 16 and num_blocks * block_size < 2^32 (an fp8
 * pool's K is widened exactly to q_dtype, V to f16, as the tiles are staged);
 * single-token sequences then run on the decode kernels, or on the tiled kernel too
 * where the decode kernels do not take the shape.  Any other supported shape (F32
 * pools, head dims 32 or 256, other block sizes) runs every token on the per-row
 * kernel, one workgroup per (token, kv head): the same results, at a small fraction
 * of the tiled kernel's rate for long prefills.
 * ALiBi and merging: the bias is counted from each row's own end - 1, so a row's
 * lse carries an offset of slopes[h] * (end - 1) from the page's form.  States of
 * calls that see a row with different ends (for example context chunks read as
 * separate sequences) are on different origins and must not be merged with
 * pa_merge_states or pa_varlen_merge; merge ALiBi states only when each row's end
 * is the same in both calls. */
int pa_varlen(const pa_kv_pool* pool, const void* q, int32_t q_dtype, void* out, int32_t out_dtype,
              float* lse, const int32_t* query_start_loc, const int32_t* seq_lens,
              const int32_t* positions, const int32_t* block_tables, int32_t max_blocks,
              int32_t num_seqs, int64_t num_tokens, int32_t max_query_len, int32_t num_heads,
              float scale, int32_t causal, int32_t sliding_window, int32_t partition_size,
              int32_t max_partitions, float* max_logits, float* exp_sums, float* tmp_out,
              const float* sinks, const float* alibi_slopes, int32_t* status, void* stream);

/* Varlen attention merged into an existing state ("cpu_mla_prefill.cpp",
 * MlaPrefillAttention then MergeAttnStates, fused): out [num_tokens, num_heads,
 * head_dim_v] float32 and lse [num_heads, num_tokens] float32 hold a state over some
 * keys; this call computes the attention of q over its visible positions, as
 * pa_varlen does, and merges it in as the suffix by pa_merge_states' rules (an lse of
 * +inf counts as -inf; when both lse are -inf the row is left as it is and its lse
 * becomes -inf).  The other arguments are pa_varlen's, without split-KV.  lse must be
 * non-NULL (else PA_EINVAL).  It saves writing this call's state and reading both
 * back, as a separate pa_merge_states would.  Supported: as pa_varlen. */
int pa_varlen_merge(const pa_kv_pool* pool, const void* q, int32_t q_dtype, float* out, float* lse,
                    const int32_t* query_start_loc, const int32_t* seq_lens, const int32_t* positions,
                    const int32_t* block_tables, int32_t max_blocks, int32_t num_seqs, int64_t num_tokens,
                    int32_t max_query_len, int32_t num_heads, float scale, int32_t causal,
                    int32_t sliding_window, const float* sinks, const float* alibi_slopes, int32_t* status,
                    void* stream);

/* Attention over a context segment and the sequence's new tokens in one pass
 * ("cpu_mla_prefill.cpp": the chunked-context prefill -- MlaPrefillAttention over a
 * context chunk and over the new tokens, MergeAttnStates to combine them -- with the
 * two key sets in one softmax).  Token t of sequence s (query_start_loc as for
 * pa_varlen) sees every position [0, ctx_lens[s]) of ctx_tables (non-causal) and,
 * when new_lens[s] > 0, positions [0, new_positions[t] + 1) of new_tables (the new
 * tokens, causal; new_positions are positions within them).  With merge == 0, out
 * [num_tokens, num_heads, head_dim_v] and lse [num_heads, num_tokens] (float32, both
 * required) receive the result; with merge != 0 they hold a state and the result is
 * merged into it as the suffix, by pa_merge_states' rules.  Equal to merging the
 * context segment's state and then the new tokens' (up to rounding), without the
 * second pass over the state.  Pool element type = q_dtype, or PA_FP8_E4M3 with
 * q_dtype PA_F16 or PA_BF16 (scales as everywhere); no window, ALiBi or split-KV;
 * sinks as for pa_varlen.  Device checks (with status): query_start_loc
 * as for pa_varlen; ctx_lens and new_lens >= 0 with their first ceil(len /
 * block_size) ids in [0, num_blocks) and at most ctx_max_blocks / new_max_blocks of
 * them; every new_position in [0, new_lens[s]) where new_lens[s] > 0.  Supported:
 * the shapes pa_varlen runs on its tiled kernel (F16 / BF16 with (head_dim_k,
 * head_dim_v) in {(64,64), (128,128), (192,128)}, FP8_E4M3 with (128,128) or
 * (192,128); power-of-two block_size >= 16, num_blocks * block_size < 2^32,
 * num_heads / num_kv_heads <= 128); every sequence runs on the tiled kernel. */
int pa_varlen_ctx_new(const pa_kv_pool* pool, const void* q, int32_t q_dtype, float* out, float* lse, int32_t merge,
                      const int32_t* query_start_loc, const int32_t* ctx_lens, const int32_t* ctx_tables,
                      int32_t ctx_max_blocks, const int32_t* new_lens, const int32_t* new_positions,
                      const int32_t* new_tables, int32_t new_max_blocks, int32_t num_seqs, int64_t num_tokens,
                      int32_t max_query_len, int32_t num_heads, float scale, const float* sinks, int32_t* status,
                      void* stream);

/* Merge two attention states over disjoint key sets ("cpu_mla_prefill.cpp",
 * MergeAttnStates).  prefix_out, suffix_out, out: [num_tokens, num_heads, head_dim] in
 * dtype; prefix_lse, suffix_lse, out_lse (nullable): float32 [num_heads, num_tokens].
 * Tokens t >= prefill_tokens_with_context (when that is >= 0) copy the suffix state.
 * Otherwise an lse of +inf is treated as -inf; if both are then -inf the prefix
 * output is copied and out_lse = -inf; else with M = max of the two, weights
 * exp(lse - M) are normalised, the outputs blended and out_lse = M + ln(sum of
 * weights).  out may alias prefix_out or suffix_out. */
int pa_merge_states(void* out, float* out_lse, const void* prefix_out, const float* prefix_lse,
                    const void* suffix_out, const float* suffix_lse, int64_t num_tokens,
                    int32_t num_heads, int32_t head_dim, int64_t prefill_tokens_with_context,
                    int32_t dtype, void* stream);

/* Gather of a paged latent cache into contiguous rows ("cpu_mla_prefill.cpp",
 * GatherMlaCache): the step that lays out a context chunk of an MLA latent cache
 * before chunked prefill.  cache: num_blocks x block_size rows of head_dim elements
 * in cache_dtype, row (block, slot) at element block * cache_block_stride + slot *
 * cache_slot_stride.  dst: num_tokens rows of head_dim elements in dst_dtype, row t
 * at element t * dst_row_stride (>= head_dim).  Row t belongs to sequence
 * b = token_to_seq[t]; it is left untouched when t >= cu_seq_lens[b + 1]; otherwise
 * its position is t - cu_seq_lens[b], plus seq_starts[b] when seq_starts is
 * non-NULL, and it receives the cache row at slot position % block_size of block
 * block_table[b][position / block_size], rounded to nearest even when the dtypes
 * differ.  block_table [num_seqs, max_blocks], cu_seq_lens [num_seqs + 1],
 * token_to_seq [num_tokens], seq_starts [num_seqs] (nullable): device int32.
 * Device checks (with status): b in [0, num_seqs), position >= 0, position /
 * block_size < max_blocks, block id in [0, num_blocks); without a status word such
 * rows are skipped.  Supported: F32 / F16 / BF16 on either side. */
int pa_gather_cache(const void* cache, int32_t cache_dtype, int64_t num_blocks, int32_t block_size,
                    int32_t head_dim, int64_t cache_block_stride, int64_t cache_slot_stride, void* dst,
                    int32_t dst_dtype, int64_t dst_row_stride, const int32_t* block_table,
                    int32_t max_blocks, const int32_t* cu_seq_lens, const int32_t* token_to_seq,
                    const int32_t* seq_starts, int32_t num_seqs, int64_t num_tokens, int32_t* status,
                    void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
