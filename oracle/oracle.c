/*
 * oracle.c -- a plain, slow CPU implementation of batched paged attention over a
 * block-pooled KV cache.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load this library.  The GPU library never links, calls or
 * reads it, and the two share no source, header, table or helper.
 *
 * What each function follows (page title, then the section on that page):
 *   - "ManagedPagedAttention.cs" (TensorSharp), class summary: tensor layouts
 *     q/out [tokens, heads, dim], pools [blocks, blockSize, kvHeads, dim], and the
 *     per-sequence metadata queryStartLoc / seqLens / blockTables / positions /
 *     slotMapping with slot = blockId * blockSize + offset.
 *   - same page, Forward: the q-head -> kv-head map h / (H / Hkv) and the visible
 *     range (end = causal ? pos + 1 : seqLen, start = max(0, end - window) when the
 *     window is positive).
 *   - same page, WriteKvToPagedPool: the slot scatter, applied in token order.
 *   - "Paged attention for decode in C", sections 2.1-2.2: position j lives in slot
 *     j mod b of block table[j / b]; a decode query sits at position n - 1.
 *     Section 2.6: validation before anything is written.  Section 3: the worked
 *     example the tests pin against.
 *   - "paged_attention_v2_pytorch.py", phase 1 and phase 2: per-partition
 *     max logit, exp-sum and output, reduced by log-sum-exp weights.
 *   - "cpu_mla_prefill.cpp", MlaPrefillAttention: the two-pass softmax (max, then
 *     exp-sum and weighted sum), zero output and lse = -inf for an empty row, lse
 *     in natural log.  MergeAttnStates: the merge and its two edge cases.
 *     GatherMlaCache: the gather of a paged latent cache into contiguous rows.
 *   - "ManagedPagedAttention.cs", ForwardWithSinks: attention sinks.
 *   - "paged_attention_v2_pytorch.py", phase 1 (Alibi): a per-head slope times the
 *     key's position is added to each score.  Here the position is counted from the
 *     row's last visible position, end - 1 (slope * (j - (end - 1))): per row this
 *     differs from the page's slope * j by a constant, so every softmax weight and
 *     output is the page's, while lse and partition maxima are the page's minus
 *     slope * (end - 1).
 *   - "paged_attention_v2_pytorch.py", phase 1 (the batched KV gather): the cache's
 *     k_scale / v_scale multiply every gathered K / V element.  "Paged attention for
 *     decode in C", the table of extensions: fp8 KV caches, read here as the OCP
 *     8-bit E4M3 format (4 exponent bits with bias 7, 3 fraction bits, no
 *     infinities, one NaN pattern per sign).
 *
 * Arithmetic: every stored element is decoded exactly to binary32 and then widened
 * to binary64; every sum, exp and log is binary64.  Work is split over (sequence,
 * kv-head) tasks with a fixed assignment, so results do not depend on the number of
 * threads.  Outputs are written only after all checks pass.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_EINVAL 1
#define ORC_ESHAPE 2
#define ORC_EUNSUPPORTED 3

#define ORC_F32 0
#define ORC_F16 1
#define ORC_BF16 2
#define ORC_FP8_E4M3 3

/* ------------------------------------------------------------------------- */
/* Element decoding                                                           */
/* ------------------------------------------------------------------------- */

static int elem_bytes(int dtype) {
  if (dtype == ORC_F32) return 4;
  if (dtype == ORC_F16 || dtype == ORC_BF16) return 2;
  if (dtype == ORC_FP8_E4M3) return 1;
  return 0;
}

/* IEEE 754 binary16: sign bit, 5 exponent bits with bias 15, 10 fraction bits. */
static double half_to_double(uint16_t h) {
  int sign = h >> 15;
  int e = (h >> 10) & 0x1f;
  int f = h & 0x3ff;
  double mag;
  if (e == 0)
    mag = ldexp((double)f, -24); /* zero or subnormal: f * 2^-24 */
  else if (e == 31)
    mag = f ? NAN : INFINITY;
  else
    mag = ldexp((double)(1024 + f), e - 25); /* (1 + f / 2^10) * 2^(e - 15) */
  return sign ? -mag : mag;
}

/* bfloat16 is the high half of a binary32 word. */
static double bf16_to_double(uint16_t h) {
  uint32_t bits = (uint32_t)h << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* OCP 8-bit E4M3: sign bit, 4 exponent bits with bias 7, 3 fraction bits.  Exponent
 * field 0 is zero or subnormal (f * 2^-9); exponent 15 with fraction 7 is NaN, every
 * other pattern is finite (largest 448); there is no infinity.                     */
static double e4m3_to_double(uint8_t b) {
  int sign = b >> 7;
  int e = (b >> 3) & 0xf;
  int f = b & 0x7;
  double mag;
  if (e == 0)
    mag = ldexp((double)f, -9);
  else if (e == 15 && f == 7)
    mag = NAN;
  else
    mag = ldexp((double)(8 + f), e - 10); /* (1 + f / 8) * 2^(e - 7) */
  return sign ? -mag : mag;
}

static double load_elem(const void* base, int dtype, int64_t i) {
  if (dtype == ORC_F32) return (double)((const float*)base)[i];
  if (dtype == ORC_F16) return half_to_double(((const uint16_t*)base)[i]);
  if (dtype == ORC_FP8_E4M3) return e4m3_to_double(((const uint8_t*)base)[i]);
  return bf16_to_double(((const uint16_t*)base)[i]);
}

/* Decode n stored elements to binary64 (exposed so the decoders can be pinned). */
int orc_decode_elems(const void* src, int dtype, int64_t n, double* out) {
  if (elem_bytes(dtype) == 0) return ORC_EUNSUPPORTED;
  for (int64_t i = 0; i < n; ++i) out[i] = load_elem(src, dtype, i);
  return ORC_OK;
}

/* ------------------------------------------------------------------------- */
/* A fixed-assignment parallel loop: task i runs on thread i mod nthreads.    */
/* ------------------------------------------------------------------------- */

typedef void (*task_fn)(void* ctx, int64_t task);

struct worker_arg {
  task_fn fn;
  void* ctx;
  int64_t ntasks;
  int nthreads;
  int tid;
};

static void* worker_main(void* p) {
  struct worker_arg* a = (struct worker_arg*)p;
  for (int64_t i = a->tid; i < a->ntasks; i += a->nthreads) a->fn(a->ctx, i);
  return NULL;
}

static void parallel_for(int64_t ntasks, int nthreads, task_fn fn, void* ctx) {
  if (nthreads < 1) nthreads = 1;
  if ((int64_t)nthreads > ntasks) nthreads = (int)(ntasks > 0 ? ntasks : 1);
  if (nthreads == 1) {
    for (int64_t i = 0; i < ntasks; ++i) fn(ctx, i);
    return;
  }
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
  struct worker_arg* args = (struct worker_arg*)malloc(sizeof(struct worker_arg) * (size_t)nthreads);
  for (int i = 0; i < nthreads; ++i) {
    args[i].fn = fn;
    args[i].ctx = ctx;
    args[i].ntasks = ntasks;
    args[i].nthreads = nthreads;
    args[i].tid = i;
    pthread_create(&th[i], NULL, worker_main, &args[i]);
  }
  for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
  free(args);
  free(th);
}

/* ------------------------------------------------------------------------- */
/* Explicit gather through a block table                                      */
/* ------------------------------------------------------------------------- */

/* Copy positions 0..n-1 of one sequence, kv head g, out of a pool laid out as
 * [num_blocks, block_size, num_kv_heads, head_dim] into dst[j * head_dim + d], each
 * element multiplied by the pool's scale (k_scale or v_scale).
 * Position j is in block table[j / block_size] at offset j % block_size.        */
static void gather_head(const void* pool, int dtype, double scale, int block_size, int num_kv_heads,
                        int head_dim, const int32_t* table, int64_t n, int g, double* dst) {
  for (int64_t j = 0; j < n; ++j) {
    int64_t block_id = table[j / block_size];
    int64_t slot = block_id * block_size + j % block_size;
    int64_t base = (slot * num_kv_heads + g) * head_dim;
    for (int d = 0; d < head_dim; ++d) dst[j * head_dim + d] = load_elem(pool, dtype, base + d) * scale;
  }
}

/* Gather every kv head: out[(j * num_kv_heads + g) * head_dim + d].
 * The table must hold at least ceil(seq_len / block_size) ids below num_blocks. */
int orc_gather(const void* pool, int dtype, int64_t num_blocks, int block_size, int num_kv_heads,
               int head_dim, const int32_t* table, int32_t table_len, int32_t seq_len, double* out) {
  if (elem_bytes(dtype) == 0) return ORC_EUNSUPPORTED;
  if (block_size < 1 || num_kv_heads < 1 || head_dim < 1 || seq_len < 0) return ORC_EINVAL;
  int64_t need = ((int64_t)seq_len + block_size - 1) / block_size;
  if (need > table_len) return ORC_EINVAL;
  for (int64_t i = 0; i < need; ++i)
    if (table[i] < 0 || table[i] >= num_blocks) return ORC_EINVAL;
  for (int64_t j = 0; j < seq_len; ++j) {
    int64_t block_id = table[j / block_size];
    int64_t slot = block_id * block_size + j % block_size;
    for (int g = 0; g < num_kv_heads; ++g) {
      int64_t base = (slot * num_kv_heads + g) * head_dim;
      for (int d = 0; d < head_dim; ++d)
        out[(j * num_kv_heads + g) * head_dim + d] = load_elem(pool, dtype, base + d);
    }
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------------- */
/* The two-pass softmax over an explicitly gathered cache                    */
/* ------------------------------------------------------------------------- */

/* One query q[dk] against keys K[j * dk + d] and values V[j * dv + d] for the
 * visible positions lo <= j < hi.  Pass 1 forms each score scale * <q, k_j> plus the
 * ALiBi term slope * (j - ref) (slope 0: none) and the maximum m; pass 2 forms
 * e_j = exp(s_j - m), l = sum e_j and a = sum e_j v_j.  The
 * output is a * (1 / l).  An attention sink ("ManagedPagedAttention.cs",
 * ForwardWithSinks) is one more position with score `sink` and a zero value: it
 * enters the maximum and the exp-sum, not the numerator (sink = -inf: none).  An
 * empty range without a sink gives a zero output, m = -inf, l = 0; with a sink, a
 * zero output, m = sink, l = 1.  s is scratch of at least hi - lo doubles.        */
static void attend(const double* q, const double* K, const double* V, int dk, int dv, int64_t lo,
                   int64_t hi, double scale, double sink, double slope, int64_t ref, double* s,
                   double* out, double* m_out, double* l_out) {
  for (int d = 0; d < dv; ++d) out[d] = 0.0;
  double m = sink;
  for (int64_t j = lo; j < hi; ++j) {
    double dot = 0.0;
    for (int d = 0; d < dk; ++d) dot += q[d] * K[j * dk + d];
    s[j - lo] = scale * dot + slope * (double)(j - ref);
    if (s[j - lo] > m) m = s[j - lo];
  }
  if (m == -INFINITY) { /* nothing visible and no sink */
    *m_out = -INFINITY;
    *l_out = 0.0;
    return;
  }
  double l = sink == -INFINITY ? 0.0 : exp(sink - m);
  for (int64_t j = lo; j < hi; ++j) {
    s[j - lo] = exp(s[j - lo] - m);
    l += s[j - lo];
  }
  for (int64_t j = lo; j < hi; ++j)
    for (int d = 0; d < dv; ++d) out[d] += s[j - lo] * V[j * dv + d];
  double inv = 1.0 / l;
  for (int d = 0; d < dv; ++d) out[d] *= inv;
  *m_out = m;
  *l_out = l;
}

static double lse_of(double m, double l) { return l > 0.0 ? m + log(l) : -INFINITY; }

/* The core on caller-gathered arrays: row r has query q[r * dk ..], visible range
 * [lo[r], hi[r]) of K / V (n_keys rows).  Writes out[r * dv ..] and lse[r].      */
int orc_attend_gathered(const double* q, const double* K, const double* V, int64_t n_keys, int dk,
                        int dv, const int64_t* lo, const int64_t* hi, int64_t num_rows, double scale,
                        double* out, double* lse) {
  for (int64_t r = 0; r < num_rows; ++r)
    if (lo[r] < 0 || hi[r] > n_keys) return ORC_EINVAL;
  int64_t widest = 1;
  for (int64_t r = 0; r < num_rows; ++r)
    if (hi[r] - lo[r] > widest) widest = hi[r] - lo[r];
  double* s = (double*)malloc(sizeof(double) * (size_t)widest);
  for (int64_t r = 0; r < num_rows; ++r) {
    double m, l;
    attend(q + r * dk, K, V, dk, dv, lo[r], hi[r], scale, -INFINITY, 0.0, 0, s, out + r * dv, &m, &l);
    lse[r] = lse_of(m, l);
  }
  free(s);
  return ORC_OK;
}

/* ------------------------------------------------------------------------- */
/* Paged attention over many sequences                                         */
/* ------------------------------------------------------------------------- */

struct pool_desc {
  const void* k;
  const void* v;
  int dtype;
  double k_scale; /* multiplies every stored K element */
  double v_scale; /* multiplies every stored V element */
  int64_t num_blocks;
  int block_size;
  int num_kv_heads;
  int dk;
  int dv;
};

struct attn_job {
  struct pool_desc pool;
  const void* q;
  int q_dtype;
  int num_heads;
  int64_t num_tokens;
  const int32_t* query_start_loc;
  int num_seqs;
  const int32_t* seq_lens;
  const int32_t* positions;
  const int32_t* block_tables;
  int max_blocks;
  double scale;
  int causal;
  int sliding_window;
  const uint8_t* row_mask; /* [T * H], nullable: compute every row */
  const double* sinks;     /* [H] sink logits, nullable: none */
  const double* alibi;     /* [H] ALiBi slopes, nullable: none */
  double* out;             /* [T, H, dv] */
  double* lse;             /* [H, T], nullable */
  /* split-KV outputs (partition_size > 0) */
  int partition_size;
  int max_partitions;
  double* max_logits; /* [S, H, max_partitions] */
  double* exp_sums;   /* [S, H, max_partitions] */
  double* tmp_out;    /* [S, H, max_partitions, dv] */
};

/* Visible positions of a query: [start, end) with end = pos + 1 when causal and
 * n otherwise, and start = max(0, end - window) when the window is positive.  */
static void visible_range(const struct attn_job* job, int64_t t, int64_t n, int64_t* start,
                          int64_t* end) {
  int64_t e = job->causal ? (int64_t)job->positions[t] + 1 : n;
  int64_t s = 0;
  if (job->sliding_window > 0) {
    s = e - job->sliding_window;
    if (s < 0) s = 0;
  }
  *start = s;
  *end = e;
}

static int row_wanted(const struct attn_job* job, int64_t t, int h) {
  return job->row_mask == NULL || job->row_mask[t * job->num_heads + h];
}

/* Task = (sequence s, kv head g): gather that head's K and V once, then answer every
 * requested (token, q-head) row of the group. */
static void attn_task(void* ctx, int64_t task) {
  const struct attn_job* job = (const struct attn_job*)ctx;
  const struct pool_desc* P = &job->pool;
  int s = (int)(task / P->num_kv_heads);
  int g = (int)(task % P->num_kv_heads);
  int group = job->num_heads / P->num_kv_heads;
  int64_t t0 = job->query_start_loc[s], t1 = job->query_start_loc[s + 1];
  int64_t n = job->seq_lens[s];

  int any = 0;
  for (int64_t t = t0; t < t1 && !any; ++t)
    for (int h = g * group; h < (g + 1) * group; ++h)
      if (row_wanted(job, t, h)) any = 1;
  if (!any) return;

  const int32_t* table = job->block_tables + (int64_t)s * job->max_blocks;
  double* K = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * (size_t)P->dk);
  double* V = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * (size_t)P->dv);
  double* sc = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  double* qrow = (double*)malloc(sizeof(double) * (size_t)P->dk);
  double* orow = (double*)malloc(sizeof(double) * (size_t)P->dv);
  gather_head(P->k, P->dtype, P->k_scale, P->block_size, P->num_kv_heads, P->dk, table, n, g, K);
  gather_head(P->v, P->dtype, P->v_scale, P->block_size, P->num_kv_heads, P->dv, table, n, g, V);

  for (int64_t t = t0; t < t1; ++t) {
    int64_t start, end;
    visible_range(job, t, n, &start, &end);
    for (int h = g * group; h < (g + 1) * group; ++h) {
      if (!row_wanted(job, t, h)) continue;
      for (int d = 0; d < P->dk; ++d)
        qrow[d] = load_elem(job->q, job->q_dtype, (t * job->num_heads + h) * P->dk + d);
      /* ALiBi: slope of head h, positions counted from the row's last visible one */
      const double slope = job->alibi ? job->alibi[h] : 0.0;
      const int64_t ref = end - 1;
      if (job->partition_size <= 0) {
        double m, l;
        const double sink = job->sinks ? job->sinks[h] : -INFINITY;
        attend(qrow, K, V, P->dk, P->dv, start, end, job->scale, sink, slope, ref, sc, orow, &m, &l);
        memcpy(job->out + (t * job->num_heads + h) * P->dv, orow, sizeof(double) * (size_t)P->dv);
        if (job->lse) job->lse[(int64_t)h * job->num_tokens + t] = lse_of(m, l);
      } else {
        /* Split-KV: partition p covers [p * P, (p + 1) * P) of the sequence. */
        int64_t np = (n + job->partition_size - 1) / job->partition_size;
        for (int64_t p = 0; p < np; ++p) {
          int64_t lo = p * job->partition_size, hi = lo + job->partition_size;
          if (hi > n) hi = n;
          if (lo < start) lo = start;
          if (hi > end) hi = end;
          double m, l; /* partition states leave the sink to the reduction */
          attend(qrow, K, V, P->dk, P->dv, lo, hi, job->scale, -INFINITY, slope, ref, sc, orow, &m, &l);
          int64_t idx = ((int64_t)s * job->num_heads + h) * job->max_partitions + p;
          job->max_logits[idx] = m;
          job->exp_sums[idx] = l;
          memcpy(job->tmp_out + idx * P->dv, orow, sizeof(double) * (size_t)P->dv);
        }
      }
    }
  }
  free(orow);
  free(qrow);
  free(sc);
  free(V);
  free(K);
}

/* Synchronous checks shared by every attention entry point.  Shape errors first,
 * then the content of the tables. */
static int check_job(const struct attn_job* job) {
  const struct pool_desc* P = &job->pool;
  if (elem_bytes(P->dtype) == 0 || elem_bytes(job->q_dtype) == 0) return ORC_EUNSUPPORTED;
  if (!isfinite(P->k_scale) || !(P->k_scale > 0.0) || !isfinite(P->v_scale) || !(P->v_scale > 0.0))
    return ORC_EINVAL;
  if (P->num_kv_heads < 1 || job->num_heads < 1 || P->dk < 1 || P->dv < 1) return ORC_ESHAPE;
  if (job->num_heads % P->num_kv_heads != 0) return ORC_ESHAPE;
  if (P->block_size < 1 || P->num_blocks < 1 || job->num_seqs < 0 || job->max_blocks < 0)
    return ORC_EINVAL;
  if (job->query_start_loc[0] != 0) return ORC_EINVAL;
  for (int s = 0; s < job->num_seqs; ++s)
    if (job->query_start_loc[s + 1] < job->query_start_loc[s]) return ORC_EINVAL;
  if (job->query_start_loc[job->num_seqs] != job->num_tokens) return ORC_EINVAL;
  if (job->causal && job->num_tokens > 0 && job->positions == NULL) return ORC_EINVAL;
  for (int s = 0; s < job->num_seqs; ++s) {
    int64_t n = job->seq_lens[s];
    if (n < 0) return ORC_EINVAL;
    int64_t need = (n + P->block_size - 1) / P->block_size;
    if (need > job->max_blocks) return ORC_EINVAL;
    const int32_t* table = job->block_tables + (int64_t)s * job->max_blocks;
    for (int64_t i = 0; i < need; ++i)
      if (table[i] < 0 || table[i] >= P->num_blocks) return ORC_EINVAL;
    if (job->causal)
      for (int64_t t = job->query_start_loc[s]; t < job->query_start_loc[s + 1]; ++t)
        if (job->positions[t] < 0 || job->positions[t] >= n) return ORC_EINVAL;
  }
  return ORC_OK;
}

/* Varlen: any mix of prefill chunks and single decode tokens, packed by
 * query_start_loc.  out is [T, H, dv]; lse is [H, T] (nullable).  row_mask [T * H]
 * selects rows to compute (nullable = all); rows not selected are left untouched. */
int orc_varlen(const void* k_pool, const void* v_pool, int kv_dtype, int64_t num_blocks,
               int block_size, int num_kv_heads, int dk, int dv, const void* q, int q_dtype,
               int num_heads, int64_t num_tokens, const int32_t* query_start_loc, int num_seqs,
               const int32_t* seq_lens, const int32_t* positions, const int32_t* block_tables,
               int max_blocks, double scale, int causal, int sliding_window,
               const uint8_t* row_mask, double* out, double* lse, const double* sinks,
               const double* alibi_slopes, double k_scale, double v_scale, int num_threads) {
  struct attn_job job;
  memset(&job, 0, sizeof job);
  job.pool.k = k_pool;
  job.pool.v = v_pool;
  job.pool.dtype = kv_dtype;
  job.pool.k_scale = k_scale;
  job.pool.v_scale = v_scale;
  job.pool.num_blocks = num_blocks;
  job.pool.block_size = block_size;
  job.pool.num_kv_heads = num_kv_heads;
  job.pool.dk = dk;
  job.pool.dv = dv;
  job.q = q;
  job.q_dtype = q_dtype;
  job.num_heads = num_heads;
  job.num_tokens = num_tokens;
  job.query_start_loc = query_start_loc;
  job.num_seqs = num_seqs;
  job.seq_lens = seq_lens;
  job.positions = positions;
  job.block_tables = block_tables;
  job.max_blocks = max_blocks;
  job.scale = scale;
  job.causal = causal;
  job.sliding_window = sliding_window;
  job.row_mask = row_mask;
  job.sinks = sinks;
  job.alibi = alibi_slopes;
  job.out = out;
  job.lse = lse;
  int st = check_job(&job);
  if (st != ORC_OK) return st;
  parallel_for((int64_t)num_seqs * num_kv_heads, num_threads, attn_task, &job);
  return ORC_OK;
}

/* Decode: one query per sequence at position n - 1, causal, optional window.
 * A context length below 1 is invalid.  q and out are [S, H, dim]; lse [H, S].
 * With partition_size > 0 the per-partition states are written instead of out:
 * max_logits / exp_sums [S, H, max_partitions] and tmp_out [S, H, max_partitions,
 * dv] hold, for each partition p < ceil(n / partition_size), the maximum score, the
 * sum of exp(score - max) and the normalised partial output over the partition's
 * visible positions; an empty partition holds (-inf, 0, 0).  Entries at
 * p >= ceil(n / partition_size) are left untouched.                                */
int orc_decode(const void* k_pool, const void* v_pool, int kv_dtype, int64_t num_blocks,
               int block_size, int num_kv_heads, int dk, int dv, const void* q, int q_dtype,
               int num_heads, const int32_t* block_tables, int max_blocks, const int32_t* seq_lens,
               int num_seqs, double scale, int sliding_window, int partition_size,
               int max_partitions, double* out, double* lse, double* max_logits,
               double* exp_sums, double* tmp_out, const double* sinks, const double* alibi_slopes,
               double k_scale, double v_scale, int num_threads) {
  if (num_seqs < 0) return ORC_EINVAL;
  for (int s = 0; s < num_seqs; ++s)
    if (seq_lens[s] < 1) return ORC_EINVAL;
  if (partition_size > 0) {
    if (partition_size % block_size != 0) return ORC_EINVAL;
    for (int s = 0; s < num_seqs; ++s)
      if ((seq_lens[s] + (int64_t)partition_size - 1) / partition_size > max_partitions)
        return ORC_EINVAL;
  } else if (partition_size < 0) {
    return ORC_EINVAL;
  }
  int32_t* qsl = (int32_t*)malloc(sizeof(int32_t) * (size_t)(num_seqs + 1));
  int32_t* pos = (int32_t*)malloc(sizeof(int32_t) * (size_t)(num_seqs > 0 ? num_seqs : 1));
  for (int s = 0; s <= num_seqs; ++s) qsl[s] = s;
  for (int s = 0; s < num_seqs; ++s) pos[s] = seq_lens[s] - 1;

  struct attn_job job;
  memset(&job, 0, sizeof job);
  job.pool.k = k_pool;
  job.pool.v = v_pool;
  job.pool.dtype = kv_dtype;
  job.pool.k_scale = k_scale;
  job.pool.v_scale = v_scale;
  job.pool.num_blocks = num_blocks;
  job.pool.block_size = block_size;
  job.pool.num_kv_heads = num_kv_heads;
  job.pool.dk = dk;
  job.pool.dv = dv;
  job.q = q;
  job.q_dtype = q_dtype;
  job.num_heads = num_heads;
  job.num_tokens = num_seqs;
  job.query_start_loc = qsl;
  job.num_seqs = num_seqs;
  job.seq_lens = seq_lens;
  job.positions = pos;
  job.block_tables = block_tables;
  job.max_blocks = max_blocks;
  job.scale = scale;
  job.causal = 1;
  job.sliding_window = sliding_window;
  job.out = out;
  job.lse = lse;
  job.partition_size = partition_size;
  job.max_partitions = max_partitions;
  job.max_logits = max_logits;
  job.exp_sums = exp_sums;
  job.tmp_out = tmp_out;
  job.sinks = sinks;
  job.alibi = alibi_slopes;
  int st = check_job(&job);
  if (st == ORC_OK) parallel_for((int64_t)num_seqs * num_kv_heads, num_threads, attn_task, &job);
  free(pos);
  free(qsl);
  return st;
}

/* Phase-2 reduction of decode partitions, for each (s, h) over p < ceil(n_s / P):
 * M = max_p m_p, w_p = l_p * exp(m_p - M), out = sum_p w_p o_p / sum_p w_p.
 * The o_p are the normalised partition outputs written by orc_decode.  A sink
 * logit z_h (sinks nullable) joins once here, as a partition of weight exp(z_h - M)
 * and zero output, with M taken over the z_h too.                               */
int orc_reduce_partitions(const double* max_logits, const double* exp_sums, const double* tmp_out,
                          const int32_t* seq_lens, int num_seqs, int num_heads, int partition_size,
                          int max_partitions, int dv, const double* sinks, double* out) {
  if (partition_size < 1) return ORC_EINVAL;
  for (int s = 0; s < num_seqs; ++s) {
    int64_t np = ((int64_t)seq_lens[s] + partition_size - 1) / partition_size;
    if (np > max_partitions) return ORC_EINVAL;
    for (int h = 0; h < num_heads; ++h) {
      int64_t base = ((int64_t)s * num_heads + h) * max_partitions;
      double* o = out + ((int64_t)s * num_heads + h) * dv;
      const double sink = sinks ? sinks[h] : -INFINITY;
      double M = sink;
      for (int64_t p = 0; p < np; ++p)
        if (max_logits[base + p] > M) M = max_logits[base + p];
      for (int d = 0; d < dv; ++d) o[d] = 0.0;
      if (M == -INFINITY) continue;
      double total = sink == -INFINITY ? 0.0 : exp(sink - M);
      for (int64_t p = 0; p < np; ++p) {
        if (exp_sums[base + p] == 0.0) continue;
        double w = exp_sums[base + p] * exp(max_logits[base + p] - M);
        total += w;
        for (int d = 0; d < dv; ++d) o[d] += w * tmp_out[(base + p) * dv + d];
      }
      for (int d = 0; d < dv; ++d) o[d] /= total;
    }
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------------- */
/* Merge of two attention states                                               */
/* ------------------------------------------------------------------------- */

/* Two attention states over disjoint key sets combine into the state over their
 * union ("cpu_mla_prefill.cpp", MergeAttnStates).  By definition a state's lse is
 * the log of its softmax mass, so the union's lse is log(e^a + e^b) for the two lse
 * a and b, and each state's output enters with the share of the mass it holds,
 * e^(a - lse) and e^(b - lse).  Edge rules of that section, as read here: an lse of
 * +inf (which attention never produces) counts as an empty state, -inf; when both
 * states are empty the row keeps the prefix output and its lse is -inf.  Tokens at or
 * past prefill_tokens_with_context (when it is >= 0) take the suffix state unchanged.
 * prefix/suffix outputs are [T, H, D] in `dtype`; every lse is binary32 [H, T].    */
static double as_state_lse(float x) { return isinf(x) ? -INFINITY : (double)x; }

/* log(e^a + e^b) for a, b not both -inf, without overflow: the larger term is
 * factored out, leaving log1p of the smaller one's ratio to it. */
static double log_add_exp(double a, double b) {
  double big = a > b ? a : b, small = a > b ? b : a;
  return big + log1p(exp(small - big));
}

int orc_merge_states(const void* prefix_out, const float* prefix_lse, const void* suffix_out,
                     const float* suffix_lse, int dtype, int64_t num_tokens, int num_heads,
                     int head_dim, int64_t prefill_tokens_with_context, double* out,
                     double* out_lse) {
  if (elem_bytes(dtype) == 0 || dtype == ORC_FP8_E4M3) return ORC_EUNSUPPORTED;
  if (num_tokens < 0 || num_heads < 1 || head_dim < 1) return ORC_EINVAL;
  for (int64_t t = 0; t < num_tokens; ++t) {
    int suffix_only = prefill_tokens_with_context >= 0 && t >= prefill_tokens_with_context;
    for (int h = 0; h < num_heads; ++h) {
      int64_t row = (t * num_heads + h) * head_dim;
      int64_t li = (int64_t)h * num_tokens + t;
      double a = as_state_lse(prefix_lse[li]), b = as_state_lse(suffix_lse[li]);
      double merged;
      if (suffix_only) { /* the suffix as it is, lse included */
        for (int d = 0; d < head_dim; ++d) out[row + d] = load_elem(suffix_out, dtype, row + d);
        merged = (double)suffix_lse[li];
      } else if (a == -INFINITY && b == -INFINITY) { /* both empty */
        for (int d = 0; d < head_dim; ++d) out[row + d] = load_elem(prefix_out, dtype, row + d);
        merged = -INFINITY;
      } else {
        merged = log_add_exp(a, b);
        double wa = exp(a - merged), wb = exp(b - merged);
        for (int d = 0; d < head_dim; ++d)
          out[row + d] = wa * load_elem(prefix_out, dtype, row + d) + wb * load_elem(suffix_out, dtype, row + d);
      }
      if (out_lse) out_lse[li] = merged;
    }
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------------- */
/* Element encoding (round to nearest, ties to even)                          */
/* ------------------------------------------------------------------------- */

/* binary64 -> binary16.  Magnitudes from 65520 (half an ulp above 65504) round to
 * infinity; below 2^-14 the result is a multiple of 2^-24 (subnormal or zero). */
static uint16_t double_to_half(double x) {
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  double a = fabs(x);
  if (isnan(x)) return (uint16_t)(sign | 0x7e00);
  if (a >= 65520.0) return (uint16_t)(sign | 0x7c00);
  if (a < ldexp(1.0, -14)) return (uint16_t)(sign | (uint16_t)nearbyint(ldexp(a, 24)));
  int e;
  double m = frexp(a, &e);         /* a = m * 2^e, m in [0.5, 1) */
  double r = nearbyint(ldexp(m, 11)); /* the 11 significant bits, in [1024, 2048] */
  int biased = e + 14;             /* a = (r / 1024) * 2^(biased - 15) */
  if (r == 2048.0) {
    r = 1024.0;
    biased += 1;
  }
  if (biased >= 31) return (uint16_t)(sign | 0x7c00);
  return (uint16_t)(sign | (biased << 10) | ((int)r - 1024));
}

/* binary64 holding a binary32 value exactly -> bfloat16 (the high half of the
 * binary32 word, rounded on the low half).  NaN stays a quiet NaN. */
static uint16_t double_to_bf16(double x) {
  float f = (float)x;
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  if (isnan(f)) return (uint16_t)((u >> 16) | 0x0040);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* The types results are stored in (an fp8 cache is only ever read here). */
static int encodable(int dtype) { return dtype == ORC_F32 || dtype == ORC_F16 || dtype == ORC_BF16; }

static void store_elem(void* base, int dtype, int64_t i, double x) {
  if (dtype == ORC_F32)
    ((float*)base)[i] = (float)x;
  else if (dtype == ORC_F16)
    ((uint16_t*)base)[i] = double_to_half(x);
  else
    ((uint16_t*)base)[i] = double_to_bf16(x);
}

/* Encode n binary64 values (each a binary32 value) to storage (exposed so the
 * encoders can be pinned). */
int orc_encode_elems(const double* src, int dtype, int64_t n, void* out) {
  if (!encodable(dtype)) return ORC_EUNSUPPORTED;
  for (int64_t i = 0; i < n; ++i) store_elem(out, dtype, i, src[i]);
  return ORC_OK;
}

/* ------------------------------------------------------------------------- */
/* Gather of a paged latent cache into contiguous rows                         */
/* ------------------------------------------------------------------------- */

/* "cpu_mla_prefill.cpp", GatherMlaCache.  Output row t belongs to sequence
 * b = token_to_seq[t]; it is skipped (left untouched) when t >= cu_seq_lens[b + 1].
 * Otherwise its position in the sequence is t - cu_seq_lens[b], plus seq_starts[b]
 * when seq_starts is given, and it receives the cache row at slot position % b of
 * block block_table[b][position / block_size], converted to the output dtype.  The
 * cache row of (block, slot) starts at element block * src_block_stride + slot *
 * src_slot_stride; output row t at element t * dst_row_stride.  Every row that is
 * copied is checked before anything is written: b in [0, num_seqs), a position >= 0,
 * its block index below max_blocks and the block id in [0, num_blocks). */
int orc_gather_cache(const void* src, int src_dtype, int64_t num_blocks, int block_size, int head_dim,
                     int64_t src_block_stride, int64_t src_slot_stride, void* dst, int dst_dtype,
                     int64_t dst_row_stride, const int32_t* block_table, int max_blocks,
                     const int32_t* cu_seq_lens, const int32_t* token_to_seq, const int32_t* seq_starts,
                     int num_seqs, int64_t num_tokens) {
  if (!encodable(src_dtype) || !encodable(dst_dtype)) return ORC_EUNSUPPORTED;
  if (num_blocks < 1 || block_size < 1 || head_dim < 1 || num_seqs < 0 || num_tokens < 0 || max_blocks < 1)
    return ORC_EINVAL;
  for (int pass = 0; pass < 2; ++pass) { /* pass 0 checks, pass 1 copies */
    for (int64_t t = 0; t < num_tokens; ++t) {
      int64_t b = token_to_seq[t];
      if (b < 0 || b >= num_seqs) return ORC_EINVAL;
      if (t >= cu_seq_lens[b + 1]) continue;
      int64_t pos = t - cu_seq_lens[b] + (seq_starts ? seq_starts[b] : 0);
      if (pos < 0) return ORC_EINVAL;
      int64_t idx = pos / block_size, slot = pos % block_size;
      if (idx >= max_blocks) return ORC_EINVAL;
      int64_t block = block_table[b * max_blocks + idx];
      if (block < 0 || block >= num_blocks) return ORC_EINVAL;
      if (pass == 0) continue;
      int64_t from = block * src_block_stride + slot * src_slot_stride, to = t * dst_row_stride;
      for (int d = 0; d < head_dim; ++d) store_elem(dst, dst_dtype, to + d, load_elem(src, src_dtype, from + d));
    }
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------------- */
/* KV write through the slot mapping                                           */
/* ------------------------------------------------------------------------- */

/* Token t's K row [num_kv_heads * dk] and V row [num_kv_heads * dv] go to slot
 * slot_mapping[t], i.e. block slot / block_size at offset slot % block_size, which in
 * the [blocks, block_size, heads, dim] layout is row `slot` of the pool.  Every slot
 * is checked against [0, num_blocks * block_size) before anything is written; rows
 * are then copied byte for byte in token order, so a repeated slot keeps the last. */
int orc_write_kv(void* k_pool, void* v_pool, int dtype, int64_t num_blocks, int block_size,
                 int num_kv_heads, int dk, int dv, const void* k_new, const void* v_new,
                 const int32_t* slot_mapping, int64_t num_tokens) {
  int eb = elem_bytes(dtype);
  if (eb == 0) return ORC_EUNSUPPORTED;
  if (block_size < 1 || num_blocks < 1 || num_kv_heads < 1 || dk < 1 || dv < 1 || num_tokens < 0)
    return ORC_EINVAL;
  int64_t num_slots = num_blocks * block_size;
  for (int64_t t = 0; t < num_tokens; ++t)
    if (slot_mapping[t] < 0 || slot_mapping[t] >= num_slots) return ORC_EINVAL;
  size_t krow = (size_t)num_kv_heads * (size_t)dk * (size_t)eb;
  size_t vrow = (size_t)num_kv_heads * (size_t)dv * (size_t)eb;
  for (int64_t t = 0; t < num_tokens; ++t) {
    int64_t block_id = slot_mapping[t] / block_size;
    int64_t offset = slot_mapping[t] % block_size;
    int64_t row = block_id * block_size + offset;
    memcpy((char*)k_pool + (size_t)row * krow, (const char*)k_new + (size_t)t * krow, krow);
    memcpy((char*)v_pool + (size_t)row * vrow, (const char*)v_new + (size_t)t * vrow, vrow);
  }
  return ORC_OK;
}
