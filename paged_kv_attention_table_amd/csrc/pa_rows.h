// Paged attention for one query row per workgroup: the decode kernel, and the
// per-token kernel pa_varlen uses for rows that the tiled prefill kernel does not
// take.
//
// Method ("Paged attention for decode in C", sections 2.1-2.2; TensorSharp
// "ManagedPagedAttention.cs", Forward): the query of row r (a decode sequence at
// position n - 1, or a varlen token at its position) attends over its visible
// positions [start, end), read in position order through the sequence's block table,
// with an online softmax.  With a partition size the workgroup covers one partition
// of the context and stores its (max, exp-sum, normalised output) state, to be
// combined by log-sum-exp weights ("paged_attention_v2_pytorch.py", phases 1-2).
//
// Mapping onto gfx950.  Workgroup = (row, kv head g, partition), 4 waves.  The
// visible range is cut into 16-position tiles aligned to absolute positions, and
// the waves take tiles round-robin.  For one tile a wave:
//   * loads K: lane l fetches position 16k + l%16, 16-byte chunks 4u + l/16 of
//     the row, so every chunk lands in the register layout of a 16x16 MFMA A
//     operand; the q heads of the group (up to 16) form the B operand, preloaded
//     once.  One MFMA chain gives S^T[position][head] for the tile.
//   * loads V: lane l fetches positions 16k + 4(l/16) + i (i < 4), elements
//     [l%16 * DV/16, +DV/16), i.e. four fully coalesced row segments.
//   * updates per head the running max m (log2 units) and the lane's partial
//     exp-sum; probabilities and rescale factors go through a per-wave LDS tile so
//     that every lane can accumulate its V segment for all heads of the group.
// Positions outside [lo, hi) are neither loaded nor counted: their K and V
// registers are zero and their scores are set to -inf, so garbage in unwritten
// slots can never reach an output.  At the end the four lane groups and then the
// four waves are merged with the same max-rescaled sums.
#pragma once

#include "pa_common.h"
#include "pa_internal.h"

namespace pa {

constexpr int kRowsWaves = 4;

template <typename T, int DK, int DV, int GMAX>
__global__ __launch_bounds__(256) void attn_rows_kernel(const RowsArgs a) {
  constexpr int EB = T::bytes;
  constexpr int CE = 16 / EB;                // elements per 16-byte chunk
  constexpr int KCH = DK / (4 * CE);         // K chunks per lane
  constexpr int KW = KCH * 4;                // K words per lane
  constexpr int VE = DV / 16;                // V elements per lane per position
  constexpr int VW = VE * EB / 4;            // V words per lane per position
  constexpr int NW = kRowsWaves;
  static_assert(KCH >= 1 && DK % (4 * CE) == 0, "head dim");
  static_assert(VW >= 1 && (VE * EB) % 4 == 0, "value dim");

  __shared__ float p_lds[NW][16][16];
  __shared__ float alpha_lds[NW][16];
  __shared__ float red_m[NW][16];
  __shared__ float red_l[NW][16];
  __shared__ float red_acc[NW][GMAX][DV];

  if (status_failed(a.status)) return;

  const int row = blockIdx.x;
  const int g = blockIdx.y;
  const int part = blockIdx.z;
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int c = lane >> 4;  // lane group
  const int r16 = lane & 15;

  // --- which sequence, which position --------------------------------------------
  int s, pos;
  int64_t q_row = row;
  const int b = a.block_size;
  if (a.query_start_loc == nullptr) {
    s = row;
  } else if (a.single_token_seqs) {
    s = row;  // one workgroup per sequence; only sequences with exactly one token
    const int t0 = a.query_start_loc[s];
    if (a.query_start_loc[s + 1] - t0 != 1) return;
    q_row = t0;
  } else {
    int lo_s = 0, hi_s = a.num_seqs - 1;  // last s with query_start_loc[s] <= row
    while (lo_s < hi_s) {
      int mid = (lo_s + hi_s + 1) >> 1;
      if (a.query_start_loc[mid] <= row) lo_s = mid; else hi_s = mid - 1;
    }
    s = lo_s;
    // sequences of one token run split, in a launch of their own
    if (a.skip_single_token_seqs && a.query_start_loc[s + 1] - a.query_start_loc[s] == 1) return;
  }
  int n = a.seq_lens[s];
  const int cap = a.max_blocks * b;
  n = n < 0 ? 0 : (n > cap ? cap : n);
  int end;
  if (a.query_start_loc == nullptr) {
    pos = n - 1;
    end = n;
  } else if (a.causal) {
    pos = a.positions[q_row];
    pos = pos < 0 ? 0 : (pos >= n ? n - 1 : pos);
    end = pos + 1;
  } else {
    end = n;
  }
  if (n == 0) end = 0;
  int start = 0;
  if (a.window > 0) start = end - a.window > 0 ? end - a.window : 0;
  int lo = start, hi = end;
  if (a.partition_size > 0) {
    const int p0 = part * a.partition_size;
    if (p0 >= n) return;  // partition past the context: not part of the state
    lo = lo > p0 ? lo : p0;
    hi = hi < p0 + a.partition_size ? hi : p0 + a.partition_size;
  }

  const int32_t* table = a.block_tables + (int64_t)s * a.max_blocks;
  const int hkv = a.num_kv_heads;
  const char* kbase = static_cast<const char*>(a.k_pool);
  const char* vbase = static_cast<const char*>(a.v_pool);
  const bool aligned16 = (b % 16) == 0;

  // --- the group's q heads as the MFMA B operand ---------------------------------
  uint32_t qw[KW];
  if (r16 < a.group) {
    const char* qrow = static_cast<const char*>(a.q) + (q_row * a.num_heads + g * a.group + r16) * (int64_t)(DK * EB);
#pragma unroll
    for (int u = 0; u < KCH; ++u) load_words<16>(qrow + (4 * u + c) * 16, qw + 4 * u);
  } else {
    zero_words<KW * 4>(qw);
  }

  // ALiBi ("paged_attention_v2_pytorch.py", phase 1): head r16's slope in log2 units;
  // position j's score gains slope * (j - (end - 1)).  Positions are counted from
  // pref = hi - 1 (end - 1 unless split), so that a partition far from the query keeps
  // exact scores and exp-sums; its stored maximum gets slope * (pref - end + 1) back.
  const float slope_l = (a.alibi != nullptr && r16 < a.group) ? a.alibi[g * a.group + r16] * kLog2e : 0.f;
  const int pref = hi - 1;
  float m_run = -INFINITY;  // log2 units, for head r16
  float l_run = 0.f;        // this lane group's share of the exp-sum, head r16
  float acc[GMAX][VE];
#pragma unroll
  for (int h = 0; h < GMAX; ++h)
#pragma unroll
    for (int e = 0; e < VE; ++e) acc[h][e] = 0.f;

  if (lo < hi) {
    const int k_first = lo >> 4, k_last = (hi - 1) >> 4;
    for (int k = k_first + wave; k <= k_last; k += NW) {
      const int t0 = k << 4;
      int64_t tile_slot = 0;
      if (aligned16 && t0 < n) tile_slot = slot_of(table, t0, b, a.num_blocks);

      // K: position t0 + r16
      uint32_t kw[KW];
      {
        const int j = t0 + r16;
        if (j >= lo && j < hi) {
          const int64_t slot = aligned16 ? tile_slot + r16 : slot_of(table, j, b, a.num_blocks);
          const char* krow = kbase + (slot * hkv + g) * (int64_t)(DK * EB);
#pragma unroll
          for (int u = 0; u < KCH; ++u) load_words<16>(krow + (4 * u + c) * 16, kw + 4 * u);
        } else {
          zero_words<KW * 4>(kw);
        }
      }
      // V: positions t0 + 4c + i
      uint32_t vw[4][VW];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = t0 + 4 * c + i;
        if (j >= lo && j < hi) {
          const int64_t slot = aligned16 ? tile_slot + 4 * c + i : slot_of(table, j, b, a.num_blocks);
          const char* vrow = vbase + (slot * hkv + g) * (int64_t)(DV * EB);
          load_words<VE * EB>(vrow + r16 * (VE * EB), vw[i]);
        } else {
          zero_words<VE * EB>(vw[i]);
        }
      }

      // S^T[position 4c + i][head r16]
      f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < KW; w += Mfma16<T>::words_per_step) sc = Mfma16<T>::step(kw + w, qw + w, sc);

      float sv[4];
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = t0 + 4 * c + i;
        sv[i] = (j >= lo && j < hi) ? fmaf(slope_l, (float)(j - pref), sc[i] * a.scale_log2) : -INFINITY;
        mx = fmaxf(mx, sv[i]);
      }
      mx = max_over_groups(mx);
      const float m_new = fmaxf(m_run, mx);
      const bool live = m_new != -INFINITY;
      const float alpha = live ? exp2f(m_run - m_new) : 1.f;
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = live ? exp2f(sv[i] - m_new) : 0.f;
        p_lds[wave][4 * c + i][r16] = p;
        psum += p;
      }
      l_run = l_run * alpha + psum;
      m_run = m_new;
      if (lane < 16) alpha_lds[wave][lane] = alpha;
      wave_lds_sync();

#pragma unroll
      for (int h = 0; h < GMAX; ++h) {
        const float al = alpha_lds[wave][h];
#pragma unroll
        for (int e = 0; e < VE; ++e) acc[h][e] *= al;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float pv[GMAX];
#pragma unroll
        for (int h = 0; h < GMAX; ++h) pv[h] = p_lds[wave][4 * c + i][h];
#pragma unroll
        for (int e = 0; e < VE; ++e) {
          const float v = widen<T>(vw[i][(e * EB) / 4], ((e * EB) / 2) & 1);
#pragma unroll
          for (int h = 0; h < GMAX; ++h) acc[h][e] = fmaf(pv[h], v, acc[h][e]);
        }
      }
      wave_lds_sync();
    }
  }

  // --- merge the four lane groups (different positions, same heads) -------------
  l_run = sum_over_groups(l_run);
#pragma unroll
  for (int h = 0; h < GMAX; ++h)
#pragma unroll
    for (int e = 0; e < VE; ++e) {
      acc[h][e] = sum_over_groups(acc[h][e]);
    }
  if (lane < 16) {
    red_m[wave][lane] = m_run;
    red_l[wave][lane] = l_run;
#pragma unroll
    for (int h = 0; h < GMAX; ++h)
#pragma unroll
      for (int e = 0; e < VE; ++e) red_acc[wave][h][lane * VE + e] = acc[h][e];
  }
  __syncthreads();

  // --- merge the waves and write ---------------------------------------------------
  const int G = a.group;
  // merging into a state held by out (float32) and lse: every head's previous lse is
  // read before any is written
  __shared__ float prev_lse[GMAX];
  if (a.merge) {
    if ((int)threadIdx.x < G) prev_lse[threadIdx.x] = a.lse[(int64_t)(g * G + threadIdx.x) * a.num_rows + q_row];
    __syncthreads();
  }
  for (int idx = threadIdx.x; idx < G * DV; idx += blockDim.x) {
    const int h = idx / DV, d = idx - h * DV;
    const int hq = g * G + h;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, red_m[w][h]);
    // an attention sink (unsplit calls): one more position with score z (z log2(e)
    // in these log2 units) and a zero value; split calls leave it to the reduction
    const float zl = (a.sinks != nullptr && a.partition_size == 0) ? a.sinks[hq] * kLog2e : -INFINITY;
    M = fmaxf(M, zl);
    float L = 0.f, O = 0.f;
    if (M != -INFINITY) {
      L = exp2f(zl - M);
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float f = exp2f(red_m[w][h] - M);
        L = fmaf(red_l[w][h], f, L);
        O = fmaf(red_acc[w][h][d], f, O);
      }
    }
    const float o = L > 0.f ? O * (a.v_scale / L) : 0.f;
    if (a.partition_size == 0) {
      const int64_t oi = (q_row * a.num_heads + hq) * (int64_t)DV + d;
      const float lse_new = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
      if (a.merge) {  // this call is the suffix of the merge
        float wp, ws, lse_m;
        bool keep;
        merge_state_weights(prev_lse[h], lse_new, wp, ws, lse_m, keep);
        float* dst = static_cast<float*>(a.out) + oi;
        if (!keep) *dst = *dst * wp + o * ws;
        if (d == 0) a.lse[(int64_t)hq * a.num_rows + q_row] = lse_m;
      } else {
        store_as(a.out, a.out_dtype, oi, o);
        if (a.lse != nullptr && d == 0) a.lse[(int64_t)hq * a.num_rows + q_row] = lse_new;
      }
    } else {
      const int64_t pi = ((int64_t)s * a.num_heads + hq) * a.max_partitions + part;
      a.tmp_out[pi * DV + d] = o;
      if (d == 0) {
        const float off = a.alibi != nullptr ? a.alibi[hq] * kLog2e * (float)(pref - (end - 1)) : 0.f;
        a.max_logits[pi] = L > 0.f ? (M + off) * kLn2 : -INFINITY;
        a.exp_sums[pi] = L;
      }
    }
  }
}

// Launch the instantiation for (T, DK, DV) with the smallest head-group width that
// holds `group`.
template <typename T, int DK, int DV>
hipError_t launch_rows_dims(const RowsArgs& a, dim3 grid, hipStream_t stream) {
  const dim3 block(kRowsWaves * kWave);
  if (a.group <= 1) {
    hipLaunchKernelGGL((attn_rows_kernel<T, DK, DV, 1>), grid, block, 0, stream, a);
  } else if (a.group <= 2) {
    hipLaunchKernelGGL((attn_rows_kernel<T, DK, DV, 2>), grid, block, 0, stream, a);
  } else if (a.group <= 4) {
    hipLaunchKernelGGL((attn_rows_kernel<T, DK, DV, 4>), grid, block, 0, stream, a);
  } else if (a.group <= 8) {
    hipLaunchKernelGGL((attn_rows_kernel<T, DK, DV, 8>), grid, block, 0, stream, a);
  } else if constexpr (DV <= 128) {
    if (a.group <= 16) {
      hipLaunchKernelGGL((attn_rows_kernel<T, DK, DV, 16>), grid, block, 0, stream, a);
    } else {
      return hipErrorInvalidValue;
    }
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_rows_typed(const RowsArgs& a, int dk, int dv, dim3 grid, hipStream_t stream) {
  if (dk == 32 && dv == 32) return launch_rows_dims<T, 32, 32>(a, grid, stream);
  if (dk == 64 && dv == 64) return launch_rows_dims<T, 64, 64>(a, grid, stream);
  if (dk == 128 && dv == 128) return launch_rows_dims<T, 128, 128>(a, grid, stream);
  if (dk == 256 && dv == 256) return launch_rows_dims<T, 256, 256>(a, grid, stream);
  if (dk == 192 && dv == 128) return launch_rows_dims<T, 192, 128>(a, grid, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
