// Tiled varlen prefill on MFMA: the dense QK^T and PV products of a query tile
// against paged K/V tiles (TensorSharp "ManagedPagedAttention.cs", Forward, for the
// semantics; the online softmax of "Paged attention for decode in C", section 2.2,
// applied per key tile).
//
// Workgroup = (query tile, sequence, kv head g): 128 rows, each a (token, q head)
// pair of the group, 4 waves of 32 rows (two 16-row blocks).  Key tiles of 32
// positions aligned to absolute positions are gathered through the block table into
// LDS (double-buffered, loads for tile t+1 in flight while tile t is computed).
//   S^T[key][row] = K_tile . Q^T  -- 16x16x32 MFMA; A = K rows read from LDS with
//                                    16-byte reads, B = the rows' q, kept in VGPRs.
//   O^T[d][row]  += V^T . P^T     -- 16x16x32 MFMA; A = V^T obtained from the
//                                    row-major V tile with LDS transpose reads
//                                    (ds_read_tr16_b64), B = the probabilities,
//                                    which are already in the B layout because
//                                    S^T's accumulator holds 4 keys x 1 row per lane.
// Each lane therefore owns one row in both products, so the running max, exp-sum
// and the rescale of O stay in registers.  Probabilities enter the PV product as
// f16 for f16 caches; for bf16 caches they are split into bf16 high and low parts
// (two MFMAs) so that the rounding of P stays far below the accuracy bound.
// Keys outside a row's visible range get score -inf; K/V slots past the sequence
// are stored as zeros in LDS, so unwritten pool slots never reach the product.
#pragma once

#include "pa_common.h"
#include "pa_internal.h"

namespace pa {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

struct PrefillArgs {
  const void* k_pool;
  const void* v_pool;
  int64_t num_blocks;
  int block_size;
  int num_kv_heads;
  const void* q;
  void* out;
  int out_dtype;
  float* lse;
  const int32_t* block_tables;
  int max_blocks;
  const int32_t* seq_lens;
  const int32_t* query_start_loc;
  const int32_t* positions;
  int num_seqs;
  int64_t num_tokens;
  int num_heads;
  int group;
  int tokens_per_tile;  // 128 / group (rounded down)
  int min_q_len;        // sequences with fewer tokens are left to the per-row kernel
  float scale_log2;
  int causal;
  int window;
  const int32_t* status;
};

constexpr int kPrefillRows = 128;
constexpr int kPrefillKeys = 32;

template <typename T>
__device__ __forceinline__ f32x4 mfma_16x16x32(u32x4 a, u32x4 b, f32x4 c);
template <>
__device__ __forceinline__ f32x4 mfma_16x16x32<BF16>(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x4 mfma_16x16x32<F16>(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                0, 0);
}

__device__ __forceinline__ uint32_t pack2(uint32_t lo, uint32_t hi) { return lo | (hi << 16); }

template <typename T, int DK, int DV>
__global__ __launch_bounds__(256, 2) void prefill_kernel(const PrefillArgs a) {
  constexpr int KT = kPrefillKeys;
  constexpr int KPAD = 16;  // elements of padding per LDS row (32 bytes)
  constexpr int KROW = DK + KPAD, VROW = DV + KPAD;
  constexpr int KCH = DK / 8, VCH = DV / 8;         // 16-byte chunks per row
  constexpr int KLD = KT * KCH / 256, VLD = KT * VCH / 256;  // chunks per thread
  constexpr int KSTEPS = DK / 32;
  constexpr int ND = DV / 16;
  static_assert(KT * KCH % 256 == 0 && KT * VCH % 256 == 0, "tile split");

  __shared__ __align__(16) uint16_t k_lds[2][KT][KROW];
  __shared__ __align__(16) uint16_t v_lds[2][KT][VROW];
  __shared__ int range_lo, range_hi;

  if (status_failed(a.status)) return;
  const int tile = blockIdx.x, s = blockIdx.y, g = blockIdx.z;
  const int q0 = a.query_start_loc[s];
  const int q_len = a.query_start_loc[s + 1] - q0;
  const int TPT = a.tokens_per_tile;
  if (q_len < a.min_q_len || tile * TPT >= q_len) return;

  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int c = lane >> 4, r16 = lane & 15;
  const int G = a.group;
  int n = a.seq_lens[s];
  const int cap = a.max_blocks * a.block_size;
  n = n < 0 ? 0 : (n > cap ? cap : n);

  if (tid == 0) {
    range_lo = 0x7fffffff;
    range_hi = 0;
  }

  // --- this lane's two rows (one per 16-row block) --------------------------------
  int vis_lo[2], vis_hi[2];
  int64_t row_tok[2];
  int row_head[2];
  bool row_ok[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int r = wave * 32 + rb * 16 + r16;
    const int tl = tile * TPT + r / G;
    row_ok[rb] = (r < TPT * G) && (tl < q_len);
    row_tok[rb] = q0 + (row_ok[rb] ? tl : 0);
    row_head[rb] = g * G + r % G;
    int end = n, start = 0;
    if (a.causal) {
      int pos = a.positions[row_tok[rb]];
      pos = pos < 0 ? 0 : (pos >= n ? n - 1 : pos);
      end = n > 0 ? pos + 1 : 0;
    }
    if (a.window > 0) start = end - a.window > 0 ? end - a.window : 0;
    vis_lo[rb] = row_ok[rb] ? start : 0;
    vis_hi[rb] = row_ok[rb] ? end : 0;
  }
  __syncthreads();
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
    if (vis_lo[rb] < vis_hi[rb]) {
      atomicMin(&range_lo, vis_lo[rb]);
      atomicMax(&range_hi, vis_hi[rb]);
    }

  // --- q rows as the B operand of S^T = K Q^T ---------------------------------------
  u32x4 qb[2][KSTEPS];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + (row_tok[rb] * a.num_heads + row_head[rb]) * DK;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      if (row_ok[rb])
        qb[rb][kk] = *reinterpret_cast<const u32x4*>(qrow + 32 * kk + 8 * c);
      else
        qb[rb][kk] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  __syncthreads();
  const int klo = range_lo, khi = range_hi;

  f32x4 o[ND][2];
#pragma unroll
  for (int nd = 0; nd < ND; ++nd)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) o[nd][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.f, 0.f};

  if (klo < khi) {
    const int32_t* table = a.block_tables + (int64_t)s * a.max_blocks;
    const char* kbase = static_cast<const char*>(a.k_pool);
    const char* vbase = static_cast<const char*>(a.v_pool);
    const int hkv = a.num_kv_heads, b = a.block_size;
    const int t_first = klo & ~(KT - 1);

    u32x4 kreg[KLD], vreg[VLD];
    auto fetch = [&](int t0) {
#pragma unroll
      for (int u = 0; u < KLD; ++u) {
        const int id = tid + 256 * u, key = id / KCH, ch = id % KCH;
        const int j = t0 + key;
        if (j >= klo && j < khi) {
          const int64_t slot = slot_of(table, j, b, a.num_blocks);
          kreg[u] = *reinterpret_cast<const u32x4*>(kbase + ((slot * hkv + g) * DK + ch * 8) * 2);
        } else {
          kreg[u] = u32x4{0u, 0u, 0u, 0u};
        }
      }
#pragma unroll
      for (int u = 0; u < VLD; ++u) {
        const int id = tid + 256 * u, key = id / VCH, ch = id % VCH;
        const int j = t0 + key;
        if (j >= klo && j < khi) {
          const int64_t slot = slot_of(table, j, b, a.num_blocks);
          vreg[u] = *reinterpret_cast<const u32x4*>(vbase + ((slot * hkv + g) * DV + ch * 8) * 2);
        } else {
          vreg[u] = u32x4{0u, 0u, 0u, 0u};
        }
      }
    };
    auto stash = [&](int buf) {
#pragma unroll
      for (int u = 0; u < KLD; ++u) {
        const int id = tid + 256 * u, key = id / KCH, ch = id % KCH;
        *reinterpret_cast<u32x4*>(&k_lds[buf][key][ch * 8]) = kreg[u];
      }
#pragma unroll
      for (int u = 0; u < VLD; ++u) {
        const int id = tid + 256 * u, key = id / VCH, ch = id % VCH;
        *reinterpret_cast<u32x4*>(&v_lds[buf][key][ch * 8]) = vreg[u];
      }
    };

    fetch(t_first);
    stash(0);
    __syncthreads();
    int buf = 0;
    for (int t0 = t_first; t0 < khi; t0 += KT) {
      const bool more = t0 + KT < khi;
      if (more) fetch(t0 + KT);

      // does any row of this wave see a key of the tile?
      bool mine = false;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) mine |= (vis_lo[rb] < t0 + KT) && (vis_hi[rb] > t0) && (vis_lo[rb] < vis_hi[rb]);
      if (__any(mine)) {
        // S^T for two 16-key blocks and both row blocks
        f32x4 sc[2][2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) sc[kb][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < KSTEPS; ++kk) {
            const u32x4 ka = *reinterpret_cast<const u32x4*>(&k_lds[buf][kb * 16 + r16][32 * kk + 8 * c]);
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) sc[kb][rb] = mfma_16x16x32<T>(ka, qb[rb][kk], sc[kb][rb]);
          }
        }
        // online softmax per row; P^T packed as the B operand of the PV product
        u32x4 pb[2], pl[2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          float sv[8];
          float mx = -INFINITY;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int j = t0 + kb * 16 + 4 * c + i;
              const bool vis = j >= vis_lo[rb] && j < vis_hi[rb];
              sv[kb * 4 + i] = vis ? sc[kb][rb][i] * a.scale_log2 : -INFINITY;
              mx = fmaxf(mx, sv[kb * 4 + i]);
            }
          mx = fmaxf(mx, shfl_xor(mx, 16));
          mx = fmaxf(mx, shfl_xor(mx, 32));
          const float m_new = fmaxf(m_run[rb], mx);
          const bool live = m_new != -INFINITY;
          const float alpha = live ? exp2f(m_run[rb] - m_new) : 1.f;
          float p[8], psum = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            p[e] = live ? exp2f(sv[e] - m_new) : 0.f;
            psum += p[e];
          }
          l_run[rb] = l_run[rb] * alpha + psum;
          m_run[rb] = m_new;
#pragma unroll
          for (int nd = 0; nd < ND; ++nd) o[nd][rb] *= alpha;
          if constexpr (T::code == PA_F16) {
            uint32_t w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = pack2(narrow<F16>(p[2 * e]), narrow<F16>(p[2 * e + 1]));
            pb[rb] = u32x4{w[0], w[1], w[2], w[3]};
          } else {
            uint32_t w[4], wl[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t h0 = narrow<BF16>(p[2 * e]), h1 = narrow<BF16>(p[2 * e + 1]);
              const float r0 = p[2 * e] - __uint_as_float(h0 << 16), r1 = p[2 * e + 1] - __uint_as_float(h1 << 16);
              w[e] = pack2(h0, h1);
              wl[e] = pack2(narrow<BF16>(r0), narrow<BF16>(r1));
            }
            pb[rb] = u32x4{w[0], w[1], w[2], w[3]};
            pl[rb] = u32x4{wl[0], wl[1], wl[2], wl[3]};
          }
        }
        // O^T += V^T P^T, V^T via transpose reads of the row-major V tile
        const int tr_r = r16 >> 2, tr_q = r16 & 3;
#pragma unroll
        for (int nd = 0; nd < ND; ++nd) {
          const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4*)(&v_lds[buf][4 * c + tr_r][16 * nd + 4 * tr_q]));
          const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4*)(&v_lds[buf][16 + 4 * c + tr_r][16 * nd + 4 * tr_q]));
          const u32x2 w0 = __builtin_bit_cast(u32x2, v0), w1 = __builtin_bit_cast(u32x2, v1);
          const u32x4 va = u32x4{w0.x, w0.y, w1.x, w1.y};
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) {
            if constexpr (T::code == PA_F16) {
              o[nd][rb] = mfma_16x16x32<F16>(va, pb[rb], o[nd][rb]);
            } else {
              o[nd][rb] = mfma_16x16x32<BF16>(va, pb[rb], o[nd][rb]);
              o[nd][rb] = mfma_16x16x32<BF16>(va, pl[rb], o[nd][rb]);
            }
          }
        }
      }
      if (more) {
        stash(buf ^ 1);
        __syncthreads();
        buf ^= 1;
      }
    }
  }

  // --- finish: sum the lane groups' exp-sums, normalise, write ---------------------
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    float l = l_run[rb];
    l += shfl_xor(l, 16);
    l += shfl_xor(l, 32);
    if (!row_ok[rb]) continue;
    const float inv = l > 0.f ? 1.0f / l : 0.f;
    const int64_t obase = (row_tok[rb] * a.num_heads + row_head[rb]) * (int64_t)DV;
#pragma unroll
    for (int nd = 0; nd < ND; ++nd) {
      const int d0 = 16 * nd + 4 * c;
      const f32x4 v = o[nd][rb] * inv;
      if (a.out_dtype == PA_F32) {
        *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + obase + d0) = v;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) store_as(a.out, a.out_dtype, obase + d0 + i, v[i]);
      }
    }
    if (a.lse != nullptr && c == 0)
      a.lse[(int64_t)row_head[rb] * a.num_tokens + row_tok[rb]] = l > 0.f ? (m_run[rb] + log2f(l)) * kLn2 : -INFINITY;
  }
}

template <typename T>
hipError_t launch_prefill_typed(const PrefillArgs& a, int dk, int dv, dim3 grid, hipStream_t stream) {
  const dim3 block(256);
  if (dk == 128 && dv == 128)
    hipLaunchKernelGGL((prefill_kernel<T, 128, 128>), grid, block, 0, stream, a);
  else if (dk == 192 && dv == 128)
    hipLaunchKernelGGL((prefill_kernel<T, 192, 128>), grid, block, 0, stream, a);
  else if (dk == 64 && dv == 64)
    hipLaunchKernelGGL((prefill_kernel<T, 64, 64>), grid, block, 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pa
