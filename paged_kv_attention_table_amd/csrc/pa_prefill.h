// Tiled varlen prefill on MFMA: the dense QK^T and PV products of a query tile
// against paged K/V tiles (TensorSharp "ManagedPagedAttention.cs", Forward, for the
// semantics; the online softmax of "Paged attention for decode in C", section 2.2,
// applied per key tile).
//
// Workgroup = (query tile, sequence, kv head g): 128 rows, each a (token, q head)
// pair of the group, 4 waves of 32 rows (two 16-row blocks); two workgroups share a
// CU.  Key tiles of 32 positions aligned to absolute positions are gathered through
// the block table: global loads for tile t+2 are issued into one of two register
// sets while tile t is computed from one of two LDS buffers, so each load has two
// tiles of compute to arrive; the 128 rows share every K/V byte brought in.
//   S^T[key][row] = K_tile . Q^T  -- 16x16x32 MFMA; A = K rows read from LDS with
//                                    16-byte reads, B = the rows' q, kept in VGPRs.
//   O^T[d][row]  += V^T . P^T     -- 16x16x32 MFMA; A = V^T obtained from the
//                                    row-major V tile with LDS transpose reads
//                                    (ds_read_tr16_b64), B = the probabilities,
//                                    which are already in the B layout because
//                                    S^T's accumulator holds 4 keys x 1 row per lane.
// Each lane therefore owns one row in both products, so the running max, exp-sum
// and the rescale of O stay in registers.  The PV product runs in f16: f16 caches
// as they are, bf16 caches with V converted to f16 as it is staged in LDS (exact
// over f16's range); a workgroup that meets a bf16 V value beyond that range redoes
// its rows with bf16 V and P split into bf16 high and low parts (two MFMAs), which
// keeps the rounding of P far below the accuracy bound; such a value shows as a
// non-finite output of the f16 pass.
// Keys outside a row's visible range get score -inf; K/V slots past the sequence
// are stored as zeros in LDS, so unwritten pool slots never reach the product.
#pragma once

#include <type_traits>

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
  int block_shift;      // log2(block_size) when it is a power of two, else -1
  int tokens_per_tile;  // kPrefillRows / group (rounded down)
  int tiles_per_seq;    // ceil(max_query_len / tokens_per_tile)
  int min_q_len;        // sequences with fewer tokens are left to the per-row kernel
  float scale_log2;     // softmax scale (with the pool's k_scale folded in) times log2(e)
  float v_scale;        // the pool's v_scale: multiplies every output
  int causal;
  int window;
  const float* sinks;  // [num_heads] sink logits, nullable
  const float* alibi;  // [num_heads] ALiBi slopes, nullable
  int merge;           // out (float32) and lse hold a state: merge this call's into it
  int rank_major;      // workgroup order: query-tile rank first (see prefill_tile)
  // Two key segments per sequence (new_lens non-null): the keys are segment A --
  // positions [0, seq_lens[s]) of block_tables, seen by every query of s -- then
  // segment B -- positions [0, new_lens[s]) of new_tables, seen causally: a query
  // sees B's positions [0, positions[t] + 1) (B's positions are not read when
  // new_lens[s] is 0).  The loop runs over one key space: A at [0, lenA), B from
  // the next multiple of 32 (the gap between them is masked).
  const int32_t* new_lens;
  const int32_t* new_tables;
  int new_max_blocks;
  const int32_t* status;
};

// 128 rows (4 waves x 32) per workgroup: two workgroups fit on a CU (registers and
// LDS), so one's Q load, pipeline fill and epilogue overlap the other's key loop.
constexpr int kPrefillRows = 128;
constexpr int kPrefillThreads = 256;
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

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two floats to packed 16-bit (round to nearest even), one v_cvt_pk each.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, f16x2));
}

// Eight bf16 values to f16 (round to nearest even): exact for |v| in [2^-14, 65504]
// (f16 holds bf16's 8-bit significands there); below 2^-14 the f16 subnormals keep
// an absolute error under 2^-25; beyond 65504 the result is inf.
__device__ __forceinline__ u32x4 bf16x8_to_f16x8(u32x4 x) {
  u32x4 y;
#pragma unroll
  for (int e = 0; e < 4; ++e) y[e] = pack_f16x2(__uint_as_float(x[e] << 16), __uint_as_float(x[e] & 0xffff0000u));
  return y;
}

// Two fp8 (E4M3) values -- bytes 0, 1 of w (HI: bytes 2, 3) -- widened exactly to the
// queries' 16-bit type, packed low element first.
template <typename T, bool HI>
__device__ __forceinline__ uint32_t widen_fp8x2(uint32_t w);
template <>
__device__ __forceinline__ uint32_t widen_fp8x2<BF16, false>(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
}
template <>
__device__ __forceinline__ uint32_t widen_fp8x2<BF16, true>(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
}
template <>
__device__ __forceinline__ uint32_t widen_fp8x2<F16, false>(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
}
template <>
__device__ __forceinline__ uint32_t widen_fp8x2<F16, true>(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true));
}

// Sixteen fp8 (E4M3) values (16 bytes, element e at byte e) widened exactly to T:
// elements 0..7 in lo, 8..15 in hi.
template <typename T>
__device__ __forceinline__ void widen_fp8x16(u32x4 x, u32x4& lo, u32x4& hi) {
  lo = u32x4{widen_fp8x2<T, false>(x[0]), widen_fp8x2<T, true>(x[0]), widen_fp8x2<T, false>(x[1]),
             widen_fp8x2<T, true>(x[1])};
  hi = u32x4{widen_fp8x2<T, false>(x[2]), widen_fp8x2<T, true>(x[2]), widen_fp8x2<T, false>(x[3]),
             widen_fp8x2<T, true>(x[3])};
}

// max(a, b, c) in one instruction (no canonicalising copies of the operands).
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

constexpr float kRescaleLog2 = 8.0f;  // move the reference max only past 2^8
constexpr float kHugeScore = 1.0e30f;

// Per-thread share of one key tile: K goes straight to LDS (KN direct 16-byte
// loads), V through registers (VN 16-byte chunks).
template <int DK, int DV>
struct TileRegs {
  static constexpr int KCH = DK / 8, VCH = DV / 8;  // 16-byte chunks per position
  static constexpr int KN = kPrefillKeys * KCH / kPrefillThreads;
  static constexpr int VN = kPrefillKeys * VCH / kPrefillThreads;
  u32x4 v[VN];
};

// LDS of one prefill workgroup: rings of K and V tiles (V rows padded by 32 bytes),
// the workgroup's key range and the flag of the exact bf16 pass.
template <int DK, int DV>
struct PrefillLds {
  static constexpr int NBUF = 3;   // ring depth, in key tiles
  static constexpr int VPAD = 16;  // elements of padding per V row (32 bytes)
  static constexpr int VROW = DV + VPAD;
  __align__(16) uint16_t k[NBUF][kPrefillKeys][DK];
  __align__(16) uint16_t v[NBUF][kPrefillKeys][VROW];
  int wave_lo[kPrefillThreads / kWave], wave_hi[kPrefillThreads / kWave];  // each wave's key range
  int v_out_of_range;
};

// One prefill workgroup's work: workgroup index L of the tile grid, its LDS in sh (a
// kernel of its own launches it alone; the fused varlen kernel beside decode rows).
// ALIBI: a.alibi is non-null; MERGE: a.merge is set; SEG2: a.new_lens is non-null
// (separate instantiations, so the loop without them keeps its registers and
// instructions).  KV8: the pools hold fp8 (E4M3) and T is the queries' type; K is
// widened to T and V to f16 as they are staged in LDS (both exact), so the products
// run as for 16-bit caches, PV always in f16.
template <typename T, int DK, int DV, bool ALIBI, bool MERGE, bool SEG2 = false, bool KV8 = false>
__device__ __forceinline__ void prefill_tile(const PrefillArgs& a, int L, PrefillLds<DK, DV>& sh) {
  static_assert(!(SEG2 && ALIBI), "two key segments take no ALiBi");
  constexpr int KT = kPrefillKeys;
  constexpr int NTH = kPrefillThreads;
  constexpr int VROW = PrefillLds<DK, DV>::VROW;
  constexpr int NBUF = PrefillLds<DK, DV>::NBUF;  // LDS ring depth, in key tiles
  using Regs = TileRegs<DK, DV>;
  constexpr int KCH = Regs::KCH, VCH = Regs::VCH;
  constexpr int KSTEPS = DK / 32;
  constexpr int ND = DV / 16;
  // Overlap S^T of the next key tile with the softmax of this one (head dims 128
  // and 192; at 64 the single-tile loop keeps three workgroups per CU).
  constexpr bool PIPE = DK >= 128;
  static_assert(!KV8 || (PIPE && DV == 128), "fp8 caches: head dims 128 or 192 for K, 128 for V");
  constexpr int EB = KV8 ? 1 : 2;  // bytes of a cached element

  // K rows sit unpadded, chunk ch of key row r in 16-byte slot ch ^ ksw(r): with
  // 256-byte rows the 16 rows one read touches get 16 distinct slots of the bank
  // space; with 128- or 384-byte rows consecutive rows alternate between its two
  // 128-byte halves, and (r / 2) % 8 spreads eight of them over each half.
  auto& k_lds = sh.k;
  auto& v_lds = sh.v;
  int& v_out_of_range = sh.v_out_of_range;

  if (status_failed(a.status)) return;
  // XCD-aware 1-D grid.  Workgroup L runs on XCD L % 8 (the dispatcher deals
  // workgroups round-robin over the 8 XCDs); all query tiles of one (sequence, kv
  // head) group get the same L % 8, so they share that XCD's L2 for the group's
  // K/V.  Tiles run last-first: under a causal mask the later tiles see more keys,
  // so the longest workgroups start first.  Group-major order (a group's tiles 8
  // workgroups apart, consecutive groups rotating over the XCDs) keeps a group's
  // tiles in flight together; rank-major order (the last tile of every group, then
  // the one before, ...; groups padded to a multiple of 8) starts the heaviest
  // tiles of all groups first, for grids that run in about one round.
  const int TPS = a.tiles_per_seq;
  int grp, tile;
  if (a.rank_major) {
    const int groups8 = (a.num_seqs * a.num_kv_heads + 7) / 8 * 8;
    grp = L % groups8;
    tile = TPS - 1 - L / groups8;
  } else {
    const int xcd = L & 7, q8 = L >> 3;
    grp = (q8 / TPS) * 8 + xcd;
    tile = TPS - 1 - q8 % TPS;
  }
  if (grp >= a.num_seqs * a.num_kv_heads) return;
  const int s = grp / a.num_kv_heads, g = grp % a.num_kv_heads;
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
  // two segments: A = [0, n), B = [base_b, base_b + len_b) of the key space; the gap
  // [n, base_b) is masked (gap_lo == gap_hi: none)
  int len_b = 0, base_b = n;
  if constexpr (SEG2) {
    const int cap_b = a.new_max_blocks * a.block_size;
    len_b = a.new_lens[s];
    len_b = len_b < 0 ? 0 : (len_b > cap_b ? cap_b : len_b);
    base_b = (n + kPrefillKeys - 1) & ~(kPrefillKeys - 1);
  }
  const int gap_lo = n, gap_hi = len_b > 0 ? base_b : n;
  // a sequence with no keys at all (an exhausted context chunk) loads no q: its rows
  // only finish (zero output, or their state merged with an empty one)
  const bool no_keys = n == 0 && len_b == 0;
  // The gap, when there is one, lies inside the one tile that starts at n rounded
  // down to the tile size (B starts at the next multiple of it): on that tile a key
  // j is in the gap when j >= n, and no other tile meets the gap.
  const int gap_tile = gap_lo < gap_hi ? (gap_lo & ~(kPrefillKeys - 1)) : -1;
  auto tile_meets_gap = [&](int t0) {
    if constexpr (SEG2) return t0 == gap_tile;
    return false;
  };
  // key j of a tile for which tile_meets_gap gave gap_t: in the gap
  auto in_gap = [&](bool gap_t, int j) {
    if constexpr (SEG2) return gap_t && j >= gap_lo;
    return false;
  };
  // start of segment B in the key space, or past every key when B is empty
  const int seg_b = len_b > 0 ? base_b : 0x7fffffff;

  if (tid == 0) v_out_of_range = 0;

  // --- this lane's two rows (one per 16-row block) --------------------------------
  int vis_lo[2], vis_hi[2];
  int64_t row_tok[2];
  int row_head[2];
  bool row_ok[2];
  int pos_in[2] = {0, 0};  // the rows' positions, where the visible range needs them
  const bool need_pos = SEG2 ? len_b > 0 : a.causal != 0;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int r = wave * 32 + rb * 16 + r16;
    const int tl = tile * TPT + r / G;
    row_ok[rb] = (r < TPT * G) && (tl < q_len);
    row_tok[rb] = q0 + (row_ok[rb] ? tl : 0);
    row_head[rb] = g * G + r % G;
    if (need_pos) pos_in[rb] = a.positions[row_tok[rb]];
  }

  // --- q rows as the B operand of S^T = K Q^T ---------------------------------------
  // (issued behind the positions loads, so both round trips overlap)
  u32x4 qb[2][KSTEPS];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + (row_tok[rb] * a.num_heads + row_head[rb]) * DK;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      if (row_ok[rb] && !no_keys)
        qb[rb][kk] = *reinterpret_cast<const u32x4*>(qrow + 32 * kk + 8 * c);
      else
        qb[rb][kk] = u32x4{0u, 0u, 0u, 0u};
    }
  }

#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    int end = n, start = 0;
    if constexpr (SEG2) {
      if (len_b > 0) {
        const int pos = pos_in[rb] < 0 ? 0 : (pos_in[rb] >= len_b ? len_b - 1 : pos_in[rb]);
        end = base_b + pos + 1;
      }
    } else if (a.causal) {
      const int pos = pos_in[rb] < 0 ? 0 : (pos_in[rb] >= n ? n - 1 : pos_in[rb]);
      end = n > 0 ? pos + 1 : 0;
    }
    if (a.window > 0) start = end - a.window > 0 ? end - a.window : 0;
    vis_lo[rb] = row_ok[rb] ? start : 0;
    vis_hi[rb] = row_ok[rb] ? end : 0;
  }
  // ALiBi ("paged_attention_v2_pytorch.py", phase 1): each row's slope in raw score
  // units; key j's score gains slope * (j - (end - 1)), end = vis_hi
  float slope_r[2] = {0.f, 0.f};
  if constexpr (ALIBI) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
      slope_r[rb] = row_ok[rb] ? a.alibi[row_head[rb]] * (kLog2e / a.scale_log2) : 0.f;
  }
  // Wave-uniform bounds of the rows' visible ranges, for the per-tile tests:
  // [w_lo_min, w_hi_max) covers every non-empty range of this wave's rows, and a
  // tile inside [w_lo_max, w_hi_min) is seen whole by every row.
  int w_lo_min = 0x7fffffff, w_hi_max = 0, w_lo_max = 0, w_hi_min = 0x7fffffff;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    if (vis_lo[rb] < vis_hi[rb]) {
      w_lo_min = min(w_lo_min, vis_lo[rb]);
      w_hi_max = max(w_hi_max, vis_hi[rb]);
    }
    if (row_ok[rb]) {
      w_lo_max = max(w_lo_max, vis_lo[rb]);
      w_hi_min = min(w_hi_min, vis_hi[rb]);
    }
  }
  w_lo_min = wave_min_i32(w_lo_min);
  w_hi_max = wave_max_i32(w_hi_max);
  w_lo_max = wave_max_i32(w_lo_max);
  w_hi_min = wave_min_i32(w_hi_min);
  // The workgroup's key range [klo, khi): the union of its waves' ranges, one LDS
  // word per wave.  (Not LDS atomics: with a divergent operand the compiler turns
  // each into a 64-step loop on the scalar unit, which the CU's waves share; four of
  // them per wave stalled every workgroup about 8 us.)
  if (lane == 0) {
    sh.wave_lo[wave] = w_lo_min;
    sh.wave_hi[wave] = w_hi_max;
  }
  // take the q loads' wait here, before any untracked K/V load is issued
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) asm volatile("" ::"v"(qb[rb][kk]));
  __syncthreads();
  int klo = sh.wave_lo[0], khi = sh.wave_hi[0];
#pragma unroll
  for (int w = 1; w < NTH / kWave; ++w) {
    klo = min(klo, sh.wave_lo[w]);
    khi = max(khi, sh.wave_hi[w]);
  }
  if (w_hi_min == 0x7fffffff) w_lo_max = 0x7fffffff;  // no row of the wave is real: mask every tile
  const bool wave_live = w_hi_min != 0x7fffffff;  // some row of the wave is real

  f32x4 o[ND][2];
  float m_run[2];
  f32x4 l_acc[2];  // exp-sums, formed by the PV MFMA against a block of ones: 4 equal values

  // Loop-invariant share of this thread in every tile's loads.  A tile's K (V)
  // chunks are dealt so that each wave's 64 lanes fall in one 16-key half of the
  // tile (a half is 16 * KCH chunks, a multiple of 64): the half -- hence the block
  // and the base address -- is wave-uniform, and a lane adds its fixed offset (key
  // within the half, chunk) to it.  K slot u of a thread is 16-byte position
  // tid + NTH u of the tile in LDS (row-major, swizzled); its global chunk is the
  // one the swizzle puts there.
  constexpr int KHALF = 16 * KCH, VHALF = 16 * VCH;
  constexpr int KN = Regs::KN, VN = Regs::VN;
  static_assert(KHALF % kWave == 0 && VHALF % kWave == 0, "tile halves of whole waves");
  static_assert(KN * NTH == 2 * KHALF && VN * NTH == 2 * VHALF, "whole loads per thread");
  const int hkv = a.num_kv_heads, b = a.block_size;
  const uint32_t krow_bytes = (uint32_t)hkv * DK * EB, vrow_bytes = (uint32_t)hkv * DV * EB;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  auto ksw = [](int r) { return DK == 128 ? (r & 15) : ((r >> 1) & 7); };
  uint32_t k_gofs[KN], v_gofs[VN], v_lofs[VN];
  int v_key[VN];
  bool k_hi[KN], v_hi[VN];  // wave-uniform
#pragma unroll
  for (int u = 0; u < KN; ++u) {
    k_hi[u] = wave_u * kWave + NTH * u >= KHALF;
    const int pos = tid + NTH * u, row = pos / KCH, ch = (pos % KCH) ^ ksw(row);
    k_gofs[u] = (uint32_t)(row & 15) * krow_bytes + (uint32_t)(ch * 16);
  }
#pragma unroll
  for (int u = 0; u < VN; ++u) {
    v_hi[u] = wave_u * kWave + NTH * u >= VHALF;
    const int within = (tid + NTH * u) % VHALF, key16 = within / VCH, ch = within % VCH;
    v_key[u] = (v_hi[u] ? 16 : 0) + key16;
    v_gofs[u] = (uint32_t)key16 * vrow_bytes + (uint32_t)(ch * 16);
    v_lofs[u] = (uint32_t)((v_key[u] * VROW + ch * 8) * 2);
  }
  // byte offsets of this lane's K reads in a tile: row kb * 16 + r16 (the kb term is
  // added as a constant), logical chunk 4 kk + c
  uint32_t k_rd[KSTEPS];
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk) k_rd[kk] = (uint32_t)(r16 * DK * 2 + (((4 * kk + c) ^ ksw(r16)) * 16));

  // fp8 caches: K and V both come through registers, one 16-byte load (16 values)
  // at a time, widened to two 16-bit chunks as they are stored to LDS.  K load u of
  // a thread is fp8 chunk tid + NTH u of the tile (DK / 16 per key row; at DK = 192
  // the second load is made by the first 128 threads only); its two halves go to
  // the swizzled slots of 16-bit chunks 2 c8 and 2 c8 + 1 of the row.  The V load
  // is fp8 chunk tid (eight per row): 16 values of key row tid / 8.  As above, the
  // 16-key half of every load is wave-uniform.
  constexpr int KCH8 = DK / 16, VCH8 = DV / 16;
  constexpr int K8N = (KT * KCH8 + NTH - 1) / NTH;  // K loads per thread
  constexpr int K8LAST = KT * KCH8 - NTH * (K8N - 1);  // threads that make the last one
  static_assert(!KV8 || (KT * VCH8 == NTH && K8LAST % kWave == 0 && (16 * KCH8) % kWave == 0), "fp8 tile shares");
  uint32_t k8_gofs[K8N], k8_l0[K8N], k8_l1[K8N], v8_gofs = 0, v8_lofs = 0;
  bool k8_hi[K8N], v8_hi = false;  // wave-uniform
  int v8_key = 0;
  if constexpr (KV8) {
#pragma unroll
    for (int u = 0; u < K8N; ++u) {
      k8_hi[u] = wave_u * kWave + NTH * u >= 16 * KCH8;
      const int pos = tid + NTH * u, row = pos / KCH8, c8 = pos % KCH8;
      k8_gofs[u] = (uint32_t)(row & 15) * krow_bytes + (uint32_t)(c8 * 16);
      k8_l0[u] = (uint32_t)((row * DK + ((2 * c8) ^ ksw(row)) * 8) * 2);
      k8_l1[u] = (uint32_t)((row * DK + ((2 * c8 + 1) ^ ksw(row)) * 8) * 2);
    }
    v8_hi = wave_u * kWave >= 16 * VCH8;
    v8_key = tid / VCH8;
    v8_gofs = (uint32_t)(v8_key & 15) * vrow_bytes + (uint32_t)(tid % VCH8 * 16);
    v8_lofs = (uint32_t)((v8_key * VROW + 16 * (tid % VCH8)) * 2);
  }

  // The whole key loop.  EXACT = false with a bf16 cache stages V as f16 and runs
  // PV on f16 MFMA with P in f16; EXACT = true keeps V in bf16 and splits P into
  // bf16 high and low parts (two MFMAs).  f16 caches always take the f16 path.
  auto run = [&](auto exact_tag) {
    constexpr bool EXACT = decltype(exact_tag)::value;
    constexpr bool F16PV = T::code == PA_F16 || !EXACT || KV8;
#pragma unroll
    for (int nd = 0; nd < ND; ++nd)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) o[nd][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
    // Reference max per row, in raw score units, with its scaled value and the
    // threshold past which it must move: a score s gives p = 2^((s - m) c) with
    // c = scale * log2(e), one fma and one v_exp; m only moves (rescaling O and l)
    // when a score exceeds it by more than 2^8 in p, so p stays below 256, which
    // f16 / bf16 and the fp32 accumulators hold as well, and O / l is unchanged.
    // The finite start makes the first visible tile move it; rows that see nothing
    // keep l = 0, and no -inf - -inf ever occurs.
    const float c2 = a.scale_log2;
    const float thr = kRescaleLog2 / c2;
    float mc[2], m_thr[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      m_run[rb] = -kHugeScore;
      l_acc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
      mc[rb] = m_run[rb] * c2;
      m_thr[rb] = m_run[rb] + thr;
    }
    if (klo >= khi) return;
    const int32_t* table = a.block_tables + (int64_t)s * a.max_blocks;
    const int32_t* table_b = SEG2 ? a.new_tables + (int64_t)s * a.new_max_blocks : table;
    const char* kbase = static_cast<const char*>(a.k_pool) + (int64_t)g * DK * EB;
    const char* vbase = static_cast<const char*>(a.v_pool) + (int64_t)g * DV * EB;
    const int t_first = klo & ~(KT - 1);
    const int num_tiles = (khi - t_first + KT - 1) / KT;
    char* const v_lds_b = reinterpret_cast<char*>(&v_lds[0][0][0]);

    // Pool rows of a tile's two 16-key halves.  The block size is a power of two of
    // at least 16, so each half lies in one block: the block of its first key (the
    // same block for both halves when b >= 32).  The ids are read with scalar loads
    // (counted apart from the vector loads, so the prefetches of earlier tiles are
    // not waited for).  Keys past the visible range are loaded from valid (clamped)
    // blocks and zeroed when stashed.  Pool rows fit 32 bits (the host sends larger
    // pools elsewhere).
    const int max_idx = a.max_blocks - 1, last_block = (int)(a.num_blocks - 1);
    struct Rows {
      uint32_t lo, hi;
    };
    const int max_idx_b = SEG2 ? a.new_max_blocks - 1 : max_idx;
    auto tile_rows = [&](int i) -> Rows {
      int u0 = __builtin_amdgcn_readfirstlane(t_first + i * KT);
      // a tile lies in one segment (B starts at a multiple of the tile size)
      const bool in_b = SEG2 && u0 >= seg_b;
      const int32_t* tab = in_b ? table_b : table;
      if (in_b) u0 -= base_b;
      const int u1 = u0 + 16, mi = in_b ? max_idx_b : max_idx;
      const int i0 = min(u0 >> a.block_shift, mi), i1 = min(u1 >> a.block_shift, mi);
      int b0, b1;
      load_scalar_i32x2(tab, (uint32_t)i0 * 4u, (uint32_t)i1 * 4u, b0, b1);
      b0 = min(max(b0, 0), last_block);
      b1 = min(max(b1, 0), last_block);
      return Rows{((uint32_t)b0 << a.block_shift) | (uint32_t)(u0 & (b - 1)),
                  ((uint32_t)b1 << a.block_shift) | (uint32_t)(u1 & (b - 1))};
    };
    // global -> LDS: the K share of one tile, KN direct loads into LDS buffer `buf`
    // (wave w's load u fills 16-byte positions NTH u + 64 w ..+ 63 of the tile, one
    // per lane); global -> registers: the V share, VN loads.  All are issued
    // untracked, so that the compiler's waits never drain the pipeline; the loop
    // waits for them explicitly.  The half of slot u is the same for every wave
    // except for at most one u.
    auto dma_k = [&](Rows r, int buf) {
      const char* lo_p = kbase + (uint64_t)r.lo * krow_bytes;
      const char* hi_p = kbase + (uint64_t)r.hi * krow_bytes;
      pin_sgpr(lo_p);
      pin_sgpr(hi_p);
      const uint32_t lds0 = lds_addr(&k_lds[buf][0][0]) + (uint32_t)wave_u * kWave * 16;
#pragma unroll
      for (int u = 0; u < KN; ++u) {
        const char* p = NTH * u + NTH <= KHALF ? lo_p : NTH * u >= KHALF ? hi_p : k_hi[u] ? hi_p : lo_p;
        load16_to_lds_untracked(p, k_gofs[u], lds0 + (uint32_t)(NTH * u * 16));
      }
    };
    auto fetch_v = [&](Rows r, Regs& R) {
      const char* lo_p = vbase + (uint64_t)r.lo * vrow_bytes;
      const char* hi_p = vbase + (uint64_t)r.hi * vrow_bytes;
      pin_sgpr(lo_p);
      pin_sgpr(hi_p);
#pragma unroll
      for (int u = 0; u < VN; ++u) {
        const char* p = NTH * u + NTH <= VHALF ? lo_p : NTH * u >= VHALF ? hi_p : v_hi[u] ? hi_p : lo_p;
        R.v[u] = load16_untracked(p, v_gofs[u]);
      }
    };
    // Wait until everything but the last KN loads (one tile's K, issued after the
    // V loads of the same step) has landed, then order the V registers after it.
    auto settle = [&](Regs& R) {
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(KN) : "memory");
#pragma unroll
      for (int u = 0; u < VN; ++u) tie_reg(R.v[u]);
    };
    // registers -> LDS: V of tile iv into buffer vb, zeros for keys outside
    // [klo, khi) on edge tiles.  (K is not cleared: scores of keys outside a row's
    // range are replaced by -inf, whatever the bytes hold.)
    auto stash_v = [&](const Regs& R, int iv, int vb) {
      const int tv = t_first + iv * KT;
      const bool gap_t = tile_meets_gap(tv);
      const bool edge = tv < klo || tv + KT > khi || gap_t;
      const u32x4 zero = {0u, 0u, 0u, 0u};
      auto put = [&](bool masking) {
#pragma unroll
        for (int u = 0; u < VN; ++u) {
          u32x4* dst = reinterpret_cast<u32x4*>(v_lds_b + vb * sizeof(v_lds[0]) + v_lofs[u]);
          u32x4 x = R.v[u];
          if constexpr (T::code == PA_BF16 && !EXACT) x = bf16x8_to_f16x8(x);
          if (masking) {
            const int j = tv + v_key[u];
            if (j < klo || j >= khi || in_gap(gap_t, j)) x = zero;
          }
          *dst = x;
        }
      };
      if (edge) {
        asm volatile("");  // keep the two copies apart: edge tiles only
        put(true);
      } else {
        put(false);
      }
    };
    // fp8 caches: global -> registers (untracked, as above), then widened into LDS.
    struct Regs8 {
      u32x4 k[K8N];
      u32x4 v;
    };
    auto fetch_k8 = [&](Rows r, Regs8& R) {
      const char* lo_p = kbase + (uint64_t)r.lo * krow_bytes;
      const char* hi_p = kbase + (uint64_t)r.hi * krow_bytes;
      pin_sgpr(lo_p);
      pin_sgpr(hi_p);
#pragma unroll
      for (int u = 0; u < K8N; ++u) {
        if (u + 1 < K8N || wave_u * kWave < K8LAST) {
          const char* p =
              NTH * u + NTH <= 16 * KCH8 ? lo_p : NTH * u >= 16 * KCH8 ? hi_p : k8_hi[u] ? hi_p : lo_p;
          R.k[u] = load16_untracked(p, k8_gofs[u]);
        }
      }
    };
    auto fetch_v8 = [&](Rows r, Regs8& R) {
      const char* lo_p = vbase + (uint64_t)r.lo * vrow_bytes;
      const char* hi_p = vbase + (uint64_t)r.hi * vrow_bytes;
      pin_sgpr(lo_p);
      pin_sgpr(hi_p);
      R.v = load16_untracked(v8_hi ? hi_p : lo_p, v8_gofs);
    };
    auto settle8 = [&](Regs8& R) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
      for (int u = 0; u < K8N; ++u) tie_reg(R.k[u]);
      tie_reg(R.v);
    };
    // K of a tile into buffer kb (not cleared, as above)
    auto stash_k8 = [&](const Regs8& R, int kb) {
      char* dst = reinterpret_cast<char*>(&k_lds[kb][0][0]);
#pragma unroll
      for (int u = 0; u < K8N; ++u) {
        if (u + 1 < K8N || wave_u * kWave < K8LAST) {
          u32x4 lo, hi;
          widen_fp8x16<T>(R.k[u], lo, hi);
          *reinterpret_cast<u32x4*>(dst + k8_l0[u]) = lo;
          *reinterpret_cast<u32x4*>(dst + k8_l1[u]) = hi;
        }
      }
    };
    // V of tile iv into buffer vb, as f16; zeros for keys outside [klo, khi)
    auto stash_v8 = [&](const Regs8& R, int iv, int vb) {
      const int tv = t_first + iv * KT;
      u32x4 lo, hi;
      widen_fp8x16<F16>(R.v, lo, hi);
      const int j = tv + v8_key;
      if (j < klo || j >= khi || in_gap(tile_meets_gap(tv), j)) lo = hi = u32x4{0u, 0u, 0u, 0u};
      char* dst = v_lds_b + vb * sizeof(v_lds[0]) + v8_lofs;
      *reinterpret_cast<u32x4*>(dst) = lo;
      *reinterpret_cast<u32x4*>(dst + 16) = hi;
    };
    // S^T of a key tile (from K buffer `buf`) for two 16-key blocks and both row blocks
    auto qk = [&](int buf, f32x4 (&sc)[2][2]) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) sc[kb][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) {
        u32x4 ka[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          ka[kb] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(&k_lds[buf][kb * 16][0]) + k_rd[kk]);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) sc[kb][rb] = mfma_16x16x32<T>(ka[kb], qb[rb][kk], sc[kb][rb]);
      }
    };
    // First half of the softmax of tile i: masking (edge tiles, and tiles no row of
    // this wave sees, which end up all masked), and the move of the reference max.
    auto soft_max = [&](int i, f32x4 (&sc)[2][2]) {
      const int t0 = t_first + i * KT;
      // Tiles inside every row's visible range skip the masking.
      // (the gap between two key segments is masked for every row)
      const bool gap_t = tile_meets_gap(t0);
      const bool masked = !(w_lo_max <= t0 && w_hi_min >= t0 + KT) || gap_t;
      if constexpr (ALIBI) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          const float jb = (float)(t0 + 4 * c - (vis_hi[rb] - 1));  // exact: |j - ref| < 2^24
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii)
              sc[kb][rb][ii] = fmaf(slope_r[rb], jb + (float)(kb * 16 + ii), sc[kb][rb][ii]);
        }
      }
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        if (masked) {
          asm volatile("");  // keep this a branch: edge tiles only
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
              const int j = t0 + kb * 16 + 4 * c + ii;
              if (j < vis_lo[rb] || j >= vis_hi[rb] || in_gap(gap_t, j)) sc[kb][rb][ii] = -INFINITY;
            }
        }
        // this lane's max; the row-wide max is only formed when the reference must move
        const float lm = max3f(max3f(sc[0][rb][0], sc[0][rb][1], sc[0][rb][2]),
                               max3f(sc[0][rb][3], sc[1][rb][0], sc[1][rb][1]),
                               max3f(sc[1][rb][2], sc[1][rb][3], sc[1][rb][3]));
        if (__any(lm > m_thr[rb])) {
          const float m_new = fmaxf(m_run[rb], max_over_groups(lm));
          const float alpha = __builtin_amdgcn_exp2f((m_run[rb] - m_new) * c2);
          l_acc[rb] *= alpha;
#pragma unroll
          for (int nd = 0; nd < ND; ++nd) o[nd][rb] *= alpha;
          m_run[rb] = m_new;
          mc[rb] = m_new * c2;
          m_thr[rb] = m_new + thr;
        }
      }
    };
    // Second half: probabilities, and O^T += V^T P^T from V buffer `buf` (V^T via
    // transpose reads of the row-major V tile), with the exp-sums.
    auto soft_pv = [&](int buf, const f32x4 (&sc)[2][2]) {
      u32x4 pb[2], pl[2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        float p[8];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) p[kb * 4 + ii] = __builtin_amdgcn_exp2f(fmaf(sc[kb][rb][ii], c2, -mc[rb]));
        if constexpr (F16PV) {
          uint32_t w[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = pack_f16x2(p[2 * e], p[2 * e + 1]);
          pb[rb] = u32x4{w[0], w[1], w[2], w[3]};
        } else {
          uint32_t w[4], wl[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t h = pack_bf16x2(p[2 * e], p[2 * e + 1]);
            w[e] = h;
            wl[e] = pack_bf16x2(p[2 * e] - __uint_as_float(h << 16), p[2 * e + 1] - __uint_as_float(h & 0xffff0000u));
          }
          pb[rb] = u32x4{w[0], w[1], w[2], w[3]};
          pl[rb] = u32x4{wl[0], wl[1], wl[2], wl[3]};
        }
      }
      // (pipelined: V reads stay below the P products; hoisted among them they push
      // the loop past 256 VGPRs)
      if constexpr (PIPE) __builtin_amdgcn_sched_barrier(0);
      // (pipelined: the PV products issue at raised wave priority, so that with two
      // waves on a SIMD the one holding MFMA work is served first; +1 %)
      if constexpr (PIPE) __builtin_amdgcn_s_setprio(1);
      const int tr_r = r16 >> 2, tr_q = r16 & 3;
#pragma unroll
      for (int nd = 0; nd < ND; ++nd) {
        const i16x4 v0 =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(&v_lds[buf][4 * c + tr_r][16 * nd + 4 * tr_q]));
        const i16x4 v1 =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(&v_lds[buf][16 + 4 * c + tr_r][16 * nd + 4 * tr_q]));
        const u32x2 w0 = __builtin_bit_cast(u32x2, v0), w1 = __builtin_bit_cast(u32x2, v1);
        const u32x4 va = u32x4{w0.x, w0.y, w1.x, w1.y};
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          if constexpr (F16PV) {
            o[nd][rb] = mfma_16x16x32<F16>(va, pb[rb], o[nd][rb]);
          } else {
            o[nd][rb] = mfma_16x16x32<BF16>(va, pb[rb], o[nd][rb]);
            o[nd][rb] = mfma_16x16x32<BF16>(va, pl[rb], o[nd][rb]);
          }
        }
      }
      // exp-sums: the same product against a V^T block of ones sums each row's
      // probabilities over the tile's 32 keys, across the lanes that hold them --
      // the same rounded values that enter O
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        if constexpr (F16PV) {
          constexpr uint32_t one2 = 0x3C003C00u;  // two f16 ones
          l_acc[rb] = mfma_16x16x32<F16>(u32x4{one2, one2, one2, one2}, pb[rb], l_acc[rb]);
        } else {
          constexpr uint32_t one2 = 0x3F803F80u;  // two bf16 ones
          l_acc[rb] = mfma_16x16x32<BF16>(u32x4{one2, one2, one2, one2}, pb[rb], l_acc[rb]);
          l_acc[rb] = mfma_16x16x32<BF16>(u32x4{one2, one2, one2, one2}, pl[rb], l_acc[rb]);
        }
      }
      if constexpr (PIPE) __builtin_amdgcn_s_setprio(0);
    };

    // Software pipeline over key tiles, in rings of NBUF LDS buffers (tile j in
    // buffer j % NBUF).  Step i loads V(i+1) into registers and K(i+KA) straight
    // into LDS, finishes tile i, and ends by stashing V(i+1) behind one barrier.
    // With PIPE, step i finishes tile i -- its softmax and PV product, from S^T
    // formed in the step before -- while it forms S^T of tile i + 1, so the MFMAs
    // of one overlap the vector work of the other; K then runs KA = 3 tiles ahead
    // (buffer i % NBUF held K(i), last read in step i - 1), else KA = 2 (buffer
    // (i + 2) % NBUF held K(i - 1)).  Loads past the last tile are clamped to it.
    // fp8 caches (always PIPE): step i loads V(i+1) and K(i+2) into registers and
    // stores both, widened, behind its compute: buffer (i+2) % NBUF held K(i-1), last
    // read in step i-2, and V(i-1), last read in step i-1.
    constexpr int KA = PIPE ? 3 : 2;
    const int last = num_tiles - 1;
    Regs RV;
    Regs8 R8;
    Rows rq[NBUF];  // pool rows of tile j in rq[j % NBUF], from its K load on
    f32x4 sc[2][2];
    if constexpr (KV8) {
      Regs8 R1;
      rq[0] = tile_rows(0);
      fetch_k8(rq[0], R8);
      fetch_v8(rq[0], R8);
      rq[1] = tile_rows(min(1, last));
      fetch_k8(rq[1], R1);
      settle8(R8);
#pragma unroll
      for (int u = 0; u < K8N; ++u) tie_reg(R1.k[u]);
      stash_k8(R8, 0);
      stash_v8(R8, 0, 0);
      stash_k8(R1, 1);
      lds_barrier();
      qk(0, sc);  // step 0 writes buffers 1 (V) and 2 (K) only: no second barrier
    } else {
      rq[0] = tile_rows(0);
      fetch_v(rq[0], RV);
#pragma unroll
      for (int j = 0; j < KA; ++j) {
        if (j > 0) rq[j] = tile_rows(min(j, last));
        dma_k(rq[j], j);
      }
      settle(RV);  // V0 and K0 .. K(KA-2) have landed
      stash_v(RV, 0, 0);
      lds_barrier();
      if constexpr (PIPE) {
        qk(0, sc);
        lds_barrier();  // every wave is past K0 before step 0 reloads its buffer
      }
    }
    // one step on tile i in buffer B = i % NBUF; `more`: i + 1 < num_tiles; LIVE: the
    // wave has a real row
    auto step = [&](int i, auto slot_tag, auto more, auto live_tag) {
      constexpr bool LIVE = decltype(live_tag)::value;
      constexpr int B = decltype(slot_tag)::value, B1 = (B + 1) % NBUF, BK = (B + KA) % NBUF;
      constexpr int B2 = (B + 2) % NBUF;
      // the next tiles' loads also issue at raised priority (pipelined), so that they
      // leave early and their latency hides under this step
      if constexpr (PIPE) __builtin_amdgcn_s_setprio(1);
      if constexpr (KV8) {
        if (more) {
          fetch_v8(rq[B1], R8);
          if (i + 2 < num_tiles) {
            rq[B2] = tile_rows(i + 2);
            fetch_k8(rq[B2], R8);
          }
        }
      } else if (more) {
        fetch_v(rq[B1], RV);
        rq[BK] = tile_rows(min(i + KA, last));
        dma_k(rq[BK], BK);
      }
      if constexpr (PIPE) __builtin_amdgcn_s_setprio(0);
      if constexpr (!LIVE) {
        // no real row in this wave: nothing to compute
      } else if constexpr (PIPE) {
        soft_max(i, sc);
        f32x4 sn[2][2];
        if (more) qk(B1, sn);
        soft_pv(B, sc);
        if (more) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) sc[kb][rb] = sn[kb][rb];
        }
      } else {
        const int t0 = t_first + i * KT;
        if (t0 < w_hi_max && t0 + KT > w_lo_min) {  // some row of this wave sees the tile
          qk(B, sc);
          soft_max(i, sc);
          soft_pv(B, sc);
        }
      }
      if constexpr (KV8) {
        if (more) {
          settle8(R8);
          stash_v8(R8, i + 1, B1);
          if (i + 2 < num_tiles) stash_k8(R8, B2);
          lds_barrier();
        }
      } else if (more) {
        settle(RV);
        stash_v(RV, i + 1, B1);
        lds_barrier();
      }
    };
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    // waves with no real row only load, stash and meet the barriers
    auto steps = [&](auto live) {
      int i = 0;
      for (; i + NBUF < num_tiles; i += NBUF) {
        step(i, S0{}, std::true_type{}, live);
        step(i + 1, S1{}, std::true_type{}, live);
        step(i + 2, S2{}, std::true_type{}, live);
      }
      step(i, S0{}, i + 1 < num_tiles, live);
      if (i + 1 < num_tiles) step(i + 1, S1{}, i + 2 < num_tiles, live);
      if (i + 2 < num_tiles) step(i + 2, S2{}, false, live);
    };
    if (wave_live)
      steps(std::true_type{});
    else
      steps(std::false_type{});
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // clamped loads past the last tile
  };
  if constexpr (T::code == PA_BF16 && !KV8) {
    run(std::false_type{});
    // A V value beyond f16's range became inf in the staged tile, which makes every
    // output it reaches inf or NaN (NaN where p = 0): any non-finite output of this
    // workgroup means its rows are done again, exactly, with bf16 V.  (Inputs that
    // are themselves inf or NaN take the exact path too; it gives the same result.)
    float sum = 0.f;
#pragma unroll
    for (int nd = 0; nd < ND; ++nd)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) sum += (o[nd][rb][0] + o[nd][rb][1]) + (o[nd][rb][2] + o[nd][rb][3]);
    if (!__builtin_isfinite(sum)) v_out_of_range = 1;
    __syncthreads();
    if (v_out_of_range) run(std::true_type{});
  } else {
    run(std::false_type{});
  }

  // --- finish: normalise, write ---------------------------------------------------
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    if (!row_ok[rb]) continue;
    // An attention sink ("ManagedPagedAttention.cs", ForwardWithSinks) is one more
    // position with score z and a zero value: in raw score units z / scale, it joins
    // the reference max and the exp-sum here (without one, mx = m_run, fo = 1, fz =
    // 0 and nothing changes).
    const float zr = a.sinks != nullptr ? a.sinks[row_head[rb]] * (kLog2e / a.scale_log2) : -INFINITY;
    const float mx = fmaxf(m_run[rb], zr);
    const float fo = __builtin_amdgcn_exp2f((m_run[rb] - mx) * a.scale_log2);
    const float fz = __builtin_amdgcn_exp2f((zr - mx) * a.scale_log2);
    const float l = fmaf(l_acc[rb][0], fo, fz);
    m_run[rb] = mx;
    const float inv = l > 0.f ? fo * a.v_scale / l : 0.f;
    const int64_t obase = (row_tok[rb] * a.num_heads + row_head[rb]) * (int64_t)DV;
    const int64_t li = (int64_t)row_head[rb] * a.num_tokens + row_tok[rb];
    const float lse_new = l > 0.f ? (m_run[rb] * a.scale_log2 + log2f(l)) * kLn2 : -INFINITY;
    if constexpr (MERGE) {
      // merge into the state held by out (float32) and lse: this call is the suffix.
      // The row's four lanes read its lse before one of them writes it (one wave).
      // An empty suffix (no visible key) leaves out as it is (weights 1 and 0), so
      // its rows touch only lse, which still turns +inf into -inf.
      float wp, ws, lse_m;
      bool keep;
      merge_state_weights(a.lse[li], lse_new, wp, ws, lse_m, keep);
      if (!keep && lse_new != -INFINITY) {
#pragma unroll
        for (int nd = 0; nd < ND; ++nd) {
          float* dst = static_cast<float*>(a.out) + obase + 16 * nd + 4 * c;
          const f32x4 prev = *reinterpret_cast<const f32x4*>(dst);
          *reinterpret_cast<f32x4*>(dst) = prev * wp + (o[nd][rb] * inv) * ws;
        }
      }
      if (c == 0) a.lse[li] = lse_m;
      continue;
    }
#pragma unroll
    for (int nd = 0; nd < ND; ++nd) {
      const int d0 = 16 * nd + 4 * c;
      const f32x4 v = o[nd][rb] * inv;
      if (a.out_dtype == PA_F32) {
        *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + obase + d0) = v;
      } else {
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) store_as(a.out, a.out_dtype, obase + d0 + ii, v[ii]);
      }
    }
    if (a.lse != nullptr && c == 0) a.lse[li] = lse_new;
  }
}

template <typename T, int DK, int DV, bool ALIBI, bool MERGE, bool SEG2 = false, bool KV8 = false>
__global__ __launch_bounds__(kPrefillThreads, 2) void prefill_kernel(const PrefillArgs a) {
  __shared__ PrefillLds<DK, DV> lds;
  prefill_tile<T, DK, DV, ALIBI, MERGE, SEG2, KV8>(a, blockIdx.x, lds);
}

// KV8: fp8 pools (head dims 128 / 128 and 192 / 128 only); T is the queries' type.
template <typename T, bool KV8, bool ALIBI, bool MERGE, bool SEG2 = false>
hipError_t launch_prefill_dims(const PrefillArgs& a, int dk, int dv, dim3 grid, hipStream_t stream) {
  const dim3 block(kPrefillThreads);
  if (dk == 128 && dv == 128)
    hipLaunchKernelGGL((prefill_kernel<T, 128, 128, ALIBI, MERGE, SEG2, KV8>), grid, block, 0, stream, a);
  else if (dk == 192 && dv == 128)
    hipLaunchKernelGGL((prefill_kernel<T, 192, 128, ALIBI, MERGE, SEG2, KV8>), grid, block, 0, stream, a);
  else if constexpr (!KV8) {
    if (dk == 64 && dv == 64)
      hipLaunchKernelGGL((prefill_kernel<T, 64, 64, ALIBI, MERGE, SEG2>), grid, block, 0, stream, a);
    else
      return hipErrorInvalidValue;
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T, bool KV8 = false>
hipError_t launch_prefill_typed(const PrefillArgs& a, int dk, int dv, dim3 grid, hipStream_t stream) {
  if (a.new_lens != nullptr) {  // two key segments (no ALiBi)
    if (a.alibi != nullptr) return hipErrorInvalidValue;
    return a.merge ? launch_prefill_dims<T, KV8, false, true, true>(a, dk, dv, grid, stream)
                   : launch_prefill_dims<T, KV8, false, false, true>(a, dk, dv, grid, stream);
  }
  if (a.merge)
    return a.alibi != nullptr ? launch_prefill_dims<T, KV8, true, true>(a, dk, dv, grid, stream)
                              : launch_prefill_dims<T, KV8, false, true>(a, dk, dv, grid, stream);
  return a.alibi != nullptr ? launch_prefill_dims<T, KV8, true, false>(a, dk, dv, grid, stream)
                            : launch_prefill_dims<T, KV8, false, false>(a, dk, dv, grid, stream);
}

}  // namespace pa
