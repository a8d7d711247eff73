// Paged decode for f16 / bf16 caches, with both products on MFMA.
//
// Method ("Paged attention for decode in C", sections 2.1-2.2; partitions and their
// states as in "paged_attention_v2_pytorch.py", phase 1): one query row per
// workgroup and kv head (all q heads of the group at once), attending over its
// visible positions [lo, hi) -- optionally one partition of them -- with an online
// softmax; the workgroup writes the normalised output, or the partition's (max,
// exp-sum, normalised output) state for the reduce kernel.
//
// Mapping onto gfx950.  Workgroup = (row, kv head g, partition), 4 waves; the
// visible range is cut into 16-position tiles aligned to absolute positions, dealt
// round-robin to the waves.  Per tile a wave
//   * brings K straight from HBM into its LDS tile (global_load_lds_dwordx4, full
//     256-byte row pieces per load, chunks XOR-swizzled) and reads the A operand of
//     a 16x16x32 MFMA from it (position l%16, 16-byte chunks 4u + l/16), against
//     the group's q heads as the B operand: S^T[position][head];
//   * brings V straight from HBM into its own LDS tile (global_load_lds_dwordx4)
//     and takes V^T back with transpose reads (ds_read_tr16_b64) as the A operand
//     of a 16x16x16 MFMA whose B operand is P^T -- already in place, since the
//     S^T accumulator holds 4 positions x 1 head per lane.  P enters as f16 for f16
//     caches and as bf16 high + low parts for bf16 caches;
//   * keeps a reference max per head that moves (rescaling O and l) only when a
//     tile's max exceeds it by more than 2^8.
// Loads are software-pipelined NB tiles ahead (NB LDS buffers per wave, each refilled
// as soon as its tile has been copied into registers), and the block ids of a wave's tiles
// are fetched up to 64 at a time with one vector load and broadcast per tile, so
// no K/V load waits on a table lookup.  Requires a power-of-two block size that is
// a multiple of 16 (a tile then lies inside one block) and head dims of 128.
//
// fp8 (E4M3) pools (F8): a tile's K and V are 2 KB each, brought in by two direct
// loads of 8 positions x 128 bytes apiece, the 16-byte chunk k of position r stored
// at chunk slot k ^ ((r >> 1) & 7).  K comes back as two 16-byte reads per lane
// (position l%16, bytes 32 (l/16) .. +32: the QK reduction runs over head-dim
// elements in that order, and q is read in the same order); V comes back through
// 8-bit transpose reads (ds_read_b64_tr_b8), each giving a lane one head-dim element
// at 4 positions for two d blocks.  Every element is widened exactly to f16 / bf16
// (the queries' type) by the packed hardware conversion and enters the same MFMAs;
// the cache's k_scale is folded into the softmax scale and v_scale into the final
// normalisation, so no per-element scaling is done.
#pragma once

#include "pa_common.h"
#include "pa_internal.h"
#include "pa_prefill.h"

namespace pa {

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

constexpr int kLoadNT = 2;  // cache-policy bits of the direct-to-LDS loads: non-temporal

template <typename T>
__device__ __forceinline__ f32x4 mfma_16x16x16(u32x2 a, u32x2 b, f32x4 c);
template <>
__device__ __forceinline__ f32x4 mfma_16x16x16<BF16>(u32x2 a, u32x2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a), __builtin_bit_cast(i16x4, b), c, 0,
                                                   0, 0);
}
template <>
__device__ __forceinline__ f32x4 mfma_16x16x16<F16>(u32x2 a, u32x2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a), __builtin_bit_cast(f16x4, b), c, 0, 0,
                                               0);
}

// Which sequence and which visible range a row workgroup covers (partition `part`
// of it in split mode), and the row's last visible position `ref` (whole range, the
// origin of ALiBi positions); false: nothing to do.
__device__ __forceinline__ bool decode_row_range(const RowsArgs& a, int row, int part, int& s, int64_t& q_row, int& n,
                                                 int& lo, int& hi, int& ref) {
  q_row = row;
  if (a.query_start_loc == nullptr) {
    s = row;
  } else if (a.single_token_seqs) {
    s = row;
    const int t0 = a.query_start_loc[s];
    if (a.query_start_loc[s + 1] - t0 != 1) return false;
    q_row = t0;
  } else {
    int lo_s = 0, hi_s = a.num_seqs - 1;
    while (lo_s < hi_s) {
      const int mid = (lo_s + hi_s + 1) >> 1;
      if (a.query_start_loc[mid] <= row) lo_s = mid; else hi_s = mid - 1;
    }
    s = lo_s;
    // sequences of one token run split, in a launch of their own
    if (a.skip_single_token_seqs && a.query_start_loc[s + 1] - a.query_start_loc[s] == 1) return false;
  }
  n = a.seq_lens[s];
  const int cap = a.max_blocks * a.block_size;
  n = n < 0 ? 0 : (n > cap ? cap : n);
  int end;
  if (a.query_start_loc == nullptr) {
    end = n;
  } else if (a.causal) {
    int pos = a.positions[q_row];
    pos = pos < 0 ? 0 : (pos >= n ? n - 1 : pos);
    end = pos + 1;
  } else {
    end = n;
  }
  if (n == 0) end = 0;
  int start = 0;
  if (a.window > 0) start = end - a.window > 0 ? end - a.window : 0;
  lo = start;
  hi = end;
  ref = end - 1;
  if (a.partition_size > 0) {
    const int p0 = part * a.partition_size;
    if (p0 >= n) return false;
    lo = lo > p0 ? lo : p0;
    hi = hi < p0 + a.partition_size ? hi : p0 + a.partition_size;
  }
  return true;
}

// NW waves per workgroup.  WP = false: the workgroup answers one (row, kv head[,
// partition]); its waves take the range's tiles round-robin and merge their states
// through LDS at the end.  WP = true (split, one wave): the wave answers one (row,
// kv head, partition) alone and writes the partition's state from registers.
// PR (fp8 only): the workgroup answers a pair of kv heads (2g, 2g + 1) and their 2G q
// heads; tile rows interleave the two heads slot by slot (row 2p + h is slot p of
// head h), so each slot's K and V are read as one 256-byte piece.
// LDS of one decode workgroup: each wave's ring of K / V tiles, reused for the
// merge of the waves' states at the end; the waves' true maxima; the prior lse of
// a merged call's rows.
template <int DK, int NW, int NB, bool F8>
struct DecodeLds {
  static constexpr int DV = 128;
  // V of a tile: four loads of four 256-byte rows, blocks 1 KB + 32 bytes apart (fp8:
  // four loads of eight 128-byte rows); K: KPIECES 256-byte pieces per row
  static constexpr int VBLK = 1024 + 32, VBUF = 4 * VBLK;
  static constexpr int KROWB = DK * 2, KPIECES = KROWB / 256, KBLK = 1024;
  static constexpr int KBUF = F8 ? 4 * KBLK : 4 * KPIECES * KBLK;
  static constexpr int VBUF8 = 4 * KBLK;
  struct Merge {
    float m[NW][16];
    float l[NW][16];
    float o[NW][16][DV];
  };
  struct Tiles {
    char k[NW][NB][KBUF];
    char v[NW][NB][F8 ? VBUF8 : VBUF];
  };
  union Ring {
    Tiles t;
    Merge r;
  };
  __align__(16) Ring u;
  float true_max[NW][16];
  float prev_lse[16];
};

// Unsplit decode of at most 64 rows: the r-th workgroup group takes the row with the
// r-th longest visible range (ties by index), so the longest rows start first and
// the last workgroups to be dispatched are the shortest.
__device__ __forceinline__ bool rows_ranked(const RowsArgs& a, uint32_t grid_rows) {
  return a.query_start_loc == nullptr && a.partition_size == 0 && grid_rows <= (uint32_t)kWave;
}
// The rows of ranks r0 and r1 (one read of the lengths, one count per lane).
__device__ __forceinline__ void rows_by_rank(const RowsArgs& a, int S, int r0, int r1, int& row0, int& row1) {
  const int lane = lane_id(), cap = a.max_blocks * a.block_size;
  int len = -1;
  if (lane < S) {
    int nl = a.seq_lens[lane];
    nl = nl < 0 ? 0 : (nl > cap ? cap : nl);
    len = a.window > 0 && nl > a.window ? a.window : nl;
  }
  int rank = 0;
  for (int r = 0; r < S; ++r) {
    const int lr = __builtin_amdgcn_readlane(len, r);
    rank += (lr > len) || (lr == len && r < lane);
  }
  const uint64_t h0 = __ballot(lane < S && rank == r0), h1 = __ballot(lane < S && rank == r1);
  row0 = h0 ? __builtin_ctzll(h0) : r0;
  row1 = h1 ? __builtin_ctzll(h1) : r1;
}

// One decode workgroup's work: workgroup index wg of a grid of num_wgs, with its
// LDS in L (a kernel of its own launches it alone; the fused varlen kernel beside
// the prefill tiles).  ranked_row >= 0: the row of the ranked order (above) this
// workgroup takes, found by the caller.
template <typename T, int DK, int NW, bool WP, int NB, bool F8, bool PR>
__device__ __forceinline__ void decode_wg(const RowsArgs& a, int block_shift, uint32_t grid_rows, uint32_t wg,
                                          uint32_t num_wgs, DecodeLds<DK, NW, NB, F8>& L, int ranked_row = -1) {
  // WP: each wave answers one (row, kv head, partition) alone -- NW > 1: the
  // workgroup's waves take NW consecutive kv heads of the same row and partition
  static_assert(NB >= 2 && NB <= 4, "2 to 4 tile buffers per wave");
  static_assert(!F8 || DK == 128, "fp8 tiles of 128-byte rows");
  static_assert(!PR || F8, "kv-head pairs on fp8 tiles only");
  using Lds = DecodeLds<DK, NW, NB, F8>;
  constexpr int EB = F8 ? 1 : 2;  // bytes per cache element
  constexpr int DV = Lds::DV;     // V rows of 256 bytes (16 lanes x 16 bytes), 128 for fp8
  constexpr int KCH = DK / 32;    // K operands (8 elements) per lane
  constexpr int ND = DV / 16;     // 16-wide d blocks of O^T
  // A tile's V arrives by direct global->LDS loads: load ii (0..3) writes
  // positions ii + 4c (c = 0..3) as four contiguous 256-byte rows (1 KB, one
  // 16-byte piece per lane); the loads' blocks are 1 KB + 32 bytes apart, so the
  // transpose reads of positions 4c + r (r = 0..3) hit distinct banks.
  constexpr int VBLK = Lds::VBLK;
  // K arrives the same way, KCH/4 * 4 loads of four 256-byte row pieces each; the
  // 16-byte chunks of a row are stored XOR-swizzled so that the A-operand reads
  // (16 positions x one chunk per 16 lanes) touch 16 distinct bank groups.
  constexpr int KPIECES = Lds::KPIECES;  // 256-byte pieces per row
  constexpr int KBLK = Lds::KBLK;        // one load: 4 rows x 256 bytes (fp8: 8 x 128)
  static_assert(Lds::KROWB % 256 == 0, "K rows of whole 256-byte pieces");
  constexpr int kTileLoads = F8 ? 8 : 4 * KPIECES + 4;  // load instructions per tile and wave
  auto& sh = L.u;
  auto& true_max = L.true_max;
  auto& prev_lse = L.prev_lse;

  if (status_failed(a.status)) return;
  // 1-D grid, kv head fastest: the workgroups of one row's kv heads are dispatched
  // together and stream the same blocks (each head's rows are interleaved with the
  // others' in every slot) at about the same time.
  // Split with one wave per partition: partition next fastest, so that the
  // workgroups in flight work on few rows at a time and their state stores fill
  // contiguous rows of the workspace (partition-major order measured about 10 %
  // slower on the long-context workload).
  const int wave_id = (int)(threadIdx.x / kWave);
  const uint32_t hkv_u = (uint32_t)(PR ? a.num_kv_heads / 2 : a.num_kv_heads) / (WP ? NW : 1);
  const int g = (int)(wg % hkv_u) * (WP ? NW : 1) + (WP ? wave_id : 0);
  int row, pz;
  if constexpr (WP) {
    const uint32_t parts_u = num_wgs / (hkv_u * grid_rows);
    pz = (int)((wg / hkv_u) % parts_u);
    row = (int)(wg / (hkv_u * parts_u));
  } else {
    row = (int)((wg / hkv_u) % grid_rows);
    pz = (int)(wg / (hkv_u * grid_rows));
  }
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  if (rows_ranked(a, grid_rows)) {
    if (ranked_row >= 0) {
      row = ranked_row;
    } else {
      int unused;
      rows_by_rank(a, (int)grid_rows, row, row, row, unused);
    }
  }
  int s, n, lo, hi, ref;
  int64_t q_row;
  if (!decode_row_range(a, row, pz, s, q_row, n, lo, hi, ref)) return;  // uniform per workgroup


  const int c = lane >> 4, r16 = lane & 15;
  const int G = a.group, hkv = a.num_kv_heads, b = a.block_size;
  const int GC = PR ? 2 * G : G, hbase = g * GC;  // q heads answered: hbase .. hbase + GC - 1
  const int my_h = PR && r16 >= G ? 1 : 0;        // PR: the kv head of this lane's q head
  const int32_t* table = a.block_tables + (int64_t)s * a.max_blocks;
  const char* kbase = static_cast<const char*>(a.k_pool) + (int64_t)(PR ? 2 * g : g) * DK * EB;
  const char* vbase = static_cast<const char*>(a.v_pool) + (int64_t)(PR ? 2 * g : g) * DV * EB;
  const int64_t krow = (int64_t)hkv * DK * EB, vrow = (int64_t)hkv * DV * EB;
  const int tr_r = r16 >> 2, tr_q = r16 & 3;

  // q heads of the group as the B operand of S^T = K Q^T: operand u of lane group c
  // holds head-dim elements 8 (4u + c) .. +8 (fp8: 32c + 8u .. +8, the order in
  // which the K reads below deliver them)
  u32x4 qb[KCH];
  {
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + (q_row * a.num_heads + hbase + r16) * DK;
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
      const int e0 = F8 ? 32 * c + 8 * u : (4 * u + c) * 8;
      qb[u] = r16 < GC ? *reinterpret_cast<const u32x4*>(qrow + e0) : u32x4{0u, 0u, 0u, 0u};
    }
  }
  // ALiBi ("paged_attention_v2_pytorch.py", phase 1): head r16's slope in raw score
  // units; position j's score gains slope * (j - ref).  The loop counts positions from
  // pref, the last one this workgroup covers (ref itself unless split), so that scores
  // and exp-sums stay exact however far the partition lies from the query; a
  // partition's maximum then gets slope * (pref - ref) added when it is stored.
  // (slope_r is loaded after the first table load, below: a load issued earlier and
  // used here would make the compiler wait for the q loads before that table load.)
  const bool alibi = a.alibi != nullptr;
  float slope_r = 0.f;
  const int pref = hi - 1;
  f32x4 o[ND];
  float m_run, m_true, l_run;  // reference max, true max (raw score units), exp-sum share
#pragma unroll
  for (int nd = 0; nd < ND; ++nd) o[nd] = f32x4{0.f, 0.f, 0.f, 0.f};
  m_run = -kHugeScore;
  m_true = -INFINITY;
  l_run = 0.f;

  // Split, one wave: the partition's state -- (true max, exp-sum against it,
  // normalised output) -- straight from registers.  Lane (head r16, group c) holds output
  // elements 16 nd + 4 c + ii of head r16.
  auto write_state = [&](int p) {
    float l = l_run;
    l = sum_over_groups(l);
    if (r16 < GC) {
      const int64_t pi = ((int64_t)s * a.num_heads + hbase + r16) * a.max_partitions + p;
      const float inv = l > 0.f ? a.v_scale / l : 0.f;
      float* dst = a.tmp_out + pi * DV + 4 * c;
#pragma unroll
      for (int nd = 0; nd < ND; ++nd) *reinterpret_cast<f32x4*>(dst + 16 * nd) = o[nd] * inv;
      if (c == 0) {
        const float m_abs = m_true + slope_r * (float)(pref - ref);  // ALiBi origin back at ref
        a.max_logits[pi] = l > 0.f ? m_abs * a.scale_log2 * kLn2 : -INFINITY;
        a.exp_sums[pi] = l > 0.f ? l * __builtin_amdgcn_exp2f((m_run - m_true) * a.scale_log2) : 0.f;
      }
    }
  };

  // Tiles of TP positions aligned to absolute positions: 16 for 16-bit caches, 32 for
  // fp8, 16 for fp8 kv-head pairs (the same 8 KB of K and V per tile).
  constexpr int TSH = F8 && !PR ? 5 : 4;
  constexpr int TP = 1 << TSH;
  // this wave's tiles: my_first + TS * i, i < my_tiles -- dealt round-robin over the
  // workgroup's waves, or (WP) all of the wave's own (kv head's) range
  constexpr int TS = WP ? 1 : NW;
  const int my_first = (lo >> TSH) + (WP ? 0 : wave);
  const int last = (hi - 1) >> TSH;
  const int my_tiles = (lo < hi && last >= my_first) ? (last - my_first) / TS + 1 : 0;

  // fp8 tiles: tile row r (0..31) holds its 16-byte chunk k in slot k ^ kswz(r) of
  // its 128-byte LDS row, which keeps both read kinds below free of bank conflicts.
  auto kswz = [](int r) { return ((r >> 1) & 3) | ((((r >> 3) ^ (r >> 4)) & 1) << 2); };
  // Lane constants: the LDS offsets of this lane's K chunks 2c and 2c + 1 of rows r16
  // (chain 0) and 16 + r16 (chain 1), and of the row piece it names for each V
  // transpose read nd: position pos(c, r16 / 2) -- 4c + k for k < 4, 16 + 4c + k - 4
  // otherwise -- bytes 16 nd + 8 (r16 % 2) .. +8.  The read then hands lane r16 the
  // element d = 16 nd + r16 of positions pos(c, 0..7): the A operand (V^T) of a
  // 16x16x32 MFMA whose reduction index 8c + k is position pos(c, k).
  uint32_t k8_off[2][2] = {{0u, 0u}, {0u, 0u}}, v8_off[ND] = {};
  if constexpr (F8) {
#pragma unroll
    for (int ch = 0; ch < 2; ++ch)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = 16 * ch + r16;
        k8_off[ch][h] = (uint32_t)((r >> 3) * KBLK + (r & 7) * 128 + 16 * ((2 * c + h) ^ kswz(r)));
      }
    const int k = r16 >> 1, pos = k < 4 ? 4 * c + k : 16 + 4 * c + (k - 4);
#pragma unroll
    for (int nd = 0; nd < ND; ++nd)
      v8_off[nd] = (uint32_t)((pos >> 3) * KBLK + (pos & 7) * 128 + 16 * (nd ^ kswz(pos)) + 8 * (r16 & 1));
  }

  // Block ids of upcoming tiles, one per lane: of tile i0 + lane (16-bit), or of the
  // 16-position half lane % 2 of tile i0 + lane / 2 (fp8 without pairs: with 16-token
  // blocks a tile spans two).  Halves past the sequence read some in-bounds entry of the row; their
  // loads are redirected into the first half below.
  constexpr int IDS_PER_TILE = F8 && !PR ? 2 : 1;
  constexpr int TILES_PER_IDS = 64 / IDS_PER_TILE;
  int ids = 0;
  auto load_ids = [&](int i0) {
    const int i = i0 + lane / IDS_PER_TILE;
    const int half = F8 && !PR ? (lane & 1) : 0;
    int idx = (((my_first + TS * (i < my_tiles ? i : 0)) << TSH) + 16 * half) >> block_shift;
    idx = idx < a.max_blocks ? idx : a.max_blocks - 1;
    const int id = table[idx];
    ids = id < 0 ? 0 : (id >= a.num_blocks ? (int)(a.num_blocks - 1) : id);
  };
  // K and V of tile i into LDS buffer i % NB by direct loads (non-temporal: the
  // data is streamed once).  16-bit: load ii writes positions ii + 4c'' (c'' = lane /
  // 16) as contiguous 256-byte rows, one 16-byte piece per lane; for K the piece a
  // lane fetches is swizzled: LDS chunk slot of logical chunk k in row c'' of load ii
  // is k ^ 4c'' ^ ii (within the 256-byte piece).  fp8: load ld writes tile rows
  // 8 ld + lane / 8, chunk slot lane % 8 receiving the row's chunk (lane % 8) ^
  // kswz(row).  Positions past the sequence read the sequence's last position instead
  // (finite data, in the same block; their scores are masked), so every tile issues
  // exactly kTileLoads loads and a counted wait can tell tiles apart.
  auto fetch = [&](int i) {
    const int t0 = (my_first + TS * i) << TSH;
    char* kl = sh.t.k[wave][i % NB];
    char* vl = sh.t.v[wave][i % NB];
    const int lim = n - 1 - t0;  // >= 0: every tile starts inside the sequence
    if constexpr (PR) {
      // 16 positions of both heads, in one block: tile row r = 8 ld + lane / 8 is slot
      // r / 2 of head r % 2; its 16-byte chunk (lane % 8) ^ kswz(r) lands in slot lane % 8
      const int blk = __builtin_amdgcn_readlane(ids, i & 63);
      const int64_t s0 = (int64_t)blk * b + (t0 & (b - 1));
      const char* k0 = kbase + s0 * krow;
      const char* v0 = vbase + s0 * vrow;
#pragma unroll
      for (int ld = 0; ld < 4; ++ld) {
        const int r = 8 * ld + (lane >> 3);
        const int pos = (r >> 1) < lim ? (r >> 1) : lim;
        const int64_t off = (int64_t)pos * krow + (r & 1) * 128 + ((lane & 7) ^ kswz(r)) * 16;
        __builtin_amdgcn_global_load_lds(k0 + off, (__attribute__((address_space(3))) void*)(kl + ld * KBLK), 16, 0,
                                         kLoadNT);
        __builtin_amdgcn_global_load_lds(v0 + off, (__attribute__((address_space(3))) void*)(vl + ld * KBLK), 16, 0,
                                         kLoadNT);
      }
      return;
    } else if constexpr (F8) {
      const int blk0 = __builtin_amdgcn_readlane(ids, (2 * i) & 63);
      const int blk1 = __builtin_amdgcn_readlane(ids, (2 * i + 1) & 63);
      const int64_t s0 = (int64_t)blk0 * b + (t0 & (b - 1));
      const int64_t s1 = (int64_t)blk1 * b + ((t0 + 16) & (b - 1));
      const char* k0 = kbase + s0 * krow;
      const char* k1 = kbase + s1 * krow;
      const char* v0 = vbase + s0 * vrow;
      const char* v1 = vbase + s1 * vrow;
#pragma unroll
      for (int ld = 0; ld < 4; ++ld) {
        const int r = 8 * ld + (lane >> 3);
        const int rr = r < lim ? r : lim;
        const int ch = (lane & 7) ^ kswz(r);
        const bool first = ld < 2 || rr < 16;  // row rr lies in the tile's first half
        const int64_t ro = (int64_t)(rr & 15);
        __builtin_amdgcn_global_load_lds((first ? k0 : k1) + ro * krow + ch * 16,
                                         (__attribute__((address_space(3))) void*)(kl + ld * KBLK), 16, 0, kLoadNT);
        __builtin_amdgcn_global_load_lds((first ? v0 : v1) + ro * vrow + ch * 16,
                                         (__attribute__((address_space(3))) void*)(vl + ld * KBLK), 16, 0, kLoadNT);
      }
      return;
    }
    const int blk = __builtin_amdgcn_readlane(ids, i & 63);
    const int64_t slot0 = (int64_t)blk * b + (t0 & (b - 1));
    const char* kt = kbase + slot0 * krow;
    const char* vt = vbase + slot0 * vrow + r16 * 16;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int rr = ii + 4 * c < lim ? ii + 4 * c : lim;
      const int kchunk = r16 ^ (4 * c) ^ ii;
#pragma unroll
      for (int pc = 0; pc < KPIECES; ++pc)
        __builtin_amdgcn_global_load_lds(kt + rr * krow + pc * 256 + kchunk * 16,
                                         (__attribute__((address_space(3))) void*)(kl + (pc * 4 + ii) * KBLK), 16, 0,
                                         kLoadNT);
      __builtin_amdgcn_global_load_lds(vt + rr * vrow, (__attribute__((address_space(3))) void*)(vl + ii * VBLK), 16,
                                       0, kLoadNT);
    }
  };
  // The waits are explicit because the direct-to-LDS loads are not otherwise
  // ordered with the LDS reads; the clobbers keep later loads from being hoisted
  // above them.  Vector-memory counts retire in order, so with the kTileLoads loads
  // of each of `ahead` later tiles issued after tile i's, "at most ahead *
  // kTileLoads outstanding" means tile i has landed.
  auto wait_tile = [&](int i) {
    const int ahead = my_tiles - 1 - i;  // tiles issued after tile i, up to NB - 1
    if (NB >= 4 && ahead >= 3)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * kTileLoads) : "memory");
    else if (NB >= 3 && ahead >= 2)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * kTileLoads) : "memory");
    else if (ahead >= 1)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kTileLoads) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  };
  auto refill = [&](int i) {
    if (i + NB < my_tiles) {
      if (((i + NB) & (TILES_PER_IDS - 1)) == 0) load_ids(i + NB);
      fetch(i + NB);
    }
  };
  // The reference-max update shared by both tile kinds: mx is the tile's max over
  // the group's lanes (raw units).
  auto rescale = [&](float mx) {
    m_true = fmaxf(m_true, mx);
    if (__any((mx - m_run) * a.scale_log2 > kRescaleLog2)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * a.scale_log2);
      l_run *= alpha;
#pragma unroll
      for (int nd = 0; nd < ND; ++nd) o[nd] *= alpha;
      m_run = m_new;
    }
  };
  // one 16-bit tile: wait for its loads (the later tiles' may stay in flight), copy
  // its K operands and transposed V from LDS into registers, refill the freed buffer
  // with tile i + NB, then S, softmax and PV from registers.  NB tiles per wave are
  // in flight while one is computed.
  auto step = [&](int i) {
    const int t0 = (my_first + TS * i) << 4;
    const char* kl = sh.t.k[wave][i % NB];
    const char* lb = sh.t.v[wave][i % NB];
    wait_tile(i);
    // The LDS reads are issued as inline asm and their results are tied to the
    // lgkmcnt wait below: the compiler would otherwise guard reads of memory that
    // direct loads write with a full vmcnt(0) wait, draining tile i + 1's loads.
    const uint32_t kl_a = lds_addr(kl), lb_a = lds_addr(lb);
    u32x4 kc[KCH];
    u32x2 va[ND];
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
      // logical chunk 4u + c of position r16 = 4 * row + block
      const int kk = 4 * u + c, piece = kk >> 4, chunk = (kk & 15) ^ (4 * tr_r) ^ tr_q;
      asm volatile("ds_read_b128 %0, %1"
                   : "=v"(kc[u])
                   : "v"(kl_a + (piece * 4 + tr_q) * KBLK + tr_r * 256 + chunk * 16));
    }
    const uint32_t va_a = lb_a + tr_r * VBLK + c * 256 + 4 * tr_q * 2;
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8\n\t"
        "ds_read_b64_tr_b16 %1, %8 offset:32\n\t"
        "ds_read_b64_tr_b16 %2, %8 offset:64\n\t"
        "ds_read_b64_tr_b16 %3, %8 offset:96\n\t"
        "ds_read_b64_tr_b16 %4, %8 offset:128\n\t"
        "ds_read_b64_tr_b16 %5, %8 offset:160\n\t"
        "ds_read_b64_tr_b16 %6, %8 offset:192\n\t"
        "ds_read_b64_tr_b16 %7, %8 offset:224"
        : "=&v"(va[0]), "=&v"(va[1]), "=&v"(va[2]), "=&v"(va[3]), "=&v"(va[4]), "=&v"(va[5]), "=&v"(va[6]),
          "=&v"(va[7])
        : "v"(va_a));
    // the reads of buffer i % NB complete (and their registers are valid) before
    // tile i + NB's loads may overwrite it
    static_assert(KCH == 4 && ND == 8, "operand wait below lists 4 K and 8 V registers");
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(kc[0]), "+v"(kc[1]), "+v"(kc[2]), "+v"(kc[3]), "+v"(va[0]), "+v"(va[1]), "+v"(va[2]),
                   "+v"(va[3]), "+v"(va[4]), "+v"(va[5]), "+v"(va[6]), "+v"(va[7])
                 :
                 : "memory");
    refill(i);

    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < KCH; ++u) sc = mfma_16x16x32<T>(kc[u], qb[u], sc);
    float sv[4] = {sc[0], sc[1], sc[2], sc[3]};
    if (alibi) {
      const float jb = (float)(t0 + 4 * c - pref);  // exact: |j - pref| < 2^24
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) sv[ii] = fmaf(slope_r, jb + (float)ii, sv[ii]);
    }
    if (t0 < lo || t0 + 16 > hi) {
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int j = t0 + 4 * c + ii;
        if (j < lo || j >= hi) sv[ii] = -INFINITY;
      }
    }
    float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    rescale(max_over_groups(mx));
    const float mc = m_run * a.scale_log2;
    float p[4];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) p[ii] = __builtin_amdgcn_exp2f(fmaf(sv[ii], a.scale_log2, -mc));
    l_run += (p[0] + p[1]) + (p[2] + p[3]);
    // O^T[d][head] += V^T[d][position] P^T[position][head]
    if constexpr (T::code == PA_F16) {
      const u32x2 pb = u32x2{pack_f16x2(p[0], p[1]), pack_f16x2(p[2], p[3])};
#pragma unroll
      for (int nd = 0; nd < ND; ++nd) o[nd] = mfma_16x16x16<F16>(va[nd], pb, o[nd]);
    } else {
      const uint32_t h0 = pack_bf16x2(p[0], p[1]), h1 = pack_bf16x2(p[2], p[3]);
      const u32x2 pb = u32x2{h0, h1};
      const u32x2 pl = u32x2{pack_bf16x2(p[0] - __uint_as_float(h0 << 16), p[1] - __uint_as_float(h0 & 0xffff0000u)),
                             pack_bf16x2(p[2] - __uint_as_float(h1 << 16), p[3] - __uint_as_float(h1 & 0xffff0000u))};
#pragma unroll
      for (int nd = 0; nd < ND; ++nd) {
        o[nd] = mfma_16x16x16<BF16>(va[nd], pb, o[nd]);
        o[nd] = mfma_16x16x16<BF16>(va[nd], pl, o[nd]);
      }
    }
  };
  // one fp8 tile of 32 positions: S^T of positions 0..15 and 16..31 as two 16-row
  // chains, one softmax step over both, and O^T += V^T P^T on 16x16x32 MFMAs whose
  // reduction index 8c + k is position pos(c, k) -- P^T's rows are already there:
  // lane (head, c) holds the two chains' positions 4c .. 4c + 3.
  auto step8 = [&](int i) {
    const int t0 = (my_first + TS * i) << TSH;
    const uint32_t kl_a = lds_addr(sh.t.k[wave][i % NB]), lb_a = lds_addr(sh.t.v[wave][i % NB]);
    wait_tile(i);
    u32x4 k8[2][2];
    u32x2 v8[ND];
#pragma unroll
    for (int ch = 0; ch < 2; ++ch)
#pragma unroll
      for (int h = 0; h < 2; ++h) asm volatile("ds_read_b128 %0, %1" : "=v"(k8[ch][h]) : "v"(kl_a + k8_off[ch][h]));
#pragma unroll
    for (int nd = 0; nd < ND; ++nd) asm volatile("ds_read_b64_tr_b8 %0, %1" : "=v"(v8[nd]) : "v"(lb_a + v8_off[nd]));
    static_assert(ND == 8, "operand wait below lists 4 K and 8 V registers");
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(k8[0][0]), "+v"(k8[0][1]), "+v"(k8[1][0]), "+v"(k8[1][1]), "+v"(v8[0]), "+v"(v8[1]),
                   "+v"(v8[2]), "+v"(v8[3]), "+v"(v8[4]), "+v"(v8[5]), "+v"(v8[6]), "+v"(v8[7])
                 :
                 : "memory");
    refill(i);

    // S^T, chain ch: K operand u = 2h + w is bytes 8w .. 8w + 7 of read (ch, h)
    f32x4 sc[2];
#pragma unroll
    for (int ch = 0; ch < 2; ++ch) {
      sc[ch] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int w = 0; w < 2; ++w) {
          const u32x4 kop = u32x4{widen_fp8x2<T, false>(k8[ch][h][2 * w]), widen_fp8x2<T, true>(k8[ch][h][2 * w]),
                                  widen_fp8x2<T, false>(k8[ch][h][2 * w + 1]),
                                  widen_fp8x2<T, true>(k8[ch][h][2 * w + 1])};
          sc[ch] = mfma_16x16x32<T>(kop, qb[2 * h + w], sc[ch]);
        }
    }
    float sv[8];  // position 16 (k / 4) + 4c + k % 4 for k = 0..7
#pragma unroll
    for (int k = 0; k < 8; ++k) sv[k] = sc[k >> 2][k & 3];
    if constexpr (PR) {
      // entry k is tile row 16 (k / 4) + 4c + k % 4: position t0 + 8 (k / 4) + 2c + (k % 4) / 2
      // of kv head k % 2; the other head's rows are not this lane's q head's keys
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int j = t0 + 8 * (k >> 2) + 2 * c + ((k & 3) >> 1);
        if (alibi) sv[k] = fmaf(slope_r, (float)(j - pref), sv[k]);  // exact: |j - pref| < 2^24
        if ((k & 1) != my_h) sv[k] = -INFINITY;
      }
      if (t0 < lo || t0 + TP > hi) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int j = t0 + 8 * (k >> 2) + 2 * c + ((k & 3) >> 1);
          if (j < lo || j >= hi) sv[k] = -INFINITY;
        }
      }
    } else {
      if (alibi) {
        const float jb = (float)(t0 + 4 * c - pref);  // exact: |j - pref| < 2^24
#pragma unroll
        for (int k = 0; k < 8; ++k) sv[k] = fmaf(slope_r, jb + (float)(16 * (k >> 2) + (k & 3)), sv[k]);
      }
      if (t0 < lo || t0 + 32 > hi) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int j = t0 + 16 * (k >> 2) + 4 * c + (k & 3);
          if (j < lo || j >= hi) sv[k] = -INFINITY;
        }
      }
    }
    const float mx = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])), fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
    rescale(max_over_groups(mx));
    const float mc = m_run * a.scale_log2;
    float p[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) p[k] = __builtin_amdgcn_exp2f(fmaf(sv[k], a.scale_log2, -mc));
    l_run += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
    // O^T[d][head] += V^T[d][position] P^T[position][head]
    u32x4 va[ND];
#pragma unroll
    for (int nd = 0; nd < ND; ++nd)
      va[nd] = u32x4{widen_fp8x2<T, false>(v8[nd][0]), widen_fp8x2<T, true>(v8[nd][0]),
                     widen_fp8x2<T, false>(v8[nd][1]), widen_fp8x2<T, true>(v8[nd][1])};
    if constexpr (T::code == PA_F16) {
      const u32x4 pb = u32x4{pack_f16x2(p[0], p[1]), pack_f16x2(p[2], p[3]), pack_f16x2(p[4], p[5]),
                             pack_f16x2(p[6], p[7])};
#pragma unroll
      for (int nd = 0; nd < ND; ++nd) o[nd] = mfma_16x16x32<F16>(va[nd], pb, o[nd]);
    } else {
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        hw[e] = pack_bf16x2(p[2 * e], p[2 * e + 1]);
        lw[e] = pack_bf16x2(p[2 * e] - __uint_as_float(hw[e] << 16), p[2 * e + 1] - __uint_as_float(hw[e] & 0xffff0000u));
      }
      const u32x4 pb = u32x4{hw[0], hw[1], hw[2], hw[3]}, pl = u32x4{lw[0], lw[1], lw[2], lw[3]};
#pragma unroll
      for (int nd = 0; nd < ND; ++nd) {
        o[nd] = mfma_16x16x32<BF16>(va[nd], pb, o[nd]);
        o[nd] = mfma_16x16x32<BF16>(va[nd], pl, o[nd]);
      }
    }
  };

  // The first block ids are loaded while the q loads are still in flight (two round
  // trips overlap); the q loads' wait is taken here, before any K/V load is in
  // flight -- otherwise the compiler guards the loop's first use of qb with a full
  // vmcnt(0) every tile.
  if (my_tiles > 0) load_ids(0);
  if (alibi && r16 < GC) slope_r = a.alibi[hbase + r16] * (kLog2e / a.scale_log2);
#pragma unroll
  for (int u = 0; u < KCH; ++u) asm volatile("" ::"v"(qb[u]));
  if (my_tiles > 0) {
#pragma unroll
    for (int j = 0; j < NB; ++j)
      if (j < my_tiles) fetch(j);
  }
  for (int i = 0; i < my_tiles; ++i) {
    if constexpr (F8)
      step8(i);
    else
      step(i);
  }
  if constexpr (WP) {
    write_state(pz);  // (-inf, 0, 0) when the window leaves the partition empty
    return;
  }

  // --- merge of the waves' states (O^T is complete per wave) ----
  l_run = sum_over_groups(l_run);
  __syncthreads();  // the tile buffers become the merge area
  if (lane < 16) {
    sh.r.m[wave][lane] = m_run;
    sh.r.l[wave][lane] = l_run;
    true_max[wave][lane] = m_true;
  }
#pragma unroll
  for (int nd = 0; nd < ND; ++nd)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) sh.r.o[wave][r16][16 * nd + 4 * c + ii] = o[nd][ii];
  __syncthreads();

  // merging into a state held by out (float32) and lse: every head's previous lse is
  // read before any is written
  if (a.merge) {
    if ((int)threadIdx.x < GC) prev_lse[threadIdx.x] = a.lse[(int64_t)(hbase + threadIdx.x) * a.num_rows + q_row];
    __syncthreads();
  }
  for (int idx = threadIdx.x; idx < GC * DV; idx += blockDim.x) {
    const int h = idx / DV, d = idx - h * DV;
    // Re-express every wave's (reference max, sums) against the true max M; the
    // factors are at most 1.
    const int hq = hbase + h;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, true_max[w][h]);
    // an attention sink (unsplit calls): one more position with score z (z / scale
    // in raw units) and a zero value; split calls leave it to the reduction
    const float zr =
        (a.sinks != nullptr && a.partition_size == 0) ? a.sinks[hq] * (kLog2e / a.scale_log2) : -INFINITY;
    M = fmaxf(M, zr);
    float L = 0.f, O = 0.f;
    if (M != -INFINITY) {
      L = __builtin_amdgcn_exp2f((zr - M) * a.scale_log2);
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float f = __builtin_amdgcn_exp2f((sh.r.m[w][h] - M) * a.scale_log2);
        L = fmaf(sh.r.l[w][h], f, L);
        O = fmaf(sh.r.o[w][h][d], f, O);
      }
    }
    const float out_v = L > 0.f ? O * (a.v_scale / L) : 0.f;
    if (a.partition_size == 0) {
      const int64_t oi = (q_row * a.num_heads + hq) * (int64_t)DV + d;
      const float lse_new = L > 0.f ? (M * a.scale_log2 + log2f(L)) * kLn2 : -INFINITY;
      if (a.merge) {  // this call is the suffix of the merge
        float wp, ws, lse_m;
        bool keep;
        merge_state_weights(prev_lse[h], lse_new, wp, ws, lse_m, keep);
        float* dst = static_cast<float*>(a.out) + oi;
        if (!keep) *dst = *dst * wp + out_v * ws;
        if (d == 0) a.lse[(int64_t)hq * a.num_rows + q_row] = lse_m;
      } else {
        store_as(a.out, a.out_dtype, oi, out_v);
        if (a.lse != nullptr && d == 0) a.lse[(int64_t)hq * a.num_rows + q_row] = lse_new;
      }
    } else {
      const int64_t pi = ((int64_t)s * a.num_heads + hq) * a.max_partitions + pz;
      a.tmp_out[pi * DV + d] = out_v;
      if (d == 0) {
        // ALiBi origin back at ref (see the loop)
        const float off = alibi ? a.alibi[hq] * (kLog2e / a.scale_log2) * (float)(pref - ref) : 0.f;
        a.max_logits[pi] = L > 0.f ? (M + off) * a.scale_log2 * kLn2 : -INFINITY;
        a.exp_sums[pi] = L;
      }
    }
  }
}

// paired_units > 0 (unsplit calls): the grid is ceil(paired_units / 2) workgroups and
// workgroup w answers unit w, then unit paired_units - 1 - w, where the units are the
// workgroup indices of the one-unit grid.  With rows taken longest first, the
// longest unit shares a workgroup with the shortest, so the pairs carry about equal
// work, the grid is one round of the chip, and no workgroup is dispatched after
// another's end; each unit's arithmetic is that of the one-unit grid, bit for bit.
template <typename T, int DK, int NW, bool WP, int NB, bool F8, bool PR = false>
__global__ __launch_bounds__(NW * 64) void decode_mfma_kernel(const RowsArgs a, int block_shift, uint32_t grid_rows,
                                                              uint32_t paired_units) {
  __shared__ DecodeLds<DK, NW, NB, F8> lds;
  if constexpr (!WP) {
    if (paired_units > 0) {
      const uint32_t w = blockIdx.x, partner = paired_units - 1 - w;
      // both units' rows from one ranking, so the second unit starts at once
      int row_w = -1, row_p = -1;
      if (rows_ranked(a, grid_rows)) {
        const uint32_t hkv_u = (uint32_t)(PR ? a.num_kv_heads / 2 : a.num_kv_heads);
        rows_by_rank(a, (int)grid_rows, (int)((w / hkv_u) % grid_rows), (int)((partner / hkv_u) % grid_rows), row_w,
                     row_p);
      }
      decode_wg<T, DK, NW, WP, NB, F8, PR>(a, block_shift, grid_rows, w, paired_units, lds, row_w);
      if (partner != w) {
        __syncthreads();  // the first unit's merge area becomes the second's tile ring
        decode_wg<T, DK, NW, WP, NB, F8, PR>(a, block_shift, grid_rows, partner, paired_units, lds, row_p);
      }
      return;
    }
  }
  decode_wg<T, DK, NW, WP, NB, F8, PR>(a, block_shift, grid_rows, blockIdx.x, gridDim.x, lds);
}

// Waves per workgroup and tile buffers per wave.  A buffer holds a tile from load
// issue until its copy into registers, so LDS bounds the loads in flight per CU:
// unsplit, 8 waves x 2 buffers = 130 KB, one workgroup per CU; split with few
// partitions, 4 waves x 2 buffers, two per CU; one-wave split, 2 buffers.  Deeper
// rings (6 waves x 3, 4 x 4) measured no faster.
constexpr int kWholeWaves = 8, kWholeBufs = 2;
constexpr int kPartWaves = 4, kPartBufs = 2;
constexpr int kOneWaveBufs = 2;
// Split mode: one wave per (row, kv head, partition) item when there are at least
// kOneWaveItems items, or when rows span at least kOneWaveParts partitions (so
// nearly every item is a whole partition, long enough to amortise a wave's start)
// and there are at least kOneWaveMinItems items (four waves per CU); otherwise
// kPartWaves waves share each partition.  On the long-context workload (8 rows of
// 32K-128K positions) one wave per item ran 0.72 / 0.73 / 0.78 of HBM at partitions
// of 1024 / 2048 / 4096 against 0.63 / 0.67 / 0.66 shared (its fp8 version at 512:
// 0.62 against 0.50); on the batched workload (64 rows of 512-4096, at most 8
// partitions) sharing stayed ahead (0.63 against 0.61 at 512, 0.64 against 0.55 at
// 1024).
constexpr int64_t kOneWaveItems = 8192, kOneWaveMinItems = 1024;
constexpr int kOneWaveParts = 16;
inline bool one_wave_split(const RowsArgs& a, uint64_t items) {
  return a.partition_size > 0 &&
         ((int64_t)items >= kOneWaveItems || (a.max_partitions >= kOneWaveParts && (int64_t)items >= kOneWaveMinItems));
}

// fp8 tiles of 32 positions hold as many bytes as 16-bit tiles of 16: the same two
// buffers per wave (unsplit: 8 waves x 2 x 8 KB = 128 KB of LDS).
constexpr int kFp8Bufs = 2;
constexpr int kFp8WholeWaves = 8;

// Split calls with many (row, kv head, partition) items run one wave per item, the
// waves of a workgroup on consecutive kv heads (or kv-head pairs) of the same row
// and partition: 4 of them when the count divides, else 2 or 1.  The waves stream
// the same blocks -- each slot's kv heads lie side by side -- at the same time on
// one CU: on the long-context workload 5.59 TB/s with 4 heads per workgroup, 5.50
// with 8, 5.27 with one (same box); a streaming probe of the access pattern alone
// gives 7.0 TB/s with a block's heads in one workgroup, 6.6 with one head per
// workgroup.
inline int split_head_waves(int units) { return units % 4 == 0 ? 4 : units % 2 == 0 ? 2 : 1; }

template <typename T, bool F8, bool PR>
hipError_t launch_split_waves(const RowsArgs& a, int block_shift, uint32_t rows, uint64_t items, int units,
                              hipStream_t stream) {
  constexpr int bufs = F8 ? kFp8Bufs : kOneWaveBufs;
  const int w = split_head_waves(units);
  const dim3 grid((uint32_t)(items / (uint64_t)w)), block(64 * w);
  if (w == 4)
    hipLaunchKernelGGL((decode_mfma_kernel<T, 128, 4, true, bufs, F8, PR>), grid, block, 0, stream, a, block_shift, rows,
                       0u);
  else if (w == 2)
    hipLaunchKernelGGL((decode_mfma_kernel<T, 128, 2, true, bufs, F8, PR>), grid, block, 0, stream, a, block_shift, rows,
                       0u);
  else
    hipLaunchKernelGGL((decode_mfma_kernel<T, 128, 1, true, bufs, F8, PR>), grid, block, 0, stream, a, block_shift, rows,
                       0u);
  return hipGetLastError();
}

// `grid` is (rows, kv heads, partitions); the kernel takes it flattened.
template <typename T, bool F8>
hipError_t launch_decode_typed(const RowsArgs& a, int block_shift, int dk, int dv, dim3 grid, hipStream_t stream) {
  if ((int)grid.y != a.num_kv_heads || dk != 128 || dv != 128) return hipErrorInvalidValue;
  const uint32_t rows = grid.x;
  const uint64_t n = (uint64_t)grid.x * grid.y * grid.z;
  if (n > 0xffffffffull) return hipErrorInvalidValue;
  constexpr int part_bufs = F8 ? kFp8Bufs : kPartBufs, whole_bufs = F8 ? kFp8Bufs : kWholeBufs;
  if constexpr (F8) {
    // split fp8 calls with an even number of kv heads and at most 8 q heads per kv
    // head: one workgroup per pair of kv heads (256-byte reads per slot)
    if (a.partition_size > 0 && a.num_kv_heads % 2 == 0 && 2 * a.group <= 16) {
      const uint64_t np = n / 2;
      if (one_wave_split(a, np))
        return launch_split_waves<T, true, true>(a, block_shift, rows, np, a.num_kv_heads / 2, stream);
      hipLaunchKernelGGL((decode_mfma_kernel<T, 128, kPartWaves, false, part_bufs, true, true>),
                         dim3((uint32_t)np), dim3(kPartWaves * 64), 0, stream, a, block_shift, rows, 0u);
      return hipGetLastError();
    }
  }
  // Unsplit varlen rows over 16-bit caches run on 4-wave workgroups, as the fused
  // varlen kernel runs them beside prefill tiles: a row's bits then do not depend on
  // whether its batch holds prefill sequences.
  const bool varlen_rows = a.query_start_loc != nullptr && a.partition_size == 0 && !F8;
  if (one_wave_split(a, n))
    return launch_split_waves<T, F8, false>(a, block_shift, rows, n, a.num_kv_heads, stream);
  if (a.partition_size > 0 || varlen_rows) {
    hipLaunchKernelGGL((decode_mfma_kernel<T, 128, kPartWaves, false, part_bufs, F8>), dim3((uint32_t)n),
                       dim3(kPartWaves * 64), 0, stream, a, block_shift, rows, 0u);
    return hipGetLastError();
  }
  // Unsplit decode (one workgroup per CU, 130 KB of LDS) of at least two rounds of
  // the chip: two units per workgroup, the longest with the shortest, so the grid
  // is one round and no unit waits for another's workgroup to end (flushed, same
  // box: batched decode 101.5 -> 101.0 us, its fp8 version 68.0 -> 66.2 us).  Fewer
  // units keep one per workgroup, where pairs would serialise units that fit side by
  // side.
  const int cus = device_cu_count();
  const bool pair = a.query_start_loc == nullptr && cus > 0 && n >= 2 * (uint64_t)cus;
  constexpr int whole_waves = F8 ? kFp8WholeWaves : kWholeWaves;
  hipLaunchKernelGGL((decode_mfma_kernel<T, 128, whole_waves, false, whole_bufs, F8>),
                     dim3((uint32_t)(pair ? (n + 1) / 2 : n)), dim3(whole_waves * 64), 0, stream, a, block_shift, rows,
                     pair ? (uint32_t)n : 0u);
  return hipGetLastError();
}

}  // namespace pa
