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
// Loads are software-pipelined one tile ahead, and the block ids of a wave's tiles
// are fetched up to 64 at a time with one vector load and broadcast per tile, so
// no K/V load waits on a table lookup.  Requires a power-of-two block size that is
// a multiple of 16 (a tile then lies inside one block) and head dims of 128.
#pragma once

#include "pa_common.h"
#include "pa_internal.h"
#include "pa_prefill.h"

namespace pa {

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

constexpr int kDecodeWaves = 4;
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

// Which sequence and which visible range a row workgroup covers; false: nothing to do.
__device__ __forceinline__ bool decode_row_range(const RowsArgs& a, int row, int part, int& s, int64_t& q_row, int& n,
                                                 int& lo, int& hi) {
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
  if (a.partition_size > 0) {
    const int p0 = part * a.partition_size;
    if (p0 >= n) return false;
    lo = lo > p0 ? lo : p0;
    hi = hi < p0 + a.partition_size ? hi : p0 + a.partition_size;
  }
  return true;
}

template <typename T, int DK>
__global__ __launch_bounds__(kDecodeWaves * 64) void decode_mfma_kernel(const RowsArgs a, int block_shift) {
  constexpr int DV = 128;        // V rows of 256 bytes: 16 lanes x 16 bytes
  constexpr int NW = kDecodeWaves;
  constexpr int KCH = DK / 32;   // 16-byte K chunks per lane
  constexpr int ND = DV / 16;    // 16-wide d blocks of O^T
  // A tile's V arrives by direct global->LDS loads: load ii (0..3) writes
  // positions ii + 4c (c = 0..3) as four contiguous 256-byte rows (1 KB, one
  // 16-byte piece per lane); the loads' blocks are 1 KB + 32 bytes apart, so the
  // transpose reads of positions 4c + r (r = 0..3) hit distinct banks.
  constexpr int VBLK = 1024 + 32;
  constexpr int VBUF = 4 * VBLK;
  // K arrives the same way, KCH/4 * 4 loads of four 256-byte row pieces each; the
  // 16-byte chunks of a row are stored XOR-swizzled so that the A-operand reads
  // (16 positions x one chunk per 16 lanes) touch 16 distinct bank groups.
  constexpr int KROWB = DK * 2;             // bytes of one K row
  constexpr int KPIECES = KROWB / 256;      // 256-byte pieces per row
  constexpr int KBLK = 1024;                // one load: 4 rows x 256 bytes
  constexpr int KBUF = 4 * KPIECES * KBLK;  // a tile's K
  static_assert(KROWB % 256 == 0, "K rows of whole 256-byte pieces");
  struct Merge {
    float m[NW][16];
    float l[NW][16];
    float o[NW][16][DV];
  };
  __shared__ float true_max[NW][16];
  struct Tiles {
    char k[NW][2][KBUF];
    char v[NW][2][VBUF];
  };
  __shared__ __align__(16) union {
    Tiles t;
    Merge r;
  } sh;

  if (status_failed(a.status)) return;
  const int row = blockIdx.x, g = blockIdx.y, part = blockIdx.z;
  int s, n, lo, hi;
  int64_t q_row;
  if (!decode_row_range(a, row, part, s, q_row, n, lo, hi)) return;

  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int c = lane >> 4, r16 = lane & 15;
  const int G = a.group, hkv = a.num_kv_heads, b = a.block_size;
  const int32_t* table = a.block_tables + (int64_t)s * a.max_blocks;
  const char* kbase = static_cast<const char*>(a.k_pool) + (int64_t)g * DK * 2;
  const char* vbase = static_cast<const char*>(a.v_pool) + (int64_t)g * DV * 2;
  const int64_t krow = (int64_t)hkv * DK * 2, vrow = (int64_t)hkv * DV * 2;
  const int tr_r = r16 >> 2, tr_q = r16 & 3;

  // q heads of the group as the B operand of S^T = K Q^T
  u32x4 qb[KCH];
  {
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + (q_row * a.num_heads + g * G + r16) * DK;
#pragma unroll
    for (int u = 0; u < KCH; ++u)
      qb[u] = r16 < G ? *reinterpret_cast<const u32x4*>(qrow + (4 * u + c) * 8) : u32x4{0u, 0u, 0u, 0u};
  }
  // Zero this wave's V buffers: slots past the sequence are never loaded, and their
  // rows (multiplied by p = 0) must hold finite values.
  {
    u32x4* z = reinterpret_cast<u32x4*>(sh.t.v[wave][0]);
    for (int x = lane; x < 2 * VBUF / 16; x += kWave) z[x] = u32x4{0u, 0u, 0u, 0u};
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // zeros land before any load into LDS

  f32x4 o[ND];
#pragma unroll
  for (int nd = 0; nd < ND; ++nd) o[nd] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -kHugeScore;  // reference max for head r16 (raw score units)
  float m_true = -INFINITY;   // true max of the scores seen, head r16
  float l_run = 0.f;          // this lane group's share of the exp-sum

  const int my_first = (lo >> 4) + wave;
  const int last = (hi - 1) >> 4;
  const int my_tiles = (lo < hi && last >= my_first) ? (last - my_first) / NW + 1 : 0;

  int ids = 0;  // block ids of up to 64 upcoming tiles, one per lane
  auto load_ids = [&](int i0) {
    const int i = i0 + lane;
    int idx = ((my_first + NW * (i < my_tiles ? i : 0)) << 4) >> block_shift;
    idx = idx < a.max_blocks ? idx : a.max_blocks - 1;
    const int id = table[idx];
    ids = id < 0 ? 0 : (id >= a.num_blocks ? (int)(a.num_blocks - 1) : id);
  };
  // K and V of tile i into LDS buffer i & 1 by direct loads (non-temporal: the
  // data is streamed once).  Load ii writes positions ii + 4c'' (c'' = lane / 16)
  // as contiguous 256-byte rows, one 16-byte piece per lane; for K the piece a lane
  // fetches is swizzled: LDS chunk slot of logical chunk k in row c'' of load ii is
  // k ^ 4c'' ^ ii (within the 256-byte piece).  Slots past the sequence are not
  // loaded.
  auto fetch = [&](int i) {
    const int t0 = (my_first + NW * i) << 4;
    const int blk = __builtin_amdgcn_readlane(ids, i & 63);
    const int64_t slot0 = (int64_t)blk * b + (t0 & (b - 1));
    const char* kt = kbase + slot0 * krow;
    const char* vt = vbase + slot0 * vrow + r16 * 16;
    char* kl = sh.t.k[wave][i & 1];
    char* vl = sh.t.v[wave][i & 1];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      if (t0 + ii + 4 * c < n) {
        const int kchunk = r16 ^ (4 * c) ^ ii;
#pragma unroll
        for (int pc = 0; pc < KPIECES; ++pc)
          __builtin_amdgcn_global_load_lds(kt + (ii + 4 * c) * krow + pc * 256 + kchunk * 16,
                                           (__attribute__((address_space(3))) void*)(kl + (pc * 4 + ii) * KBLK), 16, 0,
                                           kLoadNT);
        __builtin_amdgcn_global_load_lds(vt + (ii + 4 * c) * vrow, (__attribute__((address_space(3))) void*)(vl + ii * VBLK),
                                         16, 0, kLoadNT);
      }
    }
  };
  // one tile: its K operands and transpose reads of V first (so that no wait covers
  // the next tile's loads), then the next tile's loads, then S, softmax and PV.
  auto step = [&](int i) {
    const int t0 = (my_first + NW * i) << 4;
    const char* kl = sh.t.k[wave][i & 1];
    const char* lb = sh.t.v[wave][i & 1];
    // Tile i's loads (issued one step earlier) must have landed before its K and V
    // are read back from LDS; the waits are explicit because the direct-to-LDS
    // loads are not otherwise ordered with these reads, and the clobbers keep tile
    // i+1's loads from being hoisted above them.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    u32x4 kc[KCH];
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
      // logical chunk 4u + c of position r16 = 4 * row + block
      const int kk = 4 * u + c, piece = kk >> 4, chunk = (kk & 15) ^ (4 * tr_r) ^ tr_q;
      kc[u] = *reinterpret_cast<const u32x4*>(kl + (piece * 4 + tr_q) * KBLK + tr_r * 256 + chunk * 16);
    }
    u32x2 va[ND];
#pragma unroll
    for (int nd = 0; nd < ND; ++nd)
      va[nd] = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                            (lds_i16x4*)(lb + tr_r * VBLK + c * 256 + (16 * nd + 4 * tr_q) * 2)));
    asm volatile("" ::: "memory");
    if ((i & 63) == 63 && i + 1 < my_tiles) load_ids(i + 1);
    if (i + 1 < my_tiles) fetch(i + 1);

    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < KCH; ++u) sc = mfma_16x16x32<T>(kc[u], qb[u], sc);
    float sv[4] = {sc[0], sc[1], sc[2], sc[3]};
    if (t0 < lo || t0 + 16 > hi) {
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int j = t0 + 4 * c + ii;
        if (j < lo || j >= hi) sv[ii] = -INFINITY;
      }
    }
    float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    mx = fmaxf(mx, shfl_xor(mx, 16));
    mx = fmaxf(mx, shfl_xor(mx, 32));
    m_true = fmaxf(m_true, mx);
    if (__any((mx - m_run) * a.scale_log2 > kRescaleLog2)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * a.scale_log2);
      l_run *= alpha;
#pragma unroll
      for (int nd = 0; nd < ND; ++nd) o[nd] *= alpha;
      m_run = m_new;
    }
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

  if (my_tiles > 0) {
    load_ids(0);
    fetch(0);
  }
  for (int i = 0; i < my_tiles; ++i) step(i);

  // --- merge: lane groups (exp-sum only; O^T is complete per wave), then waves ----
  l_run += shfl_xor(l_run, 16);
  l_run += shfl_xor(l_run, 32);
  __syncthreads();  // the V buffers become the merge area
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

  for (int idx = threadIdx.x; idx < G * DV; idx += blockDim.x) {
    const int h = idx / DV, d = idx - h * DV;
    // Re-express every wave's (reference max, sums) against the true max M; the
    // factors are at most 1.
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, true_max[w][h]);
    float L = 0.f, O = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float f = __builtin_amdgcn_exp2f((sh.r.m[w][h] - M) * a.scale_log2);
        L = fmaf(sh.r.l[w][h], f, L);
        O = fmaf(sh.r.o[w][h][d], f, O);
      }
    }
    const float out_v = L > 0.f ? O * (1.0f / L) : 0.f;
    const int hq = g * G + h;
    if (a.partition_size == 0) {
      store_as(a.out, a.out_dtype, (q_row * a.num_heads + hq) * (int64_t)DV + d, out_v);
      if (a.lse != nullptr && d == 0)
        a.lse[(int64_t)hq * a.num_rows + q_row] = L > 0.f ? (M * a.scale_log2 + log2f(L)) * kLn2 : -INFINITY;
    } else {
      const int64_t pi = ((int64_t)s * a.num_heads + hq) * a.max_partitions + part;
      a.tmp_out[pi * DV + d] = out_v;
      if (d == 0) {
        a.max_logits[pi] = L > 0.f ? M * a.scale_log2 * kLn2 : -INFINITY;
        a.exp_sums[pi] = L;
      }
    }
  }
}

template <typename T>
hipError_t launch_decode_typed(const RowsArgs& a, int block_shift, int dk, int dv, dim3 grid, hipStream_t stream) {
  const dim3 block(kDecodeWaves * 64);
  if (dk == 128 && dv == 128)
    hipLaunchKernelGGL((decode_mfma_kernel<T, 128>), grid, block, 0, stream, a, block_shift);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pa
