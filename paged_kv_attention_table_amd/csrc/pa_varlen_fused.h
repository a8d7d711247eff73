// One launch for a varlen call that mixes prefill chunks with single decode tokens
// (TensorSharp "ManagedPagedAttention.cs", Forward: one call over a batch packed by
// query_start_loc).  The grid is one decode workgroup per (sequence, kv head) --
// rows that are not single tokens exit at once -- padded to a multiple of 8, then
// the prefill tile grid; both kinds share the kernel's LDS and its 256 threads.
// Over fp8 pools (F8) both halves read fp8 (E4M3) K/V; T is the queries' type.
// Small tile grids (about one round of the chip) run rank-major, heaviest tiles
// first, so the decode rows, which start at once, run beside the heavy tiles and
// the lightest tiles (early causal rows, little context) follow them.  Run on a
// launch of their own, the rows waited for the whole tile launch.
#pragma once

#include "pa_decode.h"

namespace pa {

// The decode rows' workgroup shape: the same as unsplit varlen rows on a launch of
// their own (4 waves, 2 tile buffers each), so their results match bit for bit.
constexpr int kFusedDecodeWaves = kPrefillThreads / kWave, kFusedDecodeBufs = 2;
static_assert(kFusedDecodeWaves == kPartWaves && kFusedDecodeBufs == kPartBufs, "one shape for varlen rows");
// Tile grids up to this many workgroups (two rounds of MI355X's 256 CUs at two per
// CU) run rank-major.
constexpr uint32_t kFusedRankMajorWgs = 1024;

template <typename T, bool ALIBI, bool MERGE, bool F8 = false>
__global__ __launch_bounds__(kPrefillThreads, 2) void varlen_fused_kernel(const PrefillArgs p, const RowsArgs r,
                                                                           int block_shift, uint32_t prefill_wgs) {
  __shared__ union {
    PrefillLds<128, 128> pf;
    DecodeLds<128, kFusedDecodeWaves, kFusedDecodeBufs, F8> dc;
  } lds;
  const uint32_t rows = (uint32_t)r.num_seqs * r.num_kv_heads, decode_wgs = (rows + 7) / 8 * 8;
  if (blockIdx.x >= decode_wgs) {
    prefill_tile<T, 128, 128, ALIBI, MERGE, false, F8>(p, (int)(blockIdx.x - decode_wgs), lds.pf);
  } else if (blockIdx.x < rows) {
    decode_wg<T, 128, kFusedDecodeWaves, false, kFusedDecodeBufs, F8, false>(r, block_shift, (uint32_t)r.num_seqs,
                                                                             blockIdx.x, rows, lds.dc);
  }
}

// p: the tile launch's arguments (prefill_wgs workgroups); r: the single-token rows'
// (one row per sequence, single_token_seqs set), num_seqs * num_kv_heads workgroups.
template <typename T, bool F8 = false>
hipError_t launch_varlen_fused_typed(PrefillArgs p, const RowsArgs& r, int block_shift, uint32_t prefill_wgs,
                                     hipStream_t stream) {
  p.rank_major = prefill_wgs <= kFusedRankMajorWgs;
  const uint64_t wgs = (uint64_t)prefill_wgs + ((uint64_t)r.num_seqs * r.num_kv_heads + 7) / 8 * 8;
  if (wgs > 0xffffffffull) return hipErrorInvalidValue;
  const dim3 grid((uint32_t)wgs), block(kPrefillThreads);
  if (p.merge && p.alibi != nullptr)
    hipLaunchKernelGGL((varlen_fused_kernel<T, true, true, F8>), grid, block, 0, stream, p, r, block_shift, prefill_wgs);
  else if (p.merge)
    hipLaunchKernelGGL((varlen_fused_kernel<T, false, true, F8>), grid, block, 0, stream, p, r, block_shift, prefill_wgs);
  else if (p.alibi != nullptr)
    hipLaunchKernelGGL((varlen_fused_kernel<T, true, false, F8>), grid, block, 0, stream, p, r, block_shift, prefill_wgs);
  else
    hipLaunchKernelGGL((varlen_fused_kernel<T, false, false, F8>), grid, block, 0, stream, p, r, block_shift, prefill_wgs);
  return hipGetLastError();
}

}  // namespace pa
