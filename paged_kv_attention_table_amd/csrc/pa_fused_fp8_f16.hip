// The fused varlen kernel (prefill tiles + decode rows) over fp8 (E4M3) pools, F16
// queries.
#include "pa_varlen_fused.h"

namespace pa {

hipError_t launch_varlen_fused_fp8_f16(const PrefillArgs& p, const RowsArgs& r, int block_shift,
                                      uint32_t prefill_wgs, hipStream_t stream) {
  return launch_varlen_fused_typed<F16, true>(p, r, block_shift, prefill_wgs, stream);
}

}  // namespace pa
