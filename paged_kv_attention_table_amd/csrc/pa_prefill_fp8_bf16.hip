// Tiled MFMA prefill kernel over fp8 (E4M3) pools, BF16 queries.
#include "pa_prefill.h"

namespace pa {

hipError_t launch_prefill_fp8_bf16(const PrefillArgs& a, int dk, int dv, dim3 grid, hipStream_t stream) {
  return launch_prefill_typed<BF16, true>(a, dk, dv, grid, stream);
}

}  // namespace pa
