// Tiled MFMA prefill kernel over fp8 (E4M3) pools, F16 queries.
#include "pa_prefill.h"

namespace pa {

hipError_t launch_prefill_fp8_f16(const PrefillArgs& a, int dk, int dv, dim3 grid, hipStream_t stream) {
  return launch_prefill_typed<F16, true>(a, dk, dv, grid, stream);
}

}  // namespace pa
