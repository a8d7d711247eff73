// F16 instantiations of the tiled MFMA prefill kernel.
#include "pa_prefill.h"

namespace pa {

hipError_t launch_prefill_f16(const PrefillArgs& a, int dk, int dv, dim3 grid, hipStream_t stream) {
  return launch_prefill_typed<F16>(a, dk, dv, grid, stream);
}

}  // namespace pa
