// BF16 instantiations of the tiled MFMA prefill kernel.
#include "pa_prefill.h"

namespace pa {

hipError_t launch_prefill_bf16(const PrefillArgs& a, int dk, int dv, dim3 grid, hipStream_t stream) {
  return launch_prefill_typed<BF16>(a, dk, dv, grid, stream);
}

}  // namespace pa
