// Instantiations of the MFMA decode kernel for fp8 (E4M3) pools read with F16 queries.
#include "pa_decode.h"

namespace pa {

hipError_t launch_decode_fp8_f16(const RowsArgs& a, int block_shift, int dk, int dv, dim3 grid, hipStream_t stream) {
  return launch_decode_typed<F16, true>(a, block_shift, dk, dv, grid, stream);
}

}  // namespace pa
