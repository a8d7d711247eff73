// BF16 instantiations of the MFMA decode kernel.
#include "pa_decode.h"

namespace pa {

hipError_t launch_decode_bf16(const RowsArgs& a, int block_shift, int dk, int dv, dim3 grid, hipStream_t stream) {
  return launch_decode_typed<BF16, false>(a, block_shift, dk, dv, grid, stream);
}

}  // namespace pa
