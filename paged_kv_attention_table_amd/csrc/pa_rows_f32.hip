// F32 instantiations of the per-row paged attention kernel.
#include "pa_rows.h"

namespace pa {

hipError_t launch_rows_f32(const RowsArgs& a, int dk, int dv, dim3 grid, hipStream_t stream) {
  return launch_rows_typed<F32>(a, dk, dv, grid, stream);
}

}  // namespace pa
