// Instantiations of the weight-streaming projection for workgroup shape DL_NARROW: 3 x 2 waves of 64 columns, one bf16 plane.
#include "gemm_dl_impl.h"

hipError_t dl_launch_narrow(const DlArgs& g, int max_rows, hipStream_t s) {
  return dl_impl::launch_shape<3, 2, 4, 1>(g, max_rows, s);
}
