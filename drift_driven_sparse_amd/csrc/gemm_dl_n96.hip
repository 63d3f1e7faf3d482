// Instantiations of the weight-streaming projection for workgroup shape DL_N96: 4 x 2 waves of 48 columns, one bf16 plane.
#include "gemm_dl_impl.h"

hipError_t dl_launch_n96(const DlArgs& g, int max_rows, hipStream_t s) {
  return dl_impl::launch_shape<4, 2, 3, 1>(g, max_rows, s);
}
