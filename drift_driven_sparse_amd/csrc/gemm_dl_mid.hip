// Instantiations of the weight-streaming projection for workgroup shape DL_MID: 2 x 2 waves of 64 columns, hi/lo planes.
#include "gemm_dl_impl.h"

hipError_t dl_launch_mid(const DlArgs& g, int max_rows, hipStream_t s) {
  return dl_impl::launch_shape<2, 2, 4, 2>(g, max_rows, s);
}
