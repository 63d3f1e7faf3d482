// Instantiations of the weight-streaming projection for workgroup shape DL_W192: 2 x 4 waves of 48 columns, hi/lo planes.
#include "gemm_dl_impl.h"

hipError_t dl_launch_w192(const DlArgs& g, int max_rows, hipStream_t s) {
  return dl_impl::launch_shape<2, 4, 3, 2>(g, max_rows, s);
}
