// Instantiations of the weight-streaming projection for workgroup shape DL_P160: 2 x 5 waves of 32
// columns (160-column tiles), hi/lo planes; gate/up pairs stay inside a wave.
#include "gemm_dl_impl.h"

hipError_t dl_launch_p160(const DlArgs& g, int max_rows, hipStream_t s) {
  return dl_impl::launch_shape<2, 5, 2, 2>(g, max_rows, s);
}
