// Instantiations of the weight-streaming projection for workgroup shape DL_P96: 4 x 3 waves of 32 columns, hi/lo planes
// (each wave holds one gate/up subtile pair, so the SwiGLU epilogue runs in the kernel).
#include "gemm_dl_impl.h"

hipError_t dl_launch_p96(const DlArgs& g, int max_rows, hipStream_t s) {
  return dl_impl::launch_shape<4, 3, 2, 2>(g, max_rows, s);
}
