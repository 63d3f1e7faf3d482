// Instantiations of the weight-streaming projection for workgroup shape DL_X512: 1 x 8 waves of 64
// columns (512-column tiles), hi/lo planes, at most 128 rows per launch (each wave holds the
// accumulators of every row tile).
#include "gemm_dl_impl.h"

hipError_t dl_launch_x512(const DlArgs& g, int max_rows, hipStream_t s) {
  const int rtw = PS_CEIL_DIV(max_rows, 16);
  hipError_t e = hipErrorInvalidValue;
  [&]<int... R>(std::integer_sequence<int, R...>) {
    ((rtw == R + 1 ? (e = dl_impl::launch_cfg<bf16_t, R + 1, 1, 8, 4, 2>(g, s), 0) : 0), ...);
  }(std::make_integer_sequence<int, kDlSlabX512 / 16>{});
  return e;
}
