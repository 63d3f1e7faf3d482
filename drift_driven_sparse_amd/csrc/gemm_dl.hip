// Weight-streaming projections of the gathered rows for bf16 storage (gfx950).
//
// Per sequence a projection multiplies at most 144 rows by a large weight, so
// the kernel is organised around moving bytes: every 32-wide K step is one
// pipeline stage that holds the A fragments of all row tiles and the weight
// fragments of the workgroup.  Stages are filled by direct global -> LDS loads
// (global_load_lds_dwordx4, no VGPR staging) in a ring of P buffers (P = 4, or 3
// where four do not fit); stage s is consumed after a wait that leaves the P-2
// younger stages in flight and one workgroup barrier.  Each ring buffer is its own LDS object, which lets the
// compiler see that reads of one stage do not alias the loads still landing in
// the others.
//
// Waves form RG row groups x CG column groups: the CG waves of a row group read
// the same A fragments, the RG waves of a column group the same weight
// fragments.  Row tiles are dealt to the row groups in turn.  Shapes with RG = 2
// and CG = 4 give each SIMD one wave of each row group and the same number of
// matrix products; the 512-column shape (RG = 1, CG = 8) gives every wave all row
// tiles, for many sequences, where a stage's fixed cost is best spread over more
// products.  With hi/lo planes and real data the products are what the
// projection's time depends on once the stream is fed.  Fragments are 16x16x32 MFMA operands in lane order.  Weights are
// pre-packed in groups of subtiles so that a workgroup's weights for one step are
// one contiguous block and its whole range one contiguous stream.  A operands are
// fragment-packed by their producers (one contiguous block per step), except the
// output projection's, whose rows are gathered per lane through the row map.
// Both layouts keep the number of memory requests per step low: A fragments
// gathered row by row cost twice the requests of packed ones, and the requests a
// compute unit can keep in flight bound its share of the weight stream.
//
// float32 activations (the attention output, RMSNorm(h') and the SwiGLU product)
// arrive as two bf16 planes (hi = rn(x), lo = rn(x - hi)) written by their
// producers; both planes are multiplied into the same float32 accumulators.
//
// With split-K (grid.z > 1) the raw sums go to row-major partial buffers that a
// row kernel (O, down projections) or launch_dl_finish (QKV, gate/up, next-layer
// K/V) adds in split order.  Without split-K the QKV and SwiGLU epilogues run on the
// accumulators directly.
#include "gemm_dl_impl.h"

namespace {

// Split-K finish of the element-wise epilogues: sum the partials in split order.
template <typename T, int KIND>
__global__ __launch_bounds__(256) void dl_finish_kernel(DlArgs g) {
  const int r = blockIdx.y, b = blockIdx.z;
  int rows_b = g.A.rows(b);
  if (r >= rows_b) return;
  const int c = (blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (c >= g.N) return;
  const int64_t sstride = (int64_t)g.batch * g.part_rows * g.N;
  const float* p = g.part + ((int64_t)b * g.part_rows + r) * g.N + c;
  const float4 v = sum_splits(p, sstride, g.ksplit);
  const float vv[4] = {v.x, v.y, v.z, v.w};
  if constexpr (KIND == EPI_QKV) {
    // four columns of one kind (nq and nkv are multiples of 4): queries and keys are contiguous
    // in their outputs and take one store; values (transposed cache) go element by element
    const EpiParams& e = g.e;
    if (c < e.nq + e.nkv) {
      const QkvDest dst = qkv_dest(e, b, r);
      if (e.chk) *(float4*)(e.chk + ((int64_t)b * e.chk_rows + dst.row) * e.chk_ld + c) = v;
      if (c < e.nq) *(float4*)(dst.q + c) = v;
      else if (dst.pos >= 0) Quad<T>::store((T*)e.kc + kv_index(e, b, dst.pos, c - e.nq, 0), vv);
      return;
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (KIND == EPI_QKV) epi_qkv_elem<T>(g.e, b, r, c + i, vv[i]);
    else epi_kv_elem<T>(g.e, b, r, c + i, vv[i]);
  }
}

// Split-K finish of the gate/up projection: output column oc takes gate column
// 32*(oc/16) + oc%16 and the up column 16 after it (16-column groups interleaved).
__global__ __launch_bounds__(256) void dl_finish_swiglu_kernel(DlArgs g) {
  const int r = blockIdx.y, b = blockIdx.z;
  int rows_b = g.A.rows(b);
  if (r >= rows_b) return;
  const EpiParams& e = g.e;
  const int oc = (blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (oc >= e.ffn) return;
  const int cg = (oc >> 4) * 32 + (oc & 15);
  const int64_t sstride = (int64_t)g.batch * g.part_rows * g.N;
  const float* p = g.part + ((int64_t)b * g.part_rows + r) * g.N + cg;
  const float4 gv = sum_splits(p, sstride, g.ksplit), uv = sum_splits(p + 16, sstride, g.ksplit);
  const float ga[4] = {gv.x, gv.y, gv.z, gv.w}, ua[4] = {uv.x, uv.y, uv.z, uv.w};
  bf16_t* act = (bf16_t*)e.act + (int64_t)b * 2 * e.act_rows * e.ffn;
  float hi[4], lo[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a = ga[i] / (1.f + expf(-ga[i])) * ua[i];
    hi[i] = St<bf16_t>::round(a);
    lo[i] = a - hi[i];
  }
  Quad<bf16_t>::store(act + apack(r, oc, 0, 2, e.act_tiles), hi);
  Quad<bf16_t>::store(act + apack(r, oc, 1, 2, e.act_tiles), lo);
}

}  // namespace

int dl_subtiles_per_wave(int shape) {
  switch (shape) {
    case DL_N192: case DL_W192: case DL_N96: return 3;
    case DL_MID8: case DL_P96: case DL_P160: return 2;
    default: return 4;
  }
}

int dl_tile_cols(int shape) {
  switch (shape) {
    case DL_WIDE: return 256;
    case DL_X512: return 512;
    case DL_N192: case DL_W192: return 192;
    case DL_N96: case DL_P96: return 96;
    case DL_P160: return 160;
    default: return 128;
  }
}

template <typename T>
hipError_t launch_dl(const DlArgs& g, int shape, int max_rows, hipStream_t s) {
  if constexpr (!std::is_same<T, bf16_t>::value) {
    return hipErrorInvalidValue;
  } else {
    if (max_rows <= 0) return hipSuccess;
    if (g.A.row0 != 0) return hipErrorInvalidValue;
    if (g.K % 32 || g.N % 16 || g.ksplit < 1 || g.ksplit > (g.K >> 5)) return hipErrorInvalidValue;
    if (g.wg < 1 || g.wg % (dl_tile_cols(shape) / 16) != 0) return hipErrorInvalidValue;
    const bool one_plane = shape == DL_NARROW || shape == DL_N192 || shape == DL_N96;
    if (g.planes != (one_plane ? 1 : 2)) return hipErrorInvalidValue;
    // rows past one slab (192 rows, 128 for the 512-column shape) take further launches over
    // the same weights, one per slab
    const int slab = shape == DL_X512 ? kDlSlabX512 : kDlSlab;
    for (int r0 = 0; r0 < max_rows; r0 += slab) {
      DlArgs gs = g;
      gs.A.row0 = r0;
      const int mr = max_rows - r0 < slab ? max_rows - r0 : slab;
      hipError_t e;
      switch (shape) {
        case DL_NARROW: e = dl_launch_narrow(gs, mr, s); break;
        case DL_N192: e = dl_launch_n192(gs, mr, s); break;
        case DL_N96: e = dl_launch_n96(gs, mr, s); break;
        case DL_WIDE: e = dl_launch_wide(gs, mr, s); break;
        case DL_MID: e = dl_launch_mid(gs, mr, s); break;
        case DL_W192: e = dl_launch_w192(gs, mr, s); break;
        case DL_MID8: e = dl_launch_mid8(gs, mr, s); break;
        case DL_P96: e = dl_launch_p96(gs, mr, s); break;
        case DL_P160: e = dl_launch_p160(gs, mr, s); break;
        case DL_X512: e = dl_launch_x512(gs, mr, s); break;
        default: e = hipErrorInvalidValue;
      }
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
}

template <typename T>
hipError_t launch_dl_finish(const DlArgs& g, int max_rows, hipStream_t s) {
  if (max_rows <= 0 || g.ksplit <= 1) return hipSuccess;
  if (g.N % 4) return hipErrorInvalidValue;
  if (g.e.kind == EPI_SWIGLU) {
    if (g.e.ffn % 16) return hipErrorInvalidValue;
    hipLaunchKernelGGL(dl_finish_swiglu_kernel, dim3(PS_CEIL_DIV(g.e.ffn, 1024), max_rows, g.batch), dim3(256), 0, s, g);
    return hipGetLastError();
  }
  const dim3 grid(PS_CEIL_DIV(g.N, 1024), max_rows, g.batch);
  if (g.e.kind == EPI_QKV) hipLaunchKernelGGL((dl_finish_kernel<T, EPI_QKV>), grid, dim3(256), 0, s, g);
  else if (g.e.kind == EPI_KV) hipLaunchKernelGGL((dl_finish_kernel<T, EPI_KV>), grid, dim3(256), 0, s, g);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

template hipError_t launch_dl<float>(const DlArgs&, int, int, hipStream_t);
template hipError_t launch_dl<bf16_t>(const DlArgs&, int, int, hipStream_t);
template hipError_t launch_dl_finish<float>(const DlArgs&, int, hipStream_t);
template hipError_t launch_dl_finish<bf16_t>(const DlArgs&, int, hipStream_t);
