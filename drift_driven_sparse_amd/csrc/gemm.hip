// Weight packing, the float32 projections and the split-K row reduction.
//
// Weight packing: bf16 weights are repacked once into MFMA 16x16x32 B-operand
// fragments in lane order, grouped so that a workgroup's weights for one K step
// are contiguous (gemm_dl.hip streams them); float32 weights stay row-major.
//
// float32 path (small models): a workgroup owns 64 output columns of one
// sequence and a range of K; a plain FMA inner product per (row, column) into an
// LDS tile, then the fused epilogue (QKV, SwiGLU, next-layer K/V, LM-head
// statistics, or raw split-K partial sums).  Every bf16 projection runs on the
// weight-streaming kernel of gemm_dl.hip instead.
//
// Row reduction: the partial sums of the N = d projections (added in split
// order) plus the residual, and RMSNorm of the stored row for the next
// projection.
#include "kernels.h"

namespace {

constexpr int kNT = 64;          // output columns per workgroup
constexpr int kLDT = kNT + 4;    // LDS tile row stride (floats)

PS_HD int64_t gu_src_row(int64_t p, int ffn) {
  const int64_t sub = p >> 4, i = sub >> 1;
  return (sub & 1) * (int64_t)ffn + i * 16 + (p & 15);
}

// ---- weight packing -----------------------------------------------------------------
// bf16: fragment f = (n16/G * (K/32) + k32) * G + n16%G holds
//   dst[(f*64 + lane)*8 + e] = W'[n16*16 + lane%16][k32*32 + (lane/16)*8 + e]
// (subtiles past N are zero); f32: dst[n][k] = W'[n][k].
// W' = W with rows permuted for the gate/up weight (gate and up 16-row groups interleaved).
__global__ void pack_bf16_kernel(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst, int N, int K, int G,
                                 int is_gu, int ffn) {
  const int64_t c = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;   // one 8-element chunk
  const int64_t k32n = K >> 5;
  const int64_t groups = ((N >> 4) + G - 1) / G;
  if (c >= groups * G * k32n * 64) return;
  const int lane = (int)(c & 63);
  const int64_t f = c >> 6;
  const int64_t j = f % G, rest = f / G;
  const int64_t k32 = rest % k32n, n16 = (rest / k32n) * G + j;
  if (n16 >= (N >> 4)) {
    *(uint4*)(dst + c * 8) = make_uint4(0, 0, 0, 0);
    return;
  }
  const int64_t n = n16 * 16 + (lane & 15);
  const int64_t k = k32 * 32 + (lane >> 4) * 8;
  const int64_t row = is_gu ? gu_src_row(n, ffn) : n;
  *(uint4*)(dst + c * 8) = *(const uint4*)(src + row * K + k);
}

__global__ void pack_f32_kernel(const float* __restrict__ src, float* __restrict__ dst, int N, int K, int is_gu,
                                int ffn) {
  const int64_t c = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;   // one element
  if (c >= (int64_t)N * K) return;
  const int64_t n = c / K, k = c % K;
  const int64_t row = is_gu ? gu_src_row(n, ffn) : n;
  dst[c] = src[row * K + k];
}

// ---- epilogues ------------------------------------------------------------------------
template <typename T, int KIND>
PS_DEV void epilogue(const GemmArgs& g, const EpiParams& e, int b, int rows_b, int n0, int nt,
                     const float* tile) {
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int r0 = g.A.row0;   // tile row r is row r0 + r of the sequence
  if constexpr (KIND == EPI_PARTIAL) {
    float* out = g.part + (((int64_t)blockIdx.z * g.batch + b) * g.part_rows) * g.N;
    for (int idx = tid; idx < rows_b * kNT; idx += nthr) {
      const int r = idx / kNT, c = idx % kNT, n = n0 + c;
      if (n < g.N) out[(int64_t)(r0 + r) * g.N + n] = tile[r * kLDT + c];
    }
  } else if constexpr (KIND == EPI_QKV) {
    for (int idx = tid; idx < rows_b * kNT; idx += nthr) {
      const int r = idx / kNT, c = idx % kNT, n = n0 + c;
      if (n < g.N) epi_qkv_elem<T>(e, b, r0 + r, n, tile[r * kLDT + c]);
    }
  } else if constexpr (KIND == EPI_SWIGLU) {
    // tile columns: [gate 16 | up 16] x 2 pairs -> 32 output columns starting at n0/2
    for (int idx = tid; idx < rows_b * (kNT / 2); idx += nthr) {
      const int r = idx / (kNT / 2), j = idx % (kNT / 2);
      const int p = j >> 4, jj = j & 15;
      const int oc = (n0 >> 1) + j;
      if (oc >= e.ffn) continue;
      const float gv = tile[r * kLDT + (2 * p) * 16 + jj];
      const float uv = tile[r * kLDT + (2 * p + 1) * 16 + jj];
      St<T>::store((T*)e.act, ((int64_t)b * e.act_rows + r0 + r) * e.ffn + oc, gv / (1.f + expf(-gv)) * uv);
    }
  } else if constexpr (KIND == EPI_KV) {
    for (int idx = tid; idx < rows_b * kNT; idx += nthr) {
      const int r = idx / kNT, c = idx % kNT, n = n0 + c;
      if (n < g.N) epi_kv_elem<T>(e, b, r0 + r, n, tile[r * kLDT + c]);
    }
  } else if constexpr (KIND == EPI_LMSTAT) {
    // Per row, over this tile's vocabulary ids: max logit, sum exp(logit - max), and the
    // largest logit among ids != mask_id with its id (lowest id on ties).
    const int lane = tid & 63, wave = tid >> 6, nwave = nthr >> 6;
    for (int r = wave; r < rows_b; r += nwave) {
      const int n = n0 + lane;
      const bool valid = n < e.vocab;
      const float l = valid ? tile[r * kLDT + lane] : -INFINITY;
      const float m = wave_max(l);
      const float se = wave_sum(valid ? expf(l - m) : 0.f);
      const float lb = (valid && n != e.mask_id) ? l : -INFINITY;
      const float bm = wave_max(lb);
      const unsigned long long hit = __ballot(lb == bm && bm > -INFINITY);
      const int bid = hit ? n0 + __ffsll((long long)hit) - 1 : -1;
      if (lane == 0) {
        float* st = e.lm_stats + (((int64_t)b * e.lm_rows + r0 + r) * e.lm_tiles + nt) * 4;
        st[0] = m;
        st[1] = se;
        st[2] = bm;
        st[3] = __int_as_float(bid);
      }
    }
  }
}

// ---- float32 main loop ----------------------------------------------------------------------
template <int RT, int KIND>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs g, EpiParams e) {
  __shared__ float tile[RT * 16 * kLDT];
  const int b = blockIdx.x, nt = blockIdx.y, sp = blockIdx.z;
  int rows_b = g.A.rows(b) - g.A.row0;   // this launch's slab of rows
  if (rows_b > RT * 16) rows_b = RT * 16;
  if (rows_b <= 0) return;
  const int kc = g.K >> 2;
  const int c0 = (int)((int64_t)kc * sp / g.ksplit), c1 = (int)((int64_t)kc * (sp + 1) / g.ksplit);
  const float* Ab = (const float*)g.A.base + (int64_t)b * g.A.bstride;
  const float* W = (const float*)g.W;
  const int n0 = nt * kNT;
  for (int idx = threadIdx.x; idx < rows_b * kNT; idx += blockDim.x) {
    const int r = idx / kNT, c = idx % kNT, n = n0 + c;
    float acc = 0.f;
    if (n < g.N) {
      const float4* a4 = (const float4*)(Ab + g.A.src_row(b, g.A.row0 + r) * g.A.lda);
      const float4* w4 = (const float4*)(W + (int64_t)n * g.K);
      for (int k = c0; k < c1; ++k) {
        const float4 x = a4[k], y = w4[k];
        acc = fmaf(x.x, y.x, acc);
        acc = fmaf(x.y, y.y, acc);
        acc = fmaf(x.z, y.z, acc);
        acc = fmaf(x.w, y.w, acc);
      }
    }
    tile[r * kLDT + c] = acc;
  }
  __syncthreads();
  epilogue<float, KIND>(g, e, b, rows_b, n0, nt, tile);
}

template <typename T, int RT, int KIND>
hipError_t launch_one(const GemmArgs& g, const EpiParams& e, hipStream_t s) {
  dim3 grid(g.batch, PS_CEIL_DIV(g.N, kNT), g.ksplit);
  hipLaunchKernelGGL((gemm_f32_kernel<RT, KIND>), grid, dim3(256), 0, s, g, e);
  return hipGetLastError();
}

template <typename T, int RT>
hipError_t dispatch_kind(const GemmArgs& g, const EpiParams& e, hipStream_t s) {
  switch (e.kind) {
    case EPI_PARTIAL: return launch_one<T, RT, EPI_PARTIAL>(g, e, s);
    case EPI_QKV: return launch_one<T, RT, EPI_QKV>(g, e, s);
    case EPI_SWIGLU: return launch_one<T, RT, EPI_SWIGLU>(g, e, s);
    case EPI_KV: return launch_one<T, RT, EPI_KV>(g, e, s);
    case EPI_LMSTAT: return launch_one<T, RT, EPI_LMSTAT>(g, e, s);
  }
  return hipErrorInvalidValue;
}

// ---- split-K row reduction ------------------------------------------------------------------
// Workgroup = one row: partial sums (added in split order) + residual, kept as float32 or
// rounded to the storage dtype; rows from norm_from on also get RMSNorm of the stored row, the
// input of the next projection (bf16 hi/lo planes of the float32 value, or rounded to the
// storage dtype).  Each thread re-reads only the elements it stored itself.
template <typename T>
__global__ __launch_bounds__(1024) void row_reduce_kernel(RowReduceArgs a) {
  __shared__ float red[16];
  const int r = blockIdx.x, b = blockIdx.y;
  int rows_b = a.block + (a.count ? a.count[b] : 0);
  if (rows_b > (int)gridDim.x) rows_b = gridDim.x;
  if (r >= rows_b) return;
  const void* res;
  bool res32 = false;
  if (r < a.res_split) {
    res32 = a.res_a_f32 != 0;
    res = (const char*)a.res_a + ((int64_t)b * a.res_a_bstride + (int64_t)r * a.d) * (res32 ? 4 : sizeof(T));
  } else {
    int src = a.sel_idx[(int64_t)b * a.win_max + r - a.res_split];
    src = (src < 0 || src >= a.win_max) ? 0 : src;
    res = (const T*)a.res_b + (int64_t)b * a.res_b_bstride + (int64_t)src * a.d;
  }
  const int64_t ooff = (r < a.out_split) ? (int64_t)b * a.out_a_bstride + (int64_t)r * a.d
                                         : (int64_t)b * a.out_b_bstride + (int64_t)(r - a.out_split) * a.d;
  void* obase = (r < a.out_split) ? a.out_a : a.out_b;
  const int64_t pstride = (int64_t)a.batch * a.part_rows * a.d;
  const float* p = a.part + ((int64_t)b * a.part_rows + r) * a.d;
  float* chk = a.chk ? a.chk + ((int64_t)b * a.chk_rows + r) * a.d : nullptr;
  auto load_out = [&](int n, float* x) {
    if (a.out_f32) Quad<float>::load((const float*)obase + ooff + n, x);
    else Quad<T>::load((const T*)obase + ooff + n, x);
  };
  // the first RH quads of each thread stay in registers for the normalisation pass
  constexpr int RH = 2;
  const int step = 4 * blockDim.x;
  float xs[RH][4];
  auto reduce_quad = [&](int n, float* x) __attribute__((always_inline)) {
    const float4 v = sum_splits(p + n, pstride, a.ksplit);
    if (res32) Quad<float>::load((const float*)res + n, x);
    else Quad<T>::load((const T*)res + n, x);
    x[0] += v.x; x[1] += v.y; x[2] += v.z; x[3] += v.w;
    if (chk) *(float4*)(chk + n) = make_float4(x[0], x[1], x[2], x[3]);
    if (a.out_f32) {
      Quad<float>::store((float*)obase + ooff + n, x);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = St<T>::round(x[i]);
      Quad<T>::store((T*)obase + ooff + n, x);
    }
  };
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < RH; ++i) {
    const int n = 4 * threadIdx.x + i * step;
    if (n < a.d) {
      reduce_quad(n, xs[i]);
      ss += xs[i][0] * xs[i][0] + xs[i][1] * xs[i][1] + xs[i][2] * xs[i][2] + xs[i][3] * xs[i][3];
    }
  }
  for (int n = 4 * threadIdx.x + RH * step; n < a.d; n += step) {
    float x[4];
    reduce_quad(n, x);
    ss += x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3];
  }
  if (!a.norm || r < a.norm_from) return;   // uniform over the workgroup
  ss = block_sum(ss, red);
  const float inv = 1.f / sqrtf(ss / (float)a.d + a.eps);
  const int rn = r - a.norm_from;
  const int planes = a.norm_planes ? 2 : 1;
  auto norm_quad = [&](int n, float* x) __attribute__((always_inline)) {
    x[0] *= inv; x[1] *= inv; x[2] *= inv; x[3] *= inv;
    const int64_t o0 = (int64_t)b * a.norm_bstride +
                       (a.norm_tiles > 0 ? apack(rn, n, 0, planes, a.norm_tiles) : (int64_t)rn * a.d + n);
    if (a.norm_planes) {   // bf16 hi/lo planes (fragment-packed)
      const int64_t o1 = (int64_t)b * a.norm_bstride + apack(rn, n, 1, planes, a.norm_tiles);
      float hi[4], lo[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        hi[i] = St<bf16_t>::round(x[i]);
        lo[i] = x[i] - hi[i];
      }
      Quad<bf16_t>::store((bf16_t*)a.norm + o0, hi);
      Quad<bf16_t>::store((bf16_t*)a.norm + o1, lo);
    } else {
      Quad<T>::store((T*)a.norm + o0, x);
    }
  };
#pragma unroll
  for (int i = 0; i < RH; ++i) {
    const int n = 4 * threadIdx.x + i * step;
    if (n < a.d) norm_quad(n, xs[i]);
  }
  for (int n = 4 * threadIdx.x + RH * step; n < a.d; n += step) {
    float x[4];
    load_out(n, x);
    norm_quad(n, x);
  }
}

}  // namespace

size_t packed_elems(int N, int K, int G) {
  const size_t n16 = (size_t)(N >> 4);
  return G > 1 ? (n16 + G - 1) / G * G * 16 * (size_t)K : (size_t)N * (size_t)K;
}

template <typename T>
hipError_t launch_pack(int kind, const void* src, void* dst, int N, int K, int G, int ffn, hipStream_t s) {
  const int is_gu = kind == POLESTAR_W_GU;
  if constexpr (std::is_same<T, float>::value) {
    const int64_t total = (int64_t)N * K;
    hipLaunchKernelGGL(pack_f32_kernel, dim3((unsigned)PS_CEIL_DIV(total, 256)), dim3(256), 0, s,
                       (const float*)src, (float*)dst, N, K, is_gu, ffn);
  } else {
    const int64_t total = (int64_t)packed_elems(N, K, G) / 8;
    hipLaunchKernelGGL(pack_bf16_kernel, dim3((unsigned)PS_CEIL_DIV(total, 256)), dim3(256), 0, s,
                       (const uint16_t*)src, (uint16_t*)dst, N, K, G, is_gu, ffn);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_gemm(const GemmArgs& g, const EpiParams& e, int max_rows, hipStream_t s) {
  // float32 storage only: every bf16 projection runs on the weight-streaming kernel (gemm_dl)
  if constexpr (!std::is_same<T, float>::value) return hipErrorInvalidValue;
  if (g.A.row0 != 0) return hipErrorInvalidValue;
  // one launch per slab of at most kDlSlab rows
  for (int r0 = 0; r0 < max_rows; r0 += kDlSlab) {
    GemmArgs gs = g;
    gs.A.row0 = r0;
    const int mr = max_rows - r0 < kDlSlab ? max_rows - r0 : kDlSlab;
    hipError_t err;
    if (mr <= 32) err = dispatch_kind<T, 2>(gs, e, s);
    else if (mr <= 64) err = dispatch_kind<T, 4>(gs, e, s);
    else if (mr <= 144) err = dispatch_kind<T, 9>(gs, e, s);
    else err = dispatch_kind<T, 12>(gs, e, s);
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

template <typename T>
hipError_t launch_row_reduce(const RowReduceArgs& a, int max_rows, hipStream_t s) {
  if (max_rows <= 0) return hipSuccess;
  if (a.d % 4) return hipErrorInvalidValue;
  int threads = 64 * PS_CEIL_DIV(a.d / 4, 64);
  threads = threads > 1024 ? 1024 : threads;
  hipLaunchKernelGGL(row_reduce_kernel<T>, dim3(max_rows, a.batch), dim3(threads), 0, s, a);
  return hipGetLastError();
}

template hipError_t launch_pack<float>(int, const void*, void*, int, int, int, int, hipStream_t);
template hipError_t launch_pack<bf16_t>(int, const void*, void*, int, int, int, int, hipStream_t);
template hipError_t launch_gemm<float>(const GemmArgs&, const EpiParams&, int, hipStream_t);
template hipError_t launch_gemm<bf16_t>(const GemmArgs&, const EpiParams&, int, hipStream_t);
template hipError_t launch_row_reduce<float>(const RowReduceArgs&, int, hipStream_t);
template hipError_t launch_row_reduce<bf16_t>(const RowReduceArgs&, int, hipStream_t);
