// KV-cache staleness E_i of every position against recomputed K/V rows (the
// App. C.2 measure of the Polestar page): one minus the mean of the K and V
// cosine similarities, each averaged over the KV heads.  A zero row has cosine
// 0 with any row.  Measurement only: it reads two caches and writes one float
// per position.
//
// Workgroup = 64 consecutive positions x 4 heads at a time: a thread takes one
// (position, head) pair, so the transposed V cache ([Hkv][dh][n]) is read with
// consecutive positions in consecutive lanes, and a K row (dh contiguous
// values) is one thread's run of 16-byte loads.
#include "kernels.h"

namespace {

template <typename T>
__global__ __launch_bounds__(256) void kv_staleness_kernel(StaleArgs a) {
  __shared__ float red[2][4][64];
  const int p = threadIdx.x & 63, hh = threadIdx.x >> 6;
  const int i = blockIdx.x * 64 + p, b = blockIdx.y;
  const int n = a.n_pos, H = a.hkv, dh = a.dh;
  float ck = 0.f, cv = 0.f;
  if (i < n) {
    const T* kc = (const T*)a.k + ((int64_t)b * n + i) * H * dh;
    const T* kr = (const T*)a.k_ref + ((int64_t)b * n + i) * H * dh;
    for (int h = hh; h < H; h += 4) {
      float dk = 0.f, nk = 0.f, nkr = 0.f, dv = 0.f, nv = 0.f, nvr = 0.f;
      for (int j = 0; j < dh; j += 4) {
        float x[4], y[4];
        Quad<T>::load(kc + h * dh + j, x);
        Quad<T>::load(kr + h * dh + j, y);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dk += x[e] * y[e];
          nk += x[e] * x[e];
          nkr += y[e] * y[e];
        }
      }
      const int64_t v0 = (((int64_t)b * H + h) * dh) * n + i;
      for (int j = 0; j < dh; ++j) {
        const float x = St<T>::load((const T*)a.v, v0 + (int64_t)j * n);
        const float y = St<T>::load((const T*)a.v_ref, v0 + (int64_t)j * n);
        dv += x * y;
        nv += x * x;
        nvr += y * y;
      }
      ck += (nk > 0.f && nkr > 0.f) ? dk / sqrtf(nk * nkr) : 0.f;
      cv += (nv > 0.f && nvr > 0.f) ? dv / sqrtf(nv * nvr) : 0.f;
    }
  }
  red[0][hh][p] = ck;
  red[1][hh][p] = cv;
  __syncthreads();
  if (hh == 0 && i < n) {
    const float sk = (red[0][0][p] + red[0][1][p]) + (red[0][2][p] + red[0][3][p]);
    const float sv = (red[1][0][p] + red[1][1][p]) + (red[1][2][p] + red[1][3][p]);
    a.stale[(int64_t)b * n + i] = 1.f - 0.5f * (sk / (float)H + sv / (float)H);
  }
}

}  // namespace

template <typename T>
hipError_t launch_kv_staleness(const StaleArgs& a, hipStream_t s) {
  if (a.dh % 4) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kv_staleness_kernel<T>, dim3(PS_CEIL_DIV(a.n_pos, 64), a.batch), dim3(256), 0, s, a);
  return hipGetLastError();
}

template hipError_t launch_kv_staleness<float>(const StaleArgs&, hipStream_t);
template hipError_t launch_kv_staleness<bf16_t>(const StaleArgs&, hipStream_t);
