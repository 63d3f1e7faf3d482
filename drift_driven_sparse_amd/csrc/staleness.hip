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

// Most-attended-token cosine change of one query row (the comparison policy of the drift
// ablation on the Polestar page, Fig. 6(a)): workgroup = (row, sequence), thread t owns keys
// t + 256 i.  Per query head the logits q.k/sqrt(dh) of the owned keys, the head's softmax
// (block max and sum), and the head-mean probability accumulated per key; then the argmax over
// keys (largest value, lowest position on ties) and, for that position, one minus the mean over
// KV heads of cos(k, k_ref) (0 for a zero row).  float32 throughout.
template <typename T, int PER>
__global__ __launch_bounds__(256) void attended_change_kernel(AttendArgs a) {
  extern __shared__ float qs[];          // [hq * dh]
  __shared__ float red[4];
  __shared__ float bv[4];
  __shared__ int bj[4];
  const int r = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int n = a.n_pos, dh = a.dh, hq = a.hq, hkv = a.hkv;
  const float* qr = a.q + (int64_t)b * a.q_bstride + (int64_t)r * a.q_ld;
  for (int i = tid; i < hq * dh; i += 256) qs[i] = qr[i];
  __syncthreads();
  const T* kc = (const T*)a.k + (int64_t)b * n * hkv * dh;
  const float scale = 1.f / sqrtf((float)dh);
  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
  for (int h = 0; h < hq; ++h) {
    const int g = (h * hkv) / hq;
    const float* qh = qs + h * dh;
    float lg[PER];
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int j = tid + 256 * i;
      lg[i] = -INFINITY;
      if (j < n) {
        const T* kr = kc + ((int64_t)j * hkv + g) * dh;
        float dot = 0.f;
        for (int e = 0; e < dh; e += 4) {
          float x[4];
          Quad<T>::load(kr + e, x);
          dot += (qh[e] * x[0] + qh[e + 1] * x[1]) + (qh[e + 2] * x[2] + qh[e + 3] * x[3]);
        }
        lg[i] = dot * scale;
        m = fmaxf(m, lg[i]);
      }
    }
    m = wave_max(m);
    __syncthreads();
    if (lane == 0) red[wid] = m;
    __syncthreads();
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    float z = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      lg[i] = (tid + 256 * i < n) ? expf(lg[i] - m) : 0.f;
      z += lg[i];
    }
    z = block_sum(z, red);
    const float inv = 1.f / z;
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[i] += lg[i] * inv;
  }
  // argmax of the head sums (the head mean orders the same way)
  float best = -INFINITY;
  int bjx = n;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int j = tid + 256 * i;
    if (j < n && acc[i] > best) { best = acc[i]; bjx = j; }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(best, o, 64);
    const int oj = __shfl_xor(bjx, o, 64);
    if (ov > best || (ov == best && oj < bjx)) { best = ov; bjx = oj; }
  }
  if (lane == 0) { bv[wid] = best; bj[wid] = bjx; }
  __syncthreads();
  best = bv[0];
  bjx = bj[0];
  for (int w = 1; w < 4; ++w)
    if (bv[w] > best || (bv[w] == best && bj[w] < bjx)) { best = bv[w]; bjx = bj[w]; }
  // cosine change of the chosen position's keys: one wave, lanes over KV heads
  if (wid == 0) {
    float cs = 0.f;
    if (bjx < n) {
      const T* k0 = kc + (int64_t)bjx * hkv * dh;
      const T* k1 = (const T*)a.k_ref + ((int64_t)b * n + bjx) * hkv * dh;
      for (int g = lane; g < hkv; g += 64) {
        float d = 0.f, n0 = 0.f, n1 = 0.f;
        for (int e = 0; e < dh; e += 4) {
          float x[4], y[4];
          Quad<T>::load(k0 + g * dh + e, x);
          Quad<T>::load(k1 + g * dh + e, y);
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            d += x[t] * y[t];
            n0 += x[t] * x[t];
            n1 += y[t] * y[t];
          }
        }
        cs += (n0 > 0.f && n1 > 0.f) ? d / sqrtf(n0 * n1) : 0.f;
      }
    }
    cs = wave_sum(cs);
    if (lane == 0) {
      a.top[(int64_t)b * a.rows + r] = bjx < n ? bjx : -1;
      a.score[(int64_t)b * a.rows + r] = 1.f - cs / (float)hkv;
    }
  }
}

}  // namespace

template <typename T>
hipError_t launch_attended_change(const AttendArgs& a, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  if (a.dh % 4 || a.n_pos > kMaxPos || a.hq % a.hkv || (size_t)a.hq * a.dh * 4 > 64 * 1024)
    return hipErrorInvalidValue;
  const dim3 grid(a.rows, a.batch);
  const size_t sm = (size_t)a.hq * a.dh * 4;
  if (a.n_pos <= 1024) hipLaunchKernelGGL((attended_change_kernel<T, 4>), grid, dim3(256), sm, s, a);
  else if (a.n_pos <= 2048) hipLaunchKernelGGL((attended_change_kernel<T, 8>), grid, dim3(256), sm, s, a);
  else hipLaunchKernelGGL((attended_change_kernel<T, 16>), grid, dim3(256), sm, s, a);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_kv_staleness(const StaleArgs& a, hipStream_t s) {
  if (a.dh % 4) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kv_staleness_kernel<T>, dim3(PS_CEIL_DIV(a.n_pos, 64), a.batch), dim3(256), 0, s, a);
  return hipGetLastError();
}

template hipError_t launch_kv_staleness<float>(const StaleArgs&, hipStream_t);
template hipError_t launch_kv_staleness<bf16_t>(const StaleArgs&, hipStream_t);
template hipError_t launch_attended_change<float>(const AttendArgs&, hipStream_t);
template hipError_t launch_attended_change<bf16_t>(const AttendArgs&, hipStream_t);
