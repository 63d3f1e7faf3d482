// Polestar-Commit kernels: staging of the confidence rows (active block and the
// suffix rows of the final update packet), combination of the per-tile softmax
// statistics produced by the LM-head projection, and the commit rule.
#include "kernels.h"

namespace {

template <typename T>
__global__ __launch_bounds__(256) void lm_prep_kernel(LmPrepArgs a, int32_t* meta_rows, int32_t* meta_p0) {
  __shared__ float red[4];
  __shared__ int p0_sh, cnt_sh;
  const int r = blockIdx.x, b = blockIdx.y, d = a.d;
  if (threadIdx.x == 0) {
    int cnt = a.h_full ? a.n_suf : (a.u_count ? a.u_count[b] : 0);
    cnt = cnt < 0 ? 0 : (cnt > a.win_max ? a.win_max : cnt);
    int p0 = 0;
    if (!a.h_full)
      while (p0 < cnt && a.u_idx[(int64_t)b * a.win_max + p0] < a.n_pre) ++p0;
    p0_sh = p0;
    cnt_sh = cnt;
    if (r == 0) {
      meta_rows[b] = a.block + (cnt - p0);
      meta_p0[b] = p0;
    }
  }
  __syncthreads();
  const T* src;
  if (a.h_full) {
    // block entry: the active rows, then the suffix rows, read at their positions
    if (r >= a.block + cnt_sh) return;
    src = (const T*)a.h_full + ((int64_t)b * a.n_pos + a.blk_start + r) * d;
  } else if (r < a.block) {
    src = (const T*)a.h_final + ((int64_t)b * a.block + r) * d;
  } else {
    const int j = p0_sh + (r - a.block);
    if (j >= cnt_sh) return;
    src = (const T*)a.u_rows + ((int64_t)b * a.win_max + j) * d;
  }
  T* dst = (T*)a.a_lm + ((int64_t)b * a.lm_rows + r) * d;
  rmsnorm_row<T>(src, d, a.eps, red, [&](int n, const float* x) { Quad<T>::store(dst + n, x); });
}

// Confidence and argmax of one staged row from the LM head's per-tile statistics (max, sum of
// exp(logit - max), best non-mask logit, its id): one workgroup per (row, sequence), thread t
// combines tiles t, t + 256, ... in order, then the threads' partials are combined in thread
// order (the maximum first, then the rescaled sums; the best logit with the lowest id on ties).
__global__ __launch_bounds__(256) void lm_conf_kernel(DecideArgs a, const int32_t* meta_rows) {
  __shared__ float rm[4], rz[4], rb[4];
  __shared__ int ri[4];
  const int r = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  if (r >= meta_rows[b]) return;   // uniform: rows staged for this sequence
  const float* st = a.lm_stats + ((int64_t)b * a.lm_rows + r) * a.lm_tiles * 4;
  float m = -INFINITY;
  for (int t = tid; t < a.lm_tiles; t += 256) m = fmaxf(m, st[t * 4 + 0]);
  m = wave_max(m);
  if (lane == 0) rm[wid] = m;
  __syncthreads();
  const float M = fmaxf(fmaxf(rm[0], rm[1]), fmaxf(rm[2], rm[3]));
  float z = 0.f, best = -INFINITY;
  int bid = -1;
  for (int t = tid; t < a.lm_tiles; t += 256) {
    const float4 v = *(const float4*)(st + t * 4);
    z += v.y * expf(v.x - M);
    if (v.z > best) {   // tiles ascend: the first maximum has the lowest id
      best = v.z;
      bid = __float_as_int(v.w);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    z += __shfl_xor(z, o, 64);
    const float ob = __shfl_xor(best, o, 64);
    const int oi = __shfl_xor(bid, o, 64);
    if (ob > best || (ob == best && oi >= 0 && (bid < 0 || oi < bid))) {
      best = ob;
      bid = oi;
    }
  }
  if (lane == 0) {
    rz[wid] = z;
    rb[wid] = best;
    ri[wid] = bid;
  }
  __syncthreads();
  if (tid == 0) {
    float Z = 0.f, B = -INFINITY;
    int I = -1;
    for (int w = 0; w < 4; ++w) {
      Z += rz[w];
      if (rb[w] > B || (rb[w] == B && ri[w] >= 0 && (I < 0 || ri[w] < I))) {
        B = rb[w];
        I = ri[w];
      }
    }
    const int64_t o = (int64_t)b * a.lm_rows + r;
    a.lm_conf[o] = expf(B - M) / Z;
    a.lm_yhat[o] = I;
  }
}

__global__ __launch_bounds__(64) void decide_kernel(DecideArgs a, const int32_t* meta_rows, const int32_t* meta_p0) {
  const int b = blockIdx.x, lane = threadIdx.x;
  const int H = a.hist > 0 ? a.hist : 1;
  for (int j = lane; j < a.block; j += 64) {
    const float c = a.lm_conf[(int64_t)b * a.lm_rows + j];
    const int y = a.lm_yhat[(int64_t)b * a.lm_rows + j];
    const int64_t row = (int64_t)b * a.block + j;
    if (a.entry) {   // no drift at block entry: the confidence alone decides
      a.commit_active[row] = (a.active_masked[row] != 0 && c >= a.tau_s) ? 1 : 0;
      a.conf_active[row] = c;
      a.yhat_active[row] = y;
      continue;
    }
    float* hv = a.hist_vals + row * H;
    const int cnt = a.hist_cnt[row];
    float mean = 0.f;
    if (cnt > 0) {
      float acc = 0.f;
      for (int i = 0; i < cnt; ++i) acc = __fadd_rn(acc, hv[i]);
      mean = __fdiv_rn(acc, (float)cnt);
    }
    const float dl = a.delta[row];
    const float sp = __fsub_rn(dl, mean);
    const float t = __fsub_rn(a.tau_s, c);
    const float taud = __fmul_rn(a.alpha, __fmul_rn(t, t));
    const bool masked = a.active_masked[row] != 0;
    a.commit_active[row] = (masked && (c >= a.tau_s || sp > taud)) ? 1 : 0;
    a.conf_active[row] = c;
    a.yhat_active[row] = y;
    a.spike[row] = sp;
    if (a.hist > 0) {
      if (cnt < a.hist) {
        hv[cnt] = dl;
        a.hist_cnt[row] = cnt + 1;
      } else {
        for (int i = 0; i + 1 < a.hist; ++i) hv[i] = hv[i + 1];
        hv[a.hist - 1] = dl;
      }
    }
  }
  for (int s = lane; s < a.win_suffix; s += 64) {
    a.commit_suffix[(int64_t)b * a.win_suffix + s] = 0;
    a.conf_suffix[(int64_t)b * a.win_suffix + s] = 0.f;
  }
  __syncthreads();
  const int nsuf = meta_rows[b] - a.block, p0 = meta_p0[b];
  for (int i = lane; i < nsuf; i += 64) {
    const float c = a.lm_conf[(int64_t)b * a.lm_rows + a.block + i];
    const int slot = a.entry ? i : a.u_idx[(int64_t)b * a.win_max + p0 + i] - a.n_pre;
    if (slot < 0 || slot >= a.win_suffix) continue;
    const int64_t o = (int64_t)b * a.win_suffix + slot;
    a.conf_suffix[o] = c;
    a.commit_suffix[o] = (a.suffix_masked[o] != 0 && c >= a.tau_suf) ? 1 : 0;
  }
}

}  // namespace

template <typename T>
hipError_t launch_lm_prep(const LmPrepArgs& a, hipStream_t s) {
  int32_t* meta_rows = a.meta;
  int32_t* meta_p0 = a.meta + a.batch;
  hipLaunchKernelGGL(lm_prep_kernel<T>, dim3(a.lm_rows, a.batch), dim3(256), 0, s, a, meta_rows, meta_p0);
  return hipGetLastError();
}

hipError_t launch_decide(const DecideArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(lm_conf_kernel, dim3(a.lm_rows, a.batch), dim3(256), 0, s, a, a.meta);
  hipLaunchKernelGGL(decide_kernel, dim3(a.batch), dim3(64), 0, s, a, a.meta, a.meta + a.batch);
  return hipGetLastError();
}

template hipError_t launch_lm_prep<float>(const LmPrepArgs&, hipStream_t);
template hipError_t launch_lm_prep<bf16_t>(const LmPrepArgs&, hipStream_t);
