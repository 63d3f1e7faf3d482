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

// Combine per-tile (max, sum exp, best non-mask logit, its id) in tile order.
PS_DEV void combine_stats(const float* st, int tiles, float* conf, int* yhat) {
  float M = -INFINITY;
  for (int t = 0; t < tiles; ++t) M = fmaxf(M, st[t * 4 + 0]);
  float Z = 0.f, best = -INFINITY;
  int bid = -1;
  for (int t = 0; t < tiles; ++t) {
    Z += st[t * 4 + 1] * expf(st[t * 4 + 0] - M);
    if (st[t * 4 + 2] > best) {
      best = st[t * 4 + 2];
      bid = __float_as_int(st[t * 4 + 3]);
    }
  }
  *conf = expf(best - M) / Z;
  *yhat = bid;
}

__global__ __launch_bounds__(64) void decide_kernel(DecideArgs a, const int32_t* meta_rows, const int32_t* meta_p0) {
  const int b = blockIdx.x, lane = threadIdx.x;
  const int H = a.hist > 0 ? a.hist : 1;
  for (int j = lane; j < a.block; j += 64) {
    float c;
    int y;
    combine_stats(a.lm_stats + ((int64_t)b * a.lm_rows + j) * a.lm_tiles * 4, a.lm_tiles, &c, &y);
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
    float c;
    int y;
    combine_stats(a.lm_stats + ((int64_t)b * a.lm_rows + a.block + i) * a.lm_tiles * 4, a.lm_tiles, &c, &y);
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
  hipLaunchKernelGGL(decide_kernel, dim3(a.batch), dim3(64), 0, s, a, a.meta, a.meta + a.batch);
  return hipGetLastError();
}

template hipError_t launch_lm_prep<float>(const LmPrepArgs&, hipStream_t);
template hipError_t launch_lm_prep<bf16_t>(const LmPrepArgs&, hipStream_t);
