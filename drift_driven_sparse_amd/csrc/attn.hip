// Attention of the active, window and centroid (proxy) query rows over every
// key position, the KL drift of proxy and active rows against the previous
// step's logits, and the top-k cluster selection.
//
// One workgroup handles kRG query rows of one head of one sequence.  It stages
// K (then V) in 32-key chunks through LDS, keeps all logits of its rows in LDS,
// and reduces softmax statistics and KL sums with wavefront shuffles.
#include "kernels.h"

namespace {

constexpr int kRG = 8;      // query rows per workgroup
constexpr int kKC = 32;     // keys per LDS chunk

// KL(softmax(s) || softmax(sp)) over n logits held by one wavefront (s in LDS, sp in
// global), evaluated through the logit differences so that the result keeps its
// relative accuracy when the two distributions are close:
//   u_j = exp(sp_j - max sp), e_j = (s_j - sp_j) - mean_u(s - sp),
//   S0 = sum u, S1 = sum u expm1(e), S2 = sum u exp(e) e,
//   KL = (S2/S0) / (1 + S1/S0) - log1p(S1/S0)   (invariant to the shift of e).
PS_DEV float wave_kl(const float* s, const float* sp, int n, int lane) {
  float mp = -INFINITY;
  for (int j = lane; j < n; j += 64) mp = fmaxf(mp, sp[j]);
  mp = wave_max(mp);
  float s0 = 0.f, sd = 0.f;
  for (int j = lane; j < n; j += 64) {
    const float u = expf(sp[j] - mp);
    s0 += u;
    sd += u * (s[j] - sp[j]);
  }
  s0 = wave_sum(s0);
  sd = wave_sum(sd);
  const float dbar = sd / s0;
  float s1 = 0.f, s2 = 0.f;
  for (int j = lane; j < n; j += 64) {
    const float u = expf(sp[j] - mp);
    const float e = (s[j] - sp[j]) - dbar;
    s1 += u * expm1f(e);
    s2 += u * expf(e) * e;
  }
  s1 = wave_sum(s1);
  s2 = wave_sum(s2);
  const float r1 = s1 / s0;
  return (s2 / s0) / (1.f + r1) - log1pf(r1);
}

template <typename T, int DH>
__global__ __launch_bounds__(256) void attn_kernel(AttnArgs a) {
  extern __shared__ float smem[];
  float* qs = smem;                       // [kRG][DH]
  float* kv = qs + kRG * DH;              // [kKC][DH + 1]
  float* sc = kv + kKC * (DH + 1);        // [kRG][n]
  __shared__ float rinv[kRG];

  const int n = a.n_pos;
  const int rg = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int nrows = a.n_tok + a.n_proxy;
  const int r0 = rg * kRG;
  const int nr = min(kRG, nrows - r0);
  if (nr <= 0) return;
  const int g = (h * a.hkv) / a.hq;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ldkv = a.hkv * DH;
  const T* kc = (const T*)a.kc + (int64_t)b * n * ldkv + g * DH;
  const T* vc = (const T*)a.vc + (int64_t)b * n * ldkv + g * DH;
  const float scale = 1.f / sqrtf((float)DH);

  // query rows [active; window; centroids] are float32 projections (never stored)
  for (int i = tid; i < kRG * DH; i += blockDim.x) {
    const int rr = i / DH, dd = i % DH;
    qs[i] = rr < nr ? a.q[((int64_t)b * a.mq + r0 + rr) * (a.hq * DH) + h * DH + dd] : 0.f;
  }
  // logits
  for (int c0 = 0; c0 < n; c0 += kKC) {
    const int nk = min(kKC, n - c0);
    __syncthreads();
    for (int i = tid; i < kKC * DH; i += blockDim.x) {
      const int j = i / DH, dd = i % DH;
      kv[j * (DH + 1) + dd] = j < nk ? St<T>::load(kc, (int64_t)(c0 + j) * ldkv + dd) : 0.f;
    }
    __syncthreads();
    for (int i = tid; i < kRG * kKC; i += blockDim.x) {
      const int rr = i / kKC, j = i % kKC;
      if (rr < nr && j < nk) {
        const float* qr = qs + rr * DH;
        const float* kr = kv + j * (DH + 1);
        float acc = 0.f;
#pragma unroll 8
        for (int dd = 0; dd < DH; ++dd) acc = fmaf(qr[dd], kr[dd], acc);
        sc[rr * n + c0 + j] = acc * scale;
      }
    }
  }
  __syncthreads();
  // softmax statistics, drift of proxy / active rows, logits for the next step
  for (int rr = wave; rr < nr; rr += 4) {
    const int row = r0 + rr;
    const float* s = sc + rr * n;
    float m = -INFINITY;
    for (int j = lane; j < n; j += 64) m = fmaxf(m, s[j]);
    m = wave_max(m);
    float z = 0.f;
    for (int j = lane; j < n; j += 64) z += expf(s[j] - m);
    z = wave_sum(z);
    if (lane == 0) rinv[rr] = 1.f / z;
    float* prev = nullptr;
    float* klout = nullptr;
    bool do_kl = false;
    if (row >= a.n_tok) {
      const int c = row - a.n_tok;
      prev = a.proxy_logits + (((int64_t)b * a.n_proxy + c) * a.hq + h) * n;
      klout = a.kl + ((int64_t)b * a.n_proxy + c) * a.hq + h;
      do_kl = true;
    } else if (row < a.block && a.act_logits) {
      prev = a.act_logits + (((int64_t)b * a.block + row) * a.hq + h) * n;
      klout = a.akl + ((int64_t)b * a.block + row) * a.hq + h;
      do_kl = a.act_kl != 0;
    }
    if (prev) {
      if (do_kl) {
        const float kl = wave_kl(s, prev, n, lane);
        if (lane == 0) *klout = kl;
      }
      for (int j = lane; j < n; j += 64) prev[j] = s[j];
    }
    // unnormalised probabilities replace the logits of this row
    float* sw = sc + rr * n;
    for (int j = lane; j < n; j += 64) sw[j] = expf(sw[j] - m);
  }
  __syncthreads();
  // outputs of token rows: o = sum_j p_j v_j
  const int n_out_rows = max(0, min(nr, a.n_tok - r0));
  if (n_out_rows == 0) return;
  constexpr int RPT = kRG * DH / 256;      // outputs per thread
  float acc[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) acc[i] = 0.f;
  for (int c0 = 0; c0 < n; c0 += kKC) {
    const int nk = min(kKC, n - c0);
    __syncthreads();
    for (int i = tid; i < kKC * DH; i += blockDim.x) {
      const int j = i / DH, dd = i % DH;
      kv[j * (DH + 1) + dd] = j < nk ? St<T>::load(vc, (int64_t)(c0 + j) * ldkv + dd) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int o = tid + i * 256;
      const int rr = o / DH, dd = o % DH;
      if (rr < n_out_rows) {
        const float* p = sc + rr * n + c0;
        float t = acc[i];
        for (int j = 0; j < nk; ++j) t = fmaf(p[j], kv[j * (DH + 1) + dd], t);
        acc[i] = t;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int o = tid + i * 256;
    const int rr = o / DH, dd = o % DH;
    if (rr < n_out_rows) {
      const int row = r0 + rr;
      const float v = acc[i] * rinv[rr];
      const int64_t off = ((int64_t)b * a.mt + row) * (a.hq * DH) + h * DH + dd;
      if (a.chk) a.chk[((int64_t)b * a.chk_rows + row) * (a.hq * DH) + h * DH + dd] = v;
      ((float*)a.o)[off] = v;
    }
  }
}

// Per sequence: D_c = sum_h max(0, KL_{c,h}) (heads in order); top-k clusters by
// (D desc, index asc); S = window rows whose label is selected, ascending; and the
// per-row active drift delta_j = sum_h max(0, KL_{j,h}).
__global__ __launch_bounds__(64) void topk_kernel(TopkArgs a) {
  __shared__ float D[16];
  __shared__ int chosen[16];
  const int b = blockIdx.x, lane = threadIdx.x;
  if (a.refresh) {
    const int keff = min(a.K, a.n_win);
    if (lane < a.K) {
      float s = 0.f;
      if (lane < keff)
        for (int h = 0; h < a.hq; ++h) s += fmaxf(0.f, a.kl[((int64_t)b * a.K + lane) * a.hq + h]);
      D[lane] = s;
      chosen[lane] = 0;
      if (a.D) a.D[(int64_t)b * a.K + lane] = s;
    }
    __syncthreads();
    if (lane == 0) {
      const int kk = min(a.k, keff);
      for (int t = 0; t < a.k; ++t) {
        int best = -1;
        if (t < kk) {
          for (int c = 0; c < keff; ++c)
            if (!chosen[c] && (best < 0 || D[c] > D[best])) best = c;
          chosen[best] = 1;
        }
        if (a.topk) a.topk[(int64_t)b * a.k + t] = best;
      }
    }
    __syncthreads();
    int base = 0;
    for (int w0 = 0; w0 < a.n_win; w0 += 64) {
      const int w = w0 + lane;
      int c = w < a.n_win ? a.win_m[(int64_t)b * a.win_max + w] : -1;
      const bool sel = c >= 0 && c < a.K && chosen[c];
      const unsigned long long m = __ballot(sel);
      const int before = __popcll(m & ((1ull << lane) - 1ull));
      if (sel) a.sel_idx[(int64_t)b * a.win_max + base + before] = w;
      base += __popcll(m);
    }
    if (lane == 0) a.sel_count[b] = base;
  } else {
    if (lane == 0) a.sel_count[b] = 0;
  }
  if (a.delta) {
    for (int j = lane; j < a.block; j += 64) {
      float s = 0.f;
      for (int h = 0; h < a.hq; ++h) s += fmaxf(0.f, a.akl[((int64_t)b * a.block + j) * a.hq + h]);
      a.delta[(int64_t)b * a.block + j] = s;
    }
  }
}

}  // namespace

template <typename T>
hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  const int nrows = a.n_tok + a.n_proxy;
  dim3 grid(PS_CEIL_DIV(nrows, kRG), a.hq, a.batch);
  if (a.dh == 64) {
    const size_t sm = (kRG * 64 + kKC * 65 + (size_t)kRG * a.n_pos) * sizeof(float);
    hipLaunchKernelGGL((attn_kernel<T, 64>), grid, dim3(256), sm, s, a);
  } else if (a.dh == 128) {
    const size_t sm = (kRG * 128 + kKC * 129 + (size_t)kRG * a.n_pos) * sizeof(float);
    hipLaunchKernelGGL((attn_kernel<T, 128>), grid, dim3(256), sm, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(topk_kernel, dim3(a.batch), dim3(64), 0, s, a);
  return hipGetLastError();
}

template hipError_t launch_attention<float>(const AttnArgs&, hipStream_t);
template hipError_t launch_attention<bf16_t>(const AttnArgs&, hipStream_t);
