// Attention of the active, window and centroid (proxy) query rows over every
// key position; KL drift of proxy and active rows against the previous step's
// logits; top-k cluster selection.
//
// Cache layouts: K token-major [batch][n][Hkv][dh]; V transposed
// [batch][Hkv][dh][n] so that V^T fragments are contiguous along keys.
//
// bf16 path (attn_mfma_kernel): one workgroup = 32 query rows (two 16-row MFMA
// tiles) of one head; its four waves split the keys into interleaved 32-key
// blocks.  Per block a wave computes S^T = K Q^T with MFMA 16x16x32 (the
// float32 queries as a bf16 hi + lo pair), keeps an online softmax per row, and
// accumulates O^T += V^T P^T (probabilities as a bf16 hi + lo pair), so the
// result carries float32-level accuracy.  The four partial
// (max, sum, O) states are merged in LDS.  Logits of proxy rows and (when
// requested) active rows go to a staging buffer; kl_kernel then forms the KL
// drift against the previous logits and replaces them.
//
// float32 path (attn_f32_kernel, small models): LDS-staged vector FMA.
#include "kernels.h"

namespace {

constexpr int kRG = 8;      // f32 path: query rows per workgroup
constexpr int kKC = 32;     // f32 path: keys per LDS chunk

PS_DEV floatx4_t mfma(uint4 a, uint4 b, floatx4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

PS_DEV uint32_t pack2(float a, float b) { return (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16); }

// Row kinds of the query row list [active (block); window (n_win); centroids (n_proxy)].
PS_DEV bool row_keeps_logits(const AttnArgs& a, int row) {
  return row >= a.n_tok || (row < a.block && a.act_logits != nullptr);
}
PS_DEV int stage_row(const AttnArgs& a, int row) {   // staging buffer row: [proxies; active]
  return row >= a.n_tok ? row - a.n_tok : a.n_proxy + row;
}

// ---- bf16 MFMA attention --------------------------------------------------------------------
template <int DH>
__global__ __launch_bounds__(256) void attn_mfma_kernel(AttnArgs a) {
  constexpr int DT = DH / 16;      // dh tiles of the output
  constexpr int KS = DH / 32;      // k-steps of S^T = K Q^T
  __shared__ float sm_o[4][16][DH + 1];
  __shared__ float sm_m[4][16], sm_l[4][16];

  const int n = a.n_pos;
  const int rg = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int nrows = a.n_tok + a.n_proxy;
  const int r0 = rg * 32;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g4 = lane >> 4, c16 = lane & 15;
  const int kvh = (h * a.hkv) / a.hq;
  const uint16_t* kc = (const uint16_t*)a.kc + (int64_t)b * n * a.hkv * DH + kvh * DH;
  const uint16_t* vt = (const uint16_t*)a.vc + ((int64_t)b * a.hkv + kvh) * DH * n;
  const float scale = 1.f / sqrtf((float)DH);
  const int nblk = (n + 31) >> 5;

  // query fragments (B operand of S^T): lane holds row c16, dh [32 ks + 8 g4, +8)
  uint4 qhi[2][KS], qlo[2][KS];
  bool keep[2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int row = r0 + rt * 16 + c16;
    const bool valid = row < nrows;
    bool kp = false;
    for (int i = 0; i < 16; ++i) kp |= (r0 + rt * 16 + i < nrows) && row_keeps_logits(a, r0 + rt * 16 + i);
    keep[rt] = kp;
    const float* qr = a.q + ((int64_t)b * a.mq + (valid ? row : 0)) * (a.hq * DH) + h * DH + 8 * g4;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = valid ? qr[32 * ks + e] : 0.f;
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint16_t h0 = f32_to_bf16(x[2 * e]), h1 = f32_to_bf16(x[2 * e + 1]);
        hi[e] = (uint32_t)h0 | ((uint32_t)h1 << 16);
        lo[e] = pack2(x[2 * e] - bf16_to_f32(h0), x[2 * e + 1] - bf16_to_f32(h1));
      }
      qhi[rt][ks] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
      qlo[rt][ks] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    }
  }
  const bool any_rows1 = r0 + 16 < nrows;

  floatx4_t o[2][DT];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[rt][dt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};

  for (int blk = wave; blk < nblk; blk += 4) {
    const int key0 = blk * 32;
    // S^T tiles [kt][rt]: lane holds keys key0 + 16 kt + 4 g4 + i (i < 4), row c16
    floatx4_t s[2][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      int key = key0 + 16 * kt + c16;
      key = key < n ? key : n - 1;
      const uint16_t* kr = kc + (int64_t)key * a.hkv * DH + 8 * g4;
      uint4 kf[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kf[ks] = *(const uint4*)(kr + 32 * ks);
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        floatx4_t acc = floatx4_t{0.f, 0.f, 0.f, 0.f};
        if (rt == 0 || any_rows1) {
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            acc = mfma(kf[ks], qhi[rt][ks], acc);
            acc = mfma(kf[ks], qlo[rt][ks], acc);
          }
        }
        s[kt][rt] = acc;
      }
    }
    // scale, mask, stage kept logits, online softmax, P^T fragments
    uint4 pf[2], pl[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      float v[8];
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = key0 + 16 * kt + 4 * g4 + i;
          const float x = key < n ? s[kt][rt][i] * scale : -INFINITY;
          v[kt * 4 + i] = x;
          mx = fmaxf(mx, x);
        }
      const int row = r0 + rt * 16 + c16;
      if (keep[rt] && row < nrows && row_keeps_logits(a, row)) {
        float* lg = a.lg_stage + (((int64_t)b * (a.n_proxy + a.block) + stage_row(a, row)) * a.hq + h) * n;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const int key = key0 + 16 * kt + 4 * g4;
          if (key + 3 < n) {
            *(float4*)(lg + key) = make_float4(v[kt * 4], v[kt * 4 + 1], v[kt * 4 + 2], v[kt * 4 + 3]);
          } else {
            for (int i = 0; i < 4; ++i)
              if (key + i < n) lg[key + i] = v[kt * 4 + i];
          }
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run[rt], mx);
      const float corr = m_run[rt] == -INFINITY ? 0.f : expf(m_run[rt] - m_new);
      float ps = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v[e] = v[e] == -INFINITY ? 0.f : expf(v[e] - m_new);
        ps += v[e];
      }
      ps += __shfl_xor(ps, 16, 64);
      ps += __shfl_xor(ps, 32, 64);
      l_run[rt] = l_run[rt] * corr + ps;
      m_run[rt] = m_new;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[rt][dt] *= corr;
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint16_t h0 = f32_to_bf16(v[2 * e]), h1 = f32_to_bf16(v[2 * e + 1]);
        hi[e] = (uint32_t)h0 | ((uint32_t)h1 << 16);
        lo[e] = pack2(v[2 * e] - bf16_to_f32(h0), v[2 * e + 1] - bf16_to_f32(h1));
      }
      pf[rt] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
      pl[rt] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    }
    // V^T fragments: lane holds dh row 16 dt + c16, keys {key0 + 4 g4 + i} U {key0 + 16 + 4 g4 + i};
    // key chunks at or past n (their probabilities are 0) re-read chunk 0
    int ka = key0 + 4 * g4, kb = key0 + 16 + 4 * g4;
    ka = ka < n ? ka : 0;
    kb = kb < n ? kb : 0;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const uint16_t* vr = vt + (int64_t)(16 * dt + c16) * n;
      const uint2 va = *(const uint2*)(vr + ka), vb = *(const uint2*)(vr + kb);
      const uint4 vf = make_uint4(va.x, va.y, vb.x, vb.y);
      o[0][dt] = mfma(vf, pf[0], o[0][dt]);
      o[0][dt] = mfma(vf, pl[0], o[0][dt]);
      if (any_rows1) {
        o[1][dt] = mfma(vf, pf[1], o[1][dt]);
        o[1][dt] = mfma(vf, pl[1], o[1][dt]);
      }
    }
  }
  // merge the four waves' partial states, one 16-row tile at a time
  const int n_out = min(32, a.n_tok - r0);   // token rows of this workgroup that produce outputs
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    if (rt == 1 && !any_rows1) break;
    __syncthreads();
    if (g4 == 0) {
      sm_m[wave][c16] = m_run[rt];
      sm_l[wave][c16] = l_run[rt];
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) sm_o[wave][c16][16 * dt + 4 * g4 + i] = o[rt][dt][i];
    __syncthreads();
    for (int idx = threadIdx.x; idx < 16 * DH; idx += blockDim.x) {
      const int rr = idx / DH, dd = idx % DH;
      const int lrow = rt * 16 + rr;
      if (lrow >= n_out) continue;
      float M = -INFINITY;
      for (int w = 0; w < 4; ++w) M = fmaxf(M, sm_m[w][rr]);
      float num = 0.f, den = 0.f;
      for (int w = 0; w < 4; ++w) {
        const float f = sm_m[w][rr] == -INFINITY ? 0.f : expf(sm_m[w][rr] - M);
        num += f * sm_o[w][rr][dd];
        den += f * sm_l[w][rr];
      }
      const float val = num / den;
      const int row = r0 + lrow;
      if (a.o_planes) {
        const int64_t plane = (int64_t)a.mt * a.hq * DH;
        uint16_t hi, lo;
        split_bf16(val, hi, lo);
        uint16_t* o = (uint16_t*)a.o + (int64_t)b * 2 * plane + (int64_t)row * (a.hq * DH) + h * DH + dd;
        o[0] = hi;
        o[plane] = lo;
      } else {
        ((float*)a.o)[((int64_t)b * a.mt + row) * (a.hq * DH) + h * DH + dd] = val;
      }
      if (a.chk) a.chk[((int64_t)b * a.chk_rows + row) * (a.hq * DH) + h * DH + dd] = val;
    }
  }
}

// ---- float32 attention (small models) ----------------------------------------------------------
template <int DH>
__global__ __launch_bounds__(256) void attn_f32_kernel(AttnArgs a) {
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
  const int ldk = a.hkv * DH;
  const float* kc = (const float*)a.kc + (int64_t)b * n * ldk + g * DH;
  const float* vt = (const float*)a.vc + ((int64_t)b * a.hkv + g) * DH * n;
  const float scale = 1.f / sqrtf((float)DH);
  for (int i = tid; i < kRG * DH; i += blockDim.x) {
    const int rr = i / DH, dd = i % DH;
    qs[i] = rr < nr ? a.q[((int64_t)b * a.mq + r0 + rr) * (a.hq * DH) + h * DH + dd] : 0.f;
  }
  for (int c0 = 0; c0 < n; c0 += kKC) {
    const int nk = min(kKC, n - c0);
    __syncthreads();
    for (int i = tid; i < kKC * DH; i += blockDim.x) {
      const int j = i / DH, dd = i % DH;
      kv[j * (DH + 1) + dd] = j < nk ? kc[(int64_t)(c0 + j) * ldk + dd] : 0.f;
    }
    __syncthreads();
    for (int i = tid; i < kRG * kKC; i += blockDim.x) {
      const int rr = i / kKC, j = i % kKC;
      if (rr < nr && j < nk) {
        const float* qr = qs + rr * DH;
        const float* kr = kv + j * (DH + 1);
        float acc = 0.f;
        for (int dd = 0; dd < DH; ++dd) acc = fmaf(qr[dd], kr[dd], acc);
        sc[rr * n + c0 + j] = acc * scale;
      }
    }
  }
  __syncthreads();
  for (int rr = wave; rr < nr; rr += 4) {
    const int row = r0 + rr;
    float* s = sc + rr * n;
    if (row_keeps_logits(a, row)) {
      float* lg = a.lg_stage + (((int64_t)b * (a.n_proxy + a.block) + stage_row(a, row)) * a.hq + h) * n;
      for (int j = lane; j < n; j += 64) lg[j] = s[j];
    }
    float m = -INFINITY;
    for (int j = lane; j < n; j += 64) m = fmaxf(m, s[j]);
    m = wave_max(m);
    float z = 0.f;
    for (int j = lane; j < n; j += 64) {
      const float p = expf(s[j] - m);
      s[j] = p;
      z += p;
    }
    z = wave_sum(z);
    if (lane == 0) rinv[rr] = 1.f / z;
  }
  __syncthreads();
  const int n_out_rows = max(0, min(nr, a.n_tok - r0));
  if (n_out_rows == 0) return;
  for (int o = tid; o < n_out_rows * DH; o += blockDim.x) {
    const int rr = o / DH, dd = o % DH;
    const float* p = sc + rr * n;
    const float* vr = vt + (int64_t)dd * n;
    float t = 0.f;
    for (int j = 0; j < n; ++j) t = fmaf(p[j], vr[j], t);
    const float v = t * rinv[rr];
    const int row = r0 + rr;
    ((float*)a.o)[((int64_t)b * a.mt + row) * (a.hq * DH) + h * DH + dd] = v;
    if (a.chk) a.chk[((int64_t)b * a.chk_rows + row) * (a.hq * DH) + h * DH + dd] = v;
  }
}

// KL(softmax(s) || softmax(sp)) over n logits held by one wavefront (s staged, sp in
// place), evaluated through the logit differences so that the result keeps its
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

// One wave per (staged row, head): KL against the previous logits (when wanted),
// then the staged logits replace them.  Staged rows: [proxies; active].
__global__ __launch_bounds__(256) void kl_kernel(AttnArgs a) {
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nst = a.n_proxy + (a.act_logits ? a.block : 0);
  const int b = blockIdx.y;
  if (item >= nst * a.hq) return;
  const int sr = item / a.hq, h = item % a.hq;
  const int n = a.n_pos;
  const float* s = a.lg_stage + (((int64_t)b * (a.n_proxy + a.block) + sr) * a.hq + h) * n;
  float* prev;
  float* out;
  bool do_kl;
  if (sr < a.n_proxy) {
    prev = a.proxy_logits + (((int64_t)b * a.n_proxy + sr) * a.hq + h) * n;
    out = a.kl + ((int64_t)b * a.n_proxy + sr) * a.hq + h;
    do_kl = true;
  } else {
    const int r = sr - a.n_proxy;
    prev = a.act_logits + (((int64_t)b * a.block + r) * a.hq + h) * n;
    out = a.akl + ((int64_t)b * a.block + r) * a.hq + h;
    do_kl = a.act_kl != 0;
  }
  if (do_kl) {
    const float kl = wave_kl(s, prev, n, lane);
    if (lane == 0) *out = kl;
  }
  for (int j = lane; j < n; j += 64) prev[j] = s[j];
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
  if constexpr (std::is_same<T, float>::value) {
    dim3 grid(PS_CEIL_DIV(nrows, kRG), a.hq, a.batch);
    const size_t sm = (kRG * a.dh + kKC * (a.dh + 1) + (size_t)kRG * a.n_pos) * sizeof(float);
    if (a.dh == 64) hipLaunchKernelGGL((attn_f32_kernel<64>), grid, dim3(256), sm, s, a);
    else if (a.dh == 128) hipLaunchKernelGGL((attn_f32_kernel<128>), grid, dim3(256), sm, s, a);
    else return hipErrorInvalidValue;
  } else {
    dim3 grid(PS_CEIL_DIV(nrows, 32), a.hq, a.batch);
    if (a.dh == 64) hipLaunchKernelGGL((attn_mfma_kernel<64>), grid, dim3(256), 0, s, a);
    else if (a.dh == 128) hipLaunchKernelGGL((attn_mfma_kernel<128>), grid, dim3(256), 0, s, a);
    else return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_kl(const AttnArgs& a, hipStream_t s) {
  const int nst = a.n_proxy + (a.act_logits ? a.block : 0);
  if (nst == 0) return hipSuccess;
  hipLaunchKernelGGL(kl_kernel, dim3(PS_CEIL_DIV(nst * a.hq, 4), a.batch), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(topk_kernel, dim3(a.batch), dim3(64), 0, s, a);
  return hipGetLastError();
}

template hipError_t launch_attention<float>(const AttnArgs&, hipStream_t);
template hipError_t launch_attention<bf16_t>(const AttnArgs&, hipStream_t);
