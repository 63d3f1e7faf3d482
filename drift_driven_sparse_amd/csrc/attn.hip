// Attention of the active, window and centroid (proxy) query rows over every
// key position; KL drift of proxy and active rows against the previous step's
// logits; top-k cluster selection.
//
// Cache layouts: K token-major [batch][n][Hkv][dh]; V transposed
// [batch][Hkv][dh][n] so that V^T fragments are contiguous along keys.
//
// bf16 path (attn_chunk_kernel): workgroups over (key chunk, head); MFMA 16x16x32 with the
// float32 queries as three-term bf16 splits where the logits feed the KL drift (float32
// precision), two-term splits elsewhere, and the probabilities as two-term splits (relative
// error below 2^-16, far inside what the outputs need), online softmax per chunk.  Logits
// of proxy rows and (when requested) active rows go to a staging buffer.  One following launch
// (attn_merge_kl_kernel) combines the chunks of the token rows and forms the KL drift of the
// staged rows against the previous logits, which the staged logits then replace.
//
// float32 path (attn_f32_kernel, small models): LDS-staged vector FMA.
#include <utility>

#include "kernels.h"

namespace {

constexpr int kRG = 8;      // f32 path: query rows per workgroup
constexpr int kKC = 32;     // f32 path: keys per LDS chunk

PS_DEV floatx4_t mfma(uint4 a, uint4 b, floatx4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));

// Two float32 values -> packed bf16 pair, round to nearest even (one conversion instruction).
PS_DEV uint32_t pack2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((float2_t{a, b}), bf16x2_t));
}

// Row kinds of the query row list [active (block); window (n_win); centroids (n_proxy)].
PS_DEV bool row_keeps_logits(const AttnArgs& a, int row) {
  return row >= a.n_tok || (row < a.block && a.act_logits != nullptr);
}
PS_DEV int stage_row(const AttnArgs& a, int row) {   // staging buffer row: [proxies; active]
  return row >= a.n_tok ? row - a.n_tok : a.n_stage_proxy + row;
}

// ---- bf16 MFMA attention over key chunks ------------------------------------------------------
// Workgroup = (key chunk, query head, sequence, row group); each of its NWV waves owns one
// 16-row query tile of the group, and all share the chunk's K and V^T, which stream through a
// four-stage LDS ring in 32-key steps (direct global -> LDS loads, one fragment per load
// instruction).  Splitting the rows into groups lets the key chunks be longer at the same
// workgroup count: fewer chunk states to merge, more steps to spread the prologue over.
//
// S^T = K Q^T per 16-key tile with the keys of the A operand permuted so that lane l ends up
// holding the 8 consecutive keys 8(l/16)..+8 of the step for query row l%16: A row m of tile kt
// is key 8(m/4) + 4kt + m%4.  The probabilities then form the B operand of O^T += V^T P^T
// directly, and a V^T fragment is one 16-byte load per lane.  n_pos is a multiple of 4 only, so
// the last 8-key group can hold 4 keys: its lanes load V^T from n-8 and shift their
// probabilities by 4 positions to match.
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void gbl_void;
#define AT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | (0x7 << 4) | (0xF << 8))
// ... and every LDS access of the wave complete (lgkmcnt 0): taken before the ring barrier, after
// which loads into the stage read last may land
#define AT_WAIT(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | (0x7 << 4))

PS_DEV uint4 frag_hi(const float* x) {
  uint32_t w[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) w[e] = pack2(x[2 * e], x[2 * e + 1]);
  return make_uint4(w[0], w[1], w[2], w[3]);
}
// Three-term bf16 split of eight float32 values: x = t0 + t1 + t2 + e with t0 = rn(x),
// t1 = rn(x - t0), t2 = rn(x - t0 - t1) (each difference exact in float32), |e| <= 2^-24 |x|
// roughly: the float32 operands of the attention products keep float32 precision through
// bf16 matrix products.
struct Split3 { uint4 t[3]; };
PS_DEV Split3 frag_split3(const float* x) {
  Split3 s;
  float r[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = x[e];
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    const uint4 h = frag_hi(r);
    s.t[k] = h;
    const uint32_t hw[4] = {h.x, h.y, h.z, h.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      r[2 * e] -= __uint_as_float(hw[e] << 16);
      r[2 * e + 1] -= __uint_as_float(hw[e] & 0xFFFF0000u);
    }
  }
  return s;
}

template <int DH, int NWV>
__global__ __launch_bounds__(64 * NWV) void attn_chunk_kernel(AttnArgs a) {
  constexpr int RTW = 1;                    // query tiles per wave
  constexpr int KS = DH / 32, DT = DH / 16;
  constexpr int FK = 2 * KS, F = FK + DT;   // K and V^T fragments per 32-key step
  constexpr int LPW = (F + NWV - 1) / NWV;  // loads per wave per step
  constexpr int FP = LPW * NWV;             // fragment slots per step (with padding)
  __shared__ uint4 b0[FP * 64], b1[FP * 64], b2[FP * 64], b3[FP * 64];
  auto bp = [&](auto I) -> uint4* {
    if constexpr (I == 0) return b0;
    else if constexpr (I == 1) return b1;
    else if constexpr (I == 2) return b2;
    else return b3;
  };
  const int chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z / a.row_groups, rgi = blockIdx.z % a.row_groups;
  const int n = a.n_pos, nrows = a.n_tok + a.n_proxy;
  const int tile0 = rgi * a.group_tiles;   // this workgroup's row tiles: [tile0, tile0 + group_tiles)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g4 = lane >> 4, c16 = lane & 15;
  const int kvh = (h * a.hkv) / a.hq;
  // keys [key_lo, key_hi), in chunks from key_lo rounded down to 8 keys (aligned V^T loads)
  const int k0 = (a.key_lo & ~7) + chunk * a.chunk_keys;
  const int k1 = min(a.key_hi, k0 + a.chunk_keys);
  const int nst = (k1 - k0 + 31) >> 5;
  const uint16_t* kc = (const uint16_t*)a.kc + (int64_t)b * n * a.hkv * DH + kvh * DH;
  const uint16_t* vt = (const uint16_t*)a.vc + ((int64_t)b * a.hkv + kvh) * DH * n;
  // logits are carried in log2 units: the queries are pre-scaled by log2(e)/sqrt(dh), so that
  // softmax terms are single exp2 instructions; staged logits are converted back to natural units
  const float qscale = 1.4426950408889634f / sqrtf((float)DH);
  constexpr float kLn2 = 0.6931471805599453f;

  // this lane's source for load slot i of a step starting at key0
  auto issue = [&](uint4* buf, int step) __attribute__((always_inline)) {
    step = step < nst ? step : nst - 1;
    const int key0 = k0 + 32 * step;
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int slot = i * NWV + wave;
      const int f = slot < F ? slot : 0;   // padding slots repeat fragment 0 into their own slot
      const uint16_t* src;
      if (f < FK) {
        const int kt = f / KS, ks = f % KS;
        int key = key0 + 8 * (c16 >> 2) + 4 * kt + (c16 & 3);
        key = key < n ? key : n - 1;
        src = kc + (int64_t)key * a.hkv * DH + 32 * ks + 8 * g4;
      } else {
        int kg = key0 + 8 * g4;
        kg = kg + 8 <= n ? kg : n - 8;
        src = vt + (int64_t)(16 * (f - FK) + c16) * n + kg;
      }
      __builtin_amdgcn_global_load_lds((gbl_void*)src, (lds_void*)&buf[slot * 64], 16, 0, 0);
    }
  };

  // query fragments (B operand of S^T): lane holds row c16 of each tile, dh [32 ks + 8 g4, +8)
  // (loaded before the first K/V stages are issued and converted after, so that the query
  // loads overlap the K/V loads)
  // Tiles holding a row whose logits are kept for the KL drift (centroid rows; active rows
  // when their logits are kept) multiply all three query terms: the drift of nearly equal
  // distributions needs float32 logits.  The other tiles' logits only weight the outputs, and
  // two terms (relative error below 2^-16) are far inside what those need.
  Split3 qs[RTW][KS];
  float4 qraw[RTW][KS][2];
  bool tile_on[RTW], q_valid[RTW], q3[RTW];
  auto load_q = [&](auto Tc) __attribute__((always_inline)) {
    constexpr int t = decltype(Tc)::value;
    const int tile = tile0 + wave * RTW + t;
    tile_on[t] = tile * 16 < nrows && wave * RTW + t < a.group_tiles;
    q3[t] = tile * 16 + 15 >= a.n_tok || (a.act_logits != nullptr && tile * 16 < a.block);
    const int row = tile * 16 + c16;
    q_valid[t] = row < nrows;
    const int qrow = q_valid[t] ? row : 0;
    const bool from_cache = a.q_win && qrow >= a.block && qrow < a.n_tok;   // window rows' cached queries
    const float* qr = (from_cache ? a.q_win + ((int64_t)b * a.win_max + (qrow - a.block)) * (a.hq * DH)
                                  : a.q + ((int64_t)b * a.mq + qrow) * (a.hq * DH)) + h * DH + 8 * g4;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qraw[t][ks][0] = *(const float4*)(qr + 32 * ks);
      qraw[t][ks][1] = *(const float4*)(qr + 32 * ks + 4);
    }
  };
  auto convert_q = [&](auto Tc) __attribute__((always_inline)) {
    constexpr int t = decltype(Tc)::value;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const float4 u = qraw[t][ks][0], v = qraw[t][ks][1];
      float x[8] = {u.x, u.y, u.z, u.w, v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = q_valid[t] ? x[e] * qscale : 0.f;
      qs[t][ks] = frag_split3(x);
    }
  };
  [&]<int... T>(std::integer_sequence<int, T...>) {
    (load_q(std::integral_constant<int, T>{}), ...);
  }(std::make_integer_sequence<int, RTW>{});
  floatx4_t o[RTW][DT];
  float m_run[RTW], l_run[RTW];
#pragma unroll
  for (int t = 0; t < RTW; ++t) {
    m_run[t] = -INFINITY;
    l_run[t] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[t][dt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  }

  auto compute = [&](const uint4* buf, int step) __attribute__((always_inline)) {
    const int key0 = k0 + 32 * step;
    const int kg = key0 + 8 * g4;            // first key of this lane's 8-key group
    const bool shift = kg < n && kg + 8 > n; // ragged tail: V^T was loaded from n - 8
    const bool full = key0 >= a.key_lo && key0 + 32 <= k1;   // every key of the step is in range
    auto tile_step = [&](auto Tc) __attribute__((always_inline)) {
      constexpr int t = decltype(Tc)::value;
      if (!tile_on[t]) return;
      floatx4_t sacc[2];
      if (q3[t]) {   // wave-uniform
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          floatx4_t acc = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            const uint4 kf = buf[(kt * KS + ks) * 64 + lane];
            acc = mfma(kf, qs[t][ks].t[2], acc);   // smallest terms first
            acc = mfma(kf, qs[t][ks].t[1], acc);
            acc = mfma(kf, qs[t][ks].t[0], acc);
          }
          sacc[kt] = acc;
        }
      } else {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          floatx4_t acc = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            const uint4 kf = buf[(kt * KS + ks) * 64 + lane];
            acc = mfma(kf, qs[t][ks].t[1], acc);
            acc = mfma(kf, qs[t][ks].t[0], acc);
          }
          sacc[kt] = acc;
        }
      }
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = sacc[e >> 2][e & 3];
      if (!full) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (kg + e >= a.key_lo && kg + e < k1) ? v[e] : -INFINITY;
      }
      float mx = fmaxf(fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])), fmaxf(fmaxf(v[4], v[5]), fmaxf(v[6], v[7])));
      const int row = (tile0 + wave * RTW + t) * 16 + c16;
      if (row < nrows && row_keeps_logits(a, row)) {
        float* lg = a.lg_stage + (((int64_t)b * (a.n_stage_proxy + a.block) + stage_row(a, row)) * a.hq + h) * n + kg;
        if (kg >= a.key_lo && kg + 8 <= k1) {
          *(float4*)lg = make_float4(v[0] * kLn2, v[1] * kLn2, v[2] * kLn2, v[3] * kLn2);
          *(float4*)(lg + 4) = make_float4(v[4] * kLn2, v[5] * kLn2, v[6] * kLn2, v[7] * kLn2);
        } else {
          for (int e = 0; e < 8; ++e)
            if (kg + e >= a.key_lo && kg + e < k1) lg[e] = v[e] * kLn2;
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      // every step has a key in range, so m_new is finite; exp2(-inf) = 0 covers the first step
      // and masked keys
      const float m_new = fmaxf(m_run[t], mx);
      const float corr = __builtin_amdgcn_exp2f(m_run[t] - m_new);
      float ps = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v[e] = __builtin_amdgcn_exp2f(v[e] - m_new);
        ps += v[e];
      }
      ps += __shfl_xor(ps, 16, 64);
      ps += __shfl_xor(ps, 32, 64);
      l_run[t] = l_run[t] * corr + ps;
      m_run[t] = m_new;
      const bool rescale = __builtin_amdgcn_ballot_w64(corr != 1.f) != 0;   // wave-uniform
      if (shift) {
#pragma unroll
        for (int e = 7; e >= 4; --e) v[e] = v[e - 4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = 0.f;
      }
      const Split3 pv = frag_split3(v);   // the third term is not used
      if (rescale) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[t][dt] *= corr;
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const uint4 vf = buf[(FK + dt) * 64 + lane];
        o[t][dt] = mfma(vf, pv.t[1], o[t][dt]);
        o[t][dt] = mfma(vf, pv.t[0], o[t][dt]);
      }
    };
    [&]<int... T>(std::integer_sequence<int, T...>) {
      (tile_step(std::integral_constant<int, T>{}), ...);
    }(std::make_integer_sequence<int, RTW>{});
  };

  issue(b0, 0);
  issue(b1, 1);
  issue(b2, 2);
  AT_VMCNT(LPW * 3);   // the query loads (issued before the three stages) have landed
  [&]<int... T>(std::integer_sequence<int, T...>) {
    (convert_q(std::integral_constant<int, T>{}), ...);
  }(std::make_integer_sequence<int, RTW>{});
  for (int s = 0; s < nst; s += 4) {
    [&]<int... U>(std::integer_sequence<int, U...>) {
      ([&] {
        AT_WAIT(LPW * 2);
        __builtin_amdgcn_s_barrier();
        issue(bp(std::integral_constant<int, (U + 3) % 4>{}), s + U + 3);
        if (s + U < nst) compute(bp(std::integral_constant<int, U>{}), s + U);
      }(), ...);
    }(std::make_integer_sequence<int, 4>{});
  }
  AT_VMCNT(0);

  // outputs of token rows: lane holds O^T[16 dt + 4 g4 + i][row c16]
  auto store_tile = [&](auto Tc) __attribute__((always_inline)) {
    constexpr int t = decltype(Tc)::value;
    const int row = (tile0 + wave * RTW + t) * 16 + c16;
    if (!tile_on[t] || row >= a.n_tok) return;
    if (a.n_chunks == 1) {
      const float inv = 1.f / l_run[t];
      const int64_t plane = (int64_t)a.mt * a.hq * DH;
      uint16_t* op = (uint16_t*)a.o + (int64_t)b * 2 * plane + (int64_t)row * (a.hq * DH) + h * DH;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int dd = 16 * dt + 4 * g4 + i;
          const float val = o[t][dt][i] * inv;
          uint16_t hi, lo;
          split_bf16(val, hi, lo);
          op[dd] = hi;
          op[plane + dd] = lo;
          if (a.chk) a.chk[((int64_t)b * a.chk_rows + row) * (a.hq * DH) + h * DH + dd] = val;
        }
    } else {
      const int64_t slot = (((int64_t)b * a.n_chunks + chunk) * a.hq + h) * a.mt + row;
      float* po = a.part_o + slot * DH;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        *(float4*)(po + 16 * dt + 4 * g4) = make_float4(o[t][dt][0], o[t][dt][1], o[t][dt][2], o[t][dt][3]);
      if (g4 == 0) *(float2*)(a.part_ml + slot * 2) = make_float2(m_run[t], l_run[t]);
    }
  };
  [&]<int... T>(std::integer_sequence<int, T...>) {
    (store_tile(std::integral_constant<int, T>{}), ...);
  }(std::make_integer_sequence<int, RTW>{});
}

// Merge of the per-chunk states of one (token row, head): o = sum_c 2^(m_c - M) O_c / sum_c 2^(m_c - M) l_c
// (running maxima in log2 units).  One wave per (row, head): lane c reads chunk c's (m, l), and
// each lane then adds the chunks' outputs for its DH/64 columns in chunk order.
template <int DH>
PS_DEV void attn_merge_pair(const AttnArgs& a, int pair, int b) {
  constexpr int E = DH / 64;
  const int lane = threadIdx.x & 63;
  if (pair >= a.n_tok * a.hq) return;
  const int row = pair / a.hq, h = pair % a.hq;
  const int64_t cstride = (int64_t)a.hq * a.mt;                       // slots between chunks
  const int64_t slot0 = ((int64_t)b * a.n_chunks * a.hq + h) * a.mt + row;
  float2 ml = make_float2(-INFINITY, 0.f);
  if (lane < a.n_chunks) ml = *(const float2*)(a.part_ml + (slot0 + lane * cstride) * 2);
  const float M = wave_max(ml.x);
  const float f = __builtin_amdgcn_exp2f(ml.x - M);                 // 0 for lanes past the chunks
  const float den = wave_sum(f * ml.y);
  float num[E];
#pragma unroll
  for (int e = 0; e < E; ++e) num[e] = 0.f;
  for (int c0 = 0; c0 < a.n_chunks; c0 += 8) {
    float t[8][E];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (c0 + j < a.n_chunks) {
        const float* po = a.part_o + (slot0 + (c0 + j) * cstride) * DH + E * lane;
#pragma unroll
        for (int e = 0; e < E; ++e) t[j][e] = po[e];
      }
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (c0 + j < a.n_chunks) {
        const float fc = __shfl(f, c0 + j, 64);
#pragma unroll
        for (int e = 0; e < E; ++e) num[e] += fc * t[j][e];
      }
  }
  const int64_t plane = (int64_t)a.mt * a.hq * DH;
  uint16_t* op = (uint16_t*)a.o + (int64_t)b * 2 * plane + (int64_t)row * (a.hq * DH) + h * DH + E * lane;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const float val = num[e] / den;
    uint16_t hi, lo;
    split_bf16(val, hi, lo);
    op[e] = hi;
    op[plane + e] = lo;
    if (a.chk) a.chk[((int64_t)b * a.chk_rows + row) * (a.hq * DH) + h * DH + E * lane + e] = val;
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
  const int klo = a.key_lo, khi = a.key_hi;
  for (int c0 = klo; c0 < khi; c0 += kKC) {
    const int nk = min(kKC, khi - c0);
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
      float* lg = a.lg_stage + (((int64_t)b * (a.n_stage_proxy + a.block) + stage_row(a, row)) * a.hq + h) * n;
      for (int j = klo + lane; j < khi; j += 64) lg[j] = s[j];
    }
    float m = -INFINITY;
    for (int j = klo + lane; j < khi; j += 64) m = fmaxf(m, s[j]);
    m = wave_max(m);
    float z = 0.f;
    for (int j = klo + lane; j < khi; j += 64) {
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
    for (int j = klo; j < khi; ++j) t = fmaf(p[j], vr[j], t);
    const float v = t * rinv[rr];
    const int row = r0 + rr;
    ((float*)a.o)[((int64_t)b * a.mt + row) * (a.hq * DH) + h * DH + dd] = v;
    if (a.chk) a.chk[((int64_t)b * a.chk_rows + row) * (a.hq * DH) + h * DH + dd] = v;
  }
}


// Block-wide max (fixed combination order); every thread gets the result.
PS_DEV float block_max_f(float v, float* red) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
  v = wave_max(v);
  __syncthreads();
  if (lane == 0) red[wid] = v;
  __syncthreads();
  float m = -INFINITY;
  for (int i = 0; i < nw; ++i) m = fmaxf(m, red[i]);
  __syncthreads();
  return m;
}

// Two block-wide sums in one exchange (fixed combination order); `red` holds two slots per wave.
PS_DEV void block_sum2(float& x, float& y, float* red) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
  x = wave_sum(x);
  y = wave_sum(y);
  __syncthreads();
  if (lane == 0) { red[2 * wid] = x; red[2 * wid + 1] = y; }
  __syncthreads();
  x = 0.f;
  y = 0.f;
  for (int i = 0; i < nw; ++i) { x += red[2 * i]; y += red[2 * i + 1]; }
  __syncthreads();
}

// KL(softmax(s) || softmax(p)) of one row held PER values per thread across the workgroup,
// from the logit differences: with a = p - max p, u = exp(a), dbar the u-weighted mean of s - p
// and e = s - p - dbar, KL = E_u[e^e e] / E_u[e^e] - log E_u[e^e], formed with expm1/log1p so
// that small drifts keep their relative precision.  The products u e^e are taken as exp(a + e),
// which stays bounded by the spread of s where e alone overflows (positions that p makes very
// unlikely and s does not); when even a + e exceeds 60 somewhere (a drift of tens of nats),
// the sums are scaled by exp(-max(a + e)) and the logarithm is taken directly.
template <int PER>
PS_DEV float block_kl(const float* sv, const float* pv, int n, float* red) {
  float mp = -INFINITY;
#pragma unroll
  for (int i = 0; i < PER; ++i)
    if (threadIdx.x + 256 * i < n) mp = fmaxf(mp, pv[i]);
  mp = block_max_f(mp, red);
  float u[PER];
  float s0 = 0.f, sd = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const bool ok = threadIdx.x + 256 * i < n;
    u[i] = ok ? expf(pv[i] - mp) : 0.f;
    s0 += u[i];
    sd += ok ? u[i] * (sv[i] - pv[i]) : 0.f;
  }
  block_sum2(s0, sd, red);
  const float dbar = sd / s0;
  float e[PER], ae[PER];
  float c = -INFINITY;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    e[i] = (sv[i] - pv[i]) - dbar;
    ae[i] = (pv[i] - mp) + e[i];
    if (threadIdx.x + 256 * i < n) c = fmaxf(c, ae[i]);
  }
  c = block_max_f(c, red);   // uniform over the workgroup
  float s1 = 0.f, s2 = 0.f;
  if (c <= 60.f) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (threadIdx.x + 256 * i < n) {
        const float w = expf(ae[i]);
        s1 += e[i] < 80.f ? u[i] * expm1f(e[i]) : w - u[i];
        s2 += w * e[i];
      }
    }
    block_sum2(s1, s2, red);
    const float r1 = s1 / s0;
    return (s2 / s0) / (1.f + r1) - log1pf(r1);
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if (threadIdx.x + 256 * i < n) {
      const float w = expf(ae[i] - c);
      s1 += w;
      s2 += w * e[i];
    }
  }
  block_sum2(s1, s2, red);
  return s2 / s1 - (c + logf(s1 / s0));
}

// One 256-thread workgroup per (staged row, head): KL against the previous logits (when
// wanted), then the staged logits replace them.  Staged rows: [proxies; active].
template <int PER>
PS_DEV void kl_item(const AttnArgs& a, int item, int b) {
  __shared__ float red[8];
  const int nst = a.n_proxy + (a.act_logits ? a.block : 0);
  if (item >= nst * a.hq) return;   // uniform over the workgroup
  const int sr = item / a.hq, h = item % a.hq;
  const int np = a.n_pos;
  const float* s = a.lg_stage + (((int64_t)b * (a.n_stage_proxy + a.block) + sr) * a.hq + h) * np;
  float* prev;
  float* out;
  bool do_kl;
  int lo = 0, n = np;   // key range of the row's logits
  if (sr < a.n_proxy) {
    prev = a.proxy_logits + (((int64_t)b * a.n_proxy + sr) * a.hq + h) * np;
    out = a.kl + ((int64_t)b * a.n_proxy + sr) * a.hq + h;
    do_kl = a.proxy_kl != 0;
    lo = a.pkey_lo;
    n = a.pkey_hi - a.pkey_lo;
  } else {
    const int r = sr - a.n_proxy;
    prev = a.act_logits + (((int64_t)b * a.block + r) * a.hq + h) * np;
    out = a.akl + ((int64_t)b * a.block + r) * a.hq + h;
    do_kl = a.act_kl != 0;
  }
  s += lo;
  prev += lo;
  float sv[PER], pv[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int j = threadIdx.x + 256 * i;
    sv[i] = j < n ? s[j] : 0.f;
    pv[i] = (do_kl && j < n) ? prev[j] : 0.f;
  }
  if (do_kl) {
    const float kl = block_kl<PER>(sv, pv, n, red);
    if (threadIdx.x == 0) *out = kl;
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int j = threadIdx.x + 256 * i;
    if (j < n) prev[j] = sv[i];
  }
}

// One launch for the two consumers of the chunk kernel's outputs: workgroups below
// merge_wgs merge token rows (four (row, head) pairs each, one per wave), the rest form one KL
// item each.  Both only read what the attention kernel wrote and write disjoint outputs.
// PER logits per thread: rows of up to 256 * PER positions.
template <int DH, int PER>
__global__ __launch_bounds__(256) void attn_merge_kl_kernel(AttnArgs a, int merge_wgs) {
  const int wave = threadIdx.x >> 6, b = blockIdx.y;
  if ((int)blockIdx.x < merge_wgs) attn_merge_pair<DH>(a, blockIdx.x * 4 + wave, b);
  else kl_item<PER>(a, blockIdx.x - merge_wgs, b);
}

// Per sequence: D_c = sum_h max(0, KL_{c,h}); top-k clusters by (D desc, index asc), found by
// ranking every cluster against the others; S = window rows whose label is selected, ascending;
// and the per-row active drift delta_j = sum_h max(0, KL_{j,h}).  Head sums are wavefront
// reductions (fixed order).  One 256-thread workgroup per sequence.
__global__ __launch_bounds__(256) void topk_kernel(TopkArgs a) {
  __shared__ float D[16];
  __shared__ int chosen[16];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (a.refresh) {
    // wave 0 loads the window labels first, so that their round trip overlaps the drift sums
    constexpr int kLab = 4;   // labels per lane: n_win <= 256
    int lab[kLab];
    if (wave == 0) {
#pragma unroll
      for (int i = 0; i < kLab; ++i) {
        const int w = 64 * i + lane;
        lab[i] = w < a.n_win ? a.win_m[(int64_t)b * a.win_max + w] : -1;
      }
    }
    const int keff = min(a.K, a.n_win);
    for (int c = wave; c < a.K; c += 4) {
      float s = 0.f;
      if (c < keff)
        for (int h = lane; h < a.hq; h += 64) s += fmaxf(0.f, a.kl[((int64_t)b * a.K + c) * a.hq + h]);
      s = wave_sum(s);
      if (lane == 0) {
        D[c] = s;
        if (a.D) a.D[(int64_t)b * a.K + c] = s;
      }
    }
    __syncthreads();
    const int kk = min(a.k, keff);
    if (tid < a.K) {
      int rank = 0;
      if (tid < keff)
        for (int c = 0; c < keff; ++c) rank += (D[c] > D[tid]) || (D[c] == D[tid] && c < tid);
      const int sel = tid < keff && rank < kk;
      chosen[tid] = sel;
      if (sel && a.topk) a.topk[(int64_t)b * a.k + rank] = tid;
    }
    if (tid >= kk && tid < a.k && a.topk) a.topk[(int64_t)b * a.k + tid] = -1;
    __syncthreads();
    if (wave == 0) {
      int base = 0;
#pragma unroll
      for (int i = 0; i < kLab; ++i) {
        const int w = 64 * i + lane;
        const int c = lab[i];
        const bool sel = c >= 0 && c < a.K && chosen[c];
        const unsigned long long m = __ballot(sel);
        const int before = __popcll(m & ((1ull << lane) - 1ull));
        if (sel) a.sel_idx[(int64_t)b * a.win_max + base + before] = w;
        base += __popcll(m);
      }
      if (lane == 0) a.sel_count[b] = base;
    }
    if (tid == 0 && a.q_ok) a.q_ok[b] = a.q_tag;   // every window row's query is now current for this block
  } else {
    if (tid == 0) a.sel_count[b] = 0;
  }
  if (a.delta) {
    for (int j = wave; j < a.block; j += 4) {
      float s = 0.f;
      for (int h = lane; h < a.hq; h += 64) s += fmaxf(0.f, a.akl[((int64_t)b * a.block + j) * a.hq + h]);
      s = wave_sum(s);
      if (lane == 0) a.delta[(int64_t)b * a.block + j] = s;
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
    const int tiles = PS_CEIL_DIV(nrows, 16);
    if (a.row_groups < 1 || a.group_tiles * a.row_groups < tiles) return hipErrorInvalidValue;
    const int nwv = 2 * PS_CEIL_DIV(a.group_tiles, 2);   // one wave per 16-row tile, even count
    if (nwv > 12 || a.n_pos < 8 || a.chunk_keys % 32 || a.n_chunks * a.chunk_keys < a.key_hi - (a.key_lo & ~7) ||
        a.key_lo < 0 || a.key_hi > a.n_pos || a.key_lo >= a.key_hi)
      return hipErrorInvalidValue;
    dim3 grid(a.n_chunks, a.hq, a.batch * a.row_groups);
    auto go = [&](auto DHc, auto NWc) {
      constexpr int NW = decltype(NWc)::value;
      hipLaunchKernelGGL((attn_chunk_kernel<decltype(DHc)::value, NW>), grid, dim3(64 * NW), 0, s, a);
    };
    auto by_waves = [&](auto DHc) {
      switch (nwv) {
        case 2: go(DHc, std::integral_constant<int, 2>{}); break;
        case 4: go(DHc, std::integral_constant<int, 4>{}); break;
        case 6: go(DHc, std::integral_constant<int, 6>{}); break;
        case 8: go(DHc, std::integral_constant<int, 8>{}); break;
        case 10: go(DHc, std::integral_constant<int, 10>{}); break;
        default: go(DHc, std::integral_constant<int, 12>{}); break;
      }
    };
    if (a.dh == 64) by_waves(std::integral_constant<int, 64>{});
    else if (a.dh == 128) by_waves(std::integral_constant<int, 128>{});
    else return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_merge_kl(const AttnArgs& a, bool merge, hipStream_t s) {
  merge = merge && a.n_chunks > 1 && a.n_tok > 0;
  if (merge && a.n_chunks > 64) return hipErrorInvalidValue;
  const int nst = a.n_proxy + (a.act_logits ? a.block : 0);
  if (a.n_pos > kMaxPos) return hipErrorInvalidValue;
  const int mw = merge ? PS_CEIL_DIV(a.n_tok * a.hq, 4) : 0, kw = nst * a.hq;
  if (mw + kw == 0) return hipSuccess;
  const dim3 grid(mw + kw, a.batch);
  if (merge && a.dh != 128 && a.dh != 64) return hipErrorInvalidValue;
  auto go = [&](auto PERc) {
    constexpr int PER = decltype(PERc)::value;
    if (!merge || a.dh == 128) hipLaunchKernelGGL((attn_merge_kl_kernel<128, PER>), grid, dim3(256), 0, s, a, mw);
    else hipLaunchKernelGGL((attn_merge_kl_kernel<64, PER>), grid, dim3(256), 0, s, a, mw);
  };
  if (a.n_pos <= 1024) go(std::integral_constant<int, 4>{});
  else if (a.n_pos <= 2048) go(std::integral_constant<int, 8>{});
  else go(std::integral_constant<int, 16>{});
  return hipGetLastError();
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(topk_kernel, dim3(a.batch), dim3(256), 0, s, a);
  return hipGetLastError();
}

template hipError_t launch_attention<float>(const AttnArgs&, hipStream_t);
template hipError_t launch_attention<bf16_t>(const AttnArgs&, hipStream_t);
