// Shared device/host helpers of the Polestar refresh kernels (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/polestar.h"

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

#define PS_DEV __device__ __forceinline__
#define PS_HD __host__ __device__ __forceinline__

// ---- storage dtype helpers ------------------------------------------------
// bfloat16 is carried as raw uint16 bit patterns.
struct bf16_t {
  uint16_t bits;
};

PS_HD float bf16_to_f32(uint16_t b) {
  union { uint32_t u; float f; } v;
  v.u = ((uint32_t)b) << 16;
  return v.f;
}

// float32 -> bfloat16, round to nearest, ties to even (finite inputs).
PS_HD uint16_t f32_to_bf16(float f) {
  union { uint32_t u; float f; } v;
  v.f = f;
  uint32_t u = v.u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// float64 -> bfloat16 rounded once (to 8 significant bits, ties to even), for
// values in the normal float range.
PS_HD uint16_t f64_to_bf16(double x) {
  union { uint64_t u; double d; } v;
  v.d = x;
  uint64_t u = v.u;
  u += 0x00000FFFFFFFFFFFull + ((u >> 45) & 1ull);
  u &= ~0x00001FFFFFFFFFFFull;
  v.u = u;
  const float f = (float)v.d;           // exact: at most 8 significant bits
  union { uint32_t u; float f; } w;
  w.f = f;
  return (uint16_t)(w.u >> 16);
}

template <typename T> struct St;
template <> struct St<float> {
  static PS_DEV float load(const float* p, int64_t i) { return p[i]; }
  static PS_DEV void store(float* p, int64_t i, float v) { p[i] = v; }
  static PS_DEV float round(float v) { return v; }
  static PS_DEV void store_d(float* p, int64_t i, double v) { p[i] = (float)v; }
};
template <> struct St<bf16_t> {
  static PS_DEV float load(const bf16_t* p, int64_t i) { return bf16_to_f32(p[i].bits); }
  static PS_DEV void store(bf16_t* p, int64_t i, float v) { p[i].bits = f32_to_bf16(v); }
  static PS_DEV float round(float v) { return bf16_to_f32(f32_to_bf16(v)); }
  static PS_DEV void store_d(bf16_t* p, int64_t i, double v) { p[i].bits = f64_to_bf16(v); }
};

// ---- reductions -------------------------------------------------------------
template <typename V>
PS_DEV V wave_sum(V v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
PS_DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Block-wide sum with a fixed combination order (deterministic).  `red` must
// hold one slot per wave.  All threads get the result.
template <typename V>
PS_DEV V block_sum(V v, V* red) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
  v = wave_sum(v);
  __syncthreads();
  if (lane == 0) red[wid] = v;
  __syncthreads();
  V s = 0;
  for (int i = 0; i < nw; ++i) s += red[i];
  __syncthreads();
  return s;
}

// ---- rows in the storage dtype ----------------------------------------------
// Four consecutive elements as float32 (8- or 16-byte accesses).
template <typename T> struct Quad;
template <> struct Quad<float> {
  static PS_DEV void load(const float* p, float* x) {
    const float4 v = *(const float4*)p;
    x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
  }
  static PS_DEV void store(float* p, const float* x) { *(float4*)p = make_float4(x[0], x[1], x[2], x[3]); }
};
template <> struct Quad<bf16_t> {
  static PS_DEV void load(const bf16_t* p, float* x) {
    const uint2 v = *(const uint2*)p;
    x[0] = bf16_to_f32(v.x & 0xFFFFu); x[1] = bf16_to_f32(v.x >> 16);
    x[2] = bf16_to_f32(v.y & 0xFFFFu); x[3] = bf16_to_f32(v.y >> 16);
  }
  static PS_DEV void store(bf16_t* p, const float* x) {
    *(uint2*)p = make_uint2((uint32_t)f32_to_bf16(x[0]) | ((uint32_t)f32_to_bf16(x[1]) << 16),
                            (uint32_t)f32_to_bf16(x[2]) | ((uint32_t)f32_to_bf16(x[3]) << 16));
  }
};

// RMSNorm with unit gain of one row of d elements (d a multiple of 4): calls
// store(n, x) with x[0..3] = src[n..n+3] * 1/sqrt(mean(src^2) + eps).  Every thread of the block
// takes part; `red` holds one float per wave.
template <typename T, typename Store>
PS_DEV void rmsnorm_row(const T* src, int d, float eps, float* red, Store&& store) {
  // the first QH quads of each thread stay in registers between the two passes
  constexpr int QH = 4;
  const int step = 4 * blockDim.x, n1 = 4 * threadIdx.x + QH * step;
  float xs[QH][4];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < QH; ++i) {
    const int n = 4 * threadIdx.x + i * step;
    if (n < d) {
      Quad<T>::load(src + n, xs[i]);
      ss += xs[i][0] * xs[i][0] + xs[i][1] * xs[i][1] + xs[i][2] * xs[i][2] + xs[i][3] * xs[i][3];
    }
  }
  for (int n = n1; n < d; n += step) {
    float x[4];
    Quad<T>::load(src + n, x);
    ss += x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3];
  }
  ss = block_sum(ss, red);
  const float inv = 1.f / sqrtf(ss / (float)d + eps);
#pragma unroll
  for (int i = 0; i < QH; ++i) {
    const int n = 4 * threadIdx.x + i * step;
    if (n < d) {
      float x[4] = {xs[i][0] * inv, xs[i][1] * inv, xs[i][2] * inv, xs[i][3] * inv};
      store(n, x);
    }
  }
  for (int n = n1; n < d; n += step) {
    float x[4];
    Quad<T>::load(src + n, x);
    x[0] *= inv; x[1] *= inv; x[2] *= inv; x[3] *= inv;
    store(n, x);
  }
}

// ---- window geometry -------------------------------------------------------
// Window row w -> sequence position: first the prefix rows, then the suffix rows.
struct WinGeom {
  int32_t blk_start, block, n_pre, n_win;   // n_pre prefix rows, n_win total
  PS_HD int32_t pos(int32_t w) const {
    return w < n_pre ? blk_start - n_pre + w : blk_start + block + (w - n_pre);
  }
};

PS_HD WinGeom make_geom(int32_t blk_start, int32_t n_pos, int32_t block, int32_t pre, int32_t suf) {
  WinGeom g;
  g.blk_start = blk_start;
  g.block = block;
  int32_t p0 = blk_start - pre;
  if (p0 < 0) p0 = 0;
  g.n_pre = blk_start - p0;
  int32_t s1 = blk_start + block + suf;
  if (s1 > n_pos) s1 = n_pos;
  int32_t n_suf = s1 - (blk_start + block);
  if (n_suf < 0) n_suf = 0;
  g.n_win = g.n_pre + n_suf;
  return g;
}

// ---- NVFP4 (E2M1 values, E4M3FN scale per 16) -------------------------------
PS_HD float e2m1_value(uint32_t c) {
  const uint32_t m = c & 7u;
  float v = (m == 0) ? 0.f : (m == 1) ? 0.5f : (m == 2) ? 1.f : (m == 3) ? 1.5f
          : (m == 4) ? 2.f : (m == 5) ? 3.f : (m == 6) ? 4.f : 6.f;
  return (c & 8u) ? -v : v;
}

PS_HD float e4m3_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  float mag;
  if (e == 0) {
    mag = (float)m * 0.001953125f;   // m * 2^-9
  } else {
    union { uint32_t u; float f; } v;
    v.u = ((e - 7u + 127u) << 23) | (m << 20);
    mag = v.f;
  }
  return (c & 0x80u) ? -mag : mag;
}

// Non-negative finite float -> E4M3FN byte, round to nearest even, saturate at 448.
PS_HD uint32_t e4m3_encode(float s) {
  if (!(s > 0.f)) return 0u;
  if (s >= 448.f) return 0x7Eu;
  if (s < 0.015625f) {                      // below 2^-6: subnormal grid step 2^-9
    float q = rintf(s * 512.f);             // exact scaling, then round half even
    return (uint32_t)q;                     // q == 8 encodes 2^-6 (e=1, m=0)
  }
  union { uint32_t u; float f; } v;
  v.f = s;
  int32_t ex = (int32_t)((v.u >> 23) & 0xFFu) - 127;
  uint32_t man = v.u & 0x7FFFFFu;
  uint32_t m3 = man >> 20, rem = man & 0xFFFFFu;
  if (rem > 0x80000u || (rem == 0x80000u && (m3 & 1u))) ++m3;
  if (m3 == 8u) { m3 = 0u; ++ex; }
  uint32_t code = ((uint32_t)(ex + 7) << 3) | m3;
  return code > 0x7Eu ? 0x7Eu : code;
}

// float -> E2M1 nibble, round to nearest with ties to the even code, saturate at 6.
PS_HD uint32_t e2m1_encode(float y) {
  float a = fabsf(y);
  uint32_t c;
  if (a <= 0.25f) c = 0;
  else if (a < 0.75f) c = 1;
  else if (a <= 1.25f) c = 2;
  else if (a < 1.75f) c = 3;
  else if (a <= 2.5f) c = 4;
  else if (a < 3.5f) c = 5;
  else if (a <= 5.f) c = 6;
  else c = 7;
  if (y < 0.f && c != 0) c |= 8u;
  return c;
}

// Quantise one group of 16 float32 values.  Returns the scale byte; codes[i] nibbles.
PS_HD uint32_t nvfp4_group(const float* r, uint32_t* codes) {
  float amax = 0.f;
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(r[i]));
  const float s = amax / 6.f;               // correctly rounded float32 division
  const uint32_t sc = e4m3_encode(s);
  const float sv = e4m3_value(sc);
  for (int i = 0; i < 16; ++i) codes[i] = (sv == 0.f) ? 0u : e2m1_encode(r[i] / sv);
  return sc;
}

// ---- residual formats (window storage) --------------------------------------
// Per row of d values: code bytes and scale bytes, and the values sharing one scale.
//   NVFP4:  E2M1 nibbles, E4M3FN scale per 16           (d/2 + d/16 bytes)
//   FP8:    E4M3FN byte per value, no scale             (d bytes)
//   MXINT8: int8 per value, E8M0 scale per 32 (OCP MX)  (d + d/32 bytes)
//   MXFP4:  E2M1 nibbles, E8M0 scale per 32 (OCP MX)    (d/2 + d/32 bytes)
// Element 2j of a nibble format is the low nibble of byte j.
PS_HD int64_t resid_code_bytes(int fmt, int64_t d) {
  return (fmt == POLESTAR_RESID_NVFP4 || fmt == POLESTAR_RESID_MXFP4) ? d / 2 : (fmt == POLESTAR_RESID_RAW ? 0 : d);
}
PS_HD int64_t resid_scale_bytes(int fmt, int64_t d) {
  return fmt == POLESTAR_RESID_NVFP4 ? d / 16 : ((fmt == POLESTAR_RESID_MXINT8 || fmt == POLESTAR_RESID_MXFP4) ? d / 32 : 0);
}
PS_HD int resid_group(int fmt) { return (fmt == POLESTAR_RESID_MXINT8 || fmt == POLESTAR_RESID_MXFP4) ? 32 : 16; }

// E8M0 exponent of an OCP MX block: floor(log2 amax) - emax, clamped to [-127, 127]; -127 for
// an all-zero block.
PS_HD int mx_exponent(float amax, int emax) {
  if (!(amax > 0.f)) return -127;
  int e = ilogbf(amax) - emax;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// Value n of a row's residual (codes/scales point at the row).
PS_HD float resid_value(int fmt, const uint8_t* codes, const uint8_t* scales, int n) {
  switch (fmt) {
    case POLESTAR_RESID_NVFP4:
      return e4m3_value(scales[n >> 4]) * e2m1_value((codes[n >> 1] >> (4 * (n & 1))) & 15u);
    case POLESTAR_RESID_FP8:
      return e4m3_value(codes[n]);
    case POLESTAR_RESID_MXINT8:
      return ldexpf((float)(int8_t)codes[n], (int)scales[n >> 5] - 127 - 6);
    case POLESTAR_RESID_MXFP4:
      return ldexpf(e2m1_value((codes[n >> 1] >> (4 * (n & 1))) & 15u), (int)scales[n >> 5] - 127);
    default:
      return 0.f;
  }
}

// Quantise the resid_group(fmt) values r of the group starting at column g0 of a row.
PS_HD void resid_encode_group(int fmt, const float* r, uint8_t* codes, uint8_t* scales, int g0) {
  switch (fmt) {
    case POLESTAR_RESID_NVFP4: {
      uint32_t c[16];
      scales[g0 >> 4] = (uint8_t)nvfp4_group(r, c);
      for (int e = 0; e < 8; ++e) codes[(g0 >> 1) + e] = (uint8_t)(c[2 * e] | (c[2 * e + 1] << 4));
      break;
    }
    case POLESTAR_RESID_FP8:
      for (int e = 0; e < 16; ++e) {
        const uint32_t m = e4m3_encode(fabsf(r[e]));
        codes[g0 + e] = (uint8_t)((r[e] < 0.f && m != 0u) ? (m | 0x80u) : m);
      }
      break;
    case POLESTAR_RESID_MXINT8: {
      float amax = 0.f;
      for (int e = 0; e < 32; ++e) amax = fmaxf(amax, fabsf(r[e]));
      const int ex = mx_exponent(amax, 0);
      scales[g0 >> 5] = (uint8_t)(ex + 127);
      for (int e = 0; e < 32; ++e) {
        float q = rintf(ldexpf(r[e], 6 - ex));   // exact scaling, nearest even
        q = q < -128.f ? -128.f : (q > 127.f ? 127.f : q);
        codes[g0 + e] = (uint8_t)(int8_t)(int)q;
      }
      break;
    }
    case POLESTAR_RESID_MXFP4: {
      float amax = 0.f;
      for (int e = 0; e < 32; ++e) amax = fmaxf(amax, fabsf(r[e]));
      const int ex = mx_exponent(amax, 2);
      scales[g0 >> 5] = (uint8_t)(ex + 127);
      for (int e = 0; e < 16; ++e)
        codes[(g0 >> 1) + e] = (uint8_t)(e2m1_encode(ldexpf(r[2 * e], -ex)) | (e2m1_encode(ldexpf(r[2 * e + 1], -ex)) << 4));
      break;
    }
    default:
      break;
  }
}

// ---- misc -------------------------------------------------------------------
#define PS_CEIL_DIV(a, b) (((a) + (b) - 1) / (b))

inline size_t ps_align256(size_t x) { return (x + 255) & ~(size_t)255; }
