// Weight-streaming projections of the gathered rows for bf16 storage (gfx950).
//
// Per sequence a projection multiplies at most 144 rows by a large weight, so
// the kernel is organised around moving bytes: every 32-wide K step is one
// pipeline stage that holds the A fragments of all row tiles and the weight
// fragments of the workgroup.  Stages are filled by direct global -> LDS loads
// (global_load_lds_dwordx4, no VGPR staging) in a ring of P buffers; stage s is
// consumed after a wait that leaves the P-2 younger stages in flight and one
// workgroup barrier.  Each ring buffer is its own LDS object, which lets the
// compiler see that reads of one stage do not alias the loads still landing in
// the others.
//
// Waves form RG row groups x CG column groups: the CG waves of a row group read
// the same A fragments, the RG waves of a column group the same weight
// fragments.  Row tiles are dealt to the row groups in turn and the shapes used
// have RG = 2 and CG = 4 where it matters, so each SIMD holds one wave of each row
// group and carries the same number of matrix products: with hi/lo planes and
// real data the products are what the projection's time depends on once the
// stream is fed.  Fragments are 16x16x32 MFMA operands in lane order.  Weights are
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
#include <utility>

#include "kernels.h"

namespace {

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void gbl_void;

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
#define DL_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | (0x7 << 4) | (0xF << 8))

PS_DEV floatx4_t mfma_bf16(uint4 a, uint4 w, floatx4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, w), c,
                                                 0, 0, 0);
}

template <int RTW, int RG, int CG, int NSUB, int PL>
struct DlCfg {
  static constexpr int NWV = RG * CG;              // waves per workgroup
  static constexpr int RT = RTW * RG;              // 16-row tiles per workgroup
  static constexpr int FA = PL * RT;               // A fragments per stage
  static constexpr int F = FA + CG * NSUB;         // fragments per stage
  static constexpr int LPW = (F + NWV - 1) / NWV;  // direct loads per wave per stage
  static constexpr int STAGE = F * 1024;           // bytes
  static constexpr int P0 = (150 * 1024 - 1024) / STAGE;
  static constexpr int P = P0 > 8 ? 8 : P0;        // ring depth
  static constexpr int NCOL = CG * NSUB * 16;      // columns per workgroup
  static_assert(P >= 3, "pipeline needs three stages");
  static_assert(LPW * (P - 2) < 64, "vmcnt range");
};

template <typename T, int RTW, int RG, int CG, int NSUB, int PL, int KIND>
__global__ __launch_bounds__(64 * RG * CG) void dl_kernel(DlArgs g) {
  using C = DlCfg<RTW, RG, CG, NSUB, PL>;
  constexpr int NWV = C::NWV, RT = C::RT, FA = C::FA, F = C::F, LPW = C::LPW, P = C::P;
  // ring stages (only the first P are referenced) and one slot that the padding loads of the
  // waves with fewer than LPW fragments write to and nothing reads
  __shared__ uint4 b0[F * 64], b1[F * 64], b2[F * 64], b3[F * 64], b4[F * 64], b5[F * 64], b6[F * 64],
      b7[F * 64], bd[64];
  auto bp = [&](auto I) -> uint4* {
    if constexpr (I == 0) return b0;
    else if constexpr (I == 1) return b1;
    else if constexpr (I == 2) return b2;
    else if constexpr (I == 3) return b3;
    else if constexpr (I == 4) return b4;
    else if constexpr (I == 5) return b5;
    else if constexpr (I == 6) return b6;
    else return b7;
  };
  const int nt = blockIdx.x, b = blockIdx.y, sp = blockIdx.z;
  int rows_b = g.A.rows(b);
  if (rows_b > RT * 16) rows_b = RT * 16;
  if (rows_b <= 0) return;
  const int nrt = (rows_b + 15) >> 4;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rg = wave / CG, cg = wave % CG;
  const int k32n = g.K >> 5;
  const int g0 = (int)((int64_t)k32n * sp / g.ksplit), g1 = (int)((int64_t)k32n * (sp + 1) / g.ksplit);
  const int n = g1 - g0;

  // Per load slot: source address of this lane at step 0 of the range, and the step stride.
  // Slots past the fragment count and A slots of row tiles without rows re-read one fixed
  // 16-byte location every step (stride 0): it stays in the vector L1 and costs no L2 or HBM
  // traffic, while every wave keeps the same number of loads per stage for the waits.
  const char* src[LPW];
  int stride[LPW];
  const uint16_t* Ab = (const uint16_t*)g.A.base + (int64_t)b * g.A.bstride;
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    int f = i * NWV + wave;
    const bool idle = f >= F || (f < FA && (f % RT) >= nrt);
    if (idle) {
      src[i] = (const char*)(Ab + 8 * (lane >> 4));
      stride[i] = 0;
      continue;
    }
    if (f < FA) {
      const int p = f / RT, rt = f % RT;
      if (g.A.tiles > 0) {   // fragment-packed: step s, plane p, tile rt
        src[i] = (const char*)(Ab + ((((int64_t)g0 * PL + p) * g.A.tiles + rt) * 64 + lane) * 8);
        stride[i] = PL * g.A.tiles * 1024;
      } else {
        int r = rt * 16 + (lane & 15);
        if (r >= rows_b) r = 0;
        src[i] = (const char*)(Ab + p * g.A.plane_stride + g.A.src_row(b, r) * g.A.lda + (int64_t)g0 * 32 +
                               8 * (lane >> 4));
        stride[i] = 64;
      }
    } else {
      // subtile n16 of group n16 / wg (packed groups are padded, so every subtile exists)
      const int n16 = nt * CG * NSUB + (f - FA);
      src[i] = (const char*)((const uint4*)g.W + (((int64_t)(n16 / g.wg) * k32n + g0) * g.wg + n16 % g.wg) * 64 + lane);
      stride[i] = 1024 * g.wg;
    }
  }
  auto issue = [&](uint4* buf, int step) {
    step = step < n ? step : n - 1;   // past the range: reload the last step (unused)
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int slot = i * NWV + wave;
      __builtin_amdgcn_global_load_lds((gbl_void*)(src[i] + (int64_t)step * stride[i]),
                                       (lds_void*)(slot < F ? &buf[slot * 64] : bd), 16, 0, 0);
    }
  };

  floatx4_t acc[RTW][NSUB];
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
    for (int sb = 0; sb < NSUB; ++sb) acc[rt][sb] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  // Row tiles are dealt to the row groups in turn (tile j*RG + rg is this wave's j-th), so the
  // waves of a workgroup differ by at most one tile; a wave's tile count is uniform, and the
  // loop below is instantiated once per count so that every stage reads all of its fragments
  // before its first product, with no per-tile branch.
  const int my_tiles = __builtin_amdgcn_readfirstlane(nrt > rg ? min(RTW, (nrt - rg + RG - 1) / RG) : 0);
  auto run = [&](auto NTc) {
    constexpr int NT = decltype(NTc)::value;
    auto compute = [&](const uint4* buf) {
      uint4 w[NSUB], a[PL][NT > 0 ? NT : 1];
#pragma unroll
      for (int sb = 0; sb < NSUB; ++sb) w[sb] = buf[(FA + cg * NSUB + sb) * 64 + lane];
#pragma unroll
      for (int p = 0; p < PL; ++p)
#pragma unroll
        for (int j = 0; j < NT; ++j) a[p][j] = buf[(p * RT + j * RG + rg) * 64 + lane];
#pragma unroll
      for (int p = 0; p < PL; ++p)
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
          for (int sb = 0; sb < NSUB; ++sb) acc[j][sb] = mfma_bf16(a[p][j], w[sb], acc[j][sb]);
    };
    [&]<int... U>(std::integer_sequence<int, U...>) {
      (issue(bp(std::integral_constant<int, U>{}), U), ...);
    }(std::make_integer_sequence<int, P - 1>{});
    for (int s = 0; s < n; s += P) {
      [&]<int... U>(std::integer_sequence<int, U...>) {
        ([&] {
          DL_VMCNT(LPW * (P - 2));          // this wave's loads of stage s+U have landed
          __builtin_amdgcn_s_barrier();     // ... and everyone's; stage s+U-1 is fully consumed
          issue(bp(std::integral_constant<int, (U + P - 1) % P>{}), s + U + P - 1);
          if (NT > 0 && s + U < n) compute(bp(std::integral_constant<int, U>{}));
        }(), ...);
      }(std::make_integer_sequence<int, P>{});
    }
  };
  [&]<int... V>(std::integer_sequence<int, V...>) {
    ((my_tiles == V ? (run(std::integral_constant<int, V>{}), 0) : 0), ...);
  }(std::make_integer_sequence<int, RTW + 1>{});
  DL_VMCNT(0);   // no load may land in LDS after the workgroup ends

  // accumulator element (rt, sb, i) of this lane: row r, column n
  const int col0 = (nt * CG + cg) * NSUB * 16 + (lane & 15);
  const int row0 = rg * 16 + 4 * (lane >> 4);   // accumulator tile j holds rows of tile j*RG + rg
  if (g.ksplit > 1 || KIND == EPI_PARTIAL) {
    float* out = g.part + ((int64_t)sp * g.batch + b) * g.part_rows * g.N;
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
      for (int sb = 0; sb < NSUB; ++sb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = row0 + rt * RG * 16 + i, c = col0 + sb * 16;
          if (r < rows_b && c < g.N) out[(int64_t)r * g.N + c] = acc[rt][sb][i];
        }
    return;
  }
  if constexpr (KIND == EPI_QKV || KIND == EPI_KV) {
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
      for (int sb = 0; sb < NSUB; ++sb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = row0 + rt * RG * 16 + i, c = col0 + sb * 16;
          if (r < rows_b && c < g.N) {
            if constexpr (KIND == EPI_QKV) epi_qkv_elem<T>(g.e, b, r, c, acc[rt][sb][i]);
            else epi_kv_elem<T>(g.e, b, r, c, acc[rt][sb][i]);
          }
        }
  } else if constexpr (KIND == EPI_SWIGLU) {
    // subtile pairs (2j, 2j+1) are the gate and up weights of 16 consecutive FFN columns
    static_assert(NSUB % 2 == 0, "gate/up pairs inside one wave");
    const EpiParams& e = g.e;
    bf16_t* act = (bf16_t*)e.act + (int64_t)b * 2 * e.act_rows * e.ffn;
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
      for (int j = 0; j < NSUB / 2; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = row0 + rt * RG * 16 + i;
          const int oc = ((nt * CG + cg) * NSUB / 2 + j) * 16 + (lane & 15);
          if (r < rows_b && oc < e.ffn) {
            const float gv = acc[rt][2 * j][i], uv = acc[rt][2 * j + 1][i];
            const float a = gv / (1.f + expf(-gv)) * uv;
            uint16_t hi, lo;
            split_bf16(a, hi, lo);
            act[apack(r, oc, 0, 2, e.act_tiles)].bits = hi;
            act[apack(r, oc, 1, 2, e.act_tiles)].bits = lo;
          }
        }
  }
}

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
      if (e.chk) *(float4*)(e.chk + ((int64_t)b * e.chk_rows + r) * e.chk_ld + c) = v;
      const QkvDest dst = qkv_dest(e, b, r);
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

template <typename T, int RTW, int RG, int CG, int NSUB, int PL>
hipError_t launch_cfg(const DlArgs& g, hipStream_t s) {
  using C = DlCfg<RTW, RG, CG, NSUB, PL>;
  const dim3 grid(PS_CEIL_DIV(g.N, C::NCOL), g.batch, g.ksplit), block(64 * RG * CG);
  // with split-K every kind writes raw partial sums; its epilogue runs in launch_dl_finish
  switch (g.ksplit > 1 ? (int)EPI_PARTIAL : g.e.kind) {
    case EPI_PARTIAL: hipLaunchKernelGGL((dl_kernel<T, RTW, RG, CG, NSUB, PL, EPI_PARTIAL>), grid, block, 0, s, g); break;
    case EPI_QKV: hipLaunchKernelGGL((dl_kernel<T, RTW, RG, CG, NSUB, PL, EPI_QKV>), grid, block, 0, s, g); break;
    case EPI_KV: hipLaunchKernelGGL((dl_kernel<T, RTW, RG, CG, NSUB, PL, EPI_KV>), grid, block, 0, s, g); break;
    case EPI_SWIGLU:
      if constexpr (PL == 2 && NSUB % 2 == 0) {
        hipLaunchKernelGGL((dl_kernel<T, RTW, RG, CG, NSUB, PL, EPI_SWIGLU>), grid, block, 0, s, g);
        break;
      }
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

int dl_subtiles_per_wave(int shape) {
  switch (shape) {
    case DL_N192: case DL_W192: case DL_N96: return 3;
    case DL_MID8: return 2;
    default: return 4;
  }
}

int dl_tile_cols(int shape) {
  switch (shape) {
    case DL_WIDE: return 256;
    case DL_N192: case DL_W192: return 192;
    case DL_N96: return 96;
    default: return 128;
  }
}

template <typename T>
hipError_t launch_dl(const DlArgs& g, int shape, int max_rows, hipStream_t s) {
  if constexpr (!std::is_same<T, bf16_t>::value) {
    return hipErrorInvalidValue;
  } else {
    if (max_rows <= 0) return hipSuccess;
    if (g.K % 32 || g.N % 16 || g.ksplit < 1 || g.ksplit > (g.K >> 5)) return hipErrorInvalidValue;
    if (g.wg < 1 || g.wg % (dl_tile_cols(shape) / 16) != 0) return hipErrorInvalidValue;
    if (shape == DL_NARROW || shape == DL_N192 || shape == DL_N96) {   // bf16 rows
      if (g.planes != 1) return hipErrorInvalidValue;
      if (shape == DL_N96) {   // 4 x 2 waves of 48 columns
        if (max_rows <= 64) return launch_cfg<T, 1, 4, 2, 3, 1>(g, s);
        if (max_rows <= 128) return launch_cfg<T, 2, 4, 2, 3, 1>(g, s);
        if (max_rows <= 192) return launch_cfg<T, 3, 4, 2, 3, 1>(g, s);
        return hipErrorInvalidValue;
      }
      if (shape == DL_N192) {   // 2 x 4 waves of 48 columns
        if (max_rows <= 32) return launch_cfg<T, 1, 2, 4, 3, 1>(g, s);
        if (max_rows <= 64) return launch_cfg<T, 2, 2, 4, 3, 1>(g, s);
        if (max_rows <= 96) return launch_cfg<T, 3, 2, 4, 3, 1>(g, s);
        if (max_rows <= 128) return launch_cfg<T, 4, 2, 4, 3, 1>(g, s);
        if (max_rows <= 160) return launch_cfg<T, 5, 2, 4, 3, 1>(g, s);
        if (max_rows <= 192) return launch_cfg<T, 6, 2, 4, 3, 1>(g, s);
        return hipErrorInvalidValue;
      }
      if (max_rows <= 48) return launch_cfg<T, 1, 3, 2, 4, 1>(g, s);
      if (max_rows <= 96) return launch_cfg<T, 2, 3, 2, 4, 1>(g, s);
      if (max_rows <= 144) return launch_cfg<T, 3, 3, 2, 4, 1>(g, s);
      if (max_rows <= 192) return launch_cfg<T, 4, 3, 2, 4, 1>(g, s);
      return hipErrorInvalidValue;
    }
    if (g.planes != 2) return hipErrorInvalidValue;
    if (shape == DL_MID8) {   // 2 x 4 waves of 32 columns, hi/lo planes
      if (max_rows <= 32) return launch_cfg<T, 1, 2, 4, 2, 2>(g, s);
      if (max_rows <= 64) return launch_cfg<T, 2, 2, 4, 2, 2>(g, s);
      if (max_rows <= 96) return launch_cfg<T, 3, 2, 4, 2, 2>(g, s);
      if (max_rows <= 128) return launch_cfg<T, 4, 2, 4, 2, 2>(g, s);
      if (max_rows <= 160) return launch_cfg<T, 5, 2, 4, 2, 2>(g, s);
      if (max_rows <= 192) return launch_cfg<T, 6, 2, 4, 2, 2>(g, s);
      return hipErrorInvalidValue;
    }
    if (shape == DL_W192) {   // 2 x 4 waves of 48 columns, hi/lo planes
      if (max_rows <= 32) return launch_cfg<T, 1, 2, 4, 3, 2>(g, s);
      if (max_rows <= 64) return launch_cfg<T, 2, 2, 4, 3, 2>(g, s);
      if (max_rows <= 96) return launch_cfg<T, 3, 2, 4, 3, 2>(g, s);
      if (max_rows <= 128) return launch_cfg<T, 4, 2, 4, 3, 2>(g, s);
      if (max_rows <= 160) return launch_cfg<T, 5, 2, 4, 3, 2>(g, s);
      if (max_rows <= 192) return launch_cfg<T, 6, 2, 4, 3, 2>(g, s);
      return hipErrorInvalidValue;
    }
    if (shape == DL_WIDE) {   // 2 x 4 waves, hi/lo planes
      if (max_rows <= 32) return launch_cfg<T, 1, 2, 4, 4, 2>(g, s);
      if (max_rows <= 64) return launch_cfg<T, 2, 2, 4, 4, 2>(g, s);
      if (max_rows <= 96) return launch_cfg<T, 3, 2, 4, 4, 2>(g, s);
      if (max_rows <= 128) return launch_cfg<T, 4, 2, 4, 4, 2>(g, s);
      if (max_rows <= 160) return launch_cfg<T, 5, 2, 4, 4, 2>(g, s);
      if (max_rows <= 192) return launch_cfg<T, 6, 2, 4, 4, 2>(g, s);
      return hipErrorInvalidValue;
    }
    if (shape == DL_MID) {    // 2 x 2 waves, hi/lo planes
      if (max_rows <= 32) return launch_cfg<T, 1, 2, 2, 4, 2>(g, s);
      if (max_rows <= 64) return launch_cfg<T, 2, 2, 2, 4, 2>(g, s);
      if (max_rows <= 96) return launch_cfg<T, 3, 2, 2, 4, 2>(g, s);
      if (max_rows <= 128) return launch_cfg<T, 4, 2, 2, 4, 2>(g, s);
      if (max_rows <= 160) return launch_cfg<T, 5, 2, 2, 4, 2>(g, s);
      if (max_rows <= 192) return launch_cfg<T, 6, 2, 2, 4, 2>(g, s);
      return hipErrorInvalidValue;
    }
    return hipErrorInvalidValue;
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
