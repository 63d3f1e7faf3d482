// Weight-streaming projection kernel of the gathered rows (bf16 storage, gfx950); its design is
// described at the top of gemm_dl.hip.  Included by the per-shape translation units.
#pragma once
#include <utility>

#include "kernels.h"

namespace dl_impl {

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void gbl_void;

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
#define DL_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | (0x7 << 4) | (0xF << 8))
// The same with every LDS read of the wave complete as well (lgkmcnt 0).  Taken before each ring
// barrier: the barrier releases the stage read last for the loads issued after it, and a read
// still queued in the LDS unit could otherwise return data those loads already wrote.
#define DL_WAIT(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | (0x7 << 4))

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
  // ring depth: four stages where they fit (three in flight while one is read).  The weight
  // stream is already saturated at that depth, and deeper rings only unroll more code.
  static constexpr int P0 = (150 * 1024 - 1024) / STAGE;
  static constexpr int P = P0 > 4 ? 4 : P0;
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
  __shared__ uint4 b0[F * 64], b1[F * 64], b2[F * 64], b3[F * 64], bd[64];
  auto bp = [&](auto I) -> uint4* {
    if constexpr (I == 0) return b0;
    else if constexpr (I == 1) return b1;
    else if constexpr (I == 2) return b2;
    else return b3;
  };
  // Workgroup -> (sequence b, column tile nt, split sp).  Workgroups are handed to the 8 XCDs
  // in turn (id % 8), each XCD with its own L2: the ids of one XCD take one (tile, split) for
  // all sequences in a row, so that a weight tile's repeats for the other sequences come from
  // that XCD's L2.  With one sequence this is the identity (tile-major, split outer).
  int b, nt, sp;
  {
    const int id = blockIdx.x, q = id >> 3;
    const int t = (q / g.batch) * 8 + (id & 7);
    const int ntiles = PS_CEIL_DIV(g.N, C::NCOL);
    if (t >= ntiles * g.ksplit) return;
    b = q % g.batch;
    nt = t % ntiles;
    sp = t / ntiles;
  }
  // this launch's slab: rows [row0, row0 + RT*16) of the sequence; r below is slab-local
  const int row0 = g.A.row0;
  int rows_b = g.A.rows(b) - row0;
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
        src[i] = (const char*)(Ab + ((((int64_t)g0 * PL + p) * g.A.tiles + (row0 >> 4) + rt) * 64 + lane) * 8);
        stride[i] = PL * g.A.tiles * 1024;
      } else {
        int r = rt * 16 + (lane & 15);
        if (r >= rows_b) r = 0;
        src[i] = (const char*)(Ab + p * g.A.plane_stride + g.A.src_row(b, row0 + r) * g.A.lda + (int64_t)g0 * 32 +
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
          DL_WAIT(LPW * (P - 2));           // this wave's loads of stage s+U have landed, its
          __builtin_amdgcn_s_barrier();     // reads of s+U-1 are done; after the barrier both
                                            // hold for every wave
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
  const int rrow0 = rg * 16 + 4 * (lane >> 4);   // accumulator tile j holds rows of tile j*RG + rg
  if (g.ksplit > 1 || KIND == EPI_PARTIAL) {
    float* out = g.part + ((int64_t)sp * g.batch + b) * g.part_rows * g.N;
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
      for (int sb = 0; sb < NSUB; ++sb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = rrow0 + rt * RG * 16 + i, c = col0 + sb * 16;
          if (r < rows_b && c < g.N) out[(int64_t)(row0 + r) * g.N + c] = acc[rt][sb][i];
        }
    return;
  }
  if constexpr (KIND == EPI_LMSTAT) {
    // LM-head statistics of this workgroup's NCOL vocabulary ids per row: max logit, sum of
    // exp(logit - max), best logit among ids != mask_id with its id (lowest on ties).  Each lane
    // combines its subtiles (ascending ids), the 16 lanes of a row group by an xor tree, the
    // column waves of a row in order through LDS.
    static_assert(PL == 1, "LM head: one bf16 plane");
    __shared__ float lmst[CG][RT * 16][4];
    const EpiParams& e = g.e;
    auto comb = [](float& m, float& s, float& v, int& id, float m2, float s2, float v2, int id2) {
      const float M = fmaxf(m, m2);
      s = M == -INFINITY ? 0.f : s * expf(m - M) + s2 * expf(m2 - M);
      m = M;
      if (v2 > v || (v2 == v && id2 < id)) {
        v = v2;
        id = id2;
      }
    };
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float m = -INFINITY, s = 0.f, v = -INFINITY;
        int id = 0x7fffffff;
#pragma unroll
        for (int sb = 0; sb < NSUB; ++sb) {
          const int c = col0 + sb * 16;
          const bool ok = c < e.vocab;
          const float l = ok ? acc[rt][sb][i] : -INFINITY;
          comb(m, s, v, id, l, ok ? 1.f : 0.f, (ok && c != e.mask_id) ? l : -INFINITY, c);
        }
#pragma unroll
        for (int o = 8; o > 0; o >>= 1)
          comb(m, s, v, id, __shfl_xor(m, o, 64), __shfl_xor(s, o, 64), __shfl_xor(v, o, 64), __shfl_xor(id, o, 64));
        if ((lane & 15) == 0) {
          const int rl = (rt * RG + rg) * 16 + 4 * (lane >> 4) + i;
          lmst[cg][rl][0] = m;
          lmst[cg][rl][1] = s;
          lmst[cg][rl][2] = v;
          lmst[cg][rl][3] = __int_as_float(id);
        }
      }
    __syncthreads();
    for (int rl = threadIdx.x; rl < RT * 16; rl += blockDim.x) {
      if (rl >= rows_b) continue;
      float m = lmst[0][rl][0], s = lmst[0][rl][1], v = lmst[0][rl][2];
      int id = __float_as_int(lmst[0][rl][3]);
      for (int c2 = 1; c2 < CG; ++c2)
        comb(m, s, v, id, lmst[c2][rl][0], lmst[c2][rl][1], lmst[c2][rl][2], __float_as_int(lmst[c2][rl][3]));
      float* st = e.lm_stats + (((int64_t)b * e.lm_rows + row0 + rl) * e.lm_tiles + nt) * 4;
      st[0] = m;
      st[1] = s;
      st[2] = v;
      st[3] = __int_as_float(v == -INFINITY ? -1 : id);
    }
  } else if constexpr (KIND == EPI_QKV || KIND == EPI_KV) {
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
      for (int sb = 0; sb < NSUB; ++sb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = rrow0 + rt * RG * 16 + i, c = col0 + sb * 16;
          if (r < rows_b && c < g.N) {
            if constexpr (KIND == EPI_QKV) epi_qkv_elem<T>(g.e, b, row0 + r, c, acc[rt][sb][i]);
            else epi_kv_elem<T>(g.e, b, row0 + r, c, acc[rt][sb][i]);
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
          const int r = rrow0 + rt * RG * 16 + i;
          const int oc = ((nt * CG + cg) * NSUB / 2 + j) * 16 + (lane & 15);
          if (r < rows_b && oc < e.ffn) {
            const float gv = acc[rt][2 * j][i], uv = acc[rt][2 * j + 1][i];
            const float a = gv / (1.f + expf(-gv)) * uv;
            uint16_t hi, lo;
            split_bf16(a, hi, lo);
            act[apack(row0 + r, oc, 0, 2, e.act_tiles)].bits = hi;
            act[apack(row0 + r, oc, 1, 2, e.act_tiles)].bits = lo;
          }
        }
  }
}

template <typename T, int RTW, int RG, int CG, int NSUB, int PL>
hipError_t launch_cfg(const DlArgs& g, hipStream_t s) {
  using C = DlCfg<RTW, RG, CG, NSUB, PL>;
  const int tiles = PS_CEIL_DIV(g.N, C::NCOL) * g.ksplit;
  const dim3 grid(8 * g.batch * PS_CEIL_DIV(tiles, 8)), block(64 * RG * CG);
  // with split-K every kind writes raw partial sums; its epilogue runs in launch_dl_finish
  switch (g.ksplit > 1 ? (int)EPI_PARTIAL : g.e.kind) {
    case EPI_PARTIAL: hipLaunchKernelGGL((dl_kernel<T, RTW, RG, CG, NSUB, PL, EPI_PARTIAL>), grid, block, 0, s, g); break;
    case EPI_QKV: hipLaunchKernelGGL((dl_kernel<T, RTW, RG, CG, NSUB, PL, EPI_QKV>), grid, block, 0, s, g); break;
    case EPI_KV: hipLaunchKernelGGL((dl_kernel<T, RTW, RG, CG, NSUB, PL, EPI_KV>), grid, block, 0, s, g); break;
    case EPI_LMSTAT:
      if constexpr (PL == 1) {
        hipLaunchKernelGGL((dl_kernel<T, RTW, RG, CG, NSUB, PL, EPI_LMSTAT>), grid, block, 0, s, g);
        break;
      }
      return hipErrorInvalidValue;
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


// Launch of one workgroup shape (RG x CG waves of NSUB subtiles, PL planes) with the row-tile
// count per wave that covers max_rows (at most 192 rows: one slab; the 512-column shapes have
// launchers of their own with 128-row slabs).
template <int RG, int CG, int NSUB, int PL>
hipError_t launch_shape(const DlArgs& g, int max_rows, hipStream_t s) {
  constexpr int kMax = 192 / (16 * RG);
  const int rtw = PS_CEIL_DIV(max_rows, 16 * RG);
  hipError_t e = hipErrorInvalidValue;
  [&]<int... R>(std::integer_sequence<int, R...>) {
    ((rtw == R + 1 ? (e = launch_cfg<bf16_t, R + 1, RG, CG, NSUB, PL>(g, s), 0) : 0), ...);
  }(std::make_integer_sequence<int, kMax>{});
  return e;
}

}  // namespace dl_impl

// One launcher per workgroup shape, each in its own translation unit (they compile in parallel).
hipError_t dl_launch_narrow(const DlArgs& g, int max_rows, hipStream_t s);
hipError_t dl_launch_n192(const DlArgs& g, int max_rows, hipStream_t s);
hipError_t dl_launch_n96(const DlArgs& g, int max_rows, hipStream_t s);
hipError_t dl_launch_wide(const DlArgs& g, int max_rows, hipStream_t s);
hipError_t dl_launch_mid(const DlArgs& g, int max_rows, hipStream_t s);
hipError_t dl_launch_w192(const DlArgs& g, int max_rows, hipStream_t s);
hipError_t dl_launch_mid8(const DlArgs& g, int max_rows, hipStream_t s);
hipError_t dl_launch_p96(const DlArgs& g, int max_rows, hipStream_t s);
hipError_t dl_launch_p160(const DlArgs& g, int max_rows, hipStream_t s);
hipError_t dl_launch_x512(const DlArgs& g, int max_rows, hipStream_t s);
