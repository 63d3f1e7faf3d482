// Window clustering kernels: spherical k-means at block entry, the per-step
// window update (dequantise, patch from the update packet, fixed-label centroid
// refresh, NVFP4 re-quantisation), the QKV row staging, and the NVFP4 codec
// test hooks.  Cosines and centroid sums are accumulated in float64 so that the
// integer decisions (labels) do not depend on the summation order.
#include "kernels.h"

namespace {

// Row reduction in float64 over a whole workgroup (fixed order).
PS_DEV double block_sum_d(double v, double* red) { return block_sum<double>(v, red); }

// ---- block entry: spherical k-means, spread over the chip ------------------------------------
// Lloyd iterations in float64 as a chain of small launches: unit rows (one workgroup per window
// row), then per iteration assign (one workgroup per row), update (one workgroup per 256-column
// chunk and cluster: member sums and the chunk's sum of squares) and finish (same grid: the norm
// of the whole sum from the chunk partials in chunk order, then the new centroid columns); last,
// labels and rounded centroids, and the residual codes of each row.  Every sum runs in a fixed
// order, so the labels do not depend on scheduling.

// Window row w of sequence b in the entry rows: row w of a window block, or the row at its
// position among all positions.
template <typename T>
PS_DEV const T* entry_row(const ClusterArgs& a, int b, int w) {
  const int64_t rows = a.entry_full ? a.n_pos : a.win_max;
  const int64_t r = a.entry_full ? a.geom.pos(w) : w;
  return (const T*)a.entry_h + ((int64_t)b * rows + r) * a.d;
}

// Sum of vals[0..n) in index order, the values first gathered into LDS by up to blockDim.x
// threads at once (so their loads overlap); every thread gets the sum.  n <= kGather.
constexpr int kGather = 512;
PS_DEV double gather_sum(const double* vals, int n, double* sh) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) sh[i] = vals[i];
  __syncthreads();
  double s = 0.0;
  for (int i = 0; i < n; ++i) s += sh[i];
  __syncthreads();
  return s;
}

// Unit row (a zero row stays zero); raw storage copies the row into the window; the workgroup of
// the row named by init_idx[c] seeds centroid c (row 0's workgroup zeroes the clusters with no
// valid seed).  1024 threads: a 4096-wide row is one load per thread.
template <typename T>
__global__ __launch_bounds__(1024) void km_unit_kernel(ClusterArgs a) {
  __shared__ double red[16];
  const int w = blockIdx.x, b = blockIdx.y, d = a.d, K = a.K, nwin = a.geom.n_win;
  const int keff = min(K, nwin);
  const T* src = entry_row<T>(a, b, w);
  double ss = 0.0;
  for (int n = threadIdx.x; n < d; n += blockDim.x) {
    const double x = St<T>::load(src, n);
    ss += x * x;
  }
  ss = block_sum_d(ss, red);
  const double nr = sqrt(ss);
  double* xh = a.xhat + ((int64_t)b * a.win_max + w) * d;
  const bool copy = !a.resid && (a.entry_full || a.win_h != a.entry_h);
  T* wrow = (T*)a.win_h + ((int64_t)b * a.win_max + w) * d;
  for (int n = threadIdx.x; n < d; n += blockDim.x) {
    const float x = St<T>::load(src, n);
    xh[n] = nr > 0.0 ? (double)x / nr : 0.0;
    if (copy) wrow[n] = src[n];
  }
  double* z = a.z64 + (int64_t)b * K * d;
  for (int c = 0; c < K; ++c) {
    int r = c < keff ? a.init_idx[(int64_t)b * K + c] : -1;
    if (r < 0 || r >= nwin) r = -1;
    if (r == w || (r < 0 && w == 0))
      for (int n = threadIdx.x; n < d; n += blockDim.x) z[(int64_t)c * d + n] = r >= 0 ? xh[n] : 0.0;
  }
}

// Largest cosine over the first keff centroids, lowest index on ties.  1024 threads, the column
// loop unrolled so that a thread's loads are in flight together.
constexpr int kKmMax = 16;   // clusters per sequence (the handle's limit)
__global__ __launch_bounds__(1024) void km_assign_kernel(ClusterArgs a) {
  __shared__ double red[16][kKmMax];
  const int w = blockIdx.x, b = blockIdx.y, d = a.d, K = a.K;
  const int keff = min(K, a.geom.n_win);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwv = blockDim.x >> 6;
  const double* xh = a.xhat + ((int64_t)b * a.win_max + w) * d;
  const double* z = a.z64 + (int64_t)b * K * d;
  double t[kKmMax];
#pragma unroll
  for (int c = 0; c < kKmMax; ++c) t[c] = 0.0;
  int n = threadIdx.x;
  for (; n + blockDim.x < d; n += 2 * blockDim.x) {
    const double x0 = xh[n], x1 = xh[n + blockDim.x];
#pragma unroll
    for (int c = 0; c < kKmMax; ++c)
      if (c < keff) t[c] += x0 * z[(int64_t)c * d + n] + x1 * z[(int64_t)c * d + n + blockDim.x];
  }
  if (n < d) {
    const double x0 = xh[n];
#pragma unroll
    for (int c = 0; c < kKmMax; ++c)
      if (c < keff) t[c] += x0 * z[(int64_t)c * d + n];
  }
#pragma unroll
  for (int c = 0; c < kKmMax; ++c)
    if (c < keff) {
      const double v = wave_sum(t[c]);
      if (lane == 0) red[wave][c] = v;
    }
  __syncthreads();
  if (threadIdx.x == 0) {
    int bc = 0;
    double bv = -INFINITY;
    for (int c = 0; c < keff; ++c) {
      double v = 0.0;
      for (int i = 0; i < nwv; ++i) v += red[i][c];
      if (v > bv) {
        bv = v;
        bc = c;
      }
    }
    a.km_lab[(int64_t)b * a.win_max + w] = bc;
    a.wnorm[(int64_t)b * a.win_max + w] = bv;   // best cosine of the row
  }
}

// Member sum of cluster c over one 256-column chunk, and the chunk's sum of squares.  The members
// are listed in LDS first, so each thread's loads of member values overlap.  The first workgroup
// of a sequence also records the objective after the assignment.
__global__ __launch_bounds__(256) void km_update_kernel(ClusterArgs a, int it) {
  __shared__ int lab[256];
  __shared__ int mem[256];
  __shared__ int nmem_sh;
  __shared__ double red[kGather];
  const int ch = blockIdx.x, c = blockIdx.y, b = blockIdx.z, d = a.d, K = a.K, nwin = a.geom.n_win;
  for (int w = threadIdx.x; w < nwin; w += blockDim.x) lab[w] = a.km_lab[(int64_t)b * a.win_max + w];
  __syncthreads();
  if (threadIdx.x == 0) {
    int k = 0;
    for (int w = 0; w < nwin; ++w)
      if (lab[w] == c) mem[k++] = w;
    nmem_sh = k;
    if (ch == 0) a.km_cnt[(int64_t)b * K + c] = k;
  }
  __syncthreads();
  const int nmem = nmem_sh;
  if (ch == 0 && c == 0 && a.objective) {
    const double J = gather_sum(a.wnorm + (int64_t)b * a.win_max, nwin, red);
    if (threadIdx.x == 0) a.objective[(int64_t)b * 2 * a.iters + 2 * it] = J;
  }
  if (nmem == 0) return;   // an empty cluster keeps its centroid
  const int n = ch * 256 + threadIdx.x;
  double s = 0.0;
  if (n < d) {
    const double* xh = a.xhat + (int64_t)b * a.win_max * d + n;
    int j = 0;
    for (; j + 4 <= nmem; j += 4) {
      double v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = xh[(int64_t)mem[j + u] * d];
#pragma unroll
      for (int u = 0; u < 4; ++u) s += v[u];
    }
    for (; j < nmem; ++j) s += xh[(int64_t)mem[j] * d];
    a.km_sum[((int64_t)b * K + c) * d + n] = s;
  }
  const double ss = block_sum_d(s * s, red);
  if (threadIdx.x == 0) a.cpart[((int64_t)b * K + c) * a.nchunk + ch] = ss;
}

// New centroid columns: the member sum over the norm of the whole sum (kept when the sum
// vanishes).  The first workgroup of a sequence records the objective after the update, the sum
// of those norms over the non-empty clusters.
__global__ __launch_bounds__(256) void km_finish_kernel(ClusterArgs a, int it) {
  __shared__ double sh[kGather];
  __shared__ double norms[kKmMax];
  const int ch = blockIdx.x, c = blockIdx.y, b = blockIdx.z, d = a.d, K = a.K;
  const int keff = min(K, a.geom.n_win);
  const double* cp = a.cpart + (int64_t)b * K * a.nchunk;
  if (ch == 0 && c == 0 && a.objective) {
    // norms of every cluster: chunk partials gathered at once, each cluster's added in chunk order
    for (int i = threadIdx.x; i < keff * a.nchunk; i += blockDim.x) sh[i] = cp[i];
    __syncthreads();
    if (threadIdx.x < keff) {
      double ss = 0.0;
      for (int k = 0; k < a.nchunk; ++k) ss += sh[threadIdx.x * a.nchunk + k];
      norms[threadIdx.x] = a.km_cnt[(int64_t)b * K + threadIdx.x] > 0 ? sqrt(ss) : 0.0;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      double J = 0.0;
      for (int cc = 0; cc < keff; ++cc) J += norms[cc];
      a.objective[(int64_t)b * 2 * a.iters + 2 * it + 1] = J;
    }
  }
  if (a.km_cnt[(int64_t)b * K + c] == 0) return;
  const double ns = sqrt(gather_sum(cp + (int64_t)c * a.nchunk, a.nchunk, sh));
  const int n = ch * 256 + threadIdx.x;
  if (ns > 0.0 && n < d)
    a.z64[((int64_t)b * K + c) * d + n] = a.km_sum[((int64_t)b * K + c) * d + n] / ns;
}

// Labels (0 past the window) and the centroids rounded once to the storage dtype.
template <typename T>
__global__ __launch_bounds__(256) void km_store_kernel(ClusterArgs a) {
  const int c = blockIdx.x, b = blockIdx.y, d = a.d, K = a.K, nwin = a.geom.n_win;
  if (c == 0 && threadIdx.x == 0 && a.q_ok) a.q_ok[b] = 0;   // every window row changed
  if (c == 0)
    for (int w = threadIdx.x; w < a.win_max; w += blockDim.x)
      a.win_m[(int64_t)b * a.win_max + w] = (w < nwin && a.iters > 0) ? a.km_lab[(int64_t)b * a.win_max + w] : 0;
  for (int n = threadIdx.x; n < d; n += blockDim.x)
    St<T>::store_d((T*)a.win_z + ((int64_t)b * K + c) * d, n, a.z64[((int64_t)b * K + c) * d + n]);
}

// Residual codes of window row w against its stored centroid, one group per thread.
template <typename T>
__global__ __launch_bounds__(256) void km_resid_kernel(ClusterArgs a) {
  const int w = blockIdx.x, b = blockIdx.y, d = a.d;
  const int G = resid_group(a.resid), ng = d / G;
  const int c = a.iters > 0 ? a.km_lab[(int64_t)b * a.win_max + w] : 0;
  const T* src = entry_row<T>(a, b, w);
  const T* zc = (const T*)a.win_z + ((int64_t)b * a.K + c) * d;
  const int64_t row = (int64_t)b * a.win_max + w;
  const int64_t cb = resid_code_bytes(a.resid, d), sb = resid_scale_bytes(a.resid, d);
  for (int g = threadIdx.x; g < ng; g += blockDim.x) {
    float r[32];
    for (int e = 0; e < G; ++e) r[e] = St<T>::load(src, g * G + e) - St<T>::load(zc, g * G + e);
    resid_encode_group(a.resid, r, a.codes + row * cb, a.scales + row * sb, g * G);
  }
}

// ---- per refresh step: window update ---------------------------------------------------------
// Three passes, each spread over the whole chip:
//   rows:    one workgroup per window row -> current row (packet row, else the stored row or
//            centroid + dequantised residual), patch flag, float64 norm;
//   sum:     one workgroup per (256-column chunk, cluster, sequence) -> float64 normalised
//            member sum of its columns and the chunk's sum of squares;
//   finish:  same grid -> the norm of the whole sum (chunk partials added in chunk order),
//            the new centroid columns and, for NVFP4 storage, the members' re-quantised groups.
constexpr int kChunk = 256;

// Window rows of sequence b labelled c, ascending, into mem[] (with the reciprocals of their norms,
// 0 for a zero row, when rinv != null).  Returns the member count; every thread of the
// 256-thread workgroup gets it.
PS_DEV int members_of(const ClusterArgs& a, int b, int c, int* mem, double* rinv, int* wcnt) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t wbase = (int64_t)b * a.win_max;
  // the norm is loaded with the label (one round trip for both)
  const double nr = (rinv && tid < a.geom.n_win) ? a.wnorm[wbase + tid] : 0.0;
  const bool in = tid < a.geom.n_win && a.win_m[wbase + tid] == c;
  const unsigned long long m = __ballot(in);
  if (lane == 0) wcnt[wave] = __popcll(m);
  __syncthreads();
  int off = 0, tot = 0;
  for (int w = 0; w < 4; ++w) {
    off += w < wave ? wcnt[w] : 0;
    tot += wcnt[w];
  }
  if (in) {
    const int pos = off + __popcll(m & ((1ull << lane) - 1ull));
    mem[pos] = tid;
    if (rinv) rinv[pos] = nr > 0.0 ? 1.0 / nr : 0.0;
  }
  __syncthreads();
  return tot;
}

template <typename T>
__global__ __launch_bounds__(256) void window_rows_kernel(ClusterArgs a) {
  __shared__ double red[4];
  __shared__ int pr_sh;
  const int w = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int d = a.d;
  const int64_t wbase = (int64_t)b * a.win_max;
  int c = a.win_m[wbase + w];   // issued first: its round trip overlaps the packet search
  int cnt = a.u_count ? a.u_count[b] : 0;
  cnt = cnt < 0 ? 0 : (cnt > a.win_max ? a.win_max : cnt);
  if (tid == 0) pr_sh = -1;
  __syncthreads();
  // packet row of this window row (the last one when an index repeats)
  for (int r = tid; r < cnt; r += blockDim.x)
    if (a.u_idx[wbase + r] == w) atomicMax(&pr_sh, r);
  __syncthreads();
  const int pr = pr_sh;
  c = (c < 0 || c >= a.K) ? 0 : c;
  const T* zc = (const T*)a.win_z + ((int64_t)b * a.K + c) * d;
  T* rows = (T*)a.ws_rows;
  const int64_t dst = (wbase + w) * d;
  double ss = 0.0;
  // eight consecutive elements per thread and step (d is a multiple of 16)
  for (int n0 = tid * 8; n0 < d; n0 += blockDim.x * 8) {
    float x[8];
    if (pr >= 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = St<T>::load((const T*)a.u_rows, (wbase + pr) * d + n0 + e);
    } else if (a.resid) {
      const uint8_t* cr = a.codes + (wbase + w) * resid_code_bytes(a.resid, d);
      const uint8_t* sr = a.scales + (wbase + w) * resid_scale_bytes(a.resid, d);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = St<T>::round(St<T>::load(zc, n0 + e) + resid_value(a.resid, cr, sr, n0 + e));
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = St<T>::load((const T*)a.win_h, dst + n0 + e);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      St<T>::store(rows, dst + n0 + e, x[e]);
      if (pr >= 0 && !a.resid) St<T>::store((T*)a.win_h, dst + n0 + e, x[e]);
      ss += (double)x[e] * (double)x[e];
    }
  }
  ss = block_sum_d(ss, red);
  if (tid == 0) {
    a.wnorm[wbase + w] = sqrt(ss);
    a.flags[wbase + w] = pr >= 0;
  }
}

template <typename T>
__global__ __launch_bounds__(256) void centroid_sum_kernel(ClusterArgs a) {
  __shared__ double red[4];
  __shared__ int mem[256];
  __shared__ double rinv[256];
  __shared__ int wcnt[4];
  const int ch = blockIdx.x, c = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int d = a.d, n = ch * kChunk + tid;
  const int nmem = members_of(a, b, c, mem, rinv, wcnt);
  if (nmem == 0) return;
  const int64_t wbase = (int64_t)b * a.win_max;
  const T* rows = (const T*)a.ws_rows;
  double acc = 0.0;   // unit rows added in ascending row order; a zero row adds nothing
  if (n < d) {
    constexpr int U = 16;   // members loaded per batch before they are added
    for (int m0 = 0; m0 < nmem; m0 += U) {
      float x[U];
#pragma unroll
      for (int j = 0; j < U; ++j) x[j] = St<T>::load(rows, (wbase + mem[min(m0 + j, nmem - 1)]) * d + n);
#pragma unroll
      for (int j = 0; j < U; ++j)
        if (m0 + j < nmem) acc += (double)x[j] * rinv[m0 + j];
    }
  }
  if (n < d) a.z64[((int64_t)b * a.K + c) * d + n] = acc;
  const double ss = block_sum_d(acc * acc, red);
  if (tid == 0) a.cpart[((int64_t)b * a.K + c) * a.nchunk + ch] = ss;
}

template <typename T>
__global__ __launch_bounds__(256) void centroid_finish_kernel(ClusterArgs a) {
  __shared__ int mem[256];
  __shared__ int wcnt[4];
  __shared__ float zsh[kChunk];
  __shared__ double gsh[kGather];
  const int ch = blockIdx.x, c = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int d = a.d, n0 = ch * kChunk, n = n0 + tid;
  const int64_t zrow = (int64_t)b * a.K + c;
  // chunk partials loaded before the labels, so the two round trips overlap (nchunk <= 256)
  const double cpv = tid < a.nchunk ? a.cpart[zrow * a.nchunk + tid] : 0.0;
  const int nmem = members_of(a, b, c, mem, nullptr, wcnt);
  if (nmem == 0) return;   // no members: the centroid is kept and no row refers to it
  if (tid < a.nchunk) gsh[tid] = cpv;
  __syncthreads();
  double ss = 0.0;
  for (int i = 0; i < a.nchunk; ++i) ss += gsh[i];   // chunk order
  const double ns = sqrt(ss);
  T* zc = (T*)a.win_z + zrow * d;
  if (n < d) {
    if (ns > 0.0) St<T>::store_d(zc, n, a.z64[zrow * d + n] / ns);   // kept when the sum vanishes
    zsh[tid] = St<T>::load(zc, n);
  }
  if (!a.resid) return;
  __syncthreads();
  // residuals of the members' groups in this chunk against the new centroid
  const int64_t wbase = (int64_t)b * a.win_max;
  const int G = resid_group(a.resid), gpc = min(kChunk, d - n0) / G;
  const int64_t cb = resid_code_bytes(a.resid, d), sb = resid_scale_bytes(a.resid, d);
  const T* rows = (const T*)a.ws_rows;
  for (int i = tid; i < nmem * gpc; i += blockDim.x) {
    const int w = mem[i / gpc], gi = i % gpc;
    const int64_t row = wbase + w;
    float r[32];
    for (int e = 0; e < G; ++e) r[e] = St<T>::load(rows, row * d + n0 + gi * G + e) - zsh[gi * G + e];
    resid_encode_group(a.resid, r, a.codes + row * cb, a.scales + row * sb, n0 + gi * G);
  }
}

// ---- QKV input rows: round(RMSNorm(x)) of [active; window; centroids], fragment-packed (bf16) ----
template <typename T>
__global__ __launch_bounds__(256) void prep_qkv_kernel(PrepArgs a) {
  __shared__ float red[4];
  __shared__ unsigned long long bal[4];
  const int r = blockIdx.x, b = blockIdx.y;
  const int d = a.d;
  const T* src;
  int out = r;   // staged row
  if (r < a.block) {
    src = (const T*)a.h_act + (int64_t)b * a.act_bstride + (int64_t)r * d;
  } else {
    const int w = r - a.block;
    if (a.map) {
      // query cache: window rows that need a query (all of them after block entry, else the
      // patched ones) are staged in row order after the active rows, then the centroids
      const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
      const bool all = a.q_ok[b] != a.q_tag;   // cached queries of another block position, or none
      const bool need = tid < a.n_win && (all || a.flags[(int64_t)b * a.win_max + tid] != 0);
      const unsigned long long m = __ballot(need);
      if (lane == 0) bal[wave] = m;
      __syncthreads();
      int total = 0, before = 0;   // staged window rows, and those before row w
      for (int k = 0; k < 4; ++k) total += __popcll(bal[k]);
      if (w < a.n_win) {
        const int ww = w >> 6;
        if (!((bal[ww] >> (w & 63)) & 1ull)) return;   // uniform: its query is kept from an earlier step
        for (int k = 0; k < ww; ++k) before += __popcll(bal[k]);
        before += __popcll(bal[ww] & ((1ull << (w & 63)) - 1ull));
        out = a.block + before;
        if (tid == 0) a.map[(int64_t)b * a.win_max + before] = w;
        src = (const T*)a.ws_rows + ((int64_t)b * a.win_max + w) * d;
      } else {
        const int c = w - a.n_win;
        out = a.block + total + c;
        if (c == 0 && tid == 0) a.count[b] = total;
        src = (const T*)a.win_z + ((int64_t)b * a.K + c) * d;
      }
    } else if (w < a.n_win) {
      src = (const T*)a.ws_rows + ((int64_t)b * a.win_max + w) * d;
    } else {
      src = (const T*)a.win_z + ((int64_t)b * a.K + (w - a.n_win)) * d;
    }
  }
  T* dst = (T*)a.a_qkv + (int64_t)b * a.a_bstride;
  if (a.a_tiles > 0)
    rmsnorm_row<T>(src, d, a.eps, red, [&](int n, const float* x) { Quad<T>::store(dst + apack(out, n, 0, 1, a.a_tiles), x); });
  else
    rmsnorm_row<T>(src, d, a.eps, red, [&](int n, const float* x) { Quad<T>::store(dst + (int64_t)out * d + n, x); });
}

// ---- NVFP4 test hooks ---------------------------------------------------------------------------
__global__ void nvfp4_pack_kernel(const float* x, int64_t groups, int32_t d, uint8_t* codes, uint8_t* scales) {
  const int64_t g = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (g >= groups) return;
  float r[16];
  uint32_t c[16];
  for (int e = 0; e < 16; ++e) r[e] = x[g * 16 + e];
  scales[g] = (uint8_t)nvfp4_group(r, c);
  for (int e = 0; e < 8; ++e) codes[g * 8 + e] = (uint8_t)(c[2 * e] | (c[2 * e + 1] << 4));
}

__global__ void nvfp4_unpack_kernel(const uint8_t* codes, const uint8_t* scales, int64_t groups, float* x) {
  const int64_t g = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (g >= groups) return;
  const float sv = e4m3_value(scales[g]);
  for (int e = 0; e < 8; ++e) {
    const uint8_t byte = codes[g * 8 + e];
    x[g * 16 + 2 * e] = sv * e2m1_value(byte & 15u);
    x[g * 16 + 2 * e + 1] = sv * e2m1_value(byte >> 4);
  }
}

// One thread per group of resid_group(fmt) values of a row.
__global__ void resid_pack_kernel(int fmt, const float* x, int64_t rows, int32_t d, uint8_t* codes, uint8_t* scales) {
  const int G = resid_group(fmt), ng = d / G;
  const int64_t g = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (g >= rows * ng) return;
  const int64_t row = g / ng;
  const int g0 = (int)(g % ng) * G;
  float r[32];
  for (int e = 0; e < G; ++e) r[e] = x[row * d + g0 + e];
  resid_encode_group(fmt, r, codes + row * resid_code_bytes(fmt, d), scales + row * resid_scale_bytes(fmt, d), g0);
}

__global__ void resid_unpack_kernel(int fmt, const uint8_t* codes, const uint8_t* scales, int64_t rows, int32_t d,
                                    float* x) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= rows * d) return;
  const int64_t row = i / d;
  const int n = (int)(i % d);
  x[i] = resid_value(fmt, codes + row * resid_code_bytes(fmt, d), scales + row * resid_scale_bytes(fmt, d), n);
}

}  // namespace

template <typename T>
hipError_t launch_cluster(const ClusterArgs& a, hipStream_t s) {
  if (a.mode == POLESTAR_CLUSTER_ENTRY) {
    const int nwin = a.geom.n_win, keff = a.K < nwin ? a.K : nwin;
    if (a.K > kKmMax || nwin > 256) return hipErrorInvalidValue;
    if (a.nchunk > kGather || keff * a.nchunk > kGather) return hipErrorInvalidValue;
    hipLaunchKernelGGL(km_unit_kernel<T>, dim3(nwin, a.batch), dim3(1024), 0, s, a);
    const dim3 g(a.nchunk, keff, a.batch);
    for (int it = 0; it < a.iters; ++it) {
      hipLaunchKernelGGL(km_assign_kernel, dim3(nwin, a.batch), dim3(1024), 0, s, a);
      hipLaunchKernelGGL(km_update_kernel, g, dim3(256), 0, s, a, it);
      hipLaunchKernelGGL(km_finish_kernel, g, dim3(256), 0, s, a, it);
    }
    hipLaunchKernelGGL(km_store_kernel<T>, dim3(a.K, a.batch), dim3(256), 0, s, a);
    if (a.resid) hipLaunchKernelGGL(km_resid_kernel<T>, dim3(nwin, a.batch), dim3(256), 0, s, a);
  } else {
    if (a.nchunk > 256) return hipErrorInvalidValue;
    hipLaunchKernelGGL(window_rows_kernel<T>, dim3(a.geom.n_win, a.batch), dim3(256), 0, s, a);
    const dim3 g(a.nchunk, a.K, a.batch);
    hipLaunchKernelGGL(centroid_sum_kernel<T>, g, dim3(256), 0, s, a);
    hipLaunchKernelGGL(centroid_finish_kernel<T>, g, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_prep_qkv(const PrepArgs& a, hipStream_t s) {
  const int rows = a.refresh ? a.block + a.n_win + a.K : a.block;
  hipLaunchKernelGGL(prep_qkv_kernel<T>, dim3(rows, a.batch), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_nvfp4_pack(const float* x, int64_t rows, int32_t d, uint8_t* codes, uint8_t* scales,
                             hipStream_t s) {
  const int64_t groups = rows * (d / 16);
  if (groups == 0) return hipSuccess;
  hipLaunchKernelGGL(nvfp4_pack_kernel, dim3((unsigned)PS_CEIL_DIV(groups, 256)), dim3(256), 0, s, x, groups, d,
                     codes, scales);
  return hipGetLastError();
}

hipError_t launch_nvfp4_unpack(const uint8_t* codes, const uint8_t* scales, int64_t rows, int32_t d, float* x,
                               hipStream_t s) {
  const int64_t groups = rows * (d / 16);
  if (groups == 0) return hipSuccess;
  hipLaunchKernelGGL(nvfp4_unpack_kernel, dim3((unsigned)PS_CEIL_DIV(groups, 256)), dim3(256), 0, s, codes, scales,
                     groups, x);
  return hipGetLastError();
}

hipError_t launch_resid_pack(int fmt, const float* x, int64_t rows, int32_t d, uint8_t* codes, uint8_t* scales,
                             hipStream_t s) {
  const int64_t groups = rows * (d / resid_group(fmt));
  if (groups == 0) return hipSuccess;
  hipLaunchKernelGGL(resid_pack_kernel, dim3((unsigned)PS_CEIL_DIV(groups, 256)), dim3(256), 0, s, fmt, x, rows, d,
                     codes, scales);
  return hipGetLastError();
}

hipError_t launch_resid_unpack(int fmt, const uint8_t* codes, const uint8_t* scales, int64_t rows, int32_t d, float* x,
                               hipStream_t s) {
  const int64_t n = rows * d;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(resid_unpack_kernel, dim3((unsigned)PS_CEIL_DIV(n, 256)), dim3(256), 0, s, fmt, codes, scales,
                     rows, d, x);
  return hipGetLastError();
}

template hipError_t launch_cluster<float>(const ClusterArgs&, hipStream_t);
template hipError_t launch_cluster<bf16_t>(const ClusterArgs&, hipStream_t);
template hipError_t launch_prep_qkv<float>(const PrepArgs&, hipStream_t);
template hipError_t launch_prep_qkv<bf16_t>(const PrepArgs&, hipStream_t);
