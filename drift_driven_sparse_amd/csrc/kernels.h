// Launch interfaces between the C ABI layer and the HIP kernels.
#pragma once
#include "common.h"

// Handle contents (host only).
struct WsLayout {
  size_t win_rows, flags, a_qkv, q, o, kl, akl, lg, part, hp, a_gu, act, a_kv, xhat, z64, wstat, attn_part, lm_a,
      lm_stats, lm_meta, lm_conf, q_all, qmap, km_lab, km_cnt, km_sum, total;
};

struct ProfState;   // per-kernel event records (api.hip)

struct polestar_handle {
  ProfState* prof;
  polestar_dims dm;
  polestar_params pr;
  int32_t win_max;   // win_prefix + win_suffix
  int32_t mq;        // QKV rows per sequence: B + win_max + K
  int32_t mt;        // token rows per sequence: B + win_max
  int32_t nq, nkv;   // Hq*dh, Hkv*dh
  int32_t ksplit;    // split-K factor of the N = d projections (float32 path)
  int32_t ks_qkv, ks_o, ks_gu, ks_down, ks_kv;   // split-K factors of the bf16 projections
  int32_t sh_qkv, sh_o, sh_gu, sh_down, sh_kv;   // their workgroup shapes (DlShape)
  int32_t rq, rt, rw;   // mq, mt, win_max rounded up to whole 16-row tiles (packed operands)
  int32_t ec;           // block entry: rows per slab at most (a multiple of 16, >= rq); the
                        // token-row buffers of the workspace hold this many rows per sequence
  int32_t attn_chunk, attn_nchunks;             // bf16 attention: keys per workgroup, workgroups per head
  int32_t attn_rgroups;                         // bf16 attention: workgroups along the query rows
  int32_t lm_tiles;  // LM-head vocabulary tiles: vocab / tile width of sh_lm (bf16) or 64 (f32), rounded up
  int32_t sh_lm;     // LM-head workgroup shape (bf16)
  WsLayout ws;
  polestar_check chk;
};

// ---- GEMM ---------------------------------------------------------------------
// Fragment-packed operand of the bf16 projections: per 32-column step s, plane p and 16-row
// tile t one 1 KiB MFMA 16x16x32 A fragment, so that a workgroup's operand for one step is
// contiguous; element (r, k) is element k%8 of lane (r%16) + 16*((k%32)/8).  `tiles` is the
// number of row tiles per step and plane.
PS_HD int64_t apack(int r, int k, int p, int planes, int tiles) {
  return (((((int64_t)(k >> 5) * planes + p) * tiles + (r >> 4)) * 64) + (r & 15) + 16 * ((k & 31) >> 3)) * 8 +
         (k & 7);
}

// A operand: rows of M-block b (one sequence).  Row-major: row r reads source row
//   r                                  when rowmap == nullptr or r < map_from
//   map_off + rowmap[b*map_bstride + r - map_from]   otherwise.
// Fragment-packed (tiles > 0, bf16 projections only): rows in order, no row map.
struct GemmA {
  const void* base;      // rows in the storage dtype (bf16 projections: bf16 planes)
  int32_t tiles;         // > 0: fragment-packed with this many row tiles per step and plane
  int64_t plane_stride;  // row-major bf16 planes: elements from the hi plane to the lo plane
  int64_t bstride;       // elements between sequences
  int32_t lda;           // elements between rows
  const int32_t* rowmap;
  int32_t map_bstride, map_from, map_off;
  const int32_t* rows_dev;   // rows of block b = min(rows_dev[b] + rows_add, rows_max), or rows_static
  int32_t rows_add, rows_static, rows_max;
  int32_t row0;              // first row of this launch (a multiple of 16): launches cover row slabs
  PS_DEV int rows(int b) const {
    if (!rows_dev) return rows_static;
    int r = rows_dev[b] + rows_add;
    r = r < rows_add ? rows_add : r;
    return r > rows_max ? rows_max : r;
  }
  PS_DEV int64_t src_row(int b, int r) const {
    if (rowmap != nullptr && r >= map_from) {
      int m = rowmap[b * map_bstride + r - map_from];
      m = (m < 0 || m >= map_bstride) ? 0 : m;
      return (int64_t)map_off + m;
    }
    return r;
  }
};

struct GemmArgs {
  GemmA A;
  const void* W;       // packed weight
  int32_t N, K;
  int32_t batch;
  int32_t ksplit;
  float* part;         // when set: raw sums to part[((s*batch + b)*part_rows + r)*N + n]
  int32_t part_rows;
};

enum EpiKind { EPI_PARTIAL = 0, EPI_QKV = 1, EPI_SWIGLU = 2, EPI_KV = 3, EPI_LMSTAT = 4 };

struct EpiParams {
  int kind;
  // QKV
  float* q; int32_t q_rows;     // q[(b*q_rows + r)*nq + n]
  void* kc; void* vc;           // caches (storage dtype)
  const int32_t* flags;         // patched flags [batch][win_max]
  int32_t nq, nkv, block, win_max, n_pos, dh;
  WinGeom geom;
  // query cache: rows [active; qcount staged window rows (window row qmap[b*win_max + j]); centroids];
  // window-row queries go to q_win[b][w], centroid c's to q row block + n_win + c
  float* q_win; const int32_t* qmap; const int32_t* qcount;
  float* chk; int32_t chk_rows, chk_ld;   // chk[(b*chk_rows + r)*chk_ld + n]
  // SwiGLU product: float32 rows [batch][act_rows][ffn], or for bf16 storage the hi/lo planes
  // fragment-packed with act_tiles row tiles ([batch] stride act_rows*ffn*2 elements)
  void* act; int32_t act_rows, ffn, act_tiles;
  // KV scatter of packet rows: dest pos = geom.pos(sel_idx[b*win_max + r])
  const int32_t* sel_idx;
  // LM statistics
  float* lm_stats; int32_t lm_rows, lm_tiles, vocab, mask_id;
};

// Cache element of position pos, K/V column col (= kv head * dh + d):
// K token-major [b][n][Hkv][dh]; V transposed [b][Hkv][dh][n].
PS_DEV int64_t kv_index(const EpiParams& e, int b, int pos, int col, int is_v) {
  if (!is_v) return ((int64_t)b * e.n_pos + pos) * e.nkv + col;
  return ((int64_t)b * e.nkv + col) * e.n_pos + pos;
}

// Destination of QKV row r (active block, window rows, centroids): its query row (as a pointer to
// column 0), the cache position of its K/V (-1: none, i.e. unpatched window rows and centroids)
// and its logical row [active; window row w at block + w; centroid c at block + n_win + c], the
// row of the check copy.  With the query cache only the staged window rows are projected.
struct QkvDest { float* q; int pos; int row; };
PS_DEV QkvDest qkv_dest(const EpiParams& e, int b, int r) {
  if (r < e.block) return {e.q + ((int64_t)b * e.q_rows + r) * e.nq, e.geom.blk_start + r, r};
  int w = r - e.block;
  if (e.qmap) {
    const int np = e.qcount[b];
    if (w >= np) {   // centroid rows follow the staged window rows
      const int lr = e.block + e.geom.n_win + (w - np);
      return {e.q + ((int64_t)b * e.q_rows + lr) * e.nq, -1, lr};
    }
    w = e.qmap[(int64_t)b * e.win_max + w];
    const int pos = e.flags[(int64_t)b * e.win_max + w] ? e.geom.pos(w) : -1;
    return {e.q_win + ((int64_t)b * e.win_max + w) * e.nq, pos, e.block + w};
  }
  const int pos = (w < e.geom.n_win && e.flags[(int64_t)b * e.win_max + w]) ? e.geom.pos(w) : -1;
  return {e.q + ((int64_t)b * e.q_rows + r) * e.nq, pos, r};
}

template <typename T>
PS_DEV void epi_qkv_elem(const EpiParams& e, int b, int r, int n, float v) {
  const QkvDest dst = qkv_dest(e, b, r);
  if (e.chk) e.chk[((int64_t)b * e.chk_rows + dst.row) * e.chk_ld + n] = v;
  if (n < e.nq) {
    dst.q[n] = v;
    return;
  }
  const int kv = n - e.nq;
  const int which = kv >= e.nkv;
  const int col = kv - which * e.nkv;
  if (dst.pos >= 0) St<T>::store((T*)(which ? e.vc : e.kc), kv_index(e, b, dst.pos, col, which), v);
}

// K/V of the next layer for packet row r (window row sel_idx[r]).
template <typename T>
PS_DEV void epi_kv_elem(const EpiParams& e, int b, int r, int n, float v) {
  if (e.chk) e.chk[((int64_t)b * e.chk_rows + r) * e.chk_ld + n] = v;
  const int which = n >= e.nkv;
  const int col = n - which * e.nkv;
  const int w = e.sel_idx[(int64_t)b * e.win_max + r];
  if (w < 0 || w >= e.geom.n_win) return;
  St<T>::store((T*)(which ? e.vc : e.kc), kv_index(e, b, e.geom.pos(w), col, which), v);
}

// float32 -> bf16 hi/lo pair: hi = rn(x), lo = rn(x - hi); hi + lo keeps ~16 significant bits.
PS_DEV void split_bf16(float x, uint16_t& hi, uint16_t& lo) {
  hi = f32_to_bf16(x);
  lo = f32_to_bf16(x - bf16_to_f32(hi));
}

// Sum of the split-K partials p[0], p[stride], ..., p[(ks-1)*stride] (four floats each), added
// in split order; the loads of up to eight splits are issued before their additions.
PS_DEV float4 sum_splits(const float* p, int64_t stride, int ks) {
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < ks; s0 += 8) {
    float4 t[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (s0 + j < ks) t[j] = *(const float4*)(p + (int64_t)(s0 + j) * stride);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (s0 + j < ks) {
        v.x += t[j].x; v.y += t[j].y; v.z += t[j].z; v.w += t[j].w;
      }
  }
  return v;
}

template <typename T>
hipError_t launch_gemm(const GemmArgs& g, const EpiParams& e, int max_rows, hipStream_t s);

// ---- bf16 weight-streaming projection (gemm_dl.hip) ------------------------------------
// A: bf16 planes (1 = bf16 rows, 2 = hi/lo of float32 rows), rows gathered per lane.
// ksplit > 1: raw sums to part[((s*batch + b)*part_rows + r)*N + n], finished by
// launch_dl_finish (QKV, gate/up, KV) or the row reduction (O, down).
constexpr int kMaxPos = 4096;  // key positions per sequence at most (KL rows are held in registers)
constexpr int kDlSlab = 192;       // rows per launch of the projection kernels (longer row lists take several)
constexpr int kDlSlabX512 = 128;   // rows per launch of the 512-column shape
struct DlArgs {
  GemmA A;
  int32_t planes;
  const void* W;         // packed in groups of wg 16-column subtiles (weight_group)
  int32_t N, K, batch, ksplit;
  int32_t wg;
  float* part;
  int32_t part_rows;
  EpiParams e;
};
// Workgroup shapes: row groups x column groups (waves), columns per wave.  One bf16 plane:
// NARROW, N192, N96; hi/lo planes: X512, WIDE, MID, W192, MID8, P96, P160.
enum DlShape { DL_NARROW = 0,   // 3 x 2 waves of 64 columns: 128-column tiles
               DL_WIDE = 1,     // 2 x 4 waves of 64 columns: 256-column tiles
               DL_MID = 2,      // 2 x 2 waves of 64 columns: 128-column tiles
               DL_N192 = 3,     // 2 x 4 waves of 48 columns: 192-column tiles
               DL_W192 = 4,     // 2 x 4 waves of 48 columns: 192-column tiles
               DL_N96 = 5,      // 4 x 2 waves of 48 columns: 96-column tiles
               DL_MID8 = 6,     // 2 x 4 waves of 32 columns: 128-column tiles
               DL_P96 = 7,      // 4 x 3 waves of 32 columns: 96-column tiles
               DL_P160 = 8,     // 2 x 5 waves of 32 columns: 160-column tiles
               DL_X512 = 9 };   // 1 x 8 waves of 64 columns: 512-column tiles, 128-row launches
int dl_tile_cols(int shape);
// 16-column subtiles per wave; the in-kernel SwiGLU epilogue needs an even count (gate/up pairs)
int dl_subtiles_per_wave(int shape);
template <typename T>
hipError_t launch_dl(const DlArgs& g, int shape, int max_rows, hipStream_t s);
template <typename T>
hipError_t launch_dl_finish(const DlArgs& g, int max_rows, hipStream_t s);
// Packed weights: fragment (16-column subtile n16, 32-row step k32) of the bf16 layout sits at
// ((n16/G * (K/32) + k32) * G + n16%G) KiB, so the G subtiles of one group are contiguous per
// step; the last group is padded with zeros.  float32 weights stay row-major.
template <typename T>
hipError_t launch_pack(int kind, const void* src, void* dst, int N, int K, int G, int ffn, hipStream_t s);
size_t packed_elems(int N, int K, int G);

// Row reductions after split-K projections, one row per workgroup: out = sum of partials in
// split order + residual, kept as float32 or rounded to the storage dtype, and for rows
// r >= norm_from also RMSNorm(out), the input of the next projection.
struct RowReduceArgs {
  const float* part; int32_t ksplit, part_rows, batch, d;
  const int32_t* count;   // rows of seq b = block + count[b]
  int32_t block, win_max;
  // residual row r: r < res_split -> res_a[b][r]; else res_b[b][sel_idx[b*win_max + r - res_split]]
  const void* res_a; int64_t res_a_bstride; int32_t res_split;
  int32_t res_a_f32;            // res_a holds float32 rows (else storage dtype)
  const void* res_b; int64_t res_b_bstride;
  const int32_t* sel_idx;
  // output row r: r < out_split -> out_a[b][r]; else out_b[b][r - out_split]
  void* out_a; int64_t out_a_bstride; int32_t out_split;
  void* out_b; int64_t out_b_bstride;
  int32_t out_f32;              // outputs are float32 rows (else storage dtype)
  // RMSNorm of row r >= norm_from as row r - norm_from of norm (null: none): bf16 hi/lo planes
  // of the float32 value when norm_planes, else rounded to the storage dtype; fragment-packed
  // with norm_tiles row tiles when norm_tiles > 0, else row-major
  void* norm; int64_t norm_bstride; int32_t norm_from;
  int32_t norm_planes, norm_tiles;
  float eps;
  float* chk; int32_t chk_rows;
};
template <typename T>
hipError_t launch_row_reduce(const RowReduceArgs& a, int max_rows, hipStream_t s);

// ---- window / clustering ----------------------------------------------------------
struct ClusterArgs {
  int mode;
  int32_t batch, d, K, win_max, block, n_pos, iters;
  WinGeom geom;
  void* win_h; uint8_t* codes; uint8_t* scales; void* win_z; int32_t* win_m;
  const void* entry_h;       // entry rows: [batch][win_max][d], or with entry_full the rows of
  int32_t entry_full;        // all positions [batch][n_pos][d], read at the window positions
  const int32_t* init_idx;
  double* objective;
  const void* u_rows; const int32_t* u_idx; const int32_t* u_count;
  void* ws_rows;            // patched window rows [batch][win_max][d] (storage dtype)
  int32_t* flags;           // [batch][win_max]
  double* xhat; double* z64;
  double* wnorm;            // [batch][win_max] float64 norms of the current window rows
  double* cpart;            // [batch][K][nchunk] chunk sums of squares of the member sums
  int32_t nchunk;           // ceil(d / 256)
  int32_t* km_lab;          // block entry: labels [batch][win_max], member counts [batch][K],
  int32_t* km_cnt;          //   member sums [batch][K][d] (float64); wnorm holds the best cosines
  double* km_sum;
  int resid;                // residual format of the window storage (POLESTAR_RESID_*; 0: raw rows)
  int32_t* q_ok;            // query cache validity [batch] (nullable): block entry clears it
};
template <typename T>
hipError_t launch_cluster(const ClusterArgs& a, hipStream_t s);

// Active rows, window rows and centroids -> contiguous QKV input rows round(RMSNorm(x)).
struct PrepArgs {
  int32_t batch, d, block, win_max, n_win, K, mq, refresh;
  int32_t a_tiles;        // > 0: a_qkv fragment-packed with this many row tiles (bf16)
  const void* h_act; int64_t act_bstride;   // block rows per sequence, act_bstride elements apart
  const void* ws_rows; const void* win_z;
  // query cache (map set): only the window rows that need a query (all unless q_ok[b] == q_tag,
  // the tag of this block position, else the patched ones) are staged, after the active rows and before the centroids; map[b][j] is the
  // window row of staged row block + j, count[b] their number
  const int32_t* flags; const int32_t* q_ok; int32_t q_tag; int32_t* map; int32_t* count;
  float* q_win;   // the layer's cached window-row queries (passed on to the QKV epilogue)
  void* a_qkv; int64_t a_bstride; float eps;
};
template <typename T>
hipError_t launch_prep_qkv(const PrepArgs& a, hipStream_t s);

// ---- attention / drift ------------------------------------------------------------
struct AttnArgs {
  int32_t batch, n_pos, hq, hkv, dh, mq, mt;
  int32_t n_tok;          // token query rows per sequence (block + n_win, or block)
  int32_t n_proxy;        // centroid query rows (K or 0)
  int32_t n_stage_proxy;  // proxy rows in the logit staging layout [proxies; active]
  int32_t block;
  int32_t key_lo, key_hi; // keys the query rows of this launch attend to: [key_lo, key_hi)
  int32_t pkey_lo, pkey_hi;   // KL: key range of the proxy rows' logits (active rows: all keys)
  const float* q;         // [batch][mq][hq*dh]
  const float* q_win;     // nullable: queries of token rows block.. (window rows), [batch][win_max][hq*dh]
  int32_t win_max;
  const void* kc; const void* vc;
  void* o;                // [batch][mt][hq*dh] float32, or bf16 hi/lo planes [batch][2][mt][hq*dh]
  int32_t o_planes;
  float* proxy_logits;    // [batch][K][hq][n]
  float* kl;              // [batch][K][hq]
  int32_t proxy_kl;       // 1: KL of the proxy rows against proxy_logits; 0: only store their logits
  float* act_logits;      // [batch][block][hq][n] or null
  float* lg_stage;        // staged logits of kept rows [batch][n_stage_proxy + block][hq][n]
  int32_t chunk_keys;     // bf16 path: keys per workgroup (multiple of 32)
  int32_t n_chunks;       // workgroups along the keys; > 1 -> partial states merged by launch_merge_kl
  int32_t row_groups;     // bf16 path: workgroups along the query rows, group_tiles 16-row tiles each
  int32_t group_tiles;
  float* part_o;          // [batch][n_chunks][hq][mt][dh] unnormalised outputs of token rows
  float* part_ml;         // [batch][n_chunks][hq][mt][2] running max and sum
  int32_t act_kl;         // compute active-row KL against act_logits before overwrite
  float* akl;             // [batch][block][hq]
  float* chk; int32_t chk_rows;
};
template <typename T>
hipError_t launch_attention(const AttnArgs& a, hipStream_t s);
// merge of the key chunks (bf16 path: merge = true) and the KL drift, one launch
hipError_t launch_merge_kl(const AttnArgs& a, bool merge, hipStream_t s);

struct TopkArgs {
  int32_t batch, K, k, hq, block, win_max, n_win;
  const float* kl; const int32_t* win_m;
  float* D; int32_t* topk; int32_t* sel_idx; int32_t* sel_count;
  const float* akl; float* delta;
  int32_t refresh;
  int32_t* q_ok;   // query cache validity [batch] (nullable): set to q_tag after a refresh
  int32_t q_tag;   // blk_start + 1: the block position the cached queries belong to
};
hipError_t launch_topk(const TopkArgs& a, hipStream_t s);

// ---- commit ---------------------------------------------------------------------
struct LmPrepArgs {
  int32_t batch, d, block, win_max, win_suffix, n_pre, lm_rows;
  const void* h_final; const void* u_rows; const int32_t* u_idx; const int32_t* u_count;
  // block entry (h_full set): rows of every position [batch][n_pos][d]; the active rows sit at
  // blk_start.., the n_suf suffix rows right after them
  const void* h_full; int32_t n_pos, blk_start, n_suf;
  void* a_lm; int32_t* meta; float eps;   // a_lm: round(RMSNorm(row)); meta: rows per sequence, suffix start
};
template <typename T>
hipError_t launch_lm_prep(const LmPrepArgs& a, hipStream_t s);

struct DecideArgs {
  int32_t batch, block, win_suffix, win_max, n_pre, lm_rows, lm_tiles, hist, mask_id;
  float tau_s, tau_suf, alpha;
  const float* lm_stats; const int32_t* meta; const int32_t* u_idx;
  float* lm_conf; int32_t* lm_yhat;   // [batch][lm_rows] confidence and argmax of each staged row
  const float* delta; const uint8_t* active_masked; const uint8_t* suffix_masked;
  float* hist_vals; int32_t* hist_cnt;
  uint8_t* commit_active; uint8_t* commit_suffix; float* conf_active; int32_t* yhat_active;
  float* spike; float* conf_suffix;
  int32_t entry;   // block entry: confidence alone decides (no drift, history untouched); suffix
                   // row i is suffix slot i
};
hipError_t launch_decide(const DecideArgs& a, hipStream_t s);

// ---- NVFP4 test hooks -------------------------------------------------------------
// ---- KV-cache staleness (measurement) ----------------------------------------------
struct StaleArgs {
  int32_t batch, n_pos, hkv, dh;
  const void* k; const void* v;          // caches being measured (cache layouts, storage dtype)
  const void* k_ref; const void* v_ref;  // recomputed rows, same layouts
  float* stale;                          // [batch][n_pos]
};
template <typename T>
hipError_t launch_kv_staleness(const StaleArgs& a, hipStream_t s);

// Most-attended-token policy (measurement): per query row, the key position with the largest
// head-mean attention probability over the cache k, and 1 - mean over KV heads of the cosine
// between that position's rows in k and k_ref.
struct AttendArgs {
  const float* q; int64_t q_bstride; int32_t q_ld, rows;   // q[b*q_bstride + r*q_ld + h*dh + e]
  const void* k; const void* k_ref;                        // K cache layout, storage dtype
  int32_t batch, n_pos, hq, hkv, dh;
  int32_t* top; float* score;                              // [batch][rows]
};
template <typename T>
hipError_t launch_attended_change(const AttendArgs& a, hipStream_t s);

hipError_t launch_resid_pack(int fmt, const float* x, int64_t rows, int32_t d, uint8_t* codes, uint8_t* scales,
                             hipStream_t s);
hipError_t launch_resid_unpack(int fmt, const uint8_t* codes, const uint8_t* scales, int64_t rows, int32_t d, float* x,
                               hipStream_t s);
hipError_t launch_nvfp4_pack(const float* x, int64_t rows, int32_t d, uint8_t* codes, uint8_t* scales,
                             hipStream_t s);
hipError_t launch_nvfp4_unpack(const uint8_t* codes, const uint8_t* scales, int64_t rows, int32_t d, float* x,
                               hipStream_t s);
