// C ABI of the Polestar refresh library: host-side validation, workspace layout
// and the launch sequence of each call.  Every argument is checked before the
// first launch, so a call that returns an error has enqueued nothing.
#include <algorithm>
#include <mutex>
#include <new>
#include <string.h>
#include <vector>

#include "kernels.h"

struct ProfState {
  struct Rec { int id; hipEvent_t a, b; };
  bool on = false;
  std::vector<Rec> recs;
  std::vector<hipEvent_t> pool;
  size_t used = 0;
  hipEvent_t take() {
    if (used == pool.size()) {
      hipEvent_t e = nullptr;
      if (hipEventCreate(&e) != hipSuccess) return nullptr;
      pool.push_back(e);
    }
    return pool[used++];
  }
  void clear() { recs.clear(); used = 0; }
  ~ProfState() {
    for (hipEvent_t e : pool) (void)hipEventDestroy(e);
  }
};

namespace {

// Brackets one kernel launch with profiling events when profiling is on.
struct ProfScope {
  ProfState* p;
  hipStream_t s;
  ProfState::Rec r;
  ProfScope(polestar_handle* h, hipStream_t s_, int id) : p(h->prof && h->prof->on ? h->prof : nullptr), s(s_) {
    if (!p) return;
    r.id = id;
    r.a = p->take();
    r.b = p->take();
    if (r.a && r.b) (void)hipEventRecord(r.a, s);
  }
  ~ProfScope() {
    if (!p || !r.a || !r.b) return;
    (void)hipEventRecord(r.b, s);
    p->recs.push_back(r);
  }
};
#define PROF(id) ProfScope _prof_##__LINE__(h, s, id)

constexpr int kMaxRows = 192;   // rows of one projection launch (longer row lists take several)

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

size_t elt(const polestar_handle* h) { return h->dm.dtype == POLESTAR_BF16 ? 2 : 4; }

void layout(polestar_handle* h) {
  const polestar_dims& d = h->dm;
  const size_t T = elt(h), Bt = d.batch;
  WsLayout& w = h->ws;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += ps_align256(bytes); return o; };
  w.win_rows = take(Bt * h->win_max * d.d * T);
  w.flags = take(Bt * h->win_max * 4);
  w.a_qkv = take(Bt * h->ec * d.d * T);
  w.q = take(Bt * h->mq * (size_t)h->nq * 4);
  w.o = take(Bt * h->ec * (size_t)h->nq * 4);    // float32 rows, or two bf16 planes
  w.kl = take(Bt * d.n_clusters * d.n_heads * 4);
  w.akl = take(Bt * d.block * d.n_heads * 4);
  w.lg = take(Bt * (size_t)(d.n_clusters + d.block) * d.n_heads * d.n_pos * 4);
  size_t part = (size_t)h->ksplit * Bt * h->ec * d.d;
  if (d.dtype == POLESTAR_BF16) {
    const size_t nqkv = (size_t)h->nq + 2 * (size_t)h->nkv;
    part = std::max(part, (size_t)h->ks_qkv * Bt * h->ec * nqkv);
    part = std::max(part, (size_t)h->ks_o * Bt * h->ec * d.d);
    part = std::max(part, (size_t)h->ks_down * Bt * h->ec * d.d);
    part = std::max(part, (size_t)h->ks_gu * Bt * h->ec * 2 * (size_t)d.ffn);
    part = std::max(part, (size_t)h->ks_kv * Bt * h->win_max * 2 * (size_t)h->nkv);
  }
  w.part = take(part * 4);
  w.hp = take(Bt * h->ec * d.d * 4);          // h' (float32)
  w.a_gu = take(Bt * h->ec * d.d * 4);        // RMSNorm(h'): float32 rows, or two bf16 planes
  w.attn_part = take(d.dtype == POLESTAR_BF16 && h->attn_nchunks > 1
                         ? Bt * h->attn_nchunks * d.n_heads * (size_t)h->ec * (d.head_dim + 2) * 4
                         : 0);
  w.act = take(Bt * h->ec * (size_t)d.ffn * 4);   // float32 rows, or two bf16 planes
  w.a_kv = take(Bt * h->rw * d.d * T);        // round(RMSNorm(U)): next-layer K/V input
  w.xhat = take(Bt * h->win_max * d.d * 8);
  w.z64 = take(Bt * (d.n_clusters + 1) * (size_t)d.d * 8);
  w.wstat = take(Bt * (h->win_max + (size_t)d.n_clusters * PS_CEIL_DIV(d.d, 256)) * 8);
  const size_t lm_rows = d.block + d.win_suffix;
  if (d.vocab > 0) {
    w.lm_a = take(Bt * lm_rows * d.d * T);
    w.lm_stats = take(Bt * lm_rows * (size_t)h->lm_tiles * 4 * 4);
    w.lm_meta = take(Bt * 2 * 4);
    w.lm_conf = take(Bt * lm_rows * 8);
  } else {
    w.lm_a = w.lm_stats = w.lm_meta = w.lm_conf = 0;
  }
  w.q_all = take(Bt * d.n_pos * (size_t)h->nq * 4);   // block entry: queries of every position
  w.qmap = take(Bt * (h->win_max + 1) * 4);           // query cache: staged window rows, count
  w.km_lab = take(Bt * h->win_max * 4);                // block entry: k-means labels, counts, sums
  w.km_cnt = take(Bt * d.n_clusters * 4);
  w.km_sum = take(Bt * d.n_clusters * (size_t)d.d * 8);
  w.total = off;
}

template <typename P>
P* at(void* ws, size_t off) { return (P*)((char*)ws + off); }

int check_ws(const polestar_handle* h, const void* ws, size_t ws_bytes) {
  if (!ws) return POLESTAR_E_NULL;
  if (((uintptr_t)ws & 255u) != 0) return POLESTAR_E_ALIGN;
  if (ws_bytes < h->ws.total) return POLESTAR_E_WORKSPACE;
  return POLESTAR_OK;
}

int check_blk(const polestar_handle* h, int32_t blk_start) {
  if (blk_start < 0 || blk_start + h->dm.block > h->dm.n_pos) return POLESTAR_E_ARG;
  return POLESTAR_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? POLESTAR_OK : POLESTAR_E_HIP; }

// Subtiles per packed weight group: the column width of the projection shape that streams the
// weight (bf16); the LM head and float32 weights keep one subtile per group.
int weight_group(const polestar_handle* h, int which) {
  if (h->dm.dtype != POLESTAR_BF16) return 1;
  switch (which) {
    case POLESTAR_W_QKV: return dl_tile_cols(h->sh_qkv) / 16;
    case POLESTAR_W_KV: return dl_tile_cols(h->sh_kv) / 16;
    case POLESTAR_W_O: return dl_tile_cols(h->sh_o) / 16;
    case POLESTAR_W_DOWN: return dl_tile_cols(h->sh_down) / 16;
    case POLESTAR_W_GU: return dl_tile_cols(h->sh_gu) / 16;
    case POLESTAR_W_LM: return dl_tile_cols(h->sh_lm) / 16;
    default: return 1;
  }
}

// Shape and split-K factor of one bf16 projection (n_cols x k weight, batch sequences): the
// candidate that keeps the largest share of the 256 compute units streaming weights, counting
// the columns a partial last tile wastes and the rounds of workgroups past the first; ties go
// to the smaller split (less partial-sum traffic), then to the earlier shape (the lists put
// the widest tiles first: with several sequences the projections are bound by the per-step
// work of a workgroup, which wider tiles spread over more columns, so from 8 sequences on a
// tie keeps the earlier shape at split 2 or less).  With pairs set
// (gate/up), a shape whose waves hold an odd number of subtiles is only taken with split-K,
// whose finish kernel forms the SwiGLU product.
void plan_projection(int n_cols, int k, int batch, const int* shapes, int n_shapes, int cap, bool pairs,
                     int32_t* shape, int32_t* ks) {
  double best = -1.0;
  *shape = shapes[0];
  *ks = 1;
  for (int i = 0; i < n_shapes; ++i) {
    const int tc = dl_tile_cols(shapes[i]);
    const int tiles = PS_CEIL_DIV(n_cols, tc) * batch;
    const int v0 = pairs && dl_subtiles_per_wave(shapes[i]) % 2 ? 2 : 1;
    for (int v = v0; v <= cap && v <= k / 32; ++v) {
      const int wgs = tiles * v;
      const int rounds = PS_CEIL_DIV(wgs, 256);
      const double use = (double)n_cols * batch / ((double)tiles * tc) * wgs / (256.0 * rounds);
      // a tie takes the smaller split; from 8 sequences on only over a split above 2, so that
      // the wider (earlier) shape keeps a tie at split 2 or less
      const bool smaller = batch >= 8 ? v < *ks && *ks > 2 : v < *ks;
      if (use > best + 1e-9 || (use > best - 1e-9 && smaller)) {
        best = use;
        *shape = shapes[i];
        *ks = v;
      }
    }
  }
}

WinGeom geom_of(const polestar_handle* h, int32_t blk_start) {
  return make_geom(blk_start, h->dm.n_pos, h->dm.block, h->dm.win_prefix, h->dm.win_suffix);
}

template <typename T>
int do_cluster(polestar_handle* h, int mode, const polestar_layer* L, int32_t blk_start,
               const polestar_packet* u_in, const int32_t* init_idx, const void* entry_h, double* objective,
               void* ws, hipStream_t s, bool entry_full = false) {
  const polestar_dims& d = h->dm;
  ClusterArgs a;
  memset(&a, 0, sizeof(a));
  a.mode = mode;
  a.batch = d.batch;
  a.d = d.d;
  a.K = d.n_clusters;
  a.win_max = h->win_max;
  a.block = d.block;
  a.n_pos = d.n_pos;
  a.iters = h->pr.kmeans_iters;
  a.geom = geom_of(h, blk_start);
  a.win_h = L->win_h;
  a.codes = L->win_codes;
  a.scales = L->win_scales;
  a.win_z = L->win_z;
  a.win_m = L->win_m;
  a.entry_h = entry_h;
  a.entry_full = entry_full;
  a.init_idx = init_idx;
  a.objective = objective;
  if (u_in) {
    a.u_rows = u_in->rows;
    a.u_idx = u_in->idx;
    a.u_count = u_in->count;
  }
  a.ws_rows = at<char>(ws, h->ws.win_rows);
  a.flags = at<int32_t>(ws, h->ws.flags);
  a.xhat = at<double>(ws, h->ws.xhat);
  a.z64 = at<double>(ws, h->ws.z64);
  a.wnorm = at<double>(ws, h->ws.wstat);
  a.nchunk = PS_CEIL_DIV(d.d, 256);
  a.cpart = a.wnorm + (size_t)d.batch * h->win_max;
  a.km_lab = at<int32_t>(ws, h->ws.km_lab);
  a.km_cnt = at<int32_t>(ws, h->ws.km_cnt);
  a.km_sum = at<double>(ws, h->ws.km_sum);
  a.resid = d.resid_fmt;
  a.q_ok = L->q_win ? L->q_ok : nullptr;
  if (a.geom.n_win == 0) return POLESTAR_OK;
  PROF(POLESTAR_K_CLUSTER);
  return hip_status(launch_cluster<T>(a, s));
}

// round(RMSNorm(rows)) of the rows p stages, then their Q/K/V: queries to q (float32, q_rows rows
// per sequence), K/V of rows below `block` to the cache at g.blk_start + r and of window rows
// with a patch flag at their window positions.
template <typename T>
int run_qkv(polestar_handle* h, const polestar_layer* L, const PrepArgs& p, int rows, int block, const WinGeom& g,
            float* q, int q_rows, int part_rows, bool checks, void* ws, hipStream_t s) {
  const polestar_dims& d = h->dm;
  hipError_t e;
  {
    PROF(POLESTAR_K_PREP);
    e = launch_prep_qkv<T>(p, s);
  }
  if (e != hipSuccess) return POLESTAR_E_HIP;
  GemmArgs ga;
  memset(&ga, 0, sizeof(ga));
  ga.A.base = p.a_qkv;
  ga.A.bstride = p.a_bstride;
  ga.A.tiles = p.a_tiles;
  ga.A.lda = d.d;
  ga.A.rows_static = rows;
  if (p.map) {   // block + staged window rows + K of the rows at most
    ga.A.rows_dev = p.count;
    ga.A.rows_add = block + p.K;
    ga.A.rows_max = rows;
  }
  ga.W = L->w_qkv;
  ga.N = h->nq + 2 * h->nkv;
  ga.K = d.d;
  ga.batch = d.batch;
  ga.ksplit = 1;
  EpiParams ep;
  memset(&ep, 0, sizeof(ep));
  ep.kind = EPI_QKV;
  ep.q = q;
  ep.q_rows = q_rows;
  ep.kc = L->k_cache;
  ep.vc = L->v_cache;
  ep.flags = at<int32_t>(ws, h->ws.flags);
  ep.nq = h->nq;
  ep.nkv = h->nkv;
  ep.dh = d.head_dim;
  ep.block = block;
  ep.win_max = h->win_max;
  ep.n_pos = d.n_pos;
  ep.geom = g;
  if (p.map) {   // query cache: rows [active; staged window rows; centroids]
    ep.q_win = p.q_win;
    ep.qmap = p.map;
    ep.qcount = p.count;
  }
  ep.chk = checks ? h->chk.qkv : nullptr;
  ep.chk_rows = h->mq;
  ep.chk_ld = ga.N;
  if constexpr (std::is_same<T, bf16_t>::value) {
    DlArgs dl;
    memset(&dl, 0, sizeof(dl));
    dl.A = ga.A;
    dl.planes = 1;
    dl.wg = weight_group(h, POLESTAR_W_QKV);
    dl.W = ga.W;
    dl.N = ga.N;
    dl.K = ga.K;
    dl.batch = d.batch;
    dl.ksplit = h->ks_qkv;
    dl.part = at<float>(ws, h->ws.part);
    dl.part_rows = part_rows;
    dl.e = ep;
    PROF(POLESTAR_K_QKV);
    e = launch_dl<T>(dl, h->sh_qkv, rows, s);
    if (e == hipSuccess) e = launch_dl_finish<T>(dl, rows, s);
  } else {
    PROF(POLESTAR_K_QKV);
    e = launch_gemm<T>(ga, ep, rows, s);
  }
  return hip_status(e);
}

// Attention arguments shared by every call: the layer's cache and the workspace buffers.  The
// caller sets the query rows (q, mq, n_tok, n_proxy, block) and the logit outputs.
template <typename T>
AttnArgs attn_base(polestar_handle* h, const polestar_layer* L, void* ws, int cap) {
  const polestar_dims& d = h->dm;
  AttnArgs a;
  memset(&a, 0, sizeof(a));
  a.batch = d.batch;
  a.n_pos = d.n_pos;
  a.hq = d.n_heads;
  a.hkv = d.n_kv_heads;
  a.dh = d.head_dim;
  a.mq = h->mq;
  a.mt = cap;   // token-row capacity of the output and chunk-state buffers
  a.block = d.block;
  a.kc = L->k_cache;
  a.vc = L->v_cache;
  a.key_lo = 0;
  a.key_hi = d.n_pos;
  a.pkey_lo = 0;
  a.pkey_hi = d.n_pos;
  a.o = at<char>(ws, h->ws.o);
  a.o_planes = std::is_same<T, bf16_t>::value;
  a.kl = at<float>(ws, h->ws.kl);
  a.akl = at<float>(ws, h->ws.akl);
  a.lg_stage = at<float>(ws, h->ws.lg);
  a.chunk_keys = h->attn_chunk;
  a.n_chunks = h->attn_nchunks;
  a.part_o = at<float>(ws, h->ws.attn_part);
  a.part_ml = a.part_o + (size_t)d.batch * h->attn_nchunks * d.n_heads * cap * d.head_dim;
  a.chk_rows = cap;
  return a;
}

// Attention of the query rows over all n_pos keys, then the merge of the key chunks and the KL
// drift of the kept logit rows.
void set_row_groups(const polestar_handle* h, AttnArgs& a) {
  const int tiles = PS_CEIL_DIV(a.n_tok + a.n_proxy, 16);
  a.row_groups = tiles >= 2 * h->attn_rgroups ? h->attn_rgroups : 1;
  // at most 12 row tiles (waves) per workgroup
  a.row_groups = std::max(a.row_groups, PS_CEIL_DIV(tiles, 12));
  a.group_tiles = PS_CEIL_DIV(tiles, a.row_groups);
}

template <typename T>
int run_attention(polestar_handle* h, AttnArgs& a, hipStream_t s) {
  a.n_stage_proxy = a.n_proxy;
  set_row_groups(h, a);
  hipError_t e;
  {
    PROF(POLESTAR_K_ATTN);
    e = launch_attention<T>(a, s);
  }
  if (e != hipSuccess) return POLESTAR_E_HIP;
  PROF(POLESTAR_K_KL);   // chunk merge and KL drift
  return hip_status(launch_merge_kl(a, std::is_same<T, bf16_t>::value, s));
}

// Proxy attention over the active block's keys only (POLESTAR_PROXY_ACTIVE): `a` describes the
// rows as for run_attention (n_tok token rows, then n_proxy centroid rows whose queries start at
// q_proxy); the token rows attend over every key, the centroid rows over [blk_start,
// blk_start + block) in a launch of their own; one merge/KL launch follows.
template <typename T>
int run_attention_active_keys(polestar_handle* h, AttnArgs& a, const float* q_proxy, int32_t blk_start,
                              hipStream_t s) {
  const int K = a.n_proxy;
  hipError_t e = hipSuccess;
  AttnArgs tok = a;
  tok.n_proxy = 0;
  tok.n_stage_proxy = K;
  if (tok.n_tok > 0) {
    set_row_groups(h, tok);
    PROF(POLESTAR_K_ATTN);
    e = launch_attention<T>(tok, s);
  }
  if (e != hipSuccess) return POLESTAR_E_HIP;
  AttnArgs px = a;
  px.n_tok = 0;
  px.n_stage_proxy = K;
  px.q = q_proxy;
  px.q_win = nullptr;
  px.key_lo = blk_start;
  px.key_hi = blk_start + h->dm.block;
  px.chunk_keys = 32 * PS_CEIL_DIV(px.key_hi - (px.key_lo & ~7), 32);
  px.n_chunks = 1;
  set_row_groups(h, px);
  {
    PROF(POLESTAR_K_ATTN);
    e = launch_attention<T>(px, s);
  }
  if (e != hipSuccess) return POLESTAR_E_HIP;
  tok.n_proxy = K;
  tok.pkey_lo = px.key_lo;
  tok.pkey_hi = px.key_hi;
  PROF(POLESTAR_K_KL);
  return hip_status(launch_merge_kl(tok, std::is_same<T, bf16_t>::value, s));
}

template <typename T>
int do_drift(polestar_handle* h, int mode, const polestar_layer* L, int32_t blk_start, const void* h_active,
             const polestar_packet* u_in, float* D, int32_t* topk, polestar_packet* sel, float* act_logits,
             float* delta, void* ws, hipStream_t s) {
  const polestar_dims& d = h->dm;
  const WinGeom g = geom_of(h, blk_start);
  const int refresh = mode == POLESTAR_DRIFT_REFRESH && g.n_win > 0;
  (void)u_in;
  // 1. QKV rows [active; window; centroids]; K/V of the active block and of the packet rows go
  //    to the cache
  PrepArgs p;
  memset(&p, 0, sizeof(p));
  p.batch = d.batch;
  p.d = d.d;
  p.block = d.block;
  p.win_max = h->win_max;
  p.n_win = g.n_win;
  p.K = d.n_clusters;
  p.mq = h->mq;
  p.refresh = refresh;
  p.h_act = h_active;
  p.act_bstride = (int64_t)d.block * d.d;
  p.ws_rows = at<char>(ws, h->ws.win_rows);
  p.win_z = L->win_z;
  p.a_qkv = at<char>(ws, h->ws.a_qkv);
  p.a_bstride = (int64_t)h->rq * d.d;
  p.a_tiles = std::is_same<T, bf16_t>::value ? h->rq / 16 : 0;
  p.eps = h->pr.rms_eps;
  // raw window rows change only where a packet patches them (residual formats are rebuilt
  // against a new centroid every step), so only then are the other rows' queries kept
  const bool qcache = refresh && L->q_win != nullptr && std::is_same<T, bf16_t>::value &&
                      d.resid_fmt == POLESTAR_RESID_RAW;
  if (qcache) {
    p.flags = at<int32_t>(ws, h->ws.flags);
    p.q_ok = L->q_ok;
    p.q_tag = blk_start + 1;
    p.map = at<int32_t>(ws, h->ws.qmap);
    p.count = p.map + (size_t)d.batch * h->win_max;
    p.q_win = L->q_win;
  }
  const int rows = refresh ? d.block + g.n_win + d.n_clusters : d.block;
  float* q = at<float>(ws, h->ws.q);
  int rc = run_qkv<T>(h, L, p, rows, d.block, g, q, h->mq, h->mq, true, ws, s);
  if (rc) return rc;
  // 2. attention, proxy attention and drift
  AttnArgs at_ = attn_base<T>(h, L, ws, h->mt);
  at_.n_tok = refresh ? d.block + g.n_win : d.block;
  at_.n_proxy = refresh ? d.n_clusters : 0;
  at_.q = q;
  if (qcache) {
    at_.q_win = L->q_win;
    at_.win_max = h->win_max;
  }
  at_.proxy_logits = L->proxy_logits;
  at_.proxy_kl = 1;
  at_.act_logits = act_logits;
  at_.act_kl = delta != nullptr;
  at_.chk = h->chk.attn_out;
  if (at_.n_proxy > 0 && h->pr.proxy_support == POLESTAR_PROXY_ACTIVE)
    rc = run_attention_active_keys<T>(h, at_, q + (size_t)(d.block + g.n_win) * h->nq, blk_start, s);
  else
    rc = run_attention<T>(h, at_, s);
  if (rc) return rc;
  // 3. top-k clusters and the selected rows
  TopkArgs tk;
  memset(&tk, 0, sizeof(tk));
  tk.batch = d.batch;
  tk.K = d.n_clusters;
  tk.k = d.top_k;
  tk.hq = d.n_heads;
  tk.block = d.block;
  tk.win_max = h->win_max;
  tk.n_win = g.n_win;
  tk.kl = at_.kl;
  tk.win_m = L->win_m;
  tk.D = D;
  tk.topk = topk;
  tk.sel_idx = sel->idx;
  tk.sel_count = sel->count;
  tk.akl = at_.akl;
  tk.delta = (act_logits && delta) ? delta : nullptr;
  tk.refresh = refresh;
  tk.q_ok = qcache ? L->q_ok : nullptr;
  tk.q_tag = blk_start + 1;
  PROF(POLESTAR_K_TOPK);
  return hip_status(launch_topk(tk, s));
}

// Token rows of the second half of a layer (O projection, residual, RMSNorm, SwiGLU FFN): n_act
// contiguous rows, read from h_act and written to h_out (the active block, or a slab of
// block-entry rows, whose attention output sits in rows [0, n_act) of the workspace), and with
// sel the selected window rows (attention output rows block + w, residual rows from the
// workspace window rows, outputs to u_rows).
struct TokRows {
  int32_t n_act;
  const void* h_act; int64_t act_bstride;   // elements between sequences
  void* h_out; int64_t out_bstride;
  const polestar_packet* sel;               // null: no window rows
  void* u_rows;
  bool checks;                              // fill the check buffers (per-step calls)
  int32_t cap, rcap;                        // rows per sequence of the workspace's token-row
                                            // buffers as laid out by the call (rcap: in 16-row tiles)
};

// Row count of a projection over [n_act rows; selected window rows].
void set_rows(GemmA& A, const TokRows& t, int max_rows) {
  A.rows_dev = t.sel ? t.sel->count : nullptr;
  A.rows_add = t.n_act;
  A.rows_static = t.n_act;
  A.rows_max = max_rows;
}

// bf16 storage: projections by the weight-streaming kernel; the float32 values inside the call
// (attention output, RMSNorm(h'), SwiGLU product) travel as bf16 hi/lo planes.
int do_refresh_dl(polestar_handle* h, const polestar_layer* L, int32_t blk_start, const TokRows& t,
                  const void* w_kv_next, void* k_next, void* v_next, void* ws, hipStream_t s) {
  typedef bf16_t T;
  const polestar_dims& d = h->dm;
  const WinGeom g = geom_of(h, blk_start);
  const polestar_packet* sel = t.sel;
  const int max_rows = t.n_act + (sel ? g.n_win : 0);
  const bool kv_next = w_kv_next && sel && g.n_win > 0;
  float* part = at<float>(ws, h->ws.part);
  hipError_t e;
  // 1. h' = h + o W_O^T over rows [active; S]
  DlArgs dl;
  memset(&dl, 0, sizeof(dl));
  dl.A.base = at<char>(ws, h->ws.o);
  dl.A.plane_stride = (int64_t)t.cap * h->nq;
  dl.A.bstride = 2 * dl.A.plane_stride;
  dl.A.lda = h->nq;
  dl.A.rowmap = sel ? sel->idx : nullptr;
  dl.A.map_bstride = h->win_max;
  dl.A.map_from = t.n_act;
  dl.A.map_off = d.block;
  set_rows(dl.A, t, max_rows);
  dl.planes = 2;
  dl.wg = weight_group(h, POLESTAR_W_O);
  dl.W = L->w_o;
  dl.N = d.d;
  dl.K = h->nq;
  dl.batch = d.batch;
  dl.ksplit = h->ks_o;
  dl.part = part;
  dl.part_rows = t.cap;
  dl.e.kind = EPI_PARTIAL;
  {
    PROF(POLESTAR_K_OPROJ);
    e = launch_dl<T>(dl, h->sh_o, max_rows, s);
  }
  if (e != hipSuccess) return POLESTAR_E_HIP;
  RowReduceArgs rr;
  memset(&rr, 0, sizeof(rr));
  rr.part = part;
  rr.ksplit = h->ks_o;
  rr.part_rows = t.cap;
  rr.batch = d.batch;
  rr.d = d.d;
  rr.count = sel ? sel->count : nullptr;
  rr.block = t.n_act;
  rr.win_max = h->win_max;
  rr.res_a = t.h_act;
  rr.res_a_bstride = t.act_bstride;
  rr.res_split = t.n_act;
  rr.res_b = at<char>(ws, h->ws.win_rows);
  rr.res_b_bstride = (int64_t)h->win_max * d.d;
  rr.sel_idx = sel ? sel->idx : nullptr;
  rr.out_a = at<char>(ws, h->ws.hp);
  rr.out_a_bstride = (int64_t)t.cap * d.d;
  rr.out_split = t.cap;
  rr.out_f32 = 1;
  rr.norm = at<char>(ws, h->ws.a_gu);
  rr.norm_planes = 1;
  rr.norm_tiles = t.rcap / 16;
  rr.norm_bstride = 2 * (int64_t)t.rcap * d.d;
  rr.norm_from = 0;
  rr.eps = h->pr.rms_eps;
  rr.chk = t.checks ? h->chk.hp : nullptr;
  rr.chk_rows = t.cap;
  {
    PROF(POLESTAR_K_OREDUCE);
    e = launch_row_reduce<T>(rr, max_rows, s);
  }
  if (e != hipSuccess) return POLESTAR_E_HIP;
  // 2. act = silu(g) * u with g, u the projections of RMSNorm(h')
  memset(&dl, 0, sizeof(dl));
  dl.A.base = rr.norm;
  dl.A.tiles = rr.norm_tiles;
  dl.A.bstride = rr.norm_bstride;
  dl.A.lda = d.d;
  set_rows(dl.A, t, max_rows);
  dl.planes = 2;
  dl.wg = weight_group(h, POLESTAR_W_GU);
  dl.W = L->w_gu;
  dl.N = 2 * d.ffn;
  dl.K = d.d;
  dl.batch = d.batch;
  dl.ksplit = h->ks_gu;
  dl.part = part;
  dl.part_rows = t.cap;
  dl.e.kind = EPI_SWIGLU;
  dl.e.act = at<char>(ws, h->ws.act);
  dl.e.act_rows = t.rcap;
  dl.e.act_tiles = t.rcap / 16;
  dl.e.ffn = d.ffn;
  {
    PROF(POLESTAR_K_GU);
    e = launch_dl<T>(dl, h->sh_gu, max_rows, s);
    if (e == hipSuccess) e = launch_dl_finish<T>(dl, max_rows, s);
  }
  if (e != hipSuccess) return POLESTAR_E_HIP;
  // 3. out = h' + act W_down^T -> next active rows and the update packet
  memset(&dl, 0, sizeof(dl));
  dl.A.base = at<char>(ws, h->ws.act);
  dl.A.tiles = t.rcap / 16;
  dl.A.bstride = 2 * (int64_t)t.rcap * d.ffn;
  dl.A.lda = d.ffn;
  set_rows(dl.A, t, max_rows);
  dl.planes = 2;
  dl.wg = weight_group(h, POLESTAR_W_DOWN);
  dl.W = L->w_down;
  dl.N = d.d;
  dl.K = d.ffn;
  dl.batch = d.batch;
  dl.ksplit = h->ks_down;
  dl.part = part;
  dl.part_rows = t.cap;
  dl.e.kind = EPI_PARTIAL;
  {
    PROF(POLESTAR_K_DOWN);
    e = launch_dl<T>(dl, h->sh_down, max_rows, s);
  }
  if (e != hipSuccess) return POLESTAR_E_HIP;
  // the residual stream continues from the float32 h'
  RowReduceArgs r2 = rr;
  r2.ksplit = h->ks_down;
  r2.res_a = rr.out_a;
  r2.res_a_f32 = 1;
  r2.res_a_bstride = (int64_t)t.cap * d.d;
  r2.res_split = t.cap;
  r2.res_b = nullptr;
  r2.out_a = t.h_out;
  r2.out_a_bstride = t.out_bstride;
  r2.out_split = t.n_act;
  r2.out_b = t.u_rows;
  r2.out_b_bstride = (int64_t)h->win_max * d.d;
  r2.out_f32 = 0;
  r2.norm = kv_next ? at<char>(ws, h->ws.a_kv) : nullptr;   // packet rows only, rounded
  r2.norm_planes = 0;
  r2.norm_tiles = h->rw / 16;
  r2.norm_bstride = (int64_t)h->rw * d.d;
  r2.norm_from = t.n_act;
  r2.chk = t.checks ? h->chk.out : nullptr;
  {
    PROF(POLESTAR_K_DREDUCE);
    e = launch_row_reduce<T>(r2, max_rows, s);
  }
  if (e != hipSuccess) return POLESTAR_E_HIP;
  // 4. K/V of layer l+1 for the packet rows, from round(RMSNorm(U))
  if (kv_next) {
    memset(&dl, 0, sizeof(dl));
    dl.A.base = r2.norm;
    dl.A.tiles = r2.norm_tiles;
    dl.A.bstride = r2.norm_bstride;
    dl.A.lda = d.d;
    dl.A.rows_dev = sel->count;
    dl.A.rows_max = g.n_win;
    dl.planes = 1;
    dl.wg = weight_group(h, POLESTAR_W_KV);
    dl.W = w_kv_next;
    dl.N = 2 * h->nkv;
    dl.K = d.d;
    dl.batch = d.batch;
    dl.ksplit = h->ks_kv;
    dl.part = part;
    dl.part_rows = h->win_max;
    dl.e.kind = EPI_KV;
    dl.e.kc = k_next;
    dl.e.vc = v_next;
    dl.e.nkv = h->nkv;
    dl.e.dh = d.head_dim;
    dl.e.win_max = h->win_max;
    dl.e.n_pos = d.n_pos;
    dl.e.geom = g;
    dl.e.sel_idx = sel->idx;
    dl.e.chk = h->chk.kv_next;
    dl.e.chk_rows = h->win_max;
    dl.e.chk_ld = 2 * h->nkv;
    PROF(POLESTAR_K_KVNEXT);
    e = launch_dl<T>(dl, h->sh_kv, g.n_win, s);
    if (e == hipSuccess) e = launch_dl_finish<T>(dl, g.n_win, s);
    if (e != hipSuccess) return POLESTAR_E_HIP;
  }
  return POLESTAR_OK;
}

template <typename T>
int do_refresh(polestar_handle* h, const polestar_layer* L, int32_t blk_start, const TokRows& t,
               const void* w_kv_next, void* k_next, void* v_next, void* ws, hipStream_t s) {
  if constexpr (std::is_same<T, bf16_t>::value)
    return do_refresh_dl(h, L, blk_start, t, w_kv_next, k_next, v_next, ws, s);
  const polestar_dims& d = h->dm;
  const WinGeom g = geom_of(h, blk_start);
  const polestar_packet* sel = t.sel;
  const int max_rows = t.n_act + (sel ? g.n_win : 0);
  const bool kv_next = w_kv_next && sel && g.n_win > 0;
  float* part = at<float>(ws, h->ws.part);
  // 1. h' = h + o W_O^T over rows [active; S]
  GemmArgs ga;
  memset(&ga, 0, sizeof(ga));
  ga.A.base = at<char>(ws, h->ws.o);
  ga.A.bstride = (int64_t)t.cap * h->nq;
  ga.A.lda = h->nq;
  ga.A.rowmap = sel ? sel->idx : nullptr;
  ga.A.map_bstride = h->win_max;
  ga.A.map_from = t.n_act;
  ga.A.map_off = d.block;
  set_rows(ga.A, t, max_rows);
  ga.W = L->w_o;
  ga.N = d.d;
  ga.K = h->nq;
  ga.batch = d.batch;
  ga.ksplit = h->ksplit;
  ga.part = part;
  ga.part_rows = t.cap;
  EpiParams ep;
  memset(&ep, 0, sizeof(ep));
  ep.kind = EPI_PARTIAL;
  hipError_t e;
  {
    PROF(POLESTAR_K_OPROJ);
    e = launch_gemm<T>(ga, ep, max_rows, s);
  }
  if (e != hipSuccess) return POLESTAR_E_HIP;
  RowReduceArgs rr;
  memset(&rr, 0, sizeof(rr));
  rr.part = part;
  rr.ksplit = h->ksplit;
  rr.part_rows = t.cap;
  rr.batch = d.batch;
  rr.d = d.d;
  rr.count = sel ? sel->count : nullptr;
  rr.block = t.n_act;
  rr.win_max = h->win_max;
  rr.res_a = t.h_act;
  rr.res_a_bstride = t.act_bstride;
  rr.res_split = t.n_act;
  rr.res_b = at<char>(ws, h->ws.win_rows);
  rr.res_b_bstride = (int64_t)h->win_max * d.d;
  rr.sel_idx = sel ? sel->idx : nullptr;
  rr.out_a = at<char>(ws, h->ws.hp);
  rr.out_a_bstride = (int64_t)t.cap * d.d;
  rr.out_split = t.cap;
  rr.out_f32 = 1;
  rr.norm = at<char>(ws, h->ws.a_gu);
  rr.norm_bstride = (int64_t)t.rcap * d.d;
  rr.norm_from = 0;
  rr.eps = h->pr.rms_eps;
  rr.chk = t.checks ? h->chk.hp : nullptr;
  rr.chk_rows = t.cap;
  {
    PROF(POLESTAR_K_OREDUCE);
    e = launch_row_reduce<T>(rr, max_rows, s);
  }
  if (e != hipSuccess) return POLESTAR_E_HIP;
  // 2. act = silu(g) * u with g, u the projections of RMSNorm(h')
  memset(&ga, 0, sizeof(ga));
  ga.A.base = rr.norm;
  ga.A.bstride = rr.norm_bstride;
  ga.A.lda = d.d;
  set_rows(ga.A, t, max_rows);
  ga.W = L->w_gu;
  ga.N = 2 * d.ffn;
  ga.K = d.d;
  ga.batch = d.batch;
  ga.ksplit = 1;
  memset(&ep, 0, sizeof(ep));
  ep.kind = EPI_SWIGLU;
  ep.act = at<char>(ws, h->ws.act);
  ep.act_rows = t.rcap;
  ep.ffn = d.ffn;
  {
    PROF(POLESTAR_K_GU);
    e = launch_gemm<T>(ga, ep, max_rows, s);
  }
  if (e != hipSuccess) return POLESTAR_E_HIP;
  // 3. out = h' + act W_down^T -> next active rows and the update packet
  memset(&ga, 0, sizeof(ga));
  ga.A.base = ep.act;
  ga.A.bstride = (int64_t)t.rcap * d.ffn;
  ga.A.lda = d.ffn;
  set_rows(ga.A, t, max_rows);
  ga.W = L->w_down;
  ga.N = d.d;
  ga.K = d.ffn;
  ga.batch = d.batch;
  ga.ksplit = h->ksplit;
  ga.part = part;
  ga.part_rows = t.cap;
  memset(&ep, 0, sizeof(ep));
  ep.kind = EPI_PARTIAL;
  {
    PROF(POLESTAR_K_DOWN);
    e = launch_gemm<T>(ga, ep, max_rows, s);
  }
  if (e != hipSuccess) return POLESTAR_E_HIP;
  RowReduceArgs r2 = rr;
  r2.res_a = rr.out_a;
  r2.res_a_f32 = 1;
  r2.res_a_bstride = (int64_t)t.cap * d.d;
  r2.res_split = t.cap;
  r2.res_b = nullptr;
  r2.out_a = t.h_out;
  r2.out_a_bstride = t.out_bstride;
  r2.out_split = t.n_act;
  r2.out_b = t.u_rows;
  r2.out_b_bstride = (int64_t)h->win_max * d.d;
  r2.out_f32 = 0;
  r2.norm = kv_next ? at<char>(ws, h->ws.a_kv) : nullptr;   // packet rows only
  r2.norm_bstride = (int64_t)h->rw * d.d;
  r2.norm_from = t.n_act;
  r2.chk = t.checks ? h->chk.out : nullptr;
  {
    PROF(POLESTAR_K_DREDUCE);
    e = launch_row_reduce<T>(r2, max_rows, s);
  }
  if (e != hipSuccess) return POLESTAR_E_HIP;
  // 4. K/V of layer l+1 for the packet rows, from RMSNorm(U)
  if (kv_next) {
    memset(&ga, 0, sizeof(ga));
    ga.A.base = r2.norm;
    ga.A.bstride = r2.norm_bstride;
    ga.A.lda = d.d;
    ga.A.rows_dev = sel->count;
    ga.A.rows_max = g.n_win;
    ga.W = w_kv_next;
    ga.N = 2 * h->nkv;
    ga.K = d.d;
    ga.batch = d.batch;
    ga.ksplit = 1;
    memset(&ep, 0, sizeof(ep));
    ep.kind = EPI_KV;
    ep.kc = k_next;
    ep.vc = v_next;
    ep.nkv = h->nkv;
    ep.dh = d.head_dim;
    ep.win_max = h->win_max;
    ep.n_pos = d.n_pos;
    ep.geom = g;
    ep.sel_idx = sel->idx;
    ep.chk = h->chk.kv_next;
    ep.chk_rows = h->win_max;
    ep.chk_ld = 2 * h->nkv;
    PROF(POLESTAR_K_KVNEXT);
    e = launch_gemm<T>(ga, ep, g.n_win, s);
    if (e != hipSuccess) return POLESTAR_E_HIP;
  }
  return POLESTAR_OK;
}

// Block entry of one layer: the forward of the rows at positions [r0, r1) (every position, or the
// window and the active block) with attention over the whole cache, the k-means of the window
// rows of h_in, and the centroids' proxy logits over the fresh cache.  The rows are taken in
// slabs of up to ec rows: first the Q/K/V of every slab (the cache must be complete before any
// row attends), then attention and the rest of the layer slab by slab.
template <typename T>
int do_entry(polestar_handle* h, int mode, const polestar_layer* L, int32_t blk_start, const void* h_in,
             const int32_t* init_idx, void* h_out, double* objective, float* act_logits, void* ws, hipStream_t s) {
  const polestar_dims& d = h->dm;
  const WinGeom g = geom_of(h, blk_start);
  const bool full = mode == POLESTAR_ENTRY_FULL;
  const int r0 = full ? 0 : blk_start - g.n_pre;
  const int r1 = full ? d.n_pos : blk_start + d.block + (g.n_win - g.n_pre);
  // slabs of at most ec rows, as even as 16-row tiles allow (one weight pass per slab)
  const int n_rows = r1 - r0, n_slabs = PS_CEIL_DIV(n_rows, h->ec);
  const int slab = std::min(h->ec, 16 * PS_CEIL_DIV(PS_CEIL_DIV(n_rows, n_slabs), 16));
  const int64_t hb = (int64_t)d.n_pos * d.d;   // elements between sequences of h_in, h_out
  const T* hin = (const T*)h_in;
  T* hout = (T*)h_out;
  float* q_all = at<float>(ws, h->ws.q_all);
  // 1. window clustering of the entry rows
  int rc = do_cluster<T>(h, POLESTAR_CLUSTER_ENTRY, L, blk_start, nullptr, init_idx, h_in, objective, ws, s, true);
  if (rc) return rc;
  // 2. Q/K/V of every recomputed row
  PrepArgs p;
  memset(&p, 0, sizeof(p));
  p.batch = d.batch;
  p.d = d.d;
  p.win_max = h->win_max;
  p.K = d.n_clusters;
  p.mq = h->mq;
  p.act_bstride = hb;
  p.win_z = L->win_z;
  p.a_qkv = at<char>(ws, h->ws.a_qkv);
  p.a_bstride = (int64_t)h->ec * d.d;
  p.a_tiles = std::is_same<T, bf16_t>::value ? h->ec / 16 : 0;
  p.eps = h->pr.rms_eps;
  for (int p0 = r0; p0 < r1; p0 += slab) {
    const int rows = std::min(slab, r1 - p0);
    p.block = rows;
    p.h_act = hin + (int64_t)p0 * d.d;
    const WinGeom gs = make_geom(p0, d.n_pos, rows, 0, 0);
    if ((rc = run_qkv<T>(h, L, p, rows, rows, gs, q_all + (int64_t)p0 * h->nq, d.n_pos, h->ec, false, ws, s)))
      return rc;
  }
  // 3. attention over all positions, O projection, SwiGLU FFN
  for (int p0 = r0; p0 < r1; p0 += slab) {
    const int rows = std::min(slab, r1 - p0);
    AttnArgs a = attn_base<T>(h, L, ws, h->ec);
    a.q = q_all + (int64_t)p0 * h->nq;
    a.mq = d.n_pos;
    a.n_tok = rows;
    a.block = rows;
    if ((rc = run_attention<T>(h, a, s))) return rc;
    const TokRows t = {rows, hin + (int64_t)p0 * d.d, hb, hout + (int64_t)p0 * d.d, hb, nullptr, nullptr, false,
                       h->ec, h->ec};
    if ((rc = do_refresh<T>(h, L, blk_start, t, nullptr, nullptr, nullptr, ws, s))) return rc;
  }
  // 4. (when asked) the active block's main-attention logits: the first reference of the commit
  //    drift; the block's queries are rows blk_start.. of q_all
  if (act_logits) {
    AttnArgs a = attn_base<T>(h, L, ws, h->mt);
    a.q = q_all + (int64_t)blk_start * h->nq;
    a.mq = d.n_pos;
    a.n_tok = d.block;
    a.act_logits = act_logits;
    a.act_kl = 0;
    if ((rc = run_attention<T>(h, a, s))) return rc;
  }
  // 5. proxy logits of the centroids: the first drift reference
  p.block = 0;
  p.n_win = 0;
  p.refresh = 1;
  p.h_act = nullptr;
  const WinGeom g0 = make_geom(0, d.n_pos, 0, 0, 0);
  float* q = at<float>(ws, h->ws.q);
  if ((rc = run_qkv<T>(h, L, p, d.n_clusters, 0, g0, q, h->mq, h->ec, false, ws, s))) return rc;
  AttnArgs a = attn_base<T>(h, L, ws, h->mt);
  a.q = q;
  a.n_tok = 0;
  a.n_proxy = d.n_clusters;
  a.block = 0;
  a.proxy_logits = L->proxy_logits;
  a.proxy_kl = 0;
  if (h->pr.proxy_support == POLESTAR_PROXY_ACTIVE) return run_attention_active_keys<T>(h, a, q, blk_start, s);
  return run_attention<T>(h, a, s);
}

// With h_full set (block entry): the rows are the active block and the suffix window read from the
// rows of every position, and the confidence alone decides (no drift, history untouched).
template <typename T>
int do_commit(polestar_handle* h, int32_t blk_start, const void* w_lm, const void* h_final,
              const polestar_packet* u_final, const float* delta, const uint8_t* active_masked,
              const uint8_t* suffix_masked, float* hist_vals, int32_t* hist_cnt, uint8_t* commit_active,
              uint8_t* commit_suffix, float* conf_active, int32_t* yhat_active, float* spike, float* conf_suffix,
              void* ws, hipStream_t s, const void* h_full = nullptr) {
  const polestar_dims& d = h->dm;
  const WinGeom g = geom_of(h, blk_start);
  const int lm_rows = d.block + d.win_suffix;
  LmPrepArgs lp;
  memset(&lp, 0, sizeof(lp));
  lp.batch = d.batch;
  lp.d = d.d;
  lp.block = d.block;
  lp.win_max = h->win_max;
  lp.win_suffix = d.win_suffix;
  lp.n_pre = g.n_pre;
  lp.lm_rows = lm_rows;
  lp.h_final = h_final;
  lp.h_full = h_full;
  lp.n_pos = d.n_pos;
  lp.blk_start = blk_start;
  lp.n_suf = g.n_win - g.n_pre;
  if (u_final) {
    lp.u_rows = u_final->rows;
    lp.u_idx = u_final->idx;
    lp.u_count = u_final->count;
  }
  lp.a_lm = at<char>(ws, h->ws.lm_a);
  lp.meta = at<int32_t>(ws, h->ws.lm_meta);
  lp.eps = h->pr.rms_eps;
  hipError_t e;
  {
    PROF(POLESTAR_K_LMPREP);
    e = launch_lm_prep<T>(lp, s);
  }
  if (e != hipSuccess) return POLESTAR_E_HIP;
  GemmArgs ga;
  memset(&ga, 0, sizeof(ga));
  ga.A.base = lp.a_lm;
  ga.A.bstride = (int64_t)lm_rows * d.d;
  ga.A.lda = d.d;
  ga.A.rows_dev = lp.meta;
  ga.A.rows_max = lm_rows;
  ga.W = w_lm;
  ga.N = d.vocab;
  ga.K = d.d;
  ga.batch = d.batch;
  ga.ksplit = 1;
  EpiParams ep;
  memset(&ep, 0, sizeof(ep));
  ep.kind = EPI_LMSTAT;
  ep.lm_stats = at<float>(ws, h->ws.lm_stats);
  ep.lm_rows = lm_rows;
  ep.lm_tiles = h->lm_tiles;
  ep.vocab = d.vocab;
  ep.mask_id = h->pr.mask_id;
  if constexpr (std::is_same<T, bf16_t>::value) {
    DlArgs dl;
    memset(&dl, 0, sizeof(dl));
    dl.A = ga.A;
    dl.planes = 1;
    dl.W = w_lm;
    dl.N = d.vocab;
    dl.K = d.d;
    dl.batch = d.batch;
    dl.ksplit = 1;
    dl.wg = weight_group(h, POLESTAR_W_LM);
    dl.e = ep;
    PROF(POLESTAR_K_LMHEAD);
    e = launch_dl<T>(dl, h->sh_lm, lm_rows, s);
  } else {
    PROF(POLESTAR_K_LMHEAD);
    e = launch_gemm<T>(ga, ep, lm_rows, s);
  }
  if (e != hipSuccess) return POLESTAR_E_HIP;
  DecideArgs da;
  memset(&da, 0, sizeof(da));
  da.batch = d.batch;
  da.block = d.block;
  da.win_suffix = d.win_suffix;
  da.win_max = h->win_max;
  da.n_pre = g.n_pre;
  da.lm_rows = lm_rows;
  da.lm_tiles = h->lm_tiles;
  da.hist = h->pr.hist;
  da.mask_id = h->pr.mask_id;
  da.tau_s = h->pr.tau_s;
  da.tau_suf = h->pr.tau_suf;
  da.alpha = h->pr.alpha;
  da.lm_stats = ep.lm_stats;
  da.lm_conf = at<float>(ws, h->ws.lm_conf);
  da.lm_yhat = (int32_t*)(da.lm_conf + (size_t)d.batch * lm_rows);
  da.meta = lp.meta;
  da.u_idx = lp.u_idx;
  da.delta = delta;
  da.active_masked = active_masked;
  da.suffix_masked = suffix_masked;
  da.hist_vals = hist_vals;
  da.hist_cnt = hist_cnt;
  da.commit_active = commit_active;
  da.commit_suffix = commit_suffix;
  da.conf_active = conf_active;
  da.yhat_active = yhat_active;
  da.spike = spike;
  da.conf_suffix = conf_suffix;
  da.entry = h_full != nullptr;
  PROF(POLESTAR_K_DECIDE);
  return hip_status(launch_decide(da, s));
}

}  // namespace

extern "C" {

const char* polestar_strerror(int code) {
  switch (code) {
    case POLESTAR_OK: return "ok";
    case POLESTAR_E_NULL: return "required pointer is NULL";
    case POLESTAR_E_SHAPE: return "inconsistent or out-of-range dimension";
    case POLESTAR_E_DTYPE: return "unknown dtype or residual format";
    case POLESTAR_E_UNSUPPORTED: return "configuration not supported";
    case POLESTAR_E_WORKSPACE: return "workspace too small";
    case POLESTAR_E_ALIGN: return "device pointer misaligned";
    case POLESTAR_E_HIP: return "HIP runtime error while enqueueing";
    case POLESTAR_E_ARG: return "invalid mode or scalar argument";
    case POLESTAR_E_SCRATCH:
      return "workspace larger than the library's static scratch (192 MiB): use polestar_step with a caller workspace";
  }
  return "unknown error";
}

int polestar_create(const polestar_dims* dims, const polestar_params* params, polestar_handle** out) {
  if (!dims || !params || !out) return POLESTAR_E_NULL;
  *out = nullptr;
  const polestar_dims& d = *dims;
  if (d.dtype != POLESTAR_F32 && d.dtype != POLESTAR_BF16) return POLESTAR_E_DTYPE;
  if (d.resid_fmt < POLESTAR_RESID_RAW || d.resid_fmt > POLESTAR_RESID_MXFP4) return POLESTAR_E_DTYPE;
  if (d.d <= 0 || d.n_heads <= 0 || d.n_kv_heads <= 0 || d.head_dim <= 0 || d.ffn <= 0 || d.n_pos <= 0 ||
      d.batch <= 0 || d.block <= 0 || d.win_prefix < 0 || d.win_suffix < 0 || d.n_clusters <= 0 ||
      d.top_k <= 0 || d.vocab < 0)
    return POLESTAR_E_SHAPE;
  if (d.n_heads % d.n_kv_heads != 0) return POLESTAR_E_SHAPE;
  if (d.n_pos < d.block) return POLESTAR_E_SHAPE;
  if (d.n_clusters > 16 || d.top_k > d.n_clusters) return POLESTAR_E_UNSUPPORTED;
  if (d.head_dim != 64 && d.head_dim != 128) return POLESTAR_E_UNSUPPORTED;
  if (d.block > 64 || d.win_prefix + d.win_suffix > 256) return POLESTAR_E_UNSUPPORTED;
  if (d.n_pos > kMaxPos) return POLESTAR_E_UNSUPPORTED;
  if (d.dtype == POLESTAR_F32 && d.n_pos > 1024) return POLESTAR_E_UNSUPPORTED;   // f32 attention keeps a row's scores in LDS
  if (d.d % 16 != 0) return POLESTAR_E_UNSUPPORTED;
  if (d.dtype == POLESTAR_BF16) {
    if (d.d % 128 || (d.n_heads * d.head_dim) % 128 || d.ffn % 128 || d.vocab % 16 || d.n_pos % 4 || d.n_pos < 8)
      return POLESTAR_E_UNSUPPORTED;
  } else {
    if (d.ffn % 4 || d.d % 4) return POLESTAR_E_UNSUPPORTED;
  }
  if (d.resid_fmt != POLESTAR_RESID_RAW && d.dtype != POLESTAR_BF16) return POLESTAR_E_UNSUPPORTED;
  const polestar_params& p = *params;
  if (!(p.rms_eps >= 0.f) || p.hist < 0 || p.hist > 16 || p.kmeans_iters < 0 || p.kmeans_iters > 1000)
    return POLESTAR_E_ARG;
  if (d.vocab > 0 && (p.mask_id < -1 || p.mask_id >= d.vocab)) return POLESTAR_E_ARG;
  if (p.proxy_support != POLESTAR_PROXY_ALL && p.proxy_support != POLESTAR_PROXY_ACTIVE) return POLESTAR_E_ARG;
  polestar_handle* h = new (std::nothrow) polestar_handle;
  if (!h) return POLESTAR_E_SHAPE;
  memset(h, 0, sizeof(*h));
  h->prof = new (std::nothrow) ProfState;
  if (!h->prof) {
    delete h;
    return POLESTAR_E_SHAPE;
  }
  h->dm = d;
  h->pr = p;
  h->win_max = d.win_prefix + d.win_suffix;
  h->mq = d.block + h->win_max + d.n_clusters;
  h->mt = d.block + h->win_max;
  h->nq = d.n_heads * d.head_dim;
  h->nkv = d.n_kv_heads * d.head_dim;
  h->rq = 16 * PS_CEIL_DIV(h->mq, 16);
  h->rt = 16 * PS_CEIL_DIV(h->mt, 16);
  h->ec = std::max(kMaxRows, h->rq);   // >= rq: every row list of a sequence fits one slab list
  h->rw = 16 * PS_CEIL_DIV(h->win_max, 16);
  const int ntiles = PS_CEIL_DIV(d.d, 64) * d.batch;
  int ks = PS_CEIL_DIV(256, ntiles);
  h->ksplit = ks < 1 ? 1 : (ks > 4 ? 4 : ks);
  // bf16 projections: tile width and split-K so that about 256 workgroups are busy
  {
    const int one[] = {DL_N192, DL_NARROW, DL_N96}, two[] = {DL_X512, DL_WIDE, DL_W192, DL_MID8, DL_P96, DL_P160};
    plan_projection(h->nq + 2 * h->nkv, d.d, d.batch, one, 3, 8, false, &h->sh_qkv, &h->ks_qkv);
    plan_projection(d.d, h->nq, d.batch, two, 6, 16, false, &h->sh_o, &h->ks_o);
    plan_projection(2 * d.ffn, d.d, d.batch, two, 6, 4, true, &h->sh_gu, &h->ks_gu);
    plan_projection(d.d, d.ffn, d.batch, two, 6, 16, false, &h->sh_down, &h->ks_down);
    plan_projection(2 * h->nkv, d.d, d.batch, one, 3, 16, false, &h->sh_kv, &h->ks_kv);
  }
  // bf16 attention: query rows in two groups when there are enough of them and one group per
  // (head, sequence) would leave compute units idle (a second group reads the keys and values
  // again, which at 16 sequences doubles the attention's traffic), and the keys split so that
  // about 256 workgroups run, at least 128 keys each
  {
    h->attn_rgroups = PS_CEIL_DIV(h->mq, 16) >= 6 && d.n_heads * d.batch * 2 <= 256 ? 2 : 1;
    const int blocks32 = PS_CEIL_DIV(d.n_pos, 32);
    int want = 256 / (d.n_heads * d.batch * h->attn_rgroups);
    want = want < 1 ? 1 : want;
    const int max_chunks = PS_CEIL_DIV(d.n_pos, 128);
    want = want > max_chunks ? max_chunks : want;
    h->attn_chunk = 32 * PS_CEIL_DIV(blocks32, want);
    h->attn_nchunks = PS_CEIL_DIV(d.n_pos, h->attn_chunk);
  }
  // LM head: float32 storage uses the register-streamed GEMM (64-id tiles); bf16 the weight-streaming
  // kernel without split (its epilogue forms each tile's softmax statistics) on its widest one-plane
  // tiles, 192 ids: the kernel's time per K step is set by the per-step work of a workgroup more
  // than by where the weights come from, so wider steps stream faster (measured 2.04 ms against
  // 2.77 ms for 128-id tiles at 16 sequences, n 4096 x 126464)
  h->sh_lm = DL_N192;
  if (d.dtype == POLESTAR_BF16 && d.vocab > 0) {
    h->lm_tiles = PS_CEIL_DIV(d.vocab, dl_tile_cols(h->sh_lm));
  } else {
    h->lm_tiles = PS_CEIL_DIV(d.vocab, 64);
  }
  layout(h);
  *out = h;
  return POLESTAR_OK;
}

void polestar_destroy(polestar_handle* h) {
  if (!h) return;
  delete h->prof;
  delete h;
}

int polestar_profile(polestar_handle* h, int enable) {
  if (!h) return POLESTAR_E_NULL;
  h->prof->clear();
  h->prof->on = enable != 0;
  return POLESTAR_OK;
}

int polestar_profile_read(polestar_handle* h, double* total_ms, int32_t* launches) {
  if (!h || !total_ms || !launches) return POLESTAR_E_NULL;
  for (int i = 0; i < POLESTAR_K_COUNT; ++i) {
    total_ms[i] = 0.0;
    launches[i] = 0;
  }
  for (const ProfState::Rec& r : h->prof->recs) {
    if (hipEventSynchronize(r.b) != hipSuccess) return POLESTAR_E_HIP;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) return POLESTAR_E_HIP;
    if (r.id >= 0 && r.id < POLESTAR_K_COUNT) {
      total_ms[r.id] += ms;
      launches[r.id] += 1;
    }
  }
  return POLESTAR_OK;
}

int polestar_workspace_size(const polestar_handle* h, size_t* bytes) {
  if (!h || !bytes) return POLESTAR_E_NULL;
  *bytes = h->ws.total;
  return POLESTAR_OK;
}

int polestar_set_check(polestar_handle* h, const polestar_check* chk) {
  if (!h) return POLESTAR_E_NULL;
  if (chk) h->chk = *chk;
  else memset(&h->chk, 0, sizeof(h->chk));
  return POLESTAR_OK;
}

static int weight_shape(const polestar_handle* h, int which, int* N, int* K) {
  const polestar_dims& d = h->dm;
  switch (which) {
    case POLESTAR_W_QKV: *N = h->nq + 2 * h->nkv; *K = d.d; break;
    case POLESTAR_W_O: *N = d.d; *K = h->nq; break;
    case POLESTAR_W_GU: *N = 2 * d.ffn; *K = d.d; break;
    case POLESTAR_W_DOWN: *N = d.d; *K = d.ffn; break;
    case POLESTAR_W_KV: *N = 2 * h->nkv; *K = d.d; break;
    case POLESTAR_W_LM:
      if (d.vocab <= 0) return POLESTAR_E_SHAPE;
      *N = d.vocab; *K = d.d; break;
    default: return POLESTAR_E_ARG;
  }
  return POLESTAR_OK;
}

int polestar_weight_packed_size(const polestar_handle* h, int which, size_t* bytes) {
  if (!h || !bytes) return POLESTAR_E_NULL;
  int N, K;
  int rc = weight_shape(h, which, &N, &K);
  if (rc) return rc;
  *bytes = packed_elems(N, K, weight_group(h, which)) * elt(h);
  return POLESTAR_OK;
}

int polestar_pack_weight(const polestar_handle* h, int which, const void* src, void* dst, void* stream) {
  if (!h || !src || !dst) return POLESTAR_E_NULL;
  int N, K;
  int rc = weight_shape(h, which, &N, &K);
  if (rc) return rc;
  if (!aligned16(src) || !aligned16(dst)) return POLESTAR_E_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  const int G = weight_group(h, which);
  hipError_t e = h->dm.dtype == POLESTAR_BF16 ? launch_pack<bf16_t>(which, src, dst, N, K, G, h->dm.ffn, s)
                                              : launch_pack<float>(which, src, dst, N, K, G, h->dm.ffn, s);
  return hip_status(e);
}

static int check_cluster(const polestar_handle* h, int mode, const polestar_layer* L, int32_t blk_start,
                         const polestar_packet* u_in, const int32_t* init_idx, const void* entry_h, const void* ws,
                         size_t ws_bytes) {
  if (!h || !L) return POLESTAR_E_NULL;
  if (mode != POLESTAR_CLUSTER_ENTRY && mode != POLESTAR_CLUSTER_UPDATE) return POLESTAR_E_ARG;
  int rc = check_ws(h, ws, ws_bytes);
  if (rc) return rc;
  if ((rc = check_blk(h, blk_start))) return rc;
  const bool nv = h->dm.resid_fmt != POLESTAR_RESID_RAW;   // residual codes instead of raw rows
  if (!L->win_z || !L->win_m) return POLESTAR_E_NULL;
  if (nv ? (!L->win_codes || (resid_scale_bytes(h->dm.resid_fmt, h->dm.d) > 0 && !L->win_scales)) : !L->win_h)
    return POLESTAR_E_NULL;
  if (mode == POLESTAR_CLUSTER_ENTRY && (!init_idx || !entry_h)) return POLESTAR_E_NULL;
  if (u_in && (!u_in->rows || !u_in->idx || !u_in->count)) return POLESTAR_E_NULL;
  if (!aligned16(L->win_z) || (!nv && !aligned16(L->win_h)) || (entry_h && !aligned16(entry_h)) ||
      (u_in && !aligned16(u_in->rows)))
    return POLESTAR_E_ALIGN;
  return POLESTAR_OK;
}

int polestar_cluster(polestar_handle* h, int mode, const polestar_layer* L, int32_t blk_start,
                     const polestar_packet* u_in, const int32_t* init_idx, const void* entry_h, double* objective,
                     void* ws, size_t ws_bytes, void* stream) {
  const int rc = check_cluster(h, mode, L, blk_start, u_in, init_idx, entry_h, ws, ws_bytes);
  if (rc) return rc;
  hipStream_t s = (hipStream_t)stream;
  return h->dm.dtype == POLESTAR_BF16
             ? do_cluster<bf16_t>(h, mode, L, blk_start, u_in, init_idx, entry_h, objective, ws, s)
             : do_cluster<float>(h, mode, L, blk_start, u_in, init_idx, entry_h, objective, ws, s);
}

static int check_drift(const polestar_handle* h, int mode, const polestar_layer* L, int32_t blk_start,
                       const void* h_active, const polestar_packet* u_in, const polestar_packet* sel,
                       const float* act_logits, const float* delta, const void* ws, size_t ws_bytes) {
  if (!h || !L || !h_active || !sel || !sel->idx || !sel->count) return POLESTAR_E_NULL;
  if (mode != POLESTAR_DRIFT_REFRESH && mode != POLESTAR_DRIFT_ACTIVE_ONLY) return POLESTAR_E_ARG;
  int rc = check_ws(h, ws, ws_bytes);
  if (rc) return rc;
  if ((rc = check_blk(h, blk_start))) return rc;
  if (!L->w_qkv || !L->k_cache || !L->v_cache) return POLESTAR_E_NULL;
  if (mode == POLESTAR_DRIFT_REFRESH && (!L->win_z || !L->win_m || !L->proxy_logits)) return POLESTAR_E_NULL;
  if (!aligned16(L->w_qkv) || !aligned16(h_active)) return POLESTAR_E_ALIGN;
  if (mode == POLESTAR_DRIFT_REFRESH && !aligned16(L->win_z)) return POLESTAR_E_ALIGN;
  if (delta && !act_logits) return POLESTAR_E_NULL;
  if (u_in && (!u_in->idx || !u_in->count)) return POLESTAR_E_NULL;
  if (L->q_win && (!L->q_ok)) return POLESTAR_E_NULL;
  if (L->q_win && !aligned16(L->q_win)) return POLESTAR_E_ALIGN;
  return POLESTAR_OK;
}

int polestar_drift(polestar_handle* h, int mode, const polestar_layer* L, int32_t blk_start, const void* h_active,
                   const polestar_packet* u_in, float* D, int32_t* topk, polestar_packet* sel, float* act_logits,
                   float* delta, void* ws, size_t ws_bytes, void* stream) {
  const int rc = check_drift(h, mode, L, blk_start, h_active, u_in, sel, act_logits, delta, ws, ws_bytes);
  if (rc) return rc;
  hipStream_t s = (hipStream_t)stream;
  return h->dm.dtype == POLESTAR_BF16
             ? do_drift<bf16_t>(h, mode, L, blk_start, h_active, u_in, D, topk, sel, act_logits, delta, ws, s)
             : do_drift<float>(h, mode, L, blk_start, h_active, u_in, D, topk, sel, act_logits, delta, ws, s);
}

static int check_refresh(const polestar_handle* h, const polestar_layer* L, int32_t blk_start,
                         const void* h_active, const polestar_packet* sel, const void* w_kv_next,
                         const void* k_next, const void* v_next, const void* h_active_out, const void* u_rows,
                         const void* ws, size_t ws_bytes) {
  if (!h || !L || !h_active || !sel || !sel->idx || !sel->count || !h_active_out || !u_rows) return POLESTAR_E_NULL;
  int rc = check_ws(h, ws, ws_bytes);
  if (rc) return rc;
  if ((rc = check_blk(h, blk_start))) return rc;
  if (!L->w_o || !L->w_gu || !L->w_down) return POLESTAR_E_NULL;
  if (w_kv_next && (!k_next || !v_next)) return POLESTAR_E_NULL;
  if (!aligned16(L->w_o) || !aligned16(L->w_gu) || !aligned16(L->w_down) || !aligned16(h_active) ||
      !aligned16(h_active_out) || !aligned16(u_rows) || (w_kv_next && !aligned16(w_kv_next)))
    return POLESTAR_E_ALIGN;
  return POLESTAR_OK;
}

int polestar_refresh(polestar_handle* h, const polestar_layer* L, int32_t blk_start, const void* h_active,
                     const polestar_packet* sel, const void* w_kv_next, void* k_next, void* v_next,
                     void* h_active_out, void* u_rows, void* ws, size_t ws_bytes, void* stream) {
  const int rc = check_refresh(h, L, blk_start, h_active, sel, w_kv_next, k_next, v_next, h_active_out, u_rows, ws,
                               ws_bytes);
  if (rc) return rc;
  hipStream_t s = (hipStream_t)stream;
  const int64_t bs = (int64_t)h->dm.block * h->dm.d;
  const TokRows t = {h->dm.block, h_active, bs, h_active_out, bs, sel, u_rows, true, h->mt, h->rt};
  return h->dm.dtype == POLESTAR_BF16 ? do_refresh<bf16_t>(h, L, blk_start, t, w_kv_next, k_next, v_next, ws, s)
                                      : do_refresh<float>(h, L, blk_start, t, w_kv_next, k_next, v_next, ws, s);
}

int polestar_step(polestar_handle* h, int mode, int32_t n_layers, const polestar_layer* layers, int32_t blk_start,
                  void* h_act0, void* h_act1, polestar_packet* pk0, polestar_packet* pk1, float* D, int32_t* topk,
                  float* act_logits, float* delta, void* ws, size_t ws_bytes, void* stream) {
  if (!h || !layers || !h_act0 || !h_act1 || !pk0 || !pk1 || !pk0->rows || !pk1->rows) return POLESTAR_E_NULL;
  if (n_layers < 1) return POLESTAR_E_ARG;
  if (mode != POLESTAR_DRIFT_REFRESH && mode != POLESTAR_DRIFT_ACTIVE_ONLY) return POLESTAR_E_ARG;
  void* act[2] = {h_act0, h_act1};
  polestar_packet* pk[2] = {pk0, pk1};
  const bool refresh = mode == POLESTAR_DRIFT_REFRESH;
  // every call of the step is validated before the first launch
  for (int l = 0; l < n_layers; ++l) {
    const polestar_layer* L = &layers[l];
    const bool last = l == n_layers - 1;
    const polestar_packet* u_in = refresh && l > 0 ? pk[(l - 1) % 2] : nullptr;
    int rc;
    if (refresh && (rc = check_cluster(h, POLESTAR_CLUSTER_UPDATE, L, blk_start, u_in, nullptr, nullptr, ws, ws_bytes)))
      return rc;
    if ((rc = check_drift(h, mode, L, blk_start, act[l % 2], u_in, pk[l % 2], last ? act_logits : nullptr,
                          last ? delta : nullptr, ws, ws_bytes)))
      return rc;
    if ((rc = check_refresh(h, L, blk_start, act[l % 2], pk[l % 2], nullptr, nullptr, nullptr, act[(l + 1) % 2],
                            pk[l % 2]->rows, ws, ws_bytes)))
      return rc;
  }
  hipStream_t s = (hipStream_t)stream;
  const bool bf = h->dm.dtype == POLESTAR_BF16;
  const int64_t bs = (int64_t)h->dm.block * h->dm.d;
  for (int l = 0; l < n_layers; ++l) {
    const polestar_layer* L = &layers[l];
    const bool last = l == n_layers - 1;
    const polestar_packet* u_in = refresh && l > 0 ? pk[(l - 1) % 2] : nullptr;
    float* al = last ? act_logits : nullptr;
    float* dl = last ? delta : nullptr;
    int rc = POLESTAR_OK;
    if (refresh)
      rc = bf ? do_cluster<bf16_t>(h, POLESTAR_CLUSTER_UPDATE, L, blk_start, u_in, nullptr, nullptr, nullptr, ws, s)
              : do_cluster<float>(h, POLESTAR_CLUSTER_UPDATE, L, blk_start, u_in, nullptr, nullptr, nullptr, ws, s);
    if (rc) return rc;
    rc = bf ? do_drift<bf16_t>(h, mode, L, blk_start, act[l % 2], u_in, D, topk, pk[l % 2], al, dl, ws, s)
            : do_drift<float>(h, mode, L, blk_start, act[l % 2], u_in, D, topk, pk[l % 2], al, dl, ws, s);
    if (rc) return rc;
    const TokRows t = {h->dm.block, act[l % 2], bs, act[(l + 1) % 2], bs, pk[l % 2], pk[l % 2]->rows, true,
                       h->mt, h->rt};
    rc = bf ? do_refresh<bf16_t>(h, L, blk_start, t, nullptr, nullptr, nullptr, ws, s)
            : do_refresh<float>(h, L, blk_start, t, nullptr, nullptr, nullptr, ws, s);
    if (rc) return rc;
  }
  return POLESTAR_OK;
}

int polestar_entry(polestar_handle* h, int mode, const polestar_layer* L, int32_t blk_start, const void* h_in,
                   const int32_t* init_idx, void* h_out, double* objective, float* act_logits, void* ws,
                   size_t ws_bytes, void* stream) {
  if (!h || !L || !h_in || !init_idx || !h_out) return POLESTAR_E_NULL;
  if (mode != POLESTAR_ENTRY_FULL && mode != POLESTAR_ENTRY_WINDOW) return POLESTAR_E_ARG;
  int rc = check_ws(h, ws, ws_bytes);
  if (rc) return rc;
  if ((rc = check_blk(h, blk_start))) return rc;
  const bool nv = h->dm.resid_fmt != POLESTAR_RESID_RAW;
  if (!L->w_qkv || !L->w_o || !L->w_gu || !L->w_down || !L->k_cache || !L->v_cache || !L->win_z || !L->win_m ||
      !L->proxy_logits)
    return POLESTAR_E_NULL;
  if (nv ? (!L->win_codes || (resid_scale_bytes(h->dm.resid_fmt, h->dm.d) > 0 && !L->win_scales)) : !L->win_h)
    return POLESTAR_E_NULL;
  if (!aligned16(L->w_qkv) || !aligned16(L->w_o) || !aligned16(L->w_gu) || !aligned16(L->w_down) ||
      !aligned16(L->win_z) || (!nv && !aligned16(L->win_h)) || !aligned16(h_in) || !aligned16(h_out))
    return POLESTAR_E_ALIGN;
  const size_t bytes = (size_t)h->dm.batch * h->dm.n_pos * h->dm.d * elt(h);
  const char *a0 = (const char*)h_in, *b0 = (const char*)h_out;
  if (a0 < b0 + bytes && b0 < a0 + bytes) return POLESTAR_E_ARG;   // h_out must not overlap h_in
  hipStream_t s = (hipStream_t)stream;
  return h->dm.dtype == POLESTAR_BF16
             ? do_entry<bf16_t>(h, mode, L, blk_start, h_in, init_idx, h_out, objective, act_logits, ws, s)
             : do_entry<float>(h, mode, L, blk_start, h_in, init_idx, h_out, objective, act_logits, ws, s);
}

int polestar_commit(polestar_handle* h, int32_t blk_start, const void* w_lm, const void* h_final,
                    const polestar_packet* u_final, const float* delta, const uint8_t* active_masked,
                    const uint8_t* suffix_masked, float* hist_vals, int32_t* hist_cnt, uint8_t* commit_active,
                    uint8_t* commit_suffix, float* conf_active, int32_t* yhat_active, float* spike,
                    float* conf_suffix, void* ws, size_t ws_bytes, void* stream) {
  if (!h || !w_lm || !h_final || !delta || !active_masked || !suffix_masked || !hist_vals || !hist_cnt ||
      !commit_active || !commit_suffix || !conf_active || !yhat_active || !spike || !conf_suffix)
    return POLESTAR_E_NULL;
  if (h->dm.vocab <= 0) return POLESTAR_E_SHAPE;
  int rc = check_ws(h, ws, ws_bytes);
  if (rc) return rc;
  if ((rc = check_blk(h, blk_start))) return rc;
  if (u_final && (!u_final->rows || !u_final->idx || !u_final->count)) return POLESTAR_E_NULL;
  if (!aligned16(w_lm) || !aligned16(h_final) || (u_final && !aligned16(u_final->rows))) return POLESTAR_E_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  return h->dm.dtype == POLESTAR_BF16
             ? do_commit<bf16_t>(h, blk_start, w_lm, h_final, u_final, delta, active_masked, suffix_masked,
                                 hist_vals, hist_cnt, commit_active, commit_suffix, conf_active, yhat_active, spike,
                                 conf_suffix, ws, s)
             : do_commit<float>(h, blk_start, w_lm, h_final, u_final, delta, active_masked, suffix_masked,
                                hist_vals, hist_cnt, commit_active, commit_suffix, conf_active, yhat_active, spike,
                                conf_suffix, ws, s);
}

int polestar_entry_commit(polestar_handle* h, int32_t blk_start, const void* w_lm, const void* h_full,
                          const uint8_t* active_masked, const uint8_t* suffix_masked, uint8_t* commit_active,
                          uint8_t* commit_suffix, float* conf_active, int32_t* yhat_active, float* conf_suffix,
                          void* ws, size_t ws_bytes, void* stream) {
  if (!h || !w_lm || !h_full || !active_masked || !suffix_masked || !commit_active || !commit_suffix ||
      !conf_active || !yhat_active || !conf_suffix)
    return POLESTAR_E_NULL;
  if (h->dm.vocab <= 0) return POLESTAR_E_SHAPE;
  int rc = check_ws(h, ws, ws_bytes);
  if (rc) return rc;
  if ((rc = check_blk(h, blk_start))) return rc;
  if (!aligned16(w_lm) || !aligned16(h_full)) return POLESTAR_E_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  return h->dm.dtype == POLESTAR_BF16
             ? do_commit<bf16_t>(h, blk_start, w_lm, nullptr, nullptr, nullptr, active_masked, suffix_masked, nullptr,
                                 nullptr, commit_active, commit_suffix, conf_active, yhat_active, nullptr,
                                 conf_suffix, ws, s, h_full)
             : do_commit<float>(h, blk_start, w_lm, nullptr, nullptr, nullptr, active_masked, suffix_masked, nullptr,
                                nullptr, commit_active, commit_suffix, conf_active, yhat_active, nullptr,
                                conf_suffix, ws, s, h_full);
}

}  // extern "C"

// ---- the step for callers that cannot allocate ------------------------------------------------
// The workspace of polestar_step_noalloc: one array per device, placed by the loader with the
// code object.  In host code `scratch` only names the symbol; its device address comes from
// hipGetSymbolAddress, once per device, and only that address is ever passed to kernels.
static __device__ __align__(256) unsigned char scratch[POLESTAR_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array (looked up on the first call there).
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return POLESTAR_E_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return POLESTAR_E_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return POLESTAR_OK;
}
}  // namespace

extern "C" {

int polestar_step_noalloc(polestar_handle* h, int mode, int32_t n_layers, const polestar_layer* layers,
                          int32_t blk_start, void* h_act0, void* h_act1, polestar_packet* pk0, polestar_packet* pk1,
                          float* D, int32_t* topk, float* act_logits, float* delta, void* stream) {
  if (!h) return POLESTAR_E_NULL;
  if (h->ws.total > (size_t)POLESTAR_SCRATCH_BYTES) return POLESTAR_E_SCRATCH;
  void* ws = nullptr;
  int rc = scratch_address(&ws);
  if (rc) return rc;
  // no profiling events here: recording them creates host objects on demand
  const bool prof_on = h->prof->on;
  h->prof->on = false;
  rc = polestar_step(h, mode, n_layers, layers, blk_start, h_act0, h_act1, pk0, pk1, D, topk, act_logits, delta, ws,
                     POLESTAR_SCRATCH_BYTES, stream);
  h->prof->on = prof_on;
  return rc;
}

int polestar_should_refresh(int32_t decoded_since_refresh, int32_t tau_upd) {
  if (tau_upd < 0) return 0;
  return decoded_since_refresh > tau_upd ? 1 : 0;
}

int polestar_nvfp4_pack(const float* x, int64_t rows, int32_t d, uint8_t* codes, uint8_t* scales, void* stream) {
  if (!x || !codes || !scales) return POLESTAR_E_NULL;
  if (rows < 0 || d <= 0 || d % 16) return POLESTAR_E_SHAPE;
  if (!aligned16(x)) return POLESTAR_E_ALIGN;
  return hip_status(launch_nvfp4_pack(x, rows, d, codes, scales, (hipStream_t)stream));
}

int polestar_nvfp4_unpack(const uint8_t* codes, const uint8_t* scales, int64_t rows, int32_t d, float* x,
                          void* stream) {
  if (!x || !codes || !scales) return POLESTAR_E_NULL;
  if (rows < 0 || d <= 0 || d % 16) return POLESTAR_E_SHAPE;
  return hip_status(launch_nvfp4_unpack(codes, scales, rows, d, x, (hipStream_t)stream));
}

int polestar_resid_bytes(int32_t fmt, int32_t d, int64_t* code_bytes, int64_t* scale_bytes) {
  if (!code_bytes || !scale_bytes) return POLESTAR_E_NULL;
  if (fmt < POLESTAR_RESID_RAW || fmt > POLESTAR_RESID_MXFP4) return POLESTAR_E_DTYPE;
  if (d <= 0 || d % 32) return POLESTAR_E_SHAPE;
  *code_bytes = resid_code_bytes(fmt, d);
  *scale_bytes = resid_scale_bytes(fmt, d);
  return POLESTAR_OK;
}

int polestar_resid_pack(int32_t fmt, const float* x, int64_t rows, int32_t d, uint8_t* codes, uint8_t* scales,
                        void* stream) {
  if (fmt <= POLESTAR_RESID_RAW || fmt > POLESTAR_RESID_MXFP4) return POLESTAR_E_DTYPE;
  if (rows < 0 || d <= 0 || d % 32) return POLESTAR_E_SHAPE;
  if (rows > 0 && (!x || !codes || (resid_scale_bytes(fmt, d) > 0 && !scales))) return POLESTAR_E_NULL;
  return hip_status(launch_resid_pack(fmt, x, rows, d, codes, scales, (hipStream_t)stream));
}

int polestar_resid_unpack(int32_t fmt, const uint8_t* codes, const uint8_t* scales, int64_t rows, int32_t d, float* x,
                          void* stream) {
  if (fmt <= POLESTAR_RESID_RAW || fmt > POLESTAR_RESID_MXFP4) return POLESTAR_E_DTYPE;
  if (rows < 0 || d <= 0 || d % 32) return POLESTAR_E_SHAPE;
  if (rows > 0 && (!x || !codes || (resid_scale_bytes(fmt, d) > 0 && !scales))) return POLESTAR_E_NULL;
  return hip_status(launch_resid_unpack(fmt, codes, scales, rows, d, x, (hipStream_t)stream));
}

int polestar_kv_staleness(const polestar_handle* h, const void* k_cache, const void* v_cache, const void* k_ref,
                          const void* v_ref, float* stale, void* stream) {
  if (!h || !k_cache || !v_cache || !k_ref || !v_ref || !stale) return POLESTAR_E_NULL;
  StaleArgs a;
  a.batch = h->dm.batch;
  a.n_pos = h->dm.n_pos;
  a.hkv = h->dm.n_kv_heads;
  a.dh = h->dm.head_dim;
  a.k = k_cache;
  a.v = v_cache;
  a.k_ref = k_ref;
  a.v_ref = v_ref;
  a.stale = stale;
  const hipStream_t s = (hipStream_t)stream;
  return hip_status(h->dm.dtype == POLESTAR_BF16 ? launch_kv_staleness<bf16_t>(a, s) : launch_kv_staleness<float>(a, s));
}

int polestar_attended_change(const polestar_handle* h, const float* q, int32_t rows, int32_t q_ld,
                             int64_t q_bstride, const void* k_cache, const void* k_ref, int32_t* top_pos,
                             float* score, void* stream) {
  if (!h) return POLESTAR_E_NULL;
  if (rows < 0) return POLESTAR_E_SHAPE;
  if (rows == 0) return POLESTAR_OK;
  if (!q || !k_cache || !k_ref || !top_pos || !score) return POLESTAR_E_NULL;
  const polestar_dims& d = h->dm;
  if (q_ld < d.n_heads * d.head_dim || q_bstride < (int64_t)(rows - 1) * q_ld + d.n_heads * d.head_dim)
    return POLESTAR_E_SHAPE;
  AttendArgs a;
  a.q = q;
  a.q_bstride = q_bstride;
  a.q_ld = q_ld;
  a.rows = rows;
  a.k = k_cache;
  a.k_ref = k_ref;
  a.batch = d.batch;
  a.n_pos = d.n_pos;
  a.hq = d.n_heads;
  a.hkv = d.n_kv_heads;
  a.dh = d.head_dim;
  a.top = top_pos;
  a.score = score;
  const hipStream_t s = (hipStream_t)stream;
  return hip_status(d.dtype == POLESTAR_BF16 ? launch_attended_change<bf16_t>(a, s) : launch_attended_change<float>(a, s));
}

int polestar_nvfp4_pack_host(const float* x, int64_t rows, int32_t d, uint8_t* codes, uint8_t* scales) {
  if (!x || !codes || !scales) return POLESTAR_E_NULL;
  if (rows < 0 || d <= 0 || d % 16) return POLESTAR_E_SHAPE;
  const int64_t groups = rows * (d / 16);
  for (int64_t g = 0; g < groups; ++g) {
    uint32_t c[16];
    scales[g] = (uint8_t)nvfp4_group(x + g * 16, c);
    for (int e = 0; e < 8; ++e) codes[g * 8 + e] = (uint8_t)(c[2 * e] | (c[2 * e + 1] << 4));
  }
  return POLESTAR_OK;
}

}  // extern "C"
