/*
 * polestar.h — C ABI of the drift-scored sparse KV refresh for masked-diffusion
 * LLMs (Polestar-Cache) and its drift-aware commit rule (Polestar-Commit),
 * implemented as HIP kernels for AMD Instinct MI355X (gfx950).
 *
 * Source of the method: "Polestar: Drift-Aware Cache Calibration and Token
 * Commitment for Efficient Inference of Diffusion LLMs" (arXiv 2607.14107);
 * each call below names the section, equation, table or Algorithm 1 step
 * group it implements.
 *
 * Conventions shared by every call
 * --------------------------------
 * Pointers: every tensor pointer is a DEVICE pointer unless documented as
 *   host.  The caller allocates and owns all memory (weights, caches, window
 *   state, packets, outputs and the workspace); the library never allocates
 *   device memory and keeps only host-side dimensions in the handle.
 * Storage dtype: dims.dtype selects float32 (POLESTAR_F32) or bfloat16
 *   (POLESTAR_BF16, stored as raw uint16 bit patterns) for weights, KV caches,
 *   hidden rows and centroids.  Drift logits, drift values, confidences and
 *   spikes are always float32.
 * Layouts (row-major, batch outermost):
 *   hidden rows          [batch, rows, d]
 *   K cache (per layer)  [batch, n_pos, n_kv_heads, head_dim]   (token-major)
 *   V cache (per layer)  [batch, n_kv_heads, head_dim, n_pos]   (transposed:
 *                        keys contiguous, the layout the attention streams)
 *   window rows          [batch, win_max, d], win_max = win_prefix + win_suffix;
 *                        window row w is the w-th position, ascending, of
 *                        [blk_start - win_prefix, blk_start) U
 *                        [blk_start + block, blk_start + block + win_suffix),
 *                        clipped to [0, n_pos); n_win <= win_max rows are used.
 *   window codes         [batch, win_max, code bytes per row] u8 and scales
 *                        [batch, win_max, scale bytes per row] u8 of the
 *                        residual format (polestar_resid_bytes): NVFP4 d/2
 *                        nibbles (element 2j low nibble, 2j+1 high) + d/16
 *                        E4M3FN scales; FP8 d E4M3FN bytes; MXINT8 d int8
 *                        + d/32 E8M0 scales; MXFP4 d/2 nibbles + d/32 E8M0
 *   centroids            [batch, n_clusters, d]; labels [batch, win_max] i32
 *   proxy logits         [batch, n_clusters, n_heads, n_pos] f32
 *   active-block logits  [batch, block, n_heads, n_pos] f32
 *   packed weights       produced by polestar_pack_weight (opaque layout)
 * Precision: storage dtype f32 or bf16.  Rounded to it: tensors that
 *   outlive a call (K/V caches, window rows, centroids, active outputs,
 *   update packets) and the input of each projection of such a row, its
 *   RMSNorm output with unit gain (QKV and proxy queries, next-layer K/V,
 *   LM head).  Values produced and consumed inside one call (queries,
 *   attention output, h', RMSNorm(h'), the SwiGLU product), logits, softmax,
 *   KL and every accumulation are float32.  The pages fix no rounding points
 *   (their full-precision baseline is a 16-bit model, Table 11).
 * Alignment: row tensors (hidden rows, window rows, centroids, packets) and
 *   packed weights start on 16-byte boundaries; a call that reads or writes
 *   one row-wise checks it and returns POLESTAR_E_ALIGN otherwise.
 * Streams: every call enqueues asynchronously on the given hipStream_t
 *   (passed as void*; NULL = the null stream) and never synchronises.
 *   Outputs are valid once the caller synchronises that stream.  A handle is
 *   used by one stream at a time.
 * Workspace: calls take a caller-allocated device workspace of at least
 *   polestar_workspace_size() bytes (256-byte aligned).  The calls for one
 *   layer of one refresh step must run in the order cluster -> drift ->
 *   refresh on the same workspace: cluster leaves the patched window rows in
 *   it, drift leaves the attention outputs in it.
 * Errors: every int-returning call returns POLESTAR_OK (0) or a negative
 *   code.  Arguments are validated on the host before anything is enqueued,
 *   so a failed call has launched nothing.  POLESTAR_E_HIP reports a launch
 *   error (hipGetLastError); faults inside kernels surface at the caller's
 *   synchronisation.  No C++ exception crosses this interface.
 */
#ifndef POLESTAR_H
#define POLESTAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  POLESTAR_OK = 0,
  POLESTAR_E_NULL = -1,        /* required pointer is NULL */
  POLESTAR_E_SHAPE = -2,       /* inconsistent or out-of-range dimension */
  POLESTAR_E_DTYPE = -3,       /* unknown dtype / residual format */
  POLESTAR_E_UNSUPPORTED = -4, /* valid but not implemented (K > 16, k > K, ...) */
  POLESTAR_E_WORKSPACE = -5,   /* workspace smaller than polestar_workspace_size */
  POLESTAR_E_ALIGN = -6,       /* device pointer not 16-byte aligned */
  POLESTAR_E_HIP = -7,         /* HIP runtime error while enqueueing */
  POLESTAR_E_ARG = -8,         /* invalid mode or scalar argument */
  POLESTAR_E_SCRATCH = -9      /* workspace larger than the library's static scratch (polestar_step_noalloc) */
};

enum { POLESTAR_F32 = 0, POLESTAR_BF16 = 1 };
enum {
  POLESTAR_RESID_RAW = 0,     /* window rows stored as they are */
  POLESTAR_RESID_NVFP4 = 1,   /* residual to the centroid: E2M1 + E4M3FN scale per 16 [App. C.3] */
  POLESTAR_RESID_FP8 = 2,     /* residual as E4M3FN per value, no scale [Table 11] */
  POLESTAR_RESID_MXINT8 = 3,  /* residual as int8 with an E8M0 scale per 32 (OCP MX) [Table 11 "INT8"] */
  POLESTAR_RESID_MXFP4 = 4    /* residual as E2M1 with an E8M0 scale per 32 (OCP MX) [Table 11] */
};
enum { POLESTAR_CLUSTER_ENTRY = 0, POLESTAR_CLUSTER_UPDATE = 1 };
enum { POLESTAR_DRIFT_REFRESH = 0, POLESTAR_DRIFT_ACTIVE_ONLY = 1 };
enum { POLESTAR_ENTRY_FULL = 0, POLESTAR_ENTRY_WINDOW = 1 };
/* Keys of the proxy attention [§4.1 "Measuring Drift and Layer-wise KV Updates"; Eq. 3]:
 * ALL    every position, the cached keys together with the recomputed active-block keys (the
 *        attention support the page's drift is defined over);
 * ACTIVE the active block's keys only, positions [blk_start, blk_start + block).  The proxy
 *        logits buffer then holds meaningful values at those key positions only. */
enum { POLESTAR_PROXY_ALL = 0, POLESTAR_PROXY_ACTIVE = 1 };
enum {
  POLESTAR_W_QKV = 0,  /* src [(n_heads + 2 n_kv_heads) head_dim, d] = rows of W_Q, W_K, W_V */
  POLESTAR_W_O = 1,    /* src [d, n_heads head_dim] */
  POLESTAR_W_GU = 2,   /* src [2 ffn, d] = rows of W_gate then W_up */
  POLESTAR_W_DOWN = 3, /* src [d, ffn] */
  POLESTAR_W_KV = 4,   /* src [2 n_kv_heads head_dim, d] = rows of W_K then W_V */
  POLESTAR_W_LM = 5    /* src [vocab, d] */
};

/* Model and method dimensions (host struct, copied into the handle). */
typedef struct polestar_dims {
  int32_t d;          /* hidden size */
  int32_t n_heads;    /* query heads */
  int32_t n_kv_heads; /* key/value heads; n_heads % n_kv_heads == 0 */
  int32_t head_dim;   /* 64 or 128 */
  int32_t ffn;        /* SwiGLU width */
  int32_t n_pos;      /* positions per sequence (prompt + generation); bf16: multiple of 4, at
                         most 4096; f32: at most 1024 */
  int32_t batch;      /* independent sequences processed together */
  int32_t block;      /* active block size B (<= 64) */
  int32_t win_prefix; /* |Omega_p| */
  int32_t win_suffix; /* |Omega_s|; win_prefix + win_suffix <= 256 */
  int32_t n_clusters; /* K (1..16) */
  int32_t top_k;      /* k (1..K) */
  int32_t vocab;      /* LM-head rows, 0 when polestar_commit is not used */
  int32_t dtype;      /* POLESTAR_F32 | POLESTAR_BF16 */
  int32_t resid_fmt;  /* POLESTAR_RESID_* (formats other than RAW: bf16 only) */
} polestar_dims;

/* Scalar hyper-parameters [Polestar §5.1 and Table 5]. */
typedef struct polestar_params {
  float rms_eps;        /* RMSNorm epsilon (unit gain) */
  float tau_s;          /* static confidence threshold (0.9) */
  float tau_suf;        /* suffix commit confidence (0.9) */
  float alpha;          /* drift-gate coefficient (10) */
  int32_t hist;         /* drift history length h (5), 0..16 */
  int32_t mask_id;      /* vocabulary id excluded from the confidence max */
  int32_t kmeans_iters; /* Lloyd iterations at block entry (10) */
  int32_t proxy_support; /* POLESTAR_PROXY_ALL (0) | POLESTAR_PROXY_ACTIVE */
} polestar_params;

typedef struct polestar_handle polestar_handle;

/* Per-layer device buffers.  Weights are packed (polestar_pack_weight). */
typedef struct polestar_layer {
  const void* w_qkv;    /* packed POLESTAR_W_QKV */
  const void* w_o;      /* packed POLESTAR_W_O */
  const void* w_gu;     /* packed POLESTAR_W_GU */
  const void* w_down;   /* packed POLESTAR_W_DOWN */
  void* k_cache;        /* [batch, n_pos, n_kv_heads, head_dim], in/out */
  void* v_cache;        /* [batch, n_kv_heads, head_dim, n_pos], in/out */
  void* win_h;          /* RAW: window rows [batch, win_max, d], in/out */
  uint8_t* win_codes;   /* residual formats: [batch, win_max, code bytes], in/out */
  uint8_t* win_scales;  /* residual formats: [batch, win_max, scale bytes] (FP8: unused), in/out */
  void* win_z;          /* centroids [batch, n_clusters, d], in/out */
  int32_t* win_m;       /* cluster labels [batch, win_max], in/out */
  float* proxy_logits;  /* previous proxy-attention logits [batch, K, n_heads, n_pos], in/out */
  float* q_win;         /* nullable (bf16 storage, raw window rows; ignored otherwise): the
                           window rows' queries [batch, win_max, n_heads * head_dim] f32 kept
                           across steps, in/out; a refresh-mode drift then projects only the
                           rows a packet patched (a raw row changes only there, and its query
                           depends on its stored value and W_Q alone) */
  int32_t* q_ok;        /* with q_win: [batch] i32, the block position the cached queries
                           belong to: a refresh-mode drift at blk_start sets blk_start + 1;
                           a refresh at any other blk_start, or q_ok[b] == 0, projects every
                           window row again; block entry (polestar_entry,
                           polestar_cluster(ENTRY)) sets 0.  A caller that writes win_h or the
                           packed w_qkv outside those calls (e.g. layer-0 window rows of newly
                           decoded tokens, new weights) must set q_ok to 0 first. */
} polestar_layer;

/* Update packet U(t,l): rows of selected window positions.  Row r of
 * sequence b holds window row idx[b*win_max + r]; count[b] rows are valid,
 * ascending.  count lives on the device and is never read by the host. */
typedef struct polestar_packet {
  void* rows;      /* [batch, win_max, d] storage dtype */
  int32_t* idx;    /* [batch, win_max] */
  int32_t* count;  /* [batch] */
} polestar_packet;

/* Optional float32 side outputs of values before their storage rounding,
 * for numerical checks.  Any pointer may be NULL.  Set with
 * polestar_set_check; they stay in effect until replaced. */
typedef struct polestar_check {
  float* qkv;      /* [batch, B + win_max + K, (Hq + 2 Hkv) dh] projections of the QKV rows */
  float* attn_out; /* [batch, B + win_max, Hq dh] attention outputs of token rows */
  float* hp;       /* [batch, B + win_max, d] h' = h + o W_O^T rows [active; S] */
  float* out;      /* [batch, B + win_max, d] layer outputs of rows [active; S] */
  float* kv_next;  /* [batch, win_max, 2 Hkv dh] next-layer K/V of packet rows */
} polestar_check;

/* ---- handle ------------------------------------------------------------ */
/* Validates dims/params (host only, no HIP call) and creates a handle.
 * Returns E_NULL, E_SHAPE, E_DTYPE or E_UNSUPPORTED on bad input, E_ARG on a bad scalar
 * parameter (eps < 0, hist outside 0..16, kmeans_iters outside 0..1000, mask_id, an unknown
 * proxy_support). */
int polestar_create(const polestar_dims* dims, const polestar_params* params, polestar_handle** out);
void polestar_destroy(polestar_handle* h);
const char* polestar_strerror(int code);
/* Bytes of device workspace every call needs. */
int polestar_workspace_size(const polestar_handle* h, size_t* bytes);
int polestar_set_check(polestar_handle* h, const polestar_check* chk /* NULL clears */);

/* ---- weights ----------------------------------------------------------- */
/* Bytes of a packed weight of the given kind. */
int polestar_weight_packed_size(const polestar_handle* h, int which, size_t* bytes);
/* Repack a weight from [out, in] row-major (storage dtype, device) into the
 * layout the projection kernels stream (device, caller-allocated). */
int polestar_pack_weight(const polestar_handle* h, int which, const void* src, void* dst, void* stream);

/* ---- the four refresh-path calls ---------------------------------------- */
/*
 * polestar_cluster — window clustering [§4.1 "Cluster and Quantize Hidden
 * States"; Algorithm 1: SphericalKMeans, ResidualQuantization at block entry,
 * Dequantize, Patch, ResidualQuantization inside the layer loop].
 *  ENTRY:  spherical k-means of the window rows entry_h ([batch, win_max, d],
 *          storage dtype; may alias L->win_h) with min(K, n_win) initial
 *          centroids at rows init_idx [batch, K] (i32, device), then
 *          kmeans_iters Lloyd iterations (assign by largest cosine, lowest
 *          index on ties; empty clusters keep their centroid).  Writes win_z,
 *          win_m, and win_h (RAW) or the residual codes (h - z_M(i)) in the
 *          handle's residual format.
 *          objective (nullable, device f64 [batch, 2*kmeans_iters]) receives
 *          the objective after every assignment and every update.
 *  UPDATE: per refresh step.  Rebuilds the window rows (RAW: win_h; other
 *          formats: z_M(i) + dequantised residual, stored as bf16), overwrites rows
 *          named by the packet u_in (nullable = no packet), recomputes every
 *          non-empty centroid from its members with the labels fixed (§4.1
 *          incremental centroid update), and re-quantises (residual formats).  The
 *          patched rows stay in the workspace for polestar_drift/refresh.
 */
int polestar_cluster(polestar_handle* h, int mode, const polestar_layer* L, int32_t blk_start,
                     const polestar_packet* u_in, const int32_t* init_idx, const void* entry_h,
                     double* objective, void* ws, size_t ws_bytes, void* stream);

/*
 * polestar_drift — main attention of the active block and drift scoring
 * [§2 Eq. 3; Eq. 4; §4.1 "Measuring Drift and Layer-wise KV Updates";
 * Algorithm 1 forward of the active block, ProxyAttn, KL, TopK, S = M[K]].
 *  REFRESH: projects [active rows h_active [batch, B, d]; window rows; the
 *    centroids] with W_Q/W_K/W_V (RMSNorm with unit gain), writes the active
 *    block's K/V and the K/V of the packet rows into the layer's cache (the
 *    window rows that the preceding polestar_cluster(UPDATE) on the same
 *    workspace patched from its packet; u_in itself is not read and may be
 *    NULL),
 *    runs softmax attention of the active and window rows over all n_pos
 *    keys, runs proxy attention of the centroid queries over the keys that
 *    params.proxy_support names (all positions, or the active block's),
 *    scores each cluster by D_c = sum over heads of max(0, KL(P_t || P_prev))
 *    against L->proxy_logits (then overwritten with P_t's logits), picks the
 *    top-k clusters (largest D, lowest index on ties) and writes the selected
 *    window rows S (ascending) to sel->idx / sel->count.  D [batch, K] and
 *    topk [batch, k] (-1 past min(k, n_win)) are nullable outputs.
 *  ACTIVE_ONLY: the active rows only (a step without a refresh, §4.1
 *    "Update Schedule"); sel->count is set to 0.
 *  act_logits (nullable, in/out [batch, B, Hq, n_pos]): the active block's
 *    main-attention logits of the previous step; when delta is non-NULL the
 *    per-row drift delta_j = sum_h max(0, KL(A_t || A_prev)) (f32 [batch, B])
 *    is written, then act_logits is overwritten with this step's logits
 *    (§4.2 "Current Block Commit"; Algorithm 1 main-attention drift of the
 *    last layer).
 */
int polestar_drift(polestar_handle* h, int mode, const polestar_layer* L, int32_t blk_start,
                   const void* h_active, const polestar_packet* u_in, float* D, int32_t* topk,
                   polestar_packet* sel, float* act_logits, float* delta,
                   void* ws, size_t ws_bytes, void* stream);

/*
 * polestar_refresh — gathered sparse layer forward producing the update
 * packet [§4.1: forward over the selected clusters' rows only, giving
 * U(t, l+1); Algorithm 1 sparse forward].  Rows are [active block; the
 * sel->count rows S]: h' = h + o W_O^T, out = h' + (silu(g) * u) W_down^T with
 * g, u the gate/up projections of RMSNorm(h').  Writes h_active_out
 * [batch, B, d] (the next layer's active input) and u_rows [batch, win_max, d]
 * (row r = output of window row sel->idx[r]).  When w_kv_next (packed
 * POLESTAR_W_KV of layer l+1) is given, the K/V rows of layer l+1 for S are
 * computed from the fresh U and scattered into k_next/v_next
 * (K and V caches of layer l+1, layouts as above).
 */
int polestar_refresh(polestar_handle* h, const polestar_layer* L, int32_t blk_start, const void* h_active,
                     const polestar_packet* sel, const void* w_kv_next, void* k_next, void* v_next,
                     void* h_active_out, void* u_rows, void* ws, size_t ws_bytes, void* stream);

/*
 * polestar_step — one denoising step over a stack of n_layers layers, the
 * composition of the per-layer calls above in one call [Algorithm 1 layer
 * loop; §4.1].  layers: host array [n_layers].  Layer l reads its active rows
 * from buffer l % 2 of (h_act0, h_act1) ([batch, B, d] storage dtype, device;
 * h_act0 holds layer 0's input) and writes them to the other; the output is in
 * buffer n_layers % 2.  mode POLESTAR_DRIFT_REFRESH: per layer,
 * polestar_cluster(UPDATE) with the previous layer's packet (none for layer
 * 0), polestar_drift(REFRESH) selecting into packet l % 2 of (pk0, pk1), and
 * polestar_refresh writing that packet's rows (its rows buffer
 * [batch, win_max, d]); POLESTAR_DRIFT_ACTIVE_ONLY: drift and refresh of the
 * active rows only.  D and topk (nullable) end with the last layer's values;
 * act_logits and delta (nullable) are used by the last layer as in
 * polestar_drift.  Every call is validated before the first launch (same
 * codes as the single calls); then the launches equal those of the single
 * calls issued in this order.
 */
int polestar_step(polestar_handle* h, int mode, int32_t n_layers, const polestar_layer* layers, int32_t blk_start,
                  void* h_act0, void* h_act1, polestar_packet* pk0, polestar_packet* pk1, float* D, int32_t* topk,
                  float* act_logits, float* delta, void* ws, size_t ws_bytes, void* stream);

/*
 * polestar_step_noalloc — polestar_step for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same arguments without the workspace, same validation, same launches and results.
 * The workspace is the library's own static device array of POLESTAR_SCRATCH_BYTES
 * (192 MiB) per GPU, held until the process ends; its address is looked up once per device
 * (the device current at the first call) and no call allocates or frees device memory.
 * Returns POLESTAR_E_SCRATCH, before any HIP call, when the handle's workspace
 * (polestar_workspace_size) is larger.  Every call on one GPU uses the same array, which
 * keeps the last call's contents (no step reads workspace it has not written first, so
 * nothing is cleared); calls that overlap on one GPU (other streams, other threads) race
 * and must be serialised by the caller.  Per-kernel profiling events are not recorded.
 */
#define POLESTAR_SCRATCH_BYTES (192u << 20)
int polestar_step_noalloc(polestar_handle* h, int mode, int32_t n_layers, const polestar_layer* layers,
                          int32_t blk_start, void* h_act0, void* h_act1, polestar_packet* pk0, polestar_packet* pk1,
                          float* D, int32_t* topk, float* act_logits, float* delta, void* stream);

/*
 * polestar_entry — block-entry state of one layer [§4.1 "Update Schedule"
 * (a whole-sequence forward at every other block entry) and "Cluster and
 * Quantize Hidden States"; Algorithm 1 block entry].
 *  mode POLESTAR_ENTRY_FULL recomputes every position; POLESTAR_ENTRY_WINDOW
 *  the window and the active block, positions [blk_start - win_prefix,
 *  blk_start + B + win_suffix) cut at 0 and n_pos.  For those rows of
 *  h_in [batch, n_pos, d] (storage dtype, device): their K/V (RMSNorm with unit
 *  gain, W_K/W_V) replace the layer's cache rows; then each row attends to all
 *  n_pos cache positions and the layer's residual, RMSNorm and SwiGLU steps
 *  give its row of h_out [batch, n_pos, d] (the next layer's input).  Rows of
 *  h_out outside the set, and cache rows outside it, are left as they are.
 *  h_out must not overlap h_in (POLESTAR_E_ARG).
 *  Then, as polestar_cluster(ENTRY) but on the window rows of h_in (read at
 *  their positions): k-means from init_idx [batch, K], storing win_z, win_m and
 *  the window rows or their residual codes; objective as there (nullable).
 *  act_logits (nullable, f32 [batch, B, Hq, n_pos], device): receives the
 *  active block's main-attention logits over the fresh cache, the reference
 *  of the first commit drift delta (pass it for the last layer; §4.2
 *  "Current Block Commit").  Last, the proxy logits of the new centroids over
 *  the fresh cache are written to L->proxy_logits: the reference of the
 *  first drift score (over the keys params.proxy_support names).  Needs every
 *  weight, cache and window pointer of L.
 */
int polestar_entry(polestar_handle* h, int mode, const polestar_layer* L, int32_t blk_start, const void* h_in,
                   const int32_t* init_idx, void* h_out, double* objective, float* act_logits, void* ws,
                   size_t ws_bytes, void* stream);

/*
 * polestar_commit — Polestar-Commit [§4.2 "Current Block Commit" and
 * "Suffix Block Commit"; Table 5: tau_s, h, alpha, suffix confidence].
 *  Confidence c = max over ids != mask_id of softmax(RMSNorm(x) W_lm^T),
 *  yhat its argmax, for the active rows x = h_final [batch, B, d] and for the
 *  suffix packet rows (u_final rows whose sel_final window row is in the
 *  suffix window).  Current block: with the history hist_vals
 *  [batch, B, max(hist,1)] f32 / hist_cnt [batch, B] i32 (in/out; reset to 0
 *  at block entry), spike = delta - mean(history) (0 mean when empty), then
 *  delta is pushed; tau_d = alpha (tau_s - c)^2; commit when masked and
 *  (c >= tau_s or spike > tau_d).  Suffix: commit when the row is in S,
 *  masked (suffix_masked [batch, win_suffix] u8) and c >= tau_suf.
 *  Outputs: commit_active [batch, B] u8, commit_suffix [batch, win_suffix] u8,
 *  conf_active / spike [batch, B] f32, yhat_active [batch, B] i32,
 *  conf_suffix [batch, win_suffix] f32 (0 where not a packet row).
 *  delta comes from polestar_drift of the last layer.  W_lm is packed
 *  POLESTAR_W_LM.  active_masked [batch, B] u8.
 */
int polestar_commit(polestar_handle* h, int32_t blk_start, const void* w_lm, const void* h_final,
                    const polestar_packet* u_final, const float* delta, const uint8_t* active_masked,
                    const uint8_t* suffix_masked, float* hist_vals, int32_t* hist_cnt,
                    uint8_t* commit_active, uint8_t* commit_suffix, float* conf_active,
                    int32_t* yhat_active, float* spike, float* conf_suffix,
                    void* ws, size_t ws_bytes, void* stream);

/*
 * polestar_entry_commit — the commit at block entry [§4.2 "Current Block
 * Commit" and "Suffix Block Commit"; Algorithm 1 block entry].  After the
 * entry forward there is no drift yet, so the confidence alone decides:
 * active row j commits when masked and c >= tau_s; suffix window row i
 * (positions blk_start + B + i, all of them fresh from the forward) commits
 * when masked and c >= tau_suf.  Confidences as in polestar_commit, read from
 * the last layer's output h_full [batch, n_pos, d] (storage dtype, device) at
 * those positions.  Drift history and spikes are not touched.  Outputs:
 * commit_active [batch, B] u8, conf_active [batch, B] f32, yhat_active
 * [batch, B] i32, commit_suffix / conf_suffix [batch, win_suffix] (0 past the
 * sequence end).  Masks as in polestar_commit.  Needs a vocabulary
 * (POLESTAR_E_SHAPE otherwise).
 */
int polestar_entry_commit(polestar_handle* h, int32_t blk_start, const void* w_lm, const void* h_full,
                          const uint8_t* active_masked, const uint8_t* suffix_masked, uint8_t* commit_active,
                          uint8_t* commit_suffix, float* conf_active, int32_t* yhat_active, float* conf_suffix,
                          void* ws, size_t ws_bytes, void* stream);

/* ---- per-kernel timing (diagnostics) ------------------------------------ */
enum {
  POLESTAR_K_CLUSTER = 0, POLESTAR_K_PREP, POLESTAR_K_QKV, POLESTAR_K_ATTN, POLESTAR_K_TOPK,
  POLESTAR_K_OPROJ, POLESTAR_K_OREDUCE, POLESTAR_K_GU, POLESTAR_K_DOWN, POLESTAR_K_DREDUCE,
  POLESTAR_K_KVNEXT, POLESTAR_K_LMPREP, POLESTAR_K_LMHEAD, POLESTAR_K_DECIDE, POLESTAR_K_KL, POLESTAR_K_COUNT
};
/* enable != 0: from now on every kernel this handle enqueues is bracketed by
 * a pair of hipEvents on its stream (events recorded during stream capture
 * become graph nodes and are re-recorded by every replay); enable == 0 stops.
 * Either way the previous records are dropped.  Host-side only; no device
 * memory is allocated. */
int polestar_profile(polestar_handle* h, int enable);
/* Waits for the recorded events and returns, per kernel kind (POLESTAR_K_*),
 * the summed duration in ms (total_ms[POLESTAR_K_COUNT]) and the number of
 * launches (launches[POLESTAR_K_COUNT]) of the recorded launches; the records
 * stay (a graph replay re-records them).  E_HIP if an event query fails. */
int polestar_profile_read(polestar_handle* h, double* total_ms, int32_t* launches);

/* ---- update schedule (host) --------------------------------------------- */
/* 1 when the tokens decoded since the last refresh exceed tau_upd (a refresh
 * step), else 0; tau_upd < 0 means never [§4.1 "Update Schedule"]. */
int polestar_should_refresh(int32_t decoded_since_refresh, int32_t tau_upd);

/* ---- NVFP4 codec [App. C.3] ---------------------------------------------- */
/* Quantise float32 rows x [rows, d] (device) to codes [rows, d/2] and scales
 * [rows, d/16]: per 16 channels s = amax/6, scale = E4M3(s) (round to
 * nearest even, saturating at 448), code = E2M1(x / scale) (nearest even,
 * saturating at 6; 0 when the scale is 0). */
int polestar_nvfp4_pack(const float* x, int64_t rows, int32_t d, uint8_t* codes, uint8_t* scales, void* stream);
/* Exact dequantisation scale * value(code) into float32 x [rows, d]. */
int polestar_nvfp4_unpack(const uint8_t* codes, const uint8_t* scales, int64_t rows, int32_t d, float* x,
                          void* stream);
/* Host evaluation of the same encoders (host pointers), for checks without a GPU. */
int polestar_nvfp4_pack_host(const float* x, int64_t rows, int32_t d, uint8_t* codes, uint8_t* scales);

/* ---- KV-cache staleness [App. C.2; §3 Fig. 3(a), Fig. 6(a)] ---------------- */
/* Measurement of what the refresh is for: for every position i of every
 * sequence, E_i = 1 - (mean_h cos(K_i,h, Kref_i,h) + mean_h cos(V_i,h, Vref_i,h))/2
 * over the KV heads h, written to stale [batch, n_pos] (f32, device).  k_cache,
 * v_cache are a layer's caches and k_ref, v_ref recomputed rows in the same
 * layouts and storage dtype (device).  A zero row has cosine 0 with any row.
 * float32 accumulation. */
int polestar_kv_staleness(const polestar_handle* h, const void* k_cache, const void* v_cache, const void* k_ref,
                          const void* v_ref, float* stale, void* stream);

/* The most-attended-token cosine policy that the drift ablation of §5 ("Drift Measurement
 * Policy", Fig. 6(a)) compares the KL drift with: for each query row r of each sequence (a
 * candidate window position), its most-attended token j*(r), the position whose attention
 * probability averaged over the query heads is largest when q_r attends over every position
 * of k_cache (softmax(q.k/sqrt(dh)) per head; the lowest position on ties), and the cosine
 * change of that token's keys, score = 1 - mean over KV heads of cos(k_cache[j*], k_ref[j*])
 * (a zero row has cosine 0).  Positions are ranked for refresh by score.
 * q: float32 [batch] x [rows] x [Hq dh] (element (b, r, c) at q[b q_bstride + r q_ld + c],
 * device); k_cache, k_ref: K caches [batch, n_pos, Hkv, dh] in the storage dtype (device);
 * top_pos: int32 [batch, rows] (device), score: float32 [batch, rows] (device).  float32
 * arithmetic.  E_NULL, E_SHAPE (q_ld < Hq dh, q_bstride too small); measurement only. */
int polestar_attended_change(const polestar_handle* h, const float* q, int32_t rows, int32_t q_ld,
                             int64_t q_bstride, const void* k_cache, const void* k_ref, int32_t* top_pos,
                             float* score, void* stream);

/* ---- residual formats [App. C.3; Table 11 ablation] ------------------------ */
/* Bytes per row of d values of format fmt: codes and scales (0 for RAW; FP8 has
 * no scales).  E_DTYPE for an unknown format, E_SHAPE when d is not a positive
 * multiple of 32. */
int polestar_resid_bytes(int32_t fmt, int32_t d, int64_t* code_bytes, int64_t* scale_bytes);
/* Quantise float32 rows x [rows, d] (device) in format fmt (not RAW) to codes
 * and scales laid out as polestar_resid_bytes gives:
 *   NVFP4  as polestar_nvfp4_pack;
 *   FP8    code = sign | E4M3FN(|x|) (nearest even, saturating at 448; zero +0);
 *   MXINT8 per 32 values X = 2^e, e = floor(log2 amax) (clamped to [-127, 127],
 *          -127 for zeros), byte e + 127; q = clamp(rne(x / X * 64), -128, 127);
 *   MXFP4  per 32 values X = 2^e, e = floor(log2 amax) - 2 (clamped likewise);
 *          code = E2M1(x / X) (nearest even, saturating at 6). */
int polestar_resid_pack(int32_t fmt, const float* x, int64_t rows, int32_t d, uint8_t* codes, uint8_t* scales,
                        void* stream);
/* Exact dequantisation of the same formats into float32 x [rows, d]. */
int polestar_resid_unpack(int32_t fmt, const uint8_t* codes, const uint8_t* scales, int64_t rows, int32_t d,
                          float* x, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* POLESTAR_H */
