/*
 * eta.h -- C ABI of the Elastic Threshold Attention (ETA) block-sparse decode
 * step for AMD Instinct MI355X (gfx950).
 *
 * Method: arXiv:2609.20888, "Elastic Threshold Attention: Learned Contextual
 * Sparsity for Long-Context Decoding". One decode step, per (batch, head) unit:
 *   1. predict a threshold tau from the post-RoPE query (review "Methodology
 *      Assessment", Eq. 1), or use frozen per-head constants (abstract: offline
 *      calibration);
 *   2. screen every 64-token KV block in O(1) against tau with a bound built
 *      from cached per-block metadata (abstract: a bound with a geometric
 *      and a probabilistic part; review "Summary": centroid / variance /
 *      max-norm);
 *   3. skip every block whose bound is below tau (review Q&A "What is ETA?");
 *   4. softmax attention over the admitted blocks' tokens, each logit S
 *      multiplied by the gate sigmoid(beta*(S - tau)) (Eq. 2 and Eq. 3), so a
 *      sub-threshold logit tends to 0, not to -inf.
 *
 * Conventions shared by every call
 *   - All tensors are device pointers in HBM, row-major, densely packed, owned
 *     and allocated by the caller. The library never allocates, frees or
 *     synchronises; a call validates its arguments on the host and then only
 *     enqueues kernels on `stream` (0 = the null stream).
 *   - Argument errors are returned before anything is enqueued. A failed
 *     launch returns ETA_ERR_HIP. No C++ exception crosses this boundary.
 *   - The library holds no global mutable state; calls on different streams
 *     with disjoint outputs may run concurrently.
 *   - Heads: H query heads; H_kv key/value heads (H_kv = 0 means H_kv = H,
 *     multi-head attention). With grouped heads, query head h reads key/value
 *     head h / G, G = H / H_kv.
 *   - Layouts (query unit u = b*H + h, key/value unit k = b*H_kv + h/G):
 *       q         float32 [B][H][d]        post-RoPE query (RoPE is the caller's)
 *       K, V      [B][H_kv][T_cap][d]      float32 or bfloat16 (kv_dtype);
 *                 with kv_block_stride, blocks of 64 rows kv_block_stride
 *                 elements apart (e.g. K and V interleaved block by block;
 *                 the same holds for the blocks of a page pool)
 *       tau       float32 [B][H]
 *       centroid  float32 [B][H_kv][d][nblk_cap]   dimension-major per unit
 *       var       float32 [B][H_kv][nblk_cap]
 *       maxnorm   float32 [B][H_kv][nblk_cap]
 *       adm_idx   int32   [B][H][nblk_cap]  per query head (eta_screen)
 *       adm_cnt   int32   [B][H]
 *       uni_idx   int32   [B][H_kv][nblk_cap]  per key/value head (eta_admit_union)
 *       uni_cnt   int32   [B][H_kv]
 *       out       float32 [B][H][d],  lse float32 [B][H]
 *     where nblk_cap = eta_nblk_cap(T_cap) = ceil(T_cap/64) rounded up to a
 *     multiple of 4. K and V (or their pools) start on a 16-byte boundary;
 *     bfloat16 with d = 64 needs only 8 bytes, except for K under grouped
 *     heads in the attention calls. Every other array starts on a 4-byte
 *     boundary at least (the attention calls check q, tau, adm_idx and
 *     adm_cnt: they are read with scalar loads where the index is the same
 *     across a wave).
 *   - Block beta of a unit covers tokens [64*beta, min(T_b, 64*beta + 64)) of
 *     its row b (T_b = seq_lens[b], or T); the last block may be partial.
 *     Tokens at or beyond T_b are never read. Block metadata, admitted lists
 *     and bounds are indexed by logical block in every layout; with a page
 *     table only the K/V bytes move: block beta of (b, k) is the 64 x d run
 *     K[page_table[b][beta]][k] of the pool.
 *   - eta_append_meta with seq_lens: the lengths are the ones BEFORE the
 *     append, and every row receives the same n_new tokens.
 */
#ifndef ETA_H
#define ETA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ETA_OK = 0,
    ETA_ERR_INVALID_ARG = -1, /* null pointer, bad size, misaligned buffer */
    ETA_ERR_UNSUPPORTED = -2, /* d not in {64, 128}, block != 64, bad dtype */
    ETA_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required */
    ETA_ERR_HIP = -4,         /* a kernel launch failed */
    /* range guard (never returned): every int is a valid eta_status, so the
       library reads whatever value a caller passes without undefined behaviour */
    ETA_STATUS_MAX_ENUM = 0x7fffffff
} eta_status;

typedef enum { ETA_F32 = 0, ETA_BF16 = 1, ETA_DTYPE_MAX_ENUM = 0x7fffffff } eta_dtype;

/* Bound used by the screen (see eta_screen). */
typedef enum {
    ETA_BOUND_COMBINED = 0,
    ETA_BOUND_GEO = 1,
    ETA_BOUND_CENTERED = 2,  /* needs eta_meta.maxdev2                          */
    ETA_BOUND_MAX_ENUM = 0x7fffffff
} eta_bound_mode;

typedef struct {
    int B, H;           /* batch rows and heads (MHA)                          */
    int d;              /* head dimension: 64 or 128                           */
    int T;              /* tokens present in the cache (0 <= T <= T_cap)       */
    int T_cap;          /* token capacity of the K/V layout: a positive
                           multiple of 64 (whole blocks)                       */
    int block;          /* tokens per KV block: must be 64                     */
    eta_dtype kv_dtype; /* element type of K and V                             */
    int H_kv;           /* key/value heads: 0 or H = multi-head; a divisor of H
                           with H / H_kv in {1, 2, 4, 8} = grouped heads       */
    /* Optional layout of a paged / variable-length cache (all zero: the dense
       layout K, V [B][H_kv][T_cap][d], every row holding T tokens).          */
    const int32_t *seq_lens;   /* device int32 [B]: tokens present in row b
                                  (each <= T; T is then the largest); null:
                                  every row holds T                          */
    const int32_t *page_table; /* device int32 [B][T_cap/64]: physical page of
                                  logical block j of row b; null: dense layout.
                                  With pages, K and V are pools
                                  [num_pages][H_kv][64][d] and every page id
                                  of a present block must be < num_pages (a
                                  block whose page id is out of range is
                                  skipped). Page p of K is read at
                                  K + p*H_kv*64*d and of V at the same offset
                                  from V, so one allocation may hold both
                                  pools with their pages interleaved: V = K +
                                  H_kv*64*d, even page ids only, num_pages
                                  counting both                              */
    int num_pages;             /* pages in the K/V pools (page_table only)   */
    int kv_block_stride;       /* elements from one 64-row block of K (or V)
                                  to the next: dense, block j of unit u starts
                                  at (u*T_cap/64 + j)*kv_block_stride; paged,
                                  the block of head k in page p at
                                  (p*H_kv + k)*kv_block_stride. 0 means 64*d
                                  (blocks back to back); otherwise a positive
                                  multiple of 64*d. 128*d with V = K + 64*d
                                  keeps K and V interleaved block by block in
                                  one allocation, which streams at the same
                                  rate wherever the driver places it (two
                                  separate K and V allocations read together
                                  stream faster or slower by several percent
                                  depending on their relative placement).    */
} eta_shape;

typedef struct {
    float *centroid;    /* [B][H][d][nblk_cap]                                 */
    float *var;         /* [B][H][nblk_cap]                                    */
    float *maxnorm;     /* [B][H][nblk_cap]                                    */
    int nblk_cap;       /* must equal eta_nblk_cap(T_cap); the pointers are
                           16-byte aligned                                     */
    float *maxdev2;     /* [B][H][nblk_cap] or NULL: the largest squared
                           distance of a block's keys from its centroid,
                           written by the build and append when not NULL and
                           read by ETA_BOUND_CENTERED                         */
} eta_meta;

typedef struct {
    float gate_beta;    /* gate sharpness beta of Eq. 2 (> 0); default 5       */
    float z;            /* standard deviations in the probabilistic bound
                           (>= 0, finite); default 4                           */
    int gate_hard;      /* 1: gate is the step S >= tau instead of the sigmoid */
    int bound_mode;     /* eta_bound_mode; default ETA_BOUND_COMBINED          */
    int split_blocks;   /* admitted blocks per split-KV work item (1..4096);
                           0 = library default, 8 per query head of a
                           key/value unit (8 * G), doubled when
                           B * H_kv * nblk_cap >= 2^20; see eta_split_blocks */
} eta_params;

/* Defaults: beta = 5 (the end of the 1 -> 5 anneal of Eq. 2), z = 4, soft
 * gate, combined bound, split_blocks = 0. */
eta_params eta_default_params(void);

/* Per-unit block capacity of the metadata, admitted-list and bound arrays for
 * a cache of T_cap tokens: ceil(T_cap / 64) rounded up to a multiple of 4
 * (0 if T_cap < 1). */
int eta_nblk_cap(int T_cap);

/* The split-KV item length the attention calls use for this shape and these
 * parameters: p->split_blocks if nonzero, else the default (8 * G, twice that
 * for caches of at least 2^20 unit blocks). Returns 0 if
 * s or p is null, the shape is invalid or unsupported, or p->split_blocks is
 * out of range. Host-only, no GPU work. */
int eta_split_blocks(const eta_shape *s, const eta_params *p);

/* Human-readable name of a status code (static storage). */
const char *eta_status_string(eta_status st);

/*
 * Block metadata builder (review "Summary": cached centroid / variance /
 * max-norm; abstract: cached bounds). For every unit and every block of the
 * first s->T tokens: centroid = mean key; var = mean over the block's tokens
 * and the d dimensions of (k - centroid)^2 (population); maxnorm = largest key
 * L2 norm. fp32 accumulation. Reads K once; writes blocks [0, ceil(T/64)) of
 * m. Errors: ETA_ERR_INVALID_ARG (null pointer, bad shape or meta),
 * ETA_ERR_UNSUPPORTED, ETA_ERR_HIP.
 */
eta_status eta_build_block_meta(const eta_shape *s, const void *K, const eta_meta *m,
                                hipStream_t stream);

/*
 * Incremental metadata update after new tokens (same definition as above).
 * s->T is the token count BEFORE the append; the caller has already written K
 * for tokens [s->T, s->T + n_new). Recomputes only the blocks touched by those
 * tokens, with the same per-block code as eta_build_block_meta, so the result
 * is bitwise equal to a rebuild at T + n_new. Requires n_new >= 1 and
 * s->T + n_new <= s->T_cap. Errors as eta_build_block_meta.
 */
eta_status eta_append_meta(const eta_shape *s, int n_new, const void *K, const eta_meta *m,
                           hipStream_t stream);

/*
 * Threshold predictor (review "Methodology Assessment", Eq. 1):
 *   tau[b][h] = bias[h] + sum_{g<H, i<d} q[b][g][i] * W[g*d + i][h]
 * on the concatenated post-RoPE queries of one batch row. W is float32
 * [H*d][H]; W == NULL selects frozen per-head thresholds tau[b][h] = bias[h]
 * (abstract: offline calibration removes the predictor). fp32 accumulation in
 * a fixed order. Errors: ETA_ERR_INVALID_ARG, ETA_ERR_HIP.
 */
eta_status eta_predict_tau(int B, int H, int d, const float *q, const float *W,
                           const float *bias, float *tau, hipStream_t stream);

/*
 * Constant-time block screen (abstract: a cached bound with a geometric and a
 * probabilistic part; review Q&A "What is ETA?": a block none of whose keys
 * can reach tau is skipped). With s = 1/sqrt(d), per block:
 *   U_geo  = s * |q| * maxnorm                        (Cauchy-Schwarz)
 *   U_prob = s * (q . centroid + z * |q| * sqrt(var)) (centroid + z std devs)
 *   U_cen  = s * (q . centroid + |q| * sqrt(maxdev2)) (Cauchy-Schwarz about
 *                                                      the centroid)
 *   U = min(U_geo, U_prob)  (ETA_BOUND_COMBINED),  U_geo (ETA_BOUND_GEO), or
 *   min(U_geo, U_cen) (ETA_BOUND_CENTERED: like U_geo it never skips a block
 *   holding a key that reaches tau; z is not used; m->maxdev2 must be set).
 * Block beta < ceil(T/64) is admitted iff U >= tau[b][h] (a NaN tau admits
 * nothing). Writes the admitted ids in ascending order to adm_idx[u][0..cnt)
 * and cnt to adm_cnt[u]; entries past cnt are left untouched. bound_out
 * (nullable, float32 [B][H][nblk_cap]) receives U, with -inf for blocks at or
 * beyond ceil(T/64). Deterministic: no atomics. Errors: ETA_ERR_INVALID_ARG,
 * ETA_ERR_UNSUPPORTED, ETA_ERR_HIP.
 */
eta_status eta_screen(const eta_shape *s, const float *q, const float *tau, const eta_meta *m,
                      const eta_params *p, int32_t *adm_idx, int32_t *adm_cnt,
                      float *bound_out, hipStream_t stream);

/*
 * Threshold predictor and screen in one launch: for every unit, tau[b][h] is
 * evaluated as in eta_predict_tau (W nullable: frozen tau = bias) and stored to
 * tau (float32 [B][H], read later by eta_decode_attn), then the unit is
 * screened as in eta_screen. Same layouts, outputs and errors as the two calls
 * it replaces; tau may differ from eta_predict_tau's in the last bits (another
 * fp32 summation order).
 */
eta_status eta_predict_screen(const eta_shape *s, const float *q, const float *W,
                              const float *bias, const eta_meta *m, const eta_params *p,
                              float *tau, int32_t *adm_idx, int32_t *adm_cnt, float *bound_out,
                              hipStream_t stream);

/*
 * Grouped heads: union, per key/value head, of the admitted lists of its G
 * query heads (the pages measure the fraction of blocks fetched this way;
 * abstract: the gate's floor makes tokens that only ride along with a selected
 * block harmless). uni_idx[k] = ascending union of adm_idx[k*G + j][0..cnt)
 * over j < G, uni_cnt[k] its length. Deterministic. With G = 1 it copies the
 * lists. The input lists must be ascending (as eta_screen writes them); ids
 * outside [0, ceil(T/64)) are dropped and counts are clamped to [0, nblk_cap].
 * Errors: ETA_ERR_INVALID_ARG, ETA_ERR_UNSUPPORTED, ETA_ERR_HIP.
 */
eta_status eta_admit_union(const eta_shape *s, const int32_t *adm_idx, const int32_t *adm_cnt,
                           int32_t *uni_idx, int32_t *uni_cnt, hipStream_t stream);

/*
 * eta_predict_screen followed by eta_admit_union, in one launch: with grouped
 * heads one workgroup screens the G query heads of a key/value unit together,
 * so the union of their lists is formed from the same admission bits and
 * written beside them. Outputs and errors as the two calls it replaces (tau,
 * adm_idx, adm_cnt and bound_out as eta_predict_screen; uni_idx, uni_cnt as
 * eta_admit_union, [B][H_kv][nblk_cap] and [B][H_kv]). Requires grouped heads
 * (H_kv < H): with multi-head attention the lists are already per key/value
 * unit and the call returns ETA_ERR_INVALID_ARG.
 */
eta_status eta_predict_screen_union(const eta_shape *s, const float *q, const float *W,
                                    const float *bias, const eta_meta *m, const eta_params *p,
                                    float *tau, int32_t *adm_idx, int32_t *adm_cnt,
                                    int32_t *uni_idx, int32_t *uni_cnt, float *bound_out,
                                    hipStream_t stream);

/* Bytes of device workspace the attention calls need for this shape and split
 * size (0 on invalid arguments). The layout is private to the library. */
size_t eta_decode_attn_workspace_size(const eta_shape *s, const eta_params *p);

/*
 * Block-sparse split-KV decode attention with the ETA gate (Eq. 2 and Eq. 3;
 * abstract: a logit under the threshold is multiplied down to zero). adm_idx / adm_cnt
 * are lists per key/value unit ([B][H_kv][nblk_cap], [B][H_kv]): the
 * eta_screen lists for multi-head attention, the eta_admit_union lists for
 * grouped heads. Every query head h of key/value unit k attends, with its own
 * q and tau, over the tokens (< T) of the blocks adm_idx[k][0..adm_cnt[k]):
 *   S = s * q.k,  S' = S * sigmoid(gate_beta * (S - tau))  (or S * [S >= tau]),
 *   out = softmax(S') . V,  lse = log of the softmax denominator.
 * The admitted list is cut into work items of split_blocks blocks. This call
 * is eta_decode_attn_partial followed by eta_decode_attn_combine on the same
 * stream. A unit with adm_cnt == 0 gets out = 0 and lse = -inf. lse is
 * nullable. adm_idx entries are the unit's admitted block ids (eta_screen and
 * eta_admit_union write them ascending); an entry that is not a block of the
 * unit's row (negative, or >= ceil(T_b/64)) is skipped, and a count outside
 * [0, T_cap/64] is clamped to it, so no read or write leaves the buffers.
 * ws: device workspace of at least eta_decode_attn_workspace_size() bytes,
 * 256-byte aligned; it needs no initialisation and is clobbered. Calls that
 * share a workspace must not overlap in time. Deterministic for a fixed
 * split size; results for different split sizes agree to fp32 rounding.
 * Errors: ETA_ERR_INVALID_ARG, ETA_ERR_UNSUPPORTED, ETA_ERR_WORKSPACE,
 * ETA_ERR_HIP.
 */
eta_status eta_decode_attn(const eta_shape *s, const float *q, const void *K, const void *V,
                           const float *tau, const int32_t *adm_idx, const int32_t *adm_cnt,
                           const eta_params *p, float *out, float *lse, void *ws,
                           size_t ws_bytes, hipStream_t stream);

/*
 * First phase of eta_decode_attn: every work item's online-softmax partial
 * (running max, sum of weights, weighted sum of V) over its blocks. Units
 * whose list fits one work item (or is empty) receive their final out / lse
 * here; the others' partials go to ws for eta_decode_attn_combine. Same
 * arguments, conventions and errors as eta_decode_attn.
 */
eta_status eta_decode_attn_partial(const eta_shape *s, const float *q, const void *K,
                                   const void *V, const float *tau, const int32_t *adm_idx,
                                   const int32_t *adm_cnt, const eta_params *p, float *out,
                                   float *lse, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Second phase of eta_decode_attn: for every unit with more than one work
 * item, merges the partials left in ws by eta_decode_attn_partial (same
 * shape, parameters and adm_cnt) with a log-sum-exp combine in item order:
 * M = max_i m_i, l = sum_i l_i e^(m_i - M), out = sum_i o_i e^(m_i - M) / l,
 * lse = M + log(l). Must follow the partial call on the same stream.
 * Errors: ETA_ERR_INVALID_ARG, ETA_ERR_UNSUPPORTED, ETA_ERR_WORKSPACE,
 * ETA_ERR_HIP.
 */
eta_status eta_decode_attn_combine(const eta_shape *s, const int32_t *adm_cnt,
                                   const eta_params *p, float *out, float *lse, void *ws,
                                   size_t ws_bytes, hipStream_t stream);

/* Largest workspace eta_decode_attn_noalloc can provide (128 MiB per GPU). At
 * the default split and d = 128 that covers caches of up to about 2^27.9
 * tokens in all (B * H * T_cap), e.g. B = 64, H = 16, T_cap = 128K. */
#define ETA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

/*
 * eta_decode_attn for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc. Same
 * arguments, semantics and results as eta_decode_attn (same kernels, same
 * split), but the workspace is a library-owned device array of
 * ETA_NOALLOC_SCRATCH_BYTES, one per GPU, held until the process ends. The
 * call allocates and frees nothing and needs no memset: every byte of the
 * array that a call reads it has first written itself. The kernels run on the
 * current device's copy of the array, so `stream` must belong to the current
 * device (checked when non-null). The first call on a device looks up that
 * device's address of the array (a host-side query, no launch); later calls
 * reuse it.
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents: calls that overlap in time on one GPU (on different streams, or
 * from different host threads) race and must be serialised by the caller.
 * Errors: as eta_decode_attn; ETA_ERR_WORKSPACE when the shape and split need
 * more than ETA_NOALLOC_SCRATCH_BYTES (eta_decode_attn_workspace_size tells);
 * ETA_ERR_INVALID_ARG for a stream of another device; ETA_ERR_HIP when the
 * device or the array's address cannot be queried, or a launch fails.
 */
eta_status eta_decode_attn_noalloc(const eta_shape *s, const float *q, const void *K,
                                   const void *V, const float *tau, const int32_t *adm_idx,
                                   const int32_t *adm_cnt, const eta_params *p, float *out,
                                   float *lse, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Training-time (prefill) forward
 *
 * The gate the model is trained with, applied densely: for every query token t
 * of a sequence and every key j at or before it, S = q_t . k_j / sqrt(d) and
 * the logit entering the softmax is S * sigmoid(beta * (S - tau_t)) (review
 * "Methodology Assessment", Eq. 2 and Eq. 3; abstract: in training a logit
 * under the threshold is multiplied down to zero instead of being masked
 * out), tau_t from
 * Eq. 1 on token t's concatenated queries. Causal: the T_q queries are the
 * last T_q positions of the T_k keys (T_q = T_k: a whole sequence; T_q < T_k:
 * a chunk continuing a cached prefix).
 *
 * Layouts (bfloat16 unless stated):
 *   Q     [B][H][T_q][d]         post-RoPE queries
 *   K, V  [B][H_kv][T_k][d]      (H_kv = 0 means H; query head h reads h / G)
 *   tau   float32 [B][H][T_q]
 *   out   float32 [B][H][T_q][d];  lse, gate_sum float32 [B][H][T_q]
 * d is 64 or 128; Q, K, V and out must be 16-byte aligned.
 * ------------------------------------------------------------------------ */
typedef struct {
    int B, H;      /* batch rows, query heads                                */
    int H_kv;      /* key/value heads: 0 or H, or a divisor with H/H_kv in
                      {1, 2, 4, 8}                                           */
    int d;         /* head dimension: 64 or 128                              */
    int T_q, T_k;  /* queries and keys per row; 0 <= T_q <= T_k; at most
                      65535 * 128 queries; T_k * d * 2 < 2^31 (one row's K
                      or V of one head under 2 GiB)                          */
} eta_prefill_shape;

/*
 * Eq. 1 for every query token: tau[b][h][t] = bias[h] + sum over heads g and
 * dimensions i of Q[b][g][t][i] * W[g*d + i][h], accumulated in float32 in a
 * fixed order (the bfloat16 queries are widened exactly). W: float32
 * [H*d][H] or NULL (frozen per-head thresholds: tau = bias). Only T_q and the
 * head counts of `s` are used (T_k is ignored).
 * Errors: ETA_ERR_INVALID_ARG (null pointer, bad shape, misaligned Q),
 * ETA_ERR_UNSUPPORTED (d not 64 or 128), ETA_ERR_HIP.
 */
eta_status eta_prefill_predict_tau(const eta_prefill_shape *s, const void *Q, const float *W,
                                   const float *bias, float *tau, hipStream_t stream);

/*
 * Dense causal gated attention. Per query t: softmax over its visible keys of
 * the gated logits, out = the weighted sum of V, lse = log of the softmax
 * denominator (natural log, gated-logit units), gate_sum = the sum of the
 * gates sigmoid(beta * (S - tau_t)) over the visible keys (the statistic a
 * mean-inclusion regulariser is built from; with gate_hard the number of
 * visible keys with S >= tau_t). lse and gate_sum may be NULL. Uses
 * p->gate_beta and p->gate_hard (z, bound_mode and split_blocks are ignored).
 * Precision: q.k in bfloat16 products with float32 accumulation; the softmax
 * weights and V enter the weighted sum as float16 (V must lie within
 * +-65504; magnitudes below 2^-14 keep fewer significant bits), accumulated
 * in float32.
 * Errors: ETA_ERR_INVALID_ARG, ETA_ERR_UNSUPPORTED, ETA_ERR_HIP.
 */
eta_status eta_prefill_attn(const eta_prefill_shape *s, const void *Q, const void *K,
                            const void *V, const float *tau, const eta_params *p, float *out,
                            float *lse, float *gate_sum, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* ETA_H */
