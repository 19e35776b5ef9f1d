/*
 * hstu.h -- C ABI of libhstu.so: HSTU pointwise aggregated attention on
 * AMD Instinct MI355X (gfx950).
 *
 * Source of the method: the paper review page "Actions Speak Louder than
 * Words: Trillion-Parameter Sequential Transducers for Generative
 * Recommendations" (arXiv 2402.17152), written [GR review] below.  Its
 * section 3 (core formulas) gives the HSTU layer:
 *   Eq. 1  U, V, Q, K = Split(phi1(f1(X))),  f_i(X) = W_i X + b_i
 *   Eq. 2  A(X)V(X)   = phi2(Q K^T + rab^{p,t}) V(X)
 *   Eq. 3  Y(X)       = f2(Norm(A(X)V(X)) (.) U(X))
 * and residual connections between layers; its M-FALCON subsection scores m
 * candidates in ceil(m/b_m) microbatches against cached history work.
 *
 * Readings used wherever the page leaves a step open (each is exact, not an
 * approximation):
 *   phi2(s)  = SiLU(s) / N_max, causal mask j <= i (diagonal included);
 *              masked pairs contribute exactly nothing; no 1/sqrt(d) scale.
 *   rab^p    = rab_p[h][clip(j - i, -N_max, N_max) + N_max]   (j key, i query)
 *   rab^t    = rab_t[h][min(127, floor(log2(|t_i - t_j| + 1)))] (int64 seconds)
 *   Norm     = LayerNorm over all H*d_v features of a token, no affine,
 *              biased variance, eps = hstu_dims.ln_eps.
 *   Split    = column blocks U | V | Q | K of f1's output, head-major inside.
 *   f_i      = x W^T + b with W stored [out][in];  layer: y = x + f2(.).
 *
 * Conventions for every entry point
 *   - Device pointers are HIP device memory; the caller owns every buffer.
 *     No entry point allocates or frees device memory: scratch space is the
 *     caller's workspace `ws` of at least hstu_workspace_size() bytes,
 *     256-byte aligned.
 *   - Jagged batches have no padding: sequence b owns tokens
 *     [offsets[b], offsets[b+1]) of every [T][...] array.
 *   - Matrices are row-major with a token stride `ld` in elements, so Q/K/V/U
 *     may be views into one f1 output buffer [T][4*H*d] (ld = 4*H*d).  A
 *     stride must be at least the row width and below 2^24 elements
 *     (HSTU_ERR_UNSUPPORTED otherwise).  bf16 views are moved with 16-byte
 *     accesses: their base must be 16-byte aligned and ld a multiple of 8
 *     (HSTU_ERR_ARG otherwise); so must fp32 buffers the attention writes
 *     with 16-byte stores (o_save).
 *     Per-head tensors are [T][H][d] inside a row: head h at column h*d.
 *   - Everything is enqueued on `stream` (a hipStream_t, NULL = default
 *     stream); nothing synchronises the host and nothing is copied device to
 *     host.  Outputs are overwritten, never accumulated into.
 *   - On a non-OK status nothing has been enqueued and hstu_last_error()
 *     describes the problem.  Launch failures return HSTU_ERR_DEVICE.
 *     Device-side data checks (offsets[0] == 0, non-decreasing offsets,
 *     offsets[B] == T) write a status word into the workspace; with the
 *     environment variable HSTU_DEBUG=1 (read at every call) each call
 *     synchronises the stream and reports a failed check as HSTU_ERR_ARG.
 *     hstu_attn_fwd and hstu_attn_bwd compute nothing on a batch that fails
 *     the check: their outputs are left unwritten.  The layer entry points
 *     and mfalcon_score run their linear maps before the check and leave
 *     their outputs unspecified on such a batch.
 *   - Entry points are thread-safe for distinct workspaces; calls that share
 *     a workspace must be ordered on one stream.
 */
#ifndef HSTU_H
#define HSTU_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HSTU_ABI_VERSION 2

typedef enum {
    HSTU_OK = 0,
    HSTU_ERR_ARG = 1,         /* invalid argument (null pointer, bad size, bad layout) */
    HSTU_ERR_UNSUPPORTED = 2, /* valid but not implemented (e.g. a head size) */
    HSTU_ERR_WORKSPACE = 3,   /* workspace missing, misaligned or too small */
    HSTU_ERR_DEVICE = 4       /* HIP runtime error while launching */
} hstu_status;

typedef enum { HSTU_F32 = 0, HSTU_BF16 = 1 } hstu_dtype;
typedef enum { HSTU_ACT_SILU = 0, HSTU_ACT_RELU = 1 } hstu_act; /* phi1 of Eq. 1 */

typedef enum {
    HSTU_OP_ATTN_FWD = 0,
    HSTU_OP_ATTN_BWD = 1,
    HSTU_OP_LAYER_FWD = 2,
    HSTU_OP_MFALCON = 3,
    HSTU_OP_LAYER_BWD = 4,
    HSTU_OP_LAYER_APPEND = 5
} hstu_op;

/* A jagged batch.  batch, total and n_max are host values; offsets and ts
 * are device pointers.  n_max is the N_max of phi2 and of rab^p (a constant
 * of the model, not the realised maximum length).  A batch of empty
 * sequences (total = 0) is valid: hstu_attn_fwd and hstu_attn_bwd then
 * accept NULL activation views (there are no rows), and the backward still
 * writes its bias gradients (zeros). */
typedef struct {
    int32_t batch;          /* B >= 1 */
    int32_t total;          /* T = offsets[B] (host copy), >= 0 */
    int32_t n_max;          /* N_max >= 1 */
    const int32_t *offsets; /* device [B+1], offsets[0] = 0, non-decreasing */
    const int64_t *ts;      /* device [T] int64 seconds, or NULL: no rab^t term */
} hstu_jagged;

/* Head geometry and storage dtype of activations (Q, K, V, U, outputs). */
typedef struct {
    hstu_dtype dtype; /* HSTU_BF16: MFMA path, d_qk = d_v in {32, 64, 128} for the
                       * attention entry points (hstu_attn_fwd, its _noalloc
                       * variant, hstu_softmax_attn_fwd, hstu_attn_bwd, and their
                       * workspace sizes), 128 for the layer and M-FALCON entry
                       * points; HSTU_F32: d in {16, 32, 64, 128}.  Other sizes:
                       * HSTU_ERR_UNSUPPORTED. */
    int32_t heads;    /* H >= 1 */
    int32_t d_qk;
    int32_t d_v;      /* d_qk must equal d_v */
    float ln_eps;     /* eps of Norm, > 0 */
} hstu_dims;

/* rab tables, fp32, device.  A NULL table omits that term.  hstride is the
 * distance between heads in elements; 0 shares one table across heads. */
typedef struct {
    const float *rab_p;    /* [H][2*N_max+1] */
    int64_t rab_p_hstride; /* usually 2*N_max+1 */
    const float *rab_t;    /* [H][128] */
    int64_t rab_t_hstride; /* usually 128 */
} hstu_bias;

typedef struct { const void *ptr; int64_t ld; } hstu_cmat; /* read-only row-major view */
typedef struct { void *ptr; int64_t ld; } hstu_mat;        /* writable row-major view */

/* One HSTU layer's parameters (device).  Storage dtype = hstu_dims.dtype.
 *   w1 [4*H*d][D]: output rows U | V | Q | K, head-major inside each block
 *   b1 [4*H*d] or NULL, w2 [D][H*d], b2 [D] or NULL (biases always fp32). */
typedef struct {
    const void *w1;
    const float *b1;
    const void *w2;
    const float *b2;
    hstu_bias rab;
    hstu_act phi1;
} hstu_layer;

/* Bytes of workspace an entry point needs for these sizes.  d_model and
 * total_cand are used by HSTU_OP_LAYER_FWD / HSTU_OP_LAYER_BWD /
 * HSTU_OP_MFALCON / HSTU_OP_LAYER_APPEND (d_model) and HSTU_OP_MFALCON /
 * HSTU_OP_LAYER_APPEND (total_cand: the candidates', or the new actions',
 * total) only (pass 0 otherwise); for HSTU_OP_MFALCON and
 * HSTU_OP_LAYER_APPEND `j` describes the histories (batch = users).
 * Returns 0 and sets hstu_last_error() on invalid sizes. */
size_t hstu_workspace_size(hstu_op op, const hstu_jagged *j, const hstu_dims *dims, int32_t d_model,
                           int32_t total_cand);

/*
 * Forward of Eq. 2 ([GR review] §3, spatial aggregation), optionally with
 * Eq. 3's Norm(AV) (.) U gate.
 *   q, k [T][H][d_qk], v [T][H][d_v] (storage dtype).
 *   u == NULL pointer: out = O = phi2(QK^T + rab) V, [T][H*d_v], storage dtype.
 *   u given ([T][H*d_v]): out = G = LayerNorm(O) (.) U, storage dtype.
 *   o_save (optional, fp32 [T][H*d_v], ld = H*d_v): O in fp32, for the
 *   backward; ln_stats (optional, fp32 [T][2]): per token (mean, rstd).
 */
hstu_status hstu_attn_fwd(const hstu_jagged *j, const hstu_dims *dims, const hstu_bias *bias, hstu_cmat q,
                          hstu_cmat k, hstu_cmat v, hstu_cmat u, hstu_mat out, float *o_save, float *ln_stats,
                          void *ws, size_t ws_bytes, void *stream);

/*
 * Stochastic Length ([GR review] §3, Stochastic Length): builds the sampled
 * jagged batch from full user histories.  Sequence b of `in` (n_b actions)
 * keeps L_b = min(n_b, ceil(n_b u_b^(1/alpha))) of them (at least 1 when
 * n_b > 0), a random subsequence: the L_b actions with the smallest keys
 * (ties by position), in their original order -- a uniformly random subset
 * for uniform keys (the pages give the length law and say the subsequence
 * is random; this selection rule is the plain reading).  L_b is computed in
 * fp64.
 *   u: device fp64 [B] in (0, 1]; keys: device uint32 [T] (the random
 *   numbers, drawn by the caller).
 *   out_offsets: device int32 [B+1], the sampled batch's offsets;
 *   out_index: device int32 [T] capacity, the first out_offsets[B] entries
 *   are each sampled action's row in `in`.
 *   x (optional): rows to gather, row_bytes bytes each with a stride of ldx
 *   bytes, into x_out (stride ldx_out bytes, T rows of capacity); ts_out
 *   (optional, int64 [T] capacity) gathers in->ts.
 *   Workspace: 256 bytes (a status word).  The sampled total is known on
 *   the device only (out_offsets[B]); nothing is copied to the host.
 */
hstu_status hstu_sl_sample(const hstu_jagged *in, double alpha, const double *u, const uint32_t *keys, const void *x,
                           int64_t ldx, int32_t row_bytes, int32_t *out_offsets, int32_t *out_index, void *x_out,
                           int64_t ldx_out, int64_t *ts_out, void *ws, size_t ws_bytes, void *stream);

/*
 * The comparator of pointwise aggregated attention: causal softmax attention
 * O = softmax(Q K^T / sqrt(d)) V per sequence and head, with no relative
 * bias and no gate -- the "softmax, no rab" row of [GR review] §6's
 * component ablation and the attention of the Transformer baseline of §5's
 * efficiency table -- computed on the same kernel skeleton as
 * hstu_attn_fwd (same tiles, work list and operand path; the element-wise
 * step is an online softmax), so that the two can be timed side by side.
 *   q, k, v [T][H][d], out [T][H*d] (bf16 only, d in {32, 64, 128}); lse (optional,
 *   fp32 [T][H]): the natural log of each row's sum of exp(s - max) plus the
 *   max, for a backward.  Workspace: hstu_workspace_size(HSTU_OP_ATTN_FWD).
 */
hstu_status hstu_softmax_attn_fwd(const hstu_jagged *j, const hstu_dims *dims, hstu_cmat q, hstu_cmat k,
                                  hstu_cmat v, hstu_mat out, float *lse, void *ws, size_t ws_bytes, void *stream);

/*
 * Backward of hstu_attn_fwd (chain rule through Eq. 3's Norm (.) U and
 * Eq. 2).  bf16 only, d in {32, 64, 128}.
 *   dout: upstream gradient at G when u is given (then o_save and ln_stats
 *   from the forward are required), else at O.
 *   Outputs (storage dtype): dq, dk [T][H][d], dv [T][H][d], du [T][H*d]
 *   (when u is given); fp32 drab_p [H][2*N_max+1] and drab_t [H][128] (each
 *   may be NULL to skip; contiguous, hstride as in `bias`, which must not be
 *   0 when the gradient is requested).
 *   Every output is the same bit for bit from run to run when every sequence
 *   is at most N_max long: the bias gradients are per-work-item partial
 *   sums added in a fixed order (sequence, key - query, key tile).  A batch
 *   with sequences longer than N_max may exceed the workspace's partial-sum
 *   and dS buffers (sized from N_max); such sequences fall back to fp32
 *   atomics for drab_p and dQ, whose rounding then depends on the order.
 */
hstu_status hstu_attn_bwd(const hstu_jagged *j, const hstu_dims *dims, const hstu_bias *bias, hstu_cmat q,
                          hstu_cmat k, hstu_cmat v, hstu_cmat u, const float *o_save, const float *ln_stats,
                          hstu_cmat dout, hstu_mat dq, hstu_mat dk, hstu_mat dv, hstu_mat du, float *drab_p,
                          float *drab_t, void *ws, size_t ws_bytes, void *stream);

/*
 * One HSTU layer forward ([GR review] §3 Eq. 1-3 and the residual between
 * layers): y = x + f2(LayerNorm(O) (.) U) with U, V, Q, K = Split(phi1(f1(x))).
 *   x [T][D] (storage dtype), y [T][D] (storage dtype; may not alias x).
 *   k_cache / v_cache (optional, ptr NULL to skip): this layer's K and V,
 *   [T][H][d] storage dtype -- the cacheable history work M-FALCON reuses.
 */
hstu_status hstu_layer_fwd(const hstu_jagged *j, const hstu_dims *dims, int32_t d_model, const hstu_layer *layer,
                           hstu_cmat x, hstu_mat y, hstu_mat k_cache, hstu_mat v_cache, void *ws, size_t ws_bytes,
                           void *stream);

/*
 * Backward of hstu_layer_fwd: the chain rule through f2 and the residual,
 * Eq. 3's Norm (.) U, Eq. 2, phi1 and f1 ([GR review] §3 Eq. 1-3).  The
 * forward is recomputed from x inside the call (nothing is kept between
 * calls).  bf16 storage only; d_model a multiple of 8.
 *   dy [T][D] (storage dtype): upstream gradient at y.
 *   dx [T][D] (storage dtype): gradient at x (the residual's dy plus the
 *   f1 branch); may not alias x or dy.
 *   dw1 [4*H*d][D], dw2 [D][H*d] (fp32, required), db1 [4*H*d] and
 *   db2 [D] (fp32, NULL to skip), drab_p [H][2*N_max+1] and drab_t [H][128]
 *   (fp32, NULL to skip; as in hstu_attn_bwd, which needs a per-head table
 *   for each requested gradient).  Every fp32 output is overwritten (not
 *   accumulated) and 16-byte aligned.
 *   Weight gradients are sums over all T tokens in fp32 (split over token
 *   ranges, the partial sums added in a fixed order: the result does not
 *   depend on the launch or the run).
 */
hstu_status hstu_layer_bwd(const hstu_jagged *j, const hstu_dims *dims, int32_t d_model, const hstu_layer *layer,
                           hstu_cmat x, hstu_cmat dy, hstu_mat dx, float *dw1, float *db1, float *dw2, float *db2,
                           float *drab_p, float *drab_t, void *ws, size_t ws_bytes, void *stream);

/*
 * One layer over new actions appended to cached user histories ([GR review]
 * §3, M-FALCON: the history's linear and attention computations are
 * cacheable; the architecture tree's streaming training adds actions as they
 * arrive).  User u has n_u cached history tokens (this layer's K, V in
 * k_cache / v_cache, rows hist->offsets[u]..) and a_u new tokens x_new (rows
 * add->offsets[u]..).  New token i is position n_u + i of the user's
 * sequence [history; new] with time add->ts[row]: it attends causally to
 * the whole history and to the new tokens up to itself, so y_new equals rows
 * n_u.. of hstu_layer_fwd run on the whole sequence.
 *   hist: U users (batch), total = T_hist, n_max (the model's N_max), ts
 *     [T_hist] or NULL; add: batch = U, total = T_new, offsets [U+1], ts
 *     [T_new] (NULL iff hist->ts is NULL); add->n_max is not used.
 *   k_cache, v_cache [T_hist][H][d] (may be NULL when T_hist = 0).
 *   x_new [T_new][D] in, y_new [T_new][D] out (may not alias).
 *   k_out, v_out [T_hist + T_new][H][d] out: the merged caches, user u's
 *   history rows then its new rows from row hist->offsets[u] +
 *   add->offsets[u] (the next call's caches, with offsets summed).  They may
 *   not alias the input caches.
 * bf16 storage only.  Device-side checks as for the other entry points
 * (both offset arrays start at 0, do not decrease and end at the totals).
 */
hstu_status hstu_layer_append(const hstu_jagged *hist, const hstu_jagged *add, const hstu_dims *dims, int32_t d_model,
                              const hstu_layer *layer, hstu_cmat k_cache, hstu_cmat v_cache, hstu_cmat x_new,
                              hstu_mat y_new, hstu_mat k_out, hstu_mat v_out, void *ws, size_t ws_bytes,
                              void *stream);

/*
 * M-FALCON candidate scoring ([GR review] §3, M-FALCON).  User u has a history
 * of n_u tokens (hist->offsets) whose per-layer K, V were cached by
 * hstu_layer_fwd, and candidates [cand_offsets[u], cand_offsets[u+1]) of
 * x_cand.  Every candidate sits at position n_u with time cand_ts[u] and
 * attends to the whole history and to itself, never to other candidates.
 * Candidates are processed in microbatches of b_m (>= 1); the result does not
 * depend on b_m.  Output: the candidates' final hidden states, fp32 [M][D].
 *   layers, k_cache, v_cache: host arrays of n_layers entries (device data).
 *   cand_offsets: device [U+1]; cand_ts: device [U] (NULL iff hist->ts NULL).
 *   Device-side checks: hist->offsets[0] = 0, non-decreasing,
 *   hist->offsets[U] = hist->total; cand_offsets[0] = 0, non-decreasing,
 *   cand_offsets[U] = total_cand.
 */
hstu_status mfalcon_score(const hstu_jagged *hist, const hstu_dims *dims, int32_t d_model, int32_t n_layers,
                          const hstu_layer *layers, const hstu_cmat *k_cache, const hstu_cmat *v_cache,
                          const int32_t *cand_offsets, int32_t total_cand, const int64_t *cand_ts, hstu_cmat x_cand,
                          int32_t b_m, float *y_cand, void *ws, size_t ws_bytes, void *stream);

/*
 * hstu_attn_fwd without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, results and errors as hstu_attn_fwd;
 * its scratch space (launcher work list, relative times, and the fp32 O
 * staging rows when u is given without o_save) is a static device array of
 * HSTU_NOALLOC_SCRATCH_BYTES per GPU, held by the library until the process
 * ends.  A batch needing more returns HSTU_ERR_WORKSPACE before anything is
 * enqueued (about 12 bytes per token plus 16 per 128-token tile and head,
 * plus 4*H*d_v bytes per token for the staging rows: pass o_save with u to
 * avoid them).  The call allocates nothing.  All calls on one GPU share its
 * array: calls that overlap on one GPU (other streams or threads) race and
 * must be ordered by the caller.
 */
#define HSTU_NOALLOC_SCRATCH_BYTES (16u << 20)
hstu_status hstu_attn_fwd_noalloc(const hstu_jagged *j, const hstu_dims *dims, const hstu_bias *bias, hstu_cmat q,
                                  hstu_cmat k, hstu_cmat v, hstu_cmat u, hstu_mat out, float *o_save,
                                  float *ln_stats, void *stream);

/* Kernel timing for benchmarks.  While enabled, every entry point brackets
 * each kernel (or small group of kernels) it launches with a pair of HIP
 * events recorded on the launch stream; this adds no device work and does not
 * change kernel durations.  hstu_profile_collect() waits for the recorded
 * events and returns, per kernel name, the launch count and summed duration
 * since the previous collect (at most `cap` entries; returns the number
 * written).  Off by default.  Not thread-safe against concurrent entry-point
 * calls on other threads while collecting. */
typedef struct {
    char name[48];
    int32_t launches;
    double total_ms;
} hstu_kernel_time;
void hstu_profile_enable(int32_t on);
int32_t hstu_profile_collect(hstu_kernel_time *out, int32_t cap);

/* Message of the last non-OK status on this thread ("" if none). */
const char *hstu_last_error(void);

/* HSTU_ABI_VERSION of the loaded library. */
int32_t hstu_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* HSTU_H */
