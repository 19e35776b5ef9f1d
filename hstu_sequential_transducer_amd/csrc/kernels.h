// kernels.h -- launch interfaces between the host ABI layer (api.cpp) and the
// gfx950 kernels.  Internal to libhstu; not part of the public C ABI.
#pragma once
#include "common.h"
#include "../../include/hstu.h"

// ---- entry-point internals shared by the C ABI sources (api.cpp, noalloc.hip)
namespace hstu_internal {
hstu_status set_error(hstu_status s, const char *msg);
hstu_status attn_fwd_entry(const hstu_jagged *j, const hstu_dims *dm, const hstu_bias *bias, hstu_cmat q, hstu_cmat k,
                           hstu_cmat v, hstu_cmat u, hstu_mat out, float *o_save, float *ln_stats, void *ws,
                           size_t ws_bytes, void *stream, bool lean, size_t *need);
} // namespace hstu_internal

constexpr int SCHED_BINS = 4096; // longest sequence: (SCHED_BINS - 1) tiles

// ---- launcher (sched.hip)
// rel[T] (sequence-relative times) is followed by rmin[T] and rmax[T]: at the
// first token r of every 32-token block of a sequence (r - start a multiple
// of 32), the min and max of rel over that block's tokens.
//
// Items are int2 {b, (t << 10) | (split << 9) | (part << 8) | h}: sequence b,
// tile t, head h.  With split_slots > 0 (the number of workgroups that run at
// once), tiles t >= t_split become two items (part 0 and 1, each half of the
// tile's key range) where t_split is chosen from the total work so that no
// item is much longer than the average per slot; *t_split is written (a
// large value when nothing is split).
//
// rank[B] (workspace): each sequence's rank among the sequences with the
// same tile count, by index (the tie-break of the longest-first order).
//
// SchedBwd (the backward; ds_base NULL otherwise), per sequence b with L_b
// tokens and n_b = ceil(L_b / tile) key tiles:
//   ds_base: element offset of its H planes of P x P bf16 in the dS buffer
//     (P = L rounded up to DS_PAD): the exclusive prefix sum of the plane
//     sizes, or -1 where that prefix plus the sequence's own planes exceeds
//     ds_cap elements (its dQ then goes through fp32 atomics);
//   pbase: float offset of its drab_p partial sums, H * n_b slots of L_b
//     floats, or -1 past p_cap floats (its items then add into drab_p with
//     atomics);
//   tbase: float offset of its drab_t partial sums, H * n_b slots of
//     TB_SLOTS floats (always fits: the caller sizes the buffer for every
//     tile).
// zero0[0, n0) and zero1[0, n1) (optional) are zeroed on the way.
constexpr int ITEM_T_SHIFT = 10;
constexpr int DS_PAD = 128;
constexpr int TB_SLOTS = 64; // time buckets an int64 difference can reach
struct SchedBwd {
    int64_t *ds_base;
    int64_t ds_cap;
    int64_t *pbase;
    int64_t p_cap;
    int64_t *tbase;
    float *zero0;
    int64_t n0;
    float *zero1;
    int64_t n1;
};
// Rows zeroed in the launch that follows the launcher (after validation):
// SPLIT_ROWS: the fp32 rows [offsets[b] + tile * *t_split, offsets[b + 1])
// of rows/ld/F (the rows that split forward items accumulate into);
// DQA_ROWS: the rows of rows ([T][F] fp32) of the sequences with
// ds_base[b] < 0 (their dQ goes through the fp32 accumulator).
struct ZeroRows {
    enum Mode { NONE = 0, SPLIT_ROWS = 1, DQA_ROWS = 2 } mode;
    int tile;
    const int *t_split;
    const int64_t *ds_base;
    float *rows;
    int64_t ld;
    int F;
};
void launch_sched(const int32_t *offsets, const int64_t *ts, int B, int T, int tile, int H, int *status, int *n_items,
                  int2 *items, int max_items, uint32_t *rel, int32_t *wide, int32_t *rank, int split_slots, int *t_split,
                  const SchedBwd &bw, hipStream_t st, const ZeroRows &z = ZeroRows{});
// Appending new actions to cached histories: validates hoff / aoff (first 0,
// non-decreasing, last = Th / Tn) into *status, writes the merged offsets
// moff[u] = hoff[u] + aoff[u] (user u's sequence [history; new]) and the
// work list: items (u, tile t, head h) for the query tiles that hold new
// positions, t from hoff-length / tile on (the format of launch_sched's).
// Then one wave per merged row copies that row's K and V -- from the cache
// (k_cache, v_cache) for history rows, from the new tokens' f1 output (knew,
// vnew, row aoff[u] + i) for new ones -- into kout / vout, and (when ts are
// given) its time into ts_m; then the relative times of the merged batch as
// launch_sched computes them.
struct AppendPlan {
    const int32_t *hoff, *aoff;
    int U, Th, Tn, H, tile, max_items;
    int *status, *n_items;
    int2 *items;
    int32_t *moff;
    const bf16 *kc, *vc;
    int64_t ldkc, ldvc;
    const bf16 *knew, *vnew;
    int64_t ldnew;
    bf16 *kout, *vout;
    int64_t ldko, ldvo;
    int hd;                     // H * d elements per row
    const int64_t *ts_h, *ts_a;
    int64_t *ts_m;
    uint32_t *rel;
    int32_t *wide;
};
hipError_t launch_append_plan(const AppendPlan &p, hipStream_t st);


// ---- attention forward (attn_fwd.hip)
struct AttnFwdArgs {
    const void *q, *k, *v;
    int64_t ldq, ldk, ldv;      // token strides (elements)
    const int32_t *offsets;
    const int64_t *ts;          // NULL: no time bias
    const uint32_t *rel;        // sequence-relative 32-bit times
    const int32_t *wide;        // per sequence: 1 = 64-bit time path
    const uint32_t *rmin, *rmax; // per 32-token block (at its first token): range of rel
    const float *rab_p;         // NULL: no position bias
    int64_t rp_hs;
    const float *rab_t;         // NULL: no time bias
    int64_t rt_hs;
    int H, N, d;
    float inv_n;
    const int2 *items;
    const int *n_items;
    float *o32;                 // fp32 output [T][H*d] (ld_o32) or NULL
    int64_t ld_o32;
    void *o16;                  // storage-dtype output or NULL
    int64_t ld_o16;
    // Appended actions (bf16 kernel; NULL otherwise): sequence b is
    // [history; new] with hoff[b+1] - hoff[b] history tokens; only its new
    // positions are queries, and new token i reads Q and writes O at row
    // aoff[b] + i.
    const int32_t *hoff, *aoff;
    float *lse;                 // softmax comparator: per (row, head) log-sum-exp [T][H], or NULL
};
constexpr int FWD_BM = 128; // query rows per workgroup (bf16 MFMA kernel)
// Causal softmax attention softmax(Q K^T / sqrt(d)) V, bf16, d = 128, on the
// forward's skeleton (the comparator of pointwise aggregated attention):
// items from launch_sched without splits; o16 (and o32 if given) written.
hipError_t launch_attn_softmax_fwd(const AttnFwdArgs &a, int max_items, hipStream_t st);
constexpr int F32_BM = 64;  // query rows per workgroup (fp32 kernel)
hipError_t launch_attn_fwd_bf16(const AttnFwdArgs &a, int max_items, hipStream_t st);
hipError_t launch_attn_fwd_f32(const AttnFwdArgs &a, int max_items, hipStream_t st);

// ---- LayerNorm(O) (.) U epilogue and its backward (epilogue.hip)
// G = (O - mean) * rstd * U over F features per row; out dtype per flag.
hipError_t launch_ln_gate_fwd(const float *O, int64_t ldo, int nparts, int64_t part_stride, const void *U, int64_t ldu,
                              bool bf16io, void *G, int64_t ldg, float *stats, float *o_copy, int64_t ld_oc, int T,
                              int F, float eps, const int *status, hipStream_t st);
// zrows (optional, 16-byte aligned, zF a multiple of 4): rows [T][zF] of an
// fp32 buffer zeroed on the way (the dQ accumulator).
hipError_t launch_ln_gate_bwd(const void *dG, int64_t ldg, const void *U, int64_t ldu, const float *O, int64_t ldo,
                              const float *stats, bool bf16io, void *dU, int64_t lddu, bf16 *dO, float scale, int T,
                              int F, float *zrows, int zF, const int *status, hipStream_t st);

// ---- attention backward (attn_bwd.hip)
struct AttnBwdArgs {
    const bf16 *q, *k, *v;
    int64_t ldq, ldk, ldv;
    const bf16 *dO;             // dO / N_max as bf16 hi plane [T][H*d], then lo plane [T][H*d]
    int T;
    const int32_t *offsets;
    const int64_t *ts;
    const uint32_t *rel;
    const int32_t *wide;
    const uint32_t *rmin, *rmax; // per 32-token block (at its first token): range of rel
    const float *rab_p;
    int64_t rp_hs;
    const float *rab_t;
    int64_t rt_hs;
    int H, N;
    const int2 *items;
    const int *n_items;
    bf16 *ds;                   // dS buffer (see launch_sched's ds_base), written for dQ = dS K
    const int64_t *ds_base;     // per sequence: offset of its H planes of P x P in ds, -1: did not fit
    float *dq_acc;              // fp32 [T][H*d] accumulator of the sequences that did not fit (rows zeroed)
    bf16 *dk, *dv;
    int64_t lddk, lddv;
    float *drab_p;              // fp32 [H][2N+1] (zeroed; sequences without partial slots add here) or NULL
    float *drab_t;              // NULL: no drab_t (else the partial slots below are written)
    float *dpart;               // drab_p partial slots (see launch_sched's pbase)
    const int64_t *pbase;
    float *tpart;               // drab_t partial slots (see launch_sched's tbase)
    const int64_t *tbase;
};
constexpr int BWD_BN = 128; // keys per workgroup
// d: the head size (128, 64 or 32), which selects the kernel instantiation
hipError_t launch_attn_bwd_bf16(const AttnBwdArgs &a, int d, int max_items, hipStream_t st);
// drab_p += and drab_t = the items' partial sums, added in a fixed order
// (sequence, key - query, key tile): the bias gradients do not depend on
// the order in which the backward's items ran.
struct DrabReduceArgs {
    const int32_t *offsets;
    int B, H, N;
    const int *status;
    const float *dpart;
    const int64_t *pbase;
    const float *tpart;
    const int64_t *tbase;
    float *drab_p;              // or NULL
    int64_t p_hs;
    float *drab_t;              // or NULL
    int64_t t_hs;
};
hipError_t launch_drab_reduce(const DrabReduceArgs &r, hipStream_t st);

// ---- dQ = dS K (dq.hip): one workgroup per backward item read as
// (sequence b, query tile t of 128, head h); bf16 dQ out (d = 128).
struct DqArgs {
    const bf16 *ds;             // the backward's dS buffer
    const int64_t *ds_base;     // -1: the sequence's dQ is in dq_acc (converted here)
    const float *dq_acc;
    int64_t ldacc;
    const bf16 *k;
    int64_t ldk;
    const int32_t *offsets;
    const int2 *items;
    const int *n_items;
    bf16 *dq;
    int64_t lddq;
    int d;                      // head size: 128, 64 or 32
};
hipError_t launch_dq_gemm(const DqArgs &a, int max_items, hipStream_t st);

// ---- small helpers (misc.hip)
hipError_t launch_fill_zero(void *p, size_t bytes, hipStream_t st);
hipError_t launch_cast_f32_to_bf16(const float *src, int64_t lds, bf16 *dst, int64_t ldd, int rows, int cols,
                                   const int *status, hipStream_t st);
hipError_t launch_copy_f32(const float *src, float *dst, size_t n, hipStream_t st);
hipError_t launch_scale_bf16(const bf16 *src, int64_t lds, bf16 *dst, int64_t ldd, int rows, int cols, float scale,
                             hipStream_t st);

// ---- GEMM with fused epilogues (gemm.hip)
// C[M][N] = act(A[M][K] . W[N][K]^T + bias) + R, A/W in the storage dtype.
enum GemmEpi { EPI_NONE = 0, EPI_SILU = 1, EPI_RELU = 2 };
struct GemmArgs {
    const void *A;
    int64_t lda;
    const void *W;              // [N][K] ([out][in]), ld = K
    const float *bias;          // [N] or NULL
    const float *R32;           // fp32 residual [M][N] (ld ldr) or NULL
    const void *R16;            // storage-dtype residual (ld ldr) or NULL
    int64_t ldr;
    void *C;
    int64_t ldc;
    bool c_f32;                 // C is fp32 (else storage dtype)
    void *C16;                  // optional storage-dtype copy of C
    int64_t ldc16;
    void *Cpre;                 // optional storage-dtype copy of acc + bias (before act)
    int64_t ldcpre;
    int M, N, K;
    int epi;
    // optional copies of columns [k_lo, k_lo + kv_w) and [v_lo, v_lo + kv_w)
    void *Ck;
    int64_t ldck;
    int k_lo;
    void *Cv;
    int64_t ldcv;
    int v_lo;
    int kv_w;
};
hipError_t launch_gemm_bf16(const GemmArgs &g, hipStream_t st);
hipError_t launch_gemm_f32(const GemmArgs &g, hipStream_t st);

// ---- layer backward outside the attention (layer_bwd.hip)
// Weight gradient dW[m][n] = sum_t A[t][m] B[t][n] (A [K][M], B [K][N], bf16,
// token-major), as fp32 partial sums part[splits][M][N] over token ranges
// [s chunk, (s + 1) chunk).  M, N multiples of 8; lda, ldb multiples of 8;
// A, B 16-byte aligned.
struct WgradArgs {
    const void *A;
    int64_t lda;
    const void *B;
    int64_t ldb;
    float *part;
    int M, N, K;
    int chunk, splits;
};
struct WgradPlan {
    int chunk, splits;
};
WgradPlan wgrad_plan(int M, int N, int K);
hipError_t launch_gemm_wgrad(const WgradArgs &g, hipStream_t st);
// out[e] = sum over s < S of part[s][e], e < E (E a multiple of 4)
hipError_t launch_sum_splits(const float *part, int S, int64_t E, float *out, hipStream_t st);
// act 1 (SiLU') / 2 (ReLU'): a[r][c] *= phi1'(z[r][c]) in place; act 0: no
// change.  Column sums of the (new) a per block of COLSUM_ROWS rows go to
// part[colsum_blocks(M)][N].  N a multiple of 8, rows 16-byte aligned.
constexpr int COLSUM_ROWS = 64;
int colsum_blocks(int M);
hipError_t launch_colsum_act(bf16 *a, int64_t lda, const bf16 *z, int64_t ldz, int act, int M, int N, float *part,
                             hipStream_t st);
hipError_t launch_transpose_bf16(const bf16 *in, int64_t ldi, int R, int C, bf16 *out, int64_t ldo, hipStream_t st);

// ---- M-FALCON (mfalcon.hip)
constexpr int MF_TC = 128; // candidates per attention tile
struct MfalconArgs {
    const void *q;              // candidate Q view of the f1 output [M][4*H*d] (ld ldz)
    int64_t ldz;
    const void *kc, *vc;        // this layer's cached history K, V [T_hist][H][d]
    int64_t ldkc, ldvc;
    const int32_t *hoff;        // [U+1]
    const int64_t *hts;         // [T_hist] or NULL
    const int64_t *cts;         // [U] or NULL
    const float *rab_p;
    int64_t rp_hs;
    const float *rab_t;
    int64_t rt_hs;
    int H, N, M, d;
    int kchunk;                 // history keys per split
    const int4 *items;          // (user, first row, rows, head << 16 | split)
    const int *n_items;
    float *part;                // [nsplit][M][H*d] fp32 partial sums
};
// Validates hoff (hoff[0] = 0, non-decreasing, hoff[U] = hist_total) and
// coff (coff[0] = 0, non-decreasing, coff[U] = M) into *status.
hipError_t launch_mfalcon_sched(const int32_t *hoff, const int32_t *coff, int U, int M, int H, int b_m, int nsplit,
                                int4 *items, int *n_items, int *status, int max_items, int hist_total, hipStream_t st);
hipError_t launch_mfalcon_attn(const MfalconArgs &a, int max_items, bool bf16io, hipStream_t st);
hipError_t launch_mfalcon_epilogue(const float *part, int nsplit, const void *Z, int64_t ldz, const float *rab_p,
                                   int64_t rp_hs, const float *rab_t, int64_t rt_hs, bool use_t, int N, float eps,
                                   void *G, int64_t ldg, int M, int H, int d, bool bf16io, hipStream_t st);

// ---- Stochastic Length sampling as a device gather (sl.hip)
struct SlArgs {
    const int32_t *offsets;     // input batch [B+1]
    int B, T;
    double alpha;
    const double *u;            // [B] in (0, 1]
    const uint32_t *keys;       // [T]
    int32_t *out_off;           // [B+1]
    int32_t *out_idx;           // [T] capacity (first out_off[B] written)
    const void *x;              // rows to gather, or NULL
    int64_t ldx_bytes;
    void *y;
    int64_t ldy_bytes;
    int64_t row_bytes;
    const int64_t *ts;          // [T] or NULL
    int64_t *ts_out;            // [T] capacity or NULL
    int *status;
};
hipError_t launch_sl_sample(const SlArgs &a, hipStream_t st);
