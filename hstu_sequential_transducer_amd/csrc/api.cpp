// api.cpp -- the C ABI of libhstu (declared in include/hstu.h): argument
// validation, workspace carving and kernel dispatch.  No entry point
// allocates device memory, synchronises the host (unless HSTU_DEBUG=1) or
// copies device data to the host.
#include "../../include/hstu.h"
#include "kernels.h"
#include "profile.h"

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

namespace {

thread_local std::string g_err;

hstu_status fail(hstu_status s, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return s;
}

hstu_status ok()
{
    g_err.clear();
    return HSTU_OK;
}

// HSTU_DEBUG=1: read at every call (a process may switch it on and off).
bool debug_mode()
{
    const char *e = getenv("HSTU_DEBUG");
    return e && e[0] == '1';
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Carver {
    size_t cur = 0;
    size_t take(size_t bytes)
    {
        size_t o = cur;
        cur = align256(cur + bytes);
        return o;
    }
};

size_t elem_size(hstu_dtype t) { return t == HSTU_BF16 ? 2 : 4; }

// Items bound: sum_b ceil(L_b / tile) * H <= ((T + B (tile - 1)) / tile) * H.
int max_items_for(int B, int T, int tile, int H)
{
    const int64_t n = ((int64_t)T + (int64_t)B * (tile - 1)) / tile * H;
    return (int)n;
}

// Workspace of the attention entry points.
struct AttnWs {
    size_t header, items, rel, wide, rank, obuf, dO, ds_base, ds, dq, pbase, tbase, dpart, tpart, total;
    int64_t ds_cap; // elements of the dS buffer
    int64_t p_cap;  // floats of the drab_p partial slots
};

// The backward (bwd = true) also carves the dS buffer: H planes of P x P
// bf16 per sequence, P = L rounded up to DS_PAD.  sum_b P_b^2 <= (n_max +
// DS_PAD - 1) (T + (DS_PAD - 1) B) for sequences no longer than n_max; a
// sequence beyond what is left takes the fp32-atomic dQ path instead.  The
// same bound holds for the drab_p partial slots (H n_b L_b floats per
// sequence, n_b = ceil(L_b / 128) <= ceil(n_max / 128)): sequences past it
// add their share of drab_p with atomics.  The drab_t slots (H n_b TB_SLOTS
// floats) always fit.
AttnWs attn_ws(const hstu_jagged *j, const hstu_dims *dm, int tile, bool bwd, bool with_obuf = true)
{
    AttnWs w{};
    Carver c;
    const int B = j->batch, T = j->total, H = dm->heads;
    w.header = c.take(256);
    w.items = c.take((size_t)2 * max_items_for(B, T, tile, H) * sizeof(int2)); // split items: up to 2 per tile
    w.rel = c.take((size_t)T * 4 * 3); // rel, then rmin and rmax per 32-token block
    w.wide = c.take((size_t)B * 4);
    w.rank = c.take((size_t)B * 4);
    w.obuf = with_obuf ? c.take((size_t)T * H * dm->d_v * 4) : 0;
    if (bwd) {
        w.dO = c.take((size_t)T * H * dm->d_v * 2 * 2); // hi and lo bf16 planes
        w.ds_base = c.take((size_t)B * 8);
        w.ds_cap = ((int64_t)j->n_max + DS_PAD - 1) * ((int64_t)T + (int64_t)(DS_PAD - 1) * B) * H;
        w.ds = c.take((size_t)w.ds_cap * 2);
        w.dq = c.take((size_t)T * H * dm->d_qk * 4); // dQ accumulator of sequences beyond the dS buffer
        w.pbase = c.take((size_t)B * 8);
        w.tbase = c.take((size_t)B * 8);
        w.p_cap = (int64_t)H * (((int64_t)j->n_max + BWD_BN - 1) / BWD_BN) * (int64_t)T;
        w.dpart = c.take((size_t)w.p_cap * 4);
        w.tpart = c.take((size_t)max_items_for(B, T, BWD_BN, H) * TB_SLOTS * 4);
    }
    w.total = c.cur;
    return w;
}

int fwd_tile(const hstu_dims *dm) { return dm->dtype == HSTU_BF16 ? FWD_BM : F32_BM; }

// Forward workgroups that run at once on the current device (two per
// compute unit: the kernel's LDS allows two).
int concurrent_slots()
{
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 512;
    if (cached[dev] == 0) {
        int cu = 0;
        if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu <= 0) cu = 256;
        cached[dev] = 2 * cu;
    }
    return cached[dev];
}

hstu_status check_jagged(const hstu_jagged *j)
{
    if (!j) return fail(HSTU_ERR_ARG, "jagged descriptor is NULL");
    if (j->batch < 1) return fail(HSTU_ERR_ARG, "batch must be >= 1 (got %d)", j->batch);
    if (j->total < 0) return fail(HSTU_ERR_ARG, "total must be >= 0 (got %d)", j->total);
    if (j->n_max < 1) return fail(HSTU_ERR_ARG, "n_max must be >= 1 (got %d)", j->n_max);
    if (j->n_max > (1 << 24)) return fail(HSTU_ERR_UNSUPPORTED, "n_max above 2^24 is not supported");
    if (!j->offsets) return fail(HSTU_ERR_ARG, "offsets is NULL");
    if (j->total > 0 && (int64_t)j->total * 8 > INT32_MAX * 4LL)
        return fail(HSTU_ERR_UNSUPPORTED, "total tokens too large");
    return HSTU_OK;
}

// `bf16_heads`: the bf16 head sizes the calling entry point's kernels take
// (the attention forwards and backward take 32, 64 and 128; everything else
// 128).
enum Bf16Heads { BF16_D128, BF16_D32_64_128 };

hstu_status check_dims(const hstu_dims *dm, Bf16Heads bf16_heads = BF16_D128)
{
    if (!dm) return fail(HSTU_ERR_ARG, "dims descriptor is NULL");
    if (dm->dtype != HSTU_F32 && dm->dtype != HSTU_BF16) return fail(HSTU_ERR_ARG, "unknown dtype %d", (int)dm->dtype);
    if (dm->heads < 1 || dm->heads > 255) return fail(HSTU_ERR_ARG, "heads must be in [1, 255] (got %d)", dm->heads);
    if (dm->d_qk != dm->d_v) return fail(HSTU_ERR_UNSUPPORTED, "d_qk != d_v is not supported");
    if (!(dm->ln_eps > 0.f)) return fail(HSTU_ERR_ARG, "ln_eps must be > 0");
    if (dm->dtype == HSTU_BF16 && bf16_heads == BF16_D128 && dm->d_qk != 128)
        return fail(HSTU_ERR_UNSUPPORTED, "this bf16 entry point supports d = 128 (got %d)", dm->d_qk);
    if (dm->dtype == HSTU_BF16 && dm->d_qk != 32 && dm->d_qk != 64 && dm->d_qk != 128)
        return fail(HSTU_ERR_UNSUPPORTED, "bf16 attention forward supports d in {32, 64, 128} (got %d)", dm->d_qk);
    if (dm->dtype == HSTU_F32 && dm->d_qk != 16 && dm->d_qk != 32 && dm->d_qk != 64 && dm->d_qk != 128)
        return fail(HSTU_ERR_UNSUPPORTED, "fp32 path supports d in {16, 32, 64, 128} (got %d)", dm->d_qk);
    if (dm->heads * dm->d_v > 2048) return fail(HSTU_ERR_UNSUPPORTED, "H*d_v above 2048 is not supported");
    return HSTU_OK;
}

hstu_status check_bias(const hstu_bias *bs, const hstu_jagged *j)
{
    if (!bs) return HSTU_OK;
    if (bs->rab_p && bs->rab_p_hstride != 0 && bs->rab_p_hstride < 2 * (int64_t)j->n_max + 1)
        return fail(HSTU_ERR_ARG, "rab_p_hstride must be 0 or >= 2*n_max+1");
    if (bs->rab_t && bs->rab_t_hstride != 0 && bs->rab_t_hstride < 128)
        return fail(HSTU_ERR_ARG, "rab_t_hstride must be 0 or >= 128");
    return HSTU_OK;
}

hstu_status check_view(const void *p, int64_t ld, int64_t width, const char *name, bool required = true)
{
    if (!p) return required ? fail(HSTU_ERR_ARG, "%s is NULL", name) : HSTU_OK;
    if (ld < width) return fail(HSTU_ERR_ARG, "%s: ld (%lld) < row width (%lld)", name, (long long)ld, (long long)width);
    // kernels form in-row offsets from 24-bit products
    if (ld >= ((int64_t)1 << 24))
        return fail(HSTU_ERR_UNSUPPORTED, "%s: ld (%lld) must be below 2^24 elements", name, (long long)ld);
    if (((uintptr_t)p & 3) != 0) return fail(HSTU_ERR_ARG, "%s must be 4-byte aligned", name);
    return HSTU_OK;
}

// bf16 activations are moved with 16-byte accesses (global -> LDS copies,
// vector loads and stores): base 16-byte aligned and ld a multiple of 8.
// fp32 buffers written with 16-byte stores (o_save) need the same base.
hstu_status check_vec_view(const void *p, int64_t ld, hstu_dtype dt, const char *name)
{
    if (!p) return HSTU_OK;
    if (dt == HSTU_BF16 && ((((uintptr_t)p) & 15) != 0 || (ld % 8) != 0))
        return fail(HSTU_ERR_ARG, "%s must be 16-byte aligned with ld a multiple of 8 (bf16)", name);
    if (dt == HSTU_F32 && (((uintptr_t)p) & 15) != 0)
        return fail(HSTU_ERR_ARG, "%s must be 16-byte aligned", name);
    return HSTU_OK;
}

hstu_status check_ws(void *ws, size_t ws_bytes, size_t need)
{
    if (need == 0) return HSTU_OK;
    if (!ws) return fail(HSTU_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", need);
    if (((uintptr_t)ws & 255) != 0) return fail(HSTU_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if (ws_bytes < need) return fail(HSTU_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, need);
    return HSTU_OK;
}

hstu_status launched(hipError_t e, const char *what)
{
    if (e != hipSuccess) return fail(HSTU_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
    return HSTU_OK;
}

hstu_status debug_check(void *ws, hipStream_t st)
{
    if (!debug_mode()) return HSTU_OK;
    hipError_t e = hipStreamSynchronize(st);
    if (e != hipSuccess) return fail(HSTU_ERR_DEVICE, "HSTU_DEBUG sync: %s", hipGetErrorString(e));
    int status = 0;
    e = hipMemcpy(&status, ws, sizeof(int), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return fail(HSTU_ERR_DEVICE, "HSTU_DEBUG status read: %s", hipGetErrorString(e));
    if (status & HSTU_DEV_BAD_OFFSETS)
        return fail(HSTU_ERR_ARG, "offsets invalid (offsets[0] != 0, decreasing, or offsets[B] != total)");
    if (status & HSTU_DEV_TOO_LONG) return fail(HSTU_ERR_UNSUPPORTED, "a sequence has too many tiles");
    return HSTU_OK;
}

#define TRY(x)                                                                                                     \
    do {                                                                                                           \
        hstu_status _s = (x);                                                                                      \
        if (_s != HSTU_OK) return _s;                                                                              \
    } while (0)

// Enqueue the forward (launcher, attention kernel, optional LayerNorm gate)
// on validated arguments; `wb` is the workspace carved as `w`.
hstu_status attn_fwd_launch(const hstu_jagged *j, const hstu_dims *dm, const hstu_bias *bias, hstu_cmat q, hstu_cmat k,
                            hstu_cmat v, hstu_cmat u, hstu_mat out, float *o_save, float *ln_stats, char *wb,
                            const AttnWs &w, hipStream_t st)
{
    const int H = dm->heads, d = dm->d_qk, F = H * dm->d_v;
    const int tile = fwd_tile(dm);
    int *status = (int *)(wb + w.header), *n_items = status + 1;
    int2 *items = (int2 *)(wb + w.items);
    uint32_t *rel = (uint32_t *)(wb + w.rel);
    int32_t *wide = (int32_t *)(wb + w.wide);
    const int T = j->total, B = j->batch;
    // Long query tiles are split over two workgroups (halves of the key
    // range) when the output accumulates in fp32 (the LayerNorm-gate path):
    // the halves add into zeroed rows.
    const bool split = dm->dtype == HSTU_BF16 && d == 128 && u.ptr != nullptr;
    const int max_items = (split ? 2 : 1) * max_items_for(B, T, tile, H);
    int *t_split = status + 2;
    float *obuf = u.ptr ? (o_save ? o_save : (float *)(wb + w.obuf)) : nullptr;
    {
        // (the launch after the launcher also zeroes the rows split items add into)
        ProfScope ps("sched_kernel", st);
        ZeroRows z{};
        if (split) {
            z.mode = ZeroRows::SPLIT_ROWS;
            z.tile = tile;
            z.t_split = t_split;
            z.rows = obuf;
            z.ld = F;
            z.F = F;
        }
        launch_sched(j->offsets, j->ts, B, T, tile, H, status, n_items, items, max_items, rel, wide,
                     (int32_t *)(wb + w.rank), split ? concurrent_slots() : 0, t_split, SchedBwd{}, st, z);
    }
    TRY(launched(hipGetLastError(), "schedule kernel"));

    AttnFwdArgs a{};
    a.q = q.ptr;
    a.k = k.ptr;
    a.v = v.ptr;
    a.ldq = q.ld;
    a.ldk = k.ld;
    a.ldv = v.ld;
    a.offsets = j->offsets;
    a.ts = (bias && bias->rab_t) ? j->ts : nullptr;
    a.rel = rel;
    a.wide = wide;
    a.rmin = rel + T;
    a.rmax = rel + 2 * (size_t)T;
    a.rab_p = bias ? bias->rab_p : nullptr;
    a.rp_hs = bias ? bias->rab_p_hstride : 0;
    a.rab_t = (bias && j->ts) ? bias->rab_t : nullptr;
    a.rt_hs = bias ? bias->rab_t_hstride : 0;
    a.H = H;
    a.N = j->n_max;
    a.d = d;
    a.inv_n = 1.0f / (float)j->n_max;
    a.items = items;
    a.n_items = n_items;
    if (u.ptr) {
        a.o32 = obuf;
        a.ld_o32 = F;
        a.o16 = nullptr;
    } else {
        a.o32 = o_save;
        a.ld_o32 = F;
        a.o16 = out.ptr;
        a.ld_o16 = out.ld;
    }
    hipError_t e;
    {
        ProfScope ps(dm->dtype == HSTU_BF16 ? "attn_fwd_bf16_kernel" : "attn_fwd_f32_kernel", st);
        e = dm->dtype == HSTU_BF16 ? launch_attn_fwd_bf16(a, max_items, st) : launch_attn_fwd_f32(a, max_items, st);
    }
    TRY(launched(e, "attention forward kernel"));
    if (u.ptr) {
        {
            ProfScope ps("ln_gate_fwd_kernel", st);
            e = launch_ln_gate_fwd(obuf, F, 1, 0, u.ptr, u.ld, dm->dtype == HSTU_BF16, out.ptr, out.ld, ln_stats, nullptr,
                                   0, T, F, dm->ln_eps, status, st);
        }
        TRY(launched(e, "LayerNorm gate kernel"));
    }
    return HSTU_OK;
}

// Enqueue the backward (launcher, gate backward or scaling, attention
// backward, dQ) on validated arguments; `wb` is the workspace carved as `w`.
hstu_status attn_bwd_launch(const hstu_jagged *j, const hstu_dims *dm, const hstu_bias *bias, hstu_cmat q,
                            hstu_cmat k, hstu_cmat v, hstu_cmat u, const float *o_save, const float *ln_stats,
                            hstu_cmat dout, hstu_mat dq, hstu_mat dk, hstu_mat dv, hstu_mat du, float *drab_p,
                            float *drab_t, char *wb, const AttnWs &w, hipStream_t st)
{
    const int H = dm->heads, d = dm->d_qk, F = H * dm->d_v;
    const bool has_p = bias && bias->rab_p;
    const bool has_t = bias && bias->rab_t && j->ts;
    int *status = (int *)(wb + w.header), *n_items = status + 1;
    int2 *items = (int2 *)(wb + w.items);
    uint32_t *rel = (uint32_t *)(wb + w.rel);
    int32_t *wide = (int32_t *)(wb + w.wide);
    bf16 *dO = (bf16 *)(wb + w.dO);
    int64_t *ds_base = (int64_t *)(wb + w.ds_base);
    bf16 *ds = (bf16 *)(wb + w.ds);
    float *dq_acc = (float *)(wb + w.dq);
    const int T = j->total, B = j->batch, N = j->n_max;
    const int max_items = max_items_for(B, T, BWD_BN, H);
    const int64_t p_hs = has_p ? bias->rab_p_hstride : 2 * (int64_t)N + 1;
    const int64_t t_hs = (bias && bias->rab_t) ? bias->rab_t_hstride : 128;
    int64_t *pbase = (int64_t *)(wb + w.pbase), *tbase = (int64_t *)(wb + w.tbase);
    float *dpart = (float *)(wb + w.dpart), *tpart = (float *)(wb + w.tpart);
    {
        ProfScope ps("sched_kernel", st);
        // (the scheduler also zeroes drab_p, which sequences without partial
        // slots add into)
        SchedBwd sb{};
        sb.ds_base = ds_base;
        sb.ds_cap = w.ds_cap;
        sb.pbase = pbase;
        sb.p_cap = w.p_cap;
        sb.tbase = tbase;
        sb.zero0 = drab_p;
        sb.n0 = (int64_t)H * p_hs;
        if (!has_t) { // requested without a time term: its gradient is zero
            sb.zero1 = drab_t;
            sb.n1 = (int64_t)H * t_hs;
        }
        // (and the launch after it zeroes the fp32 dQ rows of the sequences
        // whose dS planes do not fit the buffer)
        ZeroRows z{};
        z.mode = ZeroRows::DQA_ROWS;
        z.ds_base = ds_base;
        z.rows = dq_acc;
        z.F = H * d;
        launch_sched(j->offsets, j->ts, B, T, BWD_BN, H, status, n_items, items, max_items, rel, wide,
                     (int32_t *)(wb + w.rank), 0, nullptr, sb, st, z);
    }
    TRY(launched(hipGetLastError(), "schedule kernel"));
    const float inv_n = 1.0f / (float)N;
    if (u.ptr) {
        ProfScope ps("ln_gate_bwd_kernel", st);
        TRY(launched(launch_ln_gate_bwd(dout.ptr, dout.ld, u.ptr, u.ld, o_save, F, ln_stats, true, du.ptr, du.ld, dO,
                                        inv_n, T, F, nullptr, 0, status, st),
                     "LayerNorm gate backward kernel"));
    } else {
        ProfScope ps("scale_bf16_kernel", st);
        TRY(launched(launch_scale_bf16((const bf16 *)dout.ptr, dout.ld, dO, F, T, F, inv_n, st), "scale kernel"));
    }
    AttnBwdArgs a{};
    a.q = (const bf16 *)q.ptr;
    a.k = (const bf16 *)k.ptr;
    a.v = (const bf16 *)v.ptr;
    a.ldq = q.ld;
    a.ldk = k.ld;
    a.ldv = v.ld;
    a.dO = dO;
    a.T = T;
    a.offsets = j->offsets;
    a.ts = has_t ? j->ts : nullptr;
    a.rel = rel;
    a.wide = wide;
    a.rmin = rel + T;
    a.rmax = rel + 2 * (size_t)T;
    a.rab_p = has_p ? bias->rab_p : nullptr;
    a.rp_hs = p_hs;
    a.rab_t = has_t ? bias->rab_t : nullptr;
    a.rt_hs = t_hs;
    a.H = H;
    a.N = N;
    a.items = items;
    a.n_items = n_items;
    a.ds = ds;
    a.ds_base = ds_base;
    a.dq_acc = dq_acc;
    a.dk = (bf16 *)dk.ptr;
    a.dv = (bf16 *)dv.ptr;
    a.lddk = dk.ld;
    a.lddv = dv.ld;
    a.drab_p = drab_p;
    a.drab_t = has_t ? drab_t : nullptr;
    a.dpart = dpart;
    a.pbase = pbase;
    a.tpart = tpart;
    a.tbase = tbase;
    {
        ProfScope ps("attn_bwd_bf16_kernel", st);
        TRY(launched(launch_attn_bwd_bf16(a, d, max_items, st), "attention backward kernel"));
    }
    if (drab_p || (drab_t && has_t)) {
        DrabReduceArgs r{};
        r.offsets = j->offsets;
        r.B = B;
        r.H = H;
        r.N = N;
        r.status = status;
        r.dpart = dpart;
        r.pbase = pbase;
        r.tpart = tpart;
        r.tbase = tbase;
        r.drab_p = drab_p;
        r.p_hs = p_hs;
        r.drab_t = has_t ? drab_t : nullptr;
        r.t_hs = t_hs;
        ProfScope ps("drab_reduce_kernel", st);
        TRY(launched(launch_drab_reduce(r, st), "bias-gradient reduction kernel"));
    }
    {
        DqArgs qa{};
        qa.ds = ds;
        qa.ds_base = ds_base;
        qa.dq_acc = dq_acc;
        qa.ldacc = (int64_t)H * d;
        qa.k = (const bf16 *)k.ptr;
        qa.ldk = k.ld;
        qa.offsets = j->offsets;
        qa.items = items;
        qa.n_items = n_items;
        qa.dq = (bf16 *)dq.ptr;
        qa.lddq = dq.ld;
        qa.d = d;
        ProfScope ps("dq_gemm_kernel", st);
        TRY(launched(launch_dq_gemm(qa, max_items, st), "dQ kernel"));
    }
    return HSTU_OK;
}

// Workspace of hstu_layer_fwd: the attention's, then f1's output Z [T][4Hd]
// and the gate G [T][Hd] (storage dtype).
struct LayerWs {
    AttnWs attn;
    size_t z, g, total;
};

LayerWs layer_ws(const hstu_jagged *j, const hstu_dims *dm)
{
    LayerWs w{};
    w.attn = attn_ws(j, dm, fwd_tile(dm), false);
    Carver c;
    c.cur = w.attn.total;
    const size_t es = elem_size(dm->dtype), T = (size_t)j->total, HD = (size_t)dm->heads * dm->d_qk;
    w.z = c.take(T * 4 * HD * es);
    w.g = c.take(T * HD * es);
    w.total = c.cur;
    return w;
}

// Workspace of hstu_layer_bwd: the attention's (the forward and the backward
// share it, one after the other), then f1's pre-activation Z and output
// phi1(Z) [T][4Hd], O (fp32 [T][Hd]) and the LayerNorm stats, G and dG
// [T][Hd], the gradient at f1's output [T][4Hd] (dU | dV | dQ | dK, then dZ
// in place), W1^T [D][4Hd], W2^T [Hd][D], and the fp32 partial sums of the
// weight gradients and of the column sums.
struct LayerBwdWs {
    AttnWs af, ab;
    WgradPlan p1, p2;
    size_t zpre, zact, osave, stats, g, dg, da, w1t, w2t, part, total;
};

LayerBwdWs layer_bwd_ws(const hstu_jagged *j, const hstu_dims *dm, int32_t D)
{
    LayerBwdWs w{};
    w.af = attn_ws(j, dm, fwd_tile(dm), false);
    w.ab = attn_ws(j, dm, BWD_BN, true);
    Carver c;
    c.cur = align256(w.af.total > w.ab.total ? w.af.total : w.ab.total);
    const size_t T = (size_t)j->total, HD = (size_t)dm->heads * dm->d_qk, Z4 = 4 * HD, Dz = (size_t)D;
    w.zpre = c.take(T * Z4 * 2);
    w.zact = c.take(T * Z4 * 2);
    w.osave = c.take(T * HD * 4);
    w.stats = c.take(T * 2 * 4);
    w.g = c.take(T * HD * 2);
    w.dg = c.take(T * HD * 2);
    w.da = c.take(T * Z4 * 2);
    w.w1t = c.take(Dz * Z4 * 2);
    w.w2t = c.take(HD * Dz * 2);
    w.p1 = wgrad_plan((int)Z4, D, j->total);
    w.p2 = wgrad_plan(D, (int)HD, j->total);
    size_t pe = (size_t)w.p1.splits * Z4 * Dz;
    if ((size_t)w.p2.splits * Dz * HD > pe) pe = (size_t)w.p2.splits * Dz * HD;
    const size_t pc = (size_t)colsum_blocks(j->total) * (Z4 > Dz ? Z4 : Dz);
    if (pc > pe) pe = pc;
    w.part = c.take(pe * 4);
    w.total = c.cur;
    return w;
}

hstu_status check_gemm_operand(const void *p, int64_t ld, hstu_dtype dt, const char *name)
{
    if (dt == HSTU_BF16 && ((((uintptr_t)p) & 15) != 0 || (ld % 8) != 0))
        return fail(HSTU_ERR_ARG, "%s must be 16-byte aligned with ld a multiple of 8 (bf16)", name);
    return HSTU_OK;
}

hstu_status check_layer(const hstu_layer *lay, const hstu_jagged *j, const hstu_dims *dm, int32_t D, int idx)
{
    if (!lay) return fail(HSTU_ERR_ARG, "layer %d is NULL", idx);
    if (!lay->w1 || !lay->w2) return fail(HSTU_ERR_ARG, "layer %d: w1 and w2 are required", idx);
    if (lay->phi1 != HSTU_ACT_SILU && lay->phi1 != HSTU_ACT_RELU) return fail(HSTU_ERR_ARG, "layer %d: bad phi1", idx);
    TRY(check_bias(&lay->rab, j));
    TRY(check_gemm_operand(lay->w1, D, dm->dtype, "w1"));
    TRY(check_gemm_operand(lay->w2, (int64_t)dm->heads * dm->d_qk, dm->dtype, "w2"));
    return HSTU_OK;
}

GemmArgs gemm_args(const void *A, int64_t lda, const void *W, const float *bias, void *C, int64_t ldc, bool c_f32,
                   int M, int N, int K, int epi)
{
    GemmArgs g{};
    g.A = A;
    g.lda = lda;
    g.W = W;
    g.bias = bias;
    g.C = C;
    g.ldc = ldc;
    g.c_f32 = c_f32;
    g.M = M;
    g.N = N;
    g.K = K;
    g.epi = epi;
    return g;
}

hstu_status run_gemm(const GemmArgs &g, hstu_dtype dt, const char *name, hipStream_t st)
{
    ProfScope ps(name, st);
    return launched(dt == HSTU_BF16 ? launch_gemm_bf16(g, st) : launch_gemm_f32(g, st), "GEMM kernel");
}

// M-FALCON plan: key splits so a small number of candidate tiles still fills
// the chip; at most 8 splits (16 measured 9 % slower for one user, 4 slower
// still).  Depends only on sizes known on the host.
// Workspace of hstu_layer_append: header, work list, merged offsets [U+1],
// merged times int64 [Tm] and relative times (12 B per merged token), wide
// flags, the new tokens' f1 output Z [Tn][4Hd] (bf16), their fp32 O [Tn][Hd]
// and gate G [Tn][Hd].
struct AppendWs {
    size_t header, items, moff, tsm, rel, wide, z, obuf, g, total;
    int max_items;
};

AppendWs append_ws(int U, int Th, int Tn, const hstu_dims *dm)
{
    AppendWs w{};
    Carver c;
    const size_t H = dm->heads, HD = H * dm->d_qk, Tm = (size_t)Th + Tn;
    // tiles with new positions: sum_u (ceil((n+a)/BM) - floor(n/BM)) <= Tn / BM + 2 U per head
    w.max_items = (int)(((int64_t)Tn / FWD_BM + 2 * (int64_t)U) * (int64_t)H);
    w.header = c.take(256);
    w.items = c.take((size_t)w.max_items * sizeof(int2));
    w.moff = c.take((size_t)(U + 1) * 4);
    w.tsm = c.take(Tm * 8);
    w.rel = c.take(Tm * 12);
    w.wide = c.take((size_t)U * 4);
    w.z = c.take((size_t)Tn * 4 * HD * 2);
    w.obuf = c.take((size_t)Tn * HD * 4);
    w.g = c.take((size_t)Tn * HD * 2);
    w.total = c.cur;
    return w;
}

struct MfPlan {
    int nsplit, kchunk, max_items;
};

MfPlan mf_plan(const hstu_jagged *hist, const hstu_dims *dm, int32_t M)
{
    MfPlan p{};
    const int H = dm->heads, U = hist->batch;
    const int tiles_est = (M + MF_TC - 1) / MF_TC;
    int ns = (2048 + tiles_est * H - 1) / (tiles_est * H > 0 ? tiles_est * H : 1);
    ns = ns < 1 ? 1 : (ns > 8 ? 8 : ns);
    const int64_t span = hist->total > 0 ? hist->total : 1; // no user has more history than all users together
    int64_t ch = (span + ns - 1) / ns;
    ch = (ch + 63) / 64 * 64;
    p.nsplit = ns;
    p.kchunk = (int)(ch > 0 ? ch : 64);
    // tiles <= M (one candidate per microbatch at worst) + U
    p.max_items = (int)(((int64_t)M + U) * H * ns);
    return p;
}

struct MfWs {
    size_t header, items, z, part, g, x32, x16, total;
};

MfWs mf_ws(const hstu_jagged *hist, const hstu_dims *dm, int32_t D, int32_t M)
{
    MfWs w{};
    const MfPlan p = mf_plan(hist, dm, M);
    const size_t es = elem_size(dm->dtype), HD = (size_t)dm->heads * dm->d_qk;
    Carver c;
    w.header = c.take(256);
    w.items = c.take((size_t)p.max_items * sizeof(int4));
    w.z = c.take((size_t)M * 4 * HD * es);
    w.part = c.take((size_t)p.nsplit * M * HD * 4);
    w.g = c.take((size_t)M * HD * es);
    w.x32 = c.take((size_t)M * D * 4);
    w.x16 = c.take((size_t)M * D * es);
    w.total = c.cur;
    return w;
}

} // namespace

namespace hstu_internal {

hstu_status set_error(hstu_status s, const char *msg) { return fail(s, "%s", msg); }

// The forward's validation and launch on the workspace ws of ws_bytes.
// lean: the fp32 O staging buffer is carved only when the gate needs it
// (u given and no o_save); with ws == NULL only the validation runs and the
// bytes needed go to *need.
hstu_status attn_fwd_entry(const hstu_jagged *j, const hstu_dims *dm, const hstu_bias *bias, hstu_cmat q, hstu_cmat k,
                           hstu_cmat v, hstu_cmat u, hstu_mat out, float *o_save, float *ln_stats, void *ws,
                           size_t ws_bytes, void *stream, bool lean, size_t *need)
{
    TRY(check_jagged(j));
    TRY(check_dims(dm, BF16_D32_64_128));
    TRY(check_bias(bias, j));
    const int H = dm->heads, d = dm->d_qk, F = H * dm->d_v;
    const bool rows = j->total > 0; // an empty batch has no rows to read or write: its views may be NULL
    TRY(check_view(q.ptr, q.ld, (int64_t)H * d, "q", rows));
    TRY(check_view(k.ptr, k.ld, (int64_t)H * d, "k", rows));
    TRY(check_view(v.ptr, v.ld, (int64_t)F, "v", rows));
    TRY(check_view(u.ptr, u.ld, (int64_t)F, "u", false));
    TRY(check_view(out.ptr, out.ld, (int64_t)F, "out", rows));
    if (ln_stats && !u.ptr && rows) return fail(HSTU_ERR_ARG, "ln_stats requires u (the epilogue)");
    if (dm->dtype == HSTU_BF16) {
        TRY(check_vec_view(q.ptr, q.ld, HSTU_BF16, "q"));
        TRY(check_vec_view(k.ptr, k.ld, HSTU_BF16, "k"));
        TRY(check_vec_view(v.ptr, v.ld, HSTU_BF16, "v"));
        TRY(check_vec_view(u.ptr, u.ld, HSTU_BF16, "u"));
        TRY(check_vec_view(out.ptr, out.ld, HSTU_BF16, "out"));
        TRY(check_vec_view(o_save, F, HSTU_F32, "o_save"));
    }
    const AttnWs w = attn_ws(j, dm, fwd_tile(dm), false, !lean || (u.ptr && !o_save));
    if (need) *need = w.total;
    if (!ws && need) return ok();
    TRY(check_ws(ws, ws_bytes, w.total));
    hipStream_t st = (hipStream_t)stream;
    TRY(attn_fwd_launch(j, dm, bias, q, k, v, u, out, o_save, ln_stats, (char *)ws, w, st));
    TRY(debug_check(ws, st));
    return ok();
}

} // namespace hstu_internal

extern "C" {

int32_t hstu_abi_version(void) { return HSTU_ABI_VERSION; }

const char *hstu_last_error(void) { return g_err.c_str(); }

size_t hstu_workspace_size(hstu_op op, const hstu_jagged *j, const hstu_dims *dims, int32_t d_model,
                           int32_t total_cand)
{
    const bool attn_op = op == HSTU_OP_ATTN_FWD || op == HSTU_OP_ATTN_BWD;
    if (check_jagged(j) != HSTU_OK || check_dims(dims, attn_op ? BF16_D32_64_128 : BF16_D128) != HSTU_OK)
        return 0;
    switch (op) {
    case HSTU_OP_ATTN_FWD: return attn_ws(j, dims, fwd_tile(dims), false).total;
    case HSTU_OP_ATTN_BWD: return attn_ws(j, dims, BWD_BN, true).total;
    case HSTU_OP_LAYER_FWD: return layer_ws(j, dims).total;
    case HSTU_OP_LAYER_BWD:
        if (d_model < 1) {
            fail(HSTU_ERR_ARG, "d_model must be >= 1");
            return 0;
        }
        return layer_bwd_ws(j, dims, d_model).total;
    case HSTU_OP_LAYER_APPEND:
        if (d_model < 1 || total_cand < 0) {
            fail(HSTU_ERR_ARG, "d_model must be >= 1 and the new actions' total (total_cand) >= 0");
            return 0;
        }
        return append_ws(j->batch, j->total, total_cand, dims).total;
    case HSTU_OP_MFALCON:
        if (d_model < 1 || total_cand < 0) {
            fail(HSTU_ERR_ARG, "d_model must be >= 1 and total_cand >= 0");
            return 0;
        }
        return mf_ws(j, dims, d_model, total_cand).total;
    default: break;
    }
    fail(HSTU_ERR_ARG, "unknown op %d", (int)op);
    return 0;
}

hstu_status hstu_attn_fwd(const hstu_jagged *j, const hstu_dims *dm, const hstu_bias *bias, hstu_cmat q, hstu_cmat k,
                          hstu_cmat v, hstu_cmat u, hstu_mat out, float *o_save, float *ln_stats, void *ws,
                          size_t ws_bytes, void *stream)
{
    return hstu_internal::attn_fwd_entry(j, dm, bias, q, k, v, u, out, o_save, ln_stats, ws, ws_bytes, stream, false,
                                         nullptr);
}

hstu_status hstu_sl_sample(const hstu_jagged *in, double alpha, const double *u, const uint32_t *keys, const void *x,
                           int64_t ldx, int32_t row_bytes, int32_t *out_offsets, int32_t *out_index, void *x_out,
                           int64_t ldx_out, int64_t *ts_out, void *ws, size_t ws_bytes, void *stream)
{
    TRY(check_jagged(in));
    if (!(alpha > 0.0)) return fail(HSTU_ERR_ARG, "alpha must be > 0");
    if (!u || !keys) return fail(HSTU_ERR_ARG, "u and keys are required");
    if (!out_offsets || !out_index) return fail(HSTU_ERR_ARG, "out_offsets and out_index are required");
    if (x) {
        if (!x_out) return fail(HSTU_ERR_ARG, "x_out is required with x");
        if (row_bytes < 1) return fail(HSTU_ERR_ARG, "row_bytes must be >= 1");
        if (ldx < row_bytes || ldx_out < row_bytes) return fail(HSTU_ERR_ARG, "ldx and ldx_out must be >= row_bytes");
    }
    if (ts_out && !in->ts) return fail(HSTU_ERR_ARG, "ts_out needs in->ts");
    TRY(check_ws(ws, ws_bytes, 256));
    SlArgs a{};
    a.offsets = in->offsets;
    a.B = in->batch;
    a.T = in->total;
    a.alpha = alpha;
    a.u = u;
    a.keys = keys;
    a.out_off = out_offsets;
    a.out_idx = out_index;
    a.x = x;
    a.ldx_bytes = ldx;
    a.y = x_out;
    a.ldy_bytes = ldx_out;
    a.row_bytes = row_bytes;
    a.ts = in->ts;
    a.ts_out = ts_out;
    a.status = (int *)ws;
    hipStream_t st = (hipStream_t)stream;
    {
        ProfScope ps("sl_sample_kernels", st);
        TRY(launched(launch_sl_sample(a, st), "Stochastic Length kernels"));
    }
    TRY(debug_check(ws, st));
    return ok();
}

hstu_status hstu_softmax_attn_fwd(const hstu_jagged *j, const hstu_dims *dm, hstu_cmat q, hstu_cmat k, hstu_cmat v,
                                  hstu_mat out, float *lse, void *ws, size_t ws_bytes, void *stream)
{
    TRY(check_jagged(j));
    TRY(check_dims(dm, BF16_D32_64_128));
    if (dm->dtype != HSTU_BF16) return fail(HSTU_ERR_UNSUPPORTED, "hstu_softmax_attn_fwd supports bf16 storage only");
    const int H = dm->heads, d = dm->d_qk, F = H * dm->d_v;
    const struct { const void *p; int64_t ld; int64_t w; const char *n; } views[] = {
        {q.ptr, q.ld, (int64_t)H * d, "q"}, {k.ptr, k.ld, (int64_t)H * d, "k"}, {v.ptr, v.ld, F, "v"},
        {out.ptr, out.ld, F, "out"}};
    for (const auto &x : views) {
        TRY(check_view(x.p, x.ld, x.w, x.n));
        TRY(check_vec_view(x.p, x.ld, HSTU_BF16, x.n));
    }
    const AttnWs w = attn_ws(j, dm, FWD_BM, false, false);
    TRY(check_ws(ws, ws_bytes, w.total));
    hipStream_t st = (hipStream_t)stream;
    char *wb = (char *)ws;
    int *status = (int *)(wb + w.header), *n_items = status + 1;
    int2 *items = (int2 *)(wb + w.items);
    const int T = j->total, B = j->batch;
    const int max_items = max_items_for(B, T, FWD_BM, H);
    {
        ProfScope ps("sched_kernel", st);
        launch_sched(j->offsets, nullptr, B, T, FWD_BM, H, status, n_items, items, max_items, (uint32_t *)(wb + w.rel),
                     (int32_t *)(wb + w.wide), (int32_t *)(wb + w.rank), 0, nullptr, SchedBwd{}, st);
    }
    TRY(launched(hipGetLastError(), "schedule kernel"));
    AttnFwdArgs a{};
    a.q = q.ptr;
    a.k = k.ptr;
    a.v = v.ptr;
    a.ldq = q.ld;
    a.ldk = k.ld;
    a.ldv = v.ld;
    a.offsets = j->offsets;
    a.wide = (int32_t *)(wb + w.wide);
    a.H = H;
    a.N = j->n_max;
    a.d = d;
    a.items = items;
    a.n_items = n_items;
    a.o16 = out.ptr;
    a.ld_o16 = out.ld;
    a.lse = lse;
    {
        ProfScope ps("attn_softmax_fwd_kernel", st);
        TRY(launched(launch_attn_softmax_fwd(a, max_items, st), "softmax attention kernel"));
    }
    TRY(debug_check(ws, st));
    return ok();
}

hstu_status hstu_attn_bwd(const hstu_jagged *j, const hstu_dims *dm, const hstu_bias *bias, hstu_cmat q, hstu_cmat k,
                          hstu_cmat v, hstu_cmat u, const float *o_save, const float *ln_stats, hstu_cmat dout,
                          hstu_mat dq, hstu_mat dk, hstu_mat dv, hstu_mat du, float *drab_p, float *drab_t, void *ws,
                          size_t ws_bytes, void *stream)
{
    TRY(check_jagged(j));
    TRY(check_dims(dm, BF16_D32_64_128));
    TRY(check_bias(bias, j));
    if (dm->dtype != HSTU_BF16) return fail(HSTU_ERR_UNSUPPORTED, "hstu_attn_bwd supports bf16 storage only");
    const int H = dm->heads, d = dm->d_qk, F = H * dm->d_v;
    const bool rows = j->total > 0; // an empty batch has no rows to read or write: its views may be NULL
    TRY(check_view(q.ptr, q.ld, (int64_t)H * d, "q", rows));
    TRY(check_view(k.ptr, k.ld, (int64_t)H * d, "k", rows));
    TRY(check_view(v.ptr, v.ld, (int64_t)F, "v", rows));
    TRY(check_view(dout.ptr, dout.ld, (int64_t)F, "dout", rows));
    TRY(check_view(dq.ptr, dq.ld, (int64_t)H * d, "dq", rows));
    TRY(check_view(dk.ptr, dk.ld, (int64_t)H * d, "dk", rows));
    TRY(check_view(dv.ptr, dv.ld, (int64_t)F, "dv", rows));
    if (u.ptr) {
        TRY(check_view(u.ptr, u.ld, (int64_t)F, "u"));
        TRY(check_view(du.ptr, du.ld, (int64_t)F, "du", rows));
        if (rows && (!o_save || !ln_stats))
            return fail(HSTU_ERR_ARG, "with u, o_save and ln_stats from the forward are required");
    }
    {
        const struct { const void *p; int64_t ld; const char *n; } views[] = {
            {q.ptr, q.ld, "q"}, {k.ptr, k.ld, "k"}, {v.ptr, v.ld, "v"}, {u.ptr, u.ld, "u"}, {dout.ptr, dout.ld, "dout"},
            {dq.ptr, dq.ld, "dq"}, {dk.ptr, dk.ld, "dk"}, {dv.ptr, dv.ld, "dv"}, {du.ptr, du.ld, "du"}};
        for (const auto &x : views) TRY(check_vec_view(x.p, x.ld, HSTU_BF16, x.n));
        TRY(check_vec_view(o_save, F, HSTU_F32, "o_save"));
    }
    const bool has_p = bias && bias->rab_p;
    const bool has_t = bias && bias->rab_t && j->ts;
    if (drab_p && has_p && bias->rab_p_hstride == 0)
        return fail(HSTU_ERR_ARG, "drab_p needs a per-head rab_p (hstride != 0)");
    if (drab_t && has_t && bias->rab_t_hstride == 0)
        return fail(HSTU_ERR_ARG, "drab_t needs a per-head rab_t (hstride != 0)");
    const AttnWs w = attn_ws(j, dm, BWD_BN, true);
    TRY(check_ws(ws, ws_bytes, w.total));
    hipStream_t st = (hipStream_t)stream;
    char *wb = (char *)ws;
    TRY(attn_bwd_launch(j, dm, bias, q, k, v, u, o_save, ln_stats, dout, dq, dk, dv, du, drab_p, drab_t, wb, w, st));
    TRY(debug_check(ws, st));
    return ok();
}

hstu_status hstu_layer_fwd(const hstu_jagged *j, const hstu_dims *dm, int32_t d_model, const hstu_layer *layer,
                           hstu_cmat x, hstu_mat y, hstu_mat k_cache, hstu_mat v_cache, void *ws, size_t ws_bytes,
                           void *stream)
{
    TRY(check_jagged(j));
    TRY(check_dims(dm));
    if (d_model < 1) return fail(HSTU_ERR_ARG, "d_model must be >= 1");
    TRY(check_layer(layer, j, dm, d_model, 0));
    const int H = dm->heads, d = dm->d_qk, HD = H * d, D = d_model;
    TRY(check_view(x.ptr, x.ld, D, "x"));
    TRY(check_view(y.ptr, y.ld, D, "y"));
    TRY(check_gemm_operand(x.ptr, x.ld, dm->dtype, "x"));
    TRY(check_view(k_cache.ptr, k_cache.ld, HD, "k_cache", false));
    TRY(check_view(v_cache.ptr, v_cache.ld, HD, "v_cache", false));
    if (x.ptr == y.ptr) return fail(HSTU_ERR_ARG, "y may not alias x");
    const LayerWs w = layer_ws(j, dm);
    TRY(check_ws(ws, ws_bytes, w.total));
    hipStream_t st = (hipStream_t)stream;
    char *wb = (char *)ws;
    const int T = j->total;
    const hstu_dtype dt = dm->dtype;
    const size_t es = elem_size(dt);
    char *Z = wb + w.z, *G = wb + w.g;
    // f1 + phi1 -> Z = U | V | Q | K, and this layer's K, V into the cache
    GemmArgs g1 = gemm_args(x.ptr, x.ld, layer->w1, layer->b1, Z, 4 * HD, dt == HSTU_F32, T, 4 * HD, D,
                            layer->phi1 == HSTU_ACT_RELU ? EPI_RELU : EPI_SILU);
    g1.Ck = k_cache.ptr;
    g1.ldck = k_cache.ld;
    g1.k_lo = 3 * HD;
    g1.Cv = v_cache.ptr;
    g1.ldcv = v_cache.ld;
    g1.v_lo = HD;
    g1.kv_w = HD;
    TRY(run_gemm(g1, dt, "gemm_f1", st));
    // attention + LayerNorm(O) (.) U on views of Z
    hstu_cmat zu{Z, 4 * HD}, zv{Z + (size_t)HD * es, 4 * HD}, zq{Z + (size_t)2 * HD * es, 4 * HD},
        zk{Z + (size_t)3 * HD * es, 4 * HD};
    hstu_mat gm{G, HD};
    TRY(attn_fwd_launch(j, dm, &layer->rab, zq, zk, zv, zu, gm, nullptr, nullptr, wb, w.attn, st));
    // y = x + G W2^T + b2
    GemmArgs g2 = gemm_args(G, HD, layer->w2, layer->b2, y.ptr, y.ld, dt == HSTU_F32, T, D, HD, EPI_NONE);
    g2.R16 = x.ptr;
    g2.ldr = x.ld;
    TRY(run_gemm(g2, dt, "gemm_f2", st));
    TRY(debug_check(ws, st));
    return ok();
}

hstu_status hstu_layer_bwd(const hstu_jagged *j, const hstu_dims *dm, int32_t d_model, const hstu_layer *layer,
                           hstu_cmat x, hstu_cmat dy, hstu_mat dx, float *dw1, float *db1, float *dw2, float *db2,
                           float *drab_p, float *drab_t, void *ws, size_t ws_bytes, void *stream)
{
    TRY(check_jagged(j));
    TRY(check_dims(dm));
    if (dm->dtype != HSTU_BF16) return fail(HSTU_ERR_UNSUPPORTED, "hstu_layer_bwd supports bf16 storage only");
    if (d_model < 8 || d_model % 8 != 0)
        return fail(HSTU_ERR_UNSUPPORTED, "hstu_layer_bwd needs d_model a multiple of 8 (got %d)", d_model);
    TRY(check_layer(layer, j, dm, d_model, 0));
    const int H = dm->heads, d = dm->d_qk, HD = H * d, Z4 = 4 * HD, D = d_model;
    TRY(check_view(x.ptr, x.ld, D, "x"));
    TRY(check_view(dy.ptr, dy.ld, D, "dy"));
    TRY(check_view(dx.ptr, dx.ld, D, "dx"));
    TRY(check_gemm_operand(x.ptr, x.ld, dm->dtype, "x"));
    TRY(check_gemm_operand(dy.ptr, dy.ld, dm->dtype, "dy"));
    if (dx.ptr == x.ptr || dx.ptr == dy.ptr) return fail(HSTU_ERR_ARG, "dx may not alias x or dy");
    if (!dw1 || !dw2) return fail(HSTU_ERR_ARG, "dw1 and dw2 are required");
    const float *f32out[4] = {dw1, dw2, db1, db2};
    for (const float *p : f32out)
        if (p && ((uintptr_t)p & 15) != 0) return fail(HSTU_ERR_ARG, "dw1, dw2, db1, db2 must be 16-byte aligned");
    const hstu_bias *bias = &layer->rab;
    if (drab_p && bias->rab_p && bias->rab_p_hstride == 0)
        return fail(HSTU_ERR_ARG, "drab_p needs a per-head rab_p (hstride != 0)");
    if (drab_t && bias->rab_t && j->ts && bias->rab_t_hstride == 0)
        return fail(HSTU_ERR_ARG, "drab_t needs a per-head rab_t (hstride != 0)");
    const LayerBwdWs w = layer_bwd_ws(j, dm, D);
    TRY(check_ws(ws, ws_bytes, w.total));
    hipStream_t st = (hipStream_t)stream;
    char *wb = (char *)ws;
    const int T = j->total;
    bf16 *Zpre = (bf16 *)(wb + w.zpre), *Zact = (bf16 *)(wb + w.zact), *G = (bf16 *)(wb + w.g);
    bf16 *dG = (bf16 *)(wb + w.dg), *dA = (bf16 *)(wb + w.da), *W1t = (bf16 *)(wb + w.w1t);
    bf16 *W2t = (bf16 *)(wb + w.w2t);
    float *osave = (float *)(wb + w.osave), *stats = (float *)(wb + w.stats), *part = (float *)(wb + w.part);
    const int act = layer->phi1 == HSTU_ACT_RELU ? 2 : 1;

    // forward again: Z and phi1(Z) = U | V | Q | K, then G = Norm(O) (.) U
    // with O and the LayerNorm statistics kept
    GemmArgs g1 = gemm_args(x.ptr, x.ld, layer->w1, layer->b1, Zact, Z4, false, T, Z4, D,
                            act == 2 ? EPI_RELU : EPI_SILU);
    g1.Cpre = Zpre;
    g1.ldcpre = Z4;
    TRY(run_gemm(g1, dm->dtype, "gemm_f1", st));
    hstu_cmat zu{Zact, Z4}, zv{Zact + HD, Z4}, zq{Zact + 2 * HD, Z4}, zk{Zact + 3 * HD, Z4};
    TRY(attn_fwd_launch(j, dm, bias, zq, zk, zv, zu, hstu_mat{G, HD}, osave, stats, wb, w.af, st));
    {
        ProfScope ps("transpose_bf16_kernel", st);
        TRY(launched(launch_transpose_bf16((const bf16 *)layer->w2, HD, D, HD, W2t, D, st), "transpose kernel"));
        TRY(launched(launch_transpose_bf16((const bf16 *)layer->w1, D, Z4, D, W1t, Z4, st), "transpose kernel"));
    }
    // f2: dG = dY W2, dW2 = dY^T G, db2 = column sums of dY
    TRY(run_gemm(gemm_args(dy.ptr, dy.ld, W2t, nullptr, dG, HD, false, T, HD, D, EPI_NONE), dm->dtype, "gemm_dg", st));
    {
        WgradArgs a{dy.ptr, dy.ld, G, HD, part, D, HD, T, w.p2.chunk, w.p2.splits};
        {
            ProfScope ps("gemm_wgrad_w2", st);
            TRY(launched(launch_gemm_wgrad(a, st), "weight-gradient kernel"));
        }
        ProfScope ps("sum_splits_kernel", st);
        TRY(launched(launch_sum_splits(part, w.p2.splits, (int64_t)D * HD, dw2, st), "split-sum kernel"));
    }
    if (db2) {
        {
            ProfScope ps("colsum_act_kernel", st);
            TRY(launched(launch_colsum_act((bf16 *)dy.ptr, dy.ld, nullptr, 0, 0, T, D, part, st), "column-sum kernel"));
        }
        ProfScope ps("sum_splits_kernel", st);
        TRY(launched(launch_sum_splits(part, colsum_blocks(T), D, db2, st), "split-sum kernel"));
    }
    // gate and attention: dU | dV | dQ | dK into dA, and the table gradients
    TRY(attn_bwd_launch(j, dm, bias, zq, zk, zv, zu, osave, stats, hstu_cmat{dG, HD}, hstu_mat{dA + 2 * HD, Z4},
                        hstu_mat{dA + 3 * HD, Z4}, hstu_mat{dA + HD, Z4}, hstu_mat{dA, Z4}, drab_p, drab_t, wb, w.ab,
                        st));
    // phi1: dZ = dA (.) phi1'(Z) in place, db1 = its column sums
    {
        ProfScope ps("colsum_act_kernel", st);
        TRY(launched(launch_colsum_act(dA, Z4, Zpre, Z4, act, T, Z4, part, st), "phi1 backward kernel"));
    }
    if (db1) {
        ProfScope ps("sum_splits_kernel", st);
        TRY(launched(launch_sum_splits(part, colsum_blocks(T), Z4, db1, st), "split-sum kernel"));
    }
    // f1 and the residual: dX = dY + dZ W1, dW1 = dZ^T X
    {
        GemmArgs gx = gemm_args(dA, Z4, W1t, nullptr, dx.ptr, dx.ld, false, T, D, Z4, EPI_NONE);
        gx.R16 = dy.ptr;
        gx.ldr = dy.ld;
        TRY(run_gemm(gx, dm->dtype, "gemm_dx", st));
    }
    {
        WgradArgs a{dA, Z4, x.ptr, x.ld, part, Z4, D, T, w.p1.chunk, w.p1.splits};
        {
            ProfScope ps("gemm_wgrad_w1", st);
            TRY(launched(launch_gemm_wgrad(a, st), "weight-gradient kernel"));
        }
        ProfScope ps("sum_splits_kernel", st);
        TRY(launched(launch_sum_splits(part, w.p1.splits, (int64_t)Z4 * D, dw1, st), "split-sum kernel"));
    }
    TRY(debug_check(ws, st));
    return ok();
}

hstu_status hstu_layer_append(const hstu_jagged *hist, const hstu_jagged *add, const hstu_dims *dm, int32_t d_model,
                              const hstu_layer *layer, hstu_cmat k_cache, hstu_cmat v_cache, hstu_cmat x_new,
                              hstu_mat y_new, hstu_mat k_out, hstu_mat v_out, void *ws, size_t ws_bytes, void *stream)
{
    TRY(check_jagged(hist));
    if (!add) return fail(HSTU_ERR_ARG, "add (the new actions) is NULL");
    if (add->batch != hist->batch)
        return fail(HSTU_ERR_ARG, "add->batch (%d) != hist->batch (%d)", add->batch, hist->batch);
    if (add->total < 0) return fail(HSTU_ERR_ARG, "add->total must be >= 0");
    if (!add->offsets) return fail(HSTU_ERR_ARG, "add->offsets is NULL");
    if ((hist->ts == nullptr) != (add->ts == nullptr))
        return fail(HSTU_ERR_ARG, "history and new-action timestamps must both be given or both be NULL");
    if ((int64_t)hist->total + add->total > INT32_MAX / 16)
        return fail(HSTU_ERR_UNSUPPORTED, "history plus new actions: too many tokens");
    TRY(check_dims(dm));
    if (dm->dtype != HSTU_BF16) return fail(HSTU_ERR_UNSUPPORTED, "hstu_layer_append supports bf16 storage only");
    if (d_model < 1) return fail(HSTU_ERR_ARG, "d_model must be >= 1");
    TRY(check_layer(layer, hist, dm, d_model, 0));
    const int H = dm->heads, d = dm->d_qk, HD = H * d, D = d_model, U = hist->batch;
    const int Th = hist->total, Tn = add->total;
    TRY(check_view(x_new.ptr, x_new.ld, D, "x_new"));
    TRY(check_view(y_new.ptr, y_new.ld, D, "y_new"));
    TRY(check_gemm_operand(x_new.ptr, x_new.ld, dm->dtype, "x_new"));
    if (x_new.ptr == y_new.ptr) return fail(HSTU_ERR_ARG, "y_new may not alias x_new");
    const struct { const void *p; int64_t ld; const char *n; } views[] = {
        {k_cache.ptr, k_cache.ld, "k_cache"}, {v_cache.ptr, v_cache.ld, "v_cache"},
        {k_out.ptr, k_out.ld, "k_out"}, {v_out.ptr, v_out.ld, "v_out"}};
    for (const auto &x : views) {
        TRY(check_view(x.p, x.ld, HD, x.n, !(Th == 0 && (x.p == k_cache.ptr || x.p == v_cache.ptr))));
        TRY(check_vec_view(x.p, x.ld, HSTU_BF16, x.n));
    }
    if (k_out.ptr == k_cache.ptr || k_out.ptr == v_cache.ptr || v_out.ptr == k_cache.ptr ||
        v_out.ptr == v_cache.ptr || k_out.ptr == v_out.ptr)
        return fail(HSTU_ERR_ARG, "k_out and v_out may not alias each other or the caches they are built from");
    const AppendWs w = append_ws(U, Th, Tn, dm);
    TRY(check_ws(ws, ws_bytes, w.total));
    hipStream_t st = (hipStream_t)stream;
    char *wb = (char *)ws;
    int *status = (int *)(wb + w.header), *n_items = status + 1;
    int2 *items = (int2 *)(wb + w.items);
    int32_t *moff = (int32_t *)(wb + w.moff);
    int64_t *ts_m = (int64_t *)(wb + w.tsm);
    uint32_t *rel = (uint32_t *)(wb + w.rel);
    int32_t *wide = (int32_t *)(wb + w.wide);
    bf16 *Z = (bf16 *)(wb + w.z), *G = (bf16 *)(wb + w.g);
    float *obuf = (float *)(wb + w.obuf);
    const int Tm = Th + Tn;
    const bool use_t = hist->ts != nullptr && layer->rab.rab_t != nullptr;
    // f1 + phi1 of the new tokens: Z = U | V | Q | K
    if (Tn > 0) {
        GemmArgs g1 = gemm_args(x_new.ptr, x_new.ld, layer->w1, layer->b1, Z, 4 * HD, false, Tn, 4 * HD, D,
                                layer->phi1 == HSTU_ACT_RELU ? EPI_RELU : EPI_SILU);
        TRY(run_gemm(g1, dm->dtype, "gemm_f1", st));
    }
    // validate, merged offsets and work list; the merged caches and times
    {
        AppendPlan p{};
        p.hoff = hist->offsets;
        p.aoff = add->offsets;
        p.U = U;
        p.Th = Th;
        p.Tn = Tn;
        p.H = H;
        p.tile = FWD_BM;
        p.max_items = w.max_items;
        p.status = status;
        p.n_items = n_items;
        p.items = items;
        p.moff = moff;
        p.kc = (const bf16 *)k_cache.ptr;
        p.vc = (const bf16 *)v_cache.ptr;
        p.ldkc = k_cache.ld;
        p.ldvc = v_cache.ld;
        p.knew = Z + 3 * HD;
        p.vnew = Z + HD;
        p.ldnew = 4 * HD;
        p.kout = (bf16 *)k_out.ptr;
        p.vout = (bf16 *)v_out.ptr;
        p.ldko = k_out.ld;
        p.ldvo = v_out.ld;
        p.hd = HD;
        p.ts_h = use_t ? hist->ts : nullptr;
        p.ts_a = use_t ? add->ts : nullptr;
        p.ts_m = use_t ? ts_m : nullptr;
        p.rel = rel;
        p.wide = wide;
        ProfScope ps("append_plan_kernel", st);
        TRY(launched(launch_append_plan(p, st), "append plan kernels"));
    }
    // attention of the new positions over [history; new]
    AttnFwdArgs a{};
    a.q = Z + 2 * HD;
    a.ldq = 4 * HD;
    a.k = k_out.ptr;
    a.v = v_out.ptr;
    a.ldk = k_out.ld;
    a.ldv = v_out.ld;
    a.offsets = moff;
    a.ts = use_t ? ts_m : nullptr;
    a.rel = rel;
    a.wide = wide;
    a.rmin = rel + Tm;
    a.rmax = rel + 2 * (size_t)Tm;
    a.rab_p = layer->rab.rab_p;
    a.rp_hs = layer->rab.rab_p_hstride;
    a.rab_t = use_t ? layer->rab.rab_t : nullptr;
    a.rt_hs = layer->rab.rab_t_hstride;
    a.H = H;
    a.N = hist->n_max;
    a.d = d;
    a.inv_n = 1.0f / (float)hist->n_max;
    a.items = items;
    a.n_items = n_items;
    a.o32 = obuf;
    a.ld_o32 = HD;
    a.o16 = nullptr;
    a.hoff = hist->offsets;
    a.aoff = add->offsets;
    {
        ProfScope ps("attn_fwd_bf16_kernel", st);
        TRY(launched(launch_attn_fwd_bf16(a, w.max_items, st), "attention forward kernel"));
    }
    if (Tn > 0) {
        {
            ProfScope ps("ln_gate_fwd_kernel", st);
            TRY(launched(launch_ln_gate_fwd(obuf, HD, 1, 0, Z, 4 * HD, true, G, HD, nullptr, nullptr, 0, Tn, HD,
                                            dm->ln_eps, status, st),
                         "LayerNorm gate kernel"));
        }
        GemmArgs g2 = gemm_args(G, HD, layer->w2, layer->b2, y_new.ptr, y_new.ld, false, Tn, D, HD, EPI_NONE);
        g2.R16 = x_new.ptr;
        g2.ldr = x_new.ld;
        TRY(run_gemm(g2, dm->dtype, "gemm_f2", st));
    }
    TRY(debug_check(ws, st));
    return ok();
}

hstu_status mfalcon_score(const hstu_jagged *hist, const hstu_dims *dm, int32_t d_model, int32_t n_layers,
                          const hstu_layer *layers, const hstu_cmat *k_cache, const hstu_cmat *v_cache,
                          const int32_t *cand_offsets, int32_t total_cand, const int64_t *cand_ts, hstu_cmat x_cand,
                          int32_t b_m, float *y_cand, void *ws, size_t ws_bytes, void *stream)
{
    TRY(check_jagged(hist));
    TRY(check_dims(dm));
    if (d_model < 1) return fail(HSTU_ERR_ARG, "d_model must be >= 1");
    if (n_layers < 1) return fail(HSTU_ERR_ARG, "n_layers must be >= 1");
    if (!layers || !k_cache || !v_cache) return fail(HSTU_ERR_ARG, "layers, k_cache and v_cache arrays are required");
    if (!cand_offsets) return fail(HSTU_ERR_ARG, "cand_offsets is NULL");
    if (total_cand < 0) return fail(HSTU_ERR_ARG, "total_cand must be >= 0");
    if (b_m < 1) return fail(HSTU_ERR_ARG, "b_m must be >= 1 (got %d)", b_m);
    if (!y_cand) return fail(HSTU_ERR_ARG, "y_cand is NULL");
    if ((hist->ts == nullptr) != (cand_ts == nullptr))
        return fail(HSTU_ERR_ARG, "history ts and cand_ts must both be given or both be NULL");
    if (dm->heads > 32) return fail(HSTU_ERR_UNSUPPORTED, "M-FALCON supports at most 32 heads");
    const int H = dm->heads, d = dm->d_qk, HD = H * d, D = d_model, M = total_cand;
    TRY(check_view(x_cand.ptr, x_cand.ld, D, "x_cand"));
    TRY(check_gemm_operand(x_cand.ptr, x_cand.ld, dm->dtype, "x_cand"));
    for (int l = 0; l < n_layers; l++) {
        TRY(check_layer(&layers[l], hist, dm, D, l));
        TRY(check_view(k_cache[l].ptr, k_cache[l].ld, HD, "k_cache[l]"));
        TRY(check_view(v_cache[l].ptr, v_cache[l].ld, HD, "v_cache[l]"));
        TRY(check_vec_view(k_cache[l].ptr, k_cache[l].ld, dm->dtype, "k_cache[l]"));
        TRY(check_vec_view(v_cache[l].ptr, v_cache[l].ld, dm->dtype, "v_cache[l]"));
    }
    const MfWs w = mf_ws(hist, dm, D, M);
    const MfPlan p = mf_plan(hist, dm, M);
    TRY(check_ws(ws, ws_bytes, w.total));
    hipStream_t st = (hipStream_t)stream;
    char *wb = (char *)ws;
    int *status = (int *)(wb + w.header), *n_items = status + 1;
    int4 *items = (int4 *)(wb + w.items);
    const hstu_dtype dt = dm->dtype;
    const size_t es = elem_size(dt);
    char *Z = wb + w.z, *G = wb + w.g, *x16 = wb + w.x16;
    float *part = (float *)(wb + w.part), *x32 = (float *)(wb + w.x32);
    {
        ProfScope ps("mfalcon_sched_kernel", st);
        TRY(launched(launch_mfalcon_sched(hist->offsets, cand_offsets, hist->batch, M, H, b_m, p.nsplit, items,
                                          n_items, status, p.max_items, hist->total, st),
                     "M-FALCON schedule kernel"));
    }
    for (int l = 0; l < n_layers; l++) {
        const hstu_layer &lay = layers[l];
        const bool last = l == n_layers - 1;
        // candidate f1 + phi1 -> Z = U | V | Q | K
        GemmArgs g1 = gemm_args(l == 0 ? x_cand.ptr : (const void *)x16, l == 0 ? x_cand.ld : D, lay.w1, lay.b1, Z,
                                4 * HD, dt == HSTU_F32, M, 4 * HD, D,
                                lay.phi1 == HSTU_ACT_RELU ? EPI_RELU : EPI_SILU);
        TRY(run_gemm(g1, dt, "gemm_f1", st));
        // history part of the attention, one partial sum per key split
        MfalconArgs a{};
        a.q = Z + (size_t)2 * HD * es;
        a.ldz = 4 * HD;
        a.kc = k_cache[l].ptr;
        a.vc = v_cache[l].ptr;
        a.ldkc = k_cache[l].ld;
        a.ldvc = v_cache[l].ld;
        a.hoff = hist->offsets;
        a.hts = (lay.rab.rab_t && hist->ts) ? hist->ts : nullptr;
        a.cts = (lay.rab.rab_t && hist->ts) ? cand_ts : nullptr;
        a.rab_p = lay.rab.rab_p;
        a.rp_hs = lay.rab.rab_p_hstride;
        a.rab_t = lay.rab.rab_t;
        a.rt_hs = lay.rab.rab_t_hstride;
        a.H = H;
        a.N = hist->n_max;
        a.M = M;
        a.d = d;
        a.kchunk = p.kchunk;
        a.items = items;
        a.n_items = n_items;
        a.part = part;
        {
            ProfScope ps("mfalcon_attn_kernel", st);
            TRY(launched(launch_mfalcon_attn(a, p.max_items, dt == HSTU_BF16, st), "M-FALCON attention kernel"));
        }
        {
            ProfScope ps("mfalcon_epilogue_kernel", st);
            TRY(launched(launch_mfalcon_epilogue(part, p.nsplit, Z, 4 * HD, lay.rab.rab_p, lay.rab.rab_p_hstride,
                                                 lay.rab.rab_t, lay.rab.rab_t_hstride,
                                                 lay.rab.rab_t != nullptr && hist->ts != nullptr, hist->n_max,
                                                 dm->ln_eps, G, HD, M, H, d, dt == HSTU_BF16, st),
                         "M-FALCON epilogue kernel"));
        }
        // x = x + G W2^T + b2 in fp32; a storage-dtype copy feeds the next layer
        GemmArgs g2 = gemm_args(G, HD, lay.w2, lay.b2, last ? (void *)y_cand : (void *)x32, D, true, M, D, HD,
                                EPI_NONE);
        if (l == 0) {
            g2.R16 = x_cand.ptr;
            g2.ldr = x_cand.ld;
        } else {
            g2.R32 = x32;
            g2.ldr = D;
        }
        if (!last) {
            g2.C16 = x16;
            g2.ldc16 = D;
        }
        TRY(run_gemm(g2, dt, "gemm_f2", st));
    }
    TRY(debug_check(ws, st));
    return ok();
}

} // extern "C"
