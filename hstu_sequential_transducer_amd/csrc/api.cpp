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

bool debug_mode()
{
    static int v = -1;
    if (v < 0) {
        const char *e = getenv("HSTU_DEBUG");
        v = (e && e[0] == '1') ? 1 : 0;
    }
    return v == 1;
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
    size_t header, items, rel, wide, obuf, dq, dO, total;
};

AttnWs attn_ws(const hstu_jagged *j, const hstu_dims *dm, int tile)
{
    AttnWs w{};
    Carver c;
    const int B = j->batch, T = j->total, H = dm->heads;
    w.header = c.take(256);
    w.items = c.take((size_t)max_items_for(B, T, tile, H) * sizeof(int2));
    w.rel = c.take((size_t)T * 4);
    w.wide = c.take((size_t)B * 4);
    w.obuf = c.take((size_t)T * H * dm->d_v * 4);
    w.dq = c.take((size_t)T * H * dm->d_qk * 4);
    w.dO = c.take((size_t)T * H * dm->d_v * 2 * 2); // hi and lo bf16 planes
    w.total = c.cur;
    return w;
}

int fwd_tile(const hstu_dims *dm) { return dm->dtype == HSTU_BF16 ? FWD_BM : F32_BM; }

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

hstu_status check_dims(const hstu_dims *dm)
{
    if (!dm) return fail(HSTU_ERR_ARG, "dims descriptor is NULL");
    if (dm->dtype != HSTU_F32 && dm->dtype != HSTU_BF16) return fail(HSTU_ERR_ARG, "unknown dtype %d", (int)dm->dtype);
    if (dm->heads < 1 || dm->heads > 255) return fail(HSTU_ERR_ARG, "heads must be in [1, 255] (got %d)", dm->heads);
    if (dm->d_qk != dm->d_v) return fail(HSTU_ERR_UNSUPPORTED, "d_qk != d_v is not supported");
    if (!(dm->ln_eps > 0.f)) return fail(HSTU_ERR_ARG, "ln_eps must be > 0");
    if (dm->dtype == HSTU_BF16 && dm->d_qk != 128)
        return fail(HSTU_ERR_UNSUPPORTED, "bf16 path supports d = 128 (got %d)", dm->d_qk);
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
    if (((uintptr_t)p & 3) != 0) return fail(HSTU_ERR_ARG, "%s must be 4-byte aligned", name);
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

} // namespace

extern "C" {

int32_t hstu_abi_version(void) { return HSTU_ABI_VERSION; }

const char *hstu_last_error(void) { return g_err.c_str(); }

size_t hstu_workspace_size(hstu_op op, const hstu_jagged *j, const hstu_dims *dims, int32_t d_model,
                           int32_t total_cand)
{
    if (check_jagged(j) != HSTU_OK || check_dims(dims) != HSTU_OK) return 0;
    switch (op) {
    case HSTU_OP_ATTN_FWD: return attn_ws(j, dims, fwd_tile(dims)).total;
    case HSTU_OP_ATTN_BWD: return attn_ws(j, dims, BWD_BN).total;
    default: break;
    }
    (void)d_model;
    (void)total_cand;
    fail(HSTU_ERR_ARG, "unknown op %d", (int)op);
    return 0;
}

hstu_status hstu_attn_fwd(const hstu_jagged *j, const hstu_dims *dm, const hstu_bias *bias, hstu_cmat q, hstu_cmat k,
                          hstu_cmat v, hstu_cmat u, hstu_mat out, float *o_save, float *ln_stats, void *ws,
                          size_t ws_bytes, void *stream)
{
    TRY(check_jagged(j));
    TRY(check_dims(dm));
    TRY(check_bias(bias, j));
    const int H = dm->heads, d = dm->d_qk, F = H * dm->d_v;
    TRY(check_view(q.ptr, q.ld, (int64_t)H * d, "q"));
    TRY(check_view(k.ptr, k.ld, (int64_t)H * d, "k"));
    TRY(check_view(v.ptr, v.ld, (int64_t)F, "v"));
    TRY(check_view(u.ptr, u.ld, (int64_t)F, "u", false));
    TRY(check_view(out.ptr, out.ld, (int64_t)F, "out"));
    if (ln_stats && !u.ptr) return fail(HSTU_ERR_ARG, "ln_stats requires u (the epilogue)");
    const int tile = fwd_tile(dm);
    const AttnWs w = attn_ws(j, dm, tile);
    TRY(check_ws(ws, ws_bytes, w.total));
    hipStream_t st = (hipStream_t)stream;
    char *wb = (char *)ws;
    int *status = (int *)(wb + w.header), *n_items = status + 1;
    int2 *items = (int2 *)(wb + w.items);
    uint32_t *rel = (uint32_t *)(wb + w.rel);
    int32_t *wide = (int32_t *)(wb + w.wide);
    const int T = j->total, B = j->batch;
    const int max_items = max_items_for(B, T, tile, H);
    {
        ProfScope ps("sched_kernel", st);
        launch_sched(j->offsets, j->ts, B, T, tile, H, status, n_items, items, max_items, rel, wide, st);
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
    float *obuf = nullptr;
    if (u.ptr) {
        obuf = o_save ? o_save : (float *)(wb + w.obuf);
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
    TRY(debug_check(ws, st));
    return ok();
}

hstu_status hstu_attn_bwd(const hstu_jagged *j, const hstu_dims *dm, const hstu_bias *bias, hstu_cmat q, hstu_cmat k,
                          hstu_cmat v, hstu_cmat u, const float *o_save, const float *ln_stats, hstu_cmat dout,
                          hstu_mat dq, hstu_mat dk, hstu_mat dv, hstu_mat du, float *drab_p, float *drab_t, void *ws,
                          size_t ws_bytes, void *stream)
{
    TRY(check_jagged(j));
    TRY(check_dims(dm));
    TRY(check_bias(bias, j));
    if (dm->dtype != HSTU_BF16) return fail(HSTU_ERR_UNSUPPORTED, "hstu_attn_bwd supports bf16 storage only");
    const int H = dm->heads, d = dm->d_qk, F = H * dm->d_v;
    TRY(check_view(q.ptr, q.ld, (int64_t)H * d, "q"));
    TRY(check_view(k.ptr, k.ld, (int64_t)H * d, "k"));
    TRY(check_view(v.ptr, v.ld, (int64_t)F, "v"));
    TRY(check_view(dout.ptr, dout.ld, (int64_t)F, "dout"));
    TRY(check_view(dq.ptr, dq.ld, (int64_t)H * d, "dq"));
    TRY(check_view(dk.ptr, dk.ld, (int64_t)H * d, "dk"));
    TRY(check_view(dv.ptr, dv.ld, (int64_t)F, "dv"));
    if (u.ptr) {
        TRY(check_view(u.ptr, u.ld, (int64_t)F, "u"));
        TRY(check_view(du.ptr, du.ld, (int64_t)F, "du"));
        if (!o_save || !ln_stats) return fail(HSTU_ERR_ARG, "with u, o_save and ln_stats from the forward are required");
    }
    const bool has_p = bias && bias->rab_p;
    const bool has_t = bias && bias->rab_t && j->ts;
    if (drab_p && has_p && bias->rab_p_hstride == 0)
        return fail(HSTU_ERR_ARG, "drab_p needs a per-head rab_p (hstride != 0)");
    if (drab_t && has_t && bias->rab_t_hstride == 0)
        return fail(HSTU_ERR_ARG, "drab_t needs a per-head rab_t (hstride != 0)");
    const AttnWs w = attn_ws(j, dm, BWD_BN);
    TRY(check_ws(ws, ws_bytes, w.total));
    hipStream_t st = (hipStream_t)stream;
    char *wb = (char *)ws;
    int *status = (int *)(wb + w.header), *n_items = status + 1;
    int2 *items = (int2 *)(wb + w.items);
    uint32_t *rel = (uint32_t *)(wb + w.rel);
    int32_t *wide = (int32_t *)(wb + w.wide);
    float *dq_acc = (float *)(wb + w.dq);
    bf16 *dO = (bf16 *)(wb + w.dO);
    const int T = j->total, B = j->batch, N = j->n_max;
    const int max_items = max_items_for(B, T, BWD_BN, H);
    const int64_t p_hs = has_p ? bias->rab_p_hstride : 2 * (int64_t)N + 1;
    const int64_t t_hs = (bias && bias->rab_t) ? bias->rab_t_hstride : 128;
    {
        ProfScope ps("sched_kernel", st);
        launch_sched(j->offsets, j->ts, B, T, BWD_BN, H, status, n_items, items, max_items, rel, wide, st);
    }
    TRY(launched(hipGetLastError(), "schedule kernel"));
    {
        ProfScope ps("fill_zero_kernel", st);
        TRY(launched(launch_fill_zero(dq_acc, (size_t)T * H * d * 4, st), "zero fill"));
        if (drab_p) TRY(launched(launch_fill_zero(drab_p, (size_t)H * p_hs * 4, st), "zero fill"));
        if (drab_t) TRY(launched(launch_fill_zero(drab_t, (size_t)H * t_hs * 4, st), "zero fill"));
    }
    const float inv_n = 1.0f / (float)N;
    if (u.ptr) {
        ProfScope ps("ln_gate_bwd_kernel", st);
        TRY(launched(launch_ln_gate_bwd(dout.ptr, dout.ld, u.ptr, u.ld, o_save, F, ln_stats, true, du.ptr, du.ld, dO,
                                        inv_n, T, F, status, st),
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
    a.rab_p = has_p ? bias->rab_p : nullptr;
    a.rp_hs = p_hs;
    a.rab_t = has_t ? bias->rab_t : nullptr;
    a.rt_hs = t_hs;
    a.H = H;
    a.N = N;
    a.items = items;
    a.n_items = n_items;
    a.dq_acc = dq_acc;
    a.dk = (bf16 *)dk.ptr;
    a.dv = (bf16 *)dv.ptr;
    a.lddk = dk.ld;
    a.lddv = dv.ld;
    a.drab_p = drab_p;
    a.drab_t = has_t ? drab_t : nullptr;
    {
        ProfScope ps("attn_bwd_bf16_kernel", st);
        TRY(launched(launch_attn_bwd_bf16(a, max_items, st), "attention backward kernel"));
    }
    {
        ProfScope ps("cast_kernel", st);
        TRY(launched(launch_cast_f32_to_bf16(dq_acc, (int64_t)H * d, (bf16 *)dq.ptr, dq.ld, T, H * d, status, st),
                     "cast kernel"));
    }
    TRY(debug_check(ws, st));
    return ok();
}

hstu_status hstu_layer_fwd(const hstu_jagged *j, const hstu_dims *dm, int32_t d_model, const hstu_layer *layer,
                           hstu_cmat x, hstu_mat y, hstu_mat k_cache, hstu_mat v_cache, void *ws, size_t ws_bytes,
                           void *stream)
{
    (void)j; (void)dm; (void)d_model; (void)layer; (void)x; (void)y; (void)k_cache; (void)v_cache; (void)ws;
    (void)ws_bytes; (void)stream;
    return fail(HSTU_ERR_UNSUPPORTED, "hstu_layer_fwd: not built yet");
}

hstu_status mfalcon_score(const hstu_jagged *hist, const hstu_dims *dm, int32_t d_model, int32_t n_layers,
                          const hstu_layer *layers, const hstu_cmat *k_cache, const hstu_cmat *v_cache,
                          const int32_t *cand_offsets, int32_t total_cand, const int64_t *cand_ts, hstu_cmat x_cand,
                          int32_t b_m, float *y_cand, void *ws, size_t ws_bytes, void *stream)
{
    (void)hist; (void)dm; (void)d_model; (void)n_layers; (void)layers; (void)k_cache; (void)v_cache;
    (void)cand_offsets; (void)total_cand; (void)cand_ts; (void)x_cand; (void)b_m; (void)y_cand; (void)ws;
    (void)ws_bytes; (void)stream;
    return fail(HSTU_ERR_UNSUPPORTED, "mfalcon_score: not built yet");
}

} // extern "C"
