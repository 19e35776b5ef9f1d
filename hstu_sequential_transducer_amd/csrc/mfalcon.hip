// mfalcon.hip -- M-FALCON candidate scoring (review of "Actions Speak Louder
// than Words", section 3, M-FALCON: m candidates are scored in ceil(m/b_m)
// microbatches whose attention operations are identical, and the history's
// linear and attention work is cached).
//
// Every candidate c of user u sits at position n_u (right after the user's
// history) with time t_c = cand_ts[u]; it attends to the whole cached history
// and to itself, never to another candidate.  For one layer and head:
//   o_c = (1/N) [ sum_{j < n_u} SiLU(q_c.k_j + beta_j) v_j + SiLU(q_c.k_c + beta_self) v_c ]
//   beta_j    = rab_p[clip(j - n_u)] + rab_t[bucket(t_c - t_j)]   (one value per key)
//   beta_self = rab_p[clip(0)] + rab_t[bucket(0)]
//
// The history part is a dense rectangle (no mask) on 32x32x16 bf16 MFMA: a
// workgroup owns up to 128 candidates of one microbatch of one user, one head
// and one chunk of the history (split-K over keys, exact because phi2 is
// pointwise: partial sums just add).  It writes its partial sum to its own
// slice of an fp32 buffer; the epilogue adds the slices in a fixed order, the
// self term, the 1/N scale, then LayerNorm (.) U -- so results do not depend
// on b_m or on the split, bit for bit.
#include "kernels.h"

namespace {

constexpr int D = 128;
constexpr int TC = MF_TC;  // candidates per tile (4 waves x 32)
constexpr int BN = 64;     // keys per LDS tile
constexpr int NT = 256;
constexpr int RS = 136; // K tile row stride (16-byte reads: 8 mod 16 elements)
constexpr int VS = 160; // V tile row stride (transposing reads)
constexpr float NLOG2E = -1.4426950408889634f;
constexpr float NLN2 = -0.69314718055994531f;

typedef short short4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4v lds_short4v;

DEV u32x2 lds_read_tr(const bf16 *p)
{
    short4v r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v *)(p));
    return __builtin_bit_cast(u32x2, r);
}

struct alignas(16) Stage {
    alignas(16) bf16 k[BN * RS];
    alignas(16) bf16 v[BN * VS];
    float beta[BN]; // -log2(e) * beta_j
};

} // namespace

// One workgroup: items in order (user u, microbatch, 128-candidate tile, head,
// split).  Per chunk of 1024 users: each thread counts its user's tiles, a
// scan gives every user's first tile, then all threads write the chunk's
// items (one per thread and pass).
__global__ void __launch_bounds__(1024) mfalcon_sched_kernel(const int32_t *__restrict__ hoff,
                                                              const int32_t *__restrict__ coff, int U, int M, int H,
                                                              int b_m, int nsplit, int4 *__restrict__ items,
                                                              int *__restrict__ n_items, int *__restrict__ status,
                                                              int max_items, int hist_total)
{
    __shared__ int cnt[1024];
    __shared__ int base_s;
    __shared__ int bad;
    const int tid = threadIdx.x;
    if (tid == 0) {
        base_s = 0;
        bad = (hoff[0] != 0 || hoff[U] != hist_total || coff[0] != 0 || coff[U] != M) ? HSTU_DEV_BAD_OFFSETS : 0;
    }
    __syncthreads();
    for (int u = tid; u < U; u += 1024)
        if (hoff[u + 1] < hoff[u] || coff[u + 1] < coff[u]) atomicOr(&bad, HSTU_DEV_BAD_OFFSETS);
    __syncthreads();
    if (bad) {
        if (tid == 0) {
            *status = bad;
            *n_items = 0;
        }
        return;
    }
    for (int c0 = 0; c0 < U; c0 += 1024) {
        const int u = c0 + tid;
        int tiles = 0;
        if (u < U) {
            const int m = coff[u + 1] - coff[u];
            for (int s = 0; s < m; s += b_m) {
                const int e = min(m, s + b_m);
                tiles += (e - s + TC - 1) / TC;
            }
        }
        cnt[tid] = tiles;
        __syncthreads();
        // inclusive Hillis-Steele scan over the chunk
        for (int o = 1; o < 1024; o <<= 1) {
            const int v = tid >= o ? cnt[tid - o] : 0;
            __syncthreads();
            cnt[tid] += v;
            __syncthreads();
        }
        // the chunk's items, all threads together: item i -> tile lt of the
        // chunk (its user found by binary search over the inclusive scan),
        // then that user's microbatch and candidate rows
        const int chunk_tiles = cnt[1023];
        const int per_tile = H * nsplit;
        const int n_chunk = min(U - c0, 1024);
        for (int i = tid; i < chunk_tiles * per_tile; i += 1024) {
            const int lt = i / per_tile, hs = i - lt * per_tile;
            int lo = 0, hi = n_chunk - 1; // first user v of the chunk with cnt[v] > lt
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (cnt[mid] > lt) hi = mid;
                else lo = mid + 1;
            }
            const int v = c0 + lo;
            const int ut = lt - (lo > 0 ? cnt[lo - 1] : 0); // tile of user v
            const int m = coff[v + 1] - coff[v];
            const int tpm = (b_m + TC - 1) / TC; // tiles of a full microbatch
            const int mb = ut / tpm, s0 = mb * b_m, e = min(m, s0 + b_m);
            const int r = s0 + (ut - mb * tpm) * TC;
            const int rows = min(TC, e - r);
            const int t = base_s + lt;
            const int idx = t * per_tile + hs;
            if (idx < max_items) items[idx] = make_int4(v, coff[v] + r, rows, ((hs / nsplit) << 16) | (hs % nsplit));
        }
        __syncthreads();
        if (tid == 1023) base_s += cnt[1023];
        __syncthreads();
    }
    if (tid == 0) {
        *n_items = base_s * H * nsplit;
        *status = 0;
    }
}

// History part of one (candidate tile, head, key chunk): part[split][c][h*d..]
// = sum over the chunk's keys of SiLU(q_c.k_j + beta_j) v_j (natural scale).
__global__ void __launch_bounds__(NT) mfalcon_attn_kernel(MfalconArgs a)
{
    extern __shared__ __align__(16) unsigned char smem_raw[];
    Stage *st = reinterpret_cast<Stage *>(smem_raw);
    const int item = blockIdx.x;
    if (item >= *a.n_items) return;
    const int4 it = a.items[item];
    const int u = it.x, c0 = it.y, rows = it.z, h = it.w >> 16, sp = it.w & 0xffff;
    const int ho = a.hoff[u];
    const int nu = a.hoff[u + 1] - ho;
    const int kbeg = sp * a.kchunk;
    const int kend = min(nu, kbeg + a.kchunk);
    const int nkt = kend > kbeg ? (kend - kbeg + BN - 1) / BN : 0;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 5, lq = l & 31;
    const bf16 *Q = (const bf16 *)a.q, *Kc = (const bf16 *)a.kc, *Vc = (const bf16 *)a.vc;
    const bool has_t = a.hts != nullptr && a.cts != nullptr && a.rab_t != nullptr;
    const int64_t tc = has_t ? a.cts[u] : 0;

    const int crow = w * 32 + lq; // candidate row inside the tile
    const bool cvalid = crow < rows;
    bf16x8 qreg[8];
    {
        const bf16 *qp = Q + (int64_t)(c0 + (cvalid ? crow : 0)) * a.ldz + h * D + g * 8;
#pragma unroll
        for (int s = 0; s < 8; s++) qreg[s] = as_bf16x8(cvalid ? *(const u32x4 *)(qp + s * 16) : u32x4{0, 0, 0, 0});
    }
    floatx16 oacc[4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int r = 0; r < 16; r++) oacc[i][r] = 0.f;

    const int lc = tid >> 4, le = tid & 15;
    u32x4 kreg[4], vreg[4];
    float breg = 0.f;
    auto gload = [&](int kt) {
        const int kb0 = kbeg + kt * BN;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int key = kb0 + lc * 4 + i;
            const bool ok = key < kend;
            const int64_t row = (int64_t)(ho + (ok ? key : 0));
            kreg[i] = ok ? *(const u32x4 *)(Kc + row * a.ldkc + h * D + le * 8) : u32x4{0, 0, 0, 0};
            vreg[i] = ok ? *(const u32x4 *)(Vc + row * a.ldvc + h * D + le * 8) : u32x4{0, 0, 0, 0};
        }
        if (tid < BN) {
            const int key = kb0 + tid;
            float bsum = 0.f;
            if (key < kend) {
                if (a.rab_p) {
                    int dl = key - nu;
                    dl = dl < -a.N ? -a.N : (dl > a.N ? a.N : dl);
                    bsum += a.rab_p[h * a.rp_hs + dl + a.N];
                }
                if (has_t) bsum += a.rab_t[h * a.rt_hs + time_bucket64(tc - a.hts[ho + key])];
            }
            breg = NLOG2E * bsum;
        }
    };
    auto sstore = [&](int buf) {
        Stage &S = st[buf];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            *(u32x4 *)&S.k[(lc * 4 + i) * RS + le * 8] = kreg[i];
            *(u32x4 *)&S.v[(lc * 4 + i) * VS + le * 8] = vreg[i];
        }
        if (tid < BN) S.beta[tid] = breg;
    };
    if (nkt > 0) {
        gload(0);
        sstore(0);
    }
    __syncthreads();
    const int tj = l & 15, tsl = tj >> 2;
    const int cpart = ((l >> 4) & 1) * 16 + 4 * (tj & 3);
    const bool wave_live = w * 32 < rows; // wave-uniform
    for (int kt = 0; kt < nkt; kt++) {
        if (kt + 1 < nkt) gload(kt + 1);
        const Stage &S = st[kt & 1];
        if (wave_live) {
#pragma unroll
            for (int kb = 0; kb < 2; kb++) {
                floatx16 sacc;
#pragma unroll
                for (int r = 0; r < 16; r++) sacc[r] = 0.f;
#pragma unroll
                for (int s = 0; s < 8; s++) {
                    const bf16x8 ka = *(const bf16x8 *)&S.k[(kb * 32 + lq) * RS + s * 16 + g * 8];
                    sacc = mfma32(ka, qreg[s], sacc);
                }
                uint32_t pk[8];
                const float *bl = &S.beta[kb * 32 + 4 * g];
#pragma unroll
                for (int r = 0; r < 16; r += 2) {
                    float p2[2];
#pragma unroll
                    for (int uu = 0; uu < 2; uu++) {
                        const int rr = r + uu, koff = 8 * (rr >> 2) + (rr & 3);
                        const float x = __builtin_fmaf(sacc[rr], NLOG2E, bl[koff]);
                        p2[uu] = x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x));
                    }
                    pk[r >> 1] = pack2_bf16(p2[0], p2[1]);
                }
#pragma unroll
                for (int m = 0; m < 2; m++) {
                    const bf16x8 pb = as_bf16x8(u32x4{pk[4 * m], pk[4 * m + 1], pk[4 * m + 2], pk[4 * m + 3]});
                    const int key1 = kb * 32 + 16 * m + 4 * g + tsl;
#pragma unroll
                    for (int db = 0; db < 4; db++) {
                        const u32x2 r1 = lds_read_tr(&S.v[key1 * VS + db * 32 + cpart]);
                        const u32x2 r2 = lds_read_tr(&S.v[(key1 + 8) * VS + db * 32 + cpart]);
                        oacc[db] = mfma32(as_bf16x8(u32x4{r1[0], r1[1], r2[0], r2[1]}), pb, oacc[db]);
                    }
                }
            }
        }
        if (kt + 1 < nkt) sstore((kt + 1) & 1);
        __syncthreads();
    }
    if (!cvalid) return;
    const int F = a.H * D;
    float *dst = a.part + (int64_t)sp * a.M * F + (int64_t)(c0 + crow) * F + h * D;
#pragma unroll
    for (int db = 0; db < 4; db++)
#pragma unroll
        for (int gr = 0; gr < 4; gr++) {
            const int d0 = db * 32 + 8 * gr + 4 * g;
            floatx4 o4 = {oacc[db][4 * gr] * NLN2, oacc[db][4 * gr + 1] * NLN2, oacc[db][4 * gr + 2] * NLN2,
                          oacc[db][4 * gr + 3] * NLN2};
            *(floatx4 *)(dst + d0) = o4;
        }
}

// Per candidate row (one wave): O = (sum_s part[s] + self term) / N, then
// G = LayerNorm(O) (.) U.  The self term of head h is SiLU(q.k + beta_self) v
// with q, k, v, u read from the candidate's own f1 output row.  Lane l owns
// features [l*VPL, l*VPL + VPL); a head spans d/VPL consecutive lanes.
template <int VPL, bool BF>
__global__ void __launch_bounds__(256) mfalcon_epilogue_kernel(const float *__restrict__ part, int nsplit,
                                                               const void *__restrict__ Z, int64_t ldz,
                                                               const float *__restrict__ rab_p, int64_t rp_hs,
                                                               const float *__restrict__ rab_t, int64_t rt_hs,
                                                               bool use_t, int N, float inv_n, float eps,
                                                               void *__restrict__ G, int64_t ldg, int M, int H, int d)
{
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= M) return;
    const int F = H * d;
    auto ld = [&](int64_t i) -> float {
        if constexpr (BF) return from_bf16(((const bf16 *)Z)[i]);
        else return ((const float *)Z)[i];
    };
    const int64_t zr = (int64_t)row * ldz;
    float x[VPL];
    float qk = 0.f;
    float vv[VPL]; // this lane's V features (the self term)
    if constexpr (BF && VPL % 4 == 0) {
        if (F == 64 * VPL) {
            // a full row per wave: 16- or 32-byte loads, consecutive lanes on
            // consecutive features (the partial sums in split order)
            const int c0 = lane * VPL;
#pragma unroll
            for (int i = 0; i < VPL; i++) x[i] = 0.f;
            const float *pr = part + (int64_t)row * F + c0;
            for (int sp = 0; sp < nsplit; sp++) {
#pragma unroll
                for (int i = 0; i < VPL; i += 4) {
                    const floatx4 p4 = *(const floatx4 *)(pr + (int64_t)sp * M * F + i);
#pragma unroll
                    for (int e = 0; e < 4; e++) x[i + e] += p4[e];
                }
            }
            const bf16 *zb = (const bf16 *)Z + zr + c0;
#pragma unroll
            for (int i = 0; i < VPL; i += 4) {
                const u32x2 q2 = *(const u32x2 *)(zb + 2 * F + i), k2 = *(const u32x2 *)(zb + 3 * F + i),
                            v2 = *(const u32x2 *)(zb + F + i);
                qk += bf16_lo(q2[0]) * bf16_lo(k2[0]) + bf16_hi(q2[0]) * bf16_hi(k2[0]) +
                      bf16_lo(q2[1]) * bf16_lo(k2[1]) + bf16_hi(q2[1]) * bf16_hi(k2[1]);
                vv[i] = bf16_lo(v2[0]);
                vv[i + 1] = bf16_hi(v2[0]);
                vv[i + 2] = bf16_lo(v2[1]);
                vv[i + 3] = bf16_hi(v2[1]);
            }
        }
    }
    if (!(BF && VPL % 4 == 0) || F != 64 * VPL) {
#pragma unroll
        for (int i = 0; i < VPL; i++) {
            const int c = lane * VPL + i;
            float v = 0.f;
            vv[i] = 0.f;
            if (c < F) {
                for (int sp = 0; sp < nsplit; sp++) v += part[(int64_t)sp * M * F + (int64_t)row * F + c];
                qk += ld(zr + 2 * F + c) * ld(zr + 3 * F + c); // q.k partial of this lane's head
                vv[i] = ld(zr + F + c);
            }
            x[i] = v;
        }
    }
    // segmented sum of q.k over the lanes of one head (d / VPL lanes)
    const int seg = d / VPL;
    for (int o = 1; o < seg; o <<= 1) qk += __shfl_xor(qk, o, 64);
    const int hh = (lane * VPL) / d;
    float beta = 0.f;
    if (hh < H) {
        if (rab_p) beta += rab_p[hh * rp_hs + N]; // clip(0) + N
        if (use_t) beta += rab_t[hh * rt_hs + 0]; // bucket(0) = 0
    }
    const float ps = silu_f(qk + beta);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < VPL; i++) {
        const int c = lane * VPL + i;
        if (c < F) x[i] = (x[i] + ps * vv[i]) * inv_n;
        s += c < F ? x[i] : 0.f;
    }
    const float mean = wave_sum(s) / (float)F;
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < VPL; i++) {
        const int c = lane * VPL + i;
        const float dl = x[i] - mean;
        q += c < F ? dl * dl : 0.f;
    }
    const float var = wave_sum(q) / (float)F;
    const float rstd = 1.0f / sqrtf(var + eps);
    if constexpr (BF && VPL % 4 == 0) {
        if (F == 64 * VPL) {
            const bf16 *ub = (const bf16 *)Z + zr + lane * VPL; // U block first
            bf16 *gb = (bf16 *)G + (int64_t)row * ldg + lane * VPL;
#pragma unroll
            for (int i = 0; i < VPL; i += 4) {
                const u32x2 u2 = *(const u32x2 *)(ub + i);
                const float u4[4] = {bf16_lo(u2[0]), bf16_hi(u2[0]), bf16_lo(u2[1]), bf16_hi(u2[1])};
                float g4[4];
#pragma unroll
                for (int e = 0; e < 4; e++) g4[e] = (x[i + e] - mean) * rstd * u4[e];
                *(u32x2 *)(gb + i) = u32x2{pack2_bf16(g4[0], g4[1]), pack2_bf16(g4[2], g4[3])};
            }
            return;
        }
    }
#pragma unroll
    for (int i = 0; i < VPL; i++) {
        const int c = lane * VPL + i;
        if (c >= F) continue;
        const float gv = (x[i] - mean) * rstd * ld(zr + c); // U block first
        if constexpr (BF) ((bf16 *)G)[(int64_t)row * ldg + c] = to_bf16(gv);
        else ((float *)G)[(int64_t)row * ldg + c] = gv;
    }
}

// fp32 history part: one thread per candidate row (small layers only).
__global__ void __launch_bounds__(64) mfalcon_attn_f32_kernel(MfalconArgs a)
{
    const int item = blockIdx.x;
    if (item >= *a.n_items) return;
    const int4 it = a.items[item];
    const int u = it.x, c0 = it.y, rows = it.z, h = it.w >> 16, sp = it.w & 0xffff;
    const int ho = a.hoff[u], nu = a.hoff[u + 1] - a.hoff[u];
    const int kbeg = sp * a.kchunk, kend = min(nu, kbeg + a.kchunk);
    const bool has_t = a.hts != nullptr && a.cts != nullptr && a.rab_t != nullptr;
    const int d = a.d;
    const float *Q = (const float *)a.q, *Kc = (const float *)a.kc, *Vc = (const float *)a.vc;
    const int F = a.H * d;
    for (int cr = threadIdx.x; cr < rows; cr += 64) {
        const int64_t c = c0 + cr;
        float *dst = a.part + (int64_t)sp * a.M * F + c * F + h * d;
        for (int e = 0; e < d; e++) dst[e] = 0.f;
        for (int j = kbeg; j < kend; j++) {
            float s = 0.f;
            for (int e = 0; e < d; e++) s = fmaf(Q[c * a.ldz + h * d + e], Kc[(int64_t)(ho + j) * a.ldkc + h * d + e], s);
            if (a.rab_p) {
                int dl = j - nu;
                dl = dl < -a.N ? -a.N : (dl > a.N ? a.N : dl);
                s += a.rab_p[h * a.rp_hs + dl + a.N];
            }
            if (has_t) s += a.rab_t[h * a.rt_hs + time_bucket64(a.cts[u] - a.hts[ho + j])];
            const float p = s / (1.0f + expf(-s));
            for (int e = 0; e < d; e++) dst[e] = fmaf(p, Vc[(int64_t)(ho + j) * a.ldvc + h * d + e], dst[e]);
        }
    }
}

hipError_t launch_mfalcon_sched(const int32_t *hoff, const int32_t *coff, int U, int M, int H, int b_m, int nsplit,
                                int4 *items, int *n_items, int *status, int max_items, int hist_total, hipStream_t st)
{
    hipLaunchKernelGGL(mfalcon_sched_kernel, dim3(1), dim3(1024), 0, st, hoff, coff, U, M, H, b_m, nsplit, items,
                       n_items, status, max_items, hist_total);
    return hipGetLastError();
}

hipError_t launch_mfalcon_attn(const MfalconArgs &a, int max_items, bool bf16io, hipStream_t st)
{
    if (max_items <= 0) return hipSuccess;
    if (!bf16io) {
        hipLaunchKernelGGL(mfalcon_attn_f32_kernel, dim3(max_items), dim3(64), 0, st, a);
        return hipGetLastError();
    }
    static bool init = false;
    const size_t smem = 2 * sizeof(Stage);
    if (!init) {
        hipError_t e = hipFuncSetAttribute((const void *)mfalcon_attn_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)smem);
        if (e != hipSuccess) return e;
        init = true;
    }
    hipLaunchKernelGGL(mfalcon_attn_kernel, dim3(max_items), dim3(NT), smem, st, a);
    return hipGetLastError();
}

#define VPL_SWITCH2(F, BODY)                                                                                        \
    do {                                                                                                            \
        const int need = ((F) + 63) / 64;                                                                           \
        if (need <= 1) { constexpr int V = 1; BODY; }                                                               \
        else if (need <= 2) { constexpr int V = 2; BODY; }                                                          \
        else if (need <= 4) { constexpr int V = 4; BODY; }                                                          \
        else if (need <= 8) { constexpr int V = 8; BODY; }                                                          \
        else if (need <= 16) { constexpr int V = 16; BODY; }                                                        \
        else if (need <= 32) { constexpr int V = 32; BODY; }                                                        \
        else return hipErrorInvalidValue;                                                                           \
    } while (0)

hipError_t launch_mfalcon_epilogue(const float *part, int nsplit, const void *Z, int64_t ldz, const float *rab_p,
                                   int64_t rp_hs, const float *rab_t, int64_t rt_hs, bool use_t, int N, float eps,
                                   void *G, int64_t ldg, int M, int H, int d, bool bf16io, hipStream_t st)
{
    if (M <= 0) return hipSuccess;
    const int F = H * d;
    const float inv_n = 1.0f / (float)N;
    dim3 grid((M + 3) / 4);
    if (bf16io)
        VPL_SWITCH2(F, hipLaunchKernelGGL((mfalcon_epilogue_kernel<V, true>), grid, dim3(256), 0, st, part, nsplit, Z,
                                          ldz, rab_p, rp_hs, rab_t, rt_hs, use_t, N, inv_n, eps, G, ldg, M, H, d));
    else
        VPL_SWITCH2(F, hipLaunchKernelGGL((mfalcon_epilogue_kernel<V, false>), grid, dim3(256), 0, st, part, nsplit, Z,
                                          ldz, rab_p, rp_hs, rab_t, rt_hs, use_t, N, inv_n, eps, G, ldg, M, H, d));
    return hipGetLastError();
}
