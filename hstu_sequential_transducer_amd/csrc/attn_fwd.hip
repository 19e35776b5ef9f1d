// attn_fwd.hip -- forward of HSTU pointwise aggregated attention on gfx950.
//
// Computes, for each sequence b, head h and query i (review of "Actions Speak
// Louder than Words", section 3, Eq. 2, with phi2 read as SiLU(s)/N_max):
//   O[i] = (1/N) * sum_{j <= i} SiLU(q_i.k_j + rab_p[h][clip(j-i)] + rab_t[h][bucket(t_i - t_j)]) v_j
//
// bf16 kernel (d = 128): a workgroup of 4 waves owns 128 query rows of one
// (sequence, head); wave w owns rows 32w..32w+31 and keeps their Q in
// registers.  Keys stream through LDS in tiles of 64 (double buffered, one
// barrier per tile).  Per 32-key block a wave computes S^T = K Q^T with
// 32x32x16 bf16 MFMA (so each lane holds one query and 16 keys), adds both
// biases in registers, applies SiLU and the causal mask, packs P to bf16 and
// accumulates O^T += V^T P^T with V^T read by the transposing LDS load.  P
// never leaves registers.  Blocks above the diagonal are skipped; blocks on
// it are masked.
//
// The element-wise step works in the base-2 domain: x' = -log2(e) (s + bias)
// (one FMA, the tables are staged pre-scaled), P' = x' / (1 + 2^x') =
// -log2(e) SiLU(s + bias), and the constant -ln(2)/N is applied to O once at
// the end.  rab_p comes from a per-tile window in LDS indexed by key - query.
// rab_t: when all pairs of a 32x32 block share one time bucket (decided per
// block from the min/max times of its 32 queries and 32 keys) the bias is a
// scalar; otherwise it is read from a 32-entry LDS table indexed by
// count-leading-zeros of |dt| + 1 (exact for sequences whose time span fits
// 32 bits; wider sequences take an exact 64-bit path).  Every variant is a
// separate compile-time instantiation, so the element-wise code has no
// branches.
#include "kernels.h"

#include <type_traits>

namespace {

constexpr int BM = FWD_BM; // 128 query rows
constexpr int BN = 64;     // keys per LDS tile
constexpr int NT = 256;
// K and V tiles are [64 keys][D] bf16 (D = 128, 64 or 32: the head size)
// with no padding; the 16-byte chunks of row r are XOR-swizzled by sw(r) =
// 4(r%4) + bitrev2((r/4)%4), masked to the row's D/8 chunks, which for D =
// 128 keeps the 16-byte K-operand reads (16 consecutive rows, one chunk) and
// the transposing V reads (4 consecutive rows, 64 bytes each) free of bank
// conflicts, and lets the tiles be copied global -> LDS directly (1 KB, i.e.
// 1024 / (2 D) rows, per wave instruction).
constexpr int WIN = 192;   // rab_p window entries per tile (BM + BN - 1 used)
constexpr float NLOG2E = -1.4426950408889634f;
constexpr float NLN2 = -0.69314718055994531f;

template <int D>
struct alignas(16) Stage {
    alignas(16) bf16 k[BN * D];
    alignas(16) bf16 v[BN * D];
    float win[WIN];        // rab_p[clip(key - query)] (unscaled)
    uint32_t kt[BN];       // sequence-relative key times
};
template <int D>
struct alignas(16) Smem {
    Stage<D> st[2];     // (D = 128, after the last tile: a split item's output transpose, 4 x 32 x 132 floats)
    float rabt_rev[32]; // -log2(e) * rab_t[31 - c], indexed by clz(|dt| + 1)
    float rabt[128];    // -log2(e) * rab_t
};
static_assert(sizeof(Stage<128>) * 2 >= 4 * 32 * 132 * sizeof(float), "split-output transpose fits in the stages");

// Swizzle of row r: the XOR applied to its 16-byte chunk index (of D/8).
template <int D>
DEV int swf(int row)
{
    const int hi = (row >> 2) & 3;
    return (((row & 3) << 2) | ((hi & 1) << 1) | (hi >> 1)) & (D / 8 - 1);
}
// Element offset of (row, col) in a swizzled [rows][D] tile.
template <int D>
DEV int swz(int row, int col) { return row * D + (((col >> 3) ^ swf<D>(row)) << 3) + (col & 7); }

typedef __attribute__((address_space(3))) void lds_void;
typedef short short4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4v lds_short4v;

// Transposing LDS read (ds_read_b64_tr_b16).  Inside each group of 16 lanes,
// lane i receives element i%4 of the 4-element chunks addressed by lanes
// i/4, i/4+4, i/4+8, i/4+12 (in that order).
DEV u32x2 lds_read_tr(const bf16 *p)
{
    short4v r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v *)(p));
    return __builtin_bit_cast(u32x2, r);
}

// TM: 0 = no time bias, 1 = 32-bit relative times, 2 = 64-bit times.
// Register r of the S^T accumulator <-> key kbase + koff(r), koff = 8(r/4) + r%4
// (kbase = block start + 4g), query = this lane's.  sacc holds s + rab_p (the
// window is loaded into the accumulator).
//
// step(s), s = 0..7, is called at the start of each two-element step, for a
// caller that interleaves other products with the element-wise work (one
// MFMA per step; in the common variant -- one time bucket, off the diagonal
// -- the order is then pinned: per step its operand reads, its MFMA, then
// the step's VALU work).  The tile loop passes a no-op: issuing the next
// block's S^T here needs about 35 more registers than the 256 a wave has at
// two waves per SIMD, and the spills cost more than the overlap gains.
template <int TM, bool DIAG, bool UNI, typename Step>
DEV void pointwise(const floatx16 &sacc, uint32_t (&pk)[8], const uint32_t *kt_lane, const float *rabt_rev,
                   const float *rabt, uint32_t tq, int64_t tq64, const int64_t *tsk, int kbase, int klast, float ubias,
                   int dmask, Step &&step)
{
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
        step(r >> 1);
        float p2[2];
#pragma unroll
        for (int u = 0; u < 2; u++) {
            const int rr = r + u, koff = 8 * (rr >> 2) + (rr & 3);
            float tb = 0.f;
            if constexpr (TM == 1) {
                if constexpr (UNI) {
                    tb = ubias;
                } else {
                    const uint32_t tk = kt_lane[koff];
                    const uint32_t dd = (tq > tk ? tq - tk : tk - tq) + 1u; // |dt| + 1
                    tb = rabt_rev[__builtin_clz(dd)];
                }
            } else if constexpr (TM == 2) {
                const int key = min(kbase + koff, klast);
                tb = rabt[time_bucket64(tq64 - tsk[key])];
            }
            const float x = __builtin_fmaf(sacc[rr], NLOG2E, tb);
            float p = x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x));
            if constexpr (DIAG) p = koff > dmask ? 0.f : p;
            p2[u] = p;
        }
        pk[r >> 1] = pack2_bf16(p2[0], p2[1]);
    }
    if constexpr ((TM == 0 || (TM == 1 && UNI)) && !DIAG) {
#pragma unroll
        for (int s = 0; s < 8; s++) {
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0); // the step's operand reads
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0); // its MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 11, 0); // two elements
        }
    }
    __builtin_amdgcn_sched_barrier(0);
}

// Softmax elements of one 32x32 block (the comparator, SM): P' = 2^(s c - m)
// with the tile's running max m (scaled domain), masked pairs exactly 0;
// the lane's share of the row sum goes to lsum.
template <bool DIAG>
DEV void pointwise_softmax(const floatx16 &sacc, uint32_t (&pk)[8], float c, float m, float &lsum, int dmask)
{
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
        float p2[2];
#pragma unroll
        for (int u = 0; u < 2; u++) {
            const int rr = r + u, koff = 8 * (rr >> 2) + (rr & 3);
            float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[rr], c, -m));
            if constexpr (DIAG) p = koff > dmask ? 0.f : p;
            lsum += p;
            p2[u] = p;
        }
        pk[r >> 1] = pack2_bf16(p2[0], p2[1]);
    }
}

// The largest scaled score of a block among the lane's unmasked pairs.
template <bool DIAG>
DEV float block_max(const floatx16 &sacc, float c, int dmask)
{
    float mx = -__builtin_inff();
#pragma unroll
    for (int rr = 0; rr < 16; rr++) {
        const int koff = 8 * (rr >> 2) + (rr & 3);
        const float x = sacc[rr] * c;
        mx = (DIAG && koff > dmask) ? mx : fmaxf(mx, x);
    }
    return mx;
}

// qs, qmap: the queries are positions [qs, L) of the sequence (qs = 0
// except when new actions are appended to a cached history: then the
// sequence is [history; new] and only the new positions are queries), and
// query position p reads Q and writes O at row qmap + p (o_b for a whole
// sequence).  SM: the softmax comparator (no bias, online softmax).
template <int D, bool HP, int TM, bool SM = false>
DEV void fwd_body(const AttnFwdArgs &a, Smem<D> &sm, int o_b, int L, int q0, int h, int split, int part, int qs,
                  int64_t qmap)
{
    constexpr int KS = D / 16;      // K steps of the S^T products (and Q registers)
    constexpr int DB = D / 32;      // 32-wide d-blocks of O^T
    constexpr int NCH = D / 8;      // 16-byte chunks per row
    constexpr int RPI = 64 / NCH;   // rows per wave copy instruction
    constexpr int NPAT = 16 / RPI;  // distinct swizzle patterns of a wave's copy rows
    const int kend = min(q0 + BM, L); // keys [0, kend) are needed
    const int nkt = (kend + BN - 1) / BN;
    // a split item covers half of the key tiles: part 0 [0, nkt / 2), part 1 the rest
    const int kt_begin = split ? (part ? nkt / 2 : 0) : 0;
    const int kt_end = split ? (part ? nkt : nkt / 2) : nkt;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 5, lq = l & 31;
    const bf16 *Q = (const bf16 *)a.q, *K = (const bf16 *)a.k, *V = (const bf16 *)a.v;

    // This lane's query and its Q fragment: Q[row][16s + 8g .. +8], s = 0..7
    // (B operand of S^T = K Q^T).
    const int qstart = q0 + w * 32; // first query of this wave
    const int qrow = qstart + lq;
    const bool qvalid = qrow < L && qrow >= qs;
    const bool wact = qstart < L && qstart + 31 >= qs; // the wave has queries (wave-uniform)
    bf16x8 qreg[KS];
    {
        const bf16 *qp = Q + (qvalid ? qmap + qrow : 0) * a.ldq + h * D + g * 8;
#pragma unroll
        for (int s = 0; s < KS; s++) {
            u32x4 x = qvalid ? *(const u32x4 *)(qp + s * 16) : u32x4{0, 0, 0, 0};
            qreg[s] = as_bf16x8(x);
        }
    }
    const uint32_t tq = (TM == 1 && qvalid) ? a.rel[o_b + qrow] : 0u;
    const int64_t tq64 = (TM == 2 && qvalid) ? a.ts[o_b + qrow] : 0;
    // time range of this wave's queries (precomputed per 32-token block), as scalars
    uint32_t tqmin = 0xFFFFFFFFu, tqmax = 0u;
    if (TM == 1 && qstart < L) {
        tqmin = a.rmin[o_b + qstart];
        tqmax = a.rmax[o_b + qstart];
    }

    floatx16 oacc[DB];
#pragma unroll
    for (int i = 0; i < DB; i++)
#pragma unroll
        for (int r = 0; r < 16; r++) oacc[i][r] = 0.f;
    // softmax comparator: running max (scaled by c = log2(e) / sqrt(d)) and
    // this lane's share of the row sum
    const float sm_c = 1.4426950408889634f * __builtin_amdgcn_rsqf((float)D);
    float sm_m = -__builtin_inff(), sm_l = 0.f;

    // ---- tile loader: every copy goes global -> LDS directly.  K and V:
    // groups of RPI rows (one wave instruction each, 2 * 64 / RPI groups,
    // IPW per wave); lane l fills physical chunk l % NCH of row
    // RPI (G % (64 / RPI)) + l / NCH (rows past the needed keys repeat the
    // last one: finite, and every pair they form is masked).  The rab_p
    // window (waves 0-2, slot 64w + lane) and the key times (wave 3) as
    // 4-byte copies.  Full tiles (every key < kend): wave w copies plane w / 2
    // (K, then V), row groups IPW (w % 2) + i; the row base is wave-uniform
    // and each lane adds one of NPAT 32-bit byte offsets (its row of the
    // group, swizzled chunk), so the copies need no per-lane 64-bit address
    // arithmetic.
    constexpr int IPP = 64 / RPI, IPW = IPP / 2;
    const int wu = __builtin_amdgcn_readfirstlane(w);
    const bool kplane = wu < 2;
    const bf16 *pbase = kplane ? K : V;
    const int64_t pld = kplane ? a.ldk : a.ldv;
    uint32_t loff[NPAT];
#pragma unroll
    for (int j = 0; j < NPAT; j++) {
        const int rr = l / NCH, sw = swf<D>(RPI * j + rr);
        loff[j] = (uint32_t)(((int64_t)rr * pld + (((l % NCH) ^ sw) << 3)) * 2);
    }
    auto gload = [&](int kt, Stage<D> &S, auto full_c) {
        constexpr bool FULL = decltype(full_c)::value;
        const int kb0 = kt * BN;
        if constexpr (FULL) {
#pragma unroll
            for (int i = 0; i < IPW; i++) {
                const int gi = IPW * (wu & 1) + i, r0 = RPI * gi;
                const char *rowp = (const char *)(pbase + (int64_t)(o_b + kb0 + r0) * pld + h * D);
                __builtin_amdgcn_global_load_lds((const void *)(rowp + loff[gi % NPAT]),
                                                 (lds_void *)((kplane ? S.k : S.v) + r0 * D), 16, 0, 0);
            }
        } else {
#pragma unroll
            for (int i = 0; i < IPW; i++) {
                const int G = IPW * w + i, plane = G / IPP, r0 = RPI * (G % IPP);
                const int row = r0 + l / NCH;
                const int c = (l % NCH) ^ swf<D>(row);
                const int key = min(kb0 + row, kend - 1);
                const bf16 *src =
                    (plane == 0 ? K + (int64_t)(o_b + key) * a.ldk : V + (int64_t)(o_b + key) * a.ldv);
                __builtin_amdgcn_global_load_lds((const void *)(src + h * D + c * 8),
                                                 (lds_void *)((plane == 0 ? S.k : S.v) + r0 * D), 16, 0, 0);
            }
        }
        if constexpr (HP) {
            if (wu < 3) {
                int dl = kb0 - q0 - (BM - 1) + 64 * wu + l; // key - query of window slot 64w + l
                dl = dl < -a.N ? -a.N : (dl > a.N ? a.N : dl);
                __builtin_amdgcn_global_load_lds((const void *)(a.rab_p + h * a.rp_hs + dl + a.N),
                                                 (lds_void *)(S.win + 64 * wu), 4, 0, 0);
            }
        }
        if constexpr (TM == 1) {
            if (wu == 3) {
                const int key = FULL ? kb0 + l : min(kb0 + l, kend - 1);
                __builtin_amdgcn_global_load_lds((const void *)(a.rel + o_b + key), (lds_void *)S.kt, 4, 0, 0);
            }
        }
    };

    // transposing-read lane constants for the V operand
    const int tj = l & 15, tsl = tj >> 2;
    const int cpart = ((l >> 4) & 1) * 16 + 4 * (tj & 3);
    const int64_t *tsk = TM == 2 ? a.ts + o_b : nullptr;
    // Key tiles strictly below every query of the workgroup need no masking
    // and are full: the MAIN iterations, compiled without the per-block checks.
    const int n_main = q0 / BN; // tiles [0, n_main)

    // S^T of 32-key block kb (keys kb0 + 32 kb ..) in KS steps of one MFMA:
    // s_init starts the accumulator at the block's rab_p window (so the
    // products add the bias for free) and reads the first two K operands;
    // s_step(s) reads the operand two steps ahead and issues MFMA s.
    auto s_init = [&](const Stage<D> &S, int kb, floatx16 &sacc, bf16x8 (&fk)[3]) {
#pragma unroll
        for (int r = 0; r < 16; r++) {
            const int koff = 8 * (r >> 2) + (r & 3);
            sacc[r] = HP ? S.win[kb * 32 + 4 * g - w * 32 - lq + (BM - 1) + koff] : 0.f;
        }
        fk[0] = *(const bf16x8 *)&S.k[swz<D>(kb * 32 + lq, g * 8)];
        fk[1] = *(const bf16x8 *)&S.k[swz<D>(kb * 32 + lq, 16 + g * 8)];
    };
    auto s_step = [&](const Stage<D> &S, int kb, floatx16 &sacc, bf16x8 (&fk)[3], int st) {
        if (st + 2 < KS) fk[(st + 2) % 3] = *(const bf16x8 *)&S.k[swz<D>(kb * 32 + lq, (st + 2) * 16 + g * 8)];
        sacc = mfma32(fk[st % 3], qreg[st], sacc);
    };
    // The whole S^T of a block, reads two steps ahead of the MFMAs.
    auto s_block = [&](const Stage<D> &S, int kb, floatx16 &sacc) {
        __builtin_amdgcn_sched_barrier(0);
        bf16x8 fk[3];
        s_init(S, kb, sacc, fk);
#pragma unroll
        for (int st = 0; st < KS; st++) s_step(S, kb, sacc, fk, st);
        __builtin_amdgcn_sched_group_barrier(0x100, 18, 0); // the window and the first K operands
#pragma unroll
        for (int st = 0; st < KS; st++) {
            if (st + 2 < KS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    // O^T += V^T P^T for block kb in OS = 2 DB steps of one MFMA,
    // transposing V reads three steps ahead.  Step j: m = j / DB (keys
    // 16m..16m+15 of the block), db = j % DB.
    constexpr int OS = 2 * DB;
    auto o_fetch = [&](const Stage<D> &S, int kb, bf16x8 (&fv)[4], int jj) {
        const int m = jj / DB, db = jj % DB;
        // keys for element e of this lane's operand: 16m + 8(e/4) + 4g + e%4
        const int key1 = kb * 32 + 16 * m + 4 * g + tsl;
        const u32x2 r1 = lds_read_tr(&S.v[swz<D>(key1, db * 32 + cpart)]);
        const u32x2 r2 = lds_read_tr(&S.v[swz<D>(key1 + 8, db * 32 + cpart)]);
        fv[jj & 3] = as_bf16x8(u32x4{r1[0], r1[1], r2[0], r2[1]});
    };
    auto o_init = [&](const Stage<D> &S, int kb, bf16x8 (&fv)[4]) {
#pragma unroll
        for (int jj = 0; jj < 3 && jj < OS; jj++) o_fetch(S, kb, fv, jj);
    };
    auto o_step = [&](const Stage<D> &S, int kb, const uint32_t (&pk)[8], bf16x8 (&fv)[4], int jj) {
        if (jj + 3 < OS) o_fetch(S, kb, fv, jj + 3);
        const int m = jj / DB, db = jj % DB;
        const bf16x8 pb = as_bf16x8(u32x4{pk[4 * m], pk[4 * m + 1], pk[4 * m + 2], pk[4 * m + 3]});
        oacc[db] = mfma32(fv[jj & 3], pb, oacc[db]);
    };
    auto o_block = [&](const Stage<D> &S, int kb, const uint32_t (&pk)[8]) {
        __builtin_amdgcn_sched_barrier(0);
        bf16x8 fv[4];
        o_init(S, kb, fv);
#pragma unroll
        for (int jj = 0; jj < OS; jj++) o_step(S, kb, pk, fv, jj);
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * (OS < 3 ? OS : 3), 0);
#pragma unroll
        for (int jj = 0; jj < OS; jj++) {
            if (jj + 3 < OS) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    // The element-wise step of block kb (sacc holds s + rab_p): time-bias
    // mode from the block's key-time range [ka, kb_], then P' packed to bf16.
    auto pw_block = [&](const Stage<D> &S, int kt, int kb, const floatx16 &sacc, uint32_t (&pk)[8], bool diag,
                        uint32_t ka, uint32_t kb_, auto &&step) {
        const int kstart = kt * BN + kb * 32;
        const uint32_t *kt_lane = &S.kt[kb * 32 + 4 * g];
        const int kbase = kstart + 4 * g;
        bool uni = false;
        float ubias = 0.f;
        if constexpr (TM == 1) {
            // all pairs in one bucket iff floor(log2(min|dt| + 1)) == floor(log2(max|dt| + 1));
            // relative times of one non-wide sequence differ by less than 2^32 - 1
            if (tqmin <= tqmax) {
                const uint32_t lo = ka > tqmax ? ka - tqmax : (tqmin > kb_ ? tqmin - kb_ : 0u);
                const uint32_t h1 = tqmax > ka ? tqmax - ka : 0u, h2 = kb_ > tqmin ? kb_ - tqmin : 0u;
                const uint32_t hi = h1 > h2 ? h1 : h2;
                const int blo = floor_log2_u32(lo + 1u), bhi = floor_log2_u32(hi + 1u);
                uni = blo == bhi;
                ubias = sm.rabt[blo];
            }
        }
        if (diag)
            pointwise<TM, true, false>(sacc, pk, kt_lane, sm.rabt_rev, sm.rabt, tq, tq64, tsk, kbase, L - 1, ubias,
                                       lq - 4 * g, step);
        else if (TM == 1 && uni)
            pointwise<TM, false, true>(sacc, pk, kt_lane, sm.rabt_rev, sm.rabt, tq, tq64, tsk, kbase, L - 1, ubias, 0,
                                       step);
        else
            pointwise<TM, false, false>(sacc, pk, kt_lane, sm.rabt_rev, sm.rabt, tq, tq64, tsk, kbase, L - 1, ubias, 0,
                                        step);
    };

    // The key-time ranges of the two 32-key blocks of a tile, loaded one
    // tile ahead: the loads of tile kt + 1 are issued during tile kt, whose
    // final wait retires them.  (Loaded in the tile itself, after its copies,
    // they made the element-wise step wait for every copy of the next tile:
    // loads retire in order.)
    uint32_t krn[2] = {0u, 0u}, krx[2] = {0u, 0u};
    auto load_kr = [&](int kt) {
#pragma unroll
        for (int kb = 0; kb < 2; kb++) {
            const int ks = min(kt * BN + kb * 32, L - 1) & ~31; // past the sequence: its last block (unused)
            krn[kb] = a.rmin[o_b + ks];
            krx[kb] = a.rmax[o_b + ks];
        }
    };
    // One 64-key tile in stage par: the next tile's copies are issued first;
    // the transposing V reads (which wait for copies in flight) come last,
    // after both blocks' S^T and element-wise steps.
    auto iteration = [&](auto main_c, int kt, auto par) {
        constexpr bool MAIN = decltype(main_c)::value;
        if (kt + 1 < kt_end) {
            if ((kt + 2) * BN <= kend) gload(kt + 1, sm.st[1 - par], std::true_type{});
            else gload(kt + 1, sm.st[1 - par], std::false_type{});
        }
        const uint32_t kmn[2] = {krn[0], krn[1]}, kmx[2] = {krx[0], krx[1]};
        if constexpr (TM == 1)
            if (kt + 1 < kt_end) load_kr(kt + 1);
        const Stage<D> &S = sm.st[par];
        bool need[2], diag[2];
#pragma unroll
        for (int kb = 0; kb < 2; kb++) {
            const int kstart = kt * BN + kb * 32;
            need[kb] = wact && (MAIN ? true : kstart <= qstart + 31); // wave-uniform
            diag[kb] = MAIN ? false : kstart + 31 > qstart;
        }
        floatx16 sacc0, sacc1;
        uint32_t pk0[8], pk1[8];
        if constexpr (SM) {
            // online softmax over the tile: both blocks' scores, the tile's
            // max (shared by the two lanes of a query), the rescale of the
            // running sum and of O when the max grew, then P of both blocks
            if (need[0]) s_block(S, 0, sacc0);
            if (need[1]) s_block(S, 1, sacc1);
            float mx = -__builtin_inff();
            if (need[0]) mx = diag[0] ? block_max<true>(sacc0, sm_c, lq - 4 * g) : block_max<false>(sacc0, sm_c, 0);
            if (need[1])
                mx = fmaxf(mx, diag[1] ? block_max<true>(sacc1, sm_c, lq - 4 * g) : block_max<false>(sacc1, sm_c, 0));
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            const float m_new = fmaxf(sm_m, mx);
            if (__any(m_new > sm_m)) { // wave-uniform: some query's max grew
                const float alpha = __builtin_amdgcn_exp2f(sm_m - m_new);
                sm_l *= alpha;
#pragma unroll
                for (int i = 0; i < 4; i++)
#pragma unroll
                    for (int r = 0; r < 16; r++) oacc[i][r] *= alpha;
                sm_m = m_new;
            }
            if (need[0]) {
                if (diag[0]) pointwise_softmax<true>(sacc0, pk0, sm_c, sm_m, sm_l, lq - 4 * g);
                else pointwise_softmax<false>(sacc0, pk0, sm_c, sm_m, sm_l, 0);
            }
            if (need[1]) {
                if (diag[1]) pointwise_softmax<true>(sacc1, pk1, sm_c, sm_m, sm_l, lq - 4 * g);
                else pointwise_softmax<false>(sacc1, pk1, sm_c, sm_m, sm_l, 0);
            }
            if (need[0]) o_block(S, 0, pk0);
            if (need[1]) o_block(S, 1, pk1);
        } else if (need[1]) {
            // both blocks (need[1] implies need[0]): block 1's S^T products
            // run during block 0's element-wise step, block 0's O^T products
            // during block 1's, then block 1's O^T
            s_block(S, 0, sacc0);
            pw_block(S, kt, 0, sacc0, pk0, diag[0], kmn[0], kmx[0], [](int) {});
            s_block(S, 1, sacc1);
            pw_block(S, kt, 1, sacc1, pk1, diag[1], kmn[1], kmx[1], [](int) {});
            o_block(S, 0, pk0);
            o_block(S, 1, pk1);
        } else if (need[0]) {
            s_block(S, 0, sacc0);
            pw_block(S, kt, 0, sacc0, pk0, diag[0], kmn[0], kmx[0], [](int) {});
            o_block(S, 0, pk0);
        }
        __builtin_amdgcn_s_waitcnt(0); // the next tile's copies landed
        __syncthreads();
    };

    // Tile kt is in stage (kt - kt_begin) & 1.  The full-tile loop takes the
    // tiles in pairs, so that the stage of each is known at compile time and
    // its LDS addresses are constant offsets from per-lane bases (about a
    // fifth fewer VALU instructions per tile).
    gload(kt_begin, sm.st[0], std::false_type{});
    if constexpr (TM == 1) load_kr(kt_begin);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    const std::integral_constant<bool, false> generic{};
    const std::integral_constant<bool, true> fast{};
    int kt = kt_begin;
    if constexpr (TM != 2)
        for (; kt + 1 < min(n_main, kt_end); kt += 2) {
            iteration(fast, kt, std::integral_constant<int, 0>{});
            iteration(fast, kt + 1, std::integral_constant<int, 1>{});
        }
    for (; kt < kt_end; kt++) iteration(generic, kt, (kt - kt_begin) & 1);

    // O^T accumulator: lane holds query qrow, d = 32 db + 8(r/4) + 4g + r%4;
    // O = (-ln 2 / N) * sum P' V.
    const float sc = NLN2 * a.inv_n;
    if (D == 128 && split) { // (items are split for D = 128 only)
        // The two halves of a split item add their partial sums into the
        // (zeroed) fp32 output.  Through LDS (the stage tiles are free after
        // the last barrier) so that each atomic instruction covers 64
        // consecutive floats of one row: wave w's rows [32][132].
        float *ot = reinterpret_cast<float *>(&sm.st[0]) + w * 32 * 132;
#pragma unroll
        for (int db = 0; db < DB; db++)
#pragma unroll
            for (int gr = 0; gr < 4; gr++) {
                const int d0 = db * 32 + 8 * gr + 4 * g;
                *(floatx4 *)&ot[lq * 132 + d0] = floatx4{oacc[db][4 * gr] * sc, oacc[db][4 * gr + 1] * sc,
                                                         oacc[db][4 * gr + 2] * sc, oacc[db][4 * gr + 3] * sc};
            }
        __builtin_amdgcn_s_waitcnt(0xC07F); // lgkmcnt(0): this wave's rows are in LDS
        for (int r = 0; r < 32 && qstart + r < L; r++) {
            float *op = a.o32 + (int64_t)(o_b + qstart + r) * a.ld_o32 + h * D;
            atomicAdd(op + l, ot[r * 132 + l]);
            atomicAdd(op + 64 + l, ot[r * 132 + 64 + l]);
        }
        return;
    }
    float osc = sc;
    if constexpr (SM) {
        const float lt = sm_l + __shfl_xor(sm_l, 32, 64); // the query's whole row sum
        osc = 1.0f / lt;
        if (qvalid && g == 0 && a.lse) a.lse[(qmap + qrow) * a.H + h] = (sm_m + __log2f(lt)) * 0.69314718055994531f;
    }
    if (!qvalid) return;
    const int64_t row = qmap + qrow;
#pragma unroll
    for (int db = 0; db < DB; db++) {
#pragma unroll
        for (int gr = 0; gr < 4; gr++) {
            const int d0 = db * 32 + 8 * gr + 4 * g;
            floatx4 o4 = {oacc[db][4 * gr] * osc, oacc[db][4 * gr + 1] * osc, oacc[db][4 * gr + 2] * osc,
                          oacc[db][4 * gr + 3] * osc};
            if (a.o32) *(floatx4 *)(a.o32 + row * a.ld_o32 + h * D + d0) = o4;
            if (a.o16) {
                u32x2 pk2 = {pack2_bf16(o4[0], o4[1]), pack2_bf16(o4[2], o4[3])};
                *(u32x2 *)((bf16 *)a.o16 + row * a.ld_o16 + h * D + d0) = pk2;
            }
        }
    }
}

} // namespace

template <int D, bool HP>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2))) attn_fwd_bf16_kernel(AttnFwdArgs a)
{
    extern __shared__ __align__(16) unsigned char smem_raw[];
    Smem<D> &sm = *reinterpret_cast<Smem<D> *>(smem_raw);
    const int item = blockIdx.x;
    if (item >= *a.n_items) return;
    const int2 it = a.items[item];
    const int b = it.x, qt = it.y >> ITEM_T_SHIFT, split = (it.y >> 9) & 1, part = (it.y >> 8) & 1, h = it.y & 255;
    const int o_b = a.offsets[b];
    const int L = a.offsets[b + 1] - o_b;
    const bool has_t = a.ts != nullptr && a.rab_t != nullptr;
    const int tid = threadIdx.x;
    if (tid < 128) sm.rabt[tid] = has_t ? NLOG2E * a.rab_t[h * a.rt_hs + tid] : 0.f;
    if (tid < 32) sm.rabt_rev[tid] = has_t ? NLOG2E * a.rab_t[h * a.rt_hs + 31 - tid] : 0.f;
    // (the first barrier inside fwd_body orders these table writes before use)
    int qs = 0;
    int64_t qmap = o_b;
    if (a.aoff) { // appended actions: queries are the new positions [n_b, L)
        qs = a.hoff[b + 1] - a.hoff[b];
        qmap = (int64_t)a.aoff[b] - qs;
    }
    if (!has_t) fwd_body<D, HP, 0>(a, sm, o_b, L, qt * BM, h, split, part, qs, qmap);
    else if (a.wide[b] != 0) fwd_body<D, HP, 2>(a, sm, o_b, L, qt * BM, h, split, part, qs, qmap);
    else fwd_body<D, HP, 1>(a, sm, o_b, L, qt * BM, h, split, part, qs, qmap);
}

// The comparator: causal softmax attention O = softmax(Q K^T / sqrt(d)) V on
// the same skeleton (no bias, no gate, never split), for the pages'
// comparison of pointwise aggregated attention with softmax attention.
template <int D>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2))) attn_softmax_fwd_kernel(AttnFwdArgs a)
{
    extern __shared__ __align__(16) unsigned char smem_raw[];
    Smem<D> &sm = *reinterpret_cast<Smem<D> *>(smem_raw);
    const int item = blockIdx.x;
    if (item >= *a.n_items) return;
    const int2 it = a.items[item];
    const int b = it.x, qt = it.y >> ITEM_T_SHIFT, h = it.y & 255;
    const int o_b = a.offsets[b];
    const int L = a.offsets[b + 1] - o_b;
    fwd_body<D, false, 0, true>(a, sm, o_b, L, qt * BM, h, 0, 0, 0, o_b);
}

// ---------------------------------------------------------------------------
// fp32 kernel (any d in {16, 32, 64, 128}): one thread per query row, keys
// streamed through LDS in tiles of 32, plain fp32 FMA.  For the small fp32
// layers; the bf16 path above is the MFMA one.
template <int DD>
__global__ void __launch_bounds__(F32_BM) attn_fwd_f32_kernel(AttnFwdArgs a)
{
    constexpr int KT = 32;
    __shared__ float ks[KT][DD];
    __shared__ float vs[KT][DD];
    __shared__ int64_t kts[KT];
    const int item = blockIdx.x;
    if (item >= *a.n_items) return;
    const int2 it = a.items[item];
    const int b = it.x, qt = it.y >> ITEM_T_SHIFT, h = it.y & 255; // never split
    const int o_b = a.offsets[b];
    const int L = a.offsets[b + 1] - o_b;
    const int q0 = qt * F32_BM;
    const int i = q0 + threadIdx.x;
    const bool valid = i < L;
    const bool has_t = a.ts != nullptr && a.rab_t != nullptr;
    const float *Q = (const float *)a.q, *Kp = (const float *)a.k, *Vp = (const float *)a.v;
    float q[DD], acc[DD];
#pragma unroll
    for (int c = 0; c < DD; c++) {
        q[c] = valid ? Q[(int64_t)(o_b + i) * a.ldq + h * DD + c] : 0.f;
        acc[c] = 0.f;
    }
    const int64_t ti = (valid && has_t) ? a.ts[o_b + i] : 0;
    const int kend = min(q0 + F32_BM, L);
    for (int k0 = 0; k0 < kend; k0 += KT) {
        __syncthreads();
        for (int e = threadIdx.x; e < KT * DD; e += F32_BM) {
            const int kk = e / DD, c = e % DD, key = k0 + kk;
            const bool ok = key < kend;
            ks[kk][c] = ok ? Kp[(int64_t)(o_b + key) * a.ldk + h * DD + c] : 0.f;
            vs[kk][c] = ok ? Vp[(int64_t)(o_b + key) * a.ldv + h * DD + c] : 0.f;
        }
        if (threadIdx.x < KT) {
            const int key = k0 + threadIdx.x;
            kts[threadIdx.x] = (has_t && key < kend) ? a.ts[o_b + key] : 0;
        }
        __syncthreads();
        if (!valid) continue;
        for (int kk = 0; kk < KT; kk++) {
            const int j = k0 + kk;
            if (j > i) break;
            float s = 0.f;
#pragma unroll
            for (int c = 0; c < DD; c++) s = fmaf(q[c], ks[kk][c], s);
            if (a.rab_p) {
                int dl = j - i;
                dl = dl < -a.N ? -a.N : (dl > a.N ? a.N : dl);
                s += a.rab_p[h * a.rp_hs + dl + a.N];
            }
            if (has_t) s += a.rab_t[h * a.rt_hs + time_bucket64(ti - kts[kk])];
            const float p = s / (1.0f + expf(-s));
#pragma unroll
            for (int c = 0; c < DD; c++) acc[c] = fmaf(p, vs[kk][c], acc[c]);
        }
    }
    if (!valid) return;
    const int64_t row = o_b + i;
#pragma unroll
    for (int c = 0; c < DD; c++) {
        const float o = acc[c] * a.inv_n;
        if (a.o32) a.o32[row * a.ld_o32 + h * DD + c] = o;
        if (a.o16) ((float *)a.o16)[row * a.ld_o16 + h * DD + c] = o;
    }
}

namespace {
template <typename K>
hipError_t set_smem(K kernel, size_t smem)
{
    return hipFuncSetAttribute((const void *)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
}

template <int D>
hipError_t launch_fwd_d(const AttnFwdArgs &a, int max_items, hipStream_t st)
{
    static bool init = false;
    const size_t smem = sizeof(Smem<D>);
    if (!init) {
        hipError_t e = set_smem(attn_fwd_bf16_kernel<D, true>, smem);
        if (e == hipSuccess) e = set_smem(attn_fwd_bf16_kernel<D, false>, smem);
        if (e != hipSuccess) return e;
        init = true;
    }
    if (max_items <= 0) return hipSuccess;
    if (a.rab_p) hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, true>), dim3(max_items), dim3(NT), smem, st, a);
    else hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, false>), dim3(max_items), dim3(NT), smem, st, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_softmax_d(const AttnFwdArgs &a, int max_items, hipStream_t st)
{
    static bool init = false;
    const size_t smem = sizeof(Smem<D>);
    if (!init) {
        hipError_t e = set_smem(attn_softmax_fwd_kernel<D>, smem);
        if (e != hipSuccess) return e;
        init = true;
    }
    if (max_items <= 0) return hipSuccess;
    hipLaunchKernelGGL((attn_softmax_fwd_kernel<D>), dim3(max_items), dim3(NT), smem, st, a);
    return hipGetLastError();
}
} // namespace

hipError_t launch_attn_fwd_bf16(const AttnFwdArgs &a, int max_items, hipStream_t st)
{
    switch (a.d) {
    case 128: return launch_fwd_d<128>(a, max_items, st);
    case 64: return launch_fwd_d<64>(a, max_items, st);
    case 32: return launch_fwd_d<32>(a, max_items, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_attn_softmax_fwd(const AttnFwdArgs &a, int max_items, hipStream_t st)
{
    switch (a.d) {
    case 128: return launch_softmax_d<128>(a, max_items, st);
    case 64: return launch_softmax_d<64>(a, max_items, st);
    case 32: return launch_softmax_d<32>(a, max_items, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_attn_fwd_f32(const AttnFwdArgs &a, int max_items, hipStream_t st)
{
    if (max_items <= 0) return hipSuccess;
    switch (a.d) {
    case 16: hipLaunchKernelGGL(attn_fwd_f32_kernel<16>, dim3(max_items), dim3(F32_BM), 0, st, a); break;
    case 32: hipLaunchKernelGGL(attn_fwd_f32_kernel<32>, dim3(max_items), dim3(F32_BM), 0, st, a); break;
    case 64: hipLaunchKernelGGL(attn_fwd_f32_kernel<64>, dim3(max_items), dim3(F32_BM), 0, st, a); break;
    case 128: hipLaunchKernelGGL(attn_fwd_f32_kernel<128>, dim3(max_items), dim3(F32_BM), 0, st, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}
