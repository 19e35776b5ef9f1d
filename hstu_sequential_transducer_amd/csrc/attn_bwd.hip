// attn_bwd.hip -- backward of HSTU pointwise aggregated attention on gfx950.
//
// Chain rule through Eq. 2 of the review of "Actions Speak Louder than Words"
// (section 3), phi2 read as SiLU(s)/N_max; with dO' = dO / N_max:
//   p_ij  = SiLU(x_ij),  x_ij = q_i.k_j + rab_p[clip(j-i)] + rab_t[bucket]
//   dV_j += sum_i p_ij dO'_i          dP_ij = dO'_i . v_j
//   dS_ij = dP_ij * s(x)(1 + x(1 - s(x)))   (s = sigmoid; 0 where j > i)
//   dK_j += sum_i dS_ij q_i           dQ_i += sum_j dS_ij k_j
//   drab_p[clip(j-i)] += dS_ij        drab_t[bucket] += dS_ij
// x is recomputed from Q, K and the tables (pointwise attention keeps no
// softmax statistics, so nothing else is needed).  dO' arrives as two bf16
// planes (hi + lo) so dP keeps ~16 significant bits.
//
// A workgroup of 8 waves owns 128 keys of one (sequence, head).  Keys come in
// 4 groups of 32; each group is served by two waves that run on the same
// SIMD and split the work by kind, so that one's element-wise VALU work
// overlaps the other's MFMAs:
//   the pointwise wave (waves 4-7) keeps its keys' K and V rows in registers
//     and, for query block n, computes X = Q K^T + rab_p and dP = dO' V^T (hi
//     and lo planes), then P = SiLU(X) and dS, which it writes to LDS as bf16
//     [key][query] tiles (and fp32 dS into a tile skewed by j - i for
//     drab_p), and adds dS to drab_t;
//   the accumulating wave (waves 0-3) works one block behind: dV^T += dO'^T P
//     and dK^T += Q^T dS for its keys, stores its 32 keys of the block's dS
//     tile to a bf16 [query][key] plane in global memory (dQ = dS K is a
//     separate GEMM, dq.hip), and sums the drab_p diagonals.  A sequence
//     whose plane does not fit the dS buffer takes the other instantiation,
//     where the accumulating wave adds dQ for d-block w of all 128 keys into
//     an fp32 buffer with global atomics instead.
// X, P and dS are computed once.  All products are 32x32x16 bf16 MFMA with
// lane = key, registers = queries.  Query blocks of 32 stream through LDS,
// copied global -> LDS directly by the accumulating waves at the start of the
// preceding block (so the pointwise waves, which carry the longer chain,
// issue no copies, and the copies have a whole block to land): Q and dO' are triple
// buffered (block n + 1 lands while the pointwise waves read block n and the
// accumulating waves block n - 1), dO'-lo and the per-block tables double
// buffered (only the pointwise waves read them).  The accumulating waves'
// transposing reads are asm blocks that wait for their own results, so that
// they do not wait for the copies in flight.  The rab_p window is loaded into
// the X accumulator.  One barrier per query block.
//
// drab_p: the pointwise wave writes its fp32 dS into an LDS tile skewed by
// j - i ([key - query][key mod 32]: a diagonal crosses a 32-query block at
// 32 consecutive keys, one per residue); one block later, one thread per diagonal sums
// it into an LDS ring indexed by j - i, and an entry is flushed with one
// global atomic once no later block can reach it.  drab_t: when every pair of
// a 32x32 block falls in one time bucket (decided per block in scalar code
// from the min/max times of its queries and keys) the bias is a scalar and
// the block's dS is summed by a wave reduction; otherwise per-element adds go
// to per-wave LDS tables.  Bias presence, time mode, diagonal masking and
// uniform blocks are compile-time instantiations, so the element-wise code
// has no branches.
#include "kernels.h"

#include <cstddef>
#include <type_traits>

namespace {

constexpr int BN = BWD_BN; // 128 keys per workgroup
constexpr int BQ = 32;     // queries per block
constexpr int NW = 8;      // waves per workgroup
constexpr int NT = 64 * NW;
// The head size D (128, 64 or 32) is a template parameter.  Q, dO and dO-lo
// stage tiles (and the prologue's K tile) are [rows][D] bf16 with no
// padding; the 16-byte chunks of row r are XOR-swizzled by sw(r) = 4(r%4) +
// bitrev2((r/4)%4), masked to the row's D/8 chunks, which for D = 128 keeps
// the 16-byte operand reads (16 consecutive rows, one chunk) and the
// transposing reads (4 consecutive rows, 64 bytes each) free of bank
// conflicts, and lets full blocks be copied global -> LDS directly (1024 /
// (2 D) rows per wave instruction).
constexpr int SS = 40;     // dS tile [key][query] row stride (bf16)
constexpr int WIN = 160;   // rab_p window per block (BQ + BN - 1 used)
constexpr int RING = 256;  // drab_p ring (power of two >= WIN + BQ)
constexpr int DK = 160;    // diagonals of the skewed dS tile: key - query + BQ - 1 (159 used, row 159 stays 0)
// Row pitch (floats) of the skewed tile, whose columns are keys mod 32: 16-byte
// rows, and 40 = 8 (mod 16) makes each column write (64 lanes: 32 keys x 2
// query halves 4 rows apart) hit 64 different banks.
constexpr int DKP = 40;
constexpr int TB = TB_SLOTS; // time buckets that int64 differences can reach
constexpr int TCOPY = 2;   // copies of each K wave's drab_t table
constexpr float NLOG2E = -1.4426950408889634f;
constexpr float NLN2 = -0.69314718055994531f;

// Stage tiles read by both roles (pointwise waves: block n; accumulating
// waves: block n - 1): triple buffered.
template <int D>
struct alignas(16) StageQ {
    alignas(16) bf16 q[BQ * D];
    alignas(16) bf16 dO[BQ * D];
};
// Stage data read by the pointwise waves only: double buffered.
template <int D>
struct alignas(16) StageP {
    alignas(16) bf16 dOl[BQ * D]; // low part of dO' (dO' = dO + dOl to ~16 bits)
    float win[WIN];               // rab_p[clip(key - query)], slot = key - query + BQ - 1 - (k0 - q0)
    uint32_t qt[BQ];
    uint32_t qtmin, qtmax;        // over the block's valid queries (right after qt: one copy fills both)
    uint32_t pad_[2];
    int64_t qt64[BQ];
};
template <int D>
struct alignas(16) Smem {
    StageQ<D> sq[3];
    StageP<D> sp[2];
    alignas(16) bf16 ds[2][BN * SS];    // dS [key][query] (the prologue's K tile spans ds and pt)
    alignas(16) bf16 pt[2][BN * SS];    // P' [key][query]
    alignas(16) float dsk[2][DK * DKP]; // fp32 dS skewed: [key - query + BQ - 1][key % 32]
    float ring[RING];
    float dtab[4][TCOPY][TB];
    float rabt_rev[32];
    float rabt[128];
};
static_assert(offsetof(Smem<128>, pt) == offsetof(Smem<128>, ds) + sizeof(Smem<128>::ds) &&
                  sizeof(Smem<128>::ds) + sizeof(Smem<128>::pt) >= sizeof(bf16) * BN * 128,
              "the prologue's K tile fits in ds + pt");
static_assert(sizeof(Smem<128>) <= 160 * 1024, "LDS budget");

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
DEV uint32_t lds_byte(const void *p) { return (uint32_t)(uintptr_t)(lds_void *)p; }
// The same read, four or eight at a time at LDS byte addresses ad[i], waited
// for inside one asm block: the accumulating waves issue the next block's
// direct copies before these reads, and the compiler, not seeing which buffer
// a builtin transposing read touches, would wait for every copy in flight.
DEV void lds_tr4(u32x2 (&r)[4], const uint32_t (&ad)[4])
{
    asm volatile("ds_read_b64_tr_b16 %0, %4\n\t"
                 "ds_read_b64_tr_b16 %1, %5\n\t"
                 "ds_read_b64_tr_b16 %2, %6\n\t"
                 "ds_read_b64_tr_b16 %3, %7\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
                 : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3])
                 : "memory");
}
DEV void lds_tr8(u32x2 (&r)[8], const uint32_t (&ad)[8])
{
    asm volatile("ds_read_b64_tr_b16 %0, %8\n\t"
                 "ds_read_b64_tr_b16 %1, %9\n\t"
                 "ds_read_b64_tr_b16 %2, %10\n\t"
                 "ds_read_b64_tr_b16 %3, %11\n\t"
                 "ds_read_b64_tr_b16 %4, %12\n\t"
                 "ds_read_b64_tr_b16 %5, %13\n\t"
                 "ds_read_b64_tr_b16 %6, %14\n\t"
                 "ds_read_b64_tr_b16 %7, %15\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]),
                   "=&v"(r[7])
                 : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5]), "v"(ad[6]), "v"(ad[7])
                 : "memory");
}

struct BwdLane {
    const uint32_t *qt;   // S.qt + 4g   (index with cr)
    const int64_t *qt64;  // S.qt64 + 4g
    float *dsk;           // skewed-tile cell of (cr = 27) for this lane; cell of cr at DKP (27 - cr)
                          // (positive offsets fit the LDS instructions' offset field)
    float *dtab;          // this K wave's drab_t table copy for this lane
    uint32_t tk;
    int64_t tk64;
    int dmask;            // masked (key > query) iff cr < dmask  (diagonal blocks)
};

// Time-bias modes of a 32x32 block (TM == 1): generic (per-element bucket
// and table lookup), one bucket for every pair (a scalar bias), or two
// adjacent buckets (per-element choice between two scalars, threshold
// 2^(blo + 1) on |dt| + 1).
enum { TB_ANY = 0, TB_ONE = 1, TB_TWO = 2 };

// x' = -log2(e) x for register r of the X accumulator (which holds x minus
// the time bias; time tables are staged pre-scaled), the time bucket (TB_ANY)
// or whether the pair is in the upper bucket (TB_TWO).
template <int TM, int UB>
DEV float xprime(const floatx16 &xacc, int rr, const BwdLane &ln, const float *rabt_rev, const float *rabt,
                 float ubias, float ubias2, uint32_t thr, int &bucket, bool &upper)
{
    const int cr = 8 * (rr >> 2) + (rr & 3);
    float tb = 0.f;
    bucket = 0;
    upper = false;
    if constexpr (TM == 1) {
        if constexpr (UB == TB_ONE) {
            tb = ubias;
        } else {
            const uint32_t tq = ln.qt[cr];
            const uint32_t dd1 = (tq > ln.tk ? tq - ln.tk : ln.tk - tq) + 1u;
            if constexpr (UB == TB_TWO) {
                upper = dd1 >= thr;
                tb = upper ? ubias2 : ubias;
            } else {
                const int cz = __builtin_clz(dd1);
                tb = rabt_rev[cz];
                bucket = 31 - cz;
            }
        }
    } else if constexpr (TM == 2) {
        bucket = time_bucket64(ln.qt64[cr] - ln.tk64);
        tb = rabt[bucket];
    }
    return __builtin_fmaf(xacc[rr], NLOG2E, tb);
}

// Pointwise wave, one 32x32 block: P' = x' sigmoid(x) = -log2(e) SiLU(x)
// (the -ln 2 goes into dV's final scale) and dS = dP sg (1 + x (1 - sg)) =
// dP (sg - ln2 (p' - p' sg)), both packed to bf16; fp32 dS also into the
// skewed tile and into drab_t (TB_ONE: the lane's sum in tsum; TB_TWO: the
// lane's total in tsum and its upper-bucket part in tsum2; TB_ANY: LDS
// atomics into the wave's tables).  Register r <-> query 4g + cr(r),
// cr = 8(r/4) + r%4; this lane's key.
//
// The part that needs only X (P' and the factor multiplying dP, which
// replaces x in xacc) runs first, two elements per step, while dp_step(s)
// issues step s of the dP = dO' V^T products (pacc, updated through the
// functor); then dS = dP * factor.
template <int TM, bool DT, bool DIAG, int UB, typename DpStep>
DEV void pointwise(floatx16 &xacc, const floatx16 &pacc, DpStep &&dp_step, uint32_t (&ppk)[8], uint32_t (&dpk)[8],
                   const BwdLane &ln, const float *rabt_rev, const float *rabt, float ubias, float ubias2,
                   uint32_t thr, float &tsum, float &tsum2, bf16 *pt_row)
{
    floatx16 &fac = xacc; // each element's factor replaces its x
#pragma unroll
    for (int s = 0; s < 8; s++) {
        dp_step(s);
        float pp[2];
#pragma unroll
        for (int u = 0; u < 2; u++) {
            const int rr = 2 * s + u, cr = 8 * (rr >> 2) + (rr & 3);
            int bucket;
            bool upper;
            const float x = xprime<TM, UB>(xacc, rr, ln, rabt_rev, rabt, ubias, ubias2, thr, bucket, upper);
            const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x));
            float p = x * sg;
            float f = __builtin_fmaf(__builtin_fmaf(-p, sg, p), NLN2, sg);
            if constexpr (DIAG) {
                p = cr < ln.dmask ? 0.f : p;
                f = cr < ln.dmask ? 0.f : f;
            }
            pp[u] = p;
            fac[rr] = f;
        }
        ppk[s] = pack2_bf16(pp[0], pp[1]);
    }

    __builtin_amdgcn_sched_barrier(0);
    // P' -> LDS as [key][query] (lane row, 4 queries per r/4 group) while the
    // last dP products finish
#pragma unroll
    for (int gr = 0; gr < 4; gr++) *(u32x2 *)&pt_row[8 * gr] = u32x2{ppk[2 * gr], ppk[2 * gr + 1]};
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
        float dd[2];
#pragma unroll
        for (int u = 0; u < 2; u++) {
            const int rr = r + u, cr = 8 * (rr >> 2) + (rr & 3);
            const float ds = pacc[rr] * fac[rr];
            dd[u] = ds;
            ln.dsk[DKP * (27 - cr)] = ds;
            if constexpr (DT && TM != 0) {
                if constexpr (UB == TB_ONE) {
                    tsum += ds;
                } else {
                    int bucket;
                    bool upper;
                    (void)xprime<TM, UB>(xacc, rr, ln, rabt_rev, rabt, ubias, ubias2, thr, bucket, upper);
                    if constexpr (UB == TB_TWO) {
                        tsum += ds;
                        tsum2 += upper ? ds : 0.f;
                    } else {
                        atomicAdd(&ln.dtab[bucket], ds);
                    }
                }
            }
        }
        dpk[r >> 1] = pack2_bf16(dd[0], dd[1]);
    }
}

// Sum over the 64 lanes with DPP moves inside each row of 16 lanes and four
// lane reads (no LDS traffic); the result is wave-uniform.
template <int CTRL>
DEV float dpp_mov(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
DEV float wave_sum_dpp(float v)
{
    v += dpp_mov<0xB1>(v);  // quad_perm [1,0,3,2]
    v += dpp_mov<0x4E>(v);  // quad_perm [2,3,0,1]
    v += dpp_mov<0x141>(v); // row_half_mirror
    v += dpp_mov<0x140>(v); // row_mirror: every lane holds its row's sum
    const int b = __builtin_bit_cast(int, v);
    return (__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0)) +
            __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16))) +
           (__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32)) +
            __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48)));
}

// 16-byte slice o..o+3 of a register block as a bf16x8 MFMA operand.  (Each
// element is copied to a scalar before the bit cast: clang's bit_cast of a
// vector-element expression reads element 0.)
DEV bf16x8 slice8(const floatx16 &f, int o)
{
    const float e0 = f[o], e1 = f[o + 1], e2 = f[o + 2], e3 = f[o + 3];
    return as_bf16x8(u32x4{__builtin_bit_cast(uint32_t, e0), __builtin_bit_cast(uint32_t, e1),
                           __builtin_bit_cast(uint32_t, e2), __builtin_bit_cast(uint32_t, e3)});
}

template <int D, bool HP, int TM, bool DT, bool DQA>
DEV void bwd_body(const AttnBwdArgs &a, Smem<D> &sm, int b_seq, int o_b, int L, int k0, int h)
{
    constexpr int KS = D / 16;     // K steps of the X and dP products
    constexpr int DB = D / 32;     // 32-wide d-blocks of dV^T, dK^T (and the K/V registers)
    constexpr int NCH = D / 8;     // 16-byte chunks per row
    constexpr int RPI = 64 / NCH;  // rows per wave copy instruction
    constexpr int GPP = BQ / RPI;  // copy groups per stage plane (8, 4 or 2)
    static_assert(GPP == 8 || GPP == 4 || GPP == 2, "copy groups per plane");
    using StageQD = StageQ<D>;
    using StagePD = StageP<D>;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 5, lq = l & 31;
    const int p = w & 3;          // key group: keys 32p..32p+31 of the tile
    const bool awave = w < 4;     // accumulating wave (else pointwise wave); wave-uniform
    const bf16 *Q = a.q, *K = a.k, *V = a.v, *dO = a.dO;
    const int64_t ld_do = (int64_t)a.H * D;
    const bf16 *dOlo = dO + (int64_t)a.T * ld_do;
    // transposing-read lane constants
    const int tj = l & 15, tsl = tj >> 2;
    const int cpart = ((l >> 4) & 1) * 16 + 4 * (tj & 3);

    // ---- prologue: a pointwise wave's own K and V rows come straight from
    // memory into registers.  DQA (dQ by atomics, for a sequence whose dS
    // planes do not fit the dS buffer): the workgroup's K rows also go to LDS
    // (rows past the sequence repeat the last row: finite, and every pair
    // they form is masked or has dS = 0), from where an accumulating wave
    // keeps d-block p of all 128 rows in registers (B operand of dQ = dS K).
    bf16 *kt = &sm.ds[0][0]; // prologue only
    if constexpr (DQA) {
#pragma unroll
        for (int i = 0; i < BN / (RPI * NW); i++) {
            const int r0 = RPI * ((BN / (RPI * NW)) * w + i), row = r0 + l / NCH;
            const int c = (l % NCH) ^ swf<D>(row);
            const int key = min(k0 + row, L - 1);
            __builtin_amdgcn_global_load_lds((const void *)(K + (int64_t)(o_b + key) * a.ldk + h * D + c * 8),
                                             (lds_void *)(kt + r0 * D), 16, 0, 0);
        }
    }
    const int kw0 = k0 + 32 * p; // this key group's first key
    const int mykey = kw0 + lq;
    const bool kvalid = mykey < L;
    // acc: accumulating wave -> dV^T.  acc2: accumulating wave -> dK^T;
    // pointwise wave -> the bits of its K row (chunks 2i, 2i+1 in elements
    // 0..7 of acc2[i]) and V row (elements 8..15), 16-byte chunk s holding
    // d = 16s + 8g .. +8 (B operands of X = Q K^T and dP = dO' V^T).
    // Lane = key, d = 32 db + 8(r/4) + 4g + r%4 for the accumulators.
    floatx16 acc[DB], acc2[DB];
#pragma unroll
    for (int i = 0; i < DB; i++)
#pragma unroll
        for (int r = 0; r < 16; r++) acc[i][r] = acc2[i][r] = 0.f;
    if (!awave && kvalid) {
        const int64_t row = o_b + mykey;
        const bf16 *kp = K + row * a.ldk + h * D + g * 8, *vp = V + row * a.ldv + h * D + g * 8;
#pragma unroll
        for (int i = 0; i < DB; i++) {
            const u32x4 k1 = *(const u32x4 *)(kp + 32 * i), k2 = *(const u32x4 *)(kp + 32 * i + 16);
            const u32x4 v1 = *(const u32x4 *)(vp + 32 * i), v2 = *(const u32x4 *)(vp + 32 * i + 16);
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const uint32_t ka = k1[e], kb = k2[e], va = v1[e], vb = v2[e];
                acc2[i][e] = __builtin_bit_cast(float, ka);
                acc2[i][4 + e] = __builtin_bit_cast(float, kb);
                acc2[i][8 + e] = __builtin_bit_cast(float, va);
                acc2[i][12 + e] = __builtin_bit_cast(float, vb);
            }
        }
    }
    for (int i = tid; i < RING; i += NT) sm.ring[i] = 0.f;
    for (int i = tid; i < 2 * DK * DKP; i += NT) (&sm.dsk[0][0])[i] = 0.f;
    for (int i = tid; i < 4 * TCOPY * TB; i += NT) (&sm.dtab[0][0][0])[i] = 0.f;

    BwdLane ln;
    ln.tk = (TM == 1 && kvalid) ? a.rel[o_b + mykey] : 0u;
    ln.tk64 = (TM == 2 && kvalid) ? a.ts[o_b + mykey] : 0;
    ln.dtab = &sm.dtab[p][lq & (TCOPY - 1)][0];
    // time range of this group's valid keys (for the uniform-bucket test), as scalars
    uint32_t tkmin = kvalid ? ln.tk : 0xFFFFFFFFu, tkmax = kvalid ? ln.tk : 0u;
    if constexpr (TM == 1) {
        for (int o = 16; o >= 1; o >>= 1) {
            tkmin = min(tkmin, (uint32_t)__shfl_xor((int)tkmin, o, 64));
            tkmax = max(tkmax, (uint32_t)__shfl_xor((int)tkmax, o, 64));
        }
        tkmin = __builtin_amdgcn_readfirstlane(tkmin);
        tkmax = __builtin_amdgcn_readfirstlane(tkmax);
    }

    // ---- query-block stage loader.  Full blocks: 3 GPP groups of RPI rows
    // (Q, dO, dO-lo; 24 groups of 4 rows at D = 128) copied straight into
    // LDS, spread over the copying waves; lane l fills physical chunk l % NCH
    // of row RPI (G % GPP) + l / NCH.  The last, partial block goes through
    // registers (rows past the sequence: Q from the last row, dO = 0, so they
    // contribute nothing).
    const int lcq = tid / NCH, leq = tid % NCH; // partial path: 32 queries x NCH threads x 8 elements
    float wreg = 0.f;
    uint32_t treg = 0, tmn = 0xFFFFFFFFu, tmx = 0u;
    int64_t treg64 = 0;
    // nw waves share the copies; wi = this wave's index among them.
    // Row bases are wave-uniform 64-bit pointers; the lane part of each
    // address is a 32-bit offset (24-bit products).
    auto gload_direct = [&](auto nw_c, int wi, int q0, StageQD &SQ, StagePD &SP) {
        constexpr int NWC = decltype(nw_c)::value;
        constexpr int TOT = 3 * GPP; // copy groups of the three planes
        const int64_t rq = (int64_t)(o_b + q0);
        const bf16 *bq = Q + rq * a.ldq + h * D, *bo = dO + rq * ld_do + h * D, *bl = dOlo + rq * ld_do + h * D;
#pragma unroll
        for (int i = 0; i < (TOT + NWC - 1) / NWC; i++) {
            int G;
            if constexpr (TOT % NWC == 0) {
                G = (TOT / NWC) * wi + i;
            } else {
                G = wi + NWC * i;
                if (G >= TOT) break; // (wave-uniform)
            }
            // (GPP is a power of two: shift and mask, no signed-division fix-up)
            const int plane = G >> (GPP == 8 ? 3 : (GPP == 4 ? 2 : 1)), r0 = RPI * (G & (GPP - 1));
            const int row = r0 + l / NCH;
            const int c = (l % NCH) ^ swf<D>(row);
            const uint32_t ld = plane == 0 ? (uint32_t)a.ldq : (uint32_t)ld_do;
            const uint32_t off = __umul24((uint32_t)row, ld) + 8u * (uint32_t)c;
            const bf16 *src = (plane == 0 ? bq : (plane == 1 ? bo : bl)) + off;
            bf16 *dst = (plane == 0 ? SQ.q : (plane == 1 ? SQ.dO : SP.dOl)) + r0 * D;
            __builtin_amdgcn_global_load_lds((const void *)src, (lds_void *)dst, 16, 0, 0);
        }
    };
    // Per-block tables, loaded and stored by the threads tt = 0.. of one role.
    auto gload_tables = [&](int q0, int tt) {
        if constexpr (HP) {
            if (tt >= 0 && tt < WIN) {
                int dl = k0 - q0 - (BQ - 1) + tt; // key - query of window slot tt
                dl = dl < -a.N ? -a.N : (dl > a.N ? a.N : dl);
                wreg = a.rab_p[h * a.rp_hs + dl + a.N];
            }
        }
        if constexpr (TM != 0) {
            if (tt >= 0 && tt < 64) { // one wave: query times and (precomputed) their range
                const int q = q0 + tt;
                const bool okq = tt < BQ && q < L;
                treg = (TM == 1 && okq) ? a.rel[o_b + q] : 0u;
                treg64 = (TM == 2 && okq) ? a.ts[o_b + q] : 0;
                if constexpr (TM == 1) {
                    tmn = a.rmin[o_b + q0];
                    tmx = a.rmax[o_b + q0];
                }
            }
        }
    };
    auto load_partial = [&](int q0, StageQD &SQ, StagePD &SP) {
        if constexpr (BQ * NCH < NT)
            if (lcq >= BQ) return; // (D < 128: fewer threads than the workgroup's)
        const int qi = q0 + lcq;
        const bool ok = qi < L;
        const int64_t row = (int64_t)(o_b + (ok ? qi : L - 1));
        const int col = leq * 8;
        const u32x4 qv = *(const u32x4 *)(Q + row * a.ldq + h * D + col);
        const u32x4 dv = ok ? *(const u32x4 *)(dO + row * ld_do + h * D + col) : u32x4{0, 0, 0, 0};
        const u32x4 lv = ok ? *(const u32x4 *)(dOlo + row * ld_do + h * D + col) : u32x4{0, 0, 0, 0};
        *(u32x4 *)&SQ.q[swz<D>(lcq, col)] = qv;
        *(u32x4 *)&SQ.dO[swz<D>(lcq, col)] = dv;
        *(u32x4 *)&SP.dOl[swz<D>(lcq, col)] = lv;
    };
    auto sstore_tables = [&](StagePD &S, int tt) {
        if constexpr (HP)
            if (tt >= 0 && tt < WIN) S.win[tt] = wreg;
        if constexpr (TM != 0) {
            if (tt >= 0 && tt < BQ) {
                S.qt[tt] = treg;
                S.qt64[tt] = treg64;
            }
            if (tt == 0) {
                S.qtmin = tmn;
                S.qtmax = tmx;
            }
        }
    };

    // A full block's tables copied straight into LDS by the accumulating
    // waves (4-byte copies, lane i -> 4i bytes past the wave's LDS base): the
    // window by waves 0-2 (slots 64 w + lane), the query times and their
    // range by wave 3 (lanes 0-31, then 32, 33).
    auto gload_tables_direct = [&](int q0, StagePD &SP) {
        const int pw = w;
        if constexpr (HP) {
            if (pw < 3 && 64 * pw + l < WIN) {
                int dl = k0 - q0 - (BQ - 1) + 64 * pw + l;
                dl = dl < -a.N ? -a.N : (dl > a.N ? a.N : dl);
                __builtin_amdgcn_global_load_lds((const void *)(a.rab_p + h * a.rp_hs + dl + a.N),
                                                 (lds_void *)(SP.win + 64 * pw), 4, 0, 0);
            }
        }
        if constexpr (TM == 1) {
            if (pw == 3 && l < BQ + 2) {
                const uint32_t *src = l < BQ ? a.rel + o_b + q0 + l : (l == BQ ? a.rmin : a.rmax) + o_b + q0;
                __builtin_amdgcn_global_load_lds((const void *)src, (lds_void *)SP.qt, 4, 0, 0);
            }
        }
    };

    // stage 0
    const std::integral_constant<int, NW> all_waves{};
    const std::integral_constant<int, NW / 2> half_waves{};
    if (k0 + BQ <= L) gload_direct(all_waves, w, k0, sm.sq[0], sm.sp[0]);
    else load_partial(k0, sm.sq[0], sm.sp[0]);
    gload_tables(k0, tid);
    sstore_tables(sm.sp[0], tid);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    bf16x8 opnd[DQA ? 8 : 1]; // DQA, accumulating wave p < DB: K d-block p of all rows (dQ operand)
    if constexpr (DQA) {
        if (awave && (DB == 4 || p < DB)) {
#pragma unroll
            for (int t = 0; t < BN / 16; t++) {
                const int kr1 = 16 * t + 8 * g + tsl;
                const u32x2 k1 = lds_read_tr(&kt[swz<D>(kr1, 32 * p + cpart)]);
                const u32x2 k2 = lds_read_tr(&kt[swz<D>(kr1 + 4, 32 * p + cpart)]);
                opnd[t] = as_bf16x8(u32x4{k1[0], k1[1], k2[0], k2[1]});
            }
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads(); // the K tile is dead (ds and pt are written from block 0 on)
    }

    const int p_hs = a.rp_hs > 0 ? (int)a.rp_hs : 2 * a.N + 1;

    // Accumulating wave, block at q0m (stage SQ, tiles of buffer b), keys of
    // this group: dV^T += dO'^T P and dK^T += Q^T dS, contractions over the
    // 32 queries.  The B operands are this lane's key row of the P' and dS
    // tiles, queries 16m + {4g..4g+3, 8+4g..8+4g+3} (the order of the
    // transposing reads' k index).
    auto acc_block = [&](const StageQD &SQ, int b) {
        const bf16 *ptb = sm.pt[b], *dsb = sm.ds[b];
        const int krow = 32 * p + lq;
        __builtin_amdgcn_sched_barrier(0);
        bf16x8 pb[2], sb[2];
#pragma unroll
        for (int m = 0; m < 2; m++) {
            const u32x2 p1 = *(const u32x2 *)&ptb[krow * SS + 16 * m + 4 * g];
            const u32x2 p2 = *(const u32x2 *)&ptb[krow * SS + 16 * m + 8 + 4 * g];
            const u32x2 s1 = *(const u32x2 *)&dsb[krow * SS + 16 * m + 4 * g];
            const u32x2 s2 = *(const u32x2 *)&dsb[krow * SS + 16 * m + 8 + 4 * g];
            pb[m] = as_bf16x8(u32x4{p1[0], p1[1], p2[0], p2[1]});
            sb[m] = as_bf16x8(u32x4{s1[0], s1[1], s2[0], s2[1]});
        }
        // NJ = 4 DB steps j: m = j / (2 DB), db = (j / 2) % DB; even j: dO'^T slice
        // -> dV, odd j: Q^T slice -> dK.  Transposing reads run three steps ahead.
        constexpr int NJ = 4 * DB;
        // four steps per batch of transposing reads
#pragma unroll
        for (int j0 = 0; j0 < NJ; j0 += 4) {
            uint32_t ad[8];
#pragma unroll
            for (int jj = 0; jj < 4; jj++) {
                const int j = j0 + jj, m = j / (2 * DB), db = (j >> 1) % DB;
                const int qr1 = 16 * m + 4 * g + tsl; // query row of the transposing read
                const bf16 *t = (j & 1) ? SQ.q : SQ.dO;
                ad[2 * jj] = lds_byte(&t[swz<D>(qr1, db * 32 + cpart)]);
                ad[2 * jj + 1] = lds_byte(&t[swz<D>(qr1 + 8, db * 32 + cpart)]);
            }
            u32x2 r[8];
            lds_tr8(r, ad);
#pragma unroll
            for (int jj = 0; jj < 4; jj++) {
                const int j = j0 + jj, m = j / (2 * DB), db = (j >> 1) % DB;
                const bf16x8 fa = as_bf16x8(u32x4{r[2 * jj][0], r[2 * jj][1], r[2 * jj + 1][0], r[2 * jj + 1][1]});
                if (j & 1) acc2[db] = mfma32(fa, sb[m], acc2[db]);
                else acc[db] = mfma32(fa, pb[m], acc[db]);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    // Accumulating wave p: keys 32p..32p+31 of the block's dS tile `dst`
    // ([key][query] in LDS) go to the dS buffer ([query][key] rows of P
    // elements; dQ = dS K is a separate product).  The transposing reads give
    // each lane 8 consecutive keys of its query (lq): one 16-byte store per
    // 16-key step.
    const int64_t P_ds = ((int64_t)L + DS_PAD - 1) / DS_PAD * DS_PAD;
    bf16 *ds_plane = DQA ? nullptr : a.ds + a.ds_base[b_seq] + (int64_t)h * P_ds * P_ds;
    auto ds_store = [&](const bf16 *dst, int q0m) {
        uint32_t ad[4];
#pragma unroll
        for (int tt = 0; tt < 2; tt++) {
            const int kr1 = 16 * (2 * p + tt) + 8 * g + tsl;
            ad[2 * tt] = lds_byte(&dst[kr1 * SS + cpart]);
            ad[2 * tt + 1] = lds_byte(&dst[(kr1 + 4) * SS + cpart]);
        }
        u32x2 r[4];
        lds_tr4(r, ad);
#pragma unroll
        for (int tt = 0; tt < 2; tt++) {
            const int t = 2 * p + tt;
            *(u32x4 *)(ds_plane + (int64_t)(q0m + lq) * P_ds + k0 + 16 * t + 8 * g) =
                u32x4{r[2 * tt][0], r[2 * tt][1], r[2 * tt + 1][0], r[2 * tt + 1][1]};
        }
    };
    // DQA, accumulating wave: dQ of the block at q0m from the dS tile `dst`
    // (all 128 keys): dQ[32 queries][d-block p] = sum over the keys of
    // dS[q][key] K[key][d], added to the fp32 accumulator with atomics.
    auto dq_block = [&](const bf16 *dst, int q0m, bool full) {
        if constexpr (DB < 4)
            if (p >= DB) return; // (wave-uniform) d-block p does not exist
        floatx16 qacc;
#pragma unroll
        for (int r = 0; r < 16; r++) qacc[r] = 0.f;
#pragma unroll
        for (int t = 0; t < BN / 16; t++) {
            const int kr1 = 16 * t + 8 * g + tsl;
            const u32x2 s1 = lds_read_tr(&dst[kr1 * SS + cpart]);
            const u32x2 s2 = lds_read_tr(&dst[(kr1 + 4) * SS + cpart]);
            qacc = mfma32(as_bf16x8(u32x4{s1[0], s1[1], s2[0], s2[1]}), opnd[DQA ? t : 0], qacc);
        }
        // C layout: lane holds d = 32p + lq, queries 8(r/4) + 4g + r%4
        float *dqp = a.dq_acc + (int64_t)(o_b + q0m + 4 * g) * ld_do + h * D + 32 * p + lq;
        const int qlim = full ? BQ : L - q0m - 4 * g;
#pragma unroll
        for (int r = 0; r < 16; r++) {
            const int qq = 8 * (r >> 2) + (r & 3);
            if (qq < qlim) atomicAdd(dqp + (int64_t)qq * ld_do, qacc[r]);
        }
    };
    // Accumulating waves: drab_p of the block at q0m from its skewed tile
    // (row c = diagonal c, key - query = k0 - q0m + c - (BQ - 1); cells
    // outside the tile's keys are never written and stay 0).  One thread per
    // row; threads past the last diagonal take the all-zero row DK - 1.  The
    // ring entry is flushed once no later block can reach it (key - query >
    // k0 + BN - 1 - (q0m + BQ)  <=>  c > BN - 2).
    auto drabp_sum = [&](const float *dsk, int q0m, float &tot, int &dl) {
        const int c = tid < DK - 1 ? tid : DK - 1;
        const floatx4 *rowp = (const floatx4 *)(dsk + c * DKP);
        floatx4 acc4 = rowp[0];
#pragma unroll
        for (int i = 1; i < BQ / 4; i++) acc4 += rowp[i];
        const float sum = (acc4[0] + acc4[1]) + (acc4[2] + acc4[3]);
        dl = k0 - q0m + c - (BQ - 1);
        const int slot = dl & (RING - 1);
        tot = sm.ring[slot] + sum;
        sm.ring[slot] = c > BN - 2 ? 0.f : tot;
    };
    // A finished sum goes to this item's slot of partial sums (indexed by
    // key - query in [k0 - (L - 1), 0], the causal values this key tile
    // meets; drab_reduce_kernel adds the slots in a fixed order), or, for a
    // sequence whose slots did not fit, into drab_p with an atomic add.
    auto put_p = [&](int dl, float v) {
        const int64_t pb = a.pbase[b_seq]; // (reloaded here: nothing stays live across the loop)
        if (pb >= 0) {
            const int tk = k0 / BN, ntk = (L + BN - 1) / BN;
            if (dl <= 0 && dl >= k0 - (L - 1)) a.dpart[pb + ((int64_t)h * ntk + tk) * L + (L - 1) + dl] = v;
        } else if (v != 0.f) {
            const int cl = dl < -a.N ? -a.N : (dl > a.N ? a.N : dl);
            atomicAdd(&a.drab_p[h * p_hs + cl + a.N], v);
        }
    };
    auto drabp_flush = [&](int dl, float tot) {
        if (tid < DK - 1 && tid > BN - 2) put_p(dl, tot); // (the zero row DK - 1 is nobody's)
    };

    // ---- one query block.  MAIN: a block in the middle of the range (every
    // wave is past its diagonal block, this, the previous and the next block
    // are full), compiled without the per-block checks.
    const int nqb = (L - k0 + BQ - 1) / BQ; // query blocks [k0, L); >= 1
    const int krow = 32 * p + lq;
    // What every wave does at the end of block n: for a partial next block,
    // the register path of its stage and tables (64-bit times: the pointwise
    // waves store the next block's tables); then the wait and the barrier.
    // The accumulating waves (copies) wait for their direct copies, the
    // pointwise waves only for their LDS traffic.
    auto finish = [&](auto main_c, int n, bool copies) {
        constexpr bool MAIN = decltype(main_c)::value;
        const int q0 = k0 + n * BQ;
        const bool part = !MAIN && n + 1 < nqb && q0 + 2 * BQ > L; // the next block is partial
        if (part) {
            const int n3 = n % 3 == 2 ? 0 : n % 3 + 1;
            load_partial(q0 + BQ, sm.sq[n3], sm.sp[(n + 1) & 1]);
            if constexpr (TM != 2) {
                gload_tables(q0 + BQ, tid);
                sstore_tables(sm.sp[(n + 1) & 1], tid);
            }
        }
        if constexpr (TM == 2)
            if (!copies && (MAIN || n + 1 < nqb)) sstore_tables(sm.sp[(n + 1) & 1], tid - NT / 2);
        if (copies || part) __builtin_amdgcn_s_waitcnt(0);
        else __builtin_amdgcn_s_waitcnt(0xC07F); // lgkmcnt(0)
        __syncthreads();
    };
    // The next block's direct copies, issued by the accumulating waves at the
    // start of the block (their buffers were last read in the block before).
    auto start_copy = [&](auto main_c, int n) {
        constexpr bool MAIN = decltype(main_c)::value;
        const int q0 = k0 + n * BQ;
        const int n3 = n % 3 == 2 ? 0 : n % 3 + 1;
        if (MAIN || (n + 1 < nqb && q0 + 2 * BQ <= L)) {
            gload_direct(half_waves, w, q0 + BQ, sm.sq[n3], sm.sp[(n + 1) & 1]);
            if constexpr (TM != 2) gload_tables_direct(q0 + BQ, sm.sp[(n + 1) & 1]);
        }
    };
    // Accumulating wave, block n: the next block's copies, the previous
    // block's dS store (or dQ), drab_p, dV and dK.  (The atomic-dQ variant
    // issues the copies after its transposing reads: its dQ products read dS
    // with the builtin.)
    auto iter_acc = [&](auto main_c, int n) {
        constexpr bool MAIN = decltype(main_c)::value;
        const int q0 = k0 + n * BQ;
        int dlf = 0;
        float tot = 0.f;
        const int q0m = q0 - BQ;
        // the next block's copies first (a whole block to land)
        if constexpr (!DQA) start_copy(main_c, n);
        // the LDS/VALU work first and the MFMAs last, so that the pointwise
        // wave's X products meet an idle MFMA pipe after the barrier
        if (MAIN || n > 0) {
            if constexpr (DQA) dq_block(sm.ds[(n - 1) & 1], q0m, MAIN ? true : q0 <= L);
            else ds_store(sm.ds[(n - 1) & 1], q0m);
        }
        if (MAIN || n > 0)
            if (a.drab_p) drabp_sum(sm.dsk[(n - 1) & 1], q0m, tot, dlf);
        if (MAIN || n > 0) {
            const bool skipm = MAIN ? false : (kw0 > q0m + BQ - 1 || kw0 >= L);
            if (!skipm) acc_block(sm.sq[n % 3 == 0 ? 2 : n % 3 - 1], (n - 1) & 1);
        }
        if constexpr (DQA) start_copy(main_c, n);
        if ((MAIN || n > 0) && a.drab_p) drabp_flush(dlf, tot);
        finish(main_c, n, true);
    };
    // Pointwise wave, block n: X, dP, P', dS.
    int rb = 0;              // running drab_t sums of buckets rb, rb + 1 (rb wave-uniform;
    float rs0 = 0.f, rs1 = 0.f; // the sums per lane, reduced over the wave when flushed)
    auto iter_pw = [&](auto main_c, int n) {
        constexpr bool MAIN = decltype(main_c)::value;
        const int q0 = k0 + n * BQ;
        if constexpr (TM == 2)
            if (n + 1 < nqb) gload_tables(q0 + BQ, tid - NT / 2);
        const StageQD &SQn = sm.sq[n % 3];
        const StagePD &SPn = sm.sp[n & 1];
        const bool skip = MAIN ? false : (kw0 > q0 + BQ - 1 || kw0 >= L);
        const bool diag = MAIN ? false : kw0 + 31 > q0;
        ln.dsk = sm.dsk[n & 1] + (krow + (BQ - 1) - 4 * g - 27) * DKP + lq;
        bf16 *dsn = sm.ds[n & 1], *ptn = sm.pt[n & 1];
        if (!skip) {
            // X = rab_p window + Q K^T (the window is the products' initial
            // accumulator; operand reads two steps ahead of the MFMAs, pinned
            // with scheduling groups).  dP = dO' V^T (hi + lo planes) is
            // issued inside the element-wise step, whose X-only part overlaps
            // it.
            floatx16 xacc, pacc;
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int cr = 8 * (r >> 2) + (r & 3);
                xacc[r] = HP ? SPn.win[krow + (BQ - 1) - 4 * g - cr] : 0.f;
                pacc[r] = 0.f;
            }
            bf16x8 fd[3], fl[3]; // dP operands, read two steps ahead
            auto fetch_dp = [&](int s) {
                const int o = swz<D>(lq, s * 16 + g * 8);
                fd[s % 3] = *(const bf16x8 *)&SQn.dO[o];
                fl[s % 3] = *(const bf16x8 *)&SPn.dOl[o];
            };
            __builtin_amdgcn_sched_barrier(0);
            {
                bf16x8 fq[3];
                auto fetch = [&](int s) { fq[s % 3] = *(const bf16x8 *)&SQn.q[swz<D>(lq, s * 16 + g * 8)]; };
                fetch(0);
                fetch(1);
#pragma unroll
                for (int s = 0; s < KS; s++) {
                    if (s + 2 < KS) fetch(s + 2);
                    xacc = mfma32(fq[s % 3], slice8(acc2[s >> 1], 4 * (s & 1)), xacc);
                }
                fetch_dp(0);
                fetch_dp(1);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0); // Q reads of steps 0, 1
#pragma unroll
                for (int s = 0; s < KS; s++) {
                    if (s + 2 < KS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0); // read of step s + 2
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                 // MFMA of step s
                }
                __builtin_amdgcn_sched_group_barrier(0x100, 4, 0); // dP operands of steps 0, 1
            }
            __builtin_amdgcn_sched_barrier(0);
            auto dp_step = [&](int s) {
                if (s >= KS) return; // (D < 128: the products fill the first KS steps)
                const bf16x8 d0 = fd[s % 3], d1 = fl[s % 3];
                if (s + 2 < KS) fetch_dp(s + 2);
                pacc = mfma32(d0, slice8(acc2[s >> 1], 8 + 4 * (s & 1)), pacc);
                pacc = mfma32(d1, slice8(acc2[s >> 1], 8 + 4 * (s & 1)), pacc);
            };
            ln.qt = &SPn.qt[4 * g];
            ln.qt64 = &SPn.qt64[4 * g];
            ln.dmask = kw0 + lq - q0 - 4 * g; // key > query  <=>  cr < dmask
            int ubk = 0, nbk = 0; // the block's lowest time bucket; its number of buckets - 1
            if constexpr (TM == 1) {
                // bucket range from floor(log2(min|dt| + 1)) and floor(log2(max|dt| + 1));
                // relative times of one non-wide sequence differ by less than 2^32 - 1
                nbk = 2;
                const uint32_t qa = __builtin_amdgcn_readfirstlane(SPn.qtmin);
                const uint32_t qb = __builtin_amdgcn_readfirstlane(SPn.qtmax);
                if (qa <= qb && tkmin <= tkmax) {
                    const uint32_t lo = tkmin > qb ? tkmin - qb : (qa > tkmax ? qa - tkmax : 0u);
                    const uint32_t h1 = qb > tkmin ? qb - tkmin : 0u, h2 = tkmax > qa ? tkmax - qa : 0u;
                    const uint32_t hi = h1 > h2 ? h1 : h2;
                    const int blo = floor_log2_u32(lo + 1u), bhi = floor_log2_u32(hi + 1u);
                    ubk = blo;
                    nbk = bhi - blo;
                }
            }
            const float ubias = sm.rabt[ubk], ubias2 = sm.rabt[ubk + 1]; // ubk <= 31
            const uint32_t thr = ubk < 31 ? 2u << ubk : 0xFFFFFFFFu;      // 2^(ubk + 1)
            float tsum = 0.f, tsum2 = 0.f;
            uint32_t ppk[8], dpk[8];
            if (diag)
                pointwise<TM, DT, true, TB_ANY>(xacc, pacc, dp_step, ppk, dpk, ln, sm.rabt_rev, sm.rabt, ubias, ubias2, thr, tsum, tsum2, ptn + krow * SS + 4 * g);
            else if (TM == 1 && nbk == 0)
                pointwise<TM, DT, false, TB_ONE>(xacc, pacc, dp_step, ppk, dpk, ln, sm.rabt_rev, sm.rabt, ubias, ubias2, thr, tsum, tsum2, ptn + krow * SS + 4 * g);
            else if (TM == 1 && nbk == 1)
                pointwise<TM, DT, false, TB_TWO>(xacc, pacc, dp_step, ppk, dpk, ln, sm.rabt_rev, sm.rabt, ubias, ubias2, thr, tsum, tsum2, ptn + krow * SS + 4 * g);
            else
                pointwise<TM, DT, false, TB_ANY>(xacc, pacc, dp_step, ppk, dpk, ln, sm.rabt_rev, sm.rabt, ubias, ubias2, thr, tsum, tsum2, ptn + krow * SS + 4 * g);
            // dS -> LDS as [key][query]: lane writes 4 queries (r%4) per r/4 group
#pragma unroll
            for (int gr = 0; gr < 4; gr++) *(u32x2 *)&dsn[krow * SS + 8 * gr + 4 * g] = u32x2{dpk[2 * gr], dpk[2 * gr + 1]};
            // the lane's drab_t sums of this block (buckets ubk, ubk + 1) join
            // its running sums rs0, rs1 of buckets rb, rb + 1; when the block's
            // buckets differ, both running sums are first reduced over the wave
            // and go to the wave's LDS table (lane 0, plain read-modify-write).
            // One rarely taken branch: cheaper than carrying rs1 over when the
            // buckets move up by one (measured).
            if (DT && TM == 1 && nbk <= 1 && !diag) {
                const float v_up = nbk == 1 ? tsum2 : 0.f;
                if (ubk != rb) { // (rare: the buckets moved on) both running sums to the wave's table
                    const float f0 = wave_sum_dpp(rs0), f1 = wave_sum_dpp(rs1);
                    if (l == 0) {
                        sm.dtab[p][0][rb] += f0;
                        sm.dtab[p][0][rb + 1] += f1;
                    }
                    rb = ubk;
                    rs0 = 0.f;
                    rs1 = 0.f;
                }
                rs0 += tsum - v_up;
                rs1 += v_up;
            }
        } else {
#pragma unroll
            for (int gr = 0; gr < 4; gr++) *(u32x2 *)&dsn[krow * SS + 8 * gr + 4 * g] = u32x2{0u, 0u};
#pragma unroll
            for (int rr = 0; rr < 16; rr++) ln.dsk[DKP * (27 - (8 * (rr >> 2) + (rr & 3)))] = 0.f;
        }
        finish(main_c, n, false);
    };

    // The two roles run separate loops (so that each keeps only its own
    // registers live) with the same blocks and barriers: generic blocks at
    // both ends, main blocks in between.
    const std::integral_constant<bool, false> generic{};
    const std::integral_constant<bool, true> fast{};
    const int n_main_end = nqb - 2; // main blocks: [4, nqb - 2)
    auto run = [&](auto body) {
        int n = 0;
        if constexpr (TM == 2) { // sequences with a time span beyond 32 bits: rare, generic path only
            for (; n < nqb; n++) body(generic, n);
        } else {
            for (; n < nqb && (n < 4 || n >= n_main_end); n++) body(generic, n);
            for (; n < n_main_end; n++) body(fast, n);
            for (; n < nqb; n++) body(generic, n);
        }
    };
    const int qlast = k0 + (nqb - 1) * BQ;
    if (awave) {
        run(iter_acc);
        // the last block's dV, dK, dQ and drab_p, then dV^T and dK^T: lane
        // holds key mykey, d = 32 db + 8(r/4) + 4g + r%4 (stored here so that
        // the accumulators are dead on the pointwise waves' path)
        const bool skipm = kw0 > qlast + BQ - 1 || kw0 >= L;
        if (!skipm) acc_block(sm.sq[(nqb - 1) % 3], (nqb - 1) & 1);
        if constexpr (DQA) dq_block(sm.ds[(nqb - 1) & 1], qlast, qlast + BQ <= L);
        else ds_store(sm.ds[(nqb - 1) & 1], qlast);
        if (a.drab_p) {
            int dlf = 0;
            float tot = 0.f;
            drabp_sum(sm.dsk[(nqb - 1) & 1], qlast, tot, dlf);
            drabp_flush(dlf, tot);
        }
        if (kvalid) {
            const int64_t row = o_b + mykey;
            bf16 *dvp = a.dv + row * a.lddv + h * D, *dkp = a.dk + row * a.lddk + h * D;
#pragma unroll
            for (int db = 0; db < DB; db++)
#pragma unroll
                for (int gr = 0; gr < 4; gr++) {
                    const int d0 = db * 32 + 8 * gr + 4 * g;
                    const u32x2 vv = {pack2_bf16(NLN2 * acc[db][4 * gr], NLN2 * acc[db][4 * gr + 1]),
                                      pack2_bf16(NLN2 * acc[db][4 * gr + 2], NLN2 * acc[db][4 * gr + 3])};
                    const u32x2 kk = {pack2_bf16(acc2[db][4 * gr], acc2[db][4 * gr + 1]),
                                      pack2_bf16(acc2[db][4 * gr + 2], acc2[db][4 * gr + 3])};
                    *(u32x2 *)(dvp + d0) = vv;
                    *(u32x2 *)(dkp + d0) = kk;
                }
        }
    } else {
        run(iter_pw);
        if (DT && TM == 1) {
            const float f0 = wave_sum_dpp(rs0), f1 = wave_sum_dpp(rs1);
            if (l == 0) {
                sm.dtab[p][0][rb] += f0;
                sm.dtab[p][0][rb + 1] += f1;
            }
        }
    }

    // what is left in the ring and the time tables
    __syncthreads();
    if (a.drab_p) {
        // remaining key - query values: [k0 - qlast - (BQ - 1), k0 + BN - 1 - qlast - BQ]
        const int lo = k0 - qlast - (BQ - 1), hi = k0 + BN - 1 - qlast - BQ;
        for (int dl = lo + tid; dl <= hi; dl += NT) put_p(dl, sm.ring[dl & (RING - 1)]);
    }
    if constexpr (DT && TM != 0) {
        if (tid < TB) { // this item's slot of drab_t partial sums (added up by drab_reduce_kernel)
            float s = 0.f;
            for (int pp = 0; pp < 4; pp++)
                for (int c = 0; c < TCOPY; c++) s += sm.dtab[pp][c][tid];
            const int tk = k0 / BN, ntk = (L + BN - 1) / BN;
            a.tpart[a.tbase[b_seq] + ((int64_t)h * ntk + tk) * TB_SLOTS + tid] = s;
        }
    }
}

} // namespace

// TMODE: 0 = no time bias; 1 = time bias with drab_t; 2 = time bias without
// drab_t.  Sequences whose time span does not fit 32 bits take the exact
// 64-bit body.
template <int D, bool HP, int TMODE>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2))) attn_bwd_bf16_kernel(AttnBwdArgs a)
{
    extern __shared__ __align__(16) unsigned char smem_raw[];
    Smem<D> &sm = *reinterpret_cast<Smem<D> *>(smem_raw);
    const int item = blockIdx.x;
    if (item >= *a.n_items) return;
    const int2 it = a.items[item];
    const int b = it.x, tsched = it.y >> ITEM_T_SHIFT, h = it.y & 255; // never split
    const int o_b = a.offsets[b];
    const int L = a.offsets[b + 1] - o_b;
    const int nkt = (L + BN - 1) / BN;
    const int k0 = (nkt - 1 - tsched) * BN; // most expensive key tile (k0 = 0) first
    const int tid = threadIdx.x;
    if constexpr (TMODE != 0) {
        if (tid < 128) sm.rabt[tid] = NLOG2E * a.rab_t[h * a.rt_hs + tid];
        if (tid < 32) sm.rabt_rev[tid] = NLOG2E * a.rab_t[h * a.rt_hs + 31 - tid];
    } else {
        if (tid < 128) sm.rabt[tid] = 0.f;
        if (tid < 32) sm.rabt_rev[tid] = 0.f;
    }
    // (the first barrier inside bwd_body orders these writes before use)
    constexpr bool DT = TMODE == 1;
    const bool dqa = a.ds_base[b] < 0; // this sequence's dS planes did not fit: dQ by atomics
    if constexpr (TMODE == 0) {
        if (dqa) bwd_body<D, HP, 0, false, true>(a, sm, b, o_b, L, k0, h);
        else bwd_body<D, HP, 0, false, false>(a, sm, b, o_b, L, k0, h);
    } else if (a.wide[b] != 0) {
        if (dqa) bwd_body<D, HP, 2, DT, true>(a, sm, b, o_b, L, k0, h);
        else bwd_body<D, HP, 2, DT, false>(a, sm, b, o_b, L, k0, h);
    } else {
        if (dqa) bwd_body<D, HP, 1, DT, true>(a, sm, b, o_b, L, k0, h);
        else bwd_body<D, HP, 1, DT, false>(a, sm, b, o_b, L, k0, h);
    }
}

namespace {
template <int D, bool HP, int TMODE>
hipError_t launch_variant(const AttnBwdArgs &a, int max_items, hipStream_t st)
{
    static bool init = false;
    const size_t smem = sizeof(Smem<D>);
    if (!init) {
        hipError_t e = hipFuncSetAttribute((const void *)attn_bwd_bf16_kernel<D, HP, TMODE>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        if (e != hipSuccess) return e;
        init = true;
    }
    hipLaunchKernelGGL((attn_bwd_bf16_kernel<D, HP, TMODE>), dim3(max_items), dim3(NT), smem, st, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const AttnBwdArgs &a, int max_items, hipStream_t st)
{
    const bool has_t = a.ts != nullptr && a.rab_t != nullptr;
    const int tmode = !has_t ? 0 : (a.drab_t ? 1 : 2);
    if (a.rab_p) {
        if (tmode == 0) return launch_variant<D, true, 0>(a, max_items, st);
        if (tmode == 1) return launch_variant<D, true, 1>(a, max_items, st);
        return launch_variant<D, true, 2>(a, max_items, st);
    }
    if (tmode == 0) return launch_variant<D, false, 0>(a, max_items, st);
    if (tmode == 1) return launch_variant<D, false, 1>(a, max_items, st);
    return launch_variant<D, false, 2>(a, max_items, st);
}
} // namespace

hipError_t launch_attn_bwd_bf16(const AttnBwdArgs &a, int d, int max_items, hipStream_t st)
{
    if (max_items <= 0) return hipSuccess;
    switch (d) {
    case 128: return launch_d<128>(a, max_items, st);
    case 64: return launch_d<64>(a, max_items, st);
    case 32: return launch_d<32>(a, max_items, st);
    default: return hipErrorInvalidValue;
    }
}

// ---------------------------------------------------------------------------
// The bias gradients from the items' partial sums, added in a fixed order,
// so that drab_p and drab_t do not depend on the order in which items ran.
//
// drab_t[h][bucket] = the sum over the items' slots: one wave per entry;
// lane l adds tiles t = l, l + 64, ... of every sequence (in order of
// sequence and t), then a butterfly over the lanes (a fixed tree, the same
// on every lane).  Buckets from TB_SLOTS on are never reached and get 0.
__device__ void drab_t_reduce(const DrabReduceArgs &r, int h, int bk, int lane)
{
    float s = 0.f;
    // per-sequence tile counts and slot bases, 64 sequences at a time (one
    // per lane, read back with uniform lane reads); the first tile loads of
    // eight sequences are issued together, then added in order
    if (bk < TB_SLOTS)
        for (int b0 = 0; b0 < r.B; b0 += 64) {
            const int bl = b0 + lane;
            const int ntl = bl < r.B ? (r.offsets[bl + 1] - r.offsets[bl] + BWD_BN - 1) / BWD_BN : 0;
            const int64_t tbl = bl < r.B ? r.tbase[bl] : 0;
            const int nb = min(64, r.B - b0);
            for (int jb0 = 0; jb0 < nb; jb0 += 8) {
                float v[8];
                const float *sl[8];
                int ntu[8];
#pragma unroll
                for (int u = 0; u < 8; u++) {
                    const int jb = min(jb0 + u, nb - 1);
                    const int nt = jb0 + u < nb ? __builtin_amdgcn_readlane(ntl, jb) : 0;
                    const int64_t tb = ((int64_t)__builtin_amdgcn_readlane((int)(tbl >> 32), jb) << 32) |
                                       (uint32_t)__builtin_amdgcn_readlane((int)tbl, jb);
                    sl[u] = r.tpart + (nt > 0 ? tb + (int64_t)h * nt * TB_SLOTS + bk : 0);
                    ntu[u] = nt;
                    v[u] = lane < nt ? sl[u][(int64_t)lane * TB_SLOTS] : 0.f;
                }
#pragma unroll
                for (int u = 0; u < 8; u++) {
                    s += v[u];
                    for (int t = lane + 64; t < ntu[u]; t += 64) s += sl[u][(int64_t)t * TB_SLOTS];
                }
            }
        }
    s = wave_sum(s);
    if (lane == 0) r.drab_t[h * r.t_hs + bk] = s;
}

constexpr int RED_G = 16;
// drab_p[h][idx] += the sum of the slot entries for key - query x = idx - N
// (idx 0 collects every x <= -N) over the items that cover it.  A workgroup
// takes 64 entries of one head; its 16 waves split the key tiles by residue
// (wave g adds tiles t = g, g + 16, ... of every sequence, in order of
// sequence, x and t), then lane i of wave 0 adds the 16 wave sums in order
// of g.  drab_p was zeroed by the launcher; items of a sequence without
// slots added their share with atomics.  Entries idx > N (key after query)
// are never reached.
// One launch for both tables: workgroups x < np (np = 0 without drab_p)
// reduce drab_p, the rest drab_t (one wave per bucket).
__global__ void __launch_bounds__(64 * RED_G) drab_reduce_kernel(DrabReduceArgs r, int np)
{
    __shared__ float part[RED_G][64];
    if (*r.status) return;
    const int h = blockIdx.y, lane = threadIdx.x & 63, g = threadIdx.x >> 6;
    if ((int)blockIdx.x >= np) { // (workgroup-uniform)
        drab_t_reduce(r, h, ((int)blockIdx.x - np) * RED_G + g, lane);
        return;
    }
    const int idx = blockIdx.x * 64 + lane;
    const bool valid = idx <= r.N;
    const int dl = idx - r.N;
    float acc = 0.f;
    // per-sequence slot bases and lengths, 64 sequences at a time, one per
    // lane; the loop reads them back with uniform lane reads.  Entries idx > 0
    // take one x per sequence: the first four tiles' loads of eight sequences
    // are issued together, then added in order (sequence, tile); idx = 0
    // (every x <= -N) takes the general loop.
    for (int b0 = 0; b0 < r.B; b0 += 64) {
        const int bl = b0 + lane;
        const int64_t pbl = bl < r.B ? r.pbase[bl] : -1;
        const int Ll = bl < r.B ? r.offsets[bl + 1] - r.offsets[bl] : 0;
        const int nb = min(64, r.B - b0);
        for (int jb0 = 0; jb0 < nb; jb0 += 8) {
            float v[8][4];
            int tmx[8];
            const float *sl[8];
#pragma unroll
            for (int u = 0; u < 8; u++) {
                const int jb = min(jb0 + u, nb - 1);
                const int64_t pb = ((int64_t)__builtin_amdgcn_readlane((int)(pbl >> 32), jb) << 32) |
                                   (uint32_t)__builtin_amdgcn_readlane((int)pbl, jb);
                const int L = __builtin_amdgcn_readlane(Ll, jb);
                const bool ok = jb0 + u < nb && valid && idx > 0 && pb >= 0 && L > 0 && -dl <= L - 1;
                const int nt = (L + BWD_BN - 1) / BWD_BN;
                sl[u] = r.dpart + (ok ? pb + (int64_t)h * nt * L + (L - 1) + dl : 0);
                tmx[u] = ok ? min(nt - 1, (dl + L - 1) / BWD_BN) : -1;
                const int Ls = ok ? L : 0;
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int t = g + RED_G * i;
                    v[u][i] = t <= tmx[u] ? sl[u][(int64_t)t * Ls] : 0.f;
                }
            }
#pragma unroll
            for (int u = 0; u < 8; u++) {
                const int L = __builtin_amdgcn_readlane(Ll, min(jb0 + u, nb - 1));
#pragma unroll
                for (int i = 0; i < 4; i++) acc += v[u][i];
                for (int t = g + 4 * RED_G; t <= tmx[u]; t += RED_G) acc += sl[u][(int64_t)t * L];
            }
        }
        if (idx == 0) // (lane 0 of the first workgroup of each head: x = -N down to -(L - 1))
            for (int jb = 0; jb < nb; jb++) {
                const int64_t pb = ((int64_t)__builtin_amdgcn_readlane((int)(pbl >> 32), jb) << 32) |
                                   (uint32_t)__builtin_amdgcn_readlane((int)pbl, jb);
                const int L = __builtin_amdgcn_readlane(Ll, jb);
                if (pb < 0 || L <= 0 || -dl > L - 1) continue;
                const int nt = (L + BWD_BN - 1) / BWD_BN;
                const float *slot = r.dpart + pb + (int64_t)h * nt * L + (L - 1);
                for (int x = dl; x >= -(L - 1); x--) {
                    const int tmax = min(nt - 1, (x + L - 1) / BWD_BN);
                    for (int t = g; t <= tmax; t += RED_G) acc += slot[(int64_t)t * L + x];
                }
            }
    }
    part[g][lane] = acc;
    __syncthreads();
    if (g == 0 && valid) {
        float s = 0.f;
#pragma unroll
        for (int k = 0; k < RED_G; k++) s += part[k][lane];
        r.drab_p[h * r.p_hs + idx] += s;
    }
}

hipError_t launch_drab_reduce(const DrabReduceArgs &r, hipStream_t st)
{
    const int np = r.drab_p ? (r.N + 1 + 63) / 64 : 0, nt = r.drab_t ? 128 / RED_G : 0;
    if (np + nt > 0) hipLaunchKernelGGL(drab_reduce_kernel, dim3(np + nt, r.H), dim3(64 * RED_G), 0, st, r, np);
    return hipGetLastError();
}
