// dq.hip -- dQ = dS K, the query gradient of HSTU pointwise aggregated
// attention on gfx950.
//
// Chain rule through Eq. 2 of the review of "Actions Speak Louder than Words"
// (section 3): dQ_i = sum_{j <= i} dS_ij k_j.  The backward kernel writes dS
// (bf16) per sequence b and head h as a P x P plane of [query][key] rows, P =
// L_b rounded up to 128, with zeros wherever j > i; every entry this kernel
// reads for a valid query was written there.  Workgroup = 128 queries of one
// (sequence, head), 4 waves of 32.  Keys stream in tiles of 64 through LDS
// (dS tile [128][64] and K tile [64][d], double buffered, copied global ->
// LDS directly); each wave accumulates dQ^T = K^T dS^T on 32x32x16 bf16 MFMA
// (K^T by transposing LDS reads) and stores bf16 dQ.  The two stages are
// separate LDS objects with the tile loop unrolled by two, so the compiler
// can tell that the transposing reads of one stage never touch the copies
// into the other and issues them without waiting for those copies.
#include "kernels.h"

#include <type_traits>

namespace {

constexpr int BM = 128; // queries per workgroup
constexpr int BK = 64;  // keys per tile
constexpr int NT = 256;

// D: the head size (128, 64 or 32).
template <int D>
struct alignas(16) DqStage {
    alignas(16) bf16 s[BM * BK]; // dS tile [query][key], 128-byte rows
    alignas(16) bf16 k[BK * D];  // K tile [key][d], 2D-byte rows
};

// K tile rows: 16-byte chunk c of row r at c ^ sw(r), sw(r) = 4(r%4) +
// bitrev2((r/4)%4) masked to the row's D/8 chunks (conflict-free
// transposing reads at D = 128).
template <int D>
DEV int swf(int row)
{
    const int hi = (row >> 2) & 3;
    return (((row & 3) << 2) | ((hi & 1) << 1) | (hi >> 1)) & (D / 8 - 1);
}
template <int D>
DEV int swz(int row, int col) { return row * D + (((col >> 3) ^ swf<D>(row)) << 3) + (col & 7); }
// 128-byte rows (dS tile): chunk c of row r at c ^ ((r/2) % 8), so 16
// consecutive rows read at one chunk hit 16 different 16-byte bank groups.
DEV int s8f(int row) { return (row >> 1) & 7; }
DEV int swz8(int row, int col) { return row * BK + (((col >> 3) ^ s8f(row)) << 3) + (col & 7); }

typedef __attribute__((address_space(3))) void lds_void;
typedef short short4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4v lds_short4v;

// Transposing LDS read (ds_read_b64_tr_b16): inside each group of 16 lanes,
// lane i receives element i%4 of the 4-element chunks addressed by lanes
// i/4, i/4+4, i/4+8, i/4+12 (in that order).
DEV u32x2 lds_read_tr(const bf16 *p)
{
    short4v r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v *)(p));
    return __builtin_bit_cast(u32x2, r);
}

} // namespace

template <int D>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2))) dq_gemm_kernel(DqArgs a)
{
    constexpr int DB = D / 32;     // 32-wide d-blocks of dQ^T
    constexpr int NCH = D / 8;     // 16-byte chunks per K row
    constexpr int RPI = 64 / NCH;  // K rows per wave copy instruction
    constexpr int KPW = BK / RPI / 4; // K copy instructions per wave
    __shared__ DqStage<D> st0, st1;
    const int item = blockIdx.x;
    if (item >= *a.n_items) return;
    const int2 it = a.items[item];
    const int b = it.x, qt = it.y >> ITEM_T_SHIFT, h = it.y & 255;
    const int o_b = a.offsets[b];
    const int L = a.offsets[b + 1] - o_b;
    const int q0 = qt * BM;
    if (a.ds_base[b] < 0) {
        // dQ of this sequence went through the fp32 accumulator: convert this
        // tile's rows of head h
        for (int e = threadIdx.x; e < BM * D; e += NT) {
            const int r = e / D, c = e - r * D;
            if (q0 + r < L)
                a.dq[(int64_t)(o_b + q0 + r) * a.lddq + h * D + c] =
                    to_bf16(a.dq_acc[(int64_t)(o_b + q0 + r) * a.ldacc + h * D + c]);
        }
        return;
    }
    const int64_t P = ((int64_t)L + DS_PAD - 1) / DS_PAD * DS_PAD;
    const bf16 *plane = a.ds + a.ds_base[b] + (int64_t)h * P * P;
    const int kend = min(q0 + BM, L);
    const int nkt = (kend + BK - 1) / BK; // keys [0, 64 nkt): written entries of the rows below

    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 5, lq = l & 31;
    const int tj = l & 15, tsl = tj >> 2;
    const int cpart = ((l >> 4) & 1) * 16 + 4 * (tj & 3);

    // copies: dS 16 groups of 8 rows, K BK / RPI groups of RPI rows; 4 + KPW per wave
    auto gload = [&](int kt, DqStage<D> &S) {
        const int kb0 = kt * BK;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int r0 = 8 * (4 * w + i), row = r0 + (l >> 3);
            const int c = (l & 7) ^ s8f(row);
            __builtin_amdgcn_global_load_lds((const void *)(plane + (int64_t)(q0 + row) * P + kb0 + c * 8),
                                             (lds_void *)(S.s + r0 * BK), 16, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < KPW; i++) {
            const int r0 = RPI * (KPW * w + i), row = r0 + l / NCH;
            const int c = (l % NCH) ^ swf<D>(row);
            const int key = min(kb0 + row, L - 1);
            __builtin_amdgcn_global_load_lds((const void *)(a.k + (int64_t)(o_b + key) * a.ldk + h * D + c * 8),
                                             (lds_void *)(S.k + r0 * D), 16, 0, 0);
        }
    };

    floatx16 acc[DB];
#pragma unroll
    for (int i = 0; i < DB; i++)
#pragma unroll
        for (int r = 0; r < 16; r++) acc[i][r] = 0.f;

    // One tile: 4 steps of 16 keys.  B = dS^T fragment of this lane's query,
    // keys 16m + {4g..4g+3, 8+4g..8+4g+3} (the order of the transposing
    // reads' k index); A = K^T for d-block db.
    auto compute = [&](const DqStage<D> &S) {
        const int qrow = 32 * w + lq;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = 0; m < 4; m++) {
            const u32x2 s1 = *(const u32x2 *)&S.s[swz8(qrow, 16 * m) + 4 * g];
            const u32x2 s2 = *(const u32x2 *)&S.s[swz8(qrow, 16 * m + 8) + 4 * g];
            const bf16x8 sb = as_bf16x8(u32x4{s1[0], s1[1], s2[0], s2[1]});
            const int key1 = 16 * m + 4 * g + tsl;
#pragma unroll
            for (int db = 0; db < DB; db++) {
                const u32x2 r1 = lds_read_tr(&S.k[swz<D>(key1, db * 32 + cpart)]);
                const u32x2 r2 = lds_read_tr(&S.k[swz<D>(key1 + 8, db * 32 + cpart)]);
                acc[db] = mfma32(as_bf16x8(u32x4{r1[0], r1[1], r2[0], r2[1]}), sb, acc[db]);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    gload(0, st0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int kt = 0; kt < nkt; kt += 2) {
        if (kt + 1 < nkt) gload(kt + 1, st1);
        compute(st0);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (kt + 1 >= nkt) break;
        if (kt + 2 < nkt) gload(kt + 2, st0);
        compute(st1);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }

    // dQ^T accumulator: lane holds query qrow, d = 32 db + 8(r/4) + 4g + r%4
    const int qrow = q0 + 32 * w + lq;
    if (qrow >= L) return;
    bf16 *out = a.dq + (int64_t)(o_b + qrow) * a.lddq + h * D;
#pragma unroll
    for (int db = 0; db < DB; db++)
#pragma unroll
        for (int gr = 0; gr < 4; gr++) {
            const int d0 = db * 32 + 8 * gr + 4 * g;
            *(u32x2 *)(out + d0) = u32x2{pack2_bf16(acc[db][4 * gr], acc[db][4 * gr + 1]),
                                         pack2_bf16(acc[db][4 * gr + 2], acc[db][4 * gr + 3])};
        }
}

hipError_t launch_dq_gemm(const DqArgs &a, int max_items, hipStream_t st)
{
    if (max_items <= 0) return hipSuccess;
    switch (a.d) {
    case 128: hipLaunchKernelGGL(dq_gemm_kernel<128>, dim3(max_items), dim3(NT), 0, st, a); break;
    case 64: hipLaunchKernelGGL(dq_gemm_kernel<64>, dim3(max_items), dim3(NT), 0, st, a); break;
    case 32: hipLaunchKernelGGL(dq_gemm_kernel<32>, dim3(max_items), dim3(NT), 0, st, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}
