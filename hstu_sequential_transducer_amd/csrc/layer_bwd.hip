// layer_bwd.hip -- the parts of the HSTU layer backward outside the attention
// (review of "Actions Speak Louder than Words", section 3: the chain rule
// through Eq. 1's f1 and phi1, Eq. 3's f2 and the residual between layers).
//
//   weight gradients   dW[m][n] = sum_t A[t][m] B[t][n]  (dW2 = dY^T G,
//                      dW1 = dZ^T X): a sum over all T tokens of two
//                      token-major operands, split over token ranges, fp32
//                      partial tiles, then a reduction over the splits
//   phi1'              dZ = dA (.) phi1'(Z) in place, with per-block column
//                      sums (db1); the same kernel without phi1 gives db2
//   transposes         W1^T, W2^T, so dG = dY W2 and dX = dZ W1 + dY run on
//                      the layer GEMM (both of its operands K-contiguous)
//
// Weight-gradient GEMM: 256 x 128 output tile per workgroup of 4 waves, each
// wave 64 rows x 128 columns (2 x 4 blocks of 32x32x16 bf16 MFMA computing
// dW^T, a lane owning one row m and 4 consecutive columns per register
// group).  Tokens (the K dimension) advance 32 at a time through three LDS
// stages filled by direct global -> LDS copies two steps ahead.  Both
// operands are stored token-major, so the LDS tiles are [token][m] and
// [token][n] (256-byte rows, 16-byte chunks XOR-swizzled per row) and both
// MFMA operands come from transposing LDS reads (ds_read_b64_tr_b16), which
// deliver the same permutation of the 16 tokens of a sub-step to both.
// Token ranges are multiples of 32 except the last; in its partial step the
// B fragments' entries past the end are zeroed in registers (A's rows there
// re-read the last token, finite data times zero).
#include "kernels.h"

#include <cstddef>

namespace {

constexpr int WBM = 256, WBN = 128, WBK = 32, WSTAGES = 3, WNT = 256;

struct alignas(16) WStage {
    alignas(16) bf16 a[2][WBK * 128]; // A^T halves: [token][128 m]
    alignas(16) bf16 b[WBK * 128];    // [token][128 n]
};

// 256-byte rows: 16-byte chunk c of row r at c ^ sw(r), sw(r) = 4(r%4) +
// bitrev2((r/4)%4), conflict-free for the transposing reads below.
DEV int swf(int row)
{
    const int hi = (row >> 2) & 3;
    return ((row & 3) << 2) | ((hi & 1) << 1) | (hi >> 1);
}
DEV int swz(int row, int col) { return row * 128 + (((col >> 3) ^ swf(row)) << 3) + (col & 7); }

typedef __attribute__((address_space(3))) void lds_void;

// Twelve transposing LDS reads (ds_read_b64_tr_b16) at byte addresses
// ad[q] + OFF, waited for inside the same block.  Inside each group of 16
// lanes, lane i receives element i%4 of the 4-element chunks addressed by
// lanes i/4, i/4+4, i/4+8, i/4+12 (in that order).  Written as one asm block
// because the compiler, not seeing which stage a transposing read touches,
// would otherwise wait for every copy still flying into the other stages.
template <int OFF>
DEV void lds_read_tr12(u32x2 (&r)[12], const uint32_t (&ad)[12])
{
    asm volatile("ds_read_b64_tr_b16 %0, %12 offset:%24\n\t"
                 "ds_read_b64_tr_b16 %1, %13 offset:%24\n\t"
                 "ds_read_b64_tr_b16 %2, %14 offset:%24\n\t"
                 "ds_read_b64_tr_b16 %3, %15 offset:%24\n\t"
                 "ds_read_b64_tr_b16 %4, %16 offset:%24\n\t"
                 "ds_read_b64_tr_b16 %5, %17 offset:%24\n\t"
                 "ds_read_b64_tr_b16 %6, %18 offset:%24\n\t"
                 "ds_read_b64_tr_b16 %7, %19 offset:%24\n\t"
                 "ds_read_b64_tr_b16 %8, %20 offset:%24\n\t"
                 "ds_read_b64_tr_b16 %9, %21 offset:%24\n\t"
                 "ds_read_b64_tr_b16 %10, %22 offset:%24\n\t"
                 "ds_read_b64_tr_b16 %11, %23 offset:%24\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]),
                   "=&v"(r[7]), "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11])
                 : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5]), "v"(ad[6]), "v"(ad[7]),
                   "v"(ad[8]), "v"(ad[9]), "v"(ad[10]), "v"(ad[11]), "i"(OFF)
                 : "memory");
}

// Zero the bf16 entries of tokens >= kvalid; the 4 entries hold tokens
// kbase .. kbase + 3.
DEV u32x2 mask_tokens(u32x2 v, int kbase, int kvalid)
{
#pragma unroll
    for (int h = 0; h < 2; h++) {
        const uint32_t lo = (kbase + 2 * h < kvalid) ? 0x0000FFFFu : 0u;
        const uint32_t hi = (kbase + 2 * h + 1 < kvalid) ? 0xFFFF0000u : 0u;
        v[h] &= (lo | hi);
    }
    return v;
}

} // namespace

__global__ void __launch_bounds__(WNT) __attribute__((amdgpu_waves_per_eu(2, 2)))
gemm_wgrad_kernel(WgradArgs g, int tiles_n, int n_tiles, int per_xcd)
{
    __shared__ WStage st[WSTAGES];
    // workgroup -> (split, tile): consecutive workgroups go to different XCDs,
    // and each XCD takes the tiles of one or two whole splits, which share
    // their token rows through its L2
    const int t = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    if (t >= n_tiles * g.splits) return;
    const int split = t / n_tiles, tile = t - split * n_tiles;
    const int mt = tile / tiles_n, nt = tile - mt * tiles_n;
    const int m0 = mt * WBM, n0 = nt * WBN;
    const int k_lo = split * g.chunk, k_hi = min(k_lo + g.chunk, g.K);
    const int nk = (k_hi - k_lo + WBK - 1) / WBK;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, gq = l >> 5, lq = l & 31;
    const int tj = l & 15, tsl = tj >> 2;
    const int cpart = ((l >> 4) & 1) * 16 + 4 * (tj & 3);
    const bf16 *A = (const bf16 *)g.A, *B = (const bf16 *)g.B;

    // copies of step kt into stage S: 24 instructions of 4 rows x 256 bytes,
    // A halves 0..15, B 16..23; wave w issues 4w .. 4w+3 (A) and 2w, 2w+1 (B).
    // Per lane: token row (l / 16 within the instruction's 4 rows) and a
    // column offset; the step's first token goes into a uniform base.  Rows
    // past K (only in the last step) re-read token K - 1.
    int rowa[4], cola[4], rowb[2], colb[2];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int idx = 4 * w + i, half = idx >> 3;
        rowa[i] = 4 * (idx & 7) + (l >> 4);
        cola[i] = min(m0 + 128 * half + 8 * ((l & 15) ^ swf(rowa[i])), g.M - 8);
    }
#pragma unroll
    for (int i = 0; i < 2; i++) {
        rowb[i] = 4 * (2 * w + i) + (l >> 4);
        colb[i] = min(n0 + 8 * ((l & 15) ^ swf(rowb[i])), g.N - 8);
    }
    auto gload = [&](int kt, WStage &S) {
        const int k0 = k_lo + kt * WBK;
        const bf16 *Ak = A + (int64_t)k0 * g.lda, *Bk = B + (int64_t)k0 * g.ldb;
        const bool tail = k0 + WBK > g.K;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int idx = 4 * w + i, half = idx >> 3, r0 = 4 * (idx & 7);
            const int r = tail ? min(rowa[i], g.K - 1 - k0) : rowa[i];
            __builtin_amdgcn_global_load_lds((const void *)(Ak + (int64_t)r * g.lda + cola[i]),
                                             (lds_void *)(S.a[half] + r0 * 128), 16, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const int r0 = 4 * (2 * w + i);
            const int r = tail ? min(rowb[i], g.K - 1 - k0) : rowb[i];
            __builtin_amdgcn_global_load_lds((const void *)(Bk + (int64_t)r * g.ldb + colb[i]),
                                             (lds_void *)(S.b + r0 * 128), 16, 0, 0);
        }
    };
    constexpr int CPW = 6; // copies per wave per stage

    floatx16 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0.f;

    // one step of 32 tokens: 2 sub-steps of 16.  A fragment i: rows
    // m = 64w + 32i + lane%32; B fragment j: rows n = 32j + lane%32; both
    // hold tokens 16ks + {4g .. 4g+3, 8+4g .. 8+4g+3} in that order.  The
    // lane's byte offsets inside a stage (sub-step 1 adds 16 rows = 4096
    // bytes): A (i, +8 rows) at offs[2i + h], B (j, +8 rows) at offs[4 + 2j + h].
    uint32_t offs[12];
    {
        const int key1 = 4 * gq + tsl;
#pragma unroll
        for (int h = 0; h < 2; h++) {
#pragma unroll
            for (int i = 0; i < 2; i++)
                offs[2 * i + h] = (uint32_t)(offsetof(WStage, a) +
                                             2 * ((w >> 1) * WBK * 128 + swz(key1 + 8 * h, 64 * (w & 1) + 32 * i + cpart)));
#pragma unroll
            for (int j = 0; j < 4; j++)
                offs[4 + 2 * j + h] = (uint32_t)(offsetof(WStage, b) + 2 * swz(key1 + 8 * h, 32 * j + cpart));
        }
    }
    const uint32_t st_base = (uint32_t)(uintptr_t)(lds_void *)&st[0];
    auto compute = [&](int stage, int kvalid) {
        uint32_t ad[12];
        const uint32_t sb = st_base + (uint32_t)(stage * (int)sizeof(WStage));
#pragma unroll
        for (int q = 0; q < 12; q++) ad[q] = sb + offs[q];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < 2; ks++) {
            u32x2 r[12];
            if (ks == 0) lds_read_tr12<0>(r, ad);
            else lds_read_tr12<4096>(r, ad);
            bf16x8 af[2], bfr[4];
#pragma unroll
            for (int i = 0; i < 2; i++) af[i] = as_bf16x8(u32x4{r[2 * i][0], r[2 * i][1], r[2 * i + 1][0], r[2 * i + 1][1]});
#pragma unroll
            for (int j = 0; j < 4; j++) {
                u32x2 r1 = r[4 + 2 * j], r2 = r[5 + 2 * j];
                if (kvalid < WBK) {
                    r1 = mask_tokens(r1, 16 * ks + 4 * gq, kvalid);
                    r2 = mask_tokens(r2, 16 * ks + 8 + 4 * gq, kvalid);
                }
                bfr[j] = as_bf16x8(u32x4{r1[0], r1[1], r2[0], r2[1]});
            }
#pragma unroll
            for (int j = 0; j < 4; j++)
#pragma unroll
                for (int i = 0; i < 2; i++) acc[i][j] = mfma32(bfr[j], af[i], acc[i][j]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    if (nk > 0) gload(0, st[0]);
    if (nk > 1) gload(1, st[1]);
    for (int kt = 0; kt < nk; kt++) {
        // this wave's copies of step kt are in LDS (those of kt + 1 may still
        // fly); the barrier then makes every wave's copies visible and
        // guarantees the stage overwritten below is no longer read (every
        // wave's reads of it finished inside their read blocks)
        if (kt + 1 < nk) __builtin_amdgcn_s_waitcnt(0x0F70 | CPW); // vmcnt(CPW)
        else __builtin_amdgcn_s_waitcnt(0x0F70);                   // vmcnt(0)
        asm volatile("s_barrier" ::: "memory");
        if (kt + 2 < nk) gload(kt + 2, st[(kt + 2) % WSTAGES]);
        compute(kt % WSTAGES, min(WBK, k_hi - (k_lo + kt * WBK)));
    }

    // partial tile of this split: lane owns row m and columns
    // n0 + 32j + 8q + 4gq .. +3 for each (i, j, q)
    float *out = g.part + (int64_t)split * g.M * g.N;
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int m = m0 + 64 * w + 32 * i + lq;
        if (m >= g.M) continue;
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const int n = n0 + 32 * j + 8 * q + 4 * gq;
                if (n >= g.N) continue;
                *(floatx4 *)(out + (int64_t)m * g.N + n) =
                    floatx4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
            }
    }
}

// out[e] = sum_s part[s][e], e in [0, E), E a multiple of 4.  Workgroup = 64
// entries (16 quads) x 16 split phases; the phases meet in LDS.
__global__ void __launch_bounds__(256) sum_splits_kernel(const float *__restrict__ part, int S, int64_t E,
                                                         float *__restrict__ out)
{
    __shared__ floatx4 red[16][16];
    const int quad = threadIdx.x & 15, ph = threadIdx.x >> 4;
    const int64_t e = ((int64_t)blockIdx.x * 16 + quad) * 4;
    floatx4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    if (e < E) {
        int s = ph;
        for (; s + 16 < S; s += 32) {
            s0 += *(const floatx4 *)(part + (int64_t)s * E + e);
            s1 += *(const floatx4 *)(part + (int64_t)(s + 16) * E + e);
        }
        if (s < S) s0 += *(const floatx4 *)(part + (int64_t)s * E + e);
    }
    red[ph][quad] = s0 + s1;
    __syncthreads();
    if (ph == 0 && e < E) {
        floatx4 t = red[0][quad];
#pragma unroll
        for (int p = 1; p < 16; p++) t += red[p][quad];
        *(floatx4 *)(out + e) = t;
    }
}

// ACT: 0 = column sums of a only; 1 = SiLU', 2 = ReLU': a *= phi1'(z) in
// place, then column sums of the product (before its bf16 rounding).
// Workgroup = rows [rows_per_blk * blockIdx.x, ...) of columns
// [2048 blockIdx.y, +2048); a thread takes 8 consecutive columns and every
// P-th row, P = 256 / (column groups of the chunk).  Partial sums go to
// part[blockIdx.x][N].  N is a multiple of 8; rows are 16-byte aligned.
template <int ACT>
__global__ void __launch_bounds__(256) colsum_act_kernel(bf16 *__restrict__ a, int64_t lda,
                                                         const bf16 *__restrict__ z, int64_t ldz, int M, int N,
                                                         int rows_per_blk, float *__restrict__ part)
{
    __shared__ float red[256 * 8];
    const int c0 = 2048 * blockIdx.y;
    const int groups = min(256, (N - c0) / 8);
    const int P = 256 / groups;
    const int tid = threadIdx.x, cg = tid % groups, ph = tid / groups;
    const int r_lo = rows_per_blk * blockIdx.x, r_hi = min(r_lo + rows_per_blk, M);
    const int col = c0 + 8 * cg;
    float s[8];
#pragma unroll
    for (int e = 0; e < 8; e++) s[e] = 0.f;
    if (ph < P) {
        for (int r = r_lo + ph; r < r_hi; r += P) {
            u32x4 av = *(const u32x4 *)(a + (int64_t)r * lda + col);
            if constexpr (ACT != 0) {
                const u32x4 zv = *(const u32x4 *)(z + (int64_t)r * ldz + col);
                u32x4 o;
#pragma unroll
                for (int h = 0; h < 4; h++) {
                    float x[2] = {bf16_lo(av[h]), bf16_hi(av[h])};
                    const float zz[2] = {bf16_lo(zv[h]), bf16_hi(zv[h])};
#pragma unroll
                    for (int e = 0; e < 2; e++) {
                        float gr;
                        if constexpr (ACT == 1) {
                            // SiLU'(z) = sig (1 + z (1 - sig)), sig = 1 / (1 + 2^(-z log2 e))
                            const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(zz[e] * -1.4426950408889634f));
                            gr = sg * (1.0f + zz[e] * (1.0f - sg));
                        } else {
                            gr = zz[e] > 0.f ? 1.f : 0.f;
                        }
                        x[e] *= gr;
                        s[2 * h + e] += x[e];
                    }
                    o[h] = pack2_bf16(x[0], x[1]);
                }
                *(u32x4 *)(a + (int64_t)r * lda + col) = o;
            } else {
#pragma unroll
                for (int h = 0; h < 4; h++) {
                    s[2 * h] += bf16_lo(av[h]);
                    s[2 * h + 1] += bf16_hi(av[h]);
                }
            }
        }
    }
#pragma unroll
    for (int e = 0; e < 8; e++) red[tid * 8 + e] = s[e];
    __syncthreads();
    // thread t < 8 * groups: column c0 + t, summed over the P phases
    for (int t = tid; t < 8 * groups; t += 256) {
        const int g = t / 8, e = t % 8;
        float v = 0.f;
        for (int p = 0; p < P; p++) v += red[(p * groups + g) * 8 + e];
        part[(int64_t)blockIdx.x * N + c0 + t] = v;
    }
}

// out [C][R] = in [R][C]^T, bf16, 64 x 64 tiles through LDS.
__global__ void __launch_bounds__(256) transpose_bf16_kernel(const bf16 *__restrict__ in, int64_t ldi, int R, int C,
                                                             bf16 *__restrict__ out, int64_t ldo)
{
    __shared__ bf16 tile[64][66];
    const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    for (int r = ty; r < 64; r += 4)
        if (r0 + r < R && c0 + tx < C) tile[r][tx] = in[(int64_t)(r0 + r) * ldi + c0 + tx];
    __syncthreads();
    for (int c = ty; c < 64; c += 4)
        if (c0 + c < C && r0 + tx < R) out[(int64_t)(c0 + c) * ldo + r0 + tx] = tile[tx][c];
}

WgradPlan wgrad_plan(int M, int N, int K)
{
    WgradPlan p{};
    const int tiles = ((M + WBM - 1) / WBM) * ((N + WBN - 1) / WBN);
    // about two workgroups per CU, at least 8 steps of 32 tokens per split
    int s = (512 + tiles - 1) / tiles;
    const int smax = (K + 255) / 256;
    s = s < 1 ? 1 : (s > smax ? smax : s);
    if (s < 1) s = 1;
    int chunk = (K + s - 1) / s;
    chunk = (chunk + WBK - 1) / WBK * WBK;
    if (chunk < WBK) chunk = WBK;
    p.chunk = chunk;
    p.splits = K > 0 ? (K + chunk - 1) / chunk : 1;
    return p;
}

hipError_t launch_gemm_wgrad(const WgradArgs &g, hipStream_t st)
{
    if (g.M <= 0 || g.N <= 0) return hipSuccess;
    const int tiles_n = (g.N + WBN - 1) / WBN;
    const int n_tiles = tiles_n * ((g.M + WBM - 1) / WBM);
    const int64_t total = (int64_t)n_tiles * g.splits;
    const int per_xcd = (int)((total + 7) / 8);
    hipLaunchKernelGGL(gemm_wgrad_kernel, dim3(8 * per_xcd), dim3(WNT), 0, st, g, tiles_n, n_tiles, per_xcd);
    return hipGetLastError();
}

hipError_t launch_sum_splits(const float *part, int S, int64_t E, float *out, hipStream_t st)
{
    if (E <= 0) return hipSuccess;
    const int64_t blocks = (E / 4 + 15) / 16;
    hipLaunchKernelGGL(sum_splits_kernel, dim3((unsigned)blocks), dim3(256), 0, st, part, S, E, out);
    return hipGetLastError();
}

int colsum_blocks(int M) { return M > 0 ? (M + COLSUM_ROWS - 1) / COLSUM_ROWS : 0; }

hipError_t launch_colsum_act(bf16 *a, int64_t lda, const bf16 *z, int64_t ldz, int act, int M, int N, float *part,
                             hipStream_t st)
{
    const int nb = colsum_blocks(M);
    if (nb == 0 || N <= 0) return hipSuccess;
    const dim3 grid(nb, (N + 2047) / 2048);
    if (act == 1)
        hipLaunchKernelGGL(colsum_act_kernel<1>, grid, dim3(256), 0, st, a, lda, z, ldz, M, N, COLSUM_ROWS, part);
    else if (act == 2)
        hipLaunchKernelGGL(colsum_act_kernel<2>, grid, dim3(256), 0, st, a, lda, z, ldz, M, N, COLSUM_ROWS, part);
    else
        hipLaunchKernelGGL(colsum_act_kernel<0>, grid, dim3(256), 0, st, a, lda, z, ldz, M, N, COLSUM_ROWS, part);
    return hipGetLastError();
}

hipError_t launch_transpose_bf16(const bf16 *in, int64_t ldi, int R, int C, bf16 *out, int64_t ldo, hipStream_t st)
{
    if (R <= 0 || C <= 0) return hipSuccess;
    hipLaunchKernelGGL(transpose_bf16_kernel, dim3((C + 63) / 64, (R + 63) / 64), dim3(256), 0, st, in, ldi, R, C,
                       out, ldo);
    return hipGetLastError();
}
