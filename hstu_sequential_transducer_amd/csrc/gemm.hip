// gemm.hip -- the HSTU layer's two linear maps with fused epilogues (review of
// "Actions Speak Louder than Words", section 3: Eq. 1's f1 followed by phi1,
// Eq. 3's f2, and the residual connection between layers; section 5 notes
// the layer has only these 2 linear layers).
//
//   C[m][n] = act(sum_k A[m][k] W[n][k] + bias[n]) + R[m][n]
//
// W is stored [out][in] (y = x W^T + b).  Optional extra outputs: a
// storage-dtype copy of C (the M-FALCON hidden state feeding the next layer)
// and copies of two column ranges (this layer's K and V, the M-FALCON cache).
//
// bf16 kernel: 128x128 output tile per workgroup of 4 waves (64x64 each =
// 2x2 blocks of 32x32x16 bf16 MFMA), K in steps of 32 staged through LDS
// (double buffered).  Both operands are K-contiguous, so no transposes.
// fp32 kernel: plain VALU tiles for fp32 storage (small layers).
#include "kernels.h"

namespace {

constexpr int GBM = 128, GBN = 128, GBK = 32, GNT = 256;
constexpr int GRS = 40; // LDS row stride in bf16 (32 + 8: conflict-free 16-byte reads)

DEV float apply_act(float x, int epi)
{
    if (epi == EPI_SILU) return silu_f(x);
    if (epi == EPI_RELU) return x > 0.f ? x : 0.f;
    return x;
}

template <typename OutT>
DEV void store_out(void *p, int64_t i, float x)
{
    if constexpr (sizeof(OutT) == 2) ((bf16 *)p)[i] = to_bf16(x);
    else ((float *)p)[i] = x;
}

} // namespace

__global__ void __launch_bounds__(GNT) gemm_bf16_kernel(GemmArgs g)
{
    __shared__ __align__(16) bf16 As[2][GBM * GRS];
    __shared__ __align__(16) bf16 Ws[2][GBN * GRS];
    const int m0 = blockIdx.y * GBM, n0 = blockIdx.x * GBN;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, gq = l >> 5, lq = l & 31;
    const int wm = w >> 1, wn = w & 1;
    const bf16 *A = (const bf16 *)g.A, *W = (const bf16 *)g.W;
    const int nk = (g.K + GBK - 1) / GBK;

    // loader: thread -> (row lr, 16-element half lh) of both tiles
    const int lr = tid >> 1, lh = (tid & 1) * 16;
    u32x4 ar[2], wr[2];
    auto gload = [&](int kt) {
        const int k0 = kt * GBK + lh;
        const int am = m0 + lr, wn_ = n0 + lr;
#pragma unroll
        for (int c = 0; c < 2; c++) {
            const int kk = k0 + c * 8;
            const bool ka = am < g.M && kk + 8 <= g.K;
            const bool kw = wn_ < g.N && kk + 8 <= g.K;
            ar[c] = ka ? *(const u32x4 *)(A + (int64_t)am * g.lda + kk) : u32x4{0, 0, 0, 0};
            wr[c] = kw ? *(const u32x4 *)(W + (int64_t)wn_ * g.K + kk) : u32x4{0, 0, 0, 0};
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int c = 0; c < 2; c++) {
            *(u32x4 *)&As[buf][lr * GRS + lh + c * 8] = ar[c];
            *(u32x4 *)&Ws[buf][lr * GRS + lh + c * 8] = wr[c];
        }
    };

    floatx16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0.f;

    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; kt++) {
        if (kt + 1 < nk) gload(kt + 1);
        const bf16 *as = As[kt & 1], *ws = Ws[kt & 1];
#pragma unroll
        for (int ks = 0; ks < GBK / 16; ks++) {
            bf16x8 a[2], b[2];
#pragma unroll
            for (int i = 0; i < 2; i++) a[i] = *(const bf16x8 *)&as[(64 * wm + 32 * i + lq) * GRS + ks * 16 + gq * 8];
#pragma unroll
            for (int j = 0; j < 2; j++) b[j] = *(const bf16x8 *)&ws[(64 * wn + 32 * j + lq) * GRS + ks * 16 + gq * 8];
#pragma unroll
            for (int i = 0; i < 2; i++)
#pragma unroll
                for (int j = 0; j < 2; j++) acc[i][j] = mfma32(a[i], b[j], acc[i][j]);
        }
        if (kt + 1 < nk) sstore((kt + 1) & 1);
        __syncthreads();
    }

    // epilogue: lane holds column n = .. + lq, rows 8(r/4) + 4g + r%4
#pragma unroll
    for (int j = 0; j < 2; j++) {
        const int n = n0 + 64 * wn + 32 * j + lq;
        if (n >= g.N) continue;
        const float bn = g.bias ? g.bias[n] : 0.f;
        const bool to_k = g.Ck && n >= g.k_lo && n < g.k_lo + g.kv_w;
        const bool to_v = g.Cv && n >= g.v_lo && n < g.v_lo + g.kv_w;
#pragma unroll
        for (int i = 0; i < 2; i++) {
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int m = m0 + 64 * wm + 32 * i + 8 * (r >> 2) + 4 * gq + (r & 3);
                if (m >= g.M) continue;
                float x = apply_act(acc[i][j][r] + bn, g.epi);
                if (g.R32) x += g.R32[(int64_t)m * g.ldr + n];
                else if (g.R16) x += from_bf16(((const bf16 *)g.R16)[(int64_t)m * g.ldr + n]);
                if (g.c_f32) store_out<float>(g.C, (int64_t)m * g.ldc + n, x);
                else store_out<bf16>(g.C, (int64_t)m * g.ldc + n, x);
                if (g.C16) store_out<bf16>(g.C16, (int64_t)m * g.ldc16 + n, x);
                if (to_k) store_out<bf16>(g.Ck, (int64_t)m * g.ldck + (n - g.k_lo), x);
                if (to_v) store_out<bf16>(g.Cv, (int64_t)m * g.ldcv + (n - g.v_lo), x);
            }
        }
    }
}

// fp32: 64x64 tile, 256 threads x (4 x 4) outputs, K steps of 16 in LDS.
__global__ void __launch_bounds__(256) gemm_f32_kernel(GemmArgs g)
{
    __shared__ float As[16][64 + 1];
    __shared__ float Ws[16][64 + 1];
    const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
    const int tid = threadIdx.x, tm = (tid >> 4) * 4, tn = (tid & 15) * 4;
    const float *A = (const float *)g.A, *W = (const float *)g.W;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < g.K; k0 += 16) {
        __syncthreads();
        for (int e = tid; e < 64 * 16; e += 256) {
            const int r = e / 16, c = e % 16, k = k0 + c;
            As[c][r] = (m0 + r < g.M && k < g.K) ? A[(int64_t)(m0 + r) * g.lda + k] : 0.f;
            Ws[c][r] = (n0 + r < g.N && k < g.K) ? W[(int64_t)(n0 + r) * g.K + k] : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int c = 0; c < 16; c++)
#pragma unroll
            for (int i = 0; i < 4; i++)
#pragma unroll
                for (int j = 0; j < 4; j++) acc[i][j] = fmaf(As[c][tm + i], Ws[c][tn + j], acc[i][j]);
    }
    for (int i = 0; i < 4; i++) {
        const int m = m0 + tm + i;
        if (m >= g.M) continue;
        for (int j = 0; j < 4; j++) {
            const int n = n0 + tn + j;
            if (n >= g.N) continue;
            float x = acc[i][j] + (g.bias ? g.bias[n] : 0.f);
            if (g.epi == EPI_SILU) x = x / (1.0f + expf(-x));
            else if (g.epi == EPI_RELU) x = x > 0.f ? x : 0.f;
            if (g.R32) x += g.R32[(int64_t)m * g.ldr + n];
            else if (g.R16) x += ((const float *)g.R16)[(int64_t)m * g.ldr + n];
            ((float *)g.C)[(int64_t)m * g.ldc + n] = x;
            if (g.C16) ((float *)g.C16)[(int64_t)m * g.ldc16 + n] = x;
            if (g.Ck && n >= g.k_lo && n < g.k_lo + g.kv_w) ((float *)g.Ck)[(int64_t)m * g.ldck + (n - g.k_lo)] = x;
            if (g.Cv && n >= g.v_lo && n < g.v_lo + g.kv_w) ((float *)g.Cv)[(int64_t)m * g.ldcv + (n - g.v_lo)] = x;
        }
    }
}

hipError_t launch_gemm_bf16(const GemmArgs &g, hipStream_t st)
{
    if (g.M <= 0 || g.N <= 0) return hipSuccess;
    dim3 grid((g.N + GBN - 1) / GBN, (g.M + GBM - 1) / GBM);
    hipLaunchKernelGGL(gemm_bf16_kernel, grid, dim3(GNT), 0, st, g);
    return hipGetLastError();
}

hipError_t launch_gemm_f32(const GemmArgs &g, hipStream_t st)
{
    if (g.M <= 0 || g.N <= 0) return hipSuccess;
    dim3 grid((g.N + 63) / 64, (g.M + 63) / 64);
    hipLaunchKernelGGL(gemm_f32_kernel, grid, dim3(256), 0, st, g);
    return hipGetLastError();
}
