// epilogue.hip -- Norm(AV) (.) U of HSTU's pointwise transformation (review of
// "Actions Speak Louder than Words", section 3, Eq. 3) and its backward.
// Norm is read as LayerNorm over all H*d_v features of a token (no affine,
// biased variance).  One 64-lane wave per token row; statistics by wave
// reductions in fp32.  HBM-bound: each row is read once and written once.
#include "kernels.h"

namespace {

template <bool BF>
DEV float ld_act(const void *p, int64_t i)
{
    if constexpr (BF) return from_bf16(((const bf16 *)p)[i]);
    else return ((const float *)p)[i];
}
template <bool BF>
DEV void st_act(void *p, int64_t i, float x)
{
    if constexpr (BF) ((bf16 *)p)[i] = to_bf16(x);
    else ((float *)p)[i] = x;
}

// VPL consecutive activations at element i (i a multiple of VPL, row bases
// 16-byte aligned): vector loads/stores of 16 bytes where possible.
template <int VPL, bool BF>
DEV void ld_act_vec(const void *p, int64_t i, float (&x)[VPL])
{
    if constexpr (BF && VPL % 8 == 0) {
#pragma unroll
        for (int j = 0; j < VPL; j += 8) {
            const u32x4 w = *(const u32x4 *)((const bf16 *)p + i + j);
#pragma unroll
            for (int k = 0; k < 4; k++) {
                x[j + 2 * k] = bf16_lo(w[k]);
                x[j + 2 * k + 1] = bf16_hi(w[k]);
            }
        }
    } else if constexpr (!BF && VPL % 4 == 0) {
#pragma unroll
        for (int j = 0; j < VPL; j += 4) {
            const floatx4 w = *(const floatx4 *)((const float *)p + i + j);
#pragma unroll
            for (int k = 0; k < 4; k++) x[j + k] = w[k];
        }
    } else {
#pragma unroll
        for (int j = 0; j < VPL; j++) x[j] = ld_act<BF>(p, i + j);
    }
}
template <int VPL, bool BF>
DEV void st_act_vec(void *p, int64_t i, const float (&x)[VPL])
{
    if constexpr (BF && VPL % 8 == 0) {
#pragma unroll
        for (int j = 0; j < VPL; j += 8) {
            const u32x4 w = {pack2_bf16(x[j], x[j + 1]), pack2_bf16(x[j + 2], x[j + 3]), pack2_bf16(x[j + 4], x[j + 5]),
                             pack2_bf16(x[j + 6], x[j + 7])};
            *(u32x4 *)((bf16 *)p + i + j) = w;
        }
    } else if constexpr (!BF && VPL % 4 == 0) {
#pragma unroll
        for (int j = 0; j < VPL; j += 4) *(floatx4 *)((float *)p + i + j) = floatx4{x[j], x[j + 1], x[j + 2], x[j + 3]};
    } else {
#pragma unroll
        for (int j = 0; j < VPL; j++) st_act<BF>(p, i + j, x[j]);
    }
}

} // namespace

// G = (O - mean) * rstd * U.  O may be given as nparts partial sums spaced
// part_stride floats apart (they are added in order first).  Lane l owns
// features [l*VPL, l*VPL + VPL).
template <int VPL, bool BF>
__global__ void __launch_bounds__(256) ln_gate_fwd_kernel(const float *__restrict__ O, int64_t ldo, int nparts,
                                                          int64_t part_stride, const void *__restrict__ U, int64_t ldu,
                                                          void *__restrict__ G, int64_t ldg, float *__restrict__ stats,
                                                          float *__restrict__ o_copy, int64_t ld_oc, int T, int F,
                                                          float eps, bool vec, const int *__restrict__ status)
{
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= T) return;
    if (status && *status) return; // the batch failed the launcher's check: write nothing
    float x[VPL];
    float s = 0.f;
    const int c0 = lane * VPL;
    if (vec) { // F == 64 * VPL, rows 16-byte aligned
        ld_act_vec<VPL, false>(O, (int64_t)row * ldo + c0, x);
        for (int p = 1; p < nparts; p++) {
            float y[VPL];
            ld_act_vec<VPL, false>(O + p * part_stride, (int64_t)row * ldo + c0, y);
#pragma unroll
            for (int i = 0; i < VPL; i++) x[i] += y[i];
        }
#pragma unroll
        for (int i = 0; i < VPL; i++) s += x[i];
    } else {
#pragma unroll
        for (int i = 0; i < VPL; i++) {
            const int c = c0 + i;
            float v = 0.f;
            if (c < F)
                for (int p = 0; p < nparts; p++) v += O[p * part_stride + (int64_t)row * ldo + c];
            x[i] = v;
            s += v;
        }
    }
    const float mean = wave_sum(s) / (float)F;
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < VPL; i++) {
        const int c = c0 + i;
        const float dlt = x[i] - mean;
        q += c < F ? dlt * dlt : 0.f;
    }
    const float var = wave_sum(q) / (float)F;
    const float rstd = 1.0f / sqrtf(var + eps);
    if (vec) {
        float u[VPL], gv[VPL];
        ld_act_vec<VPL, BF>(U, (int64_t)row * ldu + c0, u);
#pragma unroll
        for (int i = 0; i < VPL; i++) gv[i] = (x[i] - mean) * rstd * u[i];
        st_act_vec<VPL, BF>(G, (int64_t)row * ldg + c0, gv);
        if (o_copy) st_act_vec<VPL, false>(o_copy, (int64_t)row * ld_oc + c0, x);
    } else {
#pragma unroll
        for (int i = 0; i < VPL; i++) {
            const int c = c0 + i;
            if (c >= F) continue;
            const float u = ld_act<BF>(U, (int64_t)row * ldu + c);
            st_act<BF>(G, (int64_t)row * ldg + c, (x[i] - mean) * rstd * u);
            if (o_copy) o_copy[(int64_t)row * ld_oc + c] = x[i];
        }
    }
    if (stats && lane == 0) {
        stats[2 * (int64_t)row] = mean;
        stats[2 * (int64_t)row + 1] = rstd;
    }
}

// Backward of G = xhat (.) U, xhat = (O - mean) * rstd:
//   dU = xhat (.) dG ;  dxhat = dG (.) U ;
//   dO = rstd * (dxhat - mean(dxhat) - xhat * mean(dxhat (.) xhat)),
// written as dO * scale (scale = 1/N_max folds phi2's normaliser) in two bf16
// planes, hi = bf16(x) and lo = bf16(x - hi), so that products with dO keep
// ~16 significant bits: plane hi at dO[0 .. T*F), plane lo at dO[T*F .. 2*T*F).
template <int VPL, bool BF>
__global__ void __launch_bounds__(256) ln_gate_bwd_kernel(const void *__restrict__ dG, int64_t ldg, const void *__restrict__ U,
                                                          int64_t ldu, const float *__restrict__ O, int64_t ldo,
                                                          const float *__restrict__ stats, void *__restrict__ dU,
                                                          int64_t lddu, bf16 *__restrict__ dO, float scale, int T, int F,
                                                          bool vec, float *__restrict__ zrows, int zF,
                                                          const int *__restrict__ status)
{
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= T) return;
    if (status && *status) return; // the batch failed the launcher's check: write nothing
    if (zrows)
        for (int c = 4 * lane; c < zF; c += 256) *(floatx4 *)(zrows + (int64_t)row * zF + c) = floatx4{0.f, 0.f, 0.f, 0.f};
    const float mean = stats[2 * (int64_t)row], rstd = stats[2 * (int64_t)row + 1];
    const int c0 = lane * VPL;
    float xh[VPL], dxh[VPL];
    float m1 = 0.f, m2 = 0.f;
    if (vec) {
        float g[VPL], u[VPL], o[VPL], du[VPL];
        ld_act_vec<VPL, BF>(dG, (int64_t)row * ldg + c0, g);
        ld_act_vec<VPL, BF>(U, (int64_t)row * ldu + c0, u);
        ld_act_vec<VPL, false>(O, (int64_t)row * ldo + c0, o);
#pragma unroll
        for (int i = 0; i < VPL; i++) {
            xh[i] = (o[i] - mean) * rstd;
            dxh[i] = g[i] * u[i];
            du[i] = xh[i] * g[i];
            m1 += dxh[i];
            m2 += dxh[i] * xh[i];
        }
        st_act_vec<VPL, BF>(dU, (int64_t)row * lddu + c0, du);
    } else {
#pragma unroll
        for (int i = 0; i < VPL; i++) {
            const int c = c0 + i;
            xh[i] = 0.f;
            dxh[i] = 0.f;
            if (c >= F) continue;
            const float g = ld_act<BF>(dG, (int64_t)row * ldg + c);
            const float u = ld_act<BF>(U, (int64_t)row * ldu + c);
            xh[i] = (O[(int64_t)row * ldo + c] - mean) * rstd;
            dxh[i] = g * u;
            st_act<BF>(dU, (int64_t)row * lddu + c, xh[i] * g);
            m1 += dxh[i];
            m2 += dxh[i] * xh[i];
        }
    }
    m1 = wave_sum(m1) / (float)F;
    m2 = wave_sum(m2) / (float)F;
    float hi[VPL], lo[VPL];
#pragma unroll
    for (int i = 0; i < VPL; i++) {
        const float g = rstd * (dxh[i] - m1 - xh[i] * m2) * scale;
        hi[i] = from_bf16(to_bf16(g));
        lo[i] = g - hi[i];
    }
    if (vec) {
        st_act_vec<VPL, true>(dO, (int64_t)row * F + c0, hi);
        st_act_vec<VPL, true>(dO + (int64_t)T * F, (int64_t)row * F + c0, lo);
    } else {
#pragma unroll
        for (int i = 0; i < VPL; i++) {
            const int c = c0 + i;
            if (c >= F) continue;
            dO[(int64_t)row * F + c] = to_bf16(hi[i]);
            dO[(int64_t)T * F + (int64_t)row * F + c] = to_bf16(lo[i]);
        }
    }
}

#define VPL_SWITCH(F, BODY)                                                                                         \
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

hipError_t launch_ln_gate_fwd(const float *O, int64_t ldo, int nparts, int64_t part_stride, const void *U, int64_t ldu,
                              bool bf16io, void *G, int64_t ldg, float *stats, float *o_copy, int64_t ld_oc, int T,
                              int F, float eps, const int *status, hipStream_t st)
{
    if (T <= 0) return hipSuccess;
    dim3 grid((T + 3) / 4);
    const int64_t es = bf16io ? 2 : 4;
    const bool aligned = (((uintptr_t)O | (uintptr_t)U | (uintptr_t)G | (uintptr_t)o_copy) & 15) == 0 &&
                         (ldo * 4) % 16 == 0 && (ldu * es) % 16 == 0 && (ldg * es) % 16 == 0 &&
                         (ld_oc * 4) % 16 == 0 && (part_stride * 4) % 16 == 0;
    if (bf16io)
        VPL_SWITCH(F, hipLaunchKernelGGL((ln_gate_fwd_kernel<V, true>), grid, dim3(256), 0, st, O, ldo, nparts,
                                         part_stride, U, ldu, G, ldg, stats, o_copy, ld_oc, T, F, eps,
                                         aligned && F == 64 * V && V % 8 == 0, status));
    else
        VPL_SWITCH(F, hipLaunchKernelGGL((ln_gate_fwd_kernel<V, false>), grid, dim3(256), 0, st, O, ldo, nparts,
                                         part_stride, U, ldu, G, ldg, stats, o_copy, ld_oc, T, F, eps,
                                         aligned && F == 64 * V && V % 8 == 0, status));
    return hipGetLastError();
}

hipError_t launch_ln_gate_bwd(const void *dG, int64_t ldg, const void *U, int64_t ldu, const float *O, int64_t ldo,
                              const float *stats, bool bf16io, void *dU, int64_t lddu, bf16 *dO, float scale, int T,
                              int F, float *zrows, int zF, const int *status, hipStream_t st)
{
    if (zrows && ((((uintptr_t)zrows) & 15) != 0 || zF % 4 != 0)) return hipErrorInvalidValue;
    if (T <= 0) return hipSuccess;
    dim3 grid((T + 3) / 4);
    const int64_t es = bf16io ? 2 : 4;
    const bool aligned = (((uintptr_t)dG | (uintptr_t)U | (uintptr_t)O | (uintptr_t)dU | (uintptr_t)dO) & 15) == 0 &&
                         (ldg * es) % 16 == 0 && (ldu * es) % 16 == 0 && (ldo * 4) % 16 == 0 &&
                         (lddu * es) % 16 == 0 && ((int64_t)T * F * 2) % 16 == 0;
    if (bf16io)
        VPL_SWITCH(F, hipLaunchKernelGGL((ln_gate_bwd_kernel<V, true>), grid, dim3(256), 0, st, dG, ldg, U, ldu, O,
                                         ldo, stats, dU, lddu, dO, scale, T, F, aligned && F == 64 * V && V % 8 == 0, zrows, zF, status));
    else
        VPL_SWITCH(F, hipLaunchKernelGGL((ln_gate_bwd_kernel<V, false>), grid, dim3(256), 0, st, dG, ldg, U, ldu, O,
                                         ldo, stats, dU, lddu, dO, scale, T, F, aligned && F == 64 * V && V % 8 == 0, zrows, zF, status));
    return hipGetLastError();
}
