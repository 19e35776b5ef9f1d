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

} // namespace

// G = (O - mean) * rstd * U.  O may be given as nparts partial sums spaced
// part_stride floats apart (they are added in order first).  Lane l owns
// features [l*VPL, l*VPL + VPL).
template <int VPL, bool BF>
__global__ void __launch_bounds__(256) ln_gate_fwd_kernel(const float *__restrict__ O, int64_t ldo, int nparts,
                                                          int64_t part_stride, const void *__restrict__ U, int64_t ldu,
                                                          void *__restrict__ G, int64_t ldg, float *__restrict__ stats,
                                                          float *__restrict__ o_copy, int64_t ld_oc, int T, int F,
                                                          float eps)
{
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= T) return;
    float x[VPL];
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < VPL; i++) {
        const int c = lane * VPL + i;
        float v = 0.f;
        if (c < F)
            for (int p = 0; p < nparts; p++) v += O[p * part_stride + (int64_t)row * ldo + c];
        x[i] = v;
        s += v;
    }
    const float mean = wave_sum(s) / (float)F;
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < VPL; i++) {
        const int c = lane * VPL + i;
        const float dlt = x[i] - mean;
        q += c < F ? dlt * dlt : 0.f;
    }
    const float var = wave_sum(q) / (float)F;
    const float rstd = 1.0f / sqrtf(var + eps);
#pragma unroll
    for (int i = 0; i < VPL; i++) {
        const int c = lane * VPL + i;
        if (c >= F) continue;
        const float u = ld_act<BF>(U, (int64_t)row * ldu + c);
        st_act<BF>(G, (int64_t)row * ldg + c, (x[i] - mean) * rstd * u);
        if (o_copy) o_copy[(int64_t)row * ld_oc + c] = x[i];
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
                                                          int64_t lddu, bf16 *__restrict__ dO, float scale, int T, int F)
{
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= T) return;
    const float mean = stats[2 * (int64_t)row], rstd = stats[2 * (int64_t)row + 1];
    float xh[VPL], dxh[VPL];
    float m1 = 0.f, m2 = 0.f;
#pragma unroll
    for (int i = 0; i < VPL; i++) {
        const int c = lane * VPL + i;
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
    m1 = wave_sum(m1) / (float)F;
    m2 = wave_sum(m2) / (float)F;
#pragma unroll
    for (int i = 0; i < VPL; i++) {
        const int c = lane * VPL + i;
        if (c >= F) continue;
        const float g = rstd * (dxh[i] - m1 - xh[i] * m2) * scale;
        const bf16 hi = to_bf16(g);
        dO[(int64_t)row * F + c] = hi;
        dO[(int64_t)T * F + (int64_t)row * F + c] = to_bf16(g - from_bf16(hi));
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
    (void)status;
    if (T <= 0) return hipSuccess;
    dim3 grid((T + 3) / 4);
    if (bf16io)
        VPL_SWITCH(F, hipLaunchKernelGGL((ln_gate_fwd_kernel<V, true>), grid, dim3(256), 0, st, O, ldo, nparts,
                                         part_stride, U, ldu, G, ldg, stats, o_copy, ld_oc, T, F, eps));
    else
        VPL_SWITCH(F, hipLaunchKernelGGL((ln_gate_fwd_kernel<V, false>), grid, dim3(256), 0, st, O, ldo, nparts,
                                         part_stride, U, ldu, G, ldg, stats, o_copy, ld_oc, T, F, eps));
    return hipGetLastError();
}

hipError_t launch_ln_gate_bwd(const void *dG, int64_t ldg, const void *U, int64_t ldu, const float *O, int64_t ldo,
                              const float *stats, bool bf16io, void *dU, int64_t lddu, bf16 *dO, float scale, int T,
                              int F, const int *status, hipStream_t st)
{
    (void)status;
    if (T <= 0) return hipSuccess;
    dim3 grid((T + 3) / 4);
    if (bf16io)
        VPL_SWITCH(F, hipLaunchKernelGGL((ln_gate_bwd_kernel<V, true>), grid, dim3(256), 0, st, dG, ldg, U, ldu, O,
                                         ldo, stats, dU, lddu, dO, scale, T, F));
    else
        VPL_SWITCH(F, hipLaunchKernelGGL((ln_gate_bwd_kernel<V, false>), grid, dim3(256), 0, st, dG, ldg, U, ldu, O,
                                         ldo, stats, dU, lddu, dO, scale, T, F));
    return hipGetLastError();
}
