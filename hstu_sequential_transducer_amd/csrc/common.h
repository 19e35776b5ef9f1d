// common.h -- device-side helpers shared by the gfx950 kernels of libhstu.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define DEV static __device__ __forceinline__

// Round-to-nearest-even fp32 -> bf16 (v_cvt_pk_bf16_f32 on gfx950).
DEV bf16 to_bf16(float x) { return (bf16)x; }
DEV float from_bf16(bf16 x) { return (float)x; }

// Two fp32 -> one dword of two bf16 (lo in bits 0..15), round to nearest even:
// a single v_cvt_pk_bf16_f32.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
DEV uint32_t pack2_bf16(float lo, float hi)
{
    const bf16x2 r = __builtin_convertvector((f32x2){lo, hi}, bf16x2);
    return __builtin_bit_cast(uint32_t, r);
}

DEV float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
DEV float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// 32x32x16 bf16 MFMA.  Lane l supplies A[l%32][8*(l/32) .. +8] and
// B[8*(l/32) .. +8][l%32]; C register r of lane l is
// C[8*(r/4) + 4*(l/32) + r%4][l%32].
DEV floatx16 mfma32(bf16x8 a, bf16x8 b, floatx16 c) { return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0); }

DEV bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// SiLU(x) = x * sigmoid(x) with the hardware exp2 and reciprocal.
DEV float silu_f(float x)
{
    float e = __builtin_amdgcn_exp2f(x * -1.4426950408889634f);
    return x * __builtin_amdgcn_rcpf(1.0f + e);
}

// floor(log2(x)) for x >= 1 (32-bit), via count of leading zeros.
DEV int floor_log2_u32(uint32_t x) { return 31 - __builtin_clz(x); }

// Exact time bucket min(127, floor(log2(|dt| + 1))) of an int64 difference.
DEV int time_bucket64(int64_t dt)
{
    uint64_t m = dt < 0 ? (uint64_t)0 - (uint64_t)dt : (uint64_t)dt;
    m += 1u;
    int b = 63 - __builtin_clzll(m);
    return b < 127 ? b : 127;
}

DEV float wave_sum(float v)
{
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// Status bits written by the schedule kernel into the workspace.
enum { HSTU_DEV_BAD_OFFSETS = 1, HSTU_DEV_TOO_LONG = 2 };
