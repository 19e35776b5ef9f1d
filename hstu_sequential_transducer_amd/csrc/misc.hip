// misc.hip -- small memory kernels: zero fill (in place of hipMemsetAsync,
// which must not be recorded into captured graphs), fp32 -> bf16 cast.
#include "kernels.h"

__global__ void __launch_bounds__(256) fill_zero_kernel(uint32_t *__restrict__ p, size_t n_words)
{
    size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    const size_t stride = (size_t)gridDim.x * 256;
    for (; i < n_words; i += stride) p[i] = 0u;
}

hipError_t launch_fill_zero(void *p, size_t bytes, hipStream_t st)
{
    const size_t words = bytes / 4;
    if (words == 0) return hipSuccess;
    size_t blocks = (words + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, st, (uint32_t *)p, words);
    return hipGetLastError();
}

__global__ void __launch_bounds__(256) cast_kernel(const float *__restrict__ src, int64_t lds, bf16 *__restrict__ dst,
                                                   int64_t ldd, int rows, int cols)
{
    const int64_t n = (int64_t)rows * cols;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (; i < n; i += stride) {
        const int64_t r = i / cols, c = i % cols;
        dst[r * ldd + c] = to_bf16(src[r * lds + c]);
    }
}

hipError_t launch_cast_f32_to_bf16(const float *src, int64_t lds, bf16 *dst, int64_t ldd, int rows, int cols,
                                   const int *status, hipStream_t st)
{
    (void)status;
    const int64_t n = (int64_t)rows * cols;
    if (n <= 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(cast_kernel, dim3((unsigned)blocks), dim3(256), 0, st, src, lds, dst, ldd, rows, cols);
    return hipGetLastError();
}

__global__ void __launch_bounds__(256) copy_f32_kernel(const float *__restrict__ s, float *__restrict__ d, size_t n)
{
    size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    const size_t stride = (size_t)gridDim.x * 256;
    for (; i < n; i += stride) d[i] = s[i];
}

hipError_t launch_copy_f32(const float *src, float *dst, size_t n, hipStream_t st)
{
    if (n == 0) return hipSuccess;
    size_t blocks = (n + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(copy_f32_kernel, dim3((unsigned)blocks), dim3(256), 0, st, src, dst, n);
    return hipGetLastError();
}

__global__ void __launch_bounds__(256) scale_bf16_kernel(const bf16 *__restrict__ src, int64_t lds, bf16 *__restrict__ dst,
                                                         int64_t ldd, int rows, int cols, float scale)
{
    const int64_t n = (int64_t)rows * cols;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (; i < n; i += stride) {
        const int64_t r = i / cols, c = i % cols;
        const float x = from_bf16(src[r * lds + c]) * scale;
        const bf16 hi = to_bf16(x);
        dst[r * ldd + c] = hi;
        dst[n + r * ldd + c] = to_bf16(x - from_bf16(hi)); // lo plane (ldd == cols)
    }
}

hipError_t launch_scale_bf16(const bf16 *src, int64_t lds, bf16 *dst, int64_t ldd, int rows, int cols, float scale,
                             hipStream_t st)
{
    const int64_t n = (int64_t)rows * cols;
    if (n <= 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(scale_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, st, src, lds, dst, ldd, rows, cols,
                       scale);
    return hipGetLastError();
}
