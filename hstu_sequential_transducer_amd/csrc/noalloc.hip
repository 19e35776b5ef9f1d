// noalloc.hip -- hstu_attn_fwd_noalloc: the forward of hstu_attn_fwd with
// its scratch space in a file-scope device array instead of a caller
// workspace, for callers that cannot allocate device memory.
//
// The array lives in the library's code object: every GPU the library runs
// on holds its own copy (at its own address) until the process ends.  Host
// code never uses the array's name as a device address: the first call on a
// device looks the address up with hipGetSymbolAddress (with that device
// current) and keeps it per device.  Nothing here allocates.  Every call on
// one device shares that device's array, so calls that overlap on one GPU
// (other streams, other threads) race; the forward needs no part of the
// array zeroed beforehand (the launcher writes everything it reads).
#include "kernels.h"

#include <mutex>

static __device__ __align__(256) unsigned char scratch[HSTU_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
void *g_ptr[MAX_DEVICES] = {nullptr};

// This device's copy of `scratch` (looked up once per device).
hstu_status scratch_ptr(void **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= MAX_DEVICES)
        return hstu_internal::set_error(HSTU_ERR_DEVICE, "hstu_attn_fwd_noalloc: no current HIP device");
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return hstu_internal::set_error(HSTU_ERR_DEVICE, "hstu_attn_fwd_noalloc: scratch symbol lookup failed");
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return HSTU_OK;
}

} // namespace

extern "C" hstu_status hstu_attn_fwd_noalloc(const hstu_jagged *j, const hstu_dims *dims, const hstu_bias *bias,
                                             hstu_cmat q, hstu_cmat k, hstu_cmat v, hstu_cmat u, hstu_mat out,
                                             float *o_save, float *ln_stats, void *stream)
{
    size_t need = 0;
    hstu_status s = hstu_internal::attn_fwd_entry(j, dims, bias, q, k, v, u, out, o_save, ln_stats, nullptr, 0,
                                                  stream, true, &need);
    if (s != HSTU_OK) return s;
    if (need > (size_t)HSTU_NOALLOC_SCRATCH_BYTES) {
        char msg[256];
        snprintf(msg, sizeof msg,
                 "hstu_attn_fwd_noalloc: this batch needs %zu bytes of scratch, above the %u-byte limit "
                 "(pass o_save with u, or call hstu_attn_fwd with a workspace)",
                 need, (unsigned)HSTU_NOALLOC_SCRATCH_BYTES);
        return hstu_internal::set_error(HSTU_ERR_WORKSPACE, msg);
    }
    void *ws = nullptr;
    s = scratch_ptr(&ws);
    if (s != HSTU_OK) return s;
    return hstu_internal::attn_fwd_entry(j, dims, bias, q, k, v, u, out, o_save, ln_stats, ws,
                                         (size_t)HSTU_NOALLOC_SCRATCH_BYTES, stream, true, nullptr);
}
