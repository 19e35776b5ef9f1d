// sl.hip -- Stochastic Length sampling as a device gather (review of
// "Actions Speak Louder than Words", section 3, Stochastic Length): every
// user's history of n actions is cut to L = min(n, ceil(n u^(1/alpha)))
// actions, a random subsequence, and the sampled batch is built jagged (no
// padding) for the attention path.  The subsequence is the L actions with
// the smallest random keys (ties by position), kept in their order: a
// uniformly random subset when the keys are uniform.  The random numbers
// (u per sequence, a 32-bit key per action) are inputs.
//
//   sl_len_kernel     one workgroup: L_b for every sequence (fp64 pow), the
//                     sampled batch's offsets by a block-wide scan.
//   sl_select_kernel  one workgroup per sequence: the L-th smallest key by
//                     four 8-bit radix passes over LDS histograms, then the
//                     kept positions in order by block-wide scans, written
//                     as source rows.
//   sl_gather_kernel  one wave per sampled row: the row's bytes (and time).
#include "kernels.h"

namespace {

constexpr int NT = 1024;
constexpr int KPT = 8; // keys per thread held in registers (histories up to NT * KPT actions)

// Exclusive prefix sum over the 1024 threads (int); `tmp` holds 16 wave totals.
__device__ int block_excl(int v, int *tmp, int *total)
{
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    int incl = v;
    for (int o = 1; o < 64; o <<= 1) {
        const int x = __shfl_up(incl, o, 64);
        if (lane >= o) incl += x;
    }
    __syncthreads();
    if (lane == 63) tmp[wv] = incl;
    __syncthreads();
    int before = 0, all = 0;
    for (int k = 0; k < 16; k++) {
        before += k < wv ? tmp[k] : 0;
        all += tmp[k];
    }
    *total = all;
    return before + incl - v;
}

__device__ int sl_length(int n, double u, double inv_alpha)
{
    if (n <= 0) return 0;
    const double x = ceil((double)n * pow(u, inv_alpha));
    return x < 1.0 ? 1 : (x > (double)n ? n : (int)x);
}

} // namespace

__global__ void __launch_bounds__(NT) sl_len_kernel(const int32_t *__restrict__ off, int B, int T, double inv_alpha,
                                                    const double *__restrict__ u, int32_t *__restrict__ out_off,
                                                    int *__restrict__ status)
{
    __shared__ int tmp[16];
    __shared__ int bad;
    const int tid = threadIdx.x;
    if (tid == 0) bad = (off[0] != 0 || off[B] != T) ? HSTU_DEV_BAD_OFFSETS : 0;
    __syncthreads();
    for (int b = tid; b < B; b += NT)
        if (off[b + 1] < off[b]) atomicOr(&bad, HSTU_DEV_BAD_OFFSETS);
    __syncthreads();
    if (bad) {
        if (tid == 0) *status = bad;
        return;
    }
    int base = 0;
    for (int b0 = 0; b0 < B; b0 += NT) {
        const int b = b0 + tid;
        const int L = b < B ? sl_length(off[b + 1] - off[b], u[b], inv_alpha) : 0;
        int tot;
        const int ex = block_excl(L, tmp, &tot);
        if (b < B) out_off[b] = base + ex;
        base += tot;
    }
    if (tid == 0) {
        out_off[B] = base;
        *status = 0;
    }
}

__global__ void __launch_bounds__(NT) sl_select_kernel(const int32_t *__restrict__ off, const uint32_t *__restrict__ keys,
                                                       const int32_t *__restrict__ out_off, int32_t *__restrict__ out_idx,
                                                       const int *__restrict__ status)
{
    __shared__ int hist[256];
    __shared__ int tmp[16];
    __shared__ uint32_t s_prefix;
    __shared__ int s_k;
    if (*status) return;
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int o = off[b], n = off[b + 1] - o;
    const int w0 = out_off[b], L = out_off[b + 1] - w0;
    if (L <= 0) return;
    // Histories of at most NT * KPT actions keep their keys in registers,
    // KPT consecutive positions per thread (all loads issued at once); longer
    // ones re-read the keys from memory in every pass.
    const bool reg = n <= NT * KPT;
    uint32_t kr[KPT];
    if (reg) {
#pragma unroll
        for (int i = 0; i < KPT; i++) kr[i] = keys[o + min(tid * KPT + i, n - 1)];
    }
    // the threshold: the L-th smallest key K (prefix) and how many keys equal
    // to K are kept (k), by radix passes over the bits from the top
    uint32_t prefix = 0;
    int k = L;
    if (L < n) {
        for (int shift = 24; shift >= 0; shift -= 8) {
            for (int i = tid; i < 256; i += NT) hist[i] = 0;
            __syncthreads();
            const uint32_t hmask = shift == 24 ? 0u : (0xFFFFFFFFu << (shift + 8));
            if (reg) {
#pragma unroll
                for (int i = 0; i < KPT; i++)
                    if (tid * KPT + i < n && (kr[i] & hmask) == prefix) atomicAdd(&hist[(kr[i] >> shift) & 255], 1);
            } else {
                for (int j = tid; j < n; j += NT) {
                    const uint32_t key = keys[o + j];
                    if ((key & hmask) == prefix) atomicAdd(&hist[(key >> shift) & 255], 1);
                }
            }
            __syncthreads();
            // the bin d holding the k-th key: counts before d < k <= counts
            // up to d (an inclusive scan of the 256 bins by the first four
            // waves; empty bins never qualify, so exactly one bin does)
            int v = 0, incl = 0;
            if (tid < 256) {
                v = hist[tid];
                incl = v;
                for (int sh = 1; sh < 64; sh <<= 1) {
                    const int x = __shfl_up(incl, sh, 64);
                    if (lane >= sh) incl += x;
                }
                if (lane == 63) tmp[wv] = incl;
            }
            __syncthreads();
            if (tid < 256) {
                int before = 0;
                for (int w = 0; w < wv; w++) before += tmp[w];
                const int cin = before + incl, cex = cin - v;
                if (cex < k && k <= cin) {
                    s_prefix = prefix | ((uint32_t)tid << shift);
                    s_k = k - cex;
                }
            }
            __syncthreads();
            prefix = s_prefix;
            k = s_k;
        }
    } else {
        prefix = 0xFFFFFFFFu; // keep every action
        k = n;
    }
    // kept: key < K, or key == K among the first k such positions.  A kept
    // position's rank among the kept ones is (#keys < K before it) +
    // min(#keys == K before it, k): one scan of both counts, packed.
    if (reg) {
        int cl = 0, ce = 0;
#pragma unroll
        for (int i = 0; i < KPT; i++) {
            const bool valid = tid * KPT + i < n;
            cl += valid && (L == n || kr[i] < prefix) ? 1 : 0;
            ce += valid && L < n && kr[i] == prefix ? 1 : 0;
        }
        int tot;
        const int ex = block_excl(cl | (ce << 16), tmp, &tot);
        int lt_before = ex & 0xFFFF, eq_before = ex >> 16;
#pragma unroll
        for (int i = 0; i < KPT; i++) {
            const int j = tid * KPT + i;
            const bool valid = j < n;
            const bool lt = valid && (L == n || kr[i] < prefix), eq = valid && L < n && kr[i] == prefix;
            if (lt || (eq && eq_before < k)) out_idx[w0 + lt_before + min(eq_before, k)] = o + j;
            lt_before += lt ? 1 : 0;
            eq_before += eq ? 1 : 0;
        }
        return;
    }
    int run_lt = 0, run_eq = 0;
    for (int j0 = 0; j0 < n; j0 += NT) {
        const int j = j0 + tid;
        bool lt = false, eq = false;
        if (j < n) {
            const uint32_t key = keys[o + j];
            lt = L == n || key < prefix;
            eq = L < n && key == prefix;
        }
        int tot;
        const int ex = block_excl((lt ? 1 : 0) | (eq ? 1 << 16 : 0), tmp, &tot);
        const int eq_before = run_eq + (ex >> 16);
        if (lt || (eq && eq_before < k)) out_idx[w0 + run_lt + (ex & 0xFFFF) + min(eq_before, k)] = o + j;
        run_lt += tot & 0xFFFF;
        run_eq += tot >> 16;
    }
}

// Sampled row r (one wave): src row out_idx[r]; `bytes` per row, 16-byte
// copies when rows and bases allow them.
__global__ void __launch_bounds__(256) sl_gather_kernel(const int32_t *__restrict__ out_off, int B,
                                                        const int32_t *__restrict__ out_idx, const char *__restrict__ x,
                                                        int64_t ldx_bytes, char *__restrict__ y, int64_t ldy_bytes,
                                                        int64_t bytes, bool vec, const int64_t *__restrict__ ts,
                                                        int64_t *__restrict__ ts_out, const int *__restrict__ status)
{
    if (*status) return;
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (r >= out_off[B]) return;
    const int64_t src = out_idx[r];
    if (ts_out && lane == 0) ts_out[r] = ts[src];
    if (!x) return;
    const char *s = x + src * ldx_bytes;
    char *d = y + r * ldy_bytes;
    if (vec)
        for (int64_t c = 16 * lane; c < bytes; c += 1024) *(u32x4 *)(d + c) = *(const u32x4 *)(s + c);
    else
        for (int64_t c = lane; c < bytes; c += 64) d[c] = s[c];
}

hipError_t launch_sl_sample(const SlArgs &a, hipStream_t st)
{
    hipLaunchKernelGGL(sl_len_kernel, dim3(1), dim3(NT), 0, st, a.offsets, a.B, a.T, 1.0 / a.alpha, a.u, a.out_off,
                       a.status);
    if (a.B > 0)
        hipLaunchKernelGGL(sl_select_kernel, dim3(a.B), dim3(NT), 0, st, a.offsets, a.keys, a.out_off, a.out_idx,
                           a.status);
    if (a.T > 0 && (a.x || a.ts_out)) {
        const bool vec = ((((uintptr_t)a.x) | ((uintptr_t)a.y) | (uintptr_t)a.ldx_bytes | (uintptr_t)a.ldy_bytes |
                           (uintptr_t)a.row_bytes) & 15) == 0;
        hipLaunchKernelGGL(sl_gather_kernel, dim3((a.T + 3) / 4), dim3(256), 0, st, a.out_off, a.B, a.out_idx,
                           (const char *)a.x, a.ldx_bytes, (char *)a.y, a.ldy_bytes, a.row_bytes, vec, a.ts, a.ts_out,
                           a.status);
    }
    return hipGetLastError();
}
