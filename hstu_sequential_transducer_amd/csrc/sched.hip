// sched.hip -- the launcher: validates the jagged offsets, orders the work
// longest-first and converts timestamps to sequence-relative 32-bit values.
//
// The pages attribute HSTU's speed to computing only real tokens (review of
// "Actions Speak Louder than Words", section 4 innovations table: a sparse,
// efficient kernel; section 3 Stochastic Length).  Here that means: no
// padding anywhere, items only for tiles that hold real tokens, and the most
// expensive items first so the tail of the launch is short.
#include "kernels.h"

// One workgroup of 1024 threads.  An item is (sequence b, tile t, head h);
// a tile t of sequence b costs t + 1 units (causal), so items are ordered by
// t descending.  With pi = the sequences sorted by tile count descending,
// the sequences that have a tile t form a prefix of pi, hence
//   index(b, t, h) = H * (S[t] + pos_pi(b)) + h,
//   S[t] = #items with a larger tile index / H = sum_{t' > t} #{b : n_b > t'}.
// Ties inside a length class are broken by an atomic counter; the results
// of every kernel are independent of the order.
__global__ void __launch_bounds__(1024) sched_kernel(const int32_t *__restrict__ offsets, int B, int T, int tile, int H,
                                                      int *__restrict__ status, int *__restrict__ n_items,
                                                      int2 *__restrict__ items, int max_items)
{
    __shared__ int hist[SCHED_BINS];
    __shared__ int fill[SCHED_BINS];
    __shared__ int S[SCHED_BINS];
    __shared__ int bad;
    __shared__ int chunk_tot[1024];
    const int tid = threadIdx.x;
    for (int i = tid; i < SCHED_BINS; i += 1024) {
        hist[i] = 0;
        fill[i] = 0;
    }
    if (tid == 0) bad = (offsets[0] != 0 || offsets[B] != T) ? HSTU_DEV_BAD_OFFSETS : 0;
    __syncthreads();
    for (int b = tid; b < B; b += 1024) {
        int L = offsets[b + 1] - offsets[b];
        if (L < 0) atomicOr(&bad, HSTU_DEV_BAD_OFFSETS);
        int n = L > 0 ? (L + tile - 1) / tile : 0;
        if (n >= SCHED_BINS) atomicOr(&bad, HSTU_DEV_TOO_LONG);
        else atomicAdd(&hist[n], 1);
    }
    __syncthreads();
    if (bad) {
        if (tid == 0) {
            *status = bad;
            *n_items = 0;
        }
        return;
    }
    // cnt_gt[t] = #{b : n_b > t} = sum_{v > t} hist[v]  (suffix sum, in place
    // into fill[]), then S[t] = sum_{t' > t} cnt_gt[t'].  Each thread owns a
    // contiguous chunk of bins; chunk totals are combined serially by thread 0.
    const int per = SCHED_BINS / 1024;
    {
        int s = 0;
        for (int i = per - 1; i >= 0; i--) s += hist[tid * per + i];
        chunk_tot[tid] = s;
    }
    __syncthreads();
    if (tid == 0) {
        int run = 0;
        for (int c = 1023; c >= 0; c--) {
            int v = chunk_tot[c];
            chunk_tot[c] = run; // exclusive suffix: sum of the chunks above c
            run += v;
        }
    }
    __syncthreads();
    {
        int run = chunk_tot[tid];
        for (int i = per - 1; i >= 0; i--) {
            int t = tid * per + i;
            fill[t] = run; // = #{b : n_b > t}
            run += hist[t];
        }
    }
    __syncthreads();
    {
        int s = 0;
        for (int i = per - 1; i >= 0; i--) s += fill[tid * per + i];
        chunk_tot[tid] = s;
    }
    __syncthreads();
    if (tid == 0) {
        int run = 0;
        for (int c = 1023; c >= 0; c--) {
            int v = chunk_tot[c];
            chunk_tot[c] = run;
            run += v;
        }
        *n_items = run * H; // sum_t cnt_gt[t] = sum_b n_b
        *status = 0;
    }
    __syncthreads();
    {
        int run = chunk_tot[tid];
        for (int i = per - 1; i >= 0; i--) {
            int t = tid * per + i;
            S[t] = run;
            run += fill[t];
        }
    }
    __syncthreads();
    // pos_pi(b) = #{b' : n_b' > n_b} + rank among equal n; hist[] becomes the
    // per-class fill counter.
    for (int i = tid; i < SCHED_BINS; i += 1024) hist[i] = 0;
    __syncthreads();
    for (int b = tid; b < B; b += 1024) {
        int L = offsets[b + 1] - offsets[b];
        int n = L > 0 ? (L + tile - 1) / tile : 0;
        if (n == 0) continue;
        int pos = fill[n] + atomicAdd(&hist[n], 1);
        for (int t = 0; t < n; t++) {
            int base = H * (S[t] + pos);
            for (int h = 0; h < H; h++) {
                int idx = base + h;
                if (idx < max_items) items[idx] = make_int2(b, (t << 8) | h);
            }
        }
    }
}

// One workgroup per sequence: rel[r] = ts[r] - min(ts of the sequence) as a
// 32-bit value when the sequence's time span fits (span <= 2^32 - 2, so
// |t_i - t_j| + 1 fits in 32 bits); otherwise wide[b] = 1 and the kernels use
// exact 64-bit arithmetic for that sequence.
__global__ void __launch_bounds__(256) reltime_kernel(const int32_t *__restrict__ offsets, const int64_t *__restrict__ ts,
                                                       uint32_t *__restrict__ rel, int32_t *__restrict__ wide, int B,
                                                       const int *__restrict__ status)
{
    if (*status) return; // offsets failed validation: touch nothing
    const int b = blockIdx.x;
    const int o = offsets[b], e = offsets[b + 1];
    int64_t mn = INT64_MAX, mx = INT64_MIN;
    for (int r = o + threadIdx.x; r < e; r += 256) {
        int64_t t = ts[r];
        mn = t < mn ? t : mn;
        mx = t > mx ? t : mx;
    }
    __shared__ int64_t smn[256], smx[256];
    smn[threadIdx.x] = mn;
    smx[threadIdx.x] = mx;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if (threadIdx.x < s) {
            smn[threadIdx.x] = smn[threadIdx.x + s] < smn[threadIdx.x] ? smn[threadIdx.x + s] : smn[threadIdx.x];
            smx[threadIdx.x] = smx[threadIdx.x + s] > smx[threadIdx.x] ? smx[threadIdx.x + s] : smx[threadIdx.x];
        }
        __syncthreads();
    }
    mn = smn[0];
    mx = smx[0];
    // span as unsigned: mx - mn may exceed INT64_MAX only for absurd inputs.
    const bool w = e > o && (uint64_t)mx - (uint64_t)mn > 0xFFFFFFFEull;
    if (threadIdx.x == 0) wide[b] = w ? 1 : 0;
    if (!w)
        for (int r = o + threadIdx.x; r < e; r += 256) rel[r] = (uint32_t)((uint64_t)ts[r] - (uint64_t)mn);
}

void launch_sched(const int32_t *offsets, const int64_t *ts, int B, int T, int tile, int H, int *status, int *n_items,
                  int2 *items, int max_items, uint32_t *rel, int32_t *wide, hipStream_t st)
{
    hipLaunchKernelGGL(sched_kernel, dim3(1), dim3(1024), 0, st, offsets, B, T, tile, H, status, n_items, items,
                       max_items);
    if (ts) hipLaunchKernelGGL(reltime_kernel, dim3(B), dim3(256), 0, st, offsets, ts, rel, wide, B, status);
}
