// sched.hip -- the launcher: validates the jagged offsets, orders the work
// longest-first and converts timestamps to sequence-relative 32-bit values.
//
// The pages attribute HSTU's speed to computing only real tokens (review of
// "Actions Speak Louder than Words", section 4 innovations table: a sparse,
// efficient kernel; section 3 Stochastic Length).  Here that means: no
// padding anywhere, items only for tiles that hold real tokens, and the most
// expensive items first so the tail of the launch is short.
#include "kernels.h"

// Exclusive suffix sum over the 1024 threads of the block: returns
// sum_{j > tid} v_j.  `tmp` is a 1024-entry LDS array.
__device__ int block_suffix_excl(int v, int *tmp)
{
    // exclusive suffix sum over the 1024 threads: sum of v over threads > tid.
    // Wave-level inclusive suffix scan with shuffles, then wave totals.
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    int incl = v;
    for (int o = 1; o < 64; o <<= 1) {
        const int x = __shfl_down(incl, o, 64);
        if (lane + o < 64) incl += x;
    }
    __syncthreads(); // tmp may still be read by a previous call
    if (lane == 0) tmp[wv] = incl; // wave total
    __syncthreads();
    int later = 0;
    for (int k = wv + 1; k < 16; k++) later += tmp[k];
    return incl - v + later;
}

// Exclusive prefix sum over the 1024 threads of the block (64-bit); `tmp` is
// a 16-entry LDS array.
__device__ long long block_prefix_excl64(long long v, long long *tmp)
{
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    long long incl = v;
    for (int o = 1; o < 64; o <<= 1) {
        const long long x = __shfl_up(incl, o, 64);
        if (lane >= o) incl += x;
    }
    __syncthreads();
    if (lane == 63) tmp[wv] = incl;
    __syncthreads();
    long long before = 0;
    for (int k = 0; k < wv; k++) before += tmp[k];
    return before + incl - v;
}

// One workgroup of 1024 threads.  An item is (sequence b, tile t, head h);
// a tile t of sequence b costs t + 1 units (causal), so items are ordered by
// t descending.  With pi = the sequences sorted by tile count descending,
// the sequences that have a tile t form a prefix of pi, hence
//   index(b, t, h) = H * (S[t] + pos_pi(b)) + h,
//   S[t] = #items with a larger tile index / H = sum_{t' > t} #{b : n_b > t'}.
// Ties inside a length class are broken by an atomic counter; the results
// of every kernel are independent of the order.
//
// Split items (split_slots > 0): a tile t costs about 2(t + 1) key tiles of
// half its width, the whole launch about sum_b n_b (n_b + 1) H of them; tiles
// t >= t_split = max(4, avg / 3), avg = that total over the split_slots
// concurrent workgroups, become two items of half the cost each.  Both
// halves of a tile count as a multiplicity m(t) = 2 in the index arithmetic
// below: index(b, t, h, part) = H * (S[t] + m(t) pos_pi(b) + part) + h.
__global__ void __launch_bounds__(1024) sched_kernel(const int32_t *__restrict__ offsets, int B, int T, int tile, int H,
                                                      int *__restrict__ status, int *__restrict__ n_items,
                                                      int2 *__restrict__ items, int max_items,
                                                      int32_t *__restrict__ wide, int split_slots,
                                                      int *__restrict__ t_split_out, int64_t *__restrict__ ds_base,
                                                      int64_t ds_cap, float *__restrict__ zero0, int64_t n0,
                                                      float *__restrict__ zero1, int64_t n1)
{
    __shared__ int hist[SCHED_BINS];
    __shared__ long long ptmp[16];
    // buffers the caller wants zeroed (the backward's bias gradients)
    for (int64_t i = threadIdx.x; i < n0; i += 1024) zero0[i] = 0.f;
    for (int64_t i = threadIdx.x; i < n1; i += 1024) zero1[i] = 0.f;
    __shared__ int fill[SCHED_BINS];
    __shared__ int S[SCHED_BINS];
    __shared__ int bad;
    __shared__ unsigned long long work;
    __shared__ int chunk_tot[1024];
    const int tid = threadIdx.x;
    for (int i = tid; i < SCHED_BINS; i += 1024) {
        hist[i] = 0;
        fill[i] = 0;
    }
    if (tid == 0) {
        bad = (offsets[0] != 0 || offsets[B] != T) ? HSTU_DEV_BAD_OFFSETS : 0;
        work = 0;
    }
    __syncthreads();
    for (int b = tid; b < B; b += 1024) {
        wide[b] = 0;
        int L = offsets[b + 1] - offsets[b];
        if (L < 0) atomicOr(&bad, HSTU_DEV_BAD_OFFSETS);
        int n = L > 0 ? (L + tile - 1) / tile : 0;
        if (n >= SCHED_BINS) atomicOr(&bad, HSTU_DEV_TOO_LONG);
        else {
            atomicAdd(&hist[n], 1);
            atomicAdd(&work, (unsigned long long)n * (unsigned long long)(n + 1));
        }
    }
    __syncthreads();
    if (ds_base && !bad) {
        // dS block offsets: thread tid owns sequences [tid * per, (tid + 1) * per)
        const int per = (B + 1023) / 1024, b0 = tid * per, b1 = min(B, b0 + per);
        long long own = 0;
        for (int b = b0; b < b1; b++) {
            const long long P = ((long long)(offsets[b + 1] - offsets[b]) + DS_PAD - 1) / DS_PAD * DS_PAD;
            own += P * P * H;
        }
        long long run = block_prefix_excl64(own, ptmp);
        for (int b = b0; b < b1; b++) {
            const long long P = ((long long)(offsets[b + 1] - offsets[b]) + DS_PAD - 1) / DS_PAD * DS_PAD;
            ds_base[b] = run + P * P * H <= ds_cap ? run : -1;
            run += P * P * H;
        }
    }
    if (bad) {
        if (tid == 0) {
            *status = bad;
            *n_items = 0;
            if (t_split_out) *t_split_out = SCHED_BINS;
        }
        return;
    }
    int t_split = SCHED_BINS; // no split
    if (split_slots > 0) {
        const unsigned long long avg = work * (unsigned long long)H / (unsigned long long)split_slots;
        const unsigned long long t3 = avg / 3;
        t_split = t3 < 4 ? 4 : (t3 > SCHED_BINS ? SCHED_BINS : (int)t3);
    }
    if (tid == 0 && t_split_out) *t_split_out = t_split;
    auto mult = [&](int t) { return t >= t_split ? 2 : 1; };
    // cnt_gt[t] = #{b : n_b > t} = sum_{v > t} hist[v]  (suffix sum, into
    // fill[]), then S[t] = sum_{t' > t} cnt_gt[t'].  Each thread owns a
    // contiguous chunk of bins; chunk totals go through a block-wide scan.
    const int per = SCHED_BINS / 1024;
    {
        int s = 0;
        for (int i = per - 1; i >= 0; i--) s += hist[tid * per + i];
        const int above = block_suffix_excl(s, chunk_tot); // sum of the chunks above tid
        int run = above;
        for (int i = per - 1; i >= 0; i--) {
            const int t = tid * per + i;
            fill[t] = run; // = #{b : n_b > t}
            run += hist[t];
        }
    }
    __syncthreads();
    {
        int s = 0;
        for (int i = per - 1; i >= 0; i--) s += fill[tid * per + i] * mult(tid * per + i);
        const int above = block_suffix_excl(s, chunk_tot);
        if (tid == 0) {
            *n_items = (above + s) * H; // sum_t m(t) cnt_gt[t]
            *status = 0;
        }
        int run = above;
        for (int i = per - 1; i >= 0; i--) {
            const int t = tid * per + i;
            S[t] = run;
            run += fill[t] * mult(t);
        }
    }
    __syncthreads();
    // pos_pi(b) = #{b' : n_b' > n_b} + rank among equal n; hist[] becomes the
    // per-class fill counter.
    for (int i = tid; i < SCHED_BINS; i += 1024) hist[i] = 0;
    __syncthreads();
    // one wave per sequence: lane 0 takes the sequence's rank in its length
    // class, the lanes write its n * H items
    const int lane = tid & 63, wv = tid >> 6;
    for (int b = wv; b < B; b += 16) {
        const int L = offsets[b + 1] - offsets[b];
        const int n = L > 0 ? (L + tile - 1) / tile : 0;
        if (n == 0) continue;
        int pos = 0;
        if (lane == 0) pos = fill[n] + atomicAdd(&hist[n], 1);
        pos = __shfl(pos, 0, 64);
        for (int k = lane; k < n * H; k += 64) {
            const int t = k / H, h = k - t * H;
            const int m = mult(t);
            for (int part = 0; part < m; part++) {
                const int idx = H * (S[t] + m * pos + part) + h;
                if (idx < max_items) items[idx] = make_int2(b, (t << ITEM_T_SHIFT) | ((m - 1) << 9) | (part << 8) | h);
            }
        }
    }
}

// One thread per token: rel[r] = ts[r] - ts[first token of its sequence] +
// 2^31 as a 32-bit value.  Differences of two such values are exact as long
// as every time of the sequence lies within 2^31 - 1 of its first time (then
// |t_i - t_j| + 1 < 2^32); otherwise wide[b] is set and the kernels use exact
// 64-bit arithmetic for that sequence.  wide[] was zeroed by sched_kernel.
__global__ void __launch_bounds__(256) reltime_kernel(const int32_t *__restrict__ offsets, const int64_t *__restrict__ ts,
                                                       uint32_t *__restrict__ rel, int32_t *__restrict__ wide, int B,
                                                       int T, const int *__restrict__ status)
{
    if (*status) return; // offsets failed validation: touch nothing
    const int r = blockIdx.x * 256 + threadIdx.x;
    if (r >= T) return;
    int lo = 0, hi = B - 1; // last b with offsets[b] <= r
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (offsets[mid] <= r) lo = mid;
        else hi = mid - 1;
    }
    while (lo < B - 1 && offsets[lo + 1] <= r) lo++; // skip empty sequences
    const int64_t t0 = ts[offsets[lo]];
    const int64_t d = ts[r] - t0;
    if (d < -(int64_t)0x7FFFFFFF || d > (int64_t)0x7FFFFFFF) atomicOr(&wide[lo], 1);
    rel[r] = (uint32_t)(d + ((int64_t)1 << 31));
    if (((r - offsets[lo]) & 31) == 0) { // first token of a 32-token block: its range of rel
        const int end = min(r + 32, offsets[lo + 1]);
        uint32_t mn = 0xFFFFFFFFu, mx = 0u;
        for (int i = r; i < end; i++) {
            const uint32_t v = (uint32_t)(ts[i] - t0 + ((int64_t)1 << 31));
            mn = min(mn, v);
            mx = max(mx, v);
        }
        rel[T + r] = mn;
        rel[2 * (int64_t)T + r] = mx;
    }
}

// Rows of split items: grid (B, 128), workgroup y takes every 128th row of
// sequence b from tile * t_split on; 16-byte stores when the rows allow them.
__global__ void __launch_bounds__(256) zero_split_rows_kernel(const int32_t *__restrict__ offsets, int tile,
                                                               const int *__restrict__ t_split, float *__restrict__ o32,
                                                               int64_t ld, int F, const int *__restrict__ status)
{
    if (*status) return;
    const int b = blockIdx.x;
    const int o_b = offsets[b], L = offsets[b + 1] - o_b;
    const int64_t r0 = (int64_t)tile * *t_split;
    if (r0 >= L) return;
    const bool vec = ((((uintptr_t)o32) | (uintptr_t)(ld * 4) | (uintptr_t)(F * 4)) & 15) == 0;
    if (vec) {
        const int f4 = F / 4;
        for (int64_t r = r0 + blockIdx.y; r < L; r += gridDim.y)
            for (int c = threadIdx.x; c < f4; c += 256)
                *(floatx4 *)(o32 + (o_b + r) * ld + 4 * c) = floatx4{0.f, 0.f, 0.f, 0.f};
    } else {
        for (int64_t r = r0 + blockIdx.y; r < L; r += gridDim.y)
            for (int c = threadIdx.x; c < F; c += 256) o32[(o_b + r) * ld + c] = 0.f;
    }
}

hipError_t launch_zero_split_rows(const int32_t *offsets, int B, int tile, const int *t_split, float *o32, int64_t ld,
                                  int F, const int *status, hipStream_t st)
{
    if (B <= 0) return hipSuccess;
    hipLaunchKernelGGL(zero_split_rows_kernel, dim3(B, 128), dim3(256), 0, st, offsets, tile, t_split, o32, ld, F,
                       status);
    return hipGetLastError();
}

// dq_acc rows of the sequences whose dS planes did not fit: grid (B, 32).
__global__ void __launch_bounds__(256) zero_dqa_rows_kernel(const int32_t *__restrict__ offsets,
                                                             const int64_t *__restrict__ ds_base,
                                                             float *__restrict__ dq_acc, int F,
                                                             const int *__restrict__ status)
{
    if (*status) return;
    const int b = blockIdx.x;
    if (ds_base[b] >= 0) return;
    const int o_b = offsets[b], L = offsets[b + 1] - o_b;
    for (int64_t r = blockIdx.y; r < L; r += gridDim.y)
        for (int c = threadIdx.x; c < F; c += 256) dq_acc[(o_b + r) * (int64_t)F + c] = 0.f;
}

hipError_t launch_zero_dqa_rows(const int32_t *offsets, int B, const int64_t *ds_base, float *dq_acc, int F,
                                const int *status, hipStream_t st)
{
    if (B <= 0) return hipSuccess;
    hipLaunchKernelGGL(zero_dqa_rows_kernel, dim3(B, 32), dim3(256), 0, st, offsets, ds_base, dq_acc, F, status);
    return hipGetLastError();
}

void launch_sched(const int32_t *offsets, const int64_t *ts, int B, int T, int tile, int H, int *status, int *n_items,
                  int2 *items, int max_items, uint32_t *rel, int32_t *wide, int split_slots, int *t_split,
                  int64_t *ds_base, int64_t ds_cap, float *zero0, int64_t n0, float *zero1, int64_t n1,
                  hipStream_t st)
{
    hipLaunchKernelGGL(sched_kernel, dim3(1), dim3(1024), 0, st, offsets, B, T, tile, H, status, n_items, items,
                       max_items, wide, split_slots, t_split, ds_base, ds_cap, zero0, zero0 ? n0 : 0, zero1,
                       zero1 ? n1 : 0);
    if (ts && T > 0)
        hipLaunchKernelGGL(reltime_kernel, dim3((T + 255) / 256), dim3(256), 0, st, offsets, ts, rel, wide, B, T, status);
}
