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
// ties by sequence index, the sequences that have a tile t form a prefix of
// pi, hence
//   index(b, t, h) = H * (S[t] + pos_pi(b)) + h,
//   S[t] = #items with a larger tile index / H = sum_{t' > t} #{b : n_b > t'}.
// pos_pi(b) = #{b' : n_b' > n_b} + rank(b), rank(b) = #{b' < b : n_b' = n_b}:
// the work list is a pure function of the offsets (the results of every
// kernel are independent of the order anyway).
//
// Split items (split_slots > 0): a tile t costs about 2(t + 1) key tiles of
// half its width, the whole launch about sum_b n_b (n_b + 1) H of them; tiles
// t >= t_split = max(4, avg / 3), avg = that total over the split_slots
// concurrent workgroups, become two items of half the cost each.  Both
// halves of a tile count as a multiplicity m(t) = 2 in the index arithmetic
// below: index(b, t, h, part) = H * (S[t] + m(t) pos_pi(b) + part) + h.
//
// A batch that fails validation gets status != 0 and no items, and nothing
// else is written (not even the buffers the caller asked to be zeroed).
__global__ void __launch_bounds__(1024) sched_kernel(const int32_t *__restrict__ offsets, int B, int T, int tile, int H,
                                                      int *__restrict__ status, int *__restrict__ n_items,
                                                      int2 *__restrict__ items, int max_items,
                                                      int32_t *__restrict__ wide, int32_t *__restrict__ rank,
                                                      int split_slots, int *__restrict__ t_split_out, SchedBwd bw)
{
    __shared__ int hist[SCHED_BINS];
    __shared__ long long ptmp[16];
    __shared__ int fill[SCHED_BINS];
    __shared__ int S[SCHED_BINS];
    __shared__ int bad;
    __shared__ unsigned long long work;
    __shared__ int chunk_tot[1024];
    __shared__ int rank_s[SCHED_BINS]; // ranks of the first SCHED_BINS sequences (the rest in rank[])
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
    if (bad) {
        if (tid == 0) {
            *status = bad;
            *n_items = 0;
            if (t_split_out) *t_split_out = SCHED_BINS;
        }
        return;
    }
    for (int b = tid; b < B; b += 1024) wide[b] = 0;
    // buffers the caller wants zeroed (the backward's bias gradients)
    for (int64_t i = tid; i < bw.n0; i += 1024) bw.zero0[i] = 0.f;
    for (int64_t i = tid; i < bw.n1; i += 1024) bw.zero1[i] = 0.f;
    if (bw.ds_base) {
        // Per sequence, exclusive prefix sums over the sequences before it:
        // dS plane offsets (H planes of P x P, P = L rounded up to DS_PAD),
        // drab_p partial slots (H * n * L floats) and drab_t partial slots
        // (H * n * TB_SLOTS floats, n = the sequence's key tiles).  Thread tid
        // owns sequences [tid * per, (tid + 1) * per).
        const int per = (B + 1023) / 1024, b0 = tid * per, b1 = min(B, b0 + per);
        long long own_ds = 0, own_p = 0, own_t = 0;
        for (int b = b0; b < b1; b++) {
            const long long L = offsets[b + 1] - offsets[b];
            const long long P = (L + DS_PAD - 1) / DS_PAD * DS_PAD, n = (L + tile - 1) / tile;
            own_ds += P * P * H;
            own_p += n * L * H;
            own_t += n * TB_SLOTS * H;
        }
        long long run_ds = block_prefix_excl64(own_ds, ptmp);
        long long run_p = block_prefix_excl64(own_p, ptmp);
        long long run_t = block_prefix_excl64(own_t, ptmp);
        for (int b = b0; b < b1; b++) {
            const long long L = offsets[b + 1] - offsets[b];
            const long long P = (L + DS_PAD - 1) / DS_PAD * DS_PAD, n = (L + tile - 1) / tile;
            bw.ds_base[b] = run_ds + P * P * H <= bw.ds_cap ? run_ds : -1;
            bw.pbase[b] = run_p + n * L * H <= bw.p_cap ? run_p : -1;
            bw.tbase[b] = run_t;
            run_ds += P * P * H;
            run_p += n * L * H;
            run_t += n * TB_SLOTS * H;
        }
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
    // rank(b) among the sequences of its length class, by index: wave 0
    // walks the sequences in order, 64 at a time; inside a group of 64 the
    // lanes of one class are ranked by a ballot, then the class counter
    // (hist[], reused) moves on.
    for (int i = tid; i < SCHED_BINS; i += 1024) hist[i] = 0;
    __syncthreads();
    const int lane = tid & 63, wv = tid >> 6;
    if (wv == 0) {
        const unsigned long long below = (1ull << lane) - 1ull;
        for (int b0 = 0; b0 < B; b0 += 64) {
            const int b = b0 + lane;
            int n = -1;
            if (b < B) {
                const int L = offsets[b + 1] - offsets[b];
                n = L > 0 ? (L + tile - 1) / tile : -1;
            }
            unsigned long long todo = __ballot(n >= 0);
            while (todo) {
                const int leader = __ffsll((long long)todo) - 1;
                const int v = __shfl(n, leader, 64);
                const unsigned long long same = __ballot(n == v) & todo;
                const int base = hist[v];
                if (n == v) {
                    const int rk = base + __popcll(same & below);
                    if (b < SCHED_BINS) rank_s[b] = rk;
                    else rank[b] = rk;
                }
                if (lane == leader) hist[v] = base + __popcll(same);
                todo &= ~same;
            }
        }
    }
    __syncthreads();
    // one wave per sequence: the lanes write its n * H items
    for (int b = wv; b < B; b += 16) {
        const int L = offsets[b + 1] - offsets[b];
        const int n = L > 0 ? (L + tile - 1) / tile : 0;
        if (n == 0) continue;
        const int pos = fill[n] + (b < SCHED_BINS ? rank_s[b] : rank[b]);
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
// 64-bit arithmetic for that sequence.  wide[] was zeroed by sched_kernel
// (which also validated the offsets: nothing runs on a batch that failed).
__device__ void reltime_rows(const int32_t *__restrict__ offsets, const int64_t *__restrict__ ts,
                             uint32_t *__restrict__ rel, int32_t *__restrict__ wide, int B, int T, int blk)
{
    const int r = blk * 256 + threadIdx.x;
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
        // every index clamped to the block's last token (repeats change
        // neither bound), so the 32 loads go out together
        const int last = min(r + 32, offsets[lo + 1]) - 1;
        uint32_t mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll
        for (int k = 0; k < 32; k++) {
            const uint32_t v = (uint32_t)(ts[min(r + k, last)] - t0 + ((int64_t)1 << 31));
            mn = min(mn, v);
            mx = max(mx, v);
        }
        rel[T + r] = mn;
        rel[2 * (int64_t)T + r] = mx;
    }
}

__global__ void __launch_bounds__(256) reltime_kernel(const int32_t *__restrict__ offsets, const int64_t *__restrict__ ts,
                                                       uint32_t *__restrict__ rel, int32_t *__restrict__ wide, int B,
                                                       int T, const int *__restrict__ status)
{
    if (*status) return; // offsets failed validation: touch nothing
    reltime_rows(offsets, ts, rel, wide, B, T, blockIdx.x);
}

// Rows of split items: workgroup y of sequence b (of ny) takes every ny-th
// row of the sequence from tile * t_split on; 16-byte stores when the rows
// allow them.
__device__ void zero_split_rows(const int32_t *__restrict__ offsets, const ZeroRows &z, int b, int y, int ny)
{
    const int o_b = offsets[b], L = offsets[b + 1] - o_b;
    const int64_t r0 = (int64_t)z.tile * *z.t_split;
    if (r0 >= L) return;
    float *o32 = z.rows;
    const int64_t ld = z.ld;
    const int F = z.F;
    const bool vec = ((((uintptr_t)o32) | (uintptr_t)(ld * 4) | (uintptr_t)(F * 4)) & 15) == 0;
    if (vec) {
        const int f4 = F / 4;
        for (int64_t r = r0 + y; r < L; r += ny)
            for (int c = threadIdx.x; c < f4; c += 256)
                *(floatx4 *)(o32 + (o_b + r) * ld + 4 * c) = floatx4{0.f, 0.f, 0.f, 0.f};
    } else {
        for (int64_t r = r0 + y; r < L; r += ny)
            for (int c = threadIdx.x; c < F; c += 256) o32[(o_b + r) * ld + c] = 0.f;
    }
}

// dq_acc rows ([T][F] fp32) of the sequences whose dS planes did not fit
// (ds_base < 0): workgroup y of sequence b (of ny) takes every ny-th row.
__device__ void zero_dqa_rows(const int32_t *__restrict__ offsets, const ZeroRows &z, int b, int y, int ny)
{
    if (z.ds_base[b] >= 0) return;
    const int o_b = offsets[b], L = offsets[b + 1] - o_b;
    for (int64_t r = y; r < L; r += ny)
        for (int c = threadIdx.x; c < z.F; c += 256) z.rows[(o_b + r) * (int64_t)z.F + c] = 0.f;
}

// What runs after the launcher, in one launch: workgroups [0, nrel) write
// the relative times, the next B * ZERO_NY zero rows (z.mode).
constexpr int ZERO_NY = 64;
__global__ void __launch_bounds__(256) post_sched_kernel(const int32_t *__restrict__ offsets,
                                                          const int64_t *__restrict__ ts, uint32_t *__restrict__ rel,
                                                          int32_t *__restrict__ wide, int B, int T, int nrel, ZeroRows z,
                                                          const int *__restrict__ status)
{
    if (*status) return; // offsets failed validation: touch nothing
    const int blk = blockIdx.x;
    if (blk < nrel) {
        reltime_rows(offsets, ts, rel, wide, B, T, blk);
        return;
    }
    const int zb = blk - nrel, b = zb / ZERO_NY, y = zb - b * ZERO_NY;
    if (z.mode == ZeroRows::SPLIT_ROWS) zero_split_rows(offsets, z, b, y, ZERO_NY);
    else zero_dqa_rows(offsets, z, b, y, ZERO_NY);
}

void launch_sched(const int32_t *offsets, const int64_t *ts, int B, int T, int tile, int H, int *status, int *n_items,
                  int2 *items, int max_items, uint32_t *rel, int32_t *wide, int32_t *rank, int split_slots, int *t_split,
                  const SchedBwd &bw, hipStream_t st, const ZeroRows &z)
{
    SchedBwd b2 = bw;
    if (!b2.zero0) b2.n0 = 0;
    if (!b2.zero1) b2.n1 = 0;
    hipLaunchKernelGGL(sched_kernel, dim3(1), dim3(1024), 0, st, offsets, B, T, tile, H, status, n_items, items,
                       max_items, wide, rank, split_slots, t_split, b2);
    const int nrel = ts && T > 0 ? (T + 255) / 256 : 0;
    const int nz = z.mode != ZeroRows::NONE && B > 0 ? B * ZERO_NY : 0;
    if (nrel + nz > 0)
        hipLaunchKernelGGL(post_sched_kernel, dim3(nrel + nz), dim3(256), 0, st, offsets, ts, rel, wide, B, T, nrel, z,
                           status);
}

// ---------------------------------------------------------------------------
// Appending new actions to cached histories (the streaming side of M-FALCON's
// cacheable history work): one workgroup of 1024 threads validates the two
// offset arrays, writes the merged offsets and the work list.  User u's
// sequence is [history (n_u); new (a_u)]; its query tiles holding new
// positions are t in [n_u / tile, ceil((n_u + a_u) / tile)).  Items are
// written user by user (block-wide scan of the per-user counts, 1024 users
// at a time), the highest tile first.
__global__ void __launch_bounds__(1024) append_plan_kernel(AppendPlan p)
{
    __shared__ int bad;
    __shared__ long long ptmp[16];
    __shared__ int base_s;
    const int tid = threadIdx.x, U = p.U;
    if (tid == 0) {
        bad = (p.hoff[0] != 0 || p.aoff[0] != 0 || p.hoff[U] != p.Th || p.aoff[U] != p.Tn) ? HSTU_DEV_BAD_OFFSETS : 0;
        base_s = 0;
    }
    __syncthreads();
    for (int u = tid; u < U; u += 1024)
        if (p.hoff[u + 1] < p.hoff[u] || p.aoff[u + 1] < p.aoff[u]) atomicOr(&bad, HSTU_DEV_BAD_OFFSETS);
    __syncthreads();
    if (bad) {
        if (tid == 0) {
            *p.status = bad;
            *p.n_items = 0;
        }
        return;
    }
    for (int u = tid; u <= U; u += 1024) p.moff[u] = p.hoff[u] + p.aoff[u];
    for (int u = tid; u < U; u += 1024) p.wide[u] = 0;
    for (int c0 = 0; c0 < U; c0 += 1024) {
        const int u = c0 + tid;
        int t0 = 0, t1 = 0;
        if (u < U) {
            const int n = p.hoff[u + 1] - p.hoff[u], a = p.aoff[u + 1] - p.aoff[u];
            if (a > 0) {
                t0 = n / p.tile;
                t1 = (n + a + p.tile - 1) / p.tile;
            }
        }
        const int mine = (t1 - t0) * p.H;
        const int ex = (int)block_prefix_excl64(mine, ptmp); // items of the chunk's earlier users
        const int first = base_s + ex;
        for (int k = 0; k < mine; k++) {
            const int t = t1 - 1 - k / p.H, h = k % p.H;
            if (first + k < p.max_items) p.items[first + k] = make_int2(u, (t << ITEM_T_SHIFT) | h);
        }
        __syncthreads(); // every thread has read base_s
        if (tid == 1023) base_s += ex + mine;
        __syncthreads();
    }
    if (tid == 0) {
        *p.n_items = base_s;
        *p.status = 0;
    }
}

// Each wave copies MERGE_ROWS consecutive merged rows r (user u, position
// i): K and V rows (hd bf16 elements, 16 bytes per lane and step) from the
// cache or from the new tokens, and the rows' times.  The user of the first
// row comes from a binary search over the merged offsets, the following rows
// walk forward from it; every row's loads are issued before its stores.
constexpr int MERGE_ROWS = 4;
__global__ void __launch_bounds__(256) append_merge_kernel(AppendPlan p)
{
    if (*p.status) return;
    const int64_t r0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * MERGE_ROWS;
    const int lane = threadIdx.x & 63;
    const int Tm = p.Th + p.Tn;
    if (r0 >= Tm) return;
    int lo = 0, hi = p.U - 1; // last u with moff[u] <= r0
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (p.moff[mid] <= r0) lo = mid;
        else hi = mid - 1;
    }
    const bf16 *ks[MERGE_ROWS], *vs[MERGE_ROWS];
    int nrow = 0;
#pragma unroll
    for (int j = 0; j < MERGE_ROWS; j++) {
        const int64_t r = r0 + j;
        ks[j] = vs[j] = nullptr;
        if (r < Tm) {
            while (lo < p.U - 1 && p.moff[lo + 1] <= r) lo++; // next user, skipping users with nothing
            const int64_t i = r - p.moff[lo];
            const int n = p.hoff[lo + 1] - p.hoff[lo];
            int64_t tsrc;
            if (i < n) {
                ks[j] = p.kc + (p.hoff[lo] + i) * p.ldkc;
                vs[j] = p.vc + (p.hoff[lo] + i) * p.ldvc;
                tsrc = p.hoff[lo] + i;
            } else {
                const int64_t rn = p.aoff[lo] + (i - n);
                ks[j] = p.knew + rn * p.ldnew;
                vs[j] = p.vnew + rn * p.ldnew;
                tsrc = -1 - rn;
            }
            if (p.ts_m && lane == j) p.ts_m[r] = tsrc >= 0 ? p.ts_h[tsrc] : p.ts_a[-1 - tsrc];
            nrow = j + 1;
        }
    }
    for (int c = 8 * lane; c < p.hd; c += 512) {
        u32x4 kx[MERGE_ROWS], vx[MERGE_ROWS];
#pragma unroll
        for (int j = 0; j < MERGE_ROWS; j++)
            if (j < nrow) {
                kx[j] = *(const u32x4 *)(ks[j] + c);
                vx[j] = *(const u32x4 *)(vs[j] + c);
            }
#pragma unroll
        for (int j = 0; j < MERGE_ROWS; j++)
            if (j < nrow) {
                *(u32x4 *)(p.kout + (r0 + j) * p.ldko + c) = kx[j];
                *(u32x4 *)(p.vout + (r0 + j) * p.ldvo + c) = vx[j];
            }
    }
}

hipError_t launch_append_plan(const AppendPlan &p, hipStream_t st)
{
    hipLaunchKernelGGL(append_plan_kernel, dim3(1), dim3(1024), 0, st, p);
    const int Tm = p.Th + p.Tn;
    if (Tm > 0) {
        hipLaunchKernelGGL(append_merge_kernel, dim3((Tm + 4 * MERGE_ROWS - 1) / (4 * MERGE_ROWS)), dim3(256), 0, st, p);
        if (p.ts_m)
            hipLaunchKernelGGL(reltime_kernel, dim3((Tm + 255) / 256), dim3(256), 0, st, p.moff, p.ts_m, p.rel, p.wide,
                               p.U, Tm, p.status);
    }
    return hipGetLastError();
}
