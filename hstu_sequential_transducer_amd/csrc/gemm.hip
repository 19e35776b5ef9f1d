// gemm.hip -- the HSTU layer's two linear maps with fused epilogues (review of
// "Actions Speak Louder than Words", section 3: Eq. 1's f1 followed by phi1,
// Eq. 3's f2, and the residual connection between layers; section 5 notes
// the layer has only these 2 linear layers).
//
//   C[m][n] = act(sum_k A[m][k] W[n][k] + bias[n]) + R[m][n]
//
// W is stored [out][in] (y = x W^T + b).  Optional extra outputs: a
// storage-dtype copy of C (the M-FALCON hidden state feeding the next layer),
// copies of two column ranges (this layer's K and V, the M-FALCON cache) and
// a storage-dtype copy of the pre-activation (for phi1' in the backward).
//
// bf16, main kernel: 256x128 output tile per workgroup of 4 waves, each wave
// 64 rows x 128 columns (2x4 blocks of 32x32x16 bf16 MFMA computing C^T, so
// a lane owns a row and 4 consecutive columns per register group); two
// workgroups per CU.  Products with fewer than two rounds of such tiles
// (M-FALCON's candidates, narrow outputs) take 128x128 tiles, each wave
// 32 rows, which doubles their workgroups; products that would still leave
// most CUs idle take 64x128 tiles of 2 waves.  K advances in steps of 32 through three LDS stages
// filled by direct global -> LDS copies two steps ahead, with a plain
// barrier per step (no wait for the copies still in flight); 64-byte stage
// rows have their 16-byte chunks XOR-swizzled by (row / 4) % 4, which keeps
// the operand reads (16 rows at one chunk) free of bank conflicts.  The
// epilogue (bias from LDS, activation, residual, stores and the K/V copies)
// runs from registers with 8- or 16-byte accesses.  Workgroup i takes tile
// (i % 8) * ceil(tiles / 8) + i / 8: consecutive workgroups go to different
// XCDs, so this keeps the column tiles of one row block (which share A rows)
// on one XCD and its L2.  Both operands are K-contiguous, so no transposes.
// (Measured alternatives: a 256x256 tile with one wave per SIMD, and 64-deep
// K steps with the tile staged through LDS for the epilogue, were slower.)
// bf16, general kernel (shapes or alignments the main kernel does not take):
// 128x128 tiles of 4 waves, K in steps of 32, register-staged loads.
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

// main kernel geometry
// (NW waves: 4 -> 256 x 128 tiles, 8 -> 256 x 256)
constexpr int TBK = 32, TSTAGES = 3;
template <int TBM, int TBN>
struct alignas(16) TStage {
    alignas(16) bf16 a[TBM * TBK]; // [row][k], 64-byte rows, swizzled
    alignas(16) bf16 w[TBN * TBK];
};
// 64-byte rows: 16-byte chunk c of row r sits at chunk c ^ ((r / 4) % 4), so
// 16 consecutive rows read at one chunk cover all 16 16-byte bank groups
DEV int tsw(int row) { return (row >> 2) & 3; }
DEV int tswz(int row, int col) { return row * TBK + (((col >> 3) ^ tsw(row)) << 3) + (col & 7); }
typedef __attribute__((address_space(3))) void lds_void;

// 4 consecutive outputs: one 16-byte fp32 store or one 8-byte bf16 store
DEV void store4(void *p, int64_t i, const floatx4 &x, bool f32)
{
    if (f32) *(floatx4 *)((float *)p + i) = x;
    else *(u32x2 *)((bf16 *)p + i) = u32x2{pack2_bf16(x[0], x[1]), pack2_bf16(x[2], x[3])};
}

} // namespace

// EPI: activation; RES: residual none (0), bf16 (1), fp32 (2).  Waves form a
// WGM x WGN grid; each wave owns 32 TI rows x 128 columns (TI x 4 MFMA
// blocks); the tile has TBM = 32 TI WGM rows.  TI = 2 runs two waves per SIMD
// (two workgroups per CU), TI = 4 one (its 256 accumulators use the whole
// register file).
template <int EPI, int RES, int TI, int WGM, int WGN>
__global__ void __launch_bounds__(64 * WGM * WGN) __attribute__((amdgpu_waves_per_eu(TI == 4 ? 1 : 2, TI == 4 ? 1 : 2)))
gemm_bf16_tiled_kernel(GemmArgs g, int tiles_n, int n_tiles, int per_xcd)
{
    constexpr int NW = WGM * WGN, TBN = 128 * WGN, TNT = 64 * NW;
    constexpr int TBM = 32 * TI * WGM;
    constexpr int CA = TBM / 16 / NW, CW = TBN / 16 / NW; // direct copies per wave per stage (16 rows each)
    __shared__ TStage<TBM, TBN> st[TSTAGES];
    __shared__ __align__(16) float bias_s[TBN];
    const int t = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    if (t >= n_tiles) return;
    const int mt = t / tiles_n, nt = t - mt * tiles_n;
    const int m0 = mt * TBM, n0 = nt * TBN;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, gq = l >> 5, lq = l & 31;
    const int wm = w % WGM, wn = w / WGM; // rows 32 TI wm, columns 128 wn of the tile
    const bf16 *A = (const bf16 *)g.A, *W = (const bf16 *)g.W;
    const int nk = g.K / TBK;
    // the tile's bias (N is a multiple of 8, so a 4-column group is all in or
    // all out); visible after the first barrier of the K loop
    if (tid < TBN / 4) {
        const int n = n0 + 4 * tid;
        *(floatx4 *)&bias_s[4 * tid] = (g.bias && n < g.N) ? *(const floatx4 *)(g.bias + n) : floatx4{0.f, 0.f, 0.f, 0.f};
    }

    // copies of step kt into stage S: 16 rows per wave instruction, A rows
    // [16 CA w, 16 CA (w + 1)) and W rows [32w, 32w + 32); rows past M or N
    // re-read the last row
    auto gload = [&](int kt, TStage<TBM, TBN> &S) {
        const int k0 = kt * TBK;
#pragma unroll
        for (int i = 0; i < CA; i++) {
            const int r0 = 16 * CA * w + 16 * i, row = r0 + (l >> 2);
            const int c = (l & 3) ^ tsw(row);
            const int m = min(m0 + row, g.M - 1);
            __builtin_amdgcn_global_load_lds((const void *)(A + (int64_t)m * g.lda + k0 + c * 8),
                                             (lds_void *)(S.a + r0 * TBK), 16, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < CW; i++) {
            const int r0 = 16 * CW * w + 16 * i, row = r0 + (l >> 2);
            const int c = (l & 3) ^ tsw(row);
            const int n = min(n0 + row, g.N - 1);
            __builtin_amdgcn_global_load_lds((const void *)(W + (int64_t)n * g.K + k0 + c * 8),
                                             (lds_void *)(S.w + r0 * TBK), 16, 0, 0);
        }
    };
    static_assert(CA + CW <= 15, "wait count field");

    // C^T blocks: acc[i][j] holds rows m = 32 TI wm + 32i + lane%32 (one per
    // lane) and columns n = 128 wn + 32j + 8(r/4) + 4(lane/32) + r%4
    // (registers)
    floatx16 acc[TI][4];
#pragma unroll
    for (int i = 0; i < TI; i++)
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0.f;

    // one K step: 2 sub-steps of 16; operands of sub-step 1 are read while
    // the MFMAs of sub-step 0 run
    auto compute = [&](const TStage<TBM, TBN> &S) {
        bf16x8 a[2][TI], b[2][4];
        auto fetch = [&](int ks) {
            const int col = 16 * ks + 8 * gq;
#pragma unroll
            for (int i = 0; i < TI; i++) a[ks][i] = *(const bf16x8 *)&S.a[tswz(32 * TI * wm + 32 * i + lq, col)];
#pragma unroll
            for (int j = 0; j < 4; j++) b[ks][j] = *(const bf16x8 *)&S.w[tswz(128 * wn + 32 * j + lq, col)];
        };
        fetch(0);
        fetch(1);
#pragma unroll
        for (int ks = 0; ks < 2; ks++)
#pragma unroll
            for (int j = 0; j < 4; j++)
#pragma unroll
                for (int i = 0; i < TI; i++) acc[i][j] = mfma32(b[ks][j], a[ks][i], acc[i][j]);
    };

    gload(0, st[0]);
    if (nk > 1) gload(1, st[1]);
    for (int kt = 0; kt < nk; kt++) {
        // this wave's copies of this step are done (the next step's may still
        // fly), then a plain barrier: every wave's copies of this step are in
        // LDS, and every wave has finished reading the stage that the copies
        // below overwrite (its reads fed the MFMAs of the last step).
        // (__syncthreads() would also wait for the next step's copies.)
        if (kt + 1 < nk) __builtin_amdgcn_s_waitcnt(0x0F70 | (CA + CW)); // vmcnt(CA + CW)
        else __builtin_amdgcn_s_waitcnt(0x0F70);                      // vmcnt(0)
        asm volatile("s_barrier" ::: "memory");
        if (kt + 2 < nk) gload(kt + 2, st[(kt + 2) % TSTAGES]);
        compute(st[kt % TSTAGES]);
    }

    // epilogue from registers: each lane owns 4 consecutive columns per
    // (j, r/4) of its TI rows.  A bf16 residual (32 TI bytes per lane) is
    // loaded in full before the first store: vector memory operations
    // complete in issue order, so a load issued after a store would also wait
    // for the store.  An fp32 residual is loaded per column block.  The bias
    // comes from LDS.
    u32x2 rh[RES == 1 ? TI : 1][4][4]; // bf16 residual by i, j, q
    if constexpr (RES == 1) {
#pragma unroll
        for (int i = 0; i < TI; i++) {
            const int m = min(m0 + 32 * TI * wm + 32 * i + lq, g.M - 1);
#pragma unroll
            for (int j = 0; j < 4; j++)
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    const int n = min(n0 + 128 * wn + 32 * j + 8 * q + 4 * gq, g.N - 4);
                    rh[i][j][q] = *(const u32x2 *)((const bf16 *)g.R16 + (int64_t)m * g.ldr + n);
                }
        }
    }
#pragma unroll
    for (int j = 0; j < 4; j++) {
#pragma unroll
        for (int i = 0; i < TI; i++) {
            const int m = m0 + 32 * TI * wm + 32 * i + lq;
            floatx4 rf[4];
            if constexpr (RES == 2) {
                const int mc = min(m, g.M - 1);
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    const int n = min(n0 + 128 * wn + 32 * j + 8 * q + 4 * gq, g.N - 4);
                    rf[q] = *(const floatx4 *)(g.R32 + (int64_t)mc * g.ldr + n);
                }
            }
            if (m >= g.M) continue;
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const int n = n0 + 128 * wn + 32 * j + 8 * q + 4 * gq;
                if (n >= g.N) continue;
                const floatx4 b4 = *(const floatx4 *)&bias_s[128 * wn + 32 * j + 8 * q + 4 * gq];
                floatx4 x, pre;
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    pre[e] = acc[i][j][4 * q + e] + b4[e];
                    x[e] = apply_act(pre[e], EPI);
                }
                if (g.Cpre) store4(g.Cpre, (int64_t)m * g.ldcpre + n, pre, false);
                if constexpr (RES == 2) x += rf[q];
                if constexpr (RES == 1) {
                    const u32x2 rv = rh[i][j][q];
                    x += floatx4{bf16_lo(rv[0]), bf16_hi(rv[0]), bf16_lo(rv[1]), bf16_hi(rv[1])};
                }
                store4(g.C, (int64_t)m * g.ldc + n, x, g.c_f32);
                if (g.C16) store4(g.C16, (int64_t)m * g.ldc16 + n, x, false);
                if (g.Ck && n >= g.k_lo && n < g.k_lo + g.kv_w) store4(g.Ck, (int64_t)m * g.ldck + (n - g.k_lo), x, false);
                if (g.Cv && n >= g.v_lo && n < g.v_lo + g.kv_w) store4(g.Cv, (int64_t)m * g.ldcv + (n - g.v_lo), x, false);
            }
        }
    }
}

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
                const float pre = acc[i][j][r] + bn;
                float x = apply_act(pre, g.epi);
                if (g.Cpre) store_out<bf16>(g.Cpre, (int64_t)m * g.ldcpre + n, pre);
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
            if (g.Cpre) ((float *)g.Cpre)[(int64_t)m * g.ldcpre + n] = x;
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

namespace {
bool al(const void *p, unsigned bytes) { return ((uintptr_t)p & (bytes - 1)) == 0; }
// shapes and alignments the main bf16 kernel takes: K a multiple of 64, N
// and every column offset a multiple of 8, and every row start of every
// operand, output and residual 16-byte aligned
bool tiled_ok(const GemmArgs &g)
{
    if (g.K % TBK != 0 || g.N % 8 != 0 || g.lda % 8 != 0 || !al(g.A, 16) || !al(g.W, 16)) return false;
    if (g.ldc % (g.c_f32 ? 4 : 8) != 0 || !al(g.C, 16)) return false;
    if (g.C16 && (g.ldc16 % 8 != 0 || !al(g.C16, 16))) return false;
    if (g.Cpre && (g.ldcpre % 8 != 0 || !al(g.Cpre, 16))) return false;
    if (g.R32 && (g.ldr % 4 != 0 || !al(g.R32, 16))) return false;
    if (g.R16 && (g.ldr % 8 != 0 || !al(g.R16, 16))) return false;
    if ((g.Ck || g.Cv) && (g.kv_w % 8 != 0 || g.k_lo % 8 != 0 || g.v_lo % 8 != 0)) return false;
    if (g.Ck && (g.ldck % 8 != 0 || !al(g.Ck, 16))) return false;
    if (g.Cv && (g.ldcv % 8 != 0 || !al(g.Cv, 16))) return false;
    return true;
}
} // namespace

hipError_t launch_gemm_bf16(const GemmArgs &g, hipStream_t st)
{
    if (g.M <= 0 || g.N <= 0) return hipSuccess;
    if (tiled_ok(g)) {
        // 256-row tiles when they make at least two rounds of workgroups
        // (two per CU), else 128-row tiles: twice the workgroups for small
        // products (M-FALCON's 1024 candidates, narrow outputs)
        const int tiles_n = (g.N + 127) / 128;
        const int64_t t256 = (int64_t)tiles_n * ((g.M + 255) / 256);
        // 64-row tiles (2 waves) when even 128-row tiles would leave most CUs idle
        const int tbm = t256 >= 1024 ? 256 : (t256 >= 128 ? 128 : 64);
        const int64_t n_tiles = (int64_t)tiles_n * ((g.M + tbm - 1) / tbm);
        const int per_xcd = (int)((n_tiles + 7) / 8);
        const dim3 grid(8 * per_xcd);
        const int res = g.R32 ? 2 : (g.R16 ? 1 : 0);
#define HSTU_GEMM_LAUNCH(E, R)                                                                                         \
    do {                                                                                                               \
        if (tbm == 256)                                                                                                \
            hipLaunchKernelGGL((gemm_bf16_tiled_kernel<E, R, 2, 4, 1>), grid, dim3(256), 0, st, g, tiles_n,            \
                               (int)n_tiles, per_xcd);                                                                 \
        else if (tbm == 128)                                                                                           \
            hipLaunchKernelGGL((gemm_bf16_tiled_kernel<E, R, 1, 4, 1>), grid, dim3(256), 0, st, g, tiles_n,            \
                               (int)n_tiles, per_xcd);                                                                 \
        else                                                                                                           \
            hipLaunchKernelGGL((gemm_bf16_tiled_kernel<E, R, 1, 2, 1>), grid, dim3(128), 0, st, g, tiles_n,            \
                               (int)n_tiles, per_xcd);                                                                 \
    } while (0)
#define HSTU_GEMM_RES(E)                                                                                               \
    do {                                                                                                               \
        if (res == 2) HSTU_GEMM_LAUNCH(E, 2);                                                                          \
        else if (res == 1) HSTU_GEMM_LAUNCH(E, 1);                                                                     \
        else HSTU_GEMM_LAUNCH(E, 0);                                                                                   \
    } while (0)
        if (g.epi == EPI_SILU) HSTU_GEMM_RES(EPI_SILU);
        else if (g.epi == EPI_RELU) HSTU_GEMM_RES(EPI_RELU);
        else HSTU_GEMM_RES(EPI_NONE);
#undef HSTU_GEMM_RES
#undef HSTU_GEMM_LAUNCH
        return hipGetLastError();
    }
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
