/*
 * hstu_oracle.c -- plain, slow, fp64 CPU reference of the HSTU layer and its
 * pointwise aggregated attention.  TEST INFRASTRUCTURE ONLY: it is what the
 * GPU library is checked against, and nothing in the library links it.
 *
 * Source of every formula: the paper review page "Actions Speak Louder than
 * Words: Trillion-Parameter Sequential Transducers for Generative
 * Recommendations" (xllm-io paper-review blog, arXiv 2402.17152), written
 * below as [GR review].  Its section 3 ("technical architecture", core
 * formulas) gives the HSTU layer as three equations:
 *   Eq. 1  U, V, Q, K = Split(phi1(f1(X)))
 *   Eq. 2  A(X)V(X)   = phi2(Q K^T + rab^{p,t}) V(X)
 *   Eq. 3  Y(X)       = f2(Norm(A(X)V(X)) (.) U(X))
 * with f_i(X) = W_i X + b_i, and its M-FALCON subsection (section 3) the
 * microbatched candidate scoring against cacheable history computations.
 * Where the page leaves a step open the reading used here is stated at the
 * function (phi2 = SiLU(s)/N_max, the rab tables, LayerNorm over all H*d_v
 * features, the U|V|Q|K split order, residual y = x + f2(.)).
 *
 * Every loop below is the definition written out, in fp64, with no tiling,
 * fusion or reordering beyond what the definition states.  Inputs arrive as
 * fp64 arrays (bf16 / fp32 workload values are exactly representable).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* floor(log2(x)) for an integer x >= 1: how many halvings reach 1. */
static int floor_log2_u64(uint64_t x)
{
    int b = 0;
    while (x > 1) {
        x >>= 1;
        b++;
    }
    return b;
}

/* Time bucket of a timestamp difference (reading of rab^t in [GR review] §3
 * Eq. 2: a learned table over 128 buckets indexed by floor(log2(|dt| + 1)),
 * the index clamped to 127). */
int oracle_time_bucket(int64_t dt)
{
    uint64_t mag = dt < 0 ? (uint64_t)0 - (uint64_t)dt : (uint64_t)dt;
    int b = floor_log2_u64(mag + 1u); /* mag <= 2^63, so mag + 1 cannot wrap */
    return b < 127 ? b : 127;
}

/* Position index of rab^p: clip(j - i, -N, N) + N, j the key, i the query. */
static int64_t pos_index(int64_t j, int64_t i, int64_t N)
{
    int64_t r = j - i;
    if (r < -N) r = -N;
    if (r > N) r = N;
    return r + N;
}

static double silu(double s) { return s / (1.0 + exp(-s)); }

/* d/ds [s * sigmoid(s)] = sigmoid(s) * (1 + s * (1 - sigmoid(s))). */
static double silu_grad(double s)
{
    double sg = 1.0 / (1.0 + exp(-s));
    return sg * (1.0 + s * (1.0 - sg));
}

/* The pre-activation s_ij of one (query i, key j, head h) pair of Eq. 2:
 * q_i . k_j + rab_p[h][clip(j-i)] + rab_t[h][bucket(t_i - t_j)].
 * qrow/krow point at the head's d_qk values; ipos/jpos are positions inside
 * the sequence; rab_p/rab_t may be NULL (term absent). */
static double pair_logit(const double *qrow, const double *krow, int dqk, int64_t ipos, int64_t jpos,
                         int64_t N, int h, const double *rab_p, const double *rab_t, int64_t ti, int64_t tj,
                         int have_t)
{
    double s = 0.0;
    for (int c = 0; c < dqk; c++) s += qrow[c] * krow[c];
    if (rab_p) s += rab_p[(int64_t)h * (2 * N + 1) + pos_index(jpos, ipos, N)];
    if (rab_t && have_t) s += rab_t[(int64_t)h * 128 + oracle_time_bucket(ti - tj)];
    return s;
}

/* Sequence that owns global token r (offsets is non-decreasing). */
static int seq_of(int B, const int32_t *off, int64_t r)
{
    int lo = 0, hi = B - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) / 2;
        if (off[mid] <= r) lo = mid;
        else hi = mid - 1;
    }
    while (lo < B - 1 && off[lo + 1] <= r) lo++;
    return lo;
}

/*
 * Pointwise aggregated attention, [GR review] §3 Eq. 2, for a jagged batch.
 *   O[r, h*dv + c] = (1/N) * sum_{j <= i} SiLU(s_ij) * v[o_b + j, h, c]
 * for the token r = o_b + i of sequence b.  phi2 is read as SiLU(s)/N_max with
 * the causal mask including the diagonal (masked pairs contribute nothing);
 * no 1/sqrt(d) scale (Eq. 2 has none).
 * q, k: [T][H][dqk]; v: [T][H][dv]; out: [T][H*dv] (rows = every token, or
 * only the n_rows tokens listed in rows[] when rows != NULL).
 */
void oracle_attn_fwd(int B, const int32_t *off, const int64_t *ts, int H, int dqk, int dv, int64_t N,
                     const double *rab_p, const double *rab_t, const double *q, const double *k,
                     const double *v, double *out, int64_t n_rows, const int64_t *rows)
{
    int64_t T = off[B];
    int64_t nr = rows ? n_rows : T;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t w = 0; w < nr * H; w++) {
        int64_t ri = w / H;
        int h = (int)(w % H);
        int64_t r = rows ? rows[ri] : ri;
        int b = seq_of(B, off, r);
        int64_t o_b = off[b], i = r - o_b;
        double *acc = out + ri * (int64_t)H * dv + (int64_t)h * dv;
        for (int c = 0; c < dv; c++) acc[c] = 0.0;
        for (int64_t j = 0; j <= i; j++) {
            int64_t rk = o_b + j;
            double s = pair_logit(q + (r * H + h) * dqk, k + (rk * H + h) * dqk, dqk, i, j, N, h, rab_p, rab_t,
                                  ts ? ts[r] : 0, ts ? ts[rk] : 0, ts != NULL);
            double p = silu(s);
            const double *vr = v + (rk * H + h) * dv;
            for (int c = 0; c < dv; c++) acc[c] += p * vr[c];
        }
        for (int c = 0; c < dv; c++) acc[c] /= (double)N;
    }
}

/*
 * Norm(AV) (.) U of [GR review] §3 Eq. 3.  Norm is read as LayerNorm over all
 * F = H*dv features of a token, no affine, biased variance:
 *   mu = mean(O_r), var = mean((O_r - mu)^2), xhat = (O_r - mu)/sqrt(var + eps)
 *   G_r = xhat (.) U_r.    stats[r] = (mu, 1/sqrt(var + eps)).
 */
void oracle_ln_gate(int64_t T, int F, const double *O, const double *U, double eps, double *G, double *stats)
{
#pragma omp parallel for
    for (int64_t r = 0; r < T; r++) {
        const double *o = O + r * F;
        double mu = 0.0, var = 0.0;
        for (int c = 0; c < F; c++) mu += o[c];
        mu /= F;
        for (int c = 0; c < F; c++) var += (o[c] - mu) * (o[c] - mu);
        var /= F;
        double rstd = 1.0 / sqrt(var + eps);
        for (int c = 0; c < F; c++) G[r * F + c] = (o[c] - mu) * rstd * (U ? U[r * F + c] : 1.0);
        if (stats) {
            stats[2 * r] = mu;
            stats[2 * r + 1] = rstd;
        }
    }
}

/*
 * Backward of Eq. 2 (+ Eq. 3's Norm (.) U when U != NULL) by the chain rule,
 * one step at a time.  dout is the upstream gradient at G (or at O when U is
 * NULL).  Outputs are overwritten: dq, dk [T][H][dqk], dv [T][H][dv],
 * du [T][H*dv] (if U), drab_p [H][2N+1], drab_t [H][128] (if the tables are
 * given).  Sequential over pairs inside one (sequence, head); parallel across
 * (sequence, head) with private accumulators for the shared tables.
 */
void oracle_attn_bwd(int B, const int32_t *off, const int64_t *ts, int H, int dqk, int dv, int64_t N,
                     const double *rab_p, const double *rab_t, const double *q, const double *k,
                     const double *v, const double *U, double eps, const double *dout, double *dq, double *dk,
                     double *dvv, double *du, double *drab_p, double *drab_t)
{
    int64_t T = off[B];
    int F = H * dv;
    /* 1. forward O (Eq. 2), then the epilogue's input gradient dO. */
    double *O = (double *)calloc((size_t)(T > 0 ? T : 1) * F, sizeof(double));
    double *dO = (double *)calloc((size_t)(T > 0 ? T : 1) * F, sizeof(double));
    oracle_attn_fwd(B, off, ts, H, dqk, dv, N, rab_p, rab_t, q, k, v, O, 0, NULL);
    if (U) {
        /* G = xhat (.) U with xhat = (O - mu) * rstd:
         *   dU = xhat (.) dG ;  dxhat = dG (.) U ;
         *   dO = rstd * (dxhat - mean(dxhat) - xhat * mean(dxhat (.) xhat)). */
#pragma omp parallel for
        for (int64_t r = 0; r < T; r++) {
            const double *o = O + r * F;
            double mu = 0.0, var = 0.0;
            for (int c = 0; c < F; c++) mu += o[c];
            mu /= F;
            for (int c = 0; c < F; c++) var += (o[c] - mu) * (o[c] - mu);
            var /= F;
            double rstd = 1.0 / sqrt(var + eps);
            double m1 = 0.0, m2 = 0.0;
            for (int c = 0; c < F; c++) {
                double xh = (o[c] - mu) * rstd;
                double dxh = dout[r * F + c] * U[r * F + c];
                du[r * F + c] = xh * dout[r * F + c];
                m1 += dxh;
                m2 += dxh * xh;
            }
            m1 /= F;
            m2 /= F;
            for (int c = 0; c < F; c++) {
                double xh = (o[c] - mu) * rstd;
                double dxh = dout[r * F + c] * U[r * F + c];
                dO[r * F + c] = rstd * (dxh - m1 - xh * m2);
            }
        }
    } else {
        memcpy(dO, dout, sizeof(double) * (size_t)T * F);
    }
    memset(dq, 0, sizeof(double) * (size_t)T * H * dqk);
    memset(dk, 0, sizeof(double) * (size_t)T * H * dqk);
    memset(dvv, 0, sizeof(double) * (size_t)T * H * dv);
    int64_t PW = 2 * N + 1;
    if (drab_p) memset(drab_p, 0, sizeof(double) * (size_t)H * PW);
    if (drab_t) memset(drab_t, 0, sizeof(double) * (size_t)H * 128);
    /* 2. per pair: p = SiLU(s); O_i = (1/N) sum_j p_ij v_j, so
     *   dv_j += p_ij dO_i / N ;  dp_ij = dO_i . v_j / N ;  ds_ij = dp_ij SiLU'(s_ij)
     *   dq_i += ds_ij k_j ;  dk_j += ds_ij q_i ;  drab_p[idx] += ds ;  drab_t[bucket] += ds. */
#pragma omp parallel
    {
        double *lp = drab_p ? (double *)calloc((size_t)H * PW, sizeof(double)) : NULL;
        double *lt = drab_t ? (double *)calloc((size_t)H * 128, sizeof(double)) : NULL;
#pragma omp for schedule(dynamic, 1)
        for (int64_t w = 0; w < (int64_t)B * H; w++) {
            int b = (int)(w / H), h = (int)(w % H);
            int64_t o_b = off[b], L = off[b + 1] - off[b];
            for (int64_t i = 0; i < L; i++) {
                int64_t r = o_b + i;
                for (int64_t j = 0; j <= i; j++) {
                    int64_t rk = o_b + j;
                    const double *qi = q + (r * H + h) * dqk, *kj = k + (rk * H + h) * dqk;
                    const double *vj = v + (rk * H + h) * dv, *doi = dO + r * F + (int64_t)h * dv;
                    double s = pair_logit(qi, kj, dqk, i, j, N, h, rab_p, rab_t, ts ? ts[r] : 0,
                                          ts ? ts[rk] : 0, ts != NULL);
                    double p = silu(s);
                    double dp = 0.0;
                    for (int c = 0; c < dv; c++) {
                        dvv[(rk * H + h) * dv + c] += p * doi[c] / (double)N;
                        dp += doi[c] * vj[c];
                    }
                    dp /= (double)N;
                    double ds = dp * silu_grad(s);
                    for (int c = 0; c < dqk; c++) {
                        dq[(r * H + h) * dqk + c] += ds * kj[c];
                        dk[(rk * H + h) * dqk + c] += ds * qi[c];
                    }
                    if (lp && rab_p) lp[(int64_t)h * PW + pos_index(j, i, N)] += ds;
                    if (lt && rab_t && ts) lt[(int64_t)h * 128 + oracle_time_bucket(ts[r] - ts[rk])] += ds;
                }
            }
        }
#pragma omp critical
        {
            if (lp)
                for (int64_t x = 0; x < (int64_t)H * PW; x++) drab_p[x] += lp[x];
            if (lt)
                for (int64_t x = 0; x < (int64_t)H * 128; x++) drab_t[x] += lt[x];
        }
        free(lp);
        free(lt);
    }
    free(O);
    free(dO);
}

/*
 * dq for a subset of token rows only (same chain as oracle_attn_bwd, restricted
 * to what those rows need): for each listed row r = o_b + i, recompute O_r
 * (all heads), the epilogue's dO_r (when U is given), then
 *   dq[r] = sum_{j <= i} dP_ij SiLU'(s_ij) k_j,  dP_ij = dO_r . v_j / N.
 * dq_rows: [n_rows][H][dqk].
 */
void oracle_attn_bwd_dq_rows(int B, const int32_t *off, const int64_t *ts, int H, int dqk, int dv, int64_t N,
                             const double *rab_p, const double *rab_t, const double *q, const double *k,
                             const double *v, const double *U, double eps, const double *dout, int64_t n_rows,
                             const int64_t *rows, double *dq_rows)
{
    int F = H * dv;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t ri = 0; ri < n_rows; ri++) {
        int64_t r = rows[ri];
        int b = seq_of(B, off, r);
        int64_t o_b = off[b], i = r - o_b;
        double *O = (double *)malloc(sizeof(double) * F);
        double *dO = (double *)malloc(sizeof(double) * F);
        oracle_attn_fwd(B, off, ts, H, dqk, dv, N, rab_p, rab_t, q, k, v, O, 1, &r);
        if (U) {
            double mu = 0.0, var = 0.0;
            for (int c = 0; c < F; c++) mu += O[c];
            mu /= F;
            for (int c = 0; c < F; c++) var += (O[c] - mu) * (O[c] - mu);
            var /= F;
            double rstd = 1.0 / sqrt(var + eps), m1 = 0.0, m2 = 0.0;
            for (int c = 0; c < F; c++) {
                double xh = (O[c] - mu) * rstd, dxh = dout[r * F + c] * U[r * F + c];
                m1 += dxh;
                m2 += dxh * xh;
            }
            m1 /= F;
            m2 /= F;
            for (int c = 0; c < F; c++) {
                double xh = (O[c] - mu) * rstd, dxh = dout[r * F + c] * U[r * F + c];
                dO[c] = rstd * (dxh - m1 - xh * m2);
            }
        } else {
            for (int c = 0; c < F; c++) dO[c] = dout[r * F + c];
        }
        for (int h = 0; h < H; h++) {
            double *dqr = dq_rows + (ri * H + h) * dqk;
            for (int c = 0; c < dqk; c++) dqr[c] = 0.0;
            for (int64_t j = 0; j <= i; j++) {
                int64_t rk = o_b + j;
                const double *qi = q + (r * H + h) * dqk, *kj = k + (rk * H + h) * dqk;
                double s = pair_logit(qi, kj, dqk, i, j, N, h, rab_p, rab_t, ts ? ts[r] : 0, ts ? ts[rk] : 0,
                                      ts != NULL);
                double dp = 0.0;
                for (int c = 0; c < dv; c++) dp += dO[h * dv + c] * v[(rk * H + h) * dv + c];
                dp /= (double)N;
                double ds = dp * silu_grad(s);
                for (int c = 0; c < dqk; c++) dqr[c] += ds * kj[c];
            }
        }
        free(O);
        free(dO);
    }
}

/* Activation phi1: 0 = SiLU, 1 = ReLU. */
static double act(int phi1, double z) { return phi1 == 1 ? (z > 0.0 ? z : 0.0) : silu(z); }

/*
 * One HSTU layer forward, [GR review] §3 Eq. 1-3 plus the residual between
 * layers (its architecture tree: "residual connections between layers"):
 *   Z = X W1^T + b1 ; A = phi1(Z) ; U | V | Q | K = A's column blocks of width
 *   H*d (head-major inside) ; O = Eq. 2 ; G = Norm(O) (.) U ; Y = X + G W2^T + b2.
 * W1: [4Hd][D] ([out][in]); W2: [D][Hd]; rab tables as in oracle_attn_fwd.
 * kv_out (optional, [2][T][H][d]): this layer's K and V, the cache M-FALCON
 * scoring reads.  d_qk = d_v = d.
 */
void oracle_layer_fwd(int B, const int32_t *off, const int64_t *ts, int H, int d, int64_t N, int D,
                      const double *W1, const double *b1, const double *W2, const double *b2,
                      const double *rab_p, const double *rab_t, int phi1, double eps, const double *X,
                      double *Y, double *kv_out)
{
    int64_t T = off[B];
    int HD = H * d, Z4 = 4 * HD;
    size_t Tn = (size_t)(T > 0 ? T : 1);
    double *A = (double *)malloc(sizeof(double) * Tn * Z4);
    double *Qm = (double *)malloc(sizeof(double) * Tn * HD);
    double *Km = (double *)malloc(sizeof(double) * Tn * HD);
    double *Vm = (double *)malloc(sizeof(double) * Tn * HD);
    double *Um = (double *)malloc(sizeof(double) * Tn * HD);
    double *O = (double *)malloc(sizeof(double) * Tn * HD);
    double *G = (double *)malloc(sizeof(double) * Tn * HD);
#pragma omp parallel for
    for (int64_t r = 0; r < T; r++) {
        for (int n = 0; n < Z4; n++) {
            double z = b1 ? b1[n] : 0.0;
            for (int c = 0; c < D; c++) z += X[r * D + c] * W1[(int64_t)n * D + c];
            A[r * Z4 + n] = act(phi1, z);
        }
        for (int c = 0; c < HD; c++) {
            Um[r * HD + c] = A[r * Z4 + c];
            Vm[r * HD + c] = A[r * Z4 + HD + c];
            Qm[r * HD + c] = A[r * Z4 + 2 * HD + c];
            Km[r * HD + c] = A[r * Z4 + 3 * HD + c];
        }
    }
    oracle_attn_fwd(B, off, ts, H, d, d, N, rab_p, rab_t, Qm, Km, Vm, O, 0, NULL);
    oracle_ln_gate(T, HD, O, Um, eps, G, NULL);
#pragma omp parallel for
    for (int64_t r = 0; r < T; r++) {
        for (int n = 0; n < D; n++) {
            double y = b2 ? b2[n] : 0.0;
            for (int c = 0; c < HD; c++) y += G[r * HD + c] * W2[(int64_t)n * HD + c];
            Y[r * D + n] = X[r * D + n] + y;
        }
    }
    if (kv_out) {
        memcpy(kv_out, Km, sizeof(double) * (size_t)T * HD);
        memcpy(kv_out + (size_t)T * HD, Vm, sizeof(double) * (size_t)T * HD);
    }
    free(A);
    free(Qm);
    free(Km);
    free(Vm);
    free(Um);
    free(O);
    free(G);
}

/*
 * The part of one layer that M-FALCON caches for a history ([GR review] §3,
 * M-FALCON: the history's linear computations are cacheable): the layer's
 * K and V, i.e. the K and V column blocks of phi1(X W1^T + b1) (Eq. 1), for
 * every token r of X [T][D].  kv_out [2][T][H][d].  (The same values
 * oracle_layer_fwd returns in kv_out, without the attention and f2 that the
 * cache does not need.)
 */
void oracle_layer_kv(int64_t T, int H, int d, int D, const double *W1, const double *b1, int phi1,
                     const double *X, double *kv_out)
{
    int HD = H * d;
#pragma omp parallel for
    for (int64_t r = 0; r < T; r++)
        for (int c = 0; c < HD; c++) {
            int nk = 3 * HD + c, nv = HD + c; /* K and V column blocks of U | V | Q | K */
            double zk = b1 ? b1[nk] : 0.0, zv = b1 ? b1[nv] : 0.0;
            for (int e = 0; e < D; e++) {
                zk += X[r * D + e] * W1[(int64_t)nk * D + e];
                zv += X[r * D + e] * W1[(int64_t)nv * D + e];
            }
            kv_out[r * HD + c] = act(phi1, zk);
            kv_out[(size_t)T * HD + r * HD + c] = act(phi1, zv);
        }
}

/* d phi1 / dz: SiLU' as above; ReLU' read as 1 for z > 0, else 0. */
static double act_grad(int phi1, double z) { return phi1 == 1 ? (z > 0.0 ? 1.0 : 0.0) : silu_grad(z); }

/*
 * Backward of oracle_layer_fwd by the chain rule, one step at a time, for the
 * upstream gradient dY at Y.  The forward is recomputed in fp64 first.
 *   f2 and the residual:  dX = dY (residual) ; dG = dY W2 ; dW2 = dY^T G ;
 *                         db2 = column sums of dY
 *   Eq. 3 and Eq. 2:      oracle_attn_bwd with upstream gradient dG gives
 *                         dU, dV, dQ, dK and the rab table gradients
 *   phi1 and f1:          dZ = [dU | dV | dQ | dK] (.) phi1'(Z) ;
 *                         dX += dZ W1 ; dW1 = dZ^T X ; db1 = column sums of dZ
 * Outputs are overwritten: dX [T][D], dW1 [4Hd][D], db1 [4Hd], dW2 [D][Hd],
 * db2 [D], drab_p [H][2N+1], drab_t [H][128] (the last two when the tables
 * are given).
 */
void oracle_layer_bwd(int B, const int32_t *off, const int64_t *ts, int H, int d, int64_t N, int D,
                      const double *W1, const double *b1, const double *W2, const double *rab_p,
                      const double *rab_t, int phi1, double eps, const double *X, const double *dY, double *dX,
                      double *dW1, double *db1, double *dW2, double *db2, double *drab_p, double *drab_t)
{
    int64_t T = off[B];
    int HD = H * d, Z4 = 4 * HD;
    size_t Tn = (size_t)(T > 0 ? T : 1);
    double *Z = (double *)malloc(sizeof(double) * Tn * Z4);
    double *Qm = (double *)malloc(sizeof(double) * Tn * HD);
    double *Km = (double *)malloc(sizeof(double) * Tn * HD);
    double *Vm = (double *)malloc(sizeof(double) * Tn * HD);
    double *Um = (double *)malloc(sizeof(double) * Tn * HD);
    double *O = (double *)malloc(sizeof(double) * Tn * HD);
    double *G = (double *)malloc(sizeof(double) * Tn * HD);
    double *dG = (double *)malloc(sizeof(double) * Tn * HD);
    double *dA = (double *)malloc(sizeof(double) * Tn * Z4);
    /* forward: Z = X W1^T + b1 (kept before phi1), U | V | Q | K = phi1(Z) */
#pragma omp parallel for
    for (int64_t r = 0; r < T; r++) {
        for (int n = 0; n < Z4; n++) {
            double z = b1 ? b1[n] : 0.0;
            for (int c = 0; c < D; c++) z += X[r * D + c] * W1[(int64_t)n * D + c];
            Z[r * Z4 + n] = z;
        }
        for (int c = 0; c < HD; c++) {
            Um[r * HD + c] = act(phi1, Z[r * Z4 + c]);
            Vm[r * HD + c] = act(phi1, Z[r * Z4 + HD + c]);
            Qm[r * HD + c] = act(phi1, Z[r * Z4 + 2 * HD + c]);
            Km[r * HD + c] = act(phi1, Z[r * Z4 + 3 * HD + c]);
        }
    }
    oracle_attn_fwd(B, off, ts, H, d, d, N, rab_p, rab_t, Qm, Km, Vm, O, 0, NULL);
    oracle_ln_gate(T, HD, O, Um, eps, G, NULL);
    /* f2: dG[r][c] = sum_n dY[r][n] W2[n][c] */
#pragma omp parallel for
    for (int64_t r = 0; r < T; r++)
        for (int c = 0; c < HD; c++) {
            double s = 0.0;
            for (int n = 0; n < D; n++) s += dY[r * D + n] * W2[(int64_t)n * HD + c];
            dG[r * HD + c] = s;
        }
    /* dW2[n][c] = sum_r dY[r][n] G[r][c] ; db2[n] = sum_r dY[r][n] */
#pragma omp parallel for
    for (int n = 0; n < D; n++) {
        for (int c = 0; c < HD; c++) {
            double s = 0.0;
            for (int64_t r = 0; r < T; r++) s += dY[r * D + n] * G[r * HD + c];
            dW2[(int64_t)n * HD + c] = s;
        }
        if (db2) {
            double s = 0.0;
            for (int64_t r = 0; r < T; r++) s += dY[r * D + n];
            db2[n] = s;
        }
    }
    /* attention and its gate: gradients at U, V, Q, K */
    {
        double *dq = (double *)malloc(sizeof(double) * Tn * HD);
        double *dk = (double *)malloc(sizeof(double) * Tn * HD);
        double *dv = (double *)malloc(sizeof(double) * Tn * HD);
        double *du = (double *)malloc(sizeof(double) * Tn * HD);
        oracle_attn_bwd(B, off, ts, H, d, d, N, rab_p, rab_t, Qm, Km, Vm, Um, eps, dG, dq, dk, dv, du, drab_p,
                        drab_t);
        for (int64_t r = 0; r < T; r++)
            for (int c = 0; c < HD; c++) {
                dA[r * Z4 + c] = du[r * HD + c];
                dA[r * Z4 + HD + c] = dv[r * HD + c];
                dA[r * Z4 + 2 * HD + c] = dq[r * HD + c];
                dA[r * Z4 + 3 * HD + c] = dk[r * HD + c];
            }
        free(dq);
        free(dk);
        free(dv);
        free(du);
    }
    /* phi1: dZ = dA (.) phi1'(Z), in dA */
    for (int64_t e = 0; e < (int64_t)T * Z4; e++) dA[e] *= act_grad(phi1, Z[e]);
    /* f1 and the residual: dX[r][c] = dY[r][c] + sum_n dZ[r][n] W1[n][c] */
#pragma omp parallel for
    for (int64_t r = 0; r < T; r++)
        for (int c = 0; c < D; c++) {
            double s = dY[r * D + c];
            for (int n = 0; n < Z4; n++) s += dA[r * Z4 + n] * W1[(int64_t)n * D + c];
            dX[r * D + c] = s;
        }
    /* dW1[n][c] = sum_r dZ[r][n] X[r][c] ; db1[n] = sum_r dZ[r][n] */
#pragma omp parallel for
    for (int n = 0; n < Z4; n++) {
        for (int c = 0; c < D; c++) {
            double s = 0.0;
            for (int64_t r = 0; r < T; r++) s += dA[r * Z4 + n] * X[r * D + c];
            dW1[(int64_t)n * D + c] = s;
        }
        if (db1) {
            double s = 0.0;
            for (int64_t r = 0; r < T; r++) s += dA[r * Z4 + n];
            db1[n] = s;
        }
    }
    free(Z);
    free(Qm);
    free(Km);
    free(Vm);
    free(Um);
    free(O);
    free(G);
    free(dG);
    free(dA);
}

/*
 * M-FALCON scoring of one candidate at a time ([GR review] §3, M-FALCON: the
 * m candidates are split into microbatches whose attention operations are
 * identical, and the history's linear and attention computations are cached).
 * Per user u with history length n_u and cache K_l, V_l ([T_hist][H][d]) for
 * each layer l, a candidate token x sits at position n_u with time cand_ts[u]
 * and attends to the whole history and to itself, never to other
 * candidates.  Per layer:
 *   u,v,q,k = Split(phi1(x W1^T + b1))
 *   o = (1/N) [ sum_{j < n_u} SiLU(q.K_j + rab_p[clip(j - n_u)] + rab_t[b(t_c - t_j)]) V_j
 *              + SiLU(q.k + rab_p[clip(0)] + rab_t[b(0)]) v ]
 *   x = x + (Norm(o) (.) u) W2^T + b2.
 * The final x (fp64) is the candidate's score vector, y [M][D].
 * Layer l's parameters are at W1 + l*4Hd*D, b1 + l*4Hd, W2 + l*D*Hd,
 * b2 + l*D, rab_p + l*H*(2N+1), rab_t + l*H*128; kv [n_layers][2][T_hist][H][d].
 */
void oracle_mfalcon(int n_users, const int32_t *hist_off, const int64_t *hist_ts, const int32_t *cand_off,
                    const int64_t *cand_ts, int n_layers, int H, int d, int64_t N, int D, const double *W1,
                    const double *b1, const double *W2, const double *b2, const double *rab_p,
                    const double *rab_t, int phi1, double eps, const double *kv, const double *x_cand,
                    double *y)
{
    int HD = H * d, Z4 = 4 * HD;
    int64_t Th = hist_off[n_users], M = cand_off[n_users];
    int64_t PW = 2 * N + 1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t c = 0; c < M; c++) {
        int u = seq_of(n_users, cand_off, c);
        int64_t ho = hist_off[u], nu = hist_off[u + 1] - hist_off[u];
        double *x = (double *)malloc(sizeof(double) * D);
        double *a = (double *)malloc(sizeof(double) * Z4);
        double *o = (double *)malloc(sizeof(double) * HD);
        double *g = (double *)malloc(sizeof(double) * HD);
        for (int n = 0; n < D; n++) x[n] = x_cand[c * D + n];
        for (int l = 0; l < n_layers; l++) {
            const double *w1 = W1 + (int64_t)l * Z4 * D, *w2 = W2 + (int64_t)l * D * HD;
            const double *bb1 = b1 ? b1 + (int64_t)l * Z4 : NULL, *bb2 = b2 ? b2 + (int64_t)l * D : NULL;
            const double *rp = rab_p ? rab_p + (int64_t)l * H * PW : NULL;
            const double *rt = rab_t ? rab_t + (int64_t)l * H * 128 : NULL;
            const double *Kc = kv + (int64_t)l * 2 * Th * HD, *Vc = Kc + Th * HD;
            for (int n = 0; n < Z4; n++) {
                double z = bb1 ? bb1[n] : 0.0;
                for (int e = 0; e < D; e++) z += x[e] * w1[(int64_t)n * D + e];
                a[n] = act(phi1, z);
            }
            const double *uu = a, *vv = a + HD, *qq = a + 2 * HD, *kk = a + 3 * HD;
            for (int h = 0; h < H; h++) {
                double *acc = o + h * d;
                for (int e = 0; e < d; e++) acc[e] = 0.0;
                for (int64_t j = 0; j < nu; j++) {
                    int64_t rk = ho + j;
                    double s = pair_logit(qq + h * d, Kc + (rk * H + h) * d, d, nu, j, N, h, rp, rt,
                                          cand_ts ? cand_ts[u] : 0, hist_ts ? hist_ts[rk] : 0,
                                          cand_ts != NULL && hist_ts != NULL);
                    double p = silu(s);
                    for (int e = 0; e < d; e++) acc[e] += p * Vc[(rk * H + h) * d + e];
                }
                double s = pair_logit(qq + h * d, kk + h * d, d, nu, nu, N, h, rp, rt, 0, 0,
                                      cand_ts != NULL && hist_ts != NULL);
                double p = silu(s);
                for (int e = 0; e < d; e++) acc[e] = (acc[e] + p * vv[h * d + e]) / (double)N;
            }
            oracle_ln_gate(1, HD, o, uu, eps, g, NULL);
            for (int n = 0; n < D; n++) {
                double yy = bb2 ? bb2[n] : 0.0;
                for (int e = 0; e < HD; e++) yy += g[e] * w2[(int64_t)n * HD + e];
                x[n] += yy;
            }
        }
        for (int n = 0; n < D; n++) y[c * D + n] = x[n];
        free(x);
        free(a);
        free(o);
        free(g);
    }
}

/*
 * Appending new actions to a user's cached history, one layer ([GR review]
 * §3: the history's linear and attention computations are cacheable, and
 * the architecture tree's streaming setting adds actions as they arrive).
 * User u has a cached history of n_u tokens (this layer's K, V in kv_cache
 * [2][T_hist][H][d], rows hist_off[u]..) and a_u new tokens x_new (rows
 * add_off[u]..).  New token i of user u is the token at position n_u + i
 * of the user's sequence, with time add_ts[r]:
 *   a = phi1(x W1^T + b1) = u | v | q | k of the new token (Eq. 1)
 *   o = (1/N) [ sum_{j < n_u} SiLU(q.K_j + rab_p[clip(j - (n_u + i))] + rab_t[b(t - t_j)]) V_j
 *             + sum_{i' <= i} SiLU(q.k_i' + rab_p[clip(i' - i)] + rab_t[b(t - t_i')]) v_i' ]   (Eq. 2)
 *   y = x + (Norm(o) (.) u) W2^T + b2                                          (Eq. 3 + residual)
 * i.e. exactly rows n_u.. of the layer over the user's whole sequence
 * [history; new], whose causal mask lets a new token see the history and
 * the new tokens up to itself.  y_new [T_new][D]; kv_out [2][T_hist + T_new]
 * [H][d] (optional): the merged cache, user u's history rows then its new
 * rows, starting at row hist_off[u] + add_off[u].
 */
void oracle_layer_append(int U, const int32_t *hist_off, const int64_t *hist_ts, const int32_t *add_off,
                         const int64_t *add_ts, int H, int d, int64_t N, int D, const double *W1, const double *b1,
                         const double *W2, const double *b2, const double *rab_p, const double *rab_t, int phi1,
                         double eps, const double *kv_cache, const double *x_new, double *y_new, double *kv_out)
{
    int HD = H * d, Z4 = 4 * HD;
    int64_t Th = hist_off[U], Tn = add_off[U];
    const double *Kc = kv_cache, *Vc = kv_cache + Th * HD;
    double *A = (double *)malloc(sizeof(double) * (size_t)(Tn > 0 ? Tn : 1) * Z4);
    int have_t = hist_ts != NULL && add_ts != NULL;
    /* f1 + phi1 of every new token */
#pragma omp parallel for
    for (int64_t r = 0; r < Tn; r++)
        for (int n = 0; n < Z4; n++) {
            double z = b1 ? b1[n] : 0.0;
            for (int e = 0; e < D; e++) z += x_new[r * D + e] * W1[(int64_t)n * D + e];
            A[r * Z4 + n] = act(phi1, z);
        }
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < Tn; r++) {
        int u = seq_of(U, add_off, r);
        int64_t ho = hist_off[u], nu = hist_off[u + 1] - hist_off[u], ao = add_off[u], i = r - ao;
        int64_t pos = nu + i;
        const double *uu = A + r * Z4, *qq = A + r * Z4 + 2 * HD;
        double *o = (double *)malloc(sizeof(double) * HD);
        double *g = (double *)malloc(sizeof(double) * HD);
        for (int h = 0; h < H; h++) {
            double *acc = o + h * d;
            for (int e = 0; e < d; e++) acc[e] = 0.0;
            for (int64_t j = 0; j < nu; j++) { /* the cached history */
                int64_t rk = ho + j;
                double s = pair_logit(qq + h * d, Kc + (rk * H + h) * d, d, pos, j, N, h, rab_p, rab_t,
                                      have_t ? add_ts[r] : 0, have_t ? hist_ts[rk] : 0, have_t);
                double p = silu(s);
                for (int e = 0; e < d; e++) acc[e] += p * Vc[(rk * H + h) * d + e];
            }
            for (int64_t i2 = 0; i2 <= i; i2++) { /* the new tokens up to this one */
                int64_t rk = ao + i2;
                const double *kk = A + rk * Z4 + 3 * HD, *vv = A + rk * Z4 + HD;
                double s = pair_logit(qq + h * d, kk + h * d, d, pos, nu + i2, N, h, rab_p, rab_t,
                                      have_t ? add_ts[r] : 0, have_t ? add_ts[rk] : 0, have_t);
                double p = silu(s);
                for (int e = 0; e < d; e++) acc[e] += p * vv[h * d + e];
            }
            for (int e = 0; e < d; e++) acc[e] /= (double)N;
        }
        oracle_ln_gate(1, HD, o, uu, eps, g, NULL);
        for (int n = 0; n < D; n++) {
            double yy = b2 ? b2[n] : 0.0;
            for (int e = 0; e < HD; e++) yy += g[e] * W2[(int64_t)n * HD + e];
            y_new[r * D + n] = x_new[r * D + n] + yy;
        }
        free(o);
        free(g);
    }
    if (kv_out) {
        int64_t Tm = Th + Tn;
        for (int u = 0; u < U; u++) {
            int64_t ho = hist_off[u], nu = hist_off[u + 1] - ho, ao = add_off[u], au = add_off[u + 1] - ao;
            int64_t mo = ho + ao; /* merged offset of user u */
            for (int64_t j = 0; j < nu; j++)
                for (int c = 0; c < HD; c++) {
                    kv_out[(mo + j) * HD + c] = Kc[(ho + j) * HD + c];
                    kv_out[Tm * HD + (mo + j) * HD + c] = Vc[(ho + j) * HD + c];
                }
            for (int64_t i = 0; i < au; i++)
                for (int c = 0; c < HD; c++) {
                    kv_out[(mo + nu + i) * HD + c] = A[(ao + i) * Z4 + 3 * HD + c];
                    kv_out[Tm * HD + (mo + nu + i) * HD + c] = A[(ao + i) * Z4 + HD + c];
                }
        }
    }
    free(A);
}

/*
 * The comparator the pages set pointwise aggregated attention against
 * ([GR review] §5 efficiency table: Transformers built on FlashAttention2;
 * §6 component ablation: softmax in place of the pointwise normalisation,
 * without rab): causal softmax attention per sequence b, head h and query
 * i, with the usual 1/sqrt(d) scale,
 *   s_ij = q_i . k_j / sqrt(dqk) for j <= i,
 *   O_i  = sum_j exp(s_ij - max_j s_ij) v_j / sum_j exp(s_ij - max_j s_ij).
 * lse (optional, [T][H]): max_j s_ij + log(sum_j exp(s_ij - max_j s_ij)).
 */
void oracle_softmax_attn_fwd(int B, const int32_t *off, int H, int dqk, int dv, const double *q, const double *k,
                             const double *v, double *out, double *lse)
{
    int64_t T = off[B];
    double scale = 1.0 / sqrt((double)dqk);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t w = 0; w < T * H; w++) {
        int64_t r = w / H;
        int h = (int)(w % H);
        int b = seq_of(B, off, r);
        int64_t o_b = off[b], i = r - o_b;
        double *s = (double *)malloc(sizeof(double) * (size_t)(i + 1));
        double mx = -INFINITY;
        for (int64_t j = 0; j <= i; j++) {
            double x = 0.0;
            for (int c = 0; c < dqk; c++) x += q[(r * H + h) * dqk + c] * k[((o_b + j) * H + h) * dqk + c];
            s[j] = x * scale;
            if (s[j] > mx) mx = s[j];
        }
        double den = 0.0;
        double *acc = out + r * (int64_t)H * dv + (int64_t)h * dv;
        for (int c = 0; c < dv; c++) acc[c] = 0.0;
        for (int64_t j = 0; j <= i; j++) {
            double p = exp(s[j] - mx);
            den += p;
            for (int c = 0; c < dv; c++) acc[c] += p * v[((o_b + j) * H + h) * dv + c];
        }
        for (int c = 0; c < dv; c++) acc[c] /= den;
        if (lse) lse[r * H + h] = mx + log(den);
        free(s);
    }
}

/*
 * Stochastic Length ([GR review] §3 SL: each user's history is cut to a
 * length drawn from L = min(n, ceil(n u^(1/alpha))), u ~ U(0, 1), and a
 * random subsequence of that length is kept).  Readings: a length is at least
 * 1 for a non-empty history; the subsequence is a uniformly random subset of
 * L of the n actions kept in their original order, drawn as the L actions
 * with the smallest random keys (ties by position).  The random numbers (u
 * per sequence, a uint32 key per action) are inputs.  Outputs: out_off [B+1]
 * (the sampled batch's offsets) and out_idx [out_off[B]] (for each sampled
 * action, its row in the input batch).  A plain O(n^2) rank count per action.
 */
void oracle_sl_sample(int B, const int32_t *off, double alpha, const double *u, const uint32_t *keys,
                      int32_t *out_off, int32_t *out_idx)
{
    out_off[0] = 0;
    for (int b = 0; b < B; b++) {
        int64_t o = off[b], n = off[b + 1] - off[b];
        int64_t L = 0;
        if (n > 0) {
            double x = ceil((double)n * pow(u[b], 1.0 / alpha));
            L = x < 1.0 ? 1 : (x > (double)n ? n : (int64_t)x);
        }
        int64_t w = out_off[b];
        for (int64_t j = 0; j < n; j++) {
            int64_t rank = 0; /* actions before j in (key, position) order */
            for (int64_t i = 0; i < n; i++)
                if (keys[o + i] < keys[o + j] || (keys[o + i] == keys[o + j] && i < j)) rank++;
            if (rank < L) out_idx[w++] = (int32_t)(o + j);
        }
        out_off[b + 1] = (int32_t)w;
    }
}

int oracle_abi_version(void) { return 1; }
