/*
 * mhc_oracle.c -- plain, slow, fp64 CPU oracle for the per-layer mHC operator.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call
 * this file: only the test suite, the smoke check and the benchmark's CPU-baseline
 * leg use it.  It shares no code, header, table or helper with the HIP kernels.
 *
 * Sources (web pages on mHC, Manifold-Constrained Hyper-Connections):
 *   [P1] chatgpz.de, "Von Residualverbindungen zu Hyperverbindungen" (the n-stream
 *        buffer, the three maps H_pre, H_post, H_res and the update rule
 *        X_{l+1} = H_res X_l + H_post^T F(H_pre X_l)),
 *        "Vielfaeltig eingeschraenkte Hyperverbindungen" (H_res projected onto the
 *        doubly stochastic matrices with Sinkhorn-Knopp, which alternates row and
 *        column normalisation, 20 iterations; non-negative pre/post maps),
 *        "Systemarbeit und Schulungsaufwand" (coefficients from fused RMSNorm,
 *        projection and gating), "Warum Hyperverbindungen instabil werden"
 *        (composite of the residual mixers over depth, Amax gain from the
 *        maximal row and column sums).
 *   [P5] staging.reportify.cn, section "mHC方法原理" notes [10] (doubly stochastic:
 *        non-negative entries, unit row and column sums), [12] (non-negative
 *        input/output maps), [15] (closure under products, spectral norm <= 1),
 *        [16] (t_max = 20 Sinkhorn-Knopp iterations); section "高效基础设施设计"
 *        note [17] (RMSNorm reordered) and [19] (Sinkhorn with its own backward),
 *        [21] (recompute in backward).
 *
 * Readings where the pages are silent (all fixed as inputs, shared with the GPU
 * side only through the seeded input generator):
 *   - coefficients: z = alpha_g * ((v*gamma) . W) / r + b with v = vec(X_t)
 *     stream-major, r = sqrt(mean(v^2) + eps); alpha_g a fixed scalar per group
 *     (pre, post, res); logit order pre[0..n), post[n..2n), res[2n..2n+n*n)
 *     row-major (res index 2n + i*n + j);
 *   - non-negativity: plain logistic sigmoid;
 *   - Sinkhorn input exp(z) (raw, no shift here), one iteration = a row
 *     normalisation then a column normalisation;
 *   - H_res[i][j] feeds stream j into output stream i;
 *   - composite P_l = H_res^(l) P_{l-1}; gains are absolute row / column sums.
 *
 * Every function works per token with fp64 arithmetic on fp64 inputs (the caller
 * widens bf16/fp32 storage exactly).  Outputs are fp64 and never rounded.
 * Layouts (row-major, contiguous): X, Xout, G, dX: [T][n][C]; F, u, g, dF: [T][C];
 * z: [T][K] with K = n*n + 2n; W: [n*C][K]; H_pre, H_post: [T][n]; H_res: [T][n][n].
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_MAXN 8
#define ORC_MAXK (ORC_MAXN * ORC_MAXN + 2 * ORC_MAXN)

static int orc_group(int k, int n) { return k < n ? 0 : (k < 2 * n ? 1 : 2); }

static double orc_sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* Coefficients and gating, per token.
 * [P1] "Systemarbeit und Schulungsaufwand": RMSNorm, projections and gating produce
 * the mHC maps; [P1] "Vielfaeltig eingeschraenkte ..." / [P5] note [12]: pre and
 * post coefficients are non-negative (sigmoid here).  Plain RMSNorm first, then the
 * matmul -- no reordering: the oracle follows the definition. */
void orc_coeffs(int64_t T, int n, int64_t C, const double* X, const double* gamma,
                double eps, const double* W, const double* bias, const double* alpha,
                double* z, double* r, double* Hpre, double* Hpost)
{
    const int64_t N = (int64_t)n * C;
    const int K = n * n + 2 * n;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        const double* v = X + t * N;
        double ss = 0.0;
        for (int64_t i = 0; i < N; ++i) ss += v[i] * v[i];
        const double rr = sqrt(ss / (double)N + eps);
        double p[ORC_MAXK];
        for (int k = 0; k < K; ++k) p[k] = 0.0;
        for (int64_t i = 0; i < N; ++i) {
            const double y = gamma[i] * (v[i] / rr); /* RMSNorm output */
            const double* wr = W + i * K;
            for (int k = 0; k < K; ++k) p[k] += y * wr[k];
        }
        double* zt = z + t * K;
        for (int k = 0; k < K; ++k) zt[k] = alpha[orc_group(k, n)] * p[k] + bias[k];
        if (r) r[t] = rr;
        for (int k = 0; k < n; ++k) {
            if (Hpre) Hpre[t * n + k] = orc_sigmoid(zt[k]);
            if (Hpost) Hpost[t * n + k] = orc_sigmoid(zt[n + k]);
        }
    }
}

/* Sinkhorn-Knopp on one n x n logit block.
 * [P1] "Vielfaeltig eingeschraenkte ...": alternate row and column normalisation;
 * [P5] note [16]: t_max iterations.  M = exp(Z); each iteration divides every row
 * by its sum, then every column by its sum.  Optionally records every divisor and
 * every intermediate matrix (after each row step and each column step). */
void orc_sinkhorn_one(int n, const double* zres, int iters, double* H,
                      double* rho, double* kap, double* Yrow, double* Ycol)
{
    double M[ORC_MAXN * ORC_MAXN];
    for (int a = 0; a < n * n; ++a) M[a] = exp(zres[a]);
    for (int s = 0; s < iters; ++s) {
        for (int i = 0; i < n; ++i) {
            double rs = 0.0;
            for (int j = 0; j < n; ++j) rs += M[i * n + j];
            if (rho) rho[s * n + i] = rs;
            for (int j = 0; j < n; ++j) M[i * n + j] /= rs;
        }
        if (Yrow) memcpy(Yrow + (size_t)s * n * n, M, sizeof(double) * n * n);
        for (int j = 0; j < n; ++j) {
            double cs = 0.0;
            for (int i = 0; i < n; ++i) cs += M[i * n + j];
            if (kap) kap[s * n + j] = cs;
            for (int i = 0; i < n; ++i) M[i * n + j] /= cs;
        }
        if (Ycol) memcpy(Ycol + (size_t)s * n * n, M, sizeof(double) * n * n);
    }
    memcpy(H, M, sizeof(double) * n * n);
}

/* H_res for T tokens from their res logits (row stride ld doubles). */
void orc_sinkhorn(int64_t T, int n, const double* zres, int64_t ld, int iters, double* Hres)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        orc_sinkhorn_one(n, zres + t * ld, iters, Hres + t * n * n, NULL, NULL, NULL, NULL);
}

/* Read map, [P1] "Von Residualverbindungen ...": u = H_pre X (1 x n times n x C). */
void orc_pre(int64_t T, int n, int64_t C, const double* X, const double* Hpre, double* u)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        for (int64_t c = 0; c < C; ++c) {
            double acc = 0.0;
            for (int k = 0; k < n; ++k) acc += Hpre[t * n + k] * X[(t * n + k) * C + c];
            u[t * C + c] = acc;
        }
}

/* Write map and residual mix, [P1] update rule: X' = H_res X + H_post^T F. */
void orc_post_res(int64_t T, int n, int64_t C, const double* X, const double* F,
                  const double* Hres, const double* Hpost, double* Xout)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        for (int i = 0; i < n; ++i)
            for (int64_t c = 0; c < C; ++c) {
                double acc = 0.0;
                for (int j = 0; j < n; ++j)
                    acc += Hres[(t * n + i) * n + j] * X[(t * n + j) * C + c];
                acc += Hpost[t * n + i] * F[t * C + c];
                Xout[(t * n + i) * C + c] = acc;
            }
}

/* Backward of the update rule with F's output held as an input.
 * G = dL/dX'.  dF = H_post^T-contracted G; dH_post[i] = <G_i, F>;
 * dH_res[i][j] = <G_i, X_j>; optional dXdir = H_res^T G (written). */
void orc_post_res_bwd(int64_t T, int n, int64_t C, const double* G, const double* X,
                      const double* F, const double* Hres, const double* Hpost,
                      double* dF, double* dHres, double* dHpost, double* dXdir)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        const double* Gt = G + t * n * C;
        const double* Xt = X + t * n * C;
        const double* Ft = F + t * C;
        for (int64_t c = 0; c < C; ++c) {
            double acc = 0.0;
            for (int i = 0; i < n; ++i) acc += Hpost[t * n + i] * Gt[i * C + c];
            dF[t * C + c] = acc;
        }
        for (int i = 0; i < n; ++i) {
            double acc = 0.0;
            for (int64_t c = 0; c < C; ++c) acc += Gt[i * C + c] * Ft[c];
            dHpost[t * n + i] = acc;
            for (int j = 0; j < n; ++j) {
                double a2 = 0.0;
                for (int64_t c = 0; c < C; ++c) a2 += Gt[i * C + c] * Xt[j * C + c];
                dHres[(t * n + i) * n + j] = a2;
            }
        }
        if (dXdir) {
            for (int j = 0; j < n; ++j)
                for (int64_t c = 0; c < C; ++c) {
                    double acc = 0.0;
                    for (int i = 0; i < n; ++i)
                        acc += Hres[(t * n + i) * n + j] * Gt[i * C + c];
                    dXdir[(t * n + j) * C + c] = acc;
                }
        }
    }
}

/* Backward of the read map: dH_pre[k] = <g, X_k>; optional dX += H_pre[k] g. */
void orc_pre_bwd(int64_t T, int n, int64_t C, const double* g, const double* X,
                 const double* Hpre, double* dHpre, double* dX)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int k = 0; k < n; ++k) {
            double acc = 0.0;
            for (int64_t c = 0; c < C; ++c) acc += g[t * C + c] * X[(t * n + k) * C + c];
            dHpre[t * n + k] = acc;
            if (dX)
                for (int64_t c = 0; c < C; ++c)
                    dX[(t * n + k) * C + c] += Hpre[t * n + k] * g[t * C + c];
        }
    }
}

/* Sinkhorn-Knopp backward ([P5] note [19]: the iterations get their own backward;
 * note [21]: intermediates are recomputed, not stored).  The forward is re-run
 * from the logits keeping every intermediate matrix, then each normalisation is
 * differentiated in reverse: for Y = M / colsum, dM_ij = (dY_ij - sum_m dY_mj Y_mj)
 * / kappa_j; for Y = M / rowsum, dM_ij = (dY_ij - sum_m dY_im Y_im) / rho_i;
 * finally d z = dM (.) exp(z). */
void orc_sinkhorn_bwd_one(int n, const double* zres, int iters, const double* dH, double* dz)
{
    double* buf = (double*)malloc(sizeof(double) * (size_t)iters * (2 * n * n + 2 * n) + 1);
    double* rho = buf;
    double* kap = rho + (size_t)iters * n;
    double* Yr = kap + (size_t)iters * n;
    double* Yc = Yr + (size_t)iters * n * n;
    double H[ORC_MAXN * ORC_MAXN], Gb[ORC_MAXN * ORC_MAXN];
    orc_sinkhorn_one(n, zres, iters, H, rho, kap, Yr, Yc);
    memcpy(Gb, dH, sizeof(double) * n * n);
    for (int s = iters - 1; s >= 0; --s) {
        const double* Y = Yc + (size_t)s * n * n;
        for (int j = 0; j < n; ++j) {
            double a = 0.0;
            for (int m = 0; m < n; ++m) a += Gb[m * n + j] * Y[m * n + j];
            for (int i = 0; i < n; ++i) Gb[i * n + j] = (Gb[i * n + j] - a) / kap[s * n + j];
        }
        Y = Yr + (size_t)s * n * n;
        for (int i = 0; i < n; ++i) {
            double b = 0.0;
            for (int m = 0; m < n; ++m) b += Gb[i * n + m] * Y[i * n + m];
            for (int j = 0; j < n; ++j) Gb[i * n + j] = (Gb[i * n + j] - b) / rho[s * n + i];
        }
    }
    for (int a = 0; a < n * n; ++a) dz[a] = Gb[a] * exp(zres[a]);
    free(buf);
}

void orc_sinkhorn_bwd(int64_t T, int n, const double* zres, int64_t ld, int iters,
                      const double* dHres, double* dzres)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        orc_sinkhorn_bwd_one(n, zres + t * ld, iters, dHres + t * n * n, dzres + t * n * n);
}

/* Backward of the sigmoid gating: dz = dH * s * (1 - s), s = sigmoid(z); writes the
 * pre and post columns [0, 2n) of dz (row stride K). */
void orc_gating_bwd(int64_t T, int n, const double* z, const double* dHpre,
                    const double* dHpost, double* dz)
{
    const int K = n * n + 2 * n;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        for (int k = 0; k < n; ++k) {
            const double sp = orc_sigmoid(z[t * K + k]);
            const double so = orc_sigmoid(z[t * K + n + k]);
            dz[t * K + k] = dHpre[t * n + k] * sp * (1.0 - sp);
            dz[t * K + n + k] = dHpost[t * n + k] * so * (1.0 - so);
        }
}

/* Backward of the coefficients (RMSNorm + projection + per-group scale + bias),
 * given dz for all K logits.  Recomputes r from X (nothing is taken from the
 * forward).  With y_i = gamma_i v_i / r and q_k = alpha_g(k) dz_k:
 *   dy_i  = sum_k W[i][k] q_k                       (gradient w.r.t. y)
 *   dv_i  = gamma_i dy_i / r - v_i (sum_m gamma_m v_m dy_m) / (N r^3)
 *   dX   += dv;  dW[i][k] = sum_t y_i q_k;  db_k = sum_t dz_k;
 *   dgamma_i = sum_t v_i dy_i / r.
 * The RMS term is computed directly from its definition (no identity). */
void orc_coeffs_bwd(int64_t T, int n, int64_t C, const double* X, const double* gamma,
                    double eps, const double* W, const double* alpha, const double* dz,
                    double* dX, double* dW, double* db, double* dgamma)
{
    const int64_t N = (int64_t)n * C;
    const int K = n * n + 2 * n;
    int nth = 1;
#ifdef _OPENMP
    nth = omp_get_max_threads();
#endif
    /* per-thread partial sums over tokens, combined in thread order */
    double* part = (double*)calloc((size_t)nth * ((size_t)N * K + K + N), sizeof(double));
#pragma omp parallel
    {
        int tid = 0;
#ifdef _OPENMP
        tid = omp_get_thread_num();
#endif
        double* pW = part + (size_t)tid * ((size_t)N * K + K + N);
        double* pb = pW + (size_t)N * K;
        double* pg = pb + K;
        double* dy = (double*)malloc(sizeof(double) * (size_t)N);
#pragma omp for schedule(static)
        for (int64_t t = 0; t < T; ++t) {
            const double* v = X + t * N;
            double ss = 0.0;
            for (int64_t i = 0; i < N; ++i) ss += v[i] * v[i];
            const double rr = sqrt(ss / (double)N + eps);
            double q[ORC_MAXK];
            for (int k = 0; k < K; ++k) q[k] = alpha[orc_group(k, n)] * dz[t * K + k];
            double S = 0.0;
            for (int64_t i = 0; i < N; ++i) {
                double a = 0.0;
                for (int k = 0; k < K; ++k) a += W[i * K + k] * q[k];
                dy[i] = a;
                S += gamma[i] * v[i] * a;
            }
            for (int64_t i = 0; i < N; ++i) {
                const double dv = gamma[i] * dy[i] / rr - v[i] * S / ((double)N * rr * rr * rr);
                if (dX) dX[t * N + i] += dv;
                const double y = gamma[i] * v[i] / rr;
                for (int k = 0; k < K; ++k) pW[i * K + k] += y * q[k];
                pg[i] += v[i] * dy[i] / rr;
            }
            for (int k = 0; k < K; ++k) pb[k] += dz[t * K + k];
        }
        free(dy);
    }
    memset(dW, 0, sizeof(double) * (size_t)N * K);
    memset(db, 0, sizeof(double) * K);
    if (dgamma) memset(dgamma, 0, sizeof(double) * (size_t)N);
    for (int th = 0; th < nth; ++th) {
        const double* pW = part + (size_t)th * ((size_t)N * K + K + N);
        for (size_t a = 0; a < (size_t)N * K; ++a) dW[a] += pW[a];
        for (int k = 0; k < K; ++k) db[k] += pW[(size_t)N * K + k];
        if (dgamma)
            for (int64_t i = 0; i < N; ++i) dgamma[i] += pW[(size_t)N * K + K + i];
    }
    free(part);
}

/* Gradient of the per-group logit scales, alpha read as a learnable parameter: with
 * p_k = (v .* gamma) . W[:,k] the unscaled projection, z_k = alpha_g(k) p_k / r + b_k,
 * so dalpha_g = sum_t sum_{k in group g} dz_k p_k / r.  Recomputes r and p from X.
 * Per-thread partial sums over tokens, combined in thread order. */
void orc_alpha_bwd(int64_t T, int n, int64_t C, const double* X, const double* gamma,
                   double eps, const double* W, const double* dz, double* dalpha)
{
    const int64_t N = (int64_t)n * C;
    const int K = n * n + 2 * n;
    int nth = 1;
#ifdef _OPENMP
    nth = omp_get_max_threads();
#endif
    double* part = (double*)calloc((size_t)nth * 3, sizeof(double));
#pragma omp parallel
    {
        int tid = 0;
#ifdef _OPENMP
        tid = omp_get_thread_num();
#endif
#pragma omp for schedule(static)
        for (int64_t t = 0; t < T; ++t) {
            const double* v = X + t * N;
            double ss = 0.0;
            for (int64_t i = 0; i < N; ++i) ss += v[i] * v[i];
            const double rr = sqrt(ss / (double)N + eps);
            double p[ORC_MAXK];
            for (int k = 0; k < K; ++k) p[k] = 0.0;
            for (int64_t i = 0; i < N; ++i) {
                const double gv = gamma[i] * v[i];
                for (int k = 0; k < K; ++k) p[k] += gv * W[i * K + k];
            }
            for (int k = 0; k < K; ++k) part[tid * 3 + orc_group(k, n)] += dz[t * K + k] * p[k] / rr;
        }
    }
    dalpha[0] = dalpha[1] = dalpha[2] = 0.0;
    for (int th = 0; th < nth; ++th)
        for (int g = 0; g < 3; ++g) dalpha[g] += part[th * 3 + g];
    free(part);
}

/* Composite residual mapping over depth ([P1] "Warum Hyperverbindungen instabil
 * werden"; [P5] note [15]): P <- H_res P per token (later layers on the left), then
 * the forward gain max_i sum_j |P_ij| and the backward gain max_j sum_i |P_ij|. */
void orc_composite(int64_t T, int n, const double* Hres, double* P, double* gain_row,
                   double* gain_col)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        const double* H = Hres + t * n * n;
        double* Pt = P + t * n * n;
        double R[ORC_MAXN * ORC_MAXN];
        for (int i = 0; i < n; ++i)
            for (int j = 0; j < n; ++j) {
                double acc = 0.0;
                for (int m = 0; m < n; ++m) acc += H[i * n + m] * Pt[m * n + j];
                R[i * n + j] = acc;
            }
        memcpy(Pt, R, sizeof(double) * n * n);
        double gr = 0.0, gc = 0.0;
        for (int i = 0; i < n; ++i) {
            double s = 0.0;
            for (int j = 0; j < n; ++j) s += fabs(R[i * n + j]);
            if (s > gr) gr = s;
        }
        for (int j = 0; j < n; ++j) {
            double s = 0.0;
            for (int i = 0; i < n; ++i) s += fabs(R[i * n + j]);
            if (s > gc) gc = s;
        }
        if (gain_row) gain_row[t] = gr;
        if (gain_col) gain_col[t] = gc;
    }
}

int orc_max_n(void) { return ORC_MAXN; }
