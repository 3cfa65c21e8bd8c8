/* Host-only driver that runs every function of the fp64 oracle (oracle/mhc_oracle.c)
 * once on small seeded inputs, for n = 1, 2, 4, 8, with the optional outputs both
 * present and absent.  test_sanitizers_host.py compiles it together with the oracle
 * under AddressSanitizer and UndefinedBehaviorSanitizer: any out-of-bounds access,
 * leak or undefined operation aborts the run.  Prints a checksum so the calls are not
 * optimised away. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

void orc_coeffs(int64_t T, int n, int64_t C, const double* X, const double* gamma, double eps,
                const double* W, const double* bias, const double* alpha, double* z, double* r,
                double* Hpre, double* Hpost);
void orc_sinkhorn_one(int n, const double* zres, int iters, double* H, double* rho, double* kap,
                      double* Yrow, double* Ycol);
void orc_sinkhorn(int64_t T, int n, const double* zres, int64_t ld, int iters, double* Hres);
void orc_pre(int64_t T, int n, int64_t C, const double* X, const double* Hpre, double* u);
void orc_post_res(int64_t T, int n, int64_t C, const double* X, const double* F,
                  const double* Hres, const double* Hpost, double* Xout);
void orc_post_res_bwd(int64_t T, int n, int64_t C, const double* G, const double* X,
                      const double* F, const double* Hres, const double* Hpost, double* dF,
                      double* dHres, double* dHpost, double* dXdir);
void orc_pre_bwd(int64_t T, int n, int64_t C, const double* g, const double* X,
                 const double* Hpre, double* dHpre, double* dX);
void orc_sinkhorn_bwd_one(int n, const double* zres, int iters, const double* dH, double* dz);
void orc_sinkhorn_bwd(int64_t T, int n, const double* zres, int64_t ld, int iters,
                      const double* dHres, double* dzres);
void orc_gating_bwd(int64_t T, int n, const double* z, const double* dHpre, const double* dHpost,
                    double* dz);
void orc_coeffs_bwd(int64_t T, int n, int64_t C, const double* X, const double* gamma, double eps,
                    const double* W, const double* alpha, const double* dz, double* dX, double* dW,
                    double* db, double* dgamma);
void orc_alpha_bwd(int64_t T, int n, int64_t C, const double* X, const double* gamma, double eps,
                   const double* W, const double* dz, double* dalpha);
void orc_composite(int64_t T, int n, const double* Hres, double* P, double* gain_row,
                   double* gain_col);

static uint64_t state = 12345;
static double rnd(void)
{
    state = state * 6364136223846793005ULL + 1442695040888963407ULL;
    return (double)(state >> 11) / 9007199254740992.0 - 0.5;
}

/* exactly-sized heap arrays, so that any overrun lands outside the allocation */
static double* arr(size_t len)
{
    double* a = (double*)malloc(sizeof(double) * (len ? len : 1));
    for (size_t i = 0; i < len; ++i) a[i] = rnd();
    return a;
}

static double sum(const double* a, size_t len)
{
    double s = 0.0;
    for (size_t i = 0; i < len; ++i) s += a[i];
    return s;
}

int main(void)
{
    const int ns[4] = {1, 2, 4, 8};
    const int64_t T = 5, C = 24;
    const int iters = 7;
    double check = 0.0;
    for (int q = 0; q < 4; ++q) {
        const int n = ns[q], K = n * n + 2 * n, NN = n * n;
        const int64_t N = n * C;
        double *X = arr(T * N), *F = arr(T * C), *G = arr(T * N), *g = arr(T * C);
        double *gamma = arr(N), *W = arr(N * K), *bias = arr(K), *alpha = arr(3);
        double *z = arr(T * K), *r = arr(T), *Hpre = arr(T * n), *Hpost = arr(T * n);
        double *Hres = arr(T * NN), *u = arr(T * C), *Xo = arr(T * N);
        double *dF = arr(T * C), *dHres = arr(T * NN), *dHpost = arr(T * n), *dX = arr(T * N);
        double *dHpre = arr(T * n), *dz = arr(T * K), *dW = arr(N * K), *db = arr(K);
        double *dgamma = arr(N), *dalpha = arr(3), *P = arr(T * NN), *gr = arr(T), *gc = arr(T);
        double *H1 = arr(NN), *rho = arr(iters * n), *kap = arr(iters * n);
        double *Yr = arr(iters * NN), *Yc = arr(iters * NN), *dz1 = arr(NN);
        orc_coeffs(T, n, C, X, gamma, 1e-6, W, bias, alpha, z, r, Hpre, Hpost);
        orc_sinkhorn_one(n, z + 2 * n, iters, H1, rho, kap, Yr, Yc);
        orc_sinkhorn(T, n, z + 2 * n, K, iters, Hres);
        orc_pre(T, n, C, X, Hpre, u);
        orc_post_res(T, n, C, X, F, Hres, Hpost, Xo);
        orc_post_res_bwd(T, n, C, G, X, F, Hres, Hpost, dF, dHres, dHpost, dX);
        orc_post_res_bwd(T, n, C, G, X, F, Hres, Hpost, dF, dHres, dHpost, NULL);
        orc_pre_bwd(T, n, C, g, X, Hpre, dHpre, dX);
        orc_pre_bwd(T, n, C, g, X, Hpre, dHpre, NULL);
        orc_sinkhorn_bwd_one(n, z + 2 * n, iters, dHres, dz1);
        orc_gating_bwd(T, n, z, dHpre, dHpost, dz);
        orc_sinkhorn_bwd(T, n, z + 2 * n, K, iters, dHres, dz + 2 * n);
        orc_coeffs_bwd(T, n, C, X, gamma, 1e-6, W, alpha, dz, dX, dW, db, dgamma);
        orc_coeffs_bwd(T, n, C, X, gamma, 1e-6, W, alpha, dz, NULL, dW, db, NULL);
        orc_alpha_bwd(T, n, C, X, gamma, 1e-6, W, dz, dalpha);
        orc_composite(T, n, Hres, P, gr, gc);
        orc_composite(T, n, Hres, P, NULL, NULL);
        check += sum(u, T * C) + sum(Xo, T * N) + sum(dX, T * N) + sum(dW, N * K) + sum(dalpha, 3)
                 + sum(P, T * NN) + sum(H1, NN) + sum(dz1, NN);
        double* all[] = {X, F, G, g, gamma, W, bias, alpha, z, r, Hpre, Hpost, Hres, u, Xo, dF,
                         dHres, dHpost, dX, dHpre, dz, dW, db, dgamma, dalpha, P, gr, gc, H1, rho,
                         kap, Yr, Yc, dz1};
        for (size_t i = 0; i < sizeof(all) / sizeof(all[0]); ++i) free(all[i]);
    }
    printf("oracle sanitize run done, checksum %.6e\n", check);
    return 0;
}
