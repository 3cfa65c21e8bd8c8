// mhc_fwd.hip -- forward kernels of the mHC layer for gfx950.
//
//   coefficients: r = rms(vec X), z = alpha_g (X.gamma) W / r + b, sigmoid gates,
//                 optional Sinkhorn epilogue (fused read side)
//   Sinkhorn:     one token per lane, 4x4 block in registers
//   pre:          u = H_pre X           (streaming, 16-byte rows)
//   post_res:     X' = H_res X + H_post^T F  (streaming)
//   composite:    P <- H_res P and its row/column gains
//
// The update rule and the maps follow chatgpz.de, "Von Residualverbindungen zu
// Hyperverbindungen"; the constraint and Sinkhorn-Knopp follow "Vielfaeltig
// eingeschraenkte Hyperverbindungen" on the same page and staging.reportify.cn,
// "mHC方法原理" notes [10], [16].
#include "mhc_device.hpp"
#include "mhc_internal.hpp"
#include "../../include/mhc.h"

namespace mhc {

// ---------------------------------------------------------------- coefficients
// Generic path (any dtype, n in {1,4}): TB tokens per 256-thread block; every
// thread walks the flattened n*C axis with stride 256, folds gamma into its W row
// and accumulates K dot products plus the sum of squares per token.  The
// projection is divided by r after the block reduction (RMSNorm reordered).
template <typename Tio, int NS, int TB>
__global__ __launch_bounds__(256) void k_coeffs_generic(
    int64_t T, int64_t C, const Tio* __restrict__ X, const float* __restrict__ gamma,
    float eps, const float* __restrict__ W, const float* __restrict__ bias, float a0,
    float a1, float a2, float* __restrict__ z, float* __restrict__ rms,
    float* __restrict__ Hpre, float* __restrict__ Hpost, int iters,
    const float* __restrict__ zres_in, float* __restrict__ Hres)
{
    constexpr int K = NS * NS + 2 * NS;
    constexpr int NV = TB * (K + 1);
    __shared__ float scratch[4 * NV];
    __shared__ float tot[NV];
    const int64_t N = NS * C;
    const int64_t t0 = (int64_t)blockIdx.x * TB;
    int nt = (int)((T - t0) < TB ? (T - t0) : TB);

    float acc[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) acc[j] = 0.f;

    for (int64_t e = threadIdx.x; e < N; e += 256) {
        const float g = gamma[e];
        float w[K];
#pragma unroll
        for (int k = 0; k < K; ++k) w[k] = g * W[e * K + k];
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
            if (tb < nt) {
                const float x = io<Tio>::load1(X + (t0 + tb) * N + e);
                acc[tb * (K + 1) + K] += x * x;
#pragma unroll
                for (int k = 0; k < K; ++k) acc[tb * (K + 1) + k] += x * w[k];
            }
        }
    }
    block_sum_256<NV>(acc, scratch, tot);

    if ((int)threadIdx.x < nt) {
        const int64_t t = t0 + threadIdx.x;
        const float* s = tot + threadIdx.x * (K + 1);
        const float r = sqrtf(s[K] / (float)N + eps);
        const float rinv = 1.0f / r;
        float zz[K];
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const float a = k < NS ? a0 : (k < 2 * NS ? a1 : a2);
            zz[k] = a * s[k] * rinv + bias[k];
            z[t * K + k] = zz[k];
        }
        if (rms) rms[t] = r;
#pragma unroll
        for (int k = 0; k < NS; ++k) {
            if (Hpre) Hpre[t * NS + k] = sigmoidf(zz[k]);
            if (Hpost) Hpost[t * NS + k] = sigmoidf(zz[NS + k]);
        }
        if (Hres) {
            float zr[NS * NS], M[NS * NS];
#pragma unroll
            for (int a = 0; a < NS * NS; ++a)
                zr[a] = zres_in ? zres_in[t * (NS * NS) + a] : zz[2 * NS + a];
            sinkhorn_fwd<NS>(zr, iters, M);
#pragma unroll
            for (int a = 0; a < NS * NS; ++a) Hres[t * (NS * NS) + a] = M[a];
        }
    }
}

// ---------------------------------------------------------------- Sinkhorn
template <int NS>
__global__ __launch_bounds__(256) void k_sinkhorn(int64_t T, const float* __restrict__ zres,
                                                  int64_t ld, int iters, float* __restrict__ Hres)
{
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= T) return;
    float zr[NS * NS], M[NS * NS];
#pragma unroll
    for (int a = 0; a < NS * NS; ++a) zr[a] = zres[t * ld + a];
    sinkhorn_fwd<NS>(zr, iters, M);
#pragma unroll
    for (int a = 0; a < NS * NS; ++a) Hres[t * (NS * NS) + a] = M[a];
}

// ---------------------------------------------------------------- pre: u = H_pre X
template <typename Tio, int NS>
__global__ __launch_bounds__(256) void k_pre(int64_t C, const Tio* __restrict__ X,
                                             const float* __restrict__ Hpre, Tio* __restrict__ u)
{
    const int64_t t = blockIdx.x;
    float h[NS];
#pragma unroll
    for (int k = 0; k < NS; ++k) h[k] = Hpre[t * NS + k];
    const Tio* xt = X + t * NS * C;
    for (int64_t c = (int64_t)threadIdx.x * 8; c < C; c += 256 * 8) {
        float acc[8], v[8];
        io<Tio>::load8(xt + c, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = h[0] * v[e];
#pragma unroll
        for (int k = 1; k < NS; ++k) {
            io<Tio>::load8(xt + k * C + c, v);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += h[k] * v[e];
        }
        io<Tio>::store8(u + t * C + c, acc);
    }
}

// ---------------------------------------------------------------- post + residual
template <typename Tio, int NS>
__global__ __launch_bounds__(256) void k_post_res(int64_t C, const Tio* __restrict__ X,
                                                  const Tio* __restrict__ F,
                                                  const float* __restrict__ Hres,
                                                  const float* __restrict__ Hpost,
                                                  Tio* __restrict__ Xout)
{
    const int64_t t = blockIdx.x;
    float hr[NS * NS], hp[NS];
#pragma unroll
    for (int a = 0; a < NS * NS; ++a) hr[a] = Hres[t * NS * NS + a];
#pragma unroll
    for (int k = 0; k < NS; ++k) hp[k] = Hpost[t * NS + k];
    const Tio* xt = X + t * NS * C;
    Tio* ot = Xout + t * NS * C;
    for (int64_t c = (int64_t)threadIdx.x * 8; c < C; c += 256 * 8) {
        float xv[NS][8], fv[8];
#pragma unroll
        for (int j = 0; j < NS; ++j) io<Tio>::load8(xt + j * C + c, xv[j]);
        io<Tio>::load8(F + t * C + c, fv);
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            float o[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float a = hp[i] * fv[e];
#pragma unroll
                for (int j = 0; j < NS; ++j) a += hr[i * NS + j] * xv[j][e];
                o[e] = a;
            }
            io<Tio>::store8(ot + i * C + c, o);
        }
    }
}

// ---------------------------------------------------------------- composite
template <int NS>
__global__ __launch_bounds__(256) void k_composite(int64_t T, const float* __restrict__ Hres,
                                                   float* __restrict__ P, float* __restrict__ gr,
                                                   float* __restrict__ gc)
{
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= T) return;
    float H[NS * NS], Q[NS * NS], R[NS * NS];
#pragma unroll
    for (int a = 0; a < NS * NS; ++a) { H[a] = Hres[t * NS * NS + a]; Q[a] = P[t * NS * NS + a]; }
#pragma unroll
    for (int i = 0; i < NS; ++i)
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            float acc = 0.f;
#pragma unroll
            for (int m = 0; m < NS; ++m) acc += H[i * NS + m] * Q[m * NS + j];
            R[i * NS + j] = acc;
        }
    float row = 0.f, col = 0.f;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        float s = 0.f, s2 = 0.f;
#pragma unroll
        for (int j = 0; j < NS; ++j) { s += fabsf(R[i * NS + j]); s2 += fabsf(R[j * NS + i]); }
        row = fmaxf(row, s); col = fmaxf(col, s2);
    }
#pragma unroll
    for (int a = 0; a < NS * NS; ++a) P[t * NS * NS + a] = R[a];
    if (gr) gr[t] = row;
    if (gc) gc[t] = col;
}

// ================================================================ launchers
static inline unsigned blocks_for(int64_t n, int per) { return (unsigned)((n + per - 1) / per); }

size_t coeffs_workspace_bytes(int64_t, int, int64_t, int) { return 0; }
bool coeffs_use_mfma(int64_t, int, int64_t, int) { return false; }

template <typename Tio, int NS>
static void coeffs_generic_launch(int64_t T, int64_t C, const void* X, const float* gamma,
                                  float eps, const float* W, const float* bias,
                                  const float* alpha, float* z, float* rms, float* Hpre,
                                  float* Hpost, int iters, const float* zres_in, float* Hres,
                                  hipStream_t s)
{
    constexpr int TB = 4;
    hipLaunchKernelGGL((k_coeffs_generic<Tio, NS, TB>), dim3(blocks_for(T, TB)), dim3(256), 0, s,
                       T, C, (const Tio*)X, gamma, eps, W, bias, alpha[0], alpha[1], alpha[2], z,
                       rms, Hpre, Hpost, iters, zres_in, Hres);
}

hipError_t launch_coeffs(int64_t T, int n, int64_t C, int dtype, const void* X,
                         const float* gamma, float eps, const float* W, const float* bias,
                         const float* alpha, float* z, float* rms, float* Hpre, float* Hpost,
                         int iters, const float* zres_in, float* Hres, void* ws, hipStream_t s)
{
    (void)ws;
    if (dtype == MHC_BF16) {
        if (n == 4) coeffs_generic_launch<bf16_t, 4>(T, C, X, gamma, eps, W, bias, alpha, z, rms, Hpre, Hpost, iters, zres_in, Hres, s);
        else        coeffs_generic_launch<bf16_t, 1>(T, C, X, gamma, eps, W, bias, alpha, z, rms, Hpre, Hpost, iters, zres_in, Hres, s);
    } else {
        if (n == 4) coeffs_generic_launch<float, 4>(T, C, X, gamma, eps, W, bias, alpha, z, rms, Hpre, Hpost, iters, zres_in, Hres, s);
        else        coeffs_generic_launch<float, 1>(T, C, X, gamma, eps, W, bias, alpha, z, rms, Hpre, Hpost, iters, zres_in, Hres, s);
    }
    return hipGetLastError();
}

hipError_t launch_sinkhorn(int64_t T, int n, const float* zres, int64_t ld, int iters,
                           float* Hres, hipStream_t s)
{
    if (n == 4)
        hipLaunchKernelGGL((k_sinkhorn<4>), dim3(blocks_for(T, 256)), dim3(256), 0, s, T, zres, ld, iters, Hres);
    else
        hipLaunchKernelGGL((k_sinkhorn<1>), dim3(blocks_for(T, 256)), dim3(256), 0, s, T, zres, ld, iters, Hres);
    return hipGetLastError();
}

hipError_t launch_pre(int64_t T, int n, int64_t C, int dtype, const void* X, const float* Hpre,
                      void* u, hipStream_t s)
{
    const dim3 g((unsigned)T), b(256);
    if (dtype == MHC_BF16) {
        if (n == 4) hipLaunchKernelGGL((k_pre<bf16_t, 4>), g, b, 0, s, C, (const bf16_t*)X, Hpre, (bf16_t*)u);
        else        hipLaunchKernelGGL((k_pre<bf16_t, 1>), g, b, 0, s, C, (const bf16_t*)X, Hpre, (bf16_t*)u);
    } else {
        if (n == 4) hipLaunchKernelGGL((k_pre<float, 4>), g, b, 0, s, C, (const float*)X, Hpre, (float*)u);
        else        hipLaunchKernelGGL((k_pre<float, 1>), g, b, 0, s, C, (const float*)X, Hpre, (float*)u);
    }
    return hipGetLastError();
}

hipError_t launch_post_res(int64_t T, int n, int64_t C, int dtype, const void* X, const void* F,
                           const float* Hres, const float* Hpost, void* Xout, hipStream_t s)
{
    const dim3 g((unsigned)T), b(256);
    if (dtype == MHC_BF16) {
        if (n == 4) hipLaunchKernelGGL((k_post_res<bf16_t, 4>), g, b, 0, s, C, (const bf16_t*)X, (const bf16_t*)F, Hres, Hpost, (bf16_t*)Xout);
        else        hipLaunchKernelGGL((k_post_res<bf16_t, 1>), g, b, 0, s, C, (const bf16_t*)X, (const bf16_t*)F, Hres, Hpost, (bf16_t*)Xout);
    } else {
        if (n == 4) hipLaunchKernelGGL((k_post_res<float, 4>), g, b, 0, s, C, (const float*)X, (const float*)F, Hres, Hpost, (float*)Xout);
        else        hipLaunchKernelGGL((k_post_res<float, 1>), g, b, 0, s, C, (const float*)X, (const float*)F, Hres, Hpost, (float*)Xout);
    }
    return hipGetLastError();
}

hipError_t launch_composite(int64_t T, int n, const float* Hres, float* P, float* gr, float* gc,
                            hipStream_t s)
{
    if (n == 4)
        hipLaunchKernelGGL((k_composite<4>), dim3(blocks_for(T, 256)), dim3(256), 0, s, T, Hres, P, gr, gc);
    else
        hipLaunchKernelGGL((k_composite<1>), dim3(blocks_for(T, 256)), dim3(256), 0, s, T, Hres, P, gr, gc);
    return hipGetLastError();
}

}  // namespace mhc
