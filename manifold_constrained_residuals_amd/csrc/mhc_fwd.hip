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
// Per-token epilogue shared by the coefficient kernels: p = projection of v.gamma
// onto the K columns of W (not yet divided by r), sumsq = sum of v^2.
//   r = sqrt(sumsq / N + eps); z = alpha_g p / r + b; H_pre, H_post = sigmoid;
//   optional Sinkhorn-Knopp of the res logits (or of injected ones) into H_res.
template <int NS>
__device__ __forceinline__ void coeff_epilogue(int64_t t, const float (&p)[NS * NS + 2 * NS],
                                               float sumsq, int64_t N, float eps,
                                               const float* __restrict__ bias, float a0,
                                               float a1, float a2, float* __restrict__ z,
                                               float* __restrict__ rms, float* __restrict__ Hpre,
                                               float* __restrict__ Hpost, int iters,
                                               const float* __restrict__ zres_in,
                                               float* __restrict__ Hres)
{
    constexpr int K = NS * NS + 2 * NS;
    const float r = sqrtf(sumsq / (float)N + eps);
    const float rinv = 1.0f / r;
    float zz[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const float a = k < NS ? a0 : (k < 2 * NS ? a1 : a2);
        zz[k] = a * p[k] * rinv + bias[k];
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
        const float* s = tot + threadIdx.x * (K + 1);
        float p[K];
#pragma unroll
        for (int k = 0; k < K; ++k) p[k] = s[k];
        coeff_epilogue<NS>(t0 + threadIdx.x, p, s[K], N, eps, bias, a0, a1, a2, z, rms, Hpre,
                           Hpost, iters, zres_in, Hres);
    }
}


// ---------------------------------------------------------------- coefficients, MFMA path
// bf16 storage, n = 4 (K = 24).  The projection is a skinny GEMM [T x N] x [N x 24].
// X is exact as a bf16 MFMA operand; W' = gamma (.) W is split into bf16 hi + lo
// (about 16 significant bits together), giving 48 B-columns [hi 0..23 | lo 0..23]
// = three 16-wide MFMA tiles.  The split is written once per call, in MFMA
// fragment order, into the workspace:
//   Wp[s][nb][h][lane][j], s = 64-element step of the flattened axis, nb = column
//   tile, h = which 32-element MFMA of the step, lane = MFMA lane, j = 8 values;
//   element k = 64 s + 16 (lane / 16) + 8 h + j, column 16 nb + lane % 16.
// A lane therefore reads 32 contiguous bytes of one token row per step, and the
// A and B operands pair the same k.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWpStep = 3 * 2 * 64 * 8;   // bf16 values of Wp per 64-element step

__global__ __launch_bounds__(256) void k_wsplit(int64_t N, int64_t nsteps,
                                                const float* __restrict__ gamma,
                                                const float* __restrict__ W,
                                                bf16_t* __restrict__ Wp)
{
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= nsteps * 384) return;
    const int64_t s = idx / 384;
    const int r = (int)(idx - s * 384);
    const int nb = r >> 7, h = (r >> 6) & 1, lane = r & 63;
    const int col = nb * 16 + (lane & 15);
    const int kc = col < 24 ? col : col - 24;
    float o[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int64_t k = s * 64 + 16 * (lane >> 4) + 8 * h + j;
        const float v = k < N ? gamma[k] * W[k * 24 + kc] : 0.f;
        const float hi = (float)(__bf16)v;
        o[j] = col < 24 ? hi : (float)(__bf16)(v - hi);
    }
    io<bf16_t>::store8(Wp + idx * 8, o);
}

// Sum of squares of 8 bf16 values in fp32 (exact squares, fp32 adds).  The packed
// bf16 dot instruction is not used here: its accumulation is not fp32-accurate.
__device__ __forceinline__ float sumsq8(u32x4_t a, float acc) {
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float lo = bf16_lo(w[i]), hi = bf16_hi(w[i]);
        acc = fmaf(lo, lo, acc);
        acc = fmaf(hi, hi, acc);
    }
    return acc;
}

__device__ __forceinline__ f32x4_t mfma16(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// MT tokens per block of NW waves; the waves split the 64-element steps of the
// flattened axis round-robin, each keeping MT/16 x 3 accumulator tiles, with the
// next step's fragments loaded before the current step's MFMAs.  Partial tiles
// and sums of squares are combined through LDS; one thread per token runs the
// epilogue (scale by 1/r, bias, gates, Sinkhorn).
template <int MT, int NW>
__global__ __launch_bounds__(NW * 64) void k_coeffs_mfma(
    int64_t T, int64_t N, int64_t nsteps, const bf16_t* __restrict__ X,
    const bf16_t* __restrict__ Wp, float eps, const float* __restrict__ bias, float a0,
    float a1, float a2, float* __restrict__ z, float* __restrict__ rms,
    float* __restrict__ Hpre, float* __restrict__ Hpost, int iters,
    const float* __restrict__ zres_in, float* __restrict__ Hres)
{
    constexpr int MB = MT / 16;
    __shared__ float red[NW][MB][16][49];
    __shared__ float ssr[NW][MB][16];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int row = lane & 15, grp = lane >> 4;
    const int64_t t0 = (int64_t)blockIdx.x * MT;

    f32x4_t acc[MB][3];
    float ss[MB];
    const bf16_t* xp[MB];
    bool rv[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        ss[mb] = 0.f;
#pragma unroll
        for (int nb = 0; nb < 3; ++nb) acc[mb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        const int64_t t = t0 + mb * 16 + row;
        rv[mb] = t < T;
        xp[mb] = X + (rv[mb] ? t : t0) * N + 16 * grp;
    }

    u32x4_t wA[3][2], xA[MB][2], wB[3][2], xB[MB][2];
    auto load = [&](int64_t s, u32x4_t (&w)[3][2], u32x4_t (&x)[MB][2]) {
        const u32x4_t* wq = reinterpret_cast<const u32x4_t*>(Wp + s * kWpStep) + lane;
#pragma unroll
        for (int nb = 0; nb < 3; ++nb)
#pragma unroll
            for (int h = 0; h < 2; ++h) w[nb][h] = wq[(nb * 2 + h) * 64];
        const int64_t k0 = s * 64;
        const bool kin = k0 + 16 * grp < N;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            if (rv[mb] && kin) {
                const u32x4_t* q = reinterpret_cast<const u32x4_t*>(xp[mb] + k0);
                x[mb][0] = q[0];
                x[mb][1] = q[1];
            } else {
                x[mb][0] = u32x4_t{0u, 0u, 0u, 0u};
                x[mb][1] = u32x4_t{0u, 0u, 0u, 0u};
            }
        }
    };
    auto compute = [&](const u32x4_t (&w)[3][2], const u32x4_t (&x)[MB][2]) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            ss[mb] = sumsq8(x[mb][0], ss[mb]);
            ss[mb] = sumsq8(x[mb][1], ss[mb]);
#pragma unroll
            for (int nb = 0; nb < 3; ++nb) {
                acc[mb][nb] = mfma16(x[mb][0], w[nb][0], acc[mb][nb]);
                acc[mb][nb] = mfma16(x[mb][1], w[nb][1], acc[mb][nb]);
            }
        }
    };

    int64_t s = wv;
    if (s < nsteps) load(s, wA, xA);
    for (; s < nsteps; s += 2 * NW) {
        if (s + NW < nsteps) load(s + NW, wB, xB);
        compute(wA, xA);
        if (s + 2 * NW < nsteps) load(s + 2 * NW, wA, xA);
        if (s + NW < nsteps) compute(wB, xB);
    }

#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        ss[mb] += __shfl_xor(ss[mb], 16, 64);
        ss[mb] += __shfl_xor(ss[mb], 32, 64);
#pragma unroll
        for (int nb = 0; nb < 3; ++nb)
#pragma unroll
            for (int i = 0; i < 4; ++i) red[wv][mb][4 * grp + i][nb * 16 + row] = acc[mb][nb][i];
        if (grp == 0) ssr[wv][mb][row] = ss[mb];
    }
    __syncthreads();
    if (threadIdx.x < MT) {
        const int j = threadIdx.x, mb = j >> 4, rr = j & 15;
        const int64_t t = t0 + j;
        if (t < T) {
            float p[24];
#pragma unroll
            for (int k = 0; k < 24; ++k) {
                float a = 0.f;
#pragma unroll
                for (int w = 0; w < NW; ++w) a += red[w][mb][rr][k] + red[w][mb][rr][24 + k];
                p[k] = a;
            }
            float sq = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) sq += ssr[w][mb][rr];
            coeff_epilogue<4>(t, p, sq, N, eps, bias, a0, a1, a2, z, rms, Hpre, Hpost, iters,
                              zres_in, Hres);
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
// One block per token.  On the fused read side the block's first lane also runs
// the token's Sinkhorn-Knopp (res logits from z, or injected ones) while the
// other lanes stream u: the many resident blocks hide that lane's latency.
template <typename Tio, int NS>
__global__ __launch_bounds__(256) void k_pre(int64_t C, const Tio* __restrict__ X,
                                             const float* __restrict__ Hpre, Tio* __restrict__ u,
                                             const float* __restrict__ zres, int64_t ldz,
                                             int iters, float* __restrict__ Hres)
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
    if (Hres && threadIdx.x == 0) {
        float zr[NS * NS], M[NS * NS];
#pragma unroll
        for (int a = 0; a < NS * NS; ++a) zr[a] = zres[t * ldz + a];
        sinkhorn_fwd<NS>(zr, iters, M);
#pragma unroll
        for (int a = 0; a < NS * NS; ++a) Hres[t * (NS * NS) + a] = M[a];
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

static inline int64_t wsplit_steps(int64_t N) { return (N + 63) / 64; }

bool coeffs_use_mfma(int64_t, int n, int64_t, int dtype) { return dtype == MHC_BF16 && n == 4; }

size_t coeffs_workspace_bytes(int64_t T, int n, int64_t C, int dtype)
{
    if (!coeffs_use_mfma(T, n, C, dtype)) return 0;
    return align256(sizeof(bf16_t) * (size_t)wsplit_steps((int64_t)n * C) * kWpStep);
}

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
    if (coeffs_use_mfma(T, n, C, dtype)) {
        constexpr int MT = 32, NW = 8;
        const int64_t N = (int64_t)n * C, ns = wsplit_steps(N);
        bf16_t* Wp = static_cast<bf16_t*>(ws);
        hipLaunchKernelGGL(k_wsplit, dim3(blocks_for(ns * 384, 256)), dim3(256), 0, s, N, ns, gamma,
                           W, Wp);
        hipLaunchKernelGGL((k_coeffs_mfma<MT, NW>), dim3(blocks_for(T, MT)), dim3(NW * 64), 0, s, T,
                           N, ns, (const bf16_t*)X, (const bf16_t*)Wp, eps, bias, alpha[0], alpha[1],
                           alpha[2], z, rms, Hpre, Hpost, iters, zres_in, Hres);
        return hipGetLastError();
    }
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
                      void* u, const float* zres, int64_t ldz, int iters, float* Hres,
                      hipStream_t s)
{
    const dim3 g((unsigned)T), b(256);
#define MHC_PRE_ARGS Hpre, zres, ldz, iters, Hres
    if (dtype == MHC_BF16) {
        if (n == 4) hipLaunchKernelGGL((k_pre<bf16_t, 4>), g, b, 0, s, C, (const bf16_t*)X, Hpre, (bf16_t*)u, zres, ldz, iters, Hres);
        else        hipLaunchKernelGGL((k_pre<bf16_t, 1>), g, b, 0, s, C, (const bf16_t*)X, Hpre, (bf16_t*)u, zres, ldz, iters, Hres);
    } else {
        if (n == 4) hipLaunchKernelGGL((k_pre<float, 4>), g, b, 0, s, C, (const float*)X, Hpre, (float*)u, zres, ldz, iters, Hres);
        else        hipLaunchKernelGGL((k_pre<float, 1>), g, b, 0, s, C, (const float*)X, Hpre, (float*)u, zres, ldz, iters, Hres);
    }
#undef MHC_PRE_ARGS
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
