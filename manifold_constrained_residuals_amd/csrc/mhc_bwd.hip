// mhc_bwd.hip -- backward kernels of the mHC layer for gfx950.
//
//   post_res_bwd:  dF, dH_post, dH_res (+ optional H_res^T G, + optional dH_pre) per token
//   pre_bwd:       dH_pre (+ optional dX += H_pre^T du) per token
//   sinkhorn_bwd:  recompute the iterations, differentiate them in reverse
//   logit grads:   gating backward (+ Sinkhorn backward), per-token record
//   coeffs_bwd:    dX through RMSNorm + projection, dW / dgamma partials over
//                  token ranges, then a fixed-order reduction (deterministic)
//
// The Sinkhorn iterations get their own backward and are recomputed instead of
// stored (staging.reportify.cn, "高效基础设施设计" notes [19], [21]).
#include "mhc_device.hpp"
#include "mhc_internal.hpp"
#include "../../include/mhc.h"

namespace mhc {

// ---------------------------------------------------------------- post_res backward
constexpr int kPrbU = 2;   // row pieces in flight per thread in k_post_res_bwd
constexpr int kPbU = 2;    // and in k_pre_bwd

// With DU, the pass also forms the read map's gradient dH_pre[t][k] = <du[t], X[t][k]>
// from the X rows it already streams (the pre backward's reduction, bitwise: the same
// per-thread order and its own block sum), so the backward reads X once less.
template <typename Tio, int NS, bool DU>
__global__ __launch_bounds__(256) void k_post_res_bwd(
    int64_t C, const Tio* __restrict__ G, const Tio* __restrict__ X, const Tio* __restrict__ F,
    const float* __restrict__ Hres, const float* __restrict__ Hpost, const Tio* __restrict__ du,
    float* __restrict__ dF, float* __restrict__ dHres, float* __restrict__ dHpost,
    float* __restrict__ dHpre, float* __restrict__ dX)
{
    constexpr int NV = NS + NS * NS;
    constexpr int U = NS <= 4 ? kPrbU : 1;     // n = 8 holds one piece (registers)
    __shared__ float scratch[4 * NV];
    __shared__ float tot[NV];
    __shared__ float totp[NS];
    const int64_t t = blockIdx.x;
    float hr[NS * NS], hp[NS];
#pragma unroll
    for (int a = 0; a < NS * NS; ++a) hr[a] = Hres[t * NS * NS + a];
#pragma unroll
    for (int k = 0; k < NS; ++k) hp[k] = Hpost[t * NS + k];
    float acc[NV], accp[NS];
#pragma unroll
    for (int j = 0; j < NV; ++j) acc[j] = 0.f;
#pragma unroll
    for (int k = 0; k < NS; ++k) accp[k] = 0.f;
    const Tio* gt = G + t * NS * C;
    const Tio* xt = X + t * NS * C;
    // U row pieces per thread are loaded before any is used
    for (int64_t c0 = (int64_t)threadIdx.x * 8; c0 < C; c0 += U * 256 * 8) {
        float gv[U][NS][8], xv[U][NS][8], fv[U][8], dv[U][DU ? 8 : 1];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t c = c0 + (int64_t)u * 256 * 8;
            if (u == 0 || c < C) {
#pragma unroll
                for (int i = 0; i < NS; ++i) io<Tio>::load8(gt + i * C + c, gv[u][i]);
#pragma unroll
                for (int i = 0; i < NS; ++i) io<Tio>::load8(xt + i * C + c, xv[u][i]);
                io<Tio>::load8(F + t * C + c, fv[u]);
                if constexpr (DU) io<Tio>::load8(du + t * C + c, dv[u]);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t c = c0 + (int64_t)u * 256 * 8;
            if (u > 0 && c >= C) break;
            float df[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float a = 0.f;
#pragma unroll
                for (int i = 0; i < NS; ++i) a += hp[i] * gv[u][i][e];
                df[e] = a;
            }
            store8_nt(dF + t * C + c, df);
            if constexpr (DU) {
#pragma unroll
                for (int k = 0; k < NS; ++k) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) accp[k] += dv[u][e] * xv[u][k][e];
                }
            }
#pragma unroll
            for (int i = 0; i < NS; ++i) {
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[i] += gv[u][i][e] * fv[u][e];
#pragma unroll
                for (int j = 0; j < NS; ++j)
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[NS + i * NS + j] += gv[u][i][e] * xv[u][j][e];
            }
            if (dX) {
#pragma unroll
                for (int j = 0; j < NS; ++j) {
                    float o[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        float a = 0.f;
#pragma unroll
                        for (int i = 0; i < NS; ++i) a += hr[i * NS + j] * gv[u][i][e];
                        o[e] = a;
                    }
                    store8_f32(dX + (t * NS + j) * C + c, o);
                }
            }
        }
    }
    block_sum_256<NV>(acc, scratch, tot);
    if (threadIdx.x < NS) dHpost[t * NS + threadIdx.x] = tot[threadIdx.x];
    else if (threadIdx.x < NV) dHres[t * NS * NS + threadIdx.x - NS] = tot[threadIdx.x];
    if constexpr (DU) {
        block_sum_256<NS>(accp, scratch, totp);
        if (threadIdx.x < NS) dHpre[t * NS + threadIdx.x] = totp[threadIdx.x];
    }
}

// ---------------------------------------------------------------- pre backward
template <typename Tio, int NS>
__device__ __forceinline__ void pre_bwd_token(int64_t t, int64_t C, const Tio* __restrict__ g,
                                              const Tio* __restrict__ X,
                                              const float* __restrict__ Hpre,
                                              float* __restrict__ dHpre, float* __restrict__ dX,
                                              float* scratch, float* tot)
{
    float hp[NS], acc[NS];
#pragma unroll
    for (int k = 0; k < NS; ++k) { hp[k] = Hpre[t * NS + k]; acc[k] = 0.f; }
    const Tio* xt = X + t * NS * C;
    // kPbU row pieces per thread are loaded before any is used
    for (int64_t c0 = (int64_t)threadIdx.x * 8; c0 < C; c0 += kPbU * 256 * 8) {
        float gv[kPbU][8], xv[kPbU][NS][8];
#pragma unroll
        for (int u = 0; u < kPbU; ++u) {
            const int64_t c = c0 + (int64_t)u * 256 * 8;
            if (u == 0 || c < C) {
                io<Tio>::load8(g + t * C + c, gv[u]);
#pragma unroll
                for (int k = 0; k < NS; ++k) io<Tio>::load8(xt + k * C + c, xv[u][k]);
            }
        }
#pragma unroll
        for (int u = 0; u < kPbU; ++u) {
            const int64_t c = c0 + (int64_t)u * 256 * 8;
            if (u > 0 && c >= C) break;
#pragma unroll
            for (int k = 0; k < NS; ++k) {
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[k] += gv[u][e] * xv[u][k][e];
            }
            if (dX) {
#pragma unroll
                for (int k = 0; k < NS; ++k) {
                    float d[8];
                    io<float>::load8(dX + (t * NS + k) * C + c, d);
#pragma unroll
                    for (int e = 0; e < 8; ++e) d[e] += hp[k] * gv[u][e];
                    store8_f32(dX + (t * NS + k) * C + c, d);
                }
            }
        }
    }
    block_sum_256<NS>(acc, scratch, tot);
    if (threadIdx.x < NS) dHpre[t * NS + threadIdx.x] = tot[threadIdx.x];
}

template <typename Tio, int NS>
__global__ __launch_bounds__(256) void k_pre_bwd(int64_t C, const Tio* __restrict__ g,
                                                 const Tio* __restrict__ X,
                                                 const float* __restrict__ Hpre,
                                                 float* __restrict__ dHpre, float* __restrict__ dX)
{
    __shared__ float scratch[4 * NS];
    __shared__ float tot[NS];
    pre_bwd_token<Tio, NS>(blockIdx.x, C, g, X, Hpre, dHpre, dX, scratch, tot);
}

// ---------------------------------------------------------------- Sinkhorn backward
// One token per lane.  Forward iterates after each row step are kept in LDS
// (layout [iteration][entry][lane], 64 lanes per block) when iters <= 20;
// otherwise each reverse step recomputes the forward up to that point.
// Reverse of iteration s, with R = matrix after its row step, Yc = R / colsum(R),
// P = matrix before the row step (exp of the shifted logits at s = 0):
//   column step: dR_ij = (dYc_ij - sum_m dYc_mj Yc_mj) / colsum_j(R)
//   row step:    dP_ij = (dR_ij - sum_m dR_im R_im) / rowsum_i(P)
template <int NS>
__device__ __forceinline__ void sk_exp0(const float (&zr)[NS * NS], float (&M0)[NS * NS]) {
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        float m = zr[i * NS];
#pragma unroll
        for (int j = 1; j < NS; ++j) m = fmaxf(m, zr[i * NS + j]);
#pragma unroll
        for (int j = 0; j < NS; ++j) M0[i * NS + j] = expf(zr[i * NS + j] - m);
    }
}

template <int NS>
__device__ __forceinline__ void sk_rowstep(float (&M)[NS * NS]) {
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        float rs = 0.f;
#pragma unroll
        for (int j = 0; j < NS; ++j) rs += M[i * NS + j];
        const float inv = 1.0f / rs;
#pragma unroll
        for (int j = 0; j < NS; ++j) M[i * NS + j] *= inv;
    }
}

template <int NS>
__device__ __forceinline__ void sk_colstep(float (&M)[NS * NS]) {
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        float cs = 0.f;
#pragma unroll
        for (int i = 0; i < NS; ++i) cs += M[i * NS + j];
        const float inv = 1.0f / cs;
#pragma unroll
        for (int i = 0; i < NS; ++i) M[i * NS + j] *= inv;
    }
}

// one reverse iteration: Gb holds dL/d(matrix after the column step) on entry and
// dL/d(matrix before the row step) on exit
template <int NS>
__device__ __forceinline__ void sk_reverse_step(float (&Gb)[NS * NS], const float (&R)[NS * NS],
                                                const float (&P)[NS * NS]) {
    float Yc[NS * NS], kinv[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        float cs = 0.f;
#pragma unroll
        for (int i = 0; i < NS; ++i) cs += R[i * NS + j];
        kinv[j] = 1.0f / cs;
#pragma unroll
        for (int i = 0; i < NS; ++i) Yc[i * NS + j] = R[i * NS + j] * kinv[j];
    }
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        float a = 0.f;
#pragma unroll
        for (int m = 0; m < NS; ++m) a += Gb[m * NS + j] * Yc[m * NS + j];
#pragma unroll
        for (int i = 0; i < NS; ++i) Gb[i * NS + j] = (Gb[i * NS + j] - a) * kinv[j];
    }
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        float rs = 0.f, b = 0.f;
#pragma unroll
        for (int j = 0; j < NS; ++j) { rs += P[i * NS + j]; b += Gb[i * NS + j] * R[i * NS + j]; }
        const float rinv = 1.0f / rs;
#pragma unroll
        for (int j = 0; j < NS; ++j) Gb[i * NS + j] = (Gb[i * NS + j] - b) * rinv;
    }
}

// Iterates are kept in LDS for NS <= 4 (kMaxStoredIters * NS * NS * 64 floats per
// 64-lane block); larger blocks take the recompute path.
template <int NS>
constexpr int sk_lds_floats() { return NS <= 4 ? kMaxStoredIters * NS * NS * 64 : 1; }

// lds: this lane's base, consecutive floats 64 apart (size sk_lds_floats<NS>())
template <int NS>
__device__ __forceinline__ void sinkhorn_bwd_token(const float (&zr)[NS * NS], int iters,
                                                   const float (&dH)[NS * NS],
                                                   float (&dz)[NS * NS], float* lds)
{
    float M0[NS * NS], Gb[NS * NS];
    sk_exp0<NS>(zr, M0);
#pragma unroll
    for (int a = 0; a < NS * NS; ++a) Gb[a] = dH[a];
    if (NS <= 4 && iters <= kMaxStoredIters) {
        float M[NS * NS];
#pragma unroll
        for (int a = 0; a < NS * NS; ++a) M[a] = M0[a];
        for (int s = 0; s < iters; ++s) {
            sk_rowstep<NS>(M);
#pragma unroll
            for (int a = 0; a < NS * NS; ++a) lds[(s * NS * NS + a) * 64] = M[a];
            sk_colstep<NS>(M);
        }
        for (int s = iters - 1; s >= 0; --s) {
            float R[NS * NS], P[NS * NS];
#pragma unroll
            for (int a = 0; a < NS * NS; ++a) R[a] = lds[(s * NS * NS + a) * 64];
            if (s > 0) {
#pragma unroll
                for (int a = 0; a < NS * NS; ++a) P[a] = lds[((s - 1) * NS * NS + a) * 64];
                sk_colstep<NS>(P);
            } else {
#pragma unroll
                for (int a = 0; a < NS * NS; ++a) P[a] = M0[a];
            }
            sk_reverse_step<NS>(Gb, R, P);
        }
    } else {
        for (int s = iters - 1; s >= 0; --s) {
            float P[NS * NS];
#pragma unroll
            for (int a = 0; a < NS * NS; ++a) P[a] = M0[a];
            for (int q = 0; q < s; ++q) { sk_rowstep<NS>(P); sk_colstep<NS>(P); }
            float R[NS * NS];
#pragma unroll
            for (int a = 0; a < NS * NS; ++a) R[a] = P[a];
            sk_rowstep<NS>(R);
            sk_reverse_step<NS>(Gb, R, P);
        }
    }
#pragma unroll
    for (int a = 0; a < NS * NS; ++a) dz[a] = Gb[a] * M0[a];
}

// n = 4: one token per 16 lanes (entry (i, j) in lane 4 i + j), the same reverse
// steps with the row and column sums taken across lanes.  Each thread keeps its
// entry's post-row-step iterates in its own LDS column; tokens past T run on zeros
// so that every lane of a group takes part in the exchanges.
__device__ __forceinline__ float sk16_reverse_step(float gb, float r, float p) {
    const float kinv = sk16_rcp(sk16_colsum(r));
    const float a = sk16_colsum(gb * (r * kinv));
    gb = (gb - a) * kinv;
    const float rinv = sk16_rcp(sk16_rowsum(p));
    const float b = sk16_rowsum(gb * r);
    return (gb - b) * rinv;
}

// Sinkhorn backward of one token on 16 lanes (lane q holds entry q of the 4 x 4
// block).  For iters <= 20 the forward iterates after each row step are recomputed
// into registers (uniform branches keep the row's lanes together), then reversed;
// beyond that each reverse step recomputes the forward up to that point.
__device__ __forceinline__ float sk16_bwd_token(float z, float dh, int iters)
{
    const float m0 = sk16_exp0(z);
    float gb = dh;
    if (iters <= kMaxStoredIters) {
        float rs[kMaxStoredIters];
        float m = m0;
#pragma unroll
        for (int s = 0; s < kMaxStoredIters; ++s) {
            if (s < iters) {
                m = sk16_rowstep(m);
                rs[s] = m;
                m = sk16_colstep(m);
            }
        }
#pragma unroll
        for (int s = kMaxStoredIters - 1; s >= 0; --s) {
            if (s < iters) {
                const float p = s > 0 ? sk16_colstep(rs[s > 0 ? s - 1 : 0]) : m0;
                gb = sk16_reverse_step(gb, rs[s], p);
            }
        }
    } else {
        for (int s = iters - 1; s >= 0; --s) {
            float p = m0;
            for (int u = 0; u < s; ++u) p = sk16_colstep(sk16_rowstep(p));
            gb = sk16_reverse_step(gb, sk16_rowstep(p), p);
        }
    }
    return gb * m0;
}

// 16 tokens per block of 256 threads (token blk * 16 + tid / 16); tokens past T run on
// zeros so that every lane of a DPP row takes part.
__device__ __forceinline__ void sk16_bwd_block(int64_t blk, int64_t T, const float* __restrict__ zres,
                                               int64_t ldz, int iters, const float* __restrict__ dHres,
                                               float* __restrict__ dzres, int64_t lddz)
{
    const int64_t t = blk * 16 + (threadIdx.x >> 4);
    const int q = threadIdx.x & 15;
    const bool valid = t < T;
    const float r = sk16_bwd_token(valid ? zres[t * ldz + q] : 0.f, valid ? dHres[t * 16 + q] : 0.f,
                                   iters);
    if (valid) dzres[t * lddz + q] = r;
}

__global__ __launch_bounds__(256) void k_sinkhorn_bwd16(int64_t T, const float* __restrict__ zres,
                                                        int64_t ldz, int iters,
                                                        const float* __restrict__ dHres,
                                                        float* __restrict__ dzres, int64_t lddz)
{
    sk16_bwd_block(blockIdx.x, T, zres, ldz, iters, dHres, dzres, lddz);
}

// One launch for two independent parts of the backward read side at n = 4: blocks
// [0, nsk) run the Sinkhorn backward (16 tokens each, VALU-bound), blocks nsk + t the
// pre backward of token t (HBM-bound); the GPU runs the two kinds side by side.
template <typename Tio>
__global__ __launch_bounds__(256) void k_pre_bwd_sk16(
    int64_t T, int64_t C, int64_t nsk, const Tio* __restrict__ g, const Tio* __restrict__ X,
    const float* __restrict__ Hpre, float* __restrict__ dHpre, const float* __restrict__ zres,
    int64_t ldz, int iters, const float* __restrict__ dHres, float* __restrict__ dzres,
    int64_t lddz)
{
    __shared__ float scratch[4 * 4];
    __shared__ float tot[4];
    if ((int64_t)blockIdx.x < nsk)
        sk16_bwd_block(blockIdx.x, T, zres, ldz, iters, dHres, dzres, lddz);
    else
        pre_bwd_token<Tio, 4>((int64_t)blockIdx.x - nsk, C, g, X, Hpre, dHpre, nullptr, scratch, tot);
}

template <int NS>
__global__ __launch_bounds__(64) void k_sinkhorn_bwd(int64_t T, const float* __restrict__ zres,
                                                     int64_t ldz, int iters,
                                                     const float* __restrict__ dHres,
                                                     float* __restrict__ dzres, int64_t lddz)
{
    __shared__ float lds[sk_lds_floats<NS>()];
    const int64_t t = (int64_t)blockIdx.x * 64 + threadIdx.x;
    if (t >= T) return;
    float zr[NS * NS], dH[NS * NS], dz[NS * NS];
#pragma unroll
    for (int a = 0; a < NS * NS; ++a) { zr[a] = zres[t * ldz + a]; dH[a] = dHres[t * NS * NS + a]; }
    sinkhorn_bwd_token<NS>(zr, iters, dH, dz, lds + threadIdx.x);
#pragma unroll
    for (int a = 0; a < NS * NS; ++a) dzres[t * lddz + a] = dz[a];
}

// ---------------------------------------------------------------- logit gradients
// One token per lane (n other than 4): gating backward (dz = dH s (1 - s) with s the
// forward's gate), the res-logit gradient (given, or recomputed through Sinkhorn), then
// the per-token record used by the coefficient backward.

// One token's logit gradients from the gates' gradients and the res-logit gradient
// dr: dz (also to dz_out) and the per-token record.  dz stays zero past T.
template <int NS>
__device__ __forceinline__ void dz_token(int64_t t, bool valid, int64_t N, const float* __restrict__ z,
                                         const float* __restrict__ bias, const float* __restrict__ rms,
                                         const float* __restrict__ Hpre, const float* __restrict__ Hpost,
                                         const float* __restrict__ dHpre, const float* __restrict__ dHpost,
                                         const float (&dr)[NS * NS], float a0, float a1, float a2,
                                         float* __restrict__ dz_out, float* __restrict__ rec,
                                         float (&dz)[NS * NS + 2 * NS])
{
    constexpr int K = NS * NS + 2 * NS;
    constexpr int RS = K + 2;
#pragma unroll
    for (int k = 0; k < K; ++k) dz[k] = 0.f;
    float rinv = 0.f;
    if (valid) {
#pragma unroll
        for (int k = 0; k < NS; ++k) {
            const float hp = Hpre[t * NS + k], ho = Hpost[t * NS + k];
            dz[k] = dHpre[t * NS + k] * hp * (1.0f - hp);
            dz[NS + k] = dHpost[t * NS + k] * ho * (1.0f - ho);
        }
#pragma unroll
        for (int a = 0; a < NS * NS; ++a) dz[2 * NS + a] = dr[a];
        float S = 0.f;
#pragma unroll
        for (int k = 0; k < K; ++k) S += dz[k] * (z[t * K + k] - bias[k]);
        rinv = 1.0f / rms[t];
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const float a = k < NS ? a0 : (k < 2 * NS ? a1 : a2);
            dz_out[t * K + k] = dz[k];
            rec[t * RS + k] = a * dz[k];
        }
        rec[t * RS + K] = rinv;
        rec[t * RS + K + 1] = S * rinv * rinv / (float)N;
    }
}

// Sums of dz over a 16-token group held by lanes 16 j .. 16 j + 15 (lane l: token
// 16 g + l), by xor-exchanges 8, 4, 2, 1 within the group; lane 16 j writes them.
template <int K>
__device__ __forceinline__ void group16_sums(const float (&dz)[K], int64_t g, int64_t ngroups,
                                             float* __restrict__ dbpart)
{
#pragma unroll
    for (int k = 0; k < K; ++k) {
        float s = dz[k];
        s += __shfl_xor(s, 8, 64);
        s += __shfl_xor(s, 4, 64);
        s += __shfl_xor(s, 2, 64);
        s += __shfl_xor(s, 1, 64);
        if ((threadIdx.x & 15) == 0 && g < ngroups) dbpart[g * K + k] = s;
    }
}

// One token per lane (64 per block): the res-logit gradient given (dzres) or
// recomputed through the Sinkhorn backward (SK), then dz_token; dz sums per 16-token
// group (dbpart, groups [0, ngroups)).
template <int NS, bool SK>
__global__ __launch_bounds__(64) void k_dz(
    int64_t T, int64_t N, const float* __restrict__ z, const float* __restrict__ bias,
    const float* __restrict__ rms, const float* __restrict__ Hpre,
    const float* __restrict__ Hpost, const float* __restrict__ dHpre,
    const float* __restrict__ dHpost, const float* __restrict__ dzres, int64_t lddzr,
    const float* __restrict__ zres, int64_t ldz, const float* __restrict__ dHres, int iters,
    float a0, float a1, float a2, float* __restrict__ dz_out, float* __restrict__ rec,
    float* __restrict__ dbpart, int64_t ngroups)
{
    constexpr int K = NS * NS + 2 * NS;
    __shared__ float lds[SK ? sk_lds_floats<NS>() : 1];
    const int64_t t = (int64_t)blockIdx.x * 64 + threadIdx.x;
    const bool valid = t < T;
    float dr[NS * NS];
#pragma unroll
    for (int a = 0; a < NS * NS; ++a) dr[a] = 0.f;
    if (valid) {
        if (SK) {
            float zr[NS * NS], dH[NS * NS];
#pragma unroll
            for (int a = 0; a < NS * NS; ++a) { zr[a] = zres[t * ldz + a]; dH[a] = dHres[t * NS * NS + a]; }
            sinkhorn_bwd_token<NS>(zr, iters, dH, dr, lds + threadIdx.x);
        } else {
#pragma unroll
            for (int a = 0; a < NS * NS; ++a) dr[a] = dzres[t * lddzr + a];
        }
    }
    float dz[K];
    dz_token<NS>(t, valid, N, z, bias, rms, Hpre, Hpost, dHpre, dHpost, dr, a0, a1, a2, dz_out, rec, dz);
    // every lane reaches these reductions (invalid lanes contribute zeros)
    group16_sums<K>(dz, (int64_t)blockIdx.x * 4 + (threadIdx.x >> 4), ngroups, dbpart);
}

// ---------------------------------------------------------------- logit gradients, n = 4
// 16 tokens per block of 256 threads, token t = 16 blk + tid / 16 on the 16 lanes of a
// DPP row: lane q holds the token's res-logit gradient dz[8 + q], lanes 0-7 also form
// the gate gradient dz[q].  The block's tokens are one fragment tile and one db group.
// Both logit-gradient kernels at n = 4 end in this tail, so their results agree bitwise.
struct alignas(16) Dz16Stage {
    float dz[16][25];                  // the tokens' dz, for the db sums
    uint16_t qf[3 * 64 * 8];           // the tile's fragments in their memory layout
    uint16_t qw[2 * 64 * 8];
};

__device__ __forceinline__ uint16_t bf16_bits(float v) {
    return __builtin_bit_cast(uint16_t, (__bf16)v);
}

template <bool FRAGS>
__device__ __forceinline__ void dz16_tail(int64_t blk, int64_t T, int64_t N, float r,
                                          const float* __restrict__ z, const float* __restrict__ bias,
                                          const float* __restrict__ rms, const float* __restrict__ Hpre,
                                          const float* __restrict__ Hpost, const float* __restrict__ dHpre,
                                          const float* __restrict__ dHpost, float a0, float a1, float a2,
                                          float* __restrict__ dz_out, float* __restrict__ rec,
                                          float* __restrict__ dbpart, int64_t ngroups,
                                          bf16_t* __restrict__ qf, bf16_t* __restrict__ qw, int64_t Tfr,
                                          Dz16Stage& st)
{
    constexpr int K = 24, RS = K + 2;
    const int tr = threadIdx.x >> 4, q = threadIdx.x & 15;
    const int64_t t = blk * 16 + tr;
    const bool valid = t < T, gate = q < 8;
    float dzr = 0.f, dzg = 0.f, part = 0.f, rinv = 0.f;
    if (valid) {
        dzr = r;
        part = dzr * (z[t * K + 8 + q] - bias[8 + q]);
        if (gate) {
            // gating backward: dz = dH s (1 - s) with s the forward's gate
            const float h = q < 4 ? Hpre[t * 4 + q] : Hpost[t * 4 + q - 4];
            const float dh = q < 4 ? dHpre[t * 4 + q] : dHpost[t * 4 + q - 4];
            dzg = dh * h * (1.0f - h);
            part += dzg * (z[t * K + q] - bias[q]);
        }
        rinv = 1.0f / rms[t];
    }
    // S = sum_k dz_k (z_k - b_k), the same bits on the token's 16 lanes
    float S = part + lane_ror8(part);
    S += lane_ror4(S);
    S += lane_xor2(S);
    S += lane_xor1(S);
    const float qr = a2 * dzr, qg = (q < 4 ? a0 : a1) * dzg;
    if (valid) {
        dz_out[t * K + 8 + q] = dzr;
        rec[t * RS + 8 + q] = qr;
        if (gate) {
            dz_out[t * K + q] = dzg;
            rec[t * RS + q] = qg;
        }
        if (q == 0) {
            rec[t * RS + K] = rinv;
            rec[t * RS + K + 1] = S * rinv * rinv / (float)N;
        }
    }
    st.dz[tr][8 + q] = dzr;
    if (gate) st.dz[tr][q] = dzg;
    if (FRAGS) {
        // this lane's two columns of q: 8 + q, and q (lanes 0-7) or the zero pad 16 + q
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int k = e == 0 ? 8 + q : (gate ? q : 16 + q);
            const float v = e == 0 ? qr : (gate ? qg : 0.f);
            const float qh = (float)(__bf16)v, ql = (float)(__bf16)(v - qh);
            const float w = v * rinv;
            const float wh = (float)(__bf16)w, wl = (float)(__bf16)(w - wh);
#pragma unroll
            for (int ch = 0; ch < 3; ++ch)
                st.qf[(ch * 64 + (k >> 3) * 16 + tr) * 8 + (k & 7)] = bf16_bits(ch == 1 ? ql : qh);
            const int wi = ((k >> 4) * 64 + 16 * (tr >> 3) + (k & 15)) * 8 + (tr & 7);
            st.qw[wi] = bf16_bits(wh);
            st.qw[wi + 32 * 8] = bf16_bits(wl);       // lanes 32..63: the lo half of K
        }
    }
    __syncthreads();
    if (FRAGS && blk * 16 < Tfr) {
        // the tile: 192 16-byte pieces of qf, then 128 of qw
        for (int i = threadIdx.x; i < 320; i += 256) {
            const u32x4_t v = i < 192 ? reinterpret_cast<const u32x4_t*>(st.qf)[i]
                                      : reinterpret_cast<const u32x4_t*>(st.qw)[i - 192];
            if (i < 192) reinterpret_cast<u32x4_t*>(qf + blk * 3 * 64 * 8)[i] = v;
            else         reinterpret_cast<u32x4_t*>(qw + blk * 2 * 64 * 8)[i - 192] = v;
        }
    }
    if (threadIdx.x < K && blk < ngroups) {
        // db over the block's 16 tokens, in the order of an xor tree 8, 4, 2, 1
        const int k = threadIdx.x;
        float a[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) a[j] = st.dz[j][k] + st.dz[j + 8][k];
        float b[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) b[j] = a[j] + a[j + 4];
        dbpart[blk * K + k] = (b[0] + b[2]) + (b[1] + b[3]);
    }
}

// The Sinkhorn backward and the rest of the logit gradients in one launch, on the
// same 16 lanes per token.
template <bool FRAGS>
__global__ __launch_bounds__(256) void k_sk_dz16(
    int64_t T, int64_t N, const float* __restrict__ z, const float* __restrict__ bias,
    const float* __restrict__ rms, const float* __restrict__ Hpre,
    const float* __restrict__ Hpost, const float* __restrict__ dHpre,
    const float* __restrict__ dHpost, const float* __restrict__ zres, int64_t ldz,
    const float* __restrict__ dHres, int iters, float a0, float a1, float a2,
    float* __restrict__ dz_out, float* __restrict__ rec, float* __restrict__ dbpart,
    bf16_t* __restrict__ qf, bf16_t* __restrict__ qw, int64_t Tfr, int64_t ngroups)
{
    __shared__ Dz16Stage st;
    const int64_t g = blockIdx.x;
    const int64_t t = g * 16 + (threadIdx.x >> 4);
    const int q = threadIdx.x & 15;
    const bool valid = t < T;
    // tokens past T run on zeros so that every lane of a DPP row takes part
    const float r = sk16_bwd_token(valid ? zres[t * ldz + q] : 0.f, valid ? dHres[t * 16 + q] : 0.f,
                                   iters);
    dz16_tail<FRAGS>(g, T, N, r, z, bias, rms, Hpre, Hpost, dHpre, dHpost, a0, a1, a2, dz_out, rec,
                     dbpart, ngroups, qf, qw, Tfr, st);
}

// The same tail with the res-logit gradients given (dzres, row stride lddzr).
template <bool FRAGS>
__global__ __launch_bounds__(256) void k_dz16(
    int64_t T, int64_t N, const float* __restrict__ z, const float* __restrict__ bias,
    const float* __restrict__ rms, const float* __restrict__ Hpre,
    const float* __restrict__ Hpost, const float* __restrict__ dHpre,
    const float* __restrict__ dHpost, const float* __restrict__ dzres, int64_t lddzr,
    float a0, float a1, float a2, float* __restrict__ dz_out, float* __restrict__ rec,
    float* __restrict__ dbpart, bf16_t* __restrict__ qf, bf16_t* __restrict__ qw, int64_t Tfr,
    int64_t ngroups)
{
    __shared__ Dz16Stage st;
    const int64_t g = blockIdx.x;
    const int64_t t = g * 16 + (threadIdx.x >> 4);
    const float r = t < T ? dzres[t * lddzr + (threadIdx.x & 15)] : 0.f;
    dz16_tail<FRAGS>(g, T, N, r, z, bias, rms, Hpre, Hpost, dHpre, dHpost, a0, a1, a2, dz_out, rec,
                     dbpart, ngroups, qf, qw, Tfr, st);
}

// ---------------------------------------------------------------- coefficient backward
// Grid (ceil(N/256), R): a block owns 256 consecutive flattened elements e = k*C + c
// and a contiguous token range.  Per token: dy_e = W[e,:] . q_t; the element's
// gradient gamma_e dy_e / r - v_e S/(N r^2) (+ direct terms when G/g are given);
// the thread accumulates x_e q_t / r (dW row e, scaled by gamma_e at the end) and
// x_e dy_e / r (dgamma_e) over its token range into fixed-order partials.  With the
// direct terms, dX is written as Tdx (fp32, or the storage type when a stack passes
// it on to the layer below).
template <typename Tio, int NS, bool DIRECT, typename Tdx = float>
__global__ __launch_bounds__(256) void k_coeffs_bwd_main(
    int64_t T, int64_t C, int64_t tpr, const Tio* __restrict__ X,
    const float* __restrict__ gamma, const float* __restrict__ W,
    const float* __restrict__ rec, const Tio* __restrict__ G, const Tio* __restrict__ g,
    const float* __restrict__ Hres, const float* __restrict__ Hpre, void* __restrict__ dXv,
    float* __restrict__ wpart, float* __restrict__ gpart)
{
    float* dX = static_cast<float*>(dXv);
    constexpr int K = NS * NS + 2 * NS;
    constexpr int RS = K + 2;
    constexpr int TBATCH = 64;
    constexpr int EXTRA = DIRECT ? NS * NS + NS : 0;
    __shared__ float srec[TBATCH * (RS + EXTRA)];
    const int64_t N = NS * C;
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const bool valid = e < N;
    const int ks = valid ? (int)(e / C) : 0;
    const int64_t c = valid ? e - (int64_t)ks * C : 0;
    const int64_t tb0 = (int64_t)blockIdx.y * tpr;
    const int64_t tb1 = (tb0 + tpr) < T ? (tb0 + tpr) : T;

    float w[K], accW[K];
    float accG = 0.f;
    const float gm = valid ? gamma[e] : 0.f;
#pragma unroll
    for (int k = 0; k < K; ++k) { w[k] = valid ? W[e * K + k] : 0.f; accW[k] = 0.f; }

    for (int64_t tb = tb0; tb < tb1; tb += TBATCH) {
        const int nb = (int)((tb1 - tb) < TBATCH ? (tb1 - tb) : TBATCH);
        __syncthreads();
        for (int i = threadIdx.x; i < nb * RS; i += 256) srec[i] = rec[tb * RS + i];
        if (DIRECT) {
            float* sx = srec + TBATCH * RS;
            for (int i = threadIdx.x; i < nb * NS * NS; i += 256) sx[i] = Hres[tb * NS * NS + i];
            for (int i = threadIdx.x; i < nb * NS; i += 256) sx[TBATCH * NS * NS + i] = Hpre[tb * NS + i];
        }
        __syncthreads();
        if (!valid) continue;
        for (int j = 0; j < nb; ++j) {
            const int64_t t = tb + j;
            const float* q = srec + j * RS;
            const float x = io<Tio>::load1(X + t * N + e);
            float dy = 0.f;
#pragma unroll
            for (int k = 0; k < K; ++k) dy += w[k] * q[k];
            const float rinv = q[K];
            float val = gm * dy * rinv - x * q[K + 1];
            if (DIRECT) {
                const float* sx = srec + TBATCH * RS;
                const float* hr = sx + j * NS * NS;
#pragma unroll
                for (int i = 0; i < NS; ++i)
                    val += hr[i * NS + ks] * io<Tio>::load1(G + (t * NS + i) * C + c);
                val += sx[TBATCH * NS * NS + j * NS + ks] * io<Tio>::load1(g + t * C + c);
                io<Tdx>::store1(static_cast<Tdx*>(dXv) + t * N + e, val);
            } else if (dX) {
                dX[t * N + e] += val;
            }
            const float xr = x * rinv;
#pragma unroll
            for (int k = 0; k < K; ++k) accW[k] += xr * q[k];
            accG += xr * dy;
        }
    }
    if (!valid) return;
    float* wp = wpart + ((int64_t)blockIdx.y * N + e) * K;
#pragma unroll
    for (int k = 0; k < K; ++k) wp[k] = gm * accW[k];
    gpart[(int64_t)blockIdx.y * N + e] = accG;
}

// dW[i] = sum_r wpart[r][i] and dgamma[e] = sum_r gpart[r][e], r in order.
// dW (and dgamma) = sum over the token ranges of their partials, in range order.
// The grid's last block instead forms dbias[k] = sum over the 64-token blocks of
// their dz sums: thread i adds blocks i, i + 256, ... in order, then a fixed tree
// over the 256 threads.
template <int K>
__global__ __launch_bounds__(256) void k_reduce_parts(int64_t NK, int64_t N, int R,
                                                      const float* __restrict__ wpart,
                                                      const float* __restrict__ gpart,
                                                      float* __restrict__ dW,
                                                      float* __restrict__ dgamma, int64_t nblk,
                                                      const float* __restrict__ dbpart,
                                                      float* __restrict__ dbias)
{
    if (blockIdx.x == gridDim.x - 1) {
        __shared__ float scratch[4 * K];
        __shared__ float tot[K];
        float s[K];
#pragma unroll
        for (int k = 0; k < K; ++k) s[k] = 0.f;
        for (int64_t b = threadIdx.x; b < nblk; b += 256)
#pragma unroll
            for (int k = 0; k < K; ++k) s[k] += dbpart[b * K + k];
        block_sum_256<K>(s, scratch, tot);
        if (threadIdx.x < K) dbias[threadIdx.x] = tot[threadIdx.x];
        return;
    }
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < NK) {
        float s = 0.f;
        for (int r = 0; r < R; ++r) s += wpart[(int64_t)r * NK + i];
        dW[i] = s;
    }
    if (dgamma && i < N) {
        float s = 0.f;
        for (int r = 0; r < R; ++r) s += gpart[(int64_t)r * N + i];
        dgamma[i] = s;
    }
}


// Gradient of the three logit scales.  z_k = alpha_g(k) proj_k + bias_k with proj the
// unscaled normalised projection p_k / r that the forward wrote, so d alpha_g = sum over
// tokens and k in group g of dz_k proj_k.  Block b covers elements [b E / G, (b+1) E / G)
// of the flat [T][K] arrays (E = T K); each product of two fp32 values is exact in fp64
// and sums run in fp64: per thread in index order, then a fixed tree over the block.
// part[b][g] is the block's sum.
constexpr int kAlphaBlocks = 256;

__global__ __launch_bounds__(256) void k_alpha_part(int64_t E, int n, const float* __restrict__ proj,
                                                    const float* __restrict__ dz,
                                                    double* __restrict__ part)
{
    const int K = n * n + 2 * n;
    const int64_t e0 = E * blockIdx.x / gridDim.x, e1 = E * (blockIdx.x + 1) / gridDim.x;
    double s[3] = {0.0, 0.0, 0.0};
    for (int64_t e = e0 + threadIdx.x; e < e1; e += 256) {
        const int k = (int)(e % K);
        const double v = (double)proj[e] * (double)dz[e];
        const int g = k < n ? 0 : (k < 2 * n ? 1 : 2);
        s[0] += g == 0 ? v : 0.0;
        s[1] += g == 1 ? v : 0.0;
        s[2] += g == 2 ? v : 0.0;
    }
    __shared__ double sh[3][256];
#pragma unroll
    for (int g = 0; g < 3; ++g) sh[g][threadIdx.x] = s[g];
    __syncthreads();
    for (int h = 128; h > 0; h >>= 1) {
        if ((int)threadIdx.x < h)
#pragma unroll
            for (int g = 0; g < 3; ++g) sh[g][threadIdx.x] += sh[g][threadIdx.x + h];
        __syncthreads();
    }
    if (threadIdx.x < 3) part[blockIdx.x * 3 + threadIdx.x] = sh[threadIdx.x][0];
}

// dalpha[g] = the sum of part[b][g] over b in order, rounded to fp32 once.
__global__ __launch_bounds__(64) void k_alpha_final(int blocks, const double* __restrict__ part,
                                                    float* __restrict__ dalpha)
{
    const int g = threadIdx.x;
    if (g >= 3) return;
    double s = 0.0;
    for (int b = 0; b < blocks; ++b) s += part[b * 3 + g];
    dalpha[g] = (float)s;
}

// ================================================================ launchers
static inline unsigned blocks_for(int64_t n, int per) { return (unsigned)((n + per - 1) / per); }

int bwd_token_ranges(int64_t T, int n, int64_t C)
{
    const int64_t N = (int64_t)n * C;
    const int64_t nsl = (N + 255) / 256;
    int64_t R = (1024 + nsl - 1) / nsl;
    const int64_t rmax = (T + 63) / 64;
    if (R > rmax) R = rmax;
    if (R < 1) R = 1;
    return (int)R;
}

static int64_t pad32(int64_t T) { return (T + 31) / 32 * 32; }

size_t bwd_workspace_bytes(int64_t T, int n, int64_t C, int dtype)
{
    const int64_t N = (int64_t)n * C;
    const int K = K_of(n);
    const bool mf = bwd_use_mfma(T, n, C, dtype);
    const int R = mf ? bwd_mfma_ranges(T, C) : bwd_token_ranges(T, n, C);
    const int64_t nblk = (pad32(T) + 15) / 16;           // 16-token groups of the dz sums
    return align256(sizeof(float) * (size_t)T * rec_stride(n)) +
           align256(sizeof(float) * (size_t)T * K) +
           align256(sizeof(float) * (size_t)R * N * K) +
           align256(sizeof(float) * (size_t)R * N) +
           align256(sizeof(float) * (size_t)nblk * K) +
           (mf ? bwd_mfma_frag_bytes(T) : 0);
}

BwdWorkspace bwd_workspace_carve(void* ws, int64_t T, int n, int64_t C, int dtype)
{
    const int64_t N = (int64_t)n * C;
    const int K = K_of(n);
    BwdWorkspace w;
    w.mfma = bwd_use_mfma(T, n, C, dtype);
    w.R = w.mfma ? bwd_mfma_ranges(T, C) : bwd_token_ranges(T, n, C);
    const int64_t nblk = (pad32(T) + 15) / 16;
    char* p = static_cast<char*>(ws);
    w.rec = reinterpret_cast<float*>(p);    p += align256(sizeof(float) * (size_t)T * rec_stride(n));
    w.dz = reinterpret_cast<float*>(p);     p += align256(sizeof(float) * (size_t)T * K);
    w.wpart = reinterpret_cast<float*>(p);  p += align256(sizeof(float) * (size_t)w.R * N * K);
    w.gpart = reinterpret_cast<float*>(p);  p += align256(sizeof(float) * (size_t)w.R * N);
    w.dbpart = reinterpret_cast<float*>(p); p += align256(sizeof(float) * (size_t)nblk * K);
    w.qf = w.mfma ? reinterpret_cast<uint16_t*>(p) : nullptr;
    if (w.mfma) p += align256((size_t)pad32(T) * 192);   // qw follows (pad32(T) * 128 bytes)
    w.qw = w.mfma ? reinterpret_cast<uint16_t*>(p) : nullptr;
    return w;
}

hipError_t launch_post_res_bwd(int64_t T, int n, int64_t C, int dtype, const void* G,
                               const void* X, const void* F, const float* Hres,
                               const float* Hpost, float* dF, float* dHres, float* dHpost,
                               float* dX, hipStream_t s, const void* du, float* dHpre)
{
    const dim3 g((unsigned)T), b(256);
    for_io(dtype == MHC_BF16, [&](auto tio) {
        using Tio = decltype(tio);
        for_n(n, [&](auto ns) {
            constexpr int NS = decltype(ns)::value;
            if (du)
                hipLaunchKernelGGL((k_post_res_bwd<Tio, NS, true>), g, b, 0, s, C, (const Tio*)G,
                                   (const Tio*)X, (const Tio*)F, Hres, Hpost, (const Tio*)du, dF,
                                   dHres, dHpost, dHpre, dX);
            else
                hipLaunchKernelGGL((k_post_res_bwd<Tio, NS, false>), g, b, 0, s, C, (const Tio*)G,
                                   (const Tio*)X, (const Tio*)F, Hres, Hpost, (const Tio*)nullptr, dF,
                                   dHres, dHpost, (float*)nullptr, dX);
        });
    });
    return hipGetLastError();
}

hipError_t launch_pre_bwd(int64_t T, int n, int64_t C, int dtype, const void* g, const void* X,
                          const float* Hpre, float* dHpre, float* dX, hipStream_t s)
{
    const dim3 gr((unsigned)T), b(256);
    for_io(dtype == MHC_BF16, [&](auto tio) {
        using Tio = decltype(tio);
        for_n(n, [&](auto ns) {
            hipLaunchKernelGGL((k_pre_bwd<Tio, decltype(ns)::value>), gr, b, 0, s, C, (const Tio*)g,
                               (const Tio*)X, Hpre, dHpre, dX);
        });
    });
    return hipGetLastError();
}

hipError_t launch_pre_bwd_sk(int64_t T, int64_t C, int dtype, const void* g, const void* X,
                             const float* Hpre, float* dHpre, const float* zres, int64_t ldz,
                             int iters, const float* dHres, float* dzres, int64_t lddz,
                             hipStream_t s)
{
    const int64_t nsk = (T + 15) / 16;
    const dim3 gr((unsigned)(nsk + T)), b(256);
    for_io(dtype == MHC_BF16, [&](auto tio) {
        using Tio = decltype(tio);
        hipLaunchKernelGGL((k_pre_bwd_sk16<Tio>), gr, b, 0, s, T, C, nsk, (const Tio*)g, (const Tio*)X,
                           Hpre, dHpre, zres, ldz, iters, dHres, dzres, lddz);
    });
    return hipGetLastError();
}

hipError_t launch_sinkhorn_bwd(int64_t T, int n, const float* zres, int64_t ldz, int iters,
                               const float* dHres, float* dzres, int64_t lddz, hipStream_t s)
{
    if (n == 4) {
        hipLaunchKernelGGL(k_sinkhorn_bwd16, dim3(blocks_for(T, 16)), dim3(256), 0, s, T, zres, ldz, iters,
                           dHres, dzres, lddz);
    } else {
        for_n(n, [&](auto ns) {
            hipLaunchKernelGGL((k_sinkhorn_bwd<decltype(ns)::value>), dim3(blocks_for(T, 64)), dim3(64), 0,
                               s, T, zres, ldz, iters, dHres, dzres, lddz);
        });
    }
    return hipGetLastError();
}

template <typename Tio, int NS>
static void coeffs_bwd_impl(int64_t T, int64_t C, int dtype, const void* X, const float* gamma,
                            const float* W, const float* alpha, const float* z,
                            const float* bias, const float* rms, const float* Hpre,
                            const float* Hpost, const float* dHpre, const float* dHpost,
                            const float* dzres, const float* zres, int64_t ldz,
                            const float* dHres, int iters, const void* G, const void* g,
                            const float* Hres, float* dX, float* dW, float* dbias,
                            float* dgamma, float* dz, void* ws, bool dx_storage, bool sk_done,
                            hipStream_t s)
{
    constexpr int K = NS * NS + 2 * NS;
    const int64_t N = NS * C;
    BwdWorkspace w = bwd_workspace_carve(ws, T, NS, C, dtype);
    float* dzo = dz ? dz : w.dz;
    const int64_t Tz = w.mfma ? pad32(T) : T;
    const unsigned nblk = blocks_for(Tz, 64);
    const int64_t ngroups = (Tz + 15) / 16;               // 16-token groups of the dz sums
    const float a0 = alpha[0], a1 = alpha[1], a2 = alpha[2];
    bf16_t* qf = reinterpret_cast<bf16_t*>(w.qf);
    bf16_t* qw = reinterpret_cast<bf16_t*>(w.qw);
#define MHC_KDZ16(FR, DZR, LDR) \
    hipLaunchKernelGGL((k_dz16<FR>), dim3((unsigned)ngroups), dim3(256), 0, s, T, N, z, bias, rms, \
                       Hpre, Hpost, dHpre, dHpost, DZR, LDR, a0, a1, a2, dzo, w.rec, w.dbpart, qf, \
                       qw, Tz, ngroups)
#define MHC_KDZ(SKF, DZR, LDR, ZR, LD, DH) \
    hipLaunchKernelGGL((k_dz<NS, SKF>), dim3(nblk), dim3(64), 0, s, T, N, z, bias, rms, Hpre, \
                       Hpost, dHpre, dHpost, DZR, LDR, ZR, LD, DH, iters, a0, a1, a2, dzo,     \
                       w.rec, w.dbpart, ngroups)
    if (dHres) {
        if constexpr (NS == 4) {
            if (!sk_done) {
                // the Sinkhorn backward on 16 lanes per token and the rest of the logit
                // gradients in one launch
#define MHC_KSKDZ(FR) \
                hipLaunchKernelGGL((k_sk_dz16<FR>), dim3((unsigned)ngroups), dim3(256), 0, s, T, N, z, bias, \
                                   rms, Hpre, Hpost, dHpre, dHpost, zres, ldz, dHres, iters, a0, a1, a2, \
                                   dzo, w.rec, w.dbpart, qf, qw, Tz, ngroups)
                if (w.mfma) MHC_KSKDZ(true);
                else        MHC_KSKDZ(false);
#undef MHC_KSKDZ
            } else {
                // the pre backward's launch left the res-logit gradients in dz's res columns
                if (w.mfma) MHC_KDZ16(true, (const float*)(dzo + 2 * NS), (int64_t)K);
                else        MHC_KDZ16(false, (const float*)(dzo + 2 * NS), (int64_t)K);
            }
        } else {
            // the MFMA path (and its fragments) is n = 4 only
            MHC_KDZ(true, (const float*)nullptr, (int64_t)0, zres, ldz, dHres);
        }
    } else {
        if constexpr (NS == 4) {
            if (w.mfma) MHC_KDZ16(true, dzres, (int64_t)(NS * NS));
            else        MHC_KDZ16(false, dzres, (int64_t)(NS * NS));
        } else {
            MHC_KDZ(false, dzres, (int64_t)(NS * NS), (const float*)nullptr, (int64_t)0, (const float*)nullptr);
        }
    }
#undef MHC_KDZ
#undef MHC_KDZ16
    int R = w.R;                                         // partial slots to reduce
    if (w.mfma) {
        R = launch_bwd_mfma(T, C, X, gamma, W, w.rec, K + 2, w.qf, w.qw, G, g, Hres, Hpre, dX,
                            w.wpart, w.gpart, dgamma != nullptr, G && dx_storage, s);
    } else {
        const int64_t tpr = (T + w.R - 1) / w.R;
        const dim3 grid(blocks_for(N, 256), (unsigned)w.R);
        if (G && dx_storage)
            hipLaunchKernelGGL((k_coeffs_bwd_main<Tio, NS, true, Tio>), grid, dim3(256), 0, s, T, C,
                               tpr, (const Tio*)X, gamma, W, w.rec, (const Tio*)G, (const Tio*)g,
                               Hres, Hpre, (void*)dX, w.wpart, w.gpart);
        else if (G)
            hipLaunchKernelGGL((k_coeffs_bwd_main<Tio, NS, true>), grid, dim3(256), 0, s, T, C, tpr,
                               (const Tio*)X, gamma, W, w.rec, (const Tio*)G, (const Tio*)g, Hres,
                               Hpre, (void*)dX, w.wpart, w.gpart);
        else
            hipLaunchKernelGGL((k_coeffs_bwd_main<Tio, NS, false>), grid, dim3(256), 0, s, T, C, tpr,
                               (const Tio*)X, gamma, W, w.rec, (const Tio*)nullptr,
                               (const Tio*)nullptr, (const float*)nullptr, (const float*)nullptr,
                               (void*)dX, w.wpart, w.gpart);
    }
    hipLaunchKernelGGL((k_reduce_parts<K>), dim3(blocks_for(N * K, 256) + 1), dim3(256), 0, s,
                       N * K, N, R, w.wpart, w.gpart, dW, dgamma, ngroups, w.dbpart, dbias);
}

hipError_t launch_coeffs_bwd(int64_t T, int n, int64_t C, int dtype, const void* X,
                             const float* gamma, const float* W, const float* alpha,
                             const float* z, const float* bias, const float* rms,
                             const float* Hpre, const float* Hpost, const float* dHpre,
                             const float* dHpost, const float* dzres, const float* zres,
                             int64_t ldz, const float* dHres, int iters, const void* G,
                             const void* g, const float* Hres, float* dX, float* dW,
                             float* dbias, float* dgamma, float* dz, void* ws, hipStream_t s,
                             bool dx_storage, bool sk_done)
{
#define MHC_CB_ARGS T, C, dtype, X, gamma, W, alpha, z, bias, rms, Hpre, Hpost, dHpre, dHpost, dzres, \
                    zres, ldz, dHres, iters, G, g, Hres, dX, dW, dbias, dgamma, dz, ws, dx_storage,   \
                    sk_done, s
    for_io(dtype == MHC_BF16, [&](auto tio) {
        for_n(n, [&](auto ns) { coeffs_bwd_impl<decltype(tio), decltype(ns)::value>(MHC_CB_ARGS); });
    });
#undef MHC_CB_ARGS
    return hipGetLastError();
}

size_t alpha_bwd_workspace_bytes() { return align256(sizeof(double) * 3 * kAlphaBlocks); }

hipError_t launch_alpha_bwd(int64_t T, int n, const float* proj, const float* dz, float* dalpha,
                            void* ws, hipStream_t s)
{
    const int64_t E = T * K_of(n);
    const int G = (int)(E < 256LL * kAlphaBlocks ? (E + 255) / 256 : kAlphaBlocks);
    double* part = reinterpret_cast<double*>(ws);
    hipLaunchKernelGGL(k_alpha_part, dim3(G), dim3(256), 0, s, E, n, proj, dz, part);
    hipLaunchKernelGGL(k_alpha_final, dim3(1), dim3(64), 0, s, G, (const double*)part, dalpha);
    return hipGetLastError();
}

}  // namespace mhc
