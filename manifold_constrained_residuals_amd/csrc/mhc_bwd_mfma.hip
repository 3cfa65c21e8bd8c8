// mhc_bwd_mfma.hip -- MFMA path of the coefficient backward (bf16 storage, n = 4).
//
// For each token t and flattened element e = k*C + c (stream k, channel c):
//   dy[e][t]  = sum_kappa W[e][kappa] q_t[kappa]                 (q = alpha (.) dz)
//   dX[t][e]  = sum_i H_res[t][i][k] G[t][i][c] + H_pre[t][k] g[t][c]      (direct)
//             + gamma_e dy[e][t] / r_t - x[t][e] S_t / (N r_t^2)
//   dW[e][kappa] = gamma_e sum_t x[t][e] q_t[kappa] / r_t
// Both contractions run on v_mfma_f32_16x16x32_bf16:
//   dy: A = W rows split into bf16 hi/lo, B = q split into hi/lo, K = 3 chunks of
//       32 pairing (W_hi, q_hi), (W_hi, q_lo), (W_lo, q_hi) -- about 16 significant
//       bits for each factor; the lo*lo term is below fp32 rounding of the sum;
//   dW: A = x transposed through LDS (exact in bf16), B = q/r split hi/lo as 48
//       columns; K = 32 tokens per MFMA, accumulated over the block's token range.
// A block owns 64 channels of all 4 streams (8 waves) and a token range;
// dW partials per token range are reduced afterwards in a fixed order.
#include "mhc_device.hpp"
#include "mhc_internal.hpp"
#include "../../include/mhc.h"

namespace mhc {

__device__ __forceinline__ uint32_t pk(float a, float b) { return pack_bf16x2(a, b); }

constexpr int kBT = 32;                 // tokens per block step
constexpr int kCS = 64;                 // channels per workgroup (full 128-byte lines of bf16 rows)
constexpr int kThreads = 512;           // 8 waves: wave w = stream w / 2, channel half w % 2
constexpr int kRowPad = 72;             // bf16 per LDS row of sX / sG / sg (64 + 8 pad)
constexpr int kTPitch = 34;             // bf16 per row of the transposed x tile: 32 tokens + 2;
                                        // the 32-bit token-pair stores of a wave hit distinct banks
constexpr int kScal = 25;               // per-token scalars in LDS: rinv, c2, Hpre[4], Hres[16], pad

// ---------------------------------------------------------------- q fragments
// qf / qw are written by the logit-gradient kernel (mhc_bwd.hip, write_qfrags):
//   qf[t/16][chunk][lane][8]: dy B operand; token t%16 = lane%16, kappa = 8*(lane/16)+j;
//       chunk 0: q_hi, 1: q_lo, 2: q_hi; kappa >= 24 is zero.
//   qw[t/32][nb][lane][8]: dW B operand; column 16*nb + lane%16 of [q'_hi | q'_lo]
//       (q' = q / r), tokens 8*(lane/16) + j of the 32-token block.

// ---------------------------------------------------------------- main kernel
// grid (C / 64) * R blocks of 512 threads; block -> (channel slice, token range
// [range * tpr, + tpr)), tpr % 32 == 0.  Wave w handles stream k = w / 2 and
// channels c0 + 32 (w % 2) + [0, 32): two 16-element MFMA row tiles.
template <bool DIRECT, bool DGAMMA>
__global__ __launch_bounds__(kThreads) void k_bwd_mfma(
    int64_t T, int64_t C, int64_t tpr, const bf16_t* __restrict__ X,
    const float* __restrict__ gamma, const float* __restrict__ W,
    const float* __restrict__ rec, int rs, const bf16_t* __restrict__ qf,
    const bf16_t* __restrict__ qw, const bf16_t* __restrict__ G, const bf16_t* __restrict__ g,
    const float* __restrict__ Hres, const float* __restrict__ Hpre, float* __restrict__ dX,
    float* __restrict__ wpart, float* __restrict__ gpart)
{
    __shared__ __attribute__((aligned(16))) bf16_t sX[4][kBT][kRowPad];    // [k][t][c]
    __shared__ __attribute__((aligned(16))) bf16_t sXT[4][kCS][kTPitch];   // [k][c][t]
    __shared__ __attribute__((aligned(16))) bf16_t sG[4][kBT][kRowPad];    // [i][t][c]
    __shared__ __attribute__((aligned(16))) bf16_t sg[kBT][kRowPad];       // [t][c]
    __shared__ float sS[kBT][kScal];
    __shared__ __attribute__((aligned(16))) u32x4_t sQ[9][64];             // qf (6 tiles) + qw (3 tiles)
    __shared__ float sW[32][49];                                           // dW combine

    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int k = wv >> 1, ch0 = 32 * (wv & 1);                // stream, first local channel
    const int col = lane & 15, grp = lane >> 4;
    const int64_t N = 4 * C;
    // 1-D grid.  Blocks are dealt round-robin to the 8 XCDs, so when the slice count
    // divides by 8, XCD x gets the contiguous slice band [x S/8, (x+1) S/8): the blocks
    // resident on one XCD then read long runs of every token row.
    const int64_t S = C / kCS, b = blockIdx.x;
    int64_t slice, range;
    if ((S & 7) == 0) {
        const int64_t per = S >> 3;
        slice = (b & 7) * per + (b >> 3) % per;
        range = b / S;
    } else {
        slice = b % S;
        range = b / S;
    }
    const int64_t c0 = slice * kCS;
    const int64_t tb0 = range * tpr;
    const int64_t tb1 = (tb0 + tpr) < T ? (tb0 + tpr) : T;

    // dy A operand: W rows of this wave's 32 elements, split hi/lo, K chunks (hi, hi, lo)
    u32x4_t aW[2][3];
    float gm[2][4];
#pragma unroll
    for (int a = 0; a < 2; ++a) {
        const int64_t e = (int64_t)k * C + c0 + ch0 + 16 * a + col;
        float w[8], wh[8], wl[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int kk = 8 * grp + j;
            w[j] = kk < 24 ? W[e * 24 + kk] : 0.f;
            wh[j] = (float)(__bf16)w[j];
            wl[j] = (float)(__bf16)(w[j] - wh[j]);
        }
        aW[a][0] = u32x4_t{pk(wh[0], wh[1]), pk(wh[2], wh[3]), pk(wh[4], wh[5]), pk(wh[6], wh[7])};
        aW[a][1] = aW[a][0];
        aW[a][2] = u32x4_t{pk(wl[0], wl[1]), pk(wl[2], wl[3]), pk(wl[4], wl[5]), pk(wl[6], wl[7])};
#pragma unroll
        for (int i = 0; i < 4; ++i) gm[a][i] = gamma[(int64_t)k * C + c0 + ch0 + 16 * a + 4 * grp + i];
    }

    f32x4_t accW[2][3];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int nb = 0; nb < 3; ++nb) accW[a][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float accG[2][4];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int i = 0; i < 4; ++i) accG[a][i] = 0.f;

    // Staging of one 32-token step.  Thread: stream kk = tid / 128, token pair tp =
    // (tid % 128) / 8 (tokens 2tp, 2tp + 1), 16-byte chunk cc = tid % 8 (channels
    // 8 cc .. 8 cc + 7).  g: threads < 256 load token tid / 8, chunk tid % 8.
    // Fragments: 6 qf tiles then 3 qw tiles of 64 lanes; scalars: 704 floats.
    // The next step's data is loaded into registers while the current step
    // computes, then written to LDS after a barrier.
    struct Regs {
        u32x4_t pX[2], pG[2], pg, pQ[2];
        float pS[2];
    };
    Regs RA, RB;
    const int skk = threadIdx.x >> 7, stp = (threadIdx.x & 127) >> 3, scc = (threadIdx.x & 7) * 8;
    auto prefetch = [&](int64_t tb, Regs& R) {
        u32x4_t (&pX)[2] = R.pX; u32x4_t (&pG)[2] = R.pG; u32x4_t& pg = R.pg;
        u32x4_t (&pQ)[2] = R.pQ; float (&pS)[2] = R.pS;
        const int nb_t = (int)((tb1 - tb) < kBT ? (tb1 - tb) : kBT);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int t = 2 * stp + h;
            pX[h] = u32x4_t{0u, 0u, 0u, 0u};
            pG[h] = u32x4_t{0u, 0u, 0u, 0u};
            if (t < nb_t) {
                const int64_t base = ((tb + t) * 4 + skk) * C + c0 + scc;
                pX[h] = *reinterpret_cast<const u32x4_t*>(X + base);
                if (DIRECT) pG[h] = *reinterpret_cast<const u32x4_t*>(G + base);
            }
        }
        pg = u32x4_t{0u, 0u, 0u, 0u};
        if (DIRECT && threadIdx.x < 256) {
            const int t = threadIdx.x >> 3, cc = (threadIdx.x & 7) * 8;
            if (t < nb_t) pg = *reinterpret_cast<const u32x4_t*>(g + (tb + t) * C + c0 + cc);
        }
        {
            const int64_t qt = tb >> 4, qb = tb >> 5;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int q = threadIdx.x + kThreads * h;
                if (q < 9 * 64) {
                    const int tile = q >> 6, ln = q & 63;
                    const bf16_t* src = tile < 6 ? qf + ((qt * 3 + tile) * 64 + ln) * 8
                                                 : qw + ((qb * 3 + (tile - 6)) * 64 + ln) * 8;
                    pQ[h] = *reinterpret_cast<const u32x4_t*>(src);
                }
            }
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int q = threadIdx.x + kThreads * h;
            pS[h] = 0.f;
            if (q < kBT * 22) {
                const int t = q / 22, j = q % 22;
                if (t < nb_t) {
                    const int64_t tt = tb + t;
                    if (j < 2) pS[h] = rec[tt * rs + 24 + j];
                    else if (DIRECT && j < 6) pS[h] = Hpre[tt * 4 + (j - 2)];
                    else if (DIRECT) pS[h] = Hres[tt * 16 + (j - 6)];
                }
            }
        }
    };
    auto stage = [&](const Regs& R) {
        const u32x4_t (&pX)[2] = R.pX; const u32x4_t (&pG)[2] = R.pG; const u32x4_t& pg = R.pg;
        const u32x4_t (&pQ)[2] = R.pQ; const float (&pS)[2] = R.pS;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            *reinterpret_cast<u32x4_t*>(&sX[skk][2 * stp + h][scc]) = pX[h];
            if (DIRECT) *reinterpret_cast<u32x4_t*>(&sG[skk][2 * stp + h][scc]) = pG[h];
        }
        // transposed copy: channel scc + j gets the 32-bit word (token 2stp, token 2stp + 1)
        const uint32_t a[4] = {pX[0].x, pX[0].y, pX[0].z, pX[0].w};
        const uint32_t b[4] = {pX[1].x, pX[1].y, pX[1].z, pX[1].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            *reinterpret_cast<uint32_t*>(&sXT[skk][scc + 2 * j][2 * stp]) = (a[j] & 0xffffu) | (b[j] << 16);
            *reinterpret_cast<uint32_t*>(&sXT[skk][scc + 2 * j + 1][2 * stp]) = (a[j] >> 16) | (b[j] & 0xffff0000u);
        }
        if (DIRECT && threadIdx.x < 256)
            *reinterpret_cast<u32x4_t*>(&sg[threadIdx.x >> 3][(threadIdx.x & 7) * 8]) = pg;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int q = threadIdx.x + kThreads * h;
            if (q < kBT * 22) sS[q / 22][q % 22] = pS[h];
            if (q < 9 * 64) sQ[q >> 6][q & 63] = pQ[h];
        }
    };

    // Two register sets: while step i computes, the loads of steps i + 1 and i + 2
    // are in flight.
    auto compute = [&](int64_t tb) {
        const int nb_t = (int)((tb1 - tb) < kBT ? (tb1 - tb) : kBT);
        // ---- dy = W q on MFMA, then the element gradient
#pragma unroll
        for (int bt = 0; bt < 2; ++bt) {
            u32x4_t bq[3];
#pragma unroll
            for (int ch = 0; ch < 3; ++ch) bq[ch] = sQ[bt * 3 + ch][lane];
            const int t = 16 * bt + col;      // token of this lane within the step
            const float rinv = sS[t][0], c2 = sS[t][1];
#pragma unroll
            for (int a = 0; a < 2; ++a) {
                f32x4_t dy = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ch = 0; ch < 3; ++ch) dy = mfma16(aW[a][ch], bq[ch], dy);
                const int cl = ch0 + 16 * a + 4 * grp;     // first local channel of this lane
                const u32x2_t xv = *reinterpret_cast<const u32x2_t*>(&sX[k][t][cl]);
                const float x[4] = {bf16_lo(xv.x), bf16_hi(xv.x), bf16_lo(xv.y), bf16_hi(xv.y)};
                float o[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) o[i] = gm[a][i] * dy[i] * rinv - x[i] * c2;
                if (DGAMMA) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) accG[a][i] += x[i] * dy[i] * rinv;
                }
                if (t < nb_t) {
                    float* dst = dX + ((tb + t) * 4 + k) * C + c0 + cl;
                    if (DIRECT) {
#pragma unroll
                        for (int ii = 0; ii < 4; ++ii) {
                            const float h = sS[t][6 + ii * 4 + k];
                            const u32x2_t gv = *reinterpret_cast<const u32x2_t*>(&sG[ii][t][cl]);
                            o[0] += h * bf16_lo(gv.x); o[1] += h * bf16_hi(gv.x);
                            o[2] += h * bf16_lo(gv.y); o[3] += h * bf16_hi(gv.y);
                        }
                        const float hp = sS[t][2 + k];
                        const u32x2_t uv = *reinterpret_cast<const u32x2_t*>(&sg[t][cl]);
                        o[0] += hp * bf16_lo(uv.x); o[1] += hp * bf16_hi(uv.x);
                        o[2] += hp * bf16_lo(uv.y); o[3] += hp * bf16_hi(uv.y);
                        *reinterpret_cast<float4*>(dst) = make_float4(o[0], o[1], o[2], o[3]);
                    } else if (dX) {
                        float4 d = *reinterpret_cast<float4*>(dst);
                        d.x += o[0]; d.y += o[1]; d.z += o[2]; d.w += o[3];
                        *reinterpret_cast<float4*>(dst) = d;
                    }
                }
            }
        }

        // ---- dW += x^T (q / r) on MFMA, K = 32 tokens of this step
        u32x4_t bw[3];
#pragma unroll
        for (int nb = 0; nb < 3; ++nb) bw[nb] = sQ[6 + nb][lane];
#pragma unroll
        for (int a = 0; a < 2; ++a) {
            // rows of sXT are 4-byte aligned: read the 8 tokens as four 32-bit words
            const uint32_t* rowp = reinterpret_cast<const uint32_t*>(&sXT[k][ch0 + 16 * a + col][8 * grp]);
            const u32x4_t ax = u32x4_t{rowp[0], rowp[1], rowp[2], rowp[3]};
#pragma unroll
            for (int nb = 0; nb < 3; ++nb) accW[a][nb] = mfma16(ax, bw[nb], accW[a][nb]);
        }
    };

    if (tb0 < tb1) prefetch(tb0, RA);
    if (tb0 + kBT < tb1) prefetch(tb0 + kBT, RB);
    for (int64_t tb = tb0; tb < tb1; tb += 2 * kBT) {
        __syncthreads();
        stage(RA);
        __syncthreads();
        if (tb + 2 * kBT < tb1) prefetch(tb + 2 * kBT, RA);
        compute(tb);
        if (tb + kBT < tb1) {
            __syncthreads();
            stage(RB);
            __syncthreads();
            if (tb + 3 * kBT < tb1) prefetch(tb + 3 * kBT, RB);
            compute(tb + kBT);
        }
    }

    // ---- dW partial of this token range: combine hi/lo columns, scale by gamma
    const int64_t r = range;
    for (int w = 0; w < kThreads / 64; ++w) {
        __syncthreads();
        if (wv == w) {
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int nb = 0; nb < 3; ++nb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) sW[16 * a + 4 * grp + i][16 * nb + col] = accW[a][nb][i];
        }
        __syncthreads();
        const int wk = w >> 1, wc = 32 * (w & 1);
        for (int q = threadIdx.x; q < 32 * 24; q += kThreads) {
            const int el = q / 24, kap = q % 24;
            const int64_t e = (int64_t)wk * C + c0 + wc + el;
            wpart[(r * N + e) * 24 + kap] = gamma[e] * (sW[el][kap] + sW[el][24 + kap]);
        }
    }
    if (DGAMMA) {
        // lanes with equal grp hold the same channels for 16 different tokens
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float v = accG[a][i];
                v += __shfl_xor(v, 1, 64); v += __shfl_xor(v, 2, 64);
                v += __shfl_xor(v, 4, 64); v += __shfl_xor(v, 8, 64);
                if (col == 0) gpart[r * N + (int64_t)k * C + c0 + ch0 + 16 * a + 4 * grp + i] = v;
            }
    }
}

bool bwd_use_mfma(int64_t T, int n, int64_t C, int dtype)
{
    (void)T;
    return dtype == MHC_BF16 && n == 4 && (C % kCS) == 0;
}

int bwd_mfma_ranges(int64_t T, int64_t C)
{
    const int64_t slices = C / kCS;
    int64_t R = (256 + slices - 1) / slices;   // one resident block per CU, one round
    const int64_t rmax = (T + 31) / 32;
    if (R > rmax) R = rmax;
    if (R < 1) R = 1;
    return (int)R;
}

size_t bwd_mfma_frag_bytes(int64_t T)
{
    const int64_t Tp = (T + 31) / 32 * 32;
    return align256((size_t)Tp * 192) + align256((size_t)Tp * 96);
}

void launch_bwd_mfma(int64_t T, int64_t C, const void* X, const float* gamma, const float* W,
                     const float* rec, int rs, const bf16_t* qf, const bf16_t* qw, const void* G,
                     const void* g, const float* Hres, const float* Hpre, float* dX,
                     float* wpart, float* gpart, bool dgamma, int R, hipStream_t s)
{
    int64_t tpr = (T + R - 1) / R;
    tpr = (tpr + kBT - 1) / kBT * kBT;
    const dim3 grid((unsigned)((C / kCS) * R));
    const dim3 block(kThreads);
#define MHC_BM_ARGS T, C, tpr, (const bf16_t*)X, gamma, W, rec, rs, qf, qw, (const bf16_t*)G, \
                    (const bf16_t*)g, Hres, Hpre, dX, wpart, gpart
    if (G) {
        if (dgamma) hipLaunchKernelGGL((k_bwd_mfma<true, true>), grid, block, 0, s, MHC_BM_ARGS);
        else        hipLaunchKernelGGL((k_bwd_mfma<true, false>), grid, block, 0, s, MHC_BM_ARGS);
    } else {
        if (dgamma) hipLaunchKernelGGL((k_bwd_mfma<false, true>), grid, block, 0, s, MHC_BM_ARGS);
        else        hipLaunchKernelGGL((k_bwd_mfma<false, false>), grid, block, 0, s, MHC_BM_ARGS);
    }
#undef MHC_BM_ARGS
}

}  // namespace mhc
