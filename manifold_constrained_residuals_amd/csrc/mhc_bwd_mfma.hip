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
//   dW: A = x transposed by transposed LDS reads (exact in bf16), B = q/r split hi/lo
//       and stacked along K (the step's 16 tokens as hi, the same 16 as lo), so one
//       MFMA per 16-column tile adds both; accumulated over the block's token range.
// A block works on 128-channel slices of all 4 streams (8 waves) over token ranges:
// one slice and range in the register-staged kernel, a chunk of the slice-major
// (slice, step) sequence in the streaming one.  dW partials, one per slice and range,
// are reduced afterwards in a fixed order.
#include <atomic>

#include "mhc_device.hpp"
#include "mhc_partition.hpp"
#include "mhc_internal.hpp"
#include "../../include/mhc.h"

namespace mhc {

__device__ __forceinline__ uint32_t pk(float a, float b) { return pack_bf16x2(a, b); }

constexpr int kBT = 16;                 // tokens per block step
constexpr int kCS = 128;                // channels per workgroup (256-byte runs of bf16 rows)
static_assert(kCS == bp::kSliceCh && kBT == 16, "the work partition's slice and step sizes");
constexpr int kThreads = 512;           // 8 waves: wave w = stream w / 2, channel half w % 2
constexpr int kRowPad = 136;            // bf16 per LDS row of sX / sG / sg (128 + 8 pad)
constexpr int kScal = 25;               // per-token scalars in LDS: rinv, c2, Hpre[4], Hres[16], pad

// ---------------------------------------------------------------- q fragments
// qf / qw are written by the logit-gradient kernels at n = 4 (mhc_bwd.hip, dz16_tail),
// for T rounded up to 32 tokens (zeros beyond T):
//   qf[t/16][chunk][lane][8]: dy B operand; token t%16 = lane%16, kappa = 8*(lane/16)+j;
//       chunk 0: q_hi, 1: q_lo, 2: q_hi; kappa >= 24 is zero.
//   qw[t/16][nb][lane][8]: dW B operand; column 16*nb + lane%16 of q' = q / r; K index
//       8*(lane/16) + j: q'_hi of token 8*(lane/16) + j for lane/16 < 2, q'_lo of token
//       8*(lane/16 - 2) + j for lane/16 >= 2 (hi and lo stacked along K).

// Transposed read of a 4 x 4 block of bf16 from LDS (ds_read_b64_tr_b16): within each
// group of 16 lanes, lane i receives element m = piece[4 m + i / 4][i % 4], where piece[j]
// is the 8 bytes at lane j's address.
__device__ __forceinline__ u32x2_t lds_read_tr16(const bf16_t* p) {
    typedef short s16x4_t __attribute__((ext_vector_type(4)));
    const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4_t*)(p));
    return __builtin_bit_cast(u32x2_t, v);
}

// ---------------------------------------------------------------- main kernel
// grid (C / 128) * R blocks of 512 threads, one per CU: block -> (channel slice,
// token range [range * tpr, + tpr)), tpr % 16 == 0.  Wave w handles stream k = w / 2
// and channels c0 + 64 (w % 2) + [0, 64): four 16-element MFMA row tiles.  A 128-channel
// slice makes every token row a 256-byte run per stream (the streaming mix of this
// pass runs near 5.1 TB/s with 256-byte runs and 4.6 TB/s with 128-byte runs).
// With OUTBF the direct-term dX is written in bf16 (round to nearest even) instead of
// fp32: a stack hands it on as the dX_out of the layer below.
template <bool DIRECT, bool DGAMMA, bool OUTBF>
__global__ __launch_bounds__(kThreads) void k_bwd_mfma(
    int64_t T, int64_t C, int64_t tpr, const bf16_t* __restrict__ X,
    const float* __restrict__ gamma, const float* __restrict__ W,
    const float* __restrict__ rec, int rs, const bf16_t* __restrict__ qf,
    const bf16_t* __restrict__ qw, const bf16_t* __restrict__ G, const bf16_t* __restrict__ g,
    const float* __restrict__ Hres, const float* __restrict__ Hpre, float* __restrict__ dX,
    float* __restrict__ wpart, float* __restrict__ gpart)
{
    __shared__ __attribute__((aligned(16))) bf16_t sX[4][kBT][kRowPad];    // [k][t][c]
    __shared__ __attribute__((aligned(16))) bf16_t sG[4][kBT][kRowPad];    // [i][t][c]
    __shared__ __attribute__((aligned(16))) bf16_t sg[kBT][kRowPad];       // [t][c]
    __shared__ float sS[kBT][kScal];
    __shared__ __attribute__((aligned(16))) u32x4_t sQ[3][64];             // qf tiles
    __shared__ __attribute__((aligned(16))) u32x4_t sQW[2][64];            // qw tiles
    __shared__ float sW[64][33];                                           // dW combine

    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int k = wv >> 1, ch0 = 64 * (wv & 1);                // stream, first local channel
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

    // dy A operand: W rows of this wave's 64 elements split hi/lo (K chunks hi, hi, lo).
    // Without the dgamma output, gamma is folded into the rows (dy then carries it).
    u32x4_t aW[4][2];
    float gm[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        const int64_t e = (int64_t)k * C + c0 + ch0 + 16 * a + col;
        const float ge = DGAMMA ? 1.f : gamma[e];
        float w[8], wh[8], wl[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int kk = 8 * grp + j;
            // unconditional load (a clamped column), then the select: a load under a
            // per-lane condition is issued alone and waited for before the next one
            const float wv = W[e * 24 + (kk < 24 ? kk : 23)];
            w[j] = kk < 24 ? wv * ge : 0.f;
            wh[j] = (float)(__bf16)w[j];
            wl[j] = (float)(__bf16)(w[j] - wh[j]);
        }
        aW[a][0] = u32x4_t{pk(wh[0], wh[1]), pk(wh[2], wh[3]), pk(wh[4], wh[5]), pk(wh[6], wh[7])};
        aW[a][1] = u32x4_t{pk(wl[0], wl[1]), pk(wl[2], wl[3]), pk(wl[4], wl[5]), pk(wl[6], wl[7])};
#pragma unroll
        for (int i = 0; i < 4; ++i)
            gm[a][i] = DGAMMA ? gamma[(int64_t)k * C + c0 + ch0 + 16 * a + 4 * grp + i] : 1.f;
    }

    f32x4_t accW[4][2];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) accW[a][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float accG[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int i = 0; i < 4; ++i) accG[a][i] = 0.f;

    // Staging of one 16-token step.  Thread: stream sk = tid / 128, token st =
    // (tid / 8) % 16, channels sc .. sc + 15 with sc = 16 (tid % 8), of X and G; threads
    // < 256 load g (token tid / 16, channels 8 (tid % 16) ..); threads < 192 one qf tile
    // lane, threads 192 .. 319 one qw tile lane; threads < 352 one per-token scalar.
    // The next steps' data is loaded into registers while the current step computes,
    // then written to LDS after a barrier.
    struct Regs {
        u32x4_t pX[2], pG[2], pg, pQ;
        float pS;
    };
    Regs RA, RB;
    const int sk = threadIdx.x >> 7, st = (threadIdx.x >> 3) & 15, sc = (threadIdx.x & 7) * 16;
    auto prefetch = [&](int64_t tb, Regs& R) {
        const int nb_t = (int)((tb1 - tb) < kBT ? (tb1 - tb) : kBT);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            R.pX[h] = u32x4_t{0u, 0u, 0u, 0u};
            R.pG[h] = u32x4_t{0u, 0u, 0u, 0u};
        }
        if (st < nb_t) {
            const int64_t base = ((tb + st) * 4 + sk) * C + c0 + sc;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                R.pX[h] = *reinterpret_cast<const u32x4_t*>(X + base + 8 * h);
                if (DIRECT) R.pG[h] = *reinterpret_cast<const u32x4_t*>(G + base + 8 * h);
            }
        }
        R.pg = u32x4_t{0u, 0u, 0u, 0u};
        if (DIRECT && threadIdx.x < 256) {
            const int t = threadIdx.x >> 4, cc = (threadIdx.x & 15) * 8;
            if (t < nb_t) R.pg = *reinterpret_cast<const u32x4_t*>(g + (tb + t) * C + c0 + cc);
        }
        R.pQ = u32x4_t{0u, 0u, 0u, 0u};
        const int64_t qt = tb >> 4;
        if (threadIdx.x < 192) {
            const int tile = threadIdx.x >> 6, ln = threadIdx.x & 63;
            R.pQ = *reinterpret_cast<const u32x4_t*>(qf + ((qt * 3 + tile) * 64 + ln) * 8);
        } else if (threadIdx.x < 320) {
            const int q = threadIdx.x - 192, tile = q >> 6, ln = q & 63;
            R.pQ = *reinterpret_cast<const u32x4_t*>(qw + ((qt * 2 + tile) * 64 + ln) * 8);
        }
        R.pS = 0.f;
        if (threadIdx.x < kBT * 22) {
            const int t = threadIdx.x / 22, j = threadIdx.x % 22;
            if (t < nb_t) {
                const int64_t tt = tb + t;
                if (j < 2) R.pS = rec[tt * rs + 24 + j];
                else if (DIRECT && j < 6) R.pS = Hpre[tt * 4 + (j - 2)];
                else if (DIRECT) R.pS = Hres[tt * 16 + (j - 6)];
            }
        }
    };
    auto stage = [&](const Regs& R) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            *reinterpret_cast<u32x4_t*>(&sX[sk][st][sc + 8 * h]) = R.pX[h];
            if (DIRECT) *reinterpret_cast<u32x4_t*>(&sG[sk][st][sc + 8 * h]) = R.pG[h];
        }
        if (DIRECT && threadIdx.x < 256)
            *reinterpret_cast<u32x4_t*>(&sg[threadIdx.x >> 4][(threadIdx.x & 15) * 8]) = R.pg;
        if (threadIdx.x < 192) {
            sQ[threadIdx.x >> 6][threadIdx.x & 63] = R.pQ;
        } else if (threadIdx.x < 320) {
            const int q = threadIdx.x - 192;
            sQW[q >> 6][q & 63] = R.pQ;
        }
        if (threadIdx.x < kBT * 22) sS[threadIdx.x / 22][threadIdx.x % 22] = R.pS;
    };

    auto compute = [&](int64_t tb) {
        const int nb_t = (int)((tb1 - tb) < kBT ? (tb1 - tb) : kBT);
        // ---- dy = W q on MFMA, then the element gradient
        u32x4_t bq[3];
#pragma unroll
        for (int ch = 0; ch < 3; ++ch) bq[ch] = sQ[ch][lane];
        const int t = col;                 // token of this lane within the step
        const float rinv = sS[t][0], c2 = sS[t][1];
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            f32x4_t dy = f32x4_t{0.f, 0.f, 0.f, 0.f};
            dy = mfma16(aW[a][0], bq[0], dy);
            dy = mfma16(aW[a][0], bq[1], dy);
            dy = mfma16(aW[a][1], bq[2], dy);
            const int cl = ch0 + 16 * a + 4 * grp;     // first local channel of this lane
            const u32x2_t xv = *reinterpret_cast<const u32x2_t*>(&sX[k][t][cl]);
            const float x[4] = {bf16_lo(xv.x), bf16_hi(xv.x), bf16_lo(xv.y), bf16_hi(xv.y)};
            float o[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = (DGAMMA ? gm[a][i] * dy[i] : dy[i]) * rinv - x[i] * c2;
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
                    if (OUTBF)
                        *reinterpret_cast<u32x2_t*>(reinterpret_cast<bf16_t*>(dX) +
                                                    (((tb + t) * 4 + k) * C + c0 + cl)) =
                            u32x2_t{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
                    else
                        *reinterpret_cast<float4*>(dst) = make_float4(o[0], o[1], o[2], o[3]);
                } else if (dX) {
                    float4 d = *reinterpret_cast<float4*>(dst);
                    d.x += o[0]; d.y += o[1]; d.z += o[2]; d.w += o[3];
                    *reinterpret_cast<float4*>(dst) = d;
                }
            }
        }

        // ---- dW += x^T (q'_hi + q'_lo) on MFMA: K = the 16 tokens of this step, twice.
        // The A operand (x transposed: 8 tokens of one element per lane) comes from two
        // transposed LDS reads of 4 tokens each.
        u32x4_t bw[2];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) bw[nb] = sQW[nb][lane];
        const int t0 = 8 * (grp & 1) + (col >> 2), e4 = 4 * (col & 3);
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const int e0 = ch0 + 16 * a;
            const u32x2_t r0 = lds_read_tr16(&sX[k][t0][e0 + e4]);
            const u32x2_t r1 = lds_read_tr16(&sX[k][t0 + 4][e0 + e4]);
            const u32x4_t ax = u32x4_t{r0.x, r0.y, r1.x, r1.y};
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) accW[a][nb] = mfma16(ax, bw[nb], accW[a][nb]);
        }
    };

    // Two register sets: while step i computes, the loads of steps i + 1 and i + 2
    // are in flight.
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

    // ---- dW partial of this token range, scaled by gamma
    const int64_t r = range;
    for (int w = 0; w < kThreads / 64; ++w) {
        __syncthreads();
        if (wv == w) {
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) sW[16 * a + 4 * grp + i][16 * nb + col] = accW[a][nb][i];
        }
        __syncthreads();
        const int wk = w >> 1, wc = 64 * (w & 1);
        for (int q = threadIdx.x; q < 64 * 24; q += kThreads) {
            const int el = q / 24, kap = q % 24;
            const int64_t e = (int64_t)wk * C + c0 + wc + el;
            wpart[(r * N + e) * 24 + kap] = gamma[e] * sW[el][kap];
        }
    }
    if (DGAMMA) {
        // lanes with equal grp hold the same channels for 16 different tokens
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float v = accG[a][i];
                v += __shfl_xor(v, 1, 64); v += __shfl_xor(v, 2, 64);
                v += __shfl_xor(v, 4, 64); v += __shfl_xor(v, 8, 64);
                if (col == 0) gpart[r * N + (int64_t)k * C + c0 + ch0 + 16 * a + 4 * grp + i] = v;
            }
    }
}

// ---------------------------------------------------------------- streaming variant
// The DIRECT path with every input of a 16-token step moved by direct-to-LDS loads
// into a ring of kD step slots.  The register-prefetch kernel above stages its loads
// through registers, so each block barrier waits for every load in flight (and for
// the dX stores, which share the counter): one step is in flight.  Here no load has
// a register destination, so the only waits on the loads are explicit counts (which
// include the wave's own dX stores), and the per-step barrier is a bare s_barrier:
// two steps stay in flight while one computes.
//
// Slot layout: X [4 streams][16 tokens] rows of 128 channels (256 bytes), G likewise,
// du [16] rows, qf chunks 0 and 1 (2 KiB of a 3 KiB area), the qw tiles (2 KiB) and 24
// scalars per token (r^-1, c2, H_pre[4], H_res[16], two spare).  A row keeps its 16-byte
// chunk j at position j ^ row, so a column read over the 16 rows of a stream hits 16
// different bank groups.  Rows move four to a 16-byte-per-lane load.

namespace dm {
constexpr int kD = 3;
constexpr int OX = 0, OG = 16384, Og = 32768, OQ = 36864, OQW = OQ + 3072, OS = OQW + 2048;
constexpr int SLOT = OS + kBT * 24 * 4;
static_assert(kD * SLOT >= (kThreads / 64) * 64 * 25 * 4, "the dW combine areas fit in the ring");
constexpr int kGroups = (64 + 64 + 16) / 4;           // 4-row groups: X, G, du
constexpr int kPieces = 2 + 2 + 6;                    // qf chunks 0-1, qw tiles, scalar pieces
static_assert(kPieces > 8 && kPieces <= 16, "every wave loads one or two pieces");
constexpr int kStores = 4;                            // dX stores per wave and step
}  // namespace dm

template <bool DGAMMA, bool OUTBF>
__global__ __launch_bounds__(kThreads) void k_bwd_mfma_dma(
    int64_t T, int64_t C, int64_t nslot, const BwdChunkTable tab, const bf16_t* __restrict__ X,
    const float* __restrict__ gamma, const float* __restrict__ W,
    const float* __restrict__ rec, int rs, const bf16_t* __restrict__ qf,
    const bf16_t* __restrict__ qw, const bf16_t* __restrict__ G, const bf16_t* __restrict__ g,
    const float* __restrict__ Hres, const float* __restrict__ Hpre, float* __restrict__ dX,
    float* __restrict__ wpart, float* __restrict__ gpart)
{
    using namespace dm;
    extern __shared__ __attribute__((aligned(16))) unsigned char ring[];     // [kD][SLOT]
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int wvu = __builtin_amdgcn_readfirstlane(wv);       // the same, in a scalar register
    const int k = wv >> 1, ch0 = 64 * (wv & 1);
    const int col = lane & 15, grp = lane >> 4;
    const int64_t N = 4 * C;
    // Blocks are dealt round-robin to the 8 XCDs; with NB % 8 == 0, XCD x takes chunks
    // [x NB / 8, (x + 1) NB / 8), a contiguous band of slices, so the blocks resident on
    // one XCD read long runs of every token row.
    const int64_t U = (T + kBT - 1) / kBT;
    const int NB = gridDim.x, b = blockIdx.x;
    const int ci = (NB & 7) == 0 ? (b & 7) * (NB >> 3) + (b >> 3) : b;
    const int64_t send = tab.s0[ci + 1], uend = tab.u0[ci + 1];
    int64_t r = tab.r0[ci];                                       // partial slot of the piece
    int64_t us = tab.u0[ci];
#pragma unroll 1
    for (int64_t slice = tab.s0[ci]; slice < send || (slice == send && us < uend); ++slice, us = 0) {
        const int64_t ue = slice == send ? uend : U;
        const int64_t c0 = slice * kCS;
        const int64_t tb0 = us * kBT;
        const int64_t tb1 = ue * kBT < T ? ue * kBT : T;

        u32x4_t aW[4][2];
        float gm[4][4];
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const int64_t e = (int64_t)k * C + c0 + ch0 + 16 * a + col;
            const float ge = DGAMMA ? 1.f : gamma[e];
            float w[8], wh[8], wl[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int kk = 8 * grp + j;
                // unconditional load (a clamped column), then the select: a load under a
                // per-lane condition is issued alone and waited for before the next one
                const float wv = W[e * 24 + (kk < 24 ? kk : 23)];
                w[j] = kk < 24 ? wv * ge : 0.f;
                wh[j] = (float)(__bf16)w[j];
                wl[j] = (float)(__bf16)(w[j] - wh[j]);
            }
            aW[a][0] = u32x4_t{pk(wh[0], wh[1]), pk(wh[2], wh[3]), pk(wh[4], wh[5]), pk(wh[6], wh[7])};
            aW[a][1] = u32x4_t{pk(wl[0], wl[1]), pk(wl[2], wl[3]), pk(wl[4], wl[5]), pk(wl[6], wl[7])};
#pragma unroll
            for (int i = 0; i < 4; ++i)
                gm[a][i] = DGAMMA ? gamma[(int64_t)k * C + c0 + ch0 + 16 * a + 4 * grp + i] : 1.f;
        }
        f32x4_t accW[4][2];
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) accW[a][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        float accG[4][4];
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int i = 0; i < 4; ++i) accG[a][i] = 0.f;

        typedef __attribute__((address_space(3))) void* lds_ptr;
        const int64_t nsteps = tb1 > tb0 ? (tb1 - tb0 + kBT - 1) / kBT : 0;
        // The wave's pieces of step si (block-uniform si): 4-row groups w, w + 8, ... of the
        // list [X rows (stream, token) 0-63, G rows 64-127, du rows 128-143], then pieces w
        // and (waves 0, 1) w + 8 of [qf chunks 0-1, qw tiles 2-3, scalar pieces 4-9].  Rows
        // past the range load a valid row of it instead (zeroed below for x; the rest only
        // feeds unstored dX).
        const uint32_t lane16 = 16u * (uint32_t)lane;
        const int lrow = lane >> 4, lpos = lane & 15;
        auto issue = [&](int64_t si) {
            const int64_t tb = tb0 + si * kBT;
            unsigned char* slot = ring + (int)(si % kD) * SLOT;
#pragma unroll 1
            for (int r = wvu; r < kGroups; r += kThreads / 64) {
                const int t = 4 * (r & 3) + lrow;
                int64_t tt = tb + t;
                if (tt >= tb1) tt = tb;
                const bf16_t* src;
                int off;
                if (r < 32) {
                    const int kk = (r & 15) >> 2;
                    src = (r < 16 ? X : G) + (tt * 4 + kk) * C;
                    off = (r < 16 ? OX : OG) + (kk * 16 + 4 * (r & 3)) * 256;
                } else {
                    src = g + tt * C;
                    off = Og + 4 * (r - 32) * 256;
                }
                __builtin_amdgcn_global_load_lds(src + c0 + 8 * (lpos ^ t), (lds_ptr)(slot + off), 16, 0, 0);
            }
            const int64_t qt = tb >> 4;
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) {
                const int j = wvu + 8 * pp;                    // wave-uniform
                if (j >= kPieces) continue;
                if (j < 4) {
                    // qf chunks 0 (q_hi) and 1 (q_lo); chunk 2 repeats q_hi and is not loaded
                    const bf16_t* tile = j < 2 ? qf + (qt * 3 + j) * 512 : qw + (qt * 2 + (j - 2)) * 512;
                    const int off = j < 2 ? OQ + j * 1024 : OQW + (j - 2) * 1024;
                    __builtin_amdgcn_global_load_lds(reinterpret_cast<const unsigned char*>(tile) + lane16,
                                                     (lds_ptr)(slot + off), 16, 0, 0);
                } else {
                    const int e = 64 * (j - 4) + lane, t = e / 24, q = e % 24;
                    int64_t tt = tb + t;
                    if (tt >= tb1) tt = tb;
                    const float* src = q < 2 ? rec + tt * rs + 24 + q
                                     : q < 6 ? Hpre + tt * 4 + (q - 2)
                                     : q < 22 ? Hres + tt * 16 + (q - 6) : rec + tt * rs + 24;
                    __builtin_amdgcn_global_load_lds(src, (lds_ptr)(slot + OS + 256 * (j - 4)), 4, 0, 0);
                }
            }
        };
        // byte offset of channels cl .. cl + 3 (cl % 4 == 0) within row `row` of a block
        auto pos = [&](int row, int cl) { return row * 256 + ((((cl >> 3) ^ row) & 15) << 4) + ((cl & 7) << 1); };

        auto compute = [&](int64_t si) {
            const int64_t tb = tb0 + si * kBT;
            const int nb_t = (int)((tb1 - tb) < kBT ? (tb1 - tb) : kBT);
            const unsigned char* slot = ring + (int)(si % kD) * SLOT;
            const u32x4_t* sQ = reinterpret_cast<const u32x4_t*>(slot + OQ);
            const u32x4_t* sQW = reinterpret_cast<const u32x4_t*>(slot + OQW);
            const float* sS = reinterpret_cast<const float*>(slot + OS);
            u32x4_t bq[2];
#pragma unroll
            for (int ch = 0; ch < 2; ++ch) bq[ch] = sQ[ch * 64 + lane];
            const int t = col;
            const float rinv = sS[t * 24], c2 = sS[t * 24 + 1];
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                f32x4_t dy = f32x4_t{0.f, 0.f, 0.f, 0.f};
                dy = mfma16(aW[a][0], bq[0], dy);
                dy = mfma16(aW[a][0], bq[1], dy);
                dy = mfma16(aW[a][1], bq[0], dy);              // W_lo q_hi
                const int cl = ch0 + 16 * a + 4 * grp;
                const int pa = pos(t, cl);
                const u32x2_t xv = *reinterpret_cast<const u32x2_t*>(slot + OX + k * 4096 + pa);
                const float x[4] = {bf16_lo(xv.x), bf16_hi(xv.x), bf16_lo(xv.y), bf16_hi(xv.y)};
                float o[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) o[i] = (DGAMMA ? gm[a][i] * dy[i] : dy[i]) * rinv - x[i] * c2;
                if (DGAMMA) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) accG[a][i] += x[i] * dy[i] * rinv;
                }
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                    const float h = sS[t * 24 + 6 + ii * 4 + k];
                    const u32x2_t gv = *reinterpret_cast<const u32x2_t*>(slot + OG + ii * 4096 + pa);
                    o[0] += h * bf16_lo(gv.x); o[1] += h * bf16_hi(gv.x);
                    o[2] += h * bf16_lo(gv.y); o[3] += h * bf16_hi(gv.y);
                }
                const float hp = sS[t * 24 + 2 + k];
                const u32x2_t uv = *reinterpret_cast<const u32x2_t*>(slot + Og + pa);
                o[0] += hp * bf16_lo(uv.x); o[1] += hp * bf16_hi(uv.x);
                o[2] += hp * bf16_lo(uv.y); o[3] += hp * bf16_hi(uv.y);
                if (t < nb_t) {
                    const int64_t di = ((tb + t) * 4 + k) * C + c0 + cl;
                    if (OUTBF)
                        *reinterpret_cast<u32x2_t*>(reinterpret_cast<bf16_t*>(dX) + di) =
                            u32x2_t{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
                    else
                        *reinterpret_cast<float4*>(dX + di) = make_float4(o[0], o[1], o[2], o[3]);
                }
            }
            u32x4_t bw[2];
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) bw[nb] = sQW[nb * 64 + lane];
            const int t0 = 8 * (grp & 1) + (col >> 2), e4 = 4 * (col & 3);
            // The eight transposed reads (rows t0 and t0 + 4, four 16-channel tiles) in one
            // asm block that waits for them itself: as builtins the compiler would put a full
            // vector-memory wait in front of them (it cannot tell them apart from the ring's
            // incoming loads), draining the steps in flight.  Their rows were published by
            // the step barrier.
            const uint32_t xb = (uint32_t)(uintptr_t)(lds_ptr)(slot + OX + k * 4096);
            uint32_t ad[8];
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                ad[2 * a] = xb + pos(t0, ch0 + 16 * a + e4);
                ad[2 * a + 1] = xb + pos(t0 + 4, ch0 + 16 * a + e4);
            }
            u32x2_t r[8];
            asm volatile(
                "ds_read_b64_tr_b16 %0, %8\n\t"
                "ds_read_b64_tr_b16 %1, %9\n\t"
                "ds_read_b64_tr_b16 %2, %10\n\t"
                "ds_read_b64_tr_b16 %3, %11\n\t"
                "ds_read_b64_tr_b16 %4, %12\n\t"
                "ds_read_b64_tr_b16 %5, %13\n\t"
                "ds_read_b64_tr_b16 %6, %14\n\t"
                "ds_read_b64_tr_b16 %7, %15\n\t"
                "s_waitcnt lgkmcnt(0)"
                : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]),
                  "=&v"(r[6]), "=&v"(r[7])
                : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5]), "v"(ad[6]),
                  "v"(ad[7])
                : "memory");
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const u32x4_t ax = u32x4_t{r[2 * a].x, r[2 * a].y, r[2 * a + 1].x, r[2 * a + 1].y};
#pragma unroll
                for (int nb = 0; nb < 2; ++nb) accW[a][nb] = mfma16(ax, bw[nb], accW[a][nb]);
            }
        };

        // loads this wave issues per step: its 4-row groups and two tile/scalar pieces
        const int nload = (kGroups - wvu + kThreads / 64 - 1) / (kThreads / 64) + (wvu + 8 < kPieces ? 2 : 1);
        // the W rows are in registers before the ring's first loads go out
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_sched_barrier(0);
        if (nsteps > 0) issue(0);
        if (nsteps > 1) issue(1);
        for (int64_t si = 0; si < nsteps; ++si) {
            // this wave's pieces of step si have landed once at most the operations it
            // issued after them are outstanding: the loads of later steps and its stores
            int after;
            if (si == 0)      after = nsteps > 1 ? nload : 0;
            else if (si == 1) after = (nsteps > 2 ? nload : 0) + kStores;
            else              after = kStores + (si + 1 < nsteps ? nload : 0) + kStores;
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            wait_vmcnt(after);
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            const int64_t tb = tb0 + si * kBT;
            const int nb_t = (int)((tb1 - tb) < kBT ? (tb1 - tb) : kBT);
            if (nb_t < kBT) {
                // x rows past the range must add nothing to dW (or dgamma).  Each lane clears
                // the 16 bytes its own load of such a row brought in (a copy of a valid row),
                // after the wait above: no other wave's load lands on them later.  The wave's
                // x groups are w and w + 8 of the list in issue().
                unsigned char* slot = ring + (int)(si % kD) * SLOT;
#pragma unroll
                for (int rr = 0; rr < 2; ++rr) {
                    const int r = wvu + 8 * rr, t = 4 * (r & 3) + lrow;
                    if (t >= nb_t)
                        *reinterpret_cast<u32x4_t*>(slot + OX + (((r >> 2) & 3) * 16 + 4 * (r & 3)) * 256 +
                                                    lane16) = u32x4_t{0u, 0u, 0u, 0u};
                }
            }
            // LDS writes done, then every wave's pieces of step si are in and every wave is
            // past step si - 1, whose slot the next issue reuses; the loads stay in flight
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            __builtin_amdgcn_s_waitcnt(0xC07F);          // lgkmcnt(0) only
            __builtin_amdgcn_s_barrier();
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            if (si + 2 < nsteps) issue(si + 2);
            // the counts above assume every load of a step is issued before its stores
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            __builtin_amdgcn_sched_barrier(0);
            compute(si);
            __builtin_amdgcn_sched_barrier(0);
        }

        // ---- dW partial of this piece, scaled by gamma.  Each wave turns its 64 x 24
        // tile into whole rows through its own LDS area (the ring is free once every wave is
        // past the loop) and writes them as 16-byte pieces: 6 per lane, no block-wide rounds.
        const int64_t e0 = (int64_t)k * C + c0 + ch0;               // the wave's first element
        float ge[6];
#pragma unroll
        for (int j = 0; j < 6; ++j) ge[j] = gamma[e0 + (4 * (lane + 64 * j)) / 24];
        __syncthreads();
        float (*sW)[25] = reinterpret_cast<float (*)[25]>(ring + wv * (64 * 25 * 4));
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (16 * nb + col < 24) sW[16 * a + 4 * grp + i][16 * nb + col] = accW[a][nb][i];
        __syncthreads();
        {
            f32x4_t* dst = reinterpret_cast<f32x4_t*>(wpart + (r * N + e0) * 24);
#pragma unroll
            for (int j = 0; j < 6; ++j) {
                const int f = 4 * (lane + 64 * j), el = f / 24, kap = f % 24;
                dst[lane + 64 * j] = f32x4_t{ge[j] * sW[el][kap], ge[j] * sW[el][kap + 1],
                                             ge[j] * sW[el][kap + 2], ge[j] * sW[el][kap + 3]};
            }
        }
        if (DGAMMA) {
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float v = accG[a][i];
                    v += __shfl_xor(v, 1, 64); v += __shfl_xor(v, 2, 64);
                    v += __shfl_xor(v, 4, 64); v += __shfl_xor(v, 8, 64);
                    if (col == 0) gpart[r * N + (int64_t)k * C + c0 + ch0 + 16 * a + 4 * grp + i] = v;
                }
        }
        if (ue == U) {
            // the slice's last piece: its unused slots add zero in the reduction
            for (int64_t q = r + 1; q < nslot; ++q) {
                f32x4_t* dst = reinterpret_cast<f32x4_t*>(wpart + (q * N + e0) * 24);
#pragma unroll
                for (int j = 0; j < 6; ++j) dst[lane + 64 * j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                if (DGAMMA) gpart[q * N + e0 + lane] = 0.f;
            }
        }
        r = 0;
        // every wave is done with its combine area before the next piece's loads reuse it
        __syncthreads();
    }
}

bool bwd_use_mfma(int64_t T, int n, int64_t C, int dtype)
{
    // the chunk table holds slice indices in 16 bits and step indices in 32
    return dtype == MHC_BF16 && n == 4 && (C % kCS) == 0 && C / kCS < 65536 &&
           (T + kBT - 1) / kBT < ((int64_t)1 << 31) && force_path() != kPathVector;
}

// token ranges per slice of the register-staged kernel (the variant without direct terms)
static int bwd_mfma_token_ranges(int64_t T, int64_t C)
{
    const int64_t slices = C / kCS;
    int64_t R = (256 + slices - 1) / slices;   // one resident block per CU, one round
    const int64_t rmax = (T + kBT - 1) / kBT;
    if (R > rmax) R = rmax;
    if (R < 1) R = 1;
    return (int)R;
}

int bwd_mfma_ranges(int64_t T, int64_t C)
{
    const int a = bwd_mfma_token_ranges(T, C), b = bwd_chunks(T, C).slots;
    return a > b ? a : b;
}

size_t bwd_mfma_frag_bytes(int64_t T)
{
    const int64_t Tp = (T + 31) / 32 * 32;
    return align256((size_t)Tp * 192) + align256((size_t)Tp * 128);
}

int launch_bwd_mfma(int64_t T, int64_t C, const void* X, const float* gamma, const float* W,
                    const float* rec, int rs, const bf16_t* qf, const bf16_t* qw, const void* G,
                    const void* g, const float* Hres, const float* Hpre, float* dX,
                    float* wpart, float* gpart, bool dgamma, bool dx_bf16, hipStream_t s)
{
    const dim3 block(kThreads);
    if (G) {
        const BwdChunks ch = bwd_chunks(T, C);
        const dim3 grid((unsigned)ch.NB);
        const int64_t nslot = ch.slots;
#define MHC_BM_ARGS T, C, nslot, ch.tab, (const bf16_t*)X, gamma, W, rec, rs, qf, qw, (const bf16_t*)G, \
                    (const bf16_t*)g, Hres, Hpre, dX, wpart, gpart
        // the streaming variant; its ring needs more than the default 64 KiB of LDS
        const size_t smem = (size_t)dm::kD * dm::SLOT;
        // once per device; callers on several host threads may get here together (the
        // attribute calls are idempotent, the flags atomic)
        static std::atomic<bool> attr_set[64] = {};
        int dev = 0;
        (void)hipGetDevice(&dev);
        if (dev < 0 || dev >= 64 || !attr_set[dev].load(std::memory_order_acquire)) {
            const void* fns[4] = {reinterpret_cast<const void*>(&k_bwd_mfma_dma<true, true>),
                                  reinterpret_cast<const void*>(&k_bwd_mfma_dma<true, false>),
                                  reinterpret_cast<const void*>(&k_bwd_mfma_dma<false, true>),
                                  reinterpret_cast<const void*>(&k_bwd_mfma_dma<false, false>)};
            for (const void* f : fns)
                (void)hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
            if (dev >= 0 && dev < 64) attr_set[dev].store(true, std::memory_order_release);
        }
        if (dgamma && dx_bf16) hipLaunchKernelGGL((k_bwd_mfma_dma<true, true>), grid, block, smem, s, MHC_BM_ARGS);
        else if (dgamma)       hipLaunchKernelGGL((k_bwd_mfma_dma<true, false>), grid, block, smem, s, MHC_BM_ARGS);
        else if (dx_bf16)      hipLaunchKernelGGL((k_bwd_mfma_dma<false, true>), grid, block, smem, s, MHC_BM_ARGS);
        else                   hipLaunchKernelGGL((k_bwd_mfma_dma<false, false>), grid, block, smem, s, MHC_BM_ARGS);
#undef MHC_BM_ARGS
        return ch.slots;
    }
    const int R = bwd_mfma_token_ranges(T, C);
    int64_t tpr = (T + R - 1) / R;
    tpr = (tpr + kBT - 1) / kBT * kBT;
    const dim3 grid((unsigned)((C / kCS) * R));
#define MHC_BM_ARGS T, C, tpr, (const bf16_t*)X, gamma, W, rec, rs, qf, qw, (const bf16_t*)G, \
                    (const bf16_t*)g, Hres, Hpre, dX, wpart, gpart
    if (dgamma) hipLaunchKernelGGL((k_bwd_mfma<false, true, false>), grid, block, 0, s, MHC_BM_ARGS);
    else        hipLaunchKernelGGL((k_bwd_mfma<false, false, false>), grid, block, 0, s, MHC_BM_ARGS);
#undef MHC_BM_ARGS
    return R;
}

}  // namespace mhc
