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
//   proj = p / r (optional: the unscaled normalised projection, for the scales' gradient).
template <int NS>
__device__ __forceinline__ void coeff_epilogue(int64_t t, const float (&p)[NS * NS + 2 * NS],
                                               float sumsq, int64_t N, float eps,
                                               const float* __restrict__ bias, float a0,
                                               float a1, float a2, float* __restrict__ z,
                                               float* __restrict__ rms, float* __restrict__ Hpre,
                                               float* __restrict__ Hpost, float* __restrict__ proj)
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
        if (proj) proj[t * K + k] = p[k] * rinv;
    }
    if (rms) rms[t] = r;
#pragma unroll
    for (int k = 0; k < NS; ++k) {
        if (Hpre) Hpre[t * NS + k] = sigmoidf(zz[k]);
        if (Hpost) Hpost[t * NS + k] = sigmoidf(zz[NS + k]);
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
    float* __restrict__ Hpre, float* __restrict__ Hpost, float* __restrict__ proj)
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
                           Hpost, proj);
    }
}


// ---------------------------------------------------------------- coefficients, MFMA path
// bf16 storage, n = 4 (K = 24).  The projection is a skinny GEMM [T x N] x [N x 24].
// X is exact as a bf16 MFMA operand; W' = gamma (.) W is split into three bf16 terms
// (hi + mid + lo, the fp32 value's 24 significant bits), giving 72 B-columns padded to
// five 16-wide MFMA tiles (wsplit3).  The split is written once per call, in MFMA
// fragment order, into the workspace:
//   Wp[s][nb][h][lane][j], s = 64-element step of the flattened axis, nb = column
//   tile, h = which 32-element MFMA of the step, lane = MFMA lane, j = 8 values;
//   element k = 64 s + 16 (lane / 16) + 8 h + j, column 16 nb + lane % 16.
// A lane therefore reads 32 contiguous bytes of one token row per step, and the
// A and B operands pair the same k.
constexpr int kWFrag = kWTiles * 2 * 64;     // 16-byte W' fragments per step
constexpr int kWpStep = kWFrag * 8;          // bf16 values of Wp per 64-element step

// With cs > 0 the flattened axis is taken member by member: member m = step / (4 cs / 64)
// owns channels [m cs, (m + 1) cs) of the 4 streams, walked stream-major, so step s of
// the listing above covers member-local elements l = 64 s' + ..., row k C + m cs + l % cs
// with k = l / cs (s' = step within the member).
__global__ __launch_bounds__(256) void k_wsplit(int64_t N, int64_t nsteps, int64_t C, int64_t cs,
                                                const float* __restrict__ gamma,
                                                const float* __restrict__ W,
                                                bf16_t* __restrict__ Wp)
{
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= nsteps * kWFrag) return;
    const int64_t s = idx / kWFrag;
    const int r = (int)(idx - s * kWFrag);
    const int nb = r >> 7, h = (r >> 6) & 1, lane = r & 63;
    const int col = nb * 16 + (lane & 15);
    const int kc = wsplit_logit(col), term = wsplit_term(col);
    const int64_t spm = cs > 0 ? (4 * cs) / 64 : 1;       // steps per member
    const int64_t m = cs > 0 ? s / spm : 0, sl = cs > 0 ? s - m * spm : s;
    // the 16 loads first, unconditional (a clamped index), then the splits: loads held
    // behind a per-lane condition or a branch go out one at a time, each waited for
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int64_t l = sl * 64 + 16 * (lane >> 4) + 8 * h + j;
        const int64_t k = cs > 0 ? (l / cs) * C + m * cs + l % cs : l;
        const int64_t kl = k < N ? k : N - 1;
        const float g = gamma[kl], w = W[kl * 24 + kc];
        v[j] = k < N && term < 3 ? g * w : 0.f;
    }
    float o[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = wsplit3(v[j], term < 3 ? term : 0);
    io<bf16_t>::store8(Wp + idx * 8, o);
}

void launch_wsplit(int64_t N, int64_t C, int64_t cs, const float* gamma, const float* W,
                   bf16_t* Wp, hipStream_t s)
{
    const int64_t ns = (N + 63) / 64;
    hipLaunchKernelGGL(k_wsplit, dim3((unsigned)((ns * kWFrag + 255) / 256)), dim3(256), 0, s, N,
                       ns, C, cs, gamma, W, Wp);
}

// Split-K partial projections.  The flattened axis is cut into `splits` ranges of
// whole 64-element steps (blockIdx.y); a block of NW waves covers MT = 16 NW tokens
// of one range, wave w the 16 tokens 16 w .. 16 w + 15 (one MFMA row tile, five
// column tiles).  The range is walked in chunks of CK steps:
//   - W' fragments of a chunk (CK x 10 KiB) are copied into LDS once per block
//     (double-buffered, one chunk ahead) and read by every wave, so W' crosses L2
//     once per MT tokens;
//   - each wave streams its own X rows through a ring of D register buffers, D - 1
//     chunks ahead (a lane reads 32 contiguous bytes per step; 4 lanes cover a
//     128-byte run of a row).
// Sums run in two levels: each chunk's MFMA products accumulate in fp32 (4 MFMAs per
// column tile), the chunk sums in fp64, so that rounding does not grow with the row
// length (the same for the sum of squares).  Partial projections and sums of squares go
// to part[split][t][0..24] (row pitch kPartPitch floats); k_coeffs_finish adds the
// ranges in a fixed order.
constexpr int kPartPitch = 32;         // floats per token row of the partials
constexpr int kCoefNW = 8, kCoefCK = 2, kCoefD = 2;
constexpr int kCoefBlocks = 256;       // target grid: one block per CU
constexpr int kCoefRot = 1;            // chunk rotation per token tile

// The epilogue shared by the split-K projection kernels: the fp64 tile sums of a wave
// (16 tokens x 80 columns, D layout) folded into 24 logits per token, plus the sum of
// squares, through the wave's LDS rows sC[16][25], then written as fp32 partial rows.
__device__ __forceinline__ void part_epilogue(const double (&accd)[kWTiles][4], double ssd,
                                              float (*sC)[25], int lane, int64_t tbase,
                                              int64_t T, float* __restrict__ dst_rows)
{
    const int row = lane & 15, grp = lane >> 4;
    ssd += __shfl_xor(ssd, 16, 64);
    ssd += __shfl_xor(ssd, 32, 64);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        double t[kWTiles];
#pragma unroll
        for (int nb = 0; nb < kWTiles; ++nb) t[nb] = accd[nb][i];
        double f0, f1;
        fold3(t, row, [](double v) { return lane_ror8_d(v); }, f0, f1);
        sC[4 * grp + i][row] = (float)f0;
        if (row < 8) sC[4 * grp + i][16 + row] = (float)f1;
    }
    if (grp == 0) sC[row][24] = (float)ssd;
    __syncthreads();
    if (lane < 16) {
        const int64_t tt = tbase + lane;
        if (tt < T) {
            float* dst = dst_rows + (int64_t)lane * kPartPitch;
            const float* c = sC[lane];
            float o[kPartPitch];
#pragma unroll
            for (int k = 0; k < 25; ++k) o[k] = c[k];
#pragma unroll
            for (int k = 25; k < kPartPitch; ++k) o[k] = 0.f;
#pragma unroll
            for (int k = 0; k < kPartPitch; k += 4)
                *reinterpret_cast<f32x4_t*>(dst + k) = f32x4_t{o[k], o[k + 1], o[k + 2], o[k + 3]};
        }
    }
}

template <int NW, int CK, int D>
__global__ __launch_bounds__(NW * 64) void k_coeffs_part(
    int64_t T, int64_t N, int64_t nsteps, int64_t spr, const bf16_t* __restrict__ X,
    const bf16_t* __restrict__ Wp, float* __restrict__ part)
{
    constexpr int NT = NW * 64;
    constexpr int CHW = CK * kWFrag;                // 16-byte W' fragments per chunk
    constexpr int WPT = (CHW + NT - 1) / NT;        // of them per thread
    __shared__ u32x4_t sW[2][CHW];
    __shared__ float sC[NW][16][25];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int row = lane & 15, grp = lane >> 4;
    const int64_t split = blockIdx.y;
    const int64_t sb = split * spr;
    const int64_t se = (sb + spr) < nsteps ? (sb + spr) : nsteps;
    const int64_t nch = se > sb ? (se - sb + CK - 1) / CK : 0;
    const int64_t t0 = (int64_t)blockIdx.x * (16 * NW);
    const int64_t t = t0 + 16 * wv + row;
    const bool rv = t < T;
    const bf16_t* xrow = X + (rv ? t : t0) * N + 16 * grp;
    const u32x4_t* wsrc = reinterpret_cast<const u32x4_t*>(Wp);
    const u32x4_t zero4 = u32x4_t{0u, 0u, 0u, 0u};

    u32x4_t xr[D][CK][2], wr[WPT];
    auto load_x = [&](int64_t c, u32x4_t (&x)[CK][2]) {
#pragma unroll
        for (int q = 0; q < CK; ++q) {
            const int64_t st = sb + c * CK + q;
            if (rv && st < se && 64 * st + 16 * grp < N) {
                const u32x4_t* src = reinterpret_cast<const u32x4_t*>(xrow + 64 * st);
                x[q][0] = src[0];
                x[q][1] = src[1];
            } else {
                x[q][0] = zero4;
                x[q][1] = zero4;
            }
        }
    };
    auto load_w = [&](int64_t c) {
#pragma unroll
        for (int j = 0; j < WPT; ++j) {
            const int i = threadIdx.x + NT * j;
            const int64_t st = sb + c * CK + i / kWFrag;
            wr[j] = (i < CHW && st < se) ? wsrc[(sb + c * CK) * kWFrag + i] : zero4;
        }
    };
    auto store_w = [&](int buf) {
#pragma unroll
        for (int j = 0; j < WPT; ++j) {
            const int i = threadIdx.x + NT * j;
            if (i < CHW) sW[buf][i] = wr[j];
        }
    };
    double accd[kWTiles][4];
#pragma unroll
    for (int nb = 0; nb < kWTiles; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) accd[nb][i] = 0.0;
    double ssd = 0.0;
    auto compute = [&](int buf, const u32x4_t (&x)[CK][2]) {
        float ssc = 0.f;
        f32x4_t acc[kWTiles];
#pragma unroll
        for (int nb = 0; nb < kWTiles; ++nb) acc[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < CK; ++q) {
            ssc = sumsq8(x[q][0], ssc);
            ssc = sumsq8(x[q][1], ssc);
#pragma unroll
            for (int nb = 0; nb < kWTiles; ++nb) {
                const u32x4_t w0 = sW[buf][(q * kWTiles + nb) * 128 + lane];
                const u32x4_t w1 = sW[buf][(q * kWTiles + nb) * 128 + 64 + lane];
                acc[nb] = mfma16(x[q][0], w0, acc[nb]);
                acc[nb] = mfma16(x[q][1], w1, acc[nb]);
            }
        }
#pragma unroll
        for (int nb = 0; nb < kWTiles; ++nb)
#pragma unroll
            for (int i = 0; i < 4; ++i) accd[nb][i] += (double)acc[nb][i];
        ssd += (double)ssc;
    };

    // Blocks start their walk at different chunks of the range (and wrap), so that
    // at any moment the grid reads many column offsets of the rows at once: rows are
    // 2N bytes apart, and blocks walking in lockstep would keep hitting the same
    // few HBM channels.
    const int64_t rot = nch > 0 ? (int64_t)(blockIdx.x * kCoefRot) % nch : 0;
    auto chunk = [&](int64_t cc) { const int64_t ci = cc + rot; return ci < nch ? ci : ci - nch; };
    if (nch > 0) load_w(chunk(0));
#pragma unroll
    for (int d = 0; d < D - 1; ++d)
        if (d < nch) load_x(chunk(d), xr[d]);
    if (nch > 0) store_w(0);
    __syncthreads();
    for (int64_t c = 0; c < nch; c += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int64_t cc = c + d;                 // block-uniform
            if (cc < nch) {
                if (cc + 1 < nch) load_w(chunk(cc + 1));
                if (cc + D - 1 < nch) load_x(chunk(cc + D - 1), xr[(d + D - 1) % D]);
                compute((int)(cc & 1), xr[d]);
                if (cc + 1 < nch) store_w((int)((cc + 1) & 1));
                __syncthreads();
            }
        }
    }
    part_epilogue(accd, ssd, sC[wv], lane, t0 + 16 * wv, T,
                  part + (split * T + t0 + 16 * wv) * kPartPitch);
}

// Finishing of the split-K projection for one token on 16 lanes (lanes base ..
// base + 15): lane q adds the split partials of values q and q + 16 in split order,
// then forms logits q (za) and, for q < 8, 16 + q (zb), with 1 / r, alpha and the
// bias.  Every caller gets bitwise the same logits for a token.
struct Fin16 {
    float za, zb, r, pa, pb;     // logits q and 16 + q; r; the unscaled p / r of both
};
__device__ __forceinline__ Fin16 finish16(int64_t t, bool valid, int q, int base, int splits,
                                          const float* __restrict__ part, int64_t T, int64_t N,
                                          float eps, const float* __restrict__ bias, float a0,
                                          float a1, float a2)
{
    float pa = 0.f, pb = 0.f;
    if (valid) {
        for (int sp = 0; sp < splits; ++sp) {
            const float* r = part + (sp * T + t) * kPartPitch;
            pa += r[q];
            if (q < 9) pb += r[16 + q];
        }
    }
    const float sq = __shfl(pb, base + 8, 64);              // value 24: the sum of squares
    Fin16 f;
    f.r = sqrtf(sq / (float)N + eps);
    const float rinv = 1.0f / f.r;
    f.za = (q < 4 ? a0 : (q < 8 ? a1 : a2)) * pa * rinv + bias[q];
    f.zb = a2 * pb * rinv + bias[16 + (q & 7)];   // logits 16..23 on lanes 0..7
    f.pa = pa * rinv;
    f.pb = pb * rinv;
    return f;
}

// Finishing pass, 16 tokens per block of 256 threads (token blk * 16 + tid / 16):
// z, r, the gates, and -- when H_res is asked for -- Sinkhorn-Knopp of the res logits
// (lane q holds res entry q; injected logits replace them when given).  Tokens past T
// run on zeros so that every lane of a group takes part in the lane exchanges.
__device__ __forceinline__ void finish_block(int64_t blk, int64_t T, int splits,
                                             const float* __restrict__ part, int64_t N, float eps,
                                             const float* __restrict__ bias, float a0, float a1,
                                             float a2, float* __restrict__ z,
                                             float* __restrict__ rms, float* __restrict__ Hpre,
                                             float* __restrict__ Hpost, int iters,
                                             const float* __restrict__ zres_in,
                                             float* __restrict__ Hres, float* __restrict__ proj)
{
    const int64_t t = blk * 16 + (threadIdx.x >> 4);
    const int q = threadIdx.x & 15;
    const bool valid = t < T;
    const int base = threadIdx.x & ~15;
    const Fin16 f = finish16(t, valid, q, base, splits, part, T, N, eps, bias, a0, a1, a2);
    const float za = f.za, zb = f.zb;
    if (valid) {
        z[t * 24 + q] = za;
        if (q < 8) z[t * 24 + 16 + q] = zb;
        if (q == 0) rms[t] = f.r;
        if (q < 4) Hpre[t * 4 + q] = sigmoidf(za);
        else if (q < 8) Hpost[t * 4 + q - 4] = sigmoidf(za);
        if (proj) {
            proj[t * 24 + q] = f.pa;
            if (q < 8) proj[t * 24 + 16 + q] = f.pb;
        }
    }
    if (Hres) {
        // res entry q is logit 8 + q: lane q + 8's za for q < 8, lane q - 8's zb otherwise
        const float from_a = __shfl(za, base + ((q + 8) & 15), 64);
        const float from_b = __shfl(zb, base + ((q + 8) & 15), 64);
        float zr = q < 8 ? from_a : from_b;
        if (zres_in) zr = valid ? zres_in[t * 16 + q] : 0.f;
        const float h = sinkhorn16_fwd(valid ? zr : 0.f, iters);
        if (valid) Hres[t * 16 + q] = h;
    }
}

__global__ __launch_bounds__(256) void k_coeffs_finish(
    int64_t T, int splits, const float* __restrict__ part, int64_t N, float eps,
    const float* __restrict__ bias, float a0, float a1, float a2, float* __restrict__ z,
    float* __restrict__ rms, float* __restrict__ Hpre, float* __restrict__ Hpost, int iters,
    const float* __restrict__ zres_in, float* __restrict__ Hres, float* __restrict__ proj)
{
    finish_block(blockIdx.x, T, splits, part, N, eps, bias, a0, a1, a2, z, rms, Hpre, Hpost, iters,
                 zres_in, Hres, proj);
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

// n = 4: one token per 16 lanes, entry (i, j) in lane 4 i + j; tokens past T run on
// zeros so that every lane of a group takes part in the lane exchanges.
__global__ __launch_bounds__(256) void k_sinkhorn16(int64_t T, const float* __restrict__ zres,
                                                    int64_t ld, int iters, float* __restrict__ Hres)
{
    const int64_t t = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
    const int q = threadIdx.x & 15;
    const bool valid = t < T;
    const float h = sinkhorn16_fwd(valid ? zres[t * ld + q] : 0.f, iters);
    if (valid) Hres[t * 16 + q] = h;
}

// ---------------------------------------------------------------- pre: u = H_pre X
// One block per token, 16-byte row pieces.
template <typename Tio, int NS>
__device__ __forceinline__ void pre_token(int64_t t, int64_t C, const Tio* __restrict__ X,
                                          const float (&h)[NS], Tio* __restrict__ u)
{
    const Tio* xt = X + t * NS * C;
    // two row pieces in flight per thread before any is used
    for (int64_t c0 = (int64_t)threadIdx.x * 8; c0 < C; c0 += 2 * 256 * 8) {
        float v[2][NS][8];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int64_t c = c0 + q * 256 * 8;
            if (q == 0 || c < C) {
#pragma unroll
                for (int k = 0; k < NS; ++k) io<Tio>::load8(xt + k * C + c, v[q][k]);
            }
        }
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int64_t c = c0 + q * 256 * 8;
            if (q > 0 && c >= C) break;
            // h_0 x_0, then one fused multiply-add per further stream, written out so that
            // every kernel forming u rounds the same way
            float acc[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = h[0] * v[q][0][e];
#pragma unroll
            for (int k = 1; k < NS; ++k)
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[e] = __builtin_fmaf(h[k], v[q][k][e], acc[e]);
            store8_nt(u + t * C + c, acc);
        }
    }
}

template <typename Tio, int NS>
__global__ __launch_bounds__(256) void k_pre(int64_t C, const Tio* __restrict__ X,
                                             const float* __restrict__ Hpre, Tio* __restrict__ u)
{
    const int64_t t = blockIdx.x;
    float h[NS];
#pragma unroll
    for (int k = 0; k < NS; ++k) h[k] = Hpre[t * NS + k];
    pre_token<Tio, NS>(t, C, X, h, u);
}

// The split-K finishing pass and the read map in one launch (bf16, n = 4): blocks
// [0, nsk) finish 16 tokens each (z, r, gates, Sinkhorn: latency-bound), blocks
// nsk + t form token t's H_pre from the same partials with the same arithmetic and
// stream u = H_pre X (HBM-bound); the GPU runs the two kinds side by side.
__global__ __launch_bounds__(256) void k_finish_pre(
    int64_t T, int64_t nsk, int splits, const float* __restrict__ part, int64_t N, int64_t C,
    float eps, const float* __restrict__ bias, float a0, float a1, float a2,
    float* __restrict__ z, float* __restrict__ rms, float* __restrict__ Hpre,
    float* __restrict__ Hpost, int iters, const float* __restrict__ zres_in,
    float* __restrict__ Hres, const bf16_t* __restrict__ X, bf16_t* __restrict__ u,
    float* __restrict__ proj)
{
    if ((int64_t)blockIdx.x < nsk) {
        finish_block(blockIdx.x, T, splits, part, N, eps, bias, a0, a1, a2, z, rms, Hpre, Hpost,
                     iters, zres_in, Hres, proj);
        return;
    }
    __shared__ float sh[4];
    const int64_t t = (int64_t)blockIdx.x - nsk;
    if (threadIdx.x < 16) {
        const Fin16 f = finish16(t, true, threadIdx.x, 0, splits, part, T, N, eps, bias, a0, a1, a2);
        if (threadIdx.x < 4) sh[threadIdx.x] = sigmoidf(f.za);
    }
    __syncthreads();
    const float h[4] = {sh[0], sh[1], sh[2], sh[3]};
    pre_token<bf16_t, 4>(t, C, X, h, u);
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
                // H_post F first, then one fused multiply-add per stream, written out so
                // that every kernel forming X' rounds the same way
                float a = hp[i] * fv[e];
#pragma unroll
                for (int j = 0; j < NS; ++j) a = __builtin_fmaf(hr[i * NS + j], xv[j][e], a);
                o[e] = a;
            }
            store8_nt(ot + i * C + c, o);
        }
    }
}

// ---------------------------------------------------------------- post + residual, next layer's logits
// Cross-layer fusion (bf16, n = 4): X' = H_res X + H_post^T F exactly as k_post_res,
// and, from the bf16 X' just rounded, the split-K partial projection of the NEXT
// layer (sums over the split of X'.gamma' W' and of X'^2) in k_coeffs_part's partial
// layout, for k_coeffs_finish.  The next layer's read side then reads X' once, for u.
// grid (ceil(T / (16 NW)), splits); split s owns channels [s cs, (s + 1) cs) of the
// 4 streams (cs % 64 == 0) and W' is split member by member with that cs.  A chunk
// is 64 channels: lane (row, grp) covers channels 16 grp .. 16 grp + 15 of the chunk
// for its token, which are exactly its MFMA fragments for the chunk's 4 steps (one
// step per stream).  W' fragments of a chunk go through LDS (double-buffered, the
// next chunk's loaded while the current one computes).
template <int NW>
__global__ __launch_bounds__(NW * 64) void k_post_res_part(
    int64_t T, int64_t C, int64_t cs, const bf16_t* __restrict__ X, const bf16_t* __restrict__ F,
    const float* __restrict__ Hres, const float* __restrict__ Hpost, bf16_t* __restrict__ Xout,
    const bf16_t* __restrict__ Wp, float* __restrict__ part)
{
    constexpr int NT = NW * 64;
    constexpr int CHW = 4 * kWFrag;                 // W' fragments of a chunk (4 steps)
    constexpr int WPT = (CHW + NT - 1) / NT;
    __shared__ u32x4_t sW[2][CHW];
    __shared__ float sC[NW][16][25];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int row = lane & 15, grp = lane >> 4;
    const int64_t split = blockIdx.y;
    const int64_t N = 4 * C;
    const int64_t nch = cs / 64, spm = cs / 16;     // chunks, and W' steps of the split
    const int64_t t0 = (int64_t)blockIdx.x * (16 * NW);
    const int64_t t = t0 + 16 * wv + row;
    const bool rv = t < T;
    const int64_t tt = rv ? t : t0;
    float hr[16], hp[4];
#pragma unroll
    for (int a = 0; a < 16; ++a) hr[a] = rv ? Hres[tt * 16 + a] : 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) hp[k] = rv ? Hpost[tt * 4 + k] : 0.f;
    const bf16_t* xrow = X + tt * N + split * cs + 16 * grp;
    const bf16_t* frow = F + tt * C + split * cs + 16 * grp;
    bf16_t* orow = Xout + tt * N + split * cs + 16 * grp;
    const u32x4_t* wsrc = reinterpret_cast<const u32x4_t*>(Wp);
    const u32x4_t zero4 = u32x4_t{0u, 0u, 0u, 0u};
    const int64_t rot = nch > 0 ? (int64_t)(blockIdx.x * kCoefRot) % nch : 0;
    auto chunk = [&](int64_t cc) { const int64_t ci = cc + rot; return ci < nch ? ci : ci - nch; };

    struct In { u32x4_t x[4][2]; u32x4_t f[2]; };
    In ia;
    u32x4_t wr[WPT];
    auto load_in = [&](int64_t c, In& in) {
        const int64_t off = 64 * c;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const u32x4_t* src = reinterpret_cast<const u32x4_t*>(xrow + k * C + off);
            in.x[k][0] = rv ? src[0] : zero4;
            in.x[k][1] = rv ? src[1] : zero4;
        }
        const u32x4_t* fs = reinterpret_cast<const u32x4_t*>(frow + off);
        in.f[0] = rv ? fs[0] : zero4;
        in.f[1] = rv ? fs[1] : zero4;
    };
    auto load_w = [&](int64_t c) {
#pragma unroll
        for (int j = 0; j < WPT; ++j) {
            const int i = threadIdx.x + NT * j;
            if (i < CHW) {
                const int64_t gs = split * spm + (i / kWFrag) * nch + c;   // stream i / kWFrag
                wr[j] = wsrc[gs * kWFrag + i % kWFrag];
            }
        }
    };
    auto store_w = [&](int buf) {
#pragma unroll
        for (int j = 0; j < WPT; ++j) {
            const int i = threadIdx.x + NT * j;
            if (i < CHW) sW[buf][i] = wr[j];
        }
    };
    // projection and sum of squares: fp32 within a chunk, fp64 across chunks
    double accd[kWTiles][4];
#pragma unroll
    for (int nb = 0; nb < kWTiles; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) accd[nb][i] = 0.0;
    double ssd = 0.0;
    auto compute = [&](int buf, const In& in, int64_t c) {
        u32x4_t xo[4][2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t xw[4][4] = {{in.x[0][h].x, in.x[0][h].y, in.x[0][h].z, in.x[0][h].w},
                                       {in.x[1][h].x, in.x[1][h].y, in.x[1][h].z, in.x[1][h].w},
                                       {in.x[2][h].x, in.x[2][h].y, in.x[2][h].z, in.x[2][h].w},
                                       {in.x[3][h].x, in.x[3][h].y, in.x[3][h].z, in.x[3][h].w}};
            const uint32_t fw[4] = {in.f[h].x, in.f[h].y, in.f[h].z, in.f[h].w};
            float xv[4][8], fv[8];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                fv[2 * q] = bf16_lo(fw[q]);
                fv[2 * q + 1] = bf16_hi(fw[q]);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    xv[j][2 * q] = bf16_lo(xw[j][q]);
                    xv[j][2 * q + 1] = bf16_hi(xw[j][q]);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float o[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    float a = hp[i] * fv[e];
#pragma unroll
                    for (int j = 0; j < 4; ++j) a = __builtin_fmaf(hr[i * 4 + j], xv[j][e], a);
                    o[e] = a;
                }
                xo[i][h] = u32x4_t{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]),
                                   pack_bf16x2(o[4], o[5]), pack_bf16x2(o[6], o[7])};
            }
        }
        if (rv) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                u32x4_t* dst = reinterpret_cast<u32x4_t*>(orow + i * C + 64 * c);
                __builtin_nontemporal_store(xo[i][0], dst);
                __builtin_nontemporal_store(xo[i][1], dst + 1);
            }
        }
        float ssc = 0.f;
        f32x4_t acc[kWTiles];
#pragma unroll
        for (int nb = 0; nb < kWTiles; ++nb) acc[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                ssc = sumsq8(xo[i][h], ssc);
#pragma unroll
                for (int nb = 0; nb < kWTiles; ++nb)
                    acc[nb] = mfma16(xo[i][h], sW[buf][(i * kWTiles + nb) * 128 + h * 64 + lane],
                                     acc[nb]);
            }
        }
#pragma unroll
        for (int nb = 0; nb < kWTiles; ++nb)
#pragma unroll
            for (int i = 0; i < 4; ++i) accd[nb][i] += (double)acc[nb][i];
        ssd += (double)ssc;
    };

    // inputs are not prefetched: the register budget goes to occupancy instead
    if (nch > 0) {
        load_w(chunk(0));
        store_w(0);
    }
    __syncthreads();
    for (int64_t c = 0; c < nch; ++c) {
        load_in(chunk(c), ia);
        if (c + 1 < nch) load_w(chunk(c + 1));
        compute((int)(c & 1), ia, chunk(c));
        if (c + 1 < nch) store_w((int)((c + 1) & 1));
        __syncthreads();
    }

    part_epilogue(accd, ssd, sC[wv], lane, t0 + 16 * wv, T,
                  part + (split * T + t0 + 16 * wv) * kPartPitch);
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

bool coeffs_use_mfma(int64_t, int n, int64_t, int dtype)
{
    return dtype == MHC_BF16 && n == 4 && force_path() != kPathVector;
}

// Split of the flattened axis for the MFMA path: enough ranges that the grid
// fills two blocks of k_coeffs_part per CU, whole chunks per range.
static inline int coeffs_splits(int64_t T, int64_t nsteps, int64_t* spr)
{
    const int64_t tiles = (T + 16 * kCoefNW - 1) / (16 * kCoefNW);
    const int64_t nch = (nsteps + kCoefCK - 1) / kCoefCK;
    int64_t sp = (kCoefBlocks + tiles - 1) / tiles;
    if (sp > nch) sp = nch;
    if (sp > 16) sp = 16;
    if (sp < 1) sp = 1;
    const int64_t cps = (nch + sp - 1) / sp;        // chunks per range
    *spr = cps * kCoefCK;
    return (int)((nch + cps - 1) / cps);
}

size_t coeffs_workspace_bytes(int64_t T, int n, int64_t C, int dtype)
{
    if (!coeffs_use_mfma(T, n, C, dtype)) return 0;
    const int64_t ns = wsplit_steps((int64_t)n * C);
    int64_t spr;
    const int sp = coeffs_splits(T, ns, &spr);
    return align256(sizeof(bf16_t) * (size_t)ns * kWpStep) +
           align256(sizeof(float) * (size_t)sp * (size_t)T * kPartPitch);
}

template <typename Tio, int NS>
static void coeffs_generic_launch(int64_t T, int64_t C, const void* X, const float* gamma,
                                  float eps, const float* W, const float* bias,
                                  const float* alpha, float* z, float* rms, float* Hpre,
                                  float* Hpost, float* proj, hipStream_t s)
{
    constexpr int TB = NS >= 8 ? 1 : 4;     // tokens per block (NS = 8: K + 1 = 81 sums each)
    hipLaunchKernelGGL((k_coeffs_generic<Tio, NS, TB>), dim3(blocks_for(T, TB)), dim3(256), 0, s,
                       T, C, (const Tio*)X, gamma, eps, W, bias, alpha[0], alpha[1], alpha[2], z,
                       rms, Hpre, Hpost, proj);
}

hipError_t launch_coeffs(int64_t T, int n, int64_t C, int dtype, const void* X,
                         const float* gamma, float eps, const float* W, const float* bias,
                         const float* alpha, float* z, float* rms, float* Hpre, float* Hpost,
                         int iters, const float* zres_in, float* Hres, float* proj, void* ws,
                         hipStream_t s)
{
    if (coeffs_use_mfma(T, n, C, dtype)) {
        constexpr int NW = kCoefNW;
        const int64_t N = (int64_t)n * C, ns = wsplit_steps(N);
        int64_t spr;
        const int sp = coeffs_splits(T, ns, &spr);
        bf16_t* Wp = static_cast<bf16_t*>(ws);
        float* part = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                               align256(sizeof(bf16_t) * (size_t)ns * kWpStep));
        launch_wsplit(N, C, 0, gamma, W, Wp, s);
        hipLaunchKernelGGL((k_coeffs_part<NW, kCoefCK, kCoefD>), dim3(blocks_for(T, 16 * NW), (unsigned)sp),
                           dim3(NW * 64), 0, s, T, N, ns, spr, (const bf16_t*)X, (const bf16_t*)Wp,
                           part);
        hipLaunchKernelGGL(k_coeffs_finish, dim3(blocks_for(T, 16)), dim3(256), 0, s, T, sp, part, N,
                           eps, bias, alpha[0], alpha[1], alpha[2], z, rms, Hpre, Hpost, iters,
                           zres_in, Hres, proj);
        return hipGetLastError();
    } else {
        for_io(dtype == MHC_BF16, [&](auto tio) {
            for_n(n, [&](auto ns) {
                coeffs_generic_launch<decltype(tio), decltype(ns)::value>(
                    T, C, X, gamma, eps, W, bias, alpha, z, rms, Hpre, Hpost, proj, s);
            });
        });
    }
    if (Hres) {
        // Sinkhorn-Knopp of the res logits (or of injected ones, rows of n*n)
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        return zres_in ? launch_sinkhorn(T, n, zres_in, (int64_t)n * n, iters, Hres, s)
                       : launch_sinkhorn(T, n, z + 2 * n, (int64_t)K_of(n), iters, Hres, s);
    }
    return hipGetLastError();
}

hipError_t launch_fwd_pre(int64_t T, int n, int64_t C, int dtype, const void* X,
                          const float* gamma, float eps, const float* W, const float* bias,
                          const float* alpha, float* z, float* rms, float* Hpre, float* Hpost,
                          int iters, const float* zres_in, float* Hres, void* u, float* proj,
                          void* ws, hipStream_t s)
{
    if (fwd_sr_available(T, n, C, dtype))
        return launch_fwd_pre_sr(T, C, X, gamma, eps, W, bias, alpha, z, rms, Hpre, Hpost, iters,
                                 zres_in, Hres, u, proj, ws, s);
    if (!coeffs_use_mfma(T, n, C, dtype)) {
        const hipError_t e = launch_coeffs(T, n, C, dtype, X, gamma, eps, W, bias, alpha, z, rms,
                                           Hpre, Hpost, iters, zres_in, Hres, proj, ws, s);
        if (e != hipSuccess) return e;
        return launch_pre(T, n, C, dtype, X, Hpre, u, s);
    }
    constexpr int NW = kCoefNW;
    const int64_t N = (int64_t)n * C, ns = wsplit_steps(N);
    int64_t spr;
    const int sp = coeffs_splits(T, ns, &spr);
    bf16_t* Wp = static_cast<bf16_t*>(ws);
    float* part = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                           align256(sizeof(bf16_t) * (size_t)ns * kWpStep));
    launch_wsplit(N, C, 0, gamma, W, Wp, s);
    hipLaunchKernelGGL((k_coeffs_part<NW, kCoefCK, kCoefD>), dim3(blocks_for(T, 16 * NW), (unsigned)sp),
                       dim3(NW * 64), 0, s, T, N, ns, spr, (const bf16_t*)X, (const bf16_t*)Wp, part);
    const int64_t nsk = (T + 15) / 16;
    hipLaunchKernelGGL(k_finish_pre, dim3((unsigned)(nsk + T)), dim3(256), 0, s, T, nsk, sp,
                       (const float*)part, N, C, eps, bias, alpha[0], alpha[1], alpha[2], z, rms,
                       Hpre, Hpost, iters, zres_in, Hres, (const bf16_t*)X, (bf16_t*)u, proj);
    return hipGetLastError();
}

hipError_t launch_post_res_fwd_pre(int64_t T, int n, int64_t C, int dtype, const void* X,
                                   const void* F, const float* Hres_prev, const float* Hpost_prev,
                                   void* Xout, const float* gamma, float eps, const float* W,
                                   const float* bias, const float* alpha, float* z, float* rms,
                                   float* Hpre, float* Hpost, int iters, const float* zres_in,
                                   float* Hres, void* u, float* proj, void* ws, hipStream_t s)
{
    if (fwd_sr_available(T, n, C, dtype)) {
        const PostResIn xf{X, F, Hres_prev, Hpost_prev, Xout};
        return launch_fwd_pre_sr(T, C, nullptr, gamma, eps, W, bias, alpha, z, rms, Hpre, Hpost, iters,
                                 zres_in, Hres, u, proj, ws, s, &xf);
    }
    const hipError_t e = launch_post_res(T, n, C, dtype, X, F, Hres_prev, Hpost_prev, Xout, s);
    if (e != hipSuccess) return e;
    return launch_fwd_pre(T, n, C, dtype, Xout, gamma, eps, W, bias, alpha, z, rms, Hpre, Hpost,
                          iters, zres_in, Hres, u, proj, ws, s);
}

hipError_t launch_sinkhorn(int64_t T, int n, const float* zres, int64_t ld, int iters,
                           float* Hres, hipStream_t s)
{
    if (n == 4) {
        hipLaunchKernelGGL(k_sinkhorn16, dim3(blocks_for(T, 16)), dim3(256), 0, s, T, zres, ld, iters, Hres);
    } else {
        for_n(n, [&](auto ns) {
            hipLaunchKernelGGL((k_sinkhorn<decltype(ns)::value>), dim3(blocks_for(T, 256)), dim3(256), 0,
                               s, T, zres, ld, iters, Hres);
        });
    }
    return hipGetLastError();
}

hipError_t launch_pre(int64_t T, int n, int64_t C, int dtype, const void* X, const float* Hpre,
                      void* u, hipStream_t s)
{
    const dim3 g((unsigned)T), b(256);
    for_io(dtype == MHC_BF16, [&](auto tio) {
        using Tio = decltype(tio);
        for_n(n, [&](auto ns) {
            hipLaunchKernelGGL((k_pre<Tio, decltype(ns)::value>), g, b, 0, s, C, (const Tio*)X, Hpre,
                               (Tio*)u);
        });
    });
    return hipGetLastError();
}

hipError_t launch_post_res(int64_t T, int n, int64_t C, int dtype, const void* X, const void* F,
                           const float* Hres, const float* Hpost, void* Xout, hipStream_t s)
{
    const dim3 g((unsigned)T), b(256);
    for_io(dtype == MHC_BF16, [&](auto tio) {
        using Tio = decltype(tio);
        for_n(n, [&](auto ns) {
            hipLaunchKernelGGL((k_post_res<Tio, decltype(ns)::value>), g, b, 0, s, C, (const Tio*)X,
                               (const Tio*)F, Hres, Hpost, (Tio*)Xout);
        });
    });
    return hipGetLastError();
}

hipError_t launch_composite(int64_t T, int n, const float* Hres, float* P, float* gr, float* gc,
                            hipStream_t s)
{
    for_n(n, [&](auto ns) {
        hipLaunchKernelGGL((k_composite<decltype(ns)::value>), dim3(blocks_for(T, 256)), dim3(256), 0, s,
                           T, Hres, P, gr, gc);
    });
    return hipGetLastError();
}

// ---- cross-layer fusion
bool next_shape_ok(int n, int64_t C, int dtype) { return dtype == MHC_BF16 && n == 4 && C % 64 == 0; }

// Channel splits of k_post_res_part: a power of two dividing C / 64, enough to give
// about two blocks per CU.
static int next_splits(int64_t T, int64_t C)
{
    const int64_t tiles = (T + 16 * kCoefNW - 1) / (16 * kCoefNW);
    int64_t sp = 1;
    while (tiles * sp < kCoefBlocks && (C / 64) % (sp * 2) == 0) sp *= 2;
    return (int)sp;
}

size_t next_workspace_bytes(int64_t T, int64_t C)
{
    const int64_t N = 4 * C;
    return align256(sizeof(bf16_t) * (size_t)wsplit_steps(N) * kWpStep) +
           align256(sizeof(float) * (size_t)next_splits(T, C) * (size_t)T * kPartPitch);
}

static float* next_partials(void* ws, int64_t C)
{
    return reinterpret_cast<float*>(static_cast<char*>(ws) +
                                    align256(sizeof(bf16_t) * (size_t)wsplit_steps(4 * C) * kWpStep));
}

hipError_t launch_post_res_next(int64_t T, int64_t C, const void* X, const void* F,
                                const float* Hres, const float* Hpost, void* Xout,
                                const float* gamma_next, const float* W_next, void* ws,
                                hipStream_t s)
{
    constexpr int NW = kCoefNW;
    const int sp = next_splits(T, C);
    const int64_t cs = C / sp;
    bf16_t* Wp = static_cast<bf16_t*>(ws);
    launch_wsplit(4 * C, C, cs, gamma_next, W_next, Wp, s);
    hipLaunchKernelGGL((k_post_res_part<NW>), dim3(blocks_for(T, 16 * NW), (unsigned)sp), dim3(NW * 64),
                       0, s, T, C, cs, (const bf16_t*)X, (const bf16_t*)F, Hres, Hpost, (bf16_t*)Xout,
                       (const bf16_t*)Wp, next_partials(ws, C));
    return hipGetLastError();
}

hipError_t launch_fwd_pre_from_next(int64_t T, int64_t C, float eps, const float* bias,
                                    const float* alpha, float* z, float* rms, float* Hpre,
                                    float* Hpost, int iters, const float* zres_in, float* Hres,
                                    const void* X, void* u, float* proj, void* ws, hipStream_t s)
{
    const int64_t nsk = (T + 15) / 16;
    hipLaunchKernelGGL(k_finish_pre, dim3((unsigned)(nsk + T)), dim3(256), 0, s, T, nsk,
                       next_splits(T, C), (const float*)next_partials(ws, C), 4 * C, C, eps, bias,
                       alpha[0], alpha[1], alpha[2], z, rms, Hpre, Hpost, iters, zres_in, Hres,
                       (const bf16_t*)X, (bf16_t*)u, proj);
    return hipGetLastError();
}

}  // namespace mhc
