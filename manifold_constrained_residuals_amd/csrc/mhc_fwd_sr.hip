// mhc_fwd_sr.hip -- the forward read side in one pass over X (bf16, n = 4).
//
// u = H_pre X needs H_pre, and H_pre needs a reduction over all n*C values of a token
// (RMSNorm and the projection).  The two-pass path (mhc_fwd.hip) therefore reads X
// twice.  Here X is read once:
//
//   * A persistent grid of one 8-wave block per CU.  Blocks form groups of G = C / 256
//     members on one XCD (blocks are dealt round-robin to the 8 XCDs, so block b sits on
//     XCD b % 8); a group walks a contiguous range of 16-token tiles.
//   * Member m owns channels [256 m, 256 m + 256) of the 4 streams; wave w of it owns
//     channels 256 m + 32 w + [0, 32).  Its slice of W' = gamma (.) W, split into three
//     bf16 terms (wsplit3), sits in registers as MFMA B fragments for the whole kernel
//     (80 VGPRs).
//   * A tile's member slice (16 tokens x 4 streams x 512 bytes) comes in by
//     direct-to-LDS loads (no register destination, so the waits are explicit counts),
//     three tiles deep, and is copied into a ring of register tiles where it stays until
//     its u is written, D tiles later.
//   * Per tile, the member's partial logits (24 projections, folded from the three terms,
//     and the sum of squares) are summed over its 8 waves and published: the 5 values that
//     H_pre needs (4 pre projections, the sum of squares) as 64-bit words that carry the
//     tile number in their upper half (so a reader needs no fence: it polls until every
//     word it needs shows its tile), all 25 as plain floats for the finishing pass.
//   * Every member reads the 5 published values of all members for the tile E tiles
//     back, forms H_pre of its 16 tokens with the finishing pass's arithmetic, and writes
//     u for its channels from the register tile.
//   * A separate finishing launch forms z, r, the gates, the Sinkhorn projection and the
//     unscaled projection from the plain partials (the same member order, so H_pre there
//     is bitwise the one u used).
//
// The update rule and the fused read side follow chatgpz.de, "Von Residualverbindungen
// zu Hyperverbindungen" and staging.reportify.cn, "高效基础设施设计" note [18] (one
// operator for the scans and matmuls).
#include <atomic>
#include <cstdlib>
#include <cstring>

#include "mhc_device.hpp"
#include "mhc_internal.hpp"
#include "../../include/mhc.h"

namespace mhc {
namespace sr {

constexpr int kNW = 8;                 // waves per block
constexpr int kThreads = kNW * 64;
constexpr int kTT = 16;                // tokens per tile
constexpr int kMC = 256;               // channels per member (8 waves x 32)
constexpr int kP = 3;                  // LDS tile slots (direct-to-LDS loads two tiles ahead)
constexpr int kE = 2;                  // exchange reads of tile j are issued E tiles after it
constexpr int kD = kE + 1;             // u of tile j is written D tiles after its projection
constexpr int kR = kD + 1;             // register tile slots
constexpr int kRing = 8;               // exchange ring slots per group (>= 2 E + 3)
constexpr int kNV = 5;                 // exchanged values per token: 4 pre projections, sum of squares
constexpr int kPairs = kTT * kNV;      // 80 (token, value) pairs per tile
constexpr int kPV = 25;                // plain partial values per token: 24 projections, sum of squares
constexpr int kRow = kMC * 2;          // bytes of a member row (one token, one stream)
constexpr int kSlot = kTT * 4 * kRow;  // 32 KiB: one tile of the member slice
constexpr int kPW = kTT * kPV;         // 400 floats: one wave's partials of a tile

// Dynamic LDS (the targets of direct-to-LDS loads; read only through asm, with explicit
// waits): X tile slots [kP][64 rows][512 bytes], then exchange words [2][kNW][2][64][16 B]
constexpr int oX = 0;
constexpr int oXW = kP * kSlot;
constexpr int kLds = oXW + 2 * kNW * 2048;
static_assert(kLds + 2 * kNW * kPW * 4 + 2 * kTT * 4 * 4 <= 160 * 1024, "LDS budget");

// VMEM operations a wave issues per iteration, all unconditional (out-of-range work goes
// to dummy addresses) so that the explicit waits below are constants:
constexpr int kXld = 2;                // exchange reads (direct-to-LDS, 16 bytes each)
constexpr int kDma = 4;                // direct-to-LDS loads of a tile (32 per tile, 8 waves)
constexpr int kU = 1;                  // u store
constexpr int kPub = 2;                // publish: one plain store, one tagged store
constexpr int kIter = kXld + kDma + kU + kPub;

constexpr uint32_t kSpinLimit = 1u << 16;      // re-reads of one word before giving up

}  // namespace sr

// The logit and rms arithmetic shared by the single-read kernel and its finishing pass
// (they must agree bitwise on H_pre): r = sqrt(ss / N + eps); z = a p (1 / r) + b.
__device__ __forceinline__ float sr_r(float ss, int64_t N, float eps) {
    return sqrtf(ss / (float)N + eps);
}
__device__ __forceinline__ float sr_logit(float a, float p, float rinv, float b) {
    return a * p * rinv + b;
}

// Member sums in a fixed order: members in quarters of G / 4, each quarter summed in
// member order, then the quarters as ((q0 + q1) + q2) + q3.
template <typename F>
__device__ __forceinline__ float sr_member_sum(int G, F&& val) {
    const int mq = G >> 2;
    float q[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float s = val(j * mq);
        for (int i = 1; i < mq; ++i) s += val(j * mq + i);
        q[j] = s;
    }
    return ((q[0] + q[1]) + q[2]) + q[3];
}

// ---------------------------------------------------------------- exchange ring clear
__global__ __launch_bounds__(256) void k_sr_clear(uint64_t* __restrict__ p, int64_t n,
                                                  uint32_t* __restrict__ err)
{
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        p[i] = 0ull;
    if (blockIdx.x == 0 && threadIdx.x == 0) err[0] = 0u;
}

// ---------------------------------------------------------------- the single-read pass
struct SrArgs {
    int64_t T, C;
    int G, NG, TPG;                     // members per group, groups, tiles per group
    float eps, a0;
    const bf16_t* X;
    const float* gamma;
    const float* W;
    const float* bias;
    bf16_t* u;
    uint64_t* xch;                      // [NG][kRing][80][G]
    float* part;                        // [ntiles][G][16][25]
    float* dummy;                       // per block: 8 KiB of discard space (out-of-range stores)
    uint64_t* dummy64;                  // per block: 4 KiB
    uint32_t* err;                      // spin timeout flag
};

// 16 bytes of LDS at a byte address, read by asm with its own wait: the compiler treats
// any LDS read after a direct-to-LDS load as possibly dependent on it and would wait for
// every load in flight; the explicit counts in the kernel cover these reads instead.
__device__ __forceinline__ u32x4_t lds_read16(uint32_t addr)
{
    u32x4_t v;
    asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
    return v;
}

__global__ __launch_bounds__(sr::kThreads) void k_fwd_sr(const SrArgs a)
{
    using namespace sr;
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    __shared__ float pw[kNW * kPW];                           // the waves' partials of a tile
    __shared__ float hp[2][kTT * 4];                          // H_pre of a tile
    __shared__ int gave_up;                                   // a re-read timed out: stop waiting
    typedef __attribute__((address_space(3))) void* lds_ptr;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int wvu = __builtin_amdgcn_readfirstlane(wv);
    const int tr = lane & 15, q = lane >> 4;
    const int G = a.G;
    const int gpx = 32 / G;                                  // groups per XCD
    const int xcd = blockIdx.x & 7, l = blockIdx.x >> 3;
    if (l >= gpx * G) return;                                // spare CU
    const int g = xcd * gpx + l / G, m = l % G;
    const int64_t ntiles = (a.T + kTT - 1) / kTT;
    const int64_t tile0 = (int64_t)g * a.TPG;
    const int ntl = (int)((ntiles - tile0) < a.TPG ? (ntiles - tile0) : a.TPG);
    if (ntl <= 0) return;                                    // the whole group idles
    const int64_t C = a.C, N = 4 * C;
    const int64_t cm = (int64_t)m * kMC;                     // the member's first channel
    // out-of-range stores go to this block's own discard space: stores of many CUs to
    // shared lines would serialise in L2 and hold up every wave's counted operations
    float* const dummy = a.dummy + (int64_t)blockIdx.x * 2048;
    uint64_t* const dummy64 = a.dummy64 + (int64_t)blockIdx.x * 512;

    // ---- W' fragments: B operand of stream s, column tile nb; lane holds column
    // 16 nb + tr, k = 8 q + j <-> channel cm + 32 w + 8 q + j of stream s; columns as in
    // wsplit3 (hi, mid, lo of logits 0..23, then padding).
    u32x4_t wf[4][kWTiles];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int nb = 0; nb < kWTiles; ++nb) {
            const int col = 16 * nb + tr;
            const int kc = wsplit_logit(col), term = wsplit_term(col);
            float o[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int64_t e = (int64_t)s * C + cm + 32 * wv + 8 * q + j;
                const float v = a.gamma[e] * a.W[e * 24 + kc];
                o[j] = term < 3 ? wsplit3(v, term) : 0.f;
            }
            wf[s][nb] = u32x4_t{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]),
                                pack_bf16x2(o[4], o[5]), pack_bf16x2(o[6], o[7])};
        }
    }
    // Exchange words: a token's 5 values x 4 member quarters on 20 consecutive lanes, three
    // tokens per wave (waves 0..5); lane 20 j + 4 v + qq of wave w reads quarter qq of
    // value v of token 3 w + j.  Other lanes read a dummy word.
    const int xt = 3 * wv + lane / 20, xv = (lane % 20) >> 2, xq = lane & 3;
    const bool xon = lane < 60 && xt < kTT;
    const int mq = G >> 2;
    const float xbias = a.bias[xv < 4 ? xv : 0], a0 = a.a0, eps = a.eps;
    if (tid == 0) gave_up = 0;
    __syncthreads();

    // direct-to-LDS: instruction k of wave w covers rows 2 (w + 8 k) and 2 (w + 8 k) + 1
    // (row = 4 token + stream); lane i of it loads chunk (i & 31) ^ token of its row, so
    // that chunk j of row r sits at position j ^ (r >> 2) (readers of one chunk over 16
    // tokens hit 16 different 16-byte positions).
    const bf16_t* X = a.X;
    auto dma = [&](int jt, int slot) {
        // jt: local tile index (a tile past the range loads the group's first tile into a
        // slot nobody reads)
        const int64_t t0 = (tile0 + (jt < ntl ? jt : 0)) * kTT;
        unsigned char* dst = lds + oX + slot * kSlot;
#pragma unroll
        for (int k = 0; k < kDma; ++k) {
            const int ins = wvu + 8 * k;
            const int r = 2 * ins + (lane >> 5), tt = r >> 2, s = r & 3;
            int64_t tok = t0 + tt;
            if (tok >= a.T) tok = a.T - 1;
            const int chunk = (lane & 31) ^ tt;
            const bf16_t* src = X + (tok * 4 + s) * C + cm + 8 * chunk;
            __builtin_amdgcn_global_load_lds(src, (lds_ptr)(dst + ins * 1024), 16, 0, 0);
        }
    };
    const uint32_t lbase = (uint32_t)(uintptr_t)(lds_ptr)lds;
    uint64_t* xg = a.xch + (int64_t)g * kRing * kPairs * G;

    u32x4_t xr[kR][4];                                       // the register tile ring

    // prologue: tiles 0 .. kP - 2 into their LDS slots
#pragma unroll
    for (int j = 0; j < kP - 1; ++j) dma(j, j);

    const int nit = ntl + kD;
    for (int ib = 0; ib < nit; ib += kR) {
#pragma unroll
        for (int c = 0; c < kR; ++c) {
            const int i = ib + c;
            if (i >= nit) break;
            // 1. this wave's loads of tile i have landed (every later VMEM operation of
            // the wave is counted: the loads are two iterations old)
            if (i < ntl) {
                __atomic_signal_fence(__ATOMIC_SEQ_CST);
                wait_vmcnt(i == 0 ? kDma : (i == 1 ? kIter : kIter + kU + kPub));
                __atomic_signal_fence(__ATOMIC_SEQ_CST);
            }
            // 2. every wave's loads of tile i are in; iteration i - 1 is done everywhere
            __builtin_amdgcn_s_waitcnt(0xC07F);                 // lgkmcnt(0)
            __builtin_amdgcn_s_barrier();
            __atomic_signal_fence(__ATOMIC_SEQ_CST);

            // 3. exchange words of tile jc = i - 1 - E (brought into LDS in iteration i - 1,
            // each lane its own 4 words): check their tags, re-read any that are not there
            // yet; quarter sums, totals, H_pre -> hp
            const int jc = i - 1 - kE;
            if (jc >= 0 && jc < ntl) {
                __atomic_signal_fence(__ATOMIC_SEQ_CST);
                wait_vmcnt(kDma + kU + kPub);
                __atomic_signal_fence(__ATOMIC_SEQ_CST);
                const uint32_t la = lbase + oXW + (uint32_t)(((jc & 1) * kNW + wv) * 2048 + 16 * lane);
                const u32x4_t wa = lds_read16(la), wb = lds_read16(la + 1024);
                float qs = 0.f;
                if (xon) {
                    const uint32_t want = (uint32_t)jc + 1u;
                    const uint64_t* src = xg + ((int64_t)(jc % kRing) * kPairs + xt * kNV + xv) * G +
                                          xq * mq;
                    uint64_t xw[4] = {((uint64_t)wa.y << 32) | wa.x, ((uint64_t)wa.w << 32) | wa.z,
                                      ((uint64_t)wb.y << 32) | wb.x, ((uint64_t)wb.w << 32) | wb.z};
                    uint32_t late = 0;
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (j < mq && (uint32_t)(xw[j] >> 32) != want) late |= 1u << j;
                    if (late) {
                        // not all there yet: re-read those words until they are (bounded; a
                        // timeout is flagged in the workspace)
                        uint32_t spins = 0;
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            if ((late >> j) & 1u) {
                                uint64_t w;
                                do {
                                    __builtin_amdgcn_s_sleep(2);
                                    w = __hip_atomic_load(src + j, __ATOMIC_RELAXED,
                                                          __HIP_MEMORY_SCOPE_AGENT);
                                } while ((uint32_t)(w >> 32) != want && ++spins < kSpinLimit &&
                                         !*(volatile int*)&gave_up);
                                if ((uint32_t)(w >> 32) != want) {
                                    a.err[0] = 1u;
                                    *(volatile int*)&gave_up = 1;
                                }
                                xw[j] = w;
                            }
                        }
                    }
                    qs = __uint_as_float((uint32_t)xw[0]);
                    for (int j = 1; j < mq; ++j) qs += __uint_as_float((uint32_t)xw[j]);
                }
                // ((q0 + q1) + q2) + q3 on the quad's first lane (sr_member_sum's order)
                const float q1 = __shfl(qs, lane + 1, 64), q2 = __shfl(qs, lane + 2, 64),
                            q3 = __shfl(qs, lane + 3, 64);
                const float tot = ((qs + q1) + q2) + q3;
                const float ssum = __shfl(tot, lane - 4 * xv + 16, 64);   // value 4 of the token
                if (xon && xq == 0 && xv < 4) {
                    const float z = sr_logit(a0, tot, 1.0f / sr_r(ssum, N, eps), xbias);
                    hp[jc & 1][xt * 4 + xv] = sigmoidf(z);
                }
            }
            // 4. the exchange words of tile jr = i - E into this lane's LDS words (checked
            // next iteration): two 16-byte direct-to-LDS loads at device scope (sc1: past
            // the CU's own cache, which may hold an old copy)
            {
                const int jr = i - kE;
                const bool ok = xon && jr >= 0 && jr < ntl;
                const uint64_t* src = ok ? xg + ((int64_t)(jr % kRing) * kPairs + xt * kNV + xv) * G +
                                               xq * mq
                                         : dummy64 + 4 * lane;
                // words 0, 1 of every lane, then words 2, 3 (a load fills 64 x 16 bytes)
                unsigned char* dst = lds + oXW + ((jr & 1) * kNW + wv) * 2048;
                __builtin_amdgcn_global_load_lds(src, (lds_ptr)dst, 16, 0, 16);
                __builtin_amdgcn_global_load_lds(src + 2, (lds_ptr)(dst + 1024), 16, 0, 16);
            }
            // 5. direct-to-LDS loads of tile i + P - 1 into the slot tile i - 1 used
            dma(i + kP - 1, (i + kP - 1) % kP);
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            // 6. tile i: LDS -> register slot c, projection and sum of squares -> pw
            if (i < ntl) {
                const uint32_t sb = lbase + oX + (uint32_t)((i % kP) * kSlot);
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    xr[c][s] = lds_read16(sb + (uint32_t)((4 * tr + s) * kRow + (((4 * wv + q) ^ tr) << 4)));
                f32x4_t acc[kWTiles];
#pragma unroll
                for (int nb = 0; nb < kWTiles; ++nb) acc[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                float ss = 0.f;
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    ss = sumsq8(xr[c][s], ss);
#pragma unroll
                    for (int nb = 0; nb < kWTiles; ++nb)
                        acc[nb] = mfma16(xr[c][s], wf[s][nb], acc[nb]);
                }
                ss += __shfl_xor(ss, 16, 64);
                ss += __shfl_xor(ss, 32, 64);
                // fold the three terms: logit k < 16 on lane k, 16 + k on lane k < 8
                float* dst = pw + wv * kPW;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float tv[kWTiles];
#pragma unroll
                    for (int nb = 0; nb < kWTiles; ++nb) tv[nb] = acc[nb][e];
                    float f0, f1;
                    fold3(tv, tr, [](float v) { return lane_ror8(v); }, f0, f1);
                    const int t = 4 * q + e;
                    dst[t * kPV + tr] = f0;
                    if (tr < 8) dst[t * kPV + 16 + tr] = f1;
                }
                if (q == 0) dst[tr * kPV + 24] = ss;
            }
            // 7. every wave's partials of tile i and H_pre of tile jc are in LDS
            __builtin_amdgcn_s_waitcnt(0xC07F);                 // lgkmcnt(0)
            __builtin_amdgcn_s_barrier();
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            // 8. u of tile ju = i - D (= jc) from register slot (c + 1) % R
            {
                const int ju = i - kD;
                const bool ok = ju >= 0 && ju < ntl;
                const int64_t tok = (tile0 + (ok ? ju : 0)) * kTT + tr;
                float h[4] = {0.f, 0.f, 0.f, 0.f};
                if (ok) {
                    const float4 hv = *reinterpret_cast<const float4*>(&hp[ju & 1][tr * 4]);
                    h[0] = hv.x; h[1] = hv.y; h[2] = hv.z; h[3] = hv.w;
                }
                const u32x4_t* xv4 = xr[(c + 1) % kR];
                float o[8];
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const uint32_t w4[4] = {xv4[s].x, xv4[s].y, xv4[s].z, xv4[s].w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        // h_0 x_0, then one fused multiply-add per stream (pre_token's order)
                        const float lo = bf16_lo(w4[e]), hi = bf16_hi(w4[e]);
                        o[2 * e] = s == 0 ? h[0] * lo : __builtin_fmaf(h[s], lo, o[2 * e]);
                        o[2 * e + 1] = s == 0 ? h[0] * hi : __builtin_fmaf(h[s], hi, o[2 * e + 1]);
                    }
                }
                const bool st = ok && tok < a.T;
                bf16_t* ud = st ? a.u + tok * C + cm + 32 * wv + 8 * q
                                : reinterpret_cast<bf16_t*>(dummy) + 8 * (tid & 255);
                store8_nt(ud, o);
            }
            // 9. publish tile i: sums over the 8 waves of pw, as plain partials for the
            // finishing pass and, for the 5 values H_pre needs, as tagged words
            {
                const bool ok = i < ntl && tid < kPW;
                const int t = tid / kPV, k = tid - t * kPV;
                float v = 0.f;
                if (ok) {
                    const float* src = pw + t * kPV + k;
#pragma unroll
                    for (int w = 0; w < kNW; ++w) v += src[w * kPW];
                }
                float* pdst = ok ? a.part + (((tile0 + i) * G + m) * kTT) * kPV + tid
                                 : dummy + (tid & 1023);
                *pdst = v;
                const bool tag = ok && (k < 4 || k == 24);
                const int pr = t * kNV + (k == 24 ? 4 : k);
                uint64_t* xdst = tag ? xg + ((int64_t)(i % kRing) * kPairs + pr) * G + m
                                     : dummy64 + (tid & 511);
                const uint64_t word = ((uint64_t)((uint32_t)i + 1u) << 32) | __float_as_uint(v);
                __hip_atomic_store(xdst, word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
}

// ---------------------------------------------------------------- finishing pass
// One block of 256 threads per tile: token tile * 16 + tid / 16 on 16 lanes.  Lane q
// sums the members' partial values q and 16 + q (q < 9; value 24 is the sum of squares)
// in the order of sr_member_sum, then forms z, r, the gates, the unscaled projection and
// -- on the same 16 lanes -- the Sinkhorn projection of the res logits (or of injected
// ones).  Tokens past T run on zeros so that every lane takes part in the exchanges.
__global__ __launch_bounds__(256) void k_sr_finish(
    int64_t T, int G, const float* __restrict__ part, int64_t N, float eps,
    const float* __restrict__ bias, float a0, float a1, float a2, float* __restrict__ z,
    float* __restrict__ rms, float* __restrict__ Hpre, float* __restrict__ Hpost, int iters,
    const float* __restrict__ zres_in, float* __restrict__ Hres, float* __restrict__ proj)
{
    using namespace sr;
    const int64_t tile = blockIdx.x;
    const int tt = threadIdx.x >> 4, q = threadIdx.x & 15, base = threadIdx.x & ~15;
    const int64_t t = tile * kTT + tt;
    const bool valid = t < T;
    const float* pt = part + (tile * G * kTT + tt) * kPV;     // member m at + m * kTT * kPV
    float pa = 0.f, pb = 0.f;
    if (valid) {
        pa = sr_member_sum(G, [&](int m) { return pt[(int64_t)m * kTT * kPV + q]; });
        if (q < 9) pb = sr_member_sum(G, [&](int m) { return pt[(int64_t)m * kTT * kPV + 16 + q]; });
    }
    const float sq = __shfl(pb, base + 8, 64);
    const float r = sr_r(sq, N, eps);
    const float rinv = 1.0f / r;
    const float za = sr_logit(q < 4 ? a0 : (q < 8 ? a1 : a2), pa, rinv, bias[q]);
    const float zb = sr_logit(a2, pb, rinv, bias[16 + (q & 7)]);
    if (valid) {
        z[t * 24 + q] = za;
        if (q < 8) z[t * 24 + 16 + q] = zb;
        if (q == 0) rms[t] = r;
        if (q < 4) Hpre[t * 4 + q] = sigmoidf(za);
        else if (q < 8) Hpost[t * 4 + q - 4] = sigmoidf(za);
        if (proj) {
            proj[t * 24 + q] = pa * rinv;
            if (q < 8) proj[t * 24 + 16 + q] = pb * rinv;
        }
    }
    // res entry q is logit 8 + q: lane q + 8's za for q < 8, lane q - 8's zb otherwise
    const float from_a = __shfl(za, base + ((q + 8) & 15), 64);
    const float from_b = __shfl(zb, base + ((q + 8) & 15), 64);
    float zr = q < 8 ? from_a : from_b;
    if (zres_in) zr = valid ? zres_in[t * 16 + q] : 0.f;
    const float h = sinkhorn16_fwd(valid ? zr : 0.f, iters);
    if (valid) Hres[t * 16 + q] = h;
}

// ---------------------------------------------------------------- host side
int force_path()
{
    static std::atomic<int> cached{-1};
    int v = cached.load(std::memory_order_relaxed);
    if (v < 0) {
        const char* e = std::getenv("MHC_FORCE_PATH");
        v = kPathAuto;
        if (e && std::strcmp(e, "vector") == 0) v = kPathVector;
        else if (e && std::strcmp(e, "twopass") == 0) v = kPathTwoPass;
        cached.store(v, std::memory_order_relaxed);
    }
    return v;
}

namespace {

struct SrLayout {
    int G, NG, TPG;
    int64_t ntiles, xwords;
    size_t oXch, oPart, oDummy, oDummy64, oErr, bytes;
};

SrLayout sr_layout(int64_t T, int64_t C)
{
    SrLayout L{};
    L.G = (int)(C / sr::kMC);
    L.NG = 256 / L.G;
    L.ntiles = (T + sr::kTT - 1) / sr::kTT;
    L.TPG = (int)((L.ntiles + L.NG - 1) / L.NG);
    L.xwords = (int64_t)L.NG * sr::kRing * sr::kPairs * L.G;
    size_t o = 0;
    L.oXch = o;     o += align256(sizeof(uint64_t) * (size_t)L.xwords + 64);   // 32-byte reads past a quarter
    L.oPart = o;    o += align256(sizeof(float) * (size_t)L.ntiles * L.G * sr::kTT * sr::kPV);
    L.oDummy = o;   o += 256 * 8192;                        // per block
    L.oDummy64 = o; o += 256 * 4096;
    L.oErr = o;     o += 256;
    L.bytes = o;
    return L;
}

}  // namespace

// Shapes the single-read pass is built for: bf16, n = 4, C = 256 G with G members per
// group dividing the 32 CUs of an XCD and a multiple of 4 (the exchange's quarters).
bool fwd_sr_shape(int n, int64_t C, int dtype)
{
    if (dtype != MHC_BF16 || n != 4 || C % sr::kMC != 0) return false;
    const int64_t G = C / sr::kMC;
    return G == 4 || G == 8 || G == 16;
}

size_t fwd_sr_workspace_bytes(int64_t T, int n, int64_t C, int dtype)
{
    return fwd_sr_shape(n, C, dtype) ? sr_layout(T, C).bytes : 0;
}

// The device can run the pass: 8 XCDs of 32 CUs (one block per CU, 256 blocks), and the
// path is not switched off.
static bool fwd_sr_device_ok()
{
    if (force_path() != kPathAuto) return false;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return false;
    static std::atomic<int> ok[64] = {};
    int v = ok[dev].load(std::memory_order_acquire);
    if (v == 0) {
        int cus = 0;
        v = 2;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
            cus == 256 &&
            hipFuncSetAttribute(reinterpret_cast<const void*>(&k_fwd_sr),
                                hipFuncAttributeMaxDynamicSharedMemorySize, sr::kLds) == hipSuccess)
            v = 1;
        ok[dev].store(v, std::memory_order_release);
    }
    return v == 1;
}

bool fwd_sr_available(int64_t T, int n, int64_t C, int dtype)
{
    (void)T;
    return fwd_sr_shape(n, C, dtype) && fwd_sr_device_ok();
}

hipError_t launch_fwd_pre_sr(int64_t T, int64_t C, const void* X, const float* gamma, float eps,
                             const float* W, const float* bias, const float* alpha, float* z,
                             float* rms, float* Hpre, float* Hpost, int iters,
                             const float* zres_in, float* Hres, void* u, float* proj, void* ws,
                             hipStream_t s)
{
    const SrLayout L = sr_layout(T, C);
    unsigned char* w = static_cast<unsigned char*>(ws);
    SrArgs a;
    a.T = T; a.C = C; a.G = L.G; a.NG = L.NG; a.TPG = L.TPG;
    a.eps = eps; a.a0 = alpha[0];
    a.X = static_cast<const bf16_t*>(X); a.gamma = gamma; a.W = W; a.bias = bias;
    a.u = static_cast<bf16_t*>(u);
    a.xch = reinterpret_cast<uint64_t*>(w + L.oXch);
    a.part = reinterpret_cast<float*>(w + L.oPart);
    a.dummy = reinterpret_cast<float*>(w + L.oDummy);
    a.dummy64 = reinterpret_cast<uint64_t*>(w + L.oDummy64);
    a.err = reinterpret_cast<uint32_t*>(w + L.oErr);
    // the ring starts empty: a tag of 0 matches no tile
    hipLaunchKernelGGL(k_sr_clear, dim3(64), dim3(256), 0, s, a.xch, L.xwords, a.err);
    hipLaunchKernelGGL(k_fwd_sr, dim3(256), dim3(sr::kThreads), (size_t)sr::kLds, s, a);
    hipLaunchKernelGGL(k_sr_finish, dim3((unsigned)L.ntiles), dim3(256), 0, s, T, L.G,
                       (const float*)a.part, 4 * C, eps, bias, alpha[0], alpha[1], alpha[2], z,
                       rms, Hpre, Hpost, iters, zres_in, Hres, proj);
    return hipGetLastError();
}

}  // namespace mhc
