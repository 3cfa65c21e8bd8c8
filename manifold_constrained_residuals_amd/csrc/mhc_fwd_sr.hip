// mhc_fwd_sr.hip -- the forward read side in one pass over X (bf16, n = 4).
//
// u = H_pre X needs H_pre, and H_pre needs a reduction over all n*C values of a token
// (RMSNorm and the projection).  The two-pass path (mhc_fwd.hip) therefore reads X
// twice.  Here X is read once:
//
//   * A persistent grid of one 8-wave block per CU.  Blocks form groups of G = C / 256
//     members on one XCD (blocks are dealt round-robin to the 8 XCDs, so block b sits on
//     XCD b % 8); a group walks a contiguous range of 16-token tiles.  Member m owns
//     channels [256 m, 256 m + 256) of the 4 streams.
//   * The waves have two roles, one wave of each per SIMD.  Projection wave p (0..3)
//     owns channels 256 m + 64 p + [0, 64): its slice of W' = gamma (.) W, split into
//     three bf16 terms (wsplit3) and cut into MFMA B fragments by a preparation launch,
//     sits in registers for the whole kernel (160 VGPRs).  Per tile it publishes the
//     member's partials of the previous tile (summed over the projection waves), then
//     multiplies the tile's slice (from LDS) into the 24 partial logits (folded from the
//     three terms) and the partial sum of squares, into LDS.  u wave v (0..3) owns
//     tokens 4 v .. 4 v + 3 of every tile: it copies their rows from LDS into a ring of
//     register tiles, gathers the published values of all members for the tile D back,
//     forms H_pre of its 4 tokens with the finishing pass's arithmetic and writes their
//     u from the register tile.
//   * Tiles (16 tokens x 4 streams x 512 bytes of the member slice) come in by
//     direct-to-LDS loads (no register destination, so the waits are explicit counts),
//     four slots deep.  One barrier per tile: the roles overlap between barriers.
//   * Published values: the 5 that H_pre needs (4 pre projections, the sum of squares)
//     as 64-bit words that carry the tile number in their upper half (a reader needs no
//     fence: it re-reads until every word it needs shows its tile), all 25 as plain
//     floats for the finishing pass.  The words are stored and read at device scope; a
//     member's words of a tile are contiguous in the ring (640 bytes), so that the stores,
//     which write through to memory, move whole lines.
//   * A separate finishing launch forms z, r, the gates, the Sinkhorn projection and the
//     unscaled projection from the plain partials (the same member order, so H_pre there
//     is bitwise the one u used).
//   * A member that waits too long for a published word (members that never became
//     resident together, say) stops waiting, flags the workspace and writes NaN into the
//     u of the tokens concerned: the outputs show it instead of holding wrong values.
//
// The update rule and the fused read side follow chatgpz.de, "Von Residualverbindungen
// zu Hyperverbindungen" and staging.reportify.cn, "高效基础设施设计" note [18] (one
// operator for the scans and matmuls).
#include <algorithm>
#include <atomic>
#include <type_traits>
#include <cstdlib>
#include <cstring>

#include "mhc_device.hpp"
#include "mhc_internal.hpp"
#include "../../include/mhc.h"

namespace mhc {
namespace sr {

constexpr int kNW = 8;                 // waves per block
constexpr int kNP = 4;                 // projection waves (the other 4 are u waves)
constexpr int kThreads = kNW * 64;
constexpr int kTT = 16;                // tokens per tile
constexpr int kMC = 256;               // channels per member
constexpr int kPC = kMC / kNP;         // 64 channels per projection wave
constexpr int kKS = 4 * kPC / 32;      // 8 MFMA k-steps (32 each) per projection wave
constexpr int kUT = kTT / 4;           // 4 tokens per u wave
constexpr int kE = 2;                  // exchange reads of tile j are issued E tiles after it
constexpr int kD = kE + 1;             // u of tile j is written D tiles after its projection
constexpr int kR = kD + 1;             // register tile slots of a u wave
constexpr int kRing = 8;               // exchange ring slots per group (>= 2 E + 3)
constexpr int kNV = 5;                 // exchanged values per token: 4 pre projections, sum of squares
constexpr int kPairs = kTT * kNV;      // 80 (token, value) pairs per tile
constexpr int kUPairs = kUT * kNV;     // 20 of them per u wave
constexpr int kPV = 25;                // plain partial values per token: 24 projections, sum of squares
constexpr int kRow = kMC * 2;          // bytes of a member row (one token, one stream)
constexpr int kSlot = kTT * 4 * kRow;  // 32 KiB: one tile of the member slice
constexpr int kPW = kTT * kPV;         // 400 floats: one projection wave's partials of a tile

// Per group size G (members; C = 256 G, G a multiple of 4 up to 32):
//   XI: exchange loads per u wave and tile (1 KiB each) for its 20 G words;
//   P:  LDS tile slots (direct-to-LDS loads P - 1 tiles ahead): 4 where they fit beside
//       the exchange words and the partials, else 3.
// Dynamic LDS (the targets of direct-to-LDS loads; read only through asm, with explicit
// waits): X tile slots [P][64 rows][512 bytes], then per u wave its exchange words
// [XI][64 lanes][16 bytes].  Static LDS: the partials, 2 x 4 x 400 floats.
constexpr int oX = 0;
constexpr int xi_of(int G) { return (kUPairs * G * 8 + 1023) / 1024; }
constexpr int lds_of(int P, int G) { return P * kSlot + 4 * xi_of(G) * 1024; }
constexpr int kStaticLds = 2 * kNP * kPW * 4 + 64;
constexpr int p_of(int G) { return lds_of(4, G) + kStaticLds <= 160 * 1024 ? 4 : 3; }
// The transform variant (XF: X = H_res X_prev + H_post^T F_prev formed in the kernel) also
// brings each tile's F rows (16 x 512 bytes), H_res (16 x 16 floats) and H_post (16 x 4
// floats) into the slot, three slots deep.
constexpr int oF = kSlot, oHR = oF + kTT * kRow, oHP = oHR + kTT * 16 * 4;
constexpr int kSlotXF = oHP + kTT * 4 * 4;
constexpr int kPXF = 3;
constexpr int slot_of(bool XF) { return XF ? kSlotXF : kSlot; }
constexpr int lds_xf(int G) { return kPXF * kSlotXF + 4 * xi_of(G) * 1024; }
constexpr bool g_ok(int G) { return G >= 4 && G <= 32 && G % 4 == 0; }

// VMEM operations per iteration, all unconditional (out-of-range work goes to dummy
// addresses) so that the explicit waits below are constants:
constexpr int kDmaP = 32 / kNP;        // a projection wave's direct-to-LDS loads of a tile
constexpr int kPubP = 3;               // a projection wave's publish: two plain stores, one tagged
constexpr int kStU = 2;                // a u wave's u stores
constexpr int kFrag = kNP * kKS * kWTiles * 64;   // W' fragments (16 bytes each) of a member

constexpr uint64_t kSpinTicks = 50000000ull;   // 0.5 s of the 100 MHz clock before giving up

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

// ---------------------------------------------------------------- preparation
// Clears the exchange ring (a tag of 0 matches no tile) and the timeout flag, and cuts
// W' = gamma (.) W of every member into the projection waves' B fragments, in the order
// the waves load them: [member][wave p][k-step ks][column tile nb][lane] x 16 bytes.
// Fragment (ks, nb) of lane (tr, q) holds column 16 nb + tr (as in wsplit3: hi, mid, lo
// of logits 0..23, then padding) for k = 8 q + j <-> stream ks / 2, channel
// 256 m + 64 p + 32 (ks % 2) + 8 q + j.
__global__ __launch_bounds__(256) void k_sr_prep(uint64_t* __restrict__ xch, int64_t nx,
                                                 uint32_t* __restrict__ err, int G, int64_t C,
                                                 const float* __restrict__ gamma,
                                                 const float* __restrict__ W,
                                                 u32x4_t* __restrict__ frag)
{
    using namespace sr;
    // one ring word and one fragment per thread (the grid covers both)
    const int64_t f = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (f < nx) xch[f] = 0ull;
    if (f == 0) err[0] = 0u;
    if (f < (int64_t)G * kFrag) {
        const int lane = (int)(f & 63), tr = lane & 15, q = lane >> 4;
        int64_t r = f >> 6;
        const int nb = (int)(r % kWTiles); r /= kWTiles;
        const int ks = (int)(r % kKS); r /= kKS;
        const int p = (int)(r % kNP);
        const int64_t m = r / kNP;
        const int col = 16 * nb + tr;
        const int kc = wsplit_logit(col), term = wsplit_term(col);
        // the 16 loads first, all unconditional (kc is a valid column on padding lanes
        // too), then the splits: loads held behind a per-lane condition or a branch would
        // go out one at a time, each waited for before the next
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int64_t e = (int64_t)(ks >> 1) * C + m * kMC + kPC * p + 32 * (ks & 1) + 8 * q + j;
            v[j] = gamma[e] * W[e * 24 + kc];
        }
        float o[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j] = wsplit3(term < 3 ? v[j] : 0.f, term < 3 ? term : 0);
        frag[f] = u32x4_t{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]),
                          pack_bf16x2(o[4], o[5]), pack_bf16x2(o[6], o[7])};
    }
}

// ---------------------------------------------------------------- the single-read pass
struct SrArgs {
    int64_t T, C;
    int NG, TPG;                        // groups, tiles per group
    float eps, a0;
    uint32_t tag_skew;                  // 0; a test of the timeout path expects tags that never come
    uint64_t spin_ticks;                // how long a reader waits for a word (100 MHz clock)
    const bf16_t* X;
    const u32x4_t* frag;                // [G][kFrag] W' fragments (k_sr_prep)
    const float* bias;
    bf16_t* u;
    uint64_t* xch;                      // [NG][kRing][80][G]
    float* part;                        // [ntiles][G][16][25]
    float* dummy;                       // per block: 16 KiB of discard space (out-of-range stores)
    uint64_t* dummy64;                  // per block: 4 KiB
    uint32_t* err;                      // spin timeout flag
    // the transform variant: the previous layer's X, F, H_res, H_post in, this layer's X out
    const bf16_t* Xp;
    const bf16_t* Fp;
    const float* Hrp;
    const float* Hpp;
    bf16_t* Xo;
};

// LDS reads at byte addresses by asm, with their wait in the same block: the compiler
// treats any LDS read after a direct-to-LDS load as possibly dependent on it and would
// wait for every load in flight; the explicit counts in the kernel cover these reads.
__device__ __forceinline__ void lds_read16x4(const uint32_t (&ad)[4], u32x4_t& v0, u32x4_t& v1,
                                             u32x4_t& v2, u32x4_t& v3)
{
    asm volatile("ds_read_b128 %0, %4\n\tds_read_b128 %1, %5\n\t"
                 "ds_read_b128 %2, %6\n\tds_read_b128 %3, %7\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(v0), "=&v"(v1), "=&v"(v2), "=&v"(v3)
                 : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3])
                 : "memory");
}
// four 16-byte reads at base + O0 .. base + O3 (byte offsets known at compile time)
template <int O0, int O1, int O2, int O3>
__device__ __forceinline__ void lds_read16x4_at(uint32_t base, u32x4_t& v0, u32x4_t& v1,
                                                u32x4_t& v2, u32x4_t& v3)
{
    asm volatile("ds_read_b128 %0, %4 offset:%5\n\tds_read_b128 %1, %4 offset:%6\n\t"
                 "ds_read_b128 %2, %4 offset:%7\n\tds_read_b128 %3, %4 offset:%8\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(v0), "=&v"(v1), "=&v"(v2), "=&v"(v3)
                 : "v"(base), "i"(O0), "i"(O1), "i"(O2), "i"(O3)
                 : "memory");
}
template <int O0, int O1>
__device__ __forceinline__ void lds_read16x2_at(uint32_t base, u32x4_t& v0, u32x4_t& v1)
{
    asm volatile("ds_read_b128 %0, %2 offset:%3\n\tds_read_b128 %1, %2 offset:%4\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(v0), "=&v"(v1)
                 : "v"(base), "i"(O0), "i"(O1)
                 : "memory");
}
// eight 16-byte reads at base + k S (k = 0..7)
template <int S>
__device__ __forceinline__ void lds_read16x8_at(uint32_t base, u32x4_t (&v)[8])
{
    asm volatile("ds_read_b128 %0, %8\n\tds_read_b128 %1, %8 offset:%9\n\t"
                 "ds_read_b128 %2, %8 offset:%10\n\tds_read_b128 %3, %8 offset:%11\n\t"
                 "ds_read_b128 %4, %8 offset:%12\n\tds_read_b128 %5, %8 offset:%13\n\t"
                 "ds_read_b128 %6, %8 offset:%14\n\tds_read_b128 %7, %8 offset:%15\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]),
                   "=&v"(v[6]), "=&v"(v[7])
                 : "v"(base), "i"(S), "i"(2 * S), "i"(3 * S), "i"(4 * S), "i"(5 * S), "i"(6 * S),
                   "i"(7 * S)
                 : "memory");
}
// Eight or four 8-byte LDS reads S bytes apart, one wait (an exchange lane's words of the
// members, 160 bytes apart)
template <int S>
__device__ __forceinline__ void lds_read8x8_at(uint32_t base, u32x2_t (&v)[8])
{
    asm volatile("ds_read_b64 %0, %8\n\tds_read_b64 %1, %8 offset:%9\n\t"
                 "ds_read_b64 %2, %8 offset:%10\n\tds_read_b64 %3, %8 offset:%11\n\t"
                 "ds_read_b64 %4, %8 offset:%12\n\tds_read_b64 %5, %8 offset:%13\n\t"
                 "ds_read_b64 %6, %8 offset:%14\n\tds_read_b64 %7, %8 offset:%15\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]),
                   "=&v"(v[6]), "=&v"(v[7])
                 : "v"(base), "i"(S), "i"(2 * S), "i"(3 * S), "i"(4 * S), "i"(5 * S), "i"(6 * S),
                   "i"(7 * S)
                 : "memory");
}
template <int S>
__device__ __forceinline__ void lds_read8x4_at(uint32_t base, u32x2_t (&v)[4])
{
    asm volatile("ds_read_b64 %0, %4\n\tds_read_b64 %1, %4 offset:%5\n\t"
                 "ds_read_b64 %2, %4 offset:%6\n\tds_read_b64 %3, %4 offset:%7\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
                 : "v"(base), "i"(S), "i"(2 * S), "i"(3 * S)
                 : "memory");
}
// The transform's LDS traffic: four 16-byte reads at a + S k plus one at b, one wait (the
// X rows of a chunk and its F row: S = 512; a token's H_res and H_post: S = 16); four
// 16-byte writes at a + S k
template <int S>
__device__ __forceinline__ void lds_read16x5(uint32_t a, uint32_t b, u32x4_t (&x)[4], u32x4_t& y)
{
    asm volatile("ds_read_b128 %0, %5\n\tds_read_b128 %1, %5 offset:%7\n\t"
                 "ds_read_b128 %2, %5 offset:%8\n\tds_read_b128 %3, %5 offset:%9\n\t"
                 "ds_read_b128 %4, %6\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(y)
                 : "v"(a), "v"(b), "i"(S), "i"(2 * S), "i"(3 * S)
                 : "memory");
}
template <int S>
__device__ __forceinline__ void lds_write16x4(uint32_t a, const u32x4_t& x0, const u32x4_t& x1,
                                              const u32x4_t& x2, const u32x4_t& x3)
{
    asm volatile("ds_write_b128 %0, %1\n\tds_write_b128 %0, %2 offset:%5\n\t"
                 "ds_write_b128 %0, %3 offset:%6\n\tds_write_b128 %0, %4 offset:%7"
                 :
                 : "v"(a), "v"(x0), "v"(x1), "v"(x2), "v"(x3), "i"(S), "i"(2 * S), "i"(3 * S)
                 : "memory");
}
__device__ __forceinline__ void bf16x8_to_f32(const u32x4_t& x, float (&f)[8])
{
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        f[2 * e] = bf16_lo(w[e]);
        f[2 * e + 1] = bf16_hi(w[e]);
    }
}
// three sums ((x0 + x1) + x2) + x3 of four floats at b + k O (k = 0..3), b = b0, b1, b2
template <int O>
__device__ __forceinline__ void lds_sum4x3(uint32_t b0, uint32_t b1, uint32_t b2, float& s0,
                                           float& s1, float& s2)
{
    float x[12];
    asm volatile("ds_read_b32 %0, %12\n\tds_read_b32 %1, %12 offset:%15\n\t"
                 "ds_read_b32 %2, %12 offset:%16\n\tds_read_b32 %3, %12 offset:%17\n\t"
                 "ds_read_b32 %4, %13\n\tds_read_b32 %5, %13 offset:%15\n\t"
                 "ds_read_b32 %6, %13 offset:%16\n\tds_read_b32 %7, %13 offset:%17\n\t"
                 "ds_read_b32 %8, %14\n\tds_read_b32 %9, %14 offset:%15\n\t"
                 "ds_read_b32 %10, %14 offset:%16\n\tds_read_b32 %11, %14 offset:%17\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]),
                   "=&v"(x[6]), "=&v"(x[7]), "=&v"(x[8]), "=&v"(x[9]), "=&v"(x[10]), "=&v"(x[11])
                 : "v"(b0), "v"(b1), "v"(b2), "i"(O), "i"(2 * O), "i"(3 * O)
                 : "memory");
    s0 = ((x[0] + x[1]) + x[2]) + x[3];
    s1 = ((x[4] + x[5]) + x[6]) + x[7];
    s2 = ((x[8] + x[9]) + x[10]) + x[11];
}
__device__ __forceinline__ void lds_write_f32(uint32_t addr, float v)
{
    asm volatile("ds_write_b32 %0, %1" : : "v"(addr), "v"(v) : "memory");
}

template <int G, bool XF>
__global__ __launch_bounds__(sr::kThreads) void k_fwd_sr(const SrArgs a)
{
    using namespace sr;
    static_assert(g_ok(G), "members per group");
    constexpr int kP = XF ? kPXF : p_of(G), kXI = xi_of(G), kSl = slot_of(XF), oXW = kP * kSl;
    static_assert((XF ? lds_xf(G) : lds_of(kP, G)) + kStaticLds <= 160 * 1024, "LDS budget");
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    __shared__ float pw[2][kNP][kPW];                         // the projection waves' partials
    __shared__ int gave_up;                                   // a re-read timed out: stop waiting
    typedef __attribute__((address_space(3))) void* lds_ptr;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    constexpr int gpx = 32 / G;                               // groups per XCD
    const int xcd = blockIdx.x & 7, l = blockIdx.x >> 3;
    if (l >= gpx * G) return;                                 // spare CU
    const int g = xcd * gpx + l / G, m = l % G;
    const int64_t ntiles = (a.T + kTT - 1) / kTT;
    const int64_t tile0 = (int64_t)g * a.TPG;
    const int ntl = (int)((ntiles - tile0) < a.TPG ? (ntiles - tile0) : a.TPG);
    if (ntl <= 0) return;                                     // the whole group idles
    const int64_t C = a.C, N = 4 * C;
    const int64_t cm = (int64_t)m * kMC;                      // the member's first channel
    // out-of-range stores go to this block's own discard space: stores of many CUs to
    // shared lines would serialise in L2 and hold up every wave's counted operations
    float* const dummy = a.dummy + (int64_t)blockIdx.x * 4096;
    uint64_t* const dummy64 = a.dummy64 + (int64_t)blockIdx.x * 512;
    uint64_t* const xg = a.xch + (int64_t)g * kRing * kPairs * G;
    const uint32_t lbase = (uint32_t)(uintptr_t)(lds_ptr)lds;
    const uint32_t pwbase = (uint32_t)(uintptr_t)(lds_ptr)&pw[0][0][0];
    if (tid == 0) gave_up = 0;
    __syncthreads();
    const int nit = ntl + kD;

    if (wv < kNP) {
        // ================================================= projection wave p
        const int p = wv, tr = lane & 15, q = lane >> 4;
        // A operand addresses within a slot: k-step ks of lane (tr, q) is token tr,
        // stream ks / 2, member chunk 8 p + 4 (ks % 2) + q, stored at position chunk ^ tr
        uint32_t aoff[kKS];
#pragma unroll
        for (int ks = 0; ks < kKS; ++ks)
            aoff[ks] = (uint32_t)((4 * tr + (ks >> 1)) * kRow + (((8 * p + 4 * (ks & 1) + q) ^ tr) << 4));

        // direct-to-LDS: instruction k of wave p covers rows 2 (p + 4 k) and
        // 2 (p + 4 k) + 1 (row = 4 token + stream); lane i of it loads chunk
        // (i & 31) ^ token of its row, so that chunk j of row r sits at position j ^ (r >> 2)
        // (readers of one chunk over 16 tokens hit 16 different 16-byte positions).
        const bf16_t* X = XF ? a.Xp : a.X;
        // (XF) the tile's F rows: instruction k of wave p covers tokens 2 (p + 4 k) and
        // 2 (p + 4 k) + 1 (k < 2), chunks swizzled like X; waves 0 and 2 bring H_res (16
        // bytes a lane: token lane / 4), waves 1 and 3 H_post (4 bytes a lane: token
        // lane / 4) -- the same bytes twice, so that every wave issues the same number of
        // loads and the waits below are constants
        constexpr int kDmaF = XF ? kTT / 2 / kNP : 0;
        constexpr int nhp = XF ? 1 : 0;
        auto dma = [&](int jt, int slot) {
            // jt: local tile index (a tile past the range reads 1 KiB of this block's
            // discard space, over and over, into a slot nobody reads).  Addresses are a
            // wave-uniform base plus a 32-bit byte offset; rows past T repeat the last
            // token's (the offset's token is clamped).
            const bool in = jt < ntl;
            const int64_t t0 = (tile0 + (in ? jt : 0)) * kTT;
            const int tlast = (int)(a.T - 1 - t0);            // the tile's last valid row
            unsigned char* dst = lds + oX + slot * kSl;
            const unsigned char* xb = in ? reinterpret_cast<const unsigned char*>(X + t0 * 4 * C)
                                         : reinterpret_cast<const unsigned char*>(dummy);
#pragma unroll
            for (int k = 0; k < kDmaP; ++k) {
                const int ins = p + kNP * k;                  // rows 2 ins, 2 ins + 1: token ins / 2
                const int tt = ins >> 1, s = 2 * (ins & 1) + (lane >> 5);
                const int tc = tt < tlast ? tt : tlast;
                const uint32_t off = in ? (uint32_t)(((tc * 4 + s) * C + cm + 8 * ((lane & 31) ^ tt)) * 2)
                                        : 16u * (uint32_t)lane;
                __builtin_amdgcn_global_load_lds(xb + off, (lds_ptr)(dst + ins * 1024), 16, 0, 0);
            }
            if constexpr (XF) {
                const unsigned char* fb = in ? reinterpret_cast<const unsigned char*>(a.Fp + t0 * C)
                                             : reinterpret_cast<const unsigned char*>(dummy);
#pragma unroll
                for (int k = 0; k < kDmaF; ++k) {
                    const int tt = 2 * (p + kNP * k) + (lane >> 5);
                    const int tc = tt < tlast ? tt : tlast;
                    const uint32_t off = in ? (uint32_t)((tc * C + cm + 8 * ((lane & 31) ^ tt)) * 2)
                                            : 16u * (uint32_t)lane;
                    __builtin_amdgcn_global_load_lds(fb + off, (lds_ptr)(dst + oF + (p + kNP * k) * 1024), 16,
                                                     0, 0);
                }
                // H_res (16 floats a token) and H_post (4) of the tile are contiguous
                if ((p & 1) == 0) {
                    const unsigned char* hb = in ? reinterpret_cast<const unsigned char*>(a.Hrp + t0 * 16)
                                                 : reinterpret_cast<const unsigned char*>(dummy);
                    const int tc = (lane >> 2) < tlast ? (lane >> 2) : tlast;
                    const uint32_t off = in ? (uint32_t)(tc * 64 + 16 * (lane & 3)) : 16u * (uint32_t)lane;
                    __builtin_amdgcn_global_load_lds(hb + off, (lds_ptr)(dst + oHR), 16, 0, 0);
                } else {
                    const unsigned char* hb = in ? reinterpret_cast<const unsigned char*>(a.Hpp + t0 * 4)
                                                 : reinterpret_cast<const unsigned char*>(dummy);
                    const int tc = (lane >> 2) < tlast ? (lane >> 2) : tlast;
                    const uint32_t off = in ? (uint32_t)(tc * 16 + 4 * (lane & 3)) : 4u * (uint32_t)lane;
                    __builtin_amdgcn_global_load_lds(hb + off, (lds_ptr)(dst + oHP), 4, 0, 0);
                }
            }
        };
        // VMEM operations of this wave: a tile's loads, and per iteration the publish and
        // a tile's loads
        constexpr int tileP = kDmaP + kDmaF + nhp;
        constexpr int iterP = kPubP + tileP;
        // prologue: this wave's W' fragments (lane-contiguous 16-byte loads), then tiles
        // 0 .. kP - 2 into their LDS slots; the loop starts once the fragments and tile 0
        // have landed
        u32x4_t wf[kKS][kWTiles];
        {
            const u32x4_t* fr = a.frag + ((int64_t)m * kNP + p) * (kKS * kWTiles * 64) + lane;
#pragma unroll
            for (int ks = 0; ks < kKS; ++ks)
#pragma unroll
                for (int nb = 0; nb < kWTiles; ++nb) wf[ks][nb] = fr[(ks * kWTiles + nb) * 64];
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < kP - 1; ++j) dma(j, j);
        wait_vmcnt((kP - 2) * tileP);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        // publish: values pub and pub + 256 of a tile (token t = value / 25, k = value % 25)
        const int pub = p * 64 + lane;
        const bool pub1 = pub + 256 < kPW;
        const int pt = pub / kNV, pk = pub % kNV;             // tagged pair pub < 80
        const int ptag = pt * kPV + (pk < 4 ? pk : 24);

        for (int i = 0; i < nit; ++i) {
            // this wave's loads of tile i have landed (every later operation of the wave is
            // counted: the prologue's tiles after i, then each iteration's publish and tile);
            // then every wave's have, and iteration i - 1 is done everywhere
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            static_assert(kP == 3 || kP == 4, "slot counts the waits are written for");
            if (kP == 4 && i == 1)
                wait_vmcnt(tileP + iterP);                    // prologue tile 2, iteration 0
            else
                wait_vmcnt((kP - 2) * iterP);                 // (tile 0: waited for above)
            __builtin_amdgcn_s_waitcnt(0xC07F);               // lgkmcnt(0)
            __builtin_amdgcn_s_barrier();
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            // publish tile jp = i - 1: sums over the projection waves (0..3 in order),
            // values pub and pub + 256 as plain partials for the finishing pass, pair
            // pub < 80 (value k < 4 or 24 of its token) as a word tagged jp + 1
            {
                const int jp = i - 1;
                const bool ok = jp >= 0 && jp < ntl;
                const uint32_t src = pwbase + (uint32_t)((jp & 1) * kNP * kPW * 4);
                float v0, v1, vt;
                lds_sum4x3<kPW * 4>(src + 4u * (uint32_t)pub, src + 4u * (uint32_t)(pub1 ? pub + 256 : pub),
                                    src + 4u * (uint32_t)ptag, v0, v1, vt);
                float* const pbase = a.part + (((tile0 + (ok ? jp : 0)) * G + m) * kTT) * kPV;
                float* const d0 = ok ? pbase + pub : dummy + 2048 + 2 * (p * 64 + lane);
                float* const d1 = ok && pub1 ? pbase + pub + 256 : dummy + 2048 + 2 * (p * 64 + lane) + 1;
                *d0 = v0;
                *d1 = v1;
                const bool tag = ok && pub < kPairs;
                uint64_t* const xd = tag ? xg + ((int64_t)(jp % kRing) * G + m) * kPairs + pub
                                         : dummy64 + 256 + (p * 64 + lane);
                const uint64_t word = ((uint64_t)((uint32_t)jp + 1u) << 32) | __float_as_uint(vt);
                __hip_atomic_store(xd, word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            // tile i + kP - 1 into the slot tile i - 1 used
            dma(i + kP - 1, (i + kP - 1) % kP);
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            if constexpr (XF) {
                // the u waves form this tile's X in place meanwhile
                __builtin_amdgcn_s_waitcnt(0xC07F);           // lgkmcnt(0)
                __builtin_amdgcn_s_barrier();
                __atomic_signal_fence(__ATOMIC_SEQ_CST);
            }
            if (i < ntl) {
                const uint32_t sb = lbase + oX + (uint32_t)((i % kP) * kSl);
                f32x4_t acc[kWTiles];
#pragma unroll
                for (int nb = 0; nb < kWTiles; ++nb) acc[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                float ss = 0.f;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    u32x4_t x4[4];
                    const uint32_t ad[4] = {sb + aoff[4 * h], sb + aoff[4 * h + 1],
                                            sb + aoff[4 * h + 2], sb + aoff[4 * h + 3]};
                    lds_read16x4(ad, x4[0], x4[1], x4[2], x4[3]);
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk) {
                        ss = sumsq8_dot2(x4[kk], ss);
#pragma unroll
                        for (int nb = 0; nb < kWTiles; ++nb)
                            acc[nb] = mfma16(x4[kk], wf[4 * h + kk][nb], acc[nb]);
                    }
                }
                ss += __shfl_xor(ss, 16, 64);
                ss += __shfl_xor(ss, 32, 64);
                // fold the three terms: logit k < 16 on lane k, 16 + k on lane k < 8
                const uint32_t dst = pwbase + (uint32_t)(((i & 1) * kNP + p) * kPW * 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float tv[kWTiles];
#pragma unroll
                    for (int nb = 0; nb < kWTiles; ++nb) tv[nb] = acc[nb][e];
                    float f0, f1;
                    fold3(tv, tr, [](float v) { return lane_ror8(v); }, f0, f1);
                    const int t = 4 * q + e;
                    lds_write_f32(dst + 4u * (uint32_t)(t * kPV + tr), f0);
                    if (tr < 8) lds_write_f32(dst + 4u * (uint32_t)(t * kPV + 16 + tr), f1);
                }
                if (q == 0) lds_write_f32(dst + 4u * (uint32_t)(tr * kPV + 24), ss);
            }
        }
        // the loads past the range land before the block's LDS is given up
        wait_vmcnt(0);
    } else {
        // ================================================= u wave v
        const int v = wv - kNP;
        const int tl = lane >> 4, cc = lane & 15;             // u: token 4 v + tl, chunks cc, cc + 16
        const int ut = kUT * v + tl;                          // tile row of that token
        // exchange: lane xp < 20 sums pair xp of the wave (token 4 v + xp / 5, value
        // xp % 5) over the G members
        const int xp = lane, xt = lane / kNV, xv = lane % kNV;
        const bool xon = lane < kUPairs;
        const float xbias = a.bias[xv < 4 ? xv : 0], a0 = a.a0, eps = a.eps;
        const uint32_t xw_lds = lbase + oXW + (uint32_t)(v * kXI * 1024);
        unsigned char* const xw_dst = lds + oXW + v * kXI * 1024;
        // ring loads within a slot: stream s, chunk cc + 16 hh of token ut sits at row
        // 4 ut + s, position (cc + 16 hh) ^ ut = (cc ^ ut) + 16 hh (ut < 16), i.e. at
        // roff + 512 s + 256 hh
        const uint32_t roff = (uint32_t)(4 * ut * kRow + ((cc ^ ut) << 4));

        // the bias load lands before the loop: a load still in flight at the loop would
        // get a full wait at its first use inside, in every iteration
        wait_vmcnt(0);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);

        u32x4_t xr[kR][8];                                    // the register tile ring

        for (int ib = 0; ib < nit; ib += kR) {
#pragma unroll
            for (int c = 0; c < kR; ++c) {
                const int i = ib + c;
                if (i >= nit) break;
                __atomic_signal_fence(__ATOMIC_SEQ_CST);
                __builtin_amdgcn_s_waitcnt(0xC07F);           // lgkmcnt(0)
                __builtin_amdgcn_s_barrier();
                __atomic_signal_fence(__ATOMIC_SEQ_CST);

                if constexpr (XF) {
                    if (i < ntl) {
                        // 1. (transform) this wave's 4 tokens of tile i formed as
                        // X = H_res X_prev + H_post^T F_prev straight into register slot c (the
                        // arithmetic of k_post_res), written back over X_prev in the LDS slot for
                        // the projection waves, and out to X
                        const uint32_t sb = lbase + oX + (uint32_t)((i % kP) * kSl);
                        u32x4_t hr4[4], hp4;
                        lds_read16x5<16>(sb + (uint32_t)(oHR + ut * 64), sb + (uint32_t)(oHP + ut * 16), hr4, hp4);
                        const float hr[16] = {__uint_as_float(hr4[0].x), __uint_as_float(hr4[0].y),
                                              __uint_as_float(hr4[0].z), __uint_as_float(hr4[0].w),
                                              __uint_as_float(hr4[1].x), __uint_as_float(hr4[1].y),
                                              __uint_as_float(hr4[1].z), __uint_as_float(hr4[1].w),
                                              __uint_as_float(hr4[2].x), __uint_as_float(hr4[2].y),
                                              __uint_as_float(hr4[2].z), __uint_as_float(hr4[2].w),
                                              __uint_as_float(hr4[3].x), __uint_as_float(hr4[3].y),
                                              __uint_as_float(hr4[3].z), __uint_as_float(hr4[3].w)};
                        const float hpv[4] = {__uint_as_float(hp4.x), __uint_as_float(hp4.y),
                                              __uint_as_float(hp4.z), __uint_as_float(hp4.w)};
                        const int64_t tok = (tile0 + i) * kTT + ut;
                        const bool st = tok < a.T;
#pragma unroll
                        for (int hh = 0; hh < 2; ++hh) {
                            // chunk cc + 16 hh of token ut: X rows 4 ut + s at roff + 512 s + 256 hh
                            const uint32_t xa = sb + roff + 256u * (uint32_t)hh;
                            u32x4_t xs[4], fs;
                            lds_read16x5<512>(xa, sb + (uint32_t)(oF + ut * kRow + (((cc ^ ut) + 16 * hh) << 4)), xs, fs);
                            float fv[8];
                            bf16x8_to_f32(fs, fv);
#pragma unroll
                            for (int si = 0; si < 4; ++si) {
                                float o[8];
#pragma unroll
                                for (int e = 0; e < 8; ++e) o[e] = hpv[si] * fv[e];
#pragma unroll
                                for (int j = 0; j < 4; ++j) {
                                    float xv[8];
                                    bf16x8_to_f32(xs[j], xv);
#pragma unroll
                                    for (int e = 0; e < 8; ++e) o[e] = __builtin_fmaf(hr[si * 4 + j], xv[e], o[e]);
                                }
                                xr[c][2 * si + hh] = u32x4_t{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]),
                                                             pack_bf16x2(o[4], o[5]), pack_bf16x2(o[6], o[7])};
                            }
                            lds_write16x4<512>(xa, xr[c][hh], xr[c][2 + hh], xr[c][4 + hh], xr[c][6 + hh]);
#pragma unroll
                            for (int si = 0; si < 4; ++si) {
                                u32x4_t* dst = st ? reinterpret_cast<u32x4_t*>(a.Xo + (tok * 4 + si) * C + cm + 8 * (cc + 16 * hh))
                                                  : reinterpret_cast<u32x4_t*>(dummy) + (2 * (v * 64 + lane) + hh);
                                __builtin_nontemporal_store(xr[c][2 * si + hh], dst);
                            }
                        }
                    }
                    // the whole tile's X is in place before the projection waves read it
                    __atomic_signal_fence(__ATOMIC_SEQ_CST);
                    __builtin_amdgcn_s_waitcnt(0xC07F);       // lgkmcnt(0)
                    __builtin_amdgcn_s_barrier();
                    __atomic_signal_fence(__ATOMIC_SEQ_CST);
                } else if (i < ntl) {
                    // 1. tile i: this wave's 4 tokens into register slot c
                    const uint32_t sb = lbase + oX + (uint32_t)((i % kP) * kSl) + roff;
                    lds_read16x8_at<256>(sb, xr[c]);
                }
                // 2. exchange words of tile jc = i - D (loaded in iteration i - 1; only that
                // iteration's u stores came after them): check their tags, re-read any that
                // are not there yet, member sum
                const int jc = i - kD;
                float tot = 0.f;
                if (jc >= 0 && jc < ntl) {
                    __atomic_signal_fence(__ATOMIC_SEQ_CST);
                    if (XF && i < ntl)
                        wait_vmcnt(kStU + 8);                     // (and the transform's stores)
                    else
                        wait_vmcnt(kStU);
                    __atomic_signal_fence(__ATOMIC_SEQ_CST);
                    // member j's word: value in the lower, tag in the upper half
                    const uint32_t want = (uint32_t)jc + 1u + a.tag_skew;
                    const uint32_t la = xw_lds + (uint32_t)((xon ? xp : 0) * 8);
                    float val[G];
                    uint32_t late = 0;
                    auto take = [&](int j, const u32x2_t& r) {      // member j's word
                        val[j] = __uint_as_float(r.x);
                        late |= (r.y != want ? 1u : 0u) << j;
                    };
                    // G 8-byte words 160 bytes apart, eight (then four) to an asm read
#pragma unroll
                    for (int k = 0; k < G; k += 8) {
                        if (G - k >= 8) {
                            u32x2_t r8[8];
                            lds_read8x8_at<kUPairs * 8>(la + kUPairs * 8 * k, r8);
#pragma unroll
                            for (int j = 0; j < 8; ++j) take(k + j, r8[j]);
                        } else {
                            u32x2_t r4[4];
                            lds_read8x4_at<kUPairs * 8>(la + kUPairs * 8 * k, r4);
#pragma unroll
                            for (int j = 0; j < 4; ++j) take(k + j, r4[j]);
                        }
                    }
                    if (xon) {
                        if (late) {
                            // not all there yet: re-read those words until they are
                            // (bounded in time; a timeout is flagged and poisons u)
                            const uint64_t* src = xg + (int64_t)(jc % kRing) * G * kPairs + kUPairs * v + xp;
                            const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
#pragma unroll
                            for (int j = 0; j < G; ++j) {
                                if (!((late >> j) & 1u)) continue;
                                uint64_t x;
                                bool ok;
                                do {
                                    __builtin_amdgcn_s_sleep(2);
                                    x = __hip_atomic_load(src + j * kPairs, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                                    ok = (uint32_t)(x >> 32) == want;
                                } while (!ok && !__hip_atomic_load(&gave_up, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) &&
                                         __builtin_amdgcn_s_memrealtime() - t0 < a.spin_ticks);
                                if (!ok) {
                                    a.err[0] = 1u;
                                    __hip_atomic_store(&gave_up, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                                    x = 0x7fc00000ull;                // NaN value
                                }
                                val[j] = __uint_as_float((uint32_t)x);
                            }
                        }
                        tot = sr_member_sum(G, [&](int j) { return val[j]; });
                    }
                }
                // 3. exchange words of tile jr = i - E into this wave's LDS words: kXI
                // direct-to-LDS loads at device scope (sc1: past the CU's own cache, which
                // may hold an old copy).  The wave's 20 pairs of member m are 160 contiguous
                // bytes of the ring; piece q = 64 k + lane (member q / 10, pairs
                // 2 (q % 10), + 1) lands at byte 16 q, i.e. word (m, p) at word 20 m + p
                {
                    const int jr = i - kE;
                    const bool ok = jr >= 0 && jr < ntl;
                    // a wave-uniform base and 32-bit byte offsets (out of range: the block's
                    // discard words)
                    const unsigned char* base =
                        ok ? reinterpret_cast<const unsigned char*>(xg + (int64_t)(jr % kRing) * G * kPairs + kUPairs * v)
                           : reinterpret_cast<const unsigned char*>(dummy64);
#pragma unroll
                    for (int k = 0; k < kXI; ++k) {
                        const int q = 64 * k + lane, qm = q / (kUPairs / 2), qw = q - qm * (kUPairs / 2);
                        const uint32_t off = ok && qm < G ? (uint32_t)(qm * kPairs + 2 * qw) * 8u : 16u * (uint32_t)lane;
                        __builtin_amdgcn_global_load_lds(base + off, (lds_ptr)(xw_dst + k * 1024), 16, 0, 16);
                    }
                }
                // 4. H_pre of tile jc for this wave's 4 tokens (the finishing pass's
                // arithmetic), then u of tile jc from register slot (c + 1) % R
                {
                    const bool ok = jc >= 0 && jc < ntl;
                    const float ssum = __shfl(tot, kNV * xt + 4, 64);     // value 4 of the token
                    float hz = 0.f;
                    if (xon && xv < 4)
                        hz = sigmoidf(sr_logit(a0, tot, 1.0f / sr_r(ssum, N, eps), xbias));
                    float h[4];
#pragma unroll
                    for (int s = 0; s < 4; ++s) h[s] = __shfl(hz, kNV * tl + s, 64);
                    const u32x4_t* xv4 = xr[(c + 1) % kR];
                    const int64_t tok = (tile0 + (ok ? jc : 0)) * kTT + ut;
                    const bool st = ok && tok < a.T;
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        float o[8];
#pragma unroll
                        for (int s = 0; s < 4; ++s) {
                            const u32x4_t x = xv4[2 * s + hh];
                            const uint32_t w4[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                // h_0 x_0, then one fused multiply-add per stream (pre_token's order)
                                const float lo = bf16_lo(w4[e]), hi = bf16_hi(w4[e]);
                                o[2 * e] = s == 0 ? h[0] * lo : __builtin_fmaf(h[s], lo, o[2 * e]);
                                o[2 * e + 1] = s == 0 ? h[0] * hi : __builtin_fmaf(h[s], hi, o[2 * e + 1]);
                            }
                        }
                        bf16_t* ud = st ? a.u + tok * C + cm + 8 * (cc + 16 * hh)
                                        : reinterpret_cast<bf16_t*>(dummy) + 8 * (2 * (v * 64 + lane) + hh);
                        store8_nt(ud, o);
                    }
                }
            }
        }
        wait_vmcnt(0);
    }
}

// ---------------------------------------------------------------- finishing pass
// One block of 256 threads per tile: token tile * 16 + tid / 16 on 16 lanes.  Lane q
// sums the members' partial values q and 16 + q (q < 9; value 24 is the sum of squares)
// in the order of sr_member_sum, then forms z, r, the gates, the unscaled projection and
// -- on the same 16 lanes -- the Sinkhorn projection of the res logits (or of injected
// ones).  Tokens past T run on zeros so that every lane takes part in the exchanges.
template <int G>
__global__ __launch_bounds__(256) void k_sr_finish(
    int64_t T, const float* __restrict__ part, int64_t N, float eps,
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
namespace {

struct SrLayout {
    int G, NG, TPG;
    int64_t ntiles, xwords;
    size_t oXch, oPart, oFrag, oDummy, oDummy64, oErr, bytes;
};

SrLayout sr_layout(int64_t T, int64_t C)
{
    SrLayout L{};
    L.G = (int)(C / sr::kMC);
    L.NG = 8 * (32 / L.G);                                  // 32 / G groups on each XCD
    L.ntiles = (T + sr::kTT - 1) / sr::kTT;
    L.TPG = (int)((L.ntiles + L.NG - 1) / L.NG);
    L.xwords = (int64_t)L.NG * sr::kRing * sr::kPairs * L.G;
    size_t o = 0;
    L.oXch = o;     o += align256(sizeof(uint64_t) * (size_t)L.xwords);
    L.oPart = o;    o += align256(sizeof(float) * (size_t)L.ntiles * L.G * sr::kTT * sr::kPV);
    L.oFrag = o;    o += (size_t)L.G * sr::kFrag * 16;     // W' fragments of every member
    L.oDummy = o;   o += 256 * 16384;                       // per block
    L.oDummy64 = o; o += 256 * 4096;
    L.oErr = o;     o += 256;
    L.bytes = o;
    return L;
}

// the kernel and its dynamic LDS for a group size
struct SrKernel {
    const void* fn;
    int lds;
};
template <int G, bool XF>
SrKernel sr_k()
{
    return {reinterpret_cast<const void*>(&k_fwd_sr<G, XF>),
            XF ? sr::lds_xf(G) : sr::lds_of(sr::p_of(G), G)};
}

template <bool XF>
SrKernel sr_kernel_for(int G)
{
    switch (G) {
        case 4: return sr_k<4, XF>();
        case 8: return sr_k<8, XF>();
        case 12: return sr_k<12, XF>();
        case 16: return sr_k<16, XF>();
        case 20: return sr_k<20, XF>();
        case 24: return sr_k<24, XF>();
        case 28: return sr_k<28, XF>();
        default: return sr_k<32, XF>();
    }
}

}  // namespace

// Shapes the single-read pass is built for: bf16, n = 4, C = 256 G with G members per
// group a multiple of 4 (the member sum's quarters) up to the 32 CUs of an XCD; 32 / G
// groups share an XCD (with G = 12, 20, 24, 28 some CUs idle).
bool fwd_sr_shape(int n, int64_t C, int dtype)
{
    if (dtype != MHC_BF16 || n != 4 || C % sr::kMC != 0) return false;
    const int64_t G = C / sr::kMC;
    return sr::g_ok((int)G);
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
            cus == 256) {
            v = 1;
            for (int G = 4; G <= 32; G += 4) {
                for (const SrKernel k : {sr_kernel_for<false>(G), sr_kernel_for<true>(G)})
                    if (hipFuncSetAttribute(k.fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                            k.lds) != hipSuccess)
                        v = 2;
            }
        }
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
                             hipStream_t s, const PostResIn* xf)
{
    const SrLayout L = sr_layout(T, C);
    unsigned char* w = static_cast<unsigned char*>(ws);
    SrArgs a;
    a.T = T; a.C = C; a.NG = L.NG; a.TPG = L.TPG;
    a.eps = eps; a.a0 = alpha[0];
    // MHC_SR_TEST_TIMEOUT (tests only): every reader waits for tags that never come, for
    // 20 us, then gives up -- the timeout path, forced from the host
    const char* te = std::getenv("MHC_SR_TEST_TIMEOUT");
    const bool test_timeout = te && *te && std::strcmp(te, "0") != 0;
    a.tag_skew = test_timeout ? (1u << 30) : 0u;
    a.spin_ticks = test_timeout ? 2000ull : sr::kSpinTicks;
    a.X = static_cast<const bf16_t*>(X); a.bias = bias;
    // the transform variant forms X (its output) from the previous layer's tensors
    a.Xp = xf ? static_cast<const bf16_t*>(xf->X) : nullptr;
    a.Fp = xf ? static_cast<const bf16_t*>(xf->F) : nullptr;
    a.Hrp = xf ? xf->Hres : nullptr;
    a.Hpp = xf ? xf->Hpost : nullptr;
    a.Xo = xf ? static_cast<bf16_t*>(xf->Xout) : nullptr;
    u32x4_t* const frag = reinterpret_cast<u32x4_t*>(w + L.oFrag);
    a.frag = frag;
    a.u = static_cast<bf16_t*>(u);
    a.xch = reinterpret_cast<uint64_t*>(w + L.oXch);
    a.part = reinterpret_cast<float*>(w + L.oPart);
    a.dummy = reinterpret_cast<float*>(w + L.oDummy);
    a.dummy64 = reinterpret_cast<uint64_t*>(w + L.oDummy64);
    a.err = reinterpret_cast<uint32_t*>(w + L.oErr);
    // the ring starts empty (a tag of 0 matches no tile); the W' fragments
    const int64_t nprep = std::max<int64_t>(L.xwords, (int64_t)L.G * sr::kFrag);
    hipLaunchKernelGGL(k_sr_prep, dim3((unsigned)((nprep + 255) / 256)), dim3(256), 0, s, a.xch,
                       L.xwords, a.err, L.G, C, gamma, W, frag);
    const dim3 grid(256), block(sr::kThreads);
    const SrKernel k = xf ? sr_kernel_for<true>(L.G) : sr_kernel_for<false>(L.G);
    void* args[] = {&a};
    const hipError_t e = hipLaunchKernel(k.fn, grid, block, args, (size_t)k.lds, s);
    if (e != hipSuccess) return e;
    // the finishing pass, one instantiation per G (its member sums unrolled, so that the
    // 2 G loads of a lane go out together)
    auto fin = [&](auto gtag) {
        constexpr int GG = decltype(gtag)::value;
        hipLaunchKernelGGL(k_sr_finish<GG>, dim3((unsigned)L.ntiles), dim3(256), 0, s, T,
                           (const float*)a.part, 4 * C, eps, bias, alpha[0], alpha[1], alpha[2],
                           z, rms, Hpre, Hpost, iters, zres_in, Hres, proj);
    };
    switch (L.G) {
        case 4: fin(std::integral_constant<int, 4>{}); break;
        case 8: fin(std::integral_constant<int, 8>{}); break;
        case 12: fin(std::integral_constant<int, 12>{}); break;
        case 16: fin(std::integral_constant<int, 16>{}); break;
        case 20: fin(std::integral_constant<int, 20>{}); break;
        case 24: fin(std::integral_constant<int, 24>{}); break;
        case 28: fin(std::integral_constant<int, 28>{}); break;
        default: fin(std::integral_constant<int, 32>{}); break;
    }
    return hipGetLastError();
}

}  // namespace mhc
