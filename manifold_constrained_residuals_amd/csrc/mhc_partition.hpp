// mhc_partition.hpp -- work partition of the streaming coefficient backward.
// Host code in plain C++: the library computes the table and passes it to the kernel
// (mhc_bwd_mfma.hip); the CPU tests compile this header on its own.
#pragma once

#include <cstdint>

namespace mhc {

// ---------------------------------------------------------------- work partition
// The streaming kernel's work is the slice-major sequence of (slice, 16-token step)
// pairs, a slice being 128 channels of all four streams, cut into one chunk per block (at most one block per CU, so one round whatever
// C / 128 is).  A step weighs 64 and the first step of each slice 96 more (the pipeline
// restart of a block whose chunk enters a new slice); the chunks have equal weight.
// The chunks that meet a slice are its pieces, numbered in token order; piece j writes
// partial slot j, and the slots up to the common slot count are zero for slices with
// fewer pieces, so the fixed-order reduction over slots is unchanged.
namespace bp {
constexpr int64_t kSliceCh = 128, kStepTok = 16;
constexpr int64_t kStep = 64, kRestart = 96;
constexpr int64_t kMaxStep = kStep + kRestart;
// weight of the slices before s (s <= S)
inline int64_t before(int64_t s, int64_t U) { return s * (kStep * U + kRestart); }
// weight of the steps before flattened step x
inline int64_t cum(int64_t x, int64_t U) {
    const int64_t s = x / U, u = x - s * U;
    return before(s, U) + (u > 0 ? kRestart + kStep * u : 0);
}
// first flattened step of chunk c (c = NB: the end), the least x with NB cum(x) >= Wt c
inline int64_t bound(int64_t c, int64_t S, int64_t U, int64_t NB) {
    if (c <= 0) return 0;
    if (c >= NB) return S * U;
    const int64_t P = before(S, U) * c;
    int64_t s = (P - 1) / (NB * before(1, U));           // the last slice with NB before(s) < P
    if (s > S - 1) s = S - 1;
    const int64_t rest = P - NB * (before(s, U) + kRestart);
    const int64_t den = NB * kStep;
    int64_t u = rest > 0 ? (rest + den - 1) / den : 1;
    if (u < 1) u = 1;
    return s * U + u;
}
// chunk holding flattened step x (x < S U)
inline int64_t chunk_of(int64_t x, int64_t S, int64_t U, int64_t NB) {
    return NB * cum(x, U) / before(S, U);
}
}  // namespace bp

// The partition as the kernel reads it (a by-value kernel argument): chunk c starts at
// step u0[c] of slice s0[c] and ends where chunk c + 1 starts; its first piece writes
// partial slot r0[c], and any later piece starts its slice, so it writes slot 0.
constexpr int kMaxChunks = 256;
struct BwdChunkTable {
    int32_t u0[kMaxChunks + 1];
    uint16_t s0[kMaxChunks + 1];
    uint8_t r0[kMaxChunks];
};

// chunks (blocks, one per CU at most) of the streaming kernel and the partial slots
// they need: the most pieces any slice is cut into.  Every chunk holds at least one
// step, since a chunk's weight is at least the largest step weight.
struct BwdChunks {
    int64_t NB;
    int slots;
    BwdChunkTable tab;
};
inline BwdChunks bwd_chunks(int64_t T, int64_t C)
{
    const int64_t S = C / bp::kSliceCh, U = (T + bp::kStepTok - 1) / bp::kStepTok;
    BwdChunks ch{};
    int64_t NB = bp::before(S, U) / bp::kMaxStep;
    if (NB > kMaxChunks) NB = kMaxChunks;
    if (NB < 1) NB = 1;
    int64_t P = 1;
    for (int64_t sl = 0; sl < S; ++sl) {
        const int64_t n = bp::chunk_of(sl * U + U - 1, S, U, NB) - bp::chunk_of(sl * U, S, U, NB) + 1;
        if (n > P) P = n;
    }
    for (int64_t c = 0; c <= NB; ++c) {
        const int64_t x = bp::bound(c, S, U, NB);
        ch.tab.s0[c] = (uint16_t)(x / U);
        ch.tab.u0[c] = (int32_t)(x % U);
        if (c < NB) ch.tab.r0[c] = (uint8_t)(c - bp::chunk_of(x / U * U, S, U, NB));
    }
    ch.NB = NB;
    ch.slots = (int)P;
    return ch;
}

}  // namespace mhc
