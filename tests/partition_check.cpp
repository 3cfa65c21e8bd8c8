// Checks of the coefficient backward's work partition (mhc_partition.hpp), compiled
// and run on the CPU by test_partition_host.py.  For each shape: every (slice, step)
// pair belongs to exactly one chunk, no chunk is empty, the table's slice/step starts
// and piece slots agree with the chunk bounds, and the slot count is the most pieces
// any slice has.  Exit status 0 when every check holds.
#include <cstdio>
#include <vector>

#include "mhc_partition.hpp"

using namespace mhc;

static int check(int64_t T, int64_t C)
{
    const int64_t S = C / bp::kSliceCh, U = (T + bp::kStepTok - 1) / bp::kStepTok;
    const BwdChunks ch = bwd_chunks(T, C);
    int bad = 0;
    auto fail = [&](const char* what, int64_t a, int64_t b) {
        if (bad++ < 5) std::printf("T=%lld C=%lld: %s (%lld, %lld)\n", (long long)T, (long long)C, what,
                                   (long long)a, (long long)b);
    };
    if (ch.NB < 1 || ch.NB > kMaxChunks) fail("chunk count", ch.NB, kMaxChunks);
    std::vector<int> owner((size_t)(S * U), -1);
    for (int64_t c = 0; c < ch.NB; ++c) {
        const int64_t x0 = ch.tab.s0[c] * U + ch.tab.u0[c];
        const int64_t x1 = ch.tab.s0[c + 1] * U + ch.tab.u0[c + 1];
        if (x0 != bp::bound(c, S, U, ch.NB)) fail("table start", c, x0);
        if (!(x0 < x1)) fail("empty chunk", c, x1 - x0);
        if (ch.tab.u0[c] < 0 || ch.tab.u0[c] >= U) fail("step start out of range", c, ch.tab.u0[c]);
        for (int64_t x = x0; x < x1 && x < S * U; ++x) {
            if (owner[(size_t)x] != -1) fail("step in two chunks", x, c);
            owner[(size_t)x] = (int)c;
            if (bp::chunk_of(x, S, U, ch.NB) != c) fail("chunk_of", x, c);
        }
    }
    if (ch.tab.s0[ch.NB] * U + ch.tab.u0[ch.NB] != S * U) fail("table end", ch.tab.s0[ch.NB], ch.tab.u0[ch.NB]);
    for (int64_t x = 0; x < S * U; ++x)
        if (owner[(size_t)x] < 0) fail("step in no chunk", x, 0);
    // the first piece's slot: the chunk's place among the chunks that meet its slice
    for (int64_t c = 0; c < ch.NB; ++c) {
        const int64_t s = ch.tab.s0[c];
        if (s < S && ch.tab.r0[c] != c - owner[(size_t)(s * U)]) fail("piece slot", c, ch.tab.r0[c]);
    }
    int64_t most = 1;
    for (int64_t s = 0; s < S; ++s) {
        const int64_t n = owner[(size_t)(s * U + U - 1)] - owner[(size_t)(s * U)] + 1;
        if (n > most) most = n;
    }
    if (most != ch.slots) fail("slot count", most, ch.slots);
    return bad;
}

int main()
{
    const int64_t Cs[] = {128, 256, 384, 1024, 1280, 4096, 7168, 8192, 65536};
    const int64_t Ts[] = {1, 2, 15, 16, 17, 33, 64, 100, 300, 1000, 4096, 16384, 65536};
    int bad = 0, cases = 0;
    for (int64_t C : Cs)
        for (int64_t T : Ts) {
            bad += check(T, C);
            ++cases;
        }
    std::printf("%d shapes, %d failures\n", cases, bad);
    return bad != 0;
}
