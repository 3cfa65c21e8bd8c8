// mhc_device.hpp -- device helpers for the gfx950 mHC kernels: 16-byte vector
// loads/stores of bf16 or fp32 rows, wave/block reductions, and the per-token
// Sinkhorn-Knopp forward used by several kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mhc {

// bf16 is carried as its 16-bit pattern; float <-> bf16 conversion uses the
// hardware round-to-nearest-even convert of gfx950.
typedef uint16_t bf16_t;
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    bf16x2_t r = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Row I/O of 8 consecutive elements (16 B for bf16, 32 B for fp32).
template <typename Tio> struct io;

template <> struct io<float> {
    static __device__ __forceinline__ void load8(const float* __restrict__ p, float (&v)[8]) {
        const float4 a = *reinterpret_cast<const float4*>(p);
        const float4 b = *reinterpret_cast<const float4*>(p + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
    static __device__ __forceinline__ void store8(float* __restrict__ p, const float (&v)[8]) {
        *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
        *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
    }
    static __device__ __forceinline__ float load1(const float* __restrict__ p) { return *p; }
    static __device__ __forceinline__ void store1(float* __restrict__ p, float v) { *p = v; }
};

template <> struct io<bf16_t> {
    static __device__ __forceinline__ void load8(const bf16_t* __restrict__ p, float (&v)[8]) {
        const uint4 q = *reinterpret_cast<const uint4*>(p);
        v[0] = bf16_lo(q.x); v[1] = bf16_hi(q.x);
        v[2] = bf16_lo(q.y); v[3] = bf16_hi(q.y);
        v[4] = bf16_lo(q.z); v[5] = bf16_hi(q.z);
        v[6] = bf16_lo(q.w); v[7] = bf16_hi(q.w);
    }
    static __device__ __forceinline__ void store8(bf16_t* __restrict__ p, const float (&v)[8]) {
        uint4 q;
        q.x = pack_bf16x2(v[0], v[1]);
        q.y = pack_bf16x2(v[2], v[3]);
        q.z = pack_bf16x2(v[4], v[5]);
        q.w = pack_bf16x2(v[6], v[7]);
        *reinterpret_cast<uint4*>(p) = q;
    }
    static __device__ __forceinline__ float load1(const bf16_t* __restrict__ p) {
        return __uint_as_float(static_cast<uint32_t>(*p) << 16);
    }
    static __device__ __forceinline__ void store1(bf16_t* __restrict__ p, float v) {
        *p = static_cast<bf16_t>(pack_bf16x2(v, 0.f) & 0xffffu);
    }
};

__device__ __forceinline__ void store8_f32(float* __restrict__ p, const float (&v)[8]) {
    io<float>::store8(p, v);
}

// Non-temporal row stores for outputs that nothing in the step reads again (u, X'):
// they do not stay in the caches as dirty lines that a later kernel would have to
// write back.
__device__ __forceinline__ void store8_nt(float* __restrict__ p, const float (&v)[8]) {
    typedef float f4v __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store(f4v{v[0], v[1], v[2], v[3]}, reinterpret_cast<f4v*>(p));
    __builtin_nontemporal_store(f4v{v[4], v[5], v[6], v[7]}, reinterpret_cast<f4v*>(p + 4));
}
__device__ __forceinline__ void store8_nt(bf16_t* __restrict__ p, const float (&v)[8]) {
    typedef uint32_t u4v __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store(u4v{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                    pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])},
                                reinterpret_cast<u4v*>(p));
}

// D += A B on v_mfma_f32_16x16x32_bf16; A lane l holds row l % 16, k = 8 (l / 16) + j;
// B lane l holds column l % 16, same k; D lane l holds rows 4 (l / 16) + i, column l % 16.
__device__ __forceinline__ f32x4_t mfma16(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// W' = gamma (.) W as three bf16 terms, hi + mid + lo: each term is the bf16 rounding of
// what the terms before it leave (exact differences in fp32), so together they carry the
// fp32 value's 24 significant bits.  The projections run on bf16 MFMA with X exact in
// bf16; the three terms are three groups of B columns: 72 columns [hi 0..23 | mid 0..23 |
// lo 0..23], padded to five 16-wide tiles.
constexpr int kWTiles = 5;
// (All three terms are formed and one is selected: no branch, so loads around it are
// not held behind one.)
__device__ __forceinline__ float wsplit3(float v, int term) {
    const float hi = (float)(__bf16)v;
    const float r1 = v - hi;
    const float mid = (float)(__bf16)r1;
    const float lo = (float)(__bf16)(r1 - mid);
    return term == 0 ? hi : (term == 1 ? mid : lo);
}
// B column c of the split (0 <= c < 80): its logit, and its term (3 = padding)
__device__ __forceinline__ int wsplit_logit(int c) { return c < 72 ? c % 24 : 0; }
__device__ __forceinline__ int wsplit_term(int c) { return c < 72 ? c / 24 : 3; }

// Sum of squares of 8 bf16 values in fp32 (exact squares, fp32 adds), as FMAs.
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

// The same sum with the dot-product instruction: each packed pair's two squares (exact in
// fp32: a bf16 product has at most 16 significant bits) added to the accumulator by one
// v_dot2 per pair, four instructions instead of sixteen.  r formed this way stays within
// 2e-7 of the fp64 value at the full-size workloads, as with the FMAs.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float sumsq8_dot2(u32x4_t a, float acc) {
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const bf16x2_t p = __builtin_bit_cast(bf16x2_t, w[i]);
        acc = __builtin_amdgcn_fdot2_f32_bf16(p, p, acc, false);
    }
    return acc;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

// Wave sums of NV <= 32 per-lane values by halving exchanges: with P the next power
// of two >= NV, each of the first log2 P xor-steps sends half of the live values to
// the partner lane and keeps the other half, then a plain butterfly finishes.  That
// is about P + 6 exchanges instead of 6 NV.  Lane l returns the wave total of value
// index l >> (6 - log2 P) (indices >= NV are padding).
template <int NV>
struct wave_rs {
    static_assert(NV >= 1 && NV <= 32, "at most 32 values per call");
    static constexpr int L = NV <= 1 ? 0 : NV <= 2 ? 1 : NV <= 4 ? 2 : NV <= 8 ? 3 : NV <= 16 ? 4 : 5;
    static constexpr int P = 1 << L;
    static constexpr int SH = 6 - L;     // lanes sharing one index: 2^SH
    static __device__ __forceinline__ float run(const float* v) {
        const int lane = threadIdx.x & 63;
        float w[P];
#pragma unroll
        for (int j = 0; j < P; ++j) w[j] = j < NV ? v[j] : 0.f;
#pragma unroll
        for (int st = 0; st < L; ++st) {
            const int m = 32 >> st, half = P >> (st + 1);
            // lanes with bit m set keep the upper half; the choice is made with bit
            // masks so that w is never indexed by a lane-dependent value
            const uint32_t hi = (lane & m) ? 0xffffffffu : 0u;
#pragma unroll
            for (int j = 0; j < P / 2; ++j) {
                if (j < half) {
                    const uint32_t a = __float_as_uint(w[j]), b = __float_as_uint(w[j + half]);
                    const float send = __uint_as_float((a & hi) | (b & ~hi));
                    const float keep = __uint_as_float((b & hi) | (a & ~hi));
                    w[j] = keep + __shfl_xor(send, m, 64);
                }
            }
        }
        float r = w[0];
#pragma unroll
        for (int m = 32 >> L; m >= 1; m >>= 1) r += __shfl_xor(r, m, 64);
        return r;
    }
};

// Sum NV per-thread values over a 256-thread block; the NV totals land in
// out[0..NV) (LDS) and are visible to every thread after the call.
// scratch must hold 4*NV floats.  The order of additions is fixed.
template <int NV>
__device__ __forceinline__ void block_sum_256(float (&v)[NV], float* scratch, float* out) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
    for (int base = 0; base < NV; base += 32) {
        if (NV - base >= 32) {
            const float r = wave_rs<32>::run(v + base);
            if ((lane & 1) == 0) scratch[wv * NV + base + (lane >> 1)] = r;
        } else {
            constexpr int REM = NV % 32 == 0 ? 32 : NV % 32;
            using R = wave_rs<REM>;
            const float r = R::run(v + base);
            const int idx = lane >> R::SH;
            if ((lane & ((1 << R::SH) - 1)) == 0 && idx < REM) scratch[wv * NV + base + idx] = r;
        }
    }
    __syncthreads();
    for (int j = threadIdx.x; j < NV; j += 256)
        out[j] = (scratch[j] + scratch[NV + j]) + (scratch[2 * NV + j] + scratch[3 * NV + j]);
    __syncthreads();
}

__device__ __forceinline__ float sigmoidf(float x) { return 1.0f / (1.0f + expf(-x)); }

// s_waitcnt immediate (gfx9 layout) that waits until at most n vector memory operations
// of this wave are outstanding, leaving the LDS and export counters alone.
constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }
// the same for a wave-uniform n in [0, 63] known only at run time (0 otherwise)
__device__ __forceinline__ void wait_vmcnt(int n) {
    switch (n) {
#define MHC_VMW(i) case i: __builtin_amdgcn_s_waitcnt(vmcnt_imm(i)); break;
#define MHC_VMW8(i) MHC_VMW(i) MHC_VMW(i + 1) MHC_VMW(i + 2) MHC_VMW(i + 3) MHC_VMW(i + 4) \
                    MHC_VMW(i + 5) MHC_VMW(i + 6) MHC_VMW(i + 7)
        MHC_VMW8(8) MHC_VMW8(16) MHC_VMW8(24) MHC_VMW8(32) MHC_VMW8(40) MHC_VMW8(48) MHC_VMW8(56)
        MHC_VMW(1) MHC_VMW(2) MHC_VMW(3) MHC_VMW(4) MHC_VMW(5) MHC_VMW(6) MHC_VMW(7)
#undef MHC_VMW8
#undef MHC_VMW
        default: __builtin_amdgcn_s_waitcnt(vmcnt_imm(0)); break;
    }
}

// ---------------------------------------------------------------- 4x4 block over 16 lanes
// Entry (i, j) of a token's 4x4 block sits in lane 4 i + j of a 16-lane DPP row.
// Row sums combine the 4 lanes of a quad (quad permutations), column sums the lanes
// 8 and then 4 apart (rotations of the 16-lane row, each one DPP operand of an add).
// Every lane of a row (column) gets the bit-identical total: each step adds a lane's
// value and its partner's, both lanes of a pair add the same two values (rotating by
// 8 pairs lanes l and l ^ 8, which then hold equal sums; lanes l + 4 and l - 4 are 8
// apart, so rotating by 4 either way meets the same partner sum), and fp32 addition
// is commutative.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float lane_xor1(float v) { return dpp_mov<0xB1>(v); }   // quad_perm 1,0,3,2
__device__ __forceinline__ float lane_xor2(float v) { return dpp_mov<0x4E>(v); }   // quad_perm 2,3,0,1
__device__ __forceinline__ float lane_ror4(float v) { return dpp_mov<0x124>(v); }   // row_ror:4
__device__ __forceinline__ float lane_ror8(float v) { return dpp_mov<0x128>(v); }   // row_ror:8
__device__ __forceinline__ double lane_ror8_d(double v) {
    const uint64_t b = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_mov_dpp((int)(uint32_t)b, 0x128, 0xF, 0xF, true);
    const int hi = __builtin_amdgcn_mov_dpp((int)(uint32_t)(b >> 32), 0x128, 0xF, 0xF, true);
    return __longlong_as_double((long long)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo));
}

// Fold of the five MFMA column tiles of the three-term projection (D layout: lane holds
// column 16 nb + lane % 16) into the 24 logits: logit k < 16 is hi (tile 0) + mid + lo
// (tile 3) on lane k; logit 16 + k (k < 8) is hi (tile 1) + mid + lo (tile 4) on lane k.
// The mid parts sit 8 lanes over (columns 24..47), brought in by a row rotation.
// Returns the logit of lane % 16 in f0 and, for lane % 16 < 8, logit 16 + lane % 16 in f1.
template <typename V, typename Ror>
__device__ __forceinline__ void fold3(const V (&t)[5], int l16, Ror ror8, V& f0, V& f1) {
    const V r1 = ror8(t[1]), r2 = ror8(t[2]);
    f0 = t[0] + ((l16 < 8 ? r1 : r2) + t[3]);
    f1 = t[1] + (r2 + t[4]);
}

__device__ __forceinline__ float sk16_rowsum(float v) {
    v += lane_xor1(v);
    return v + lane_xor2(v);
}
__device__ __forceinline__ float sk16_colsum(float v) {
    v += lane_ror8(v);
    return v + lane_ror4(v);
}
__device__ __forceinline__ float sk16_rowmax(float v) {
    v = fmaxf(v, lane_xor1(v));
    return fmaxf(v, lane_xor2(v));
}
// exp of the row-shifted logit; the shift cancels in the first row normalisation
__device__ __forceinline__ float sk16_exp0(float z) { return expf(z - sk16_rowmax(z)); }
// Normalisations multiply by the hardware reciprocal (v_rcp_f32, within 1 ulp) of the
// positive row or column sum: the iterations are issue-bound on 16 lanes per token, and
// an IEEE division costs ten instructions.  Over 20 iterations the results move by
// under 1e-6 relative.
__device__ __forceinline__ float sk16_rcp(float s) { return __builtin_amdgcn_rcpf(s); }
__device__ __forceinline__ float sk16_rowstep(float m) { return m * sk16_rcp(sk16_rowsum(m)); }
__device__ __forceinline__ float sk16_colstep(float m) { return m * sk16_rcp(sk16_colsum(m)); }

__device__ __forceinline__ float sinkhorn16_fwd(float z, int iters) {
    float m = sk16_exp0(z);
    for (int s = 0; s < iters; ++s) m = sk16_colstep(sk16_rowstep(m));
    return m;
}

// Sinkhorn-Knopp on one NS x NS logit block held by one thread: M = exp(Z - rowmax),
// then `iters` x (row normalisation, column normalisation).
template <int NS>
__device__ __forceinline__ void sinkhorn_fwd(const float (&zr)[NS * NS], int iters, float (&M)[NS * NS]) {
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        float m = zr[i * NS];
#pragma unroll
        for (int j = 1; j < NS; ++j) m = fmaxf(m, zr[i * NS + j]);
#pragma unroll
        for (int j = 0; j < NS; ++j) M[i * NS + j] = expf(zr[i * NS + j] - m);
    }
    for (int s = 0; s < iters; ++s) {
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            float rs = 0.f;
#pragma unroll
            for (int j = 0; j < NS; ++j) rs += M[i * NS + j];
            const float inv = 1.0f / rs;
#pragma unroll
            for (int j = 0; j < NS; ++j) M[i * NS + j] *= inv;
        }
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
}

}  // namespace mhc
