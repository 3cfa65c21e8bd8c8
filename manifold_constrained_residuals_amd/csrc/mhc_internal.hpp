// mhc_internal.hpp -- host-side launchers of the mHC kernels and the workspace
// layout they share with the C ABI layer.  Arguments reaching a launcher have
// already been validated by mhc_abi.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <initializer_list>
#include <type_traits>

namespace mhc {

// Host-side dispatch of the generic kernels over the supported stream counts
// n in {1, 2, 4, 8} and storage types (fp32, bf16 carried as uint16_t).
template <typename Fn>
inline void for_n(int n, Fn&& fn) {
    switch (n) {
        case 1: fn(std::integral_constant<int, 1>{}); break;
        case 2: fn(std::integral_constant<int, 2>{}); break;
        case 4: fn(std::integral_constant<int, 4>{}); break;
        case 8: fn(std::integral_constant<int, 8>{}); break;
        default: break;
    }
}
template <typename Fn>
inline void for_io(bool bf16, Fn&& fn) {
    if (bf16) fn(uint16_t{});
    else      fn(float{});
}

// MHC_FORCE_PATH (environment, read once per process) selects among kernels that compute
// the same results: "vector" runs the generic VALU kernels for the coefficients and their
// backward at every shape, "twopass" keeps the MFMA kernels but reads X twice in the
// forward read side; unset or any other value picks the fastest path for the shape.
enum { kPathAuto = 0, kPathVector = 1, kPathTwoPass = 2 };
int force_path();

constexpr int kMaxStoredIters = 20;   // Sinkhorn backward keeps up to this many iterates in LDS

inline int K_of(int n) { return n * n + 2 * n; }
inline size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

// Per-token record written by the logit-gradient kernel and read by the
// coefficient-backward kernel: alpha-scaled dz (K floats), 1/r, S/(N r^2).
inline int rec_stride(int n) { return K_of(n) + 2; }

// Token ranges of the deterministic two-stage dW / dgamma reduction.
int bwd_token_ranges(int64_t T, int n, int64_t C);

struct BwdWorkspace {
    float* rec;      // [T][rec_stride]
    float* dz;       // [T][K] (used when the caller passes no dz)
    float* wpart;    // [R][N][K]
    float* gpart;    // [R][N]
    float* dbpart;   // [ceil(T/64)][K] per-64-token sums of dz
    uint16_t* qf;    // MFMA path: dy fragments, [Tp/16][3][64][8] bf16
    uint16_t* qw;    // MFMA path: dW fragments, [Tp/32][3][64][8] bf16
    int R;
    bool mfma;
};
size_t bwd_workspace_bytes(int64_t T, int n, int64_t C, int dtype);
BwdWorkspace bwd_workspace_carve(void* ws, int64_t T, int n, int64_t C, int dtype);

// MFMA path of the coefficient backward (mhc_bwd_mfma.hip)
bool bwd_use_mfma(int64_t T, int n, int64_t C, int dtype);
int bwd_mfma_ranges(int64_t T, int64_t C);         // partial slots the workspace holds
size_t bwd_mfma_frag_bytes(int64_t T);
// returns the partial slots written (and to be reduced)
int launch_bwd_mfma(int64_t T, int64_t C, const void* X, const float* gamma, const float* W,
                    const float* rec, int rs, const uint16_t* qf, const uint16_t* qw,
                    const void* G, const void* g, const float* Hres, const float* Hpre,
                    float* dX, float* wpart, float* gpart, bool dgamma, bool dx_bf16,
                    hipStream_t s);

// Fast coefficient path (bf16, n = 4): bytes of the pre-split projection.
size_t coeffs_workspace_bytes(int64_t T, int n, int64_t C, int dtype);
bool coeffs_use_mfma(int64_t T, int n, int64_t C, int dtype);
// The forward read side in one pass over X (mhc_fwd_sr.hip): the shapes it is built for,
// its workspace, whether this device runs it, and the launch.  The read side's workspace
// covers both paths.
bool fwd_sr_shape(int n, int64_t C, int dtype);
size_t fwd_sr_workspace_bytes(int64_t T, int n, int64_t C, int dtype);
bool fwd_sr_available(int64_t T, int n, int64_t C, int dtype);
// The previous layer's write map and residual merge, X = H_res X_prev + H_post^T F_prev,
// done by the single-read pass itself: it reads X_prev and F_prev, writes X to Xout and
// projects the tile it formed (its own X argument is then not read).
struct PostResIn {
    const void* X;
    const void* F;
    const float* Hres;
    const float* Hpost;
    void* Xout;
};
hipError_t launch_fwd_pre_sr(int64_t T, int64_t C, const void* X, const float* gamma, float eps,
                             const float* W, const float* bias, const float* alpha, float* z,
                             float* rms, float* Hpre, float* Hpost, int iters,
                             const float* zres_in, float* Hres, void* u, float* proj, void* ws,
                             hipStream_t s, const PostResIn* xf = nullptr);
inline size_t fwd_pre_workspace_bytes(int64_t T, int n, int64_t C, int dtype) {
    const size_t a = coeffs_workspace_bytes(T, n, C, dtype), b = fwd_sr_workspace_bytes(T, n, C, dtype);
    return a > b ? a : b;
}

// ---- forward
// proj (nullable): the unscaled normalised projection p / r, [T][K]
hipError_t launch_coeffs(int64_t T, int n, int64_t C, int dtype, const void* X,
                         const float* gamma, float eps, const float* W, const float* bias,
                         const float* alpha, float* z, float* rms, float* Hpre, float* Hpost,
                         int iters, const float* zres_in, float* Hres, float* proj, void* ws,
                         hipStream_t s);
hipError_t launch_sinkhorn(int64_t T, int n, const float* zres, int64_t ld, int iters,
                           float* Hres, hipStream_t s);
// W' = gamma (.) W split into bf16 hi + lo in MFMA fragment order (mhc_fwd.hip); with
// cs > 0, member by member (channel ranges of cs channels of all streams).
void launch_wsplit(int64_t N, int64_t C, int64_t cs, const float* gamma, const float* W,
                   uint16_t* Wp, hipStream_t s);
// Cross-layer fusion (bf16, n = 4, C % 64 == 0): the post + residual pass of layer l
// also writes the next layer's split-K partial projection of X' into the workspace;
// the next layer's read side finishes the logits from them.
bool next_shape_ok(int n, int64_t C, int dtype);
size_t next_workspace_bytes(int64_t T, int64_t C);
hipError_t launch_post_res_next(int64_t T, int64_t C, const void* X, const void* F,
                                const float* Hres, const float* Hpost, void* Xout,
                                const float* gamma_next, const float* W_next, void* ws,
                                hipStream_t s);
hipError_t launch_fwd_pre_from_next(int64_t T, int64_t C, float eps, const float* bias,
                                    const float* alpha, float* z, float* rms, float* Hpre,
                                    float* Hpost, int iters, const float* zres_in, float* Hres,
                                    const void* X, void* u, float* proj, void* ws, hipStream_t s);
// The whole read side (coefficients, gates, Sinkhorn, u = H_pre X); on the MFMA path
// the finishing pass and the read map share one launch.
hipError_t launch_fwd_pre(int64_t T, int n, int64_t C, int dtype, const void* X,
                          const float* gamma, float eps, const float* W, const float* bias,
                          const float* alpha, float* z, float* rms, float* Hpre, float* Hpost,
                          int iters, const float* zres_in, float* Hres, void* u, float* proj,
                          void* ws, hipStream_t s);
// u = H_pre X
hipError_t launch_pre(int64_t T, int n, int64_t C, int dtype, const void* X, const float* Hpre,
                      void* u, hipStream_t s);
hipError_t launch_post_res(int64_t T, int n, int64_t C, int dtype, const void* X,
                           const void* F, const float* Hres, const float* Hpost, void* Xout,
                           hipStream_t s);
// The previous layer's write map and residual merge followed by this layer's read side:
// Xout = H_res X + H_post^T F (as launch_post_res), then launch_fwd_pre on Xout.  The
// single-read pass does both while reading X and F once; elsewhere the two launches run
// in turn.
hipError_t launch_post_res_fwd_pre(int64_t T, int n, int64_t C, int dtype, const void* X,
                                   const void* F, const float* Hres_prev, const float* Hpost_prev,
                                   void* Xout, const float* gamma, float eps, const float* W,
                                   const float* bias, const float* alpha, float* z, float* rms,
                                   float* Hpre, float* Hpost, int iters, const float* zres_in,
                                   float* Hres, void* u, float* proj, void* ws, hipStream_t s);
hipError_t launch_composite(int64_t T, int n, const float* Hres, float* P, float* gr,
                            float* gc, hipStream_t s);

// ---- backward
// With du given, also dH_pre = <du, X_k> from the same pass over X (bitwise the pre
// backward's value).
hipError_t launch_post_res_bwd(int64_t T, int n, int64_t C, int dtype, const void* G,
                               const void* X, const void* F, const float* Hres,
                               const float* Hpost, float* dF, float* dHres, float* dHpost,
                               float* dX, hipStream_t s, const void* du = nullptr,
                               float* dHpre = nullptr);
hipError_t launch_pre_bwd(int64_t T, int n, int64_t C, int dtype, const void* g,
                          const void* X, const float* Hpre, float* dHpre, float* dX,
                          hipStream_t s);
hipError_t launch_sinkhorn_bwd(int64_t T, int n, const float* zres, int64_t ldz, int iters,
                               const float* dHres, float* dzres, int64_t lddz, hipStream_t s);
// Coefficient backward.  When dHres is non-NULL the res-logit gradient is
// recomputed through Sinkhorn from zres (ld ldz); otherwise it is read from dzres.
// When G/g are non-NULL the direct terms H_res^T G + H_pre^T g are added and dX is
// written (fp32, or in the storage dtype when dx_storage is set: the stack runner
// hands it to the layer below that way); otherwise dX (if non-NULL, fp32) is
// accumulated into.
hipError_t launch_coeffs_bwd(int64_t T, int n, int64_t C, int dtype, const void* X,
                             const float* gamma, const float* W, const float* alpha,
                             const float* z, const float* bias, const float* rms,
                             const float* Hpre, const float* Hpost, const float* dHpre,
                             const float* dHpost, const float* dzres,
                             const float* zres, int64_t ldz, const float* dHres, int iters,
                             const void* G, const void* g, const float* Hres,
                             float* dX, float* dW, float* dbias, float* dgamma, float* dz,
                             void* ws, hipStream_t s, bool dx_storage = false,
                             bool sk_done = false);
// n = 4: the pre backward (dH_pre) and the Sinkhorn backward (res logit gradient into
// dzres, row stride lddz) in one launch.  With it, launch_coeffs_bwd is then called
// with sk_done = true and dz = the buffer whose res columns dzres points into.
hipError_t launch_pre_bwd_sk(int64_t T, int64_t C, int dtype, const void* g, const void* X,
                             const float* Hpre, float* dHpre, const float* zres, int64_t ldz,
                             int iters, const float* dHres, float* dzres, int64_t lddz,
                             hipStream_t s);
// Gradient of the logit scales from the forward's unscaled projection p / r and the
// backward's dz.
size_t alpha_bwd_workspace_bytes();

// ---- the optional non-finite check (mhc_check.hip)
// rows x cols elements with row pitch ld; bf16 storage or fp32; p == nullptr is skipped
struct FiniteSpan {
    const void* p;
    int64_t rows, cols, ld;
    bool bf16;
};
inline FiniteSpan f32span(const float* p, int64_t n) { return {p, 1, n, n, false}; }
inline FiniteSpan f32rows(const float* p, int64_t rows, int64_t cols, int64_t ld) {
    return {p, rows, cols, ld, false};
}
inline FiniteSpan iospan(const void* p, int64_t n, int dtype) { return {p, 1, n, n, dtype == 1}; }
bool check_finite_on();
// 0: every element finite; 1: some NaN or Inf; -1: a HIP error.  Synchronises s.
int scan_finite(hipStream_t s, std::initializer_list<FiniteSpan> spans);
hipError_t launch_alpha_bwd(int64_t T, int n, const float* proj, const float* dz, float* dalpha,
                            void* ws, hipStream_t s);

// Layer-block recomputation over a stack of L layers (mhc_stack.hip).
int stack_block_size(int L);
size_t stack_workspace_bytes(int L, int B, int64_t T, int n, int64_t C, int dtype);
hipError_t stack_forward(int L, int B, int64_t T, int n, int64_t C, int dtype, const void* X0,
                         const float* const* gamma, const float* const* W,
                         const float* const* bias, const float* alpha, const void* const* F,
                         void* const* u, float eps, int iters, void* const* Xsave, void* XL,
                         void* ws, hipStream_t s);
hipError_t stack_backward(int L, int B, int64_t T, int n, int64_t C, int dtype,
                          const void* const* Xsave, const float* const* gamma,
                          const float* const* W, const float* const* bias, const float* alpha,
                          const void* const* F, const void* const* du, int iters, const void* GL,
                          float* dX0, float* const* dW, float* const* dbias, float* const* dF,
                          void* ws, hipStream_t s);

}  // namespace mhc
