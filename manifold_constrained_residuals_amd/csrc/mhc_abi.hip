// mhc_abi.hip -- extern "C" entry points of libmhc.so: argument validation on the
// host (before anything is enqueued), workspace checks, then the launchers.
// The semantics of every call are documented in include/mhc.h.
#include <hip/hip_runtime.h>

#include <utility>

#include <atomic>
#include <cmath>
#include <mutex>

#include "mhc_internal.hpp"
#include "../../include/mhc.h"

namespace {

using mhc::K_of;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

int check_shape(int64_t T, int n, int64_t C) {
    if (T < 1 || T > 0x7fffffffLL) return MHC_ERR_SHAPE;
    if (n != 1 && n != 2 && n != 4 && n != 8) return MHC_ERR_SHAPE;
    if (C < 8 || (C % 8) != 0 || C > (1LL << 30)) return MHC_ERR_SHAPE;
    return MHC_OK;
}

int check_dtype(int dtype) { return (dtype == MHC_F32 || dtype == MHC_BF16) ? MHC_OK : MHC_ERR_DTYPE; }

int check_iters(int iters) { return (iters >= 1 && iters <= 10000) ? MHC_OK : MHC_ERR_ITERS; }

// required pointers: non-NULL and 16-byte aligned; optional: aligned when given
int req(std::initializer_list<const void*> ps) {
    for (const void* p : ps) if (!p) return MHC_ERR_NULL;
    for (const void* p : ps) if (!aligned16(p)) return MHC_ERR_ALIGN;
    return MHC_OK;
}
int opt(std::initializer_list<const void*> ps) {
    for (const void* p : ps) if (p && !aligned16(p)) return MHC_ERR_ALIGN;
    return MHC_OK;
}

int check_ws(void* ws, size_t bytes, size_t need) {
    if (need == 0) return MHC_OK;
    if (!ws || bytes < need) return MHC_ERR_WORKSPACE;
    if (!aligned16(ws)) return MHC_ERR_ALIGN;
    return MHC_OK;
}

int finish(hipError_t e) { return e == hipSuccess ? MHC_OK : MHC_ERR_HIP; }

hipStream_t S(void* s) { return reinterpret_cast<hipStream_t>(s); }

#define MHC_TRY(expr) do { const int _st = (expr); if (_st != MHC_OK) return _st; } while (0)

// The optional non-finite check: inputs before any launch, outputs after the kernels
// (each entry point sets `chk` from mhc::check_finite_on()).
int finite_status(int r) { return r == 0 ? MHC_OK : (r > 0 ? MHC_ERR_NONFINITE : MHC_ERR_HIP); }
#define MHC_FINITE_IN(...) \
    do { if (chk) MHC_TRY(finite_status(mhc::scan_finite(S(stream), {__VA_ARGS__}))); } while (0)
#define MHC_FINITE_OUT(st, ...) \
    do { const int _s = (st); \
         if (_s != MHC_OK || !chk) return _s; \
         return finite_status(mhc::scan_finite(S(stream), {__VA_ARGS__})); } while (0)
using mhc::f32span;
using mhc::f32rows;
using mhc::iospan;

constexpr int kStackMaxL = 1 << 16, kStackMaxB = 1024;

// two byte ranges [a, a + na) and [b, b + nb) share a byte
bool overlap(const void* a, size_t na, const void* b, size_t nb)
{
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return na > 0 && nb > 0 && x < y + nb && y < x + na;
}

int check_stack(int L, int B)
{
    if (L < 1 || L > kStackMaxL || B < 1 || B > L || B > kStackMaxB) return MHC_ERR_SHAPE;
    return MHC_OK;
}

// every entry of a host array of device pointers non-NULL and 16-byte aligned
template <typename P>
int req_array(P const* a, int count)
{
    if (!a) return MHC_ERR_NULL;
    for (int i = 0; i < count; ++i) if (!a[i]) return MHC_ERR_NULL;
    for (int i = 0; i < count; ++i) if (!aligned16(a[i])) return MHC_ERR_ALIGN;
    return MHC_OK;
}

// alpha: a host array of 3 finite floats per layer
int check_alpha(const float* alpha, int L = 1)
{
    if (!alpha) return MHC_ERR_NULL;
    for (int i = 0; i < 3 * L; ++i)
        if (!std::isfinite(alpha[i])) return MHC_ERR_VALUE;
    return MHC_OK;
}

// ---- device-resident scratch of mhc_fwd_pre_noalloc
// Each GPU the library runs on holds its own copy of this array from module load until
// the process ends.  In host code `scratch` is only a stand-in for the symbol: its
// device address on the current device comes from hipGetSymbolAddress, taken once per
// device and kept in scratch_dev.
static __device__ __align__(256) unsigned char scratch[MHC_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> scratch_dev[kMaxDevices];
std::mutex scratch_mu;

// device address of the current device's scratch array, or nullptr (with *err set)
void* scratch_ptr(hipError_t* err)
{
    int dev = -1;
    *err = hipGetDevice(&dev);
    if (*err != hipSuccess) return nullptr;
    if (dev < 0 || dev >= kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    void* p = scratch_dev[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lk(scratch_mu);
    p = scratch_dev[dev].load(std::memory_order_relaxed);
    if (!p) {
        *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (*err != hipSuccess || !p) {
            if (*err == hipSuccess) *err = hipErrorInvalidSymbol;
            return nullptr;
        }
        scratch_dev[dev].store(p, std::memory_order_release);
    }
    return p;
}

}  // namespace

extern "C" {

const char* mhc_status_str(int status) {
    switch (status) {
        case MHC_OK: return "MHC_OK: success";
        case MHC_ERR_NULL: return "MHC_ERR_NULL: a required pointer is NULL";
        case MHC_ERR_SHAPE: return "MHC_ERR_SHAPE: need T >= 1, n in {1,2,4,8}, C >= 8 with C % 8 == 0, ld >= n*n";
        case MHC_ERR_ALIGN: return "MHC_ERR_ALIGN: a tensor pointer is not 16-byte aligned";
        case MHC_ERR_DTYPE: return "MHC_ERR_DTYPE: dtype must be MHC_F32 or MHC_BF16";
        case MHC_ERR_ITERS: return "MHC_ERR_ITERS: iters must be in [1, 10000]";
        case MHC_ERR_WORKSPACE: return "MHC_ERR_WORKSPACE: workspace missing or smaller than mhc_workspace_size()";
        case MHC_ERR_HIP: return "MHC_ERR_HIP: a kernel launch failed";
        case MHC_ERR_VALUE: return "MHC_ERR_VALUE: alpha has a non-finite entry";
        case MHC_ERR_NONFINITE: return "MHC_ERR_NONFINITE: a NaN or Inf in an input (nothing computed) or in an output (MHC_CHECK_FINITE)";
        case MHC_ERR_SCRATCH: return "MHC_ERR_SCRATCH: the call needs more scratch than the built-in buffer holds (MHC_NOALLOC_SCRATCH_BYTES)";
        default: return "unknown mhc status";
    }
}

int mhc_abi_version(void) { return 2; }

size_t mhc_workspace_size(int op, int64_t T, int n, int64_t C, int dtype) {
    if (check_shape(T, n, C) != MHC_OK || check_dtype(dtype) != MHC_OK) return 0;
    switch (op) {
        case MHC_OP_COEFFS:
        case MHC_OP_FWD_PRE: return mhc::fwd_pre_workspace_bytes(T, n, C, dtype);
        case MHC_OP_NEXT: return mhc::next_shape_ok(n, C, dtype) ? mhc::next_workspace_bytes(T, C) : 0;
        case MHC_OP_COEFFS_BWD:
        case MHC_OP_BWD_PRE: return mhc::bwd_workspace_bytes(T, n, C, dtype);
        case MHC_OP_ALPHA_BWD: return mhc::alpha_bwd_workspace_bytes();
        default: return 0;
    }
}

int mhc_coeffs(int64_t T, int n, int64_t C, int dtype, const void* X, const float* gamma,
               float eps, const float* W, const float* bias, const float* alpha, float* z,
               float* rms, float* H_pre, float* H_post, float* proj, void* workspace,
               size_t workspace_bytes, void* stream) {
    MHC_TRY(check_shape(T, n, C));
    MHC_TRY(check_dtype(dtype));
    MHC_TRY(check_alpha(alpha));
    MHC_TRY(req({X, gamma, W, bias, z}));
    MHC_TRY(opt({rms, H_pre, H_post, proj}));
    MHC_TRY(check_ws(workspace, workspace_bytes, mhc::coeffs_workspace_bytes(T, n, C, dtype)));
    const bool chk = mhc::check_finite_on();
    MHC_FINITE_IN(iospan(X, T * n * C, dtype), f32span(gamma, n * C), f32span(W, n * C * K_of(n)),
                  f32span(bias, K_of(n)));
    (void)hipGetLastError();
    const int st = finish(mhc::launch_coeffs(T, n, C, dtype, X, gamma, eps, W, bias, alpha, z, rms,
                                             H_pre, H_post, 20, nullptr, nullptr, proj, workspace,
                                             S(stream)));
    MHC_FINITE_OUT(st, f32span(z, T * K_of(n)), f32span(rms, T), f32span(H_pre, T * n),
                   f32span(H_post, T * n), f32span(proj, T * K_of(n)));
}

int mhc_sinkhorn(int64_t T, int n, const float* z_res, int64_t ld_z, int iters, float* H_res,
                 void* stream) {
    MHC_TRY(check_shape(T, n, 8));
    MHC_TRY(check_iters(iters));
    if (!z_res || !H_res) return MHC_ERR_NULL;
    if (ld_z < (int64_t)n * n) return MHC_ERR_SHAPE;
    if (!aligned4(z_res) || !aligned16(H_res)) return MHC_ERR_ALIGN;
    const bool chk = mhc::check_finite_on();
    MHC_FINITE_IN(f32rows(z_res, T, n * n, ld_z));
    (void)hipGetLastError();
    const int st = finish(mhc::launch_sinkhorn(T, n, z_res, ld_z, iters, H_res, S(stream)));
    MHC_FINITE_OUT(st, f32span(H_res, T * n * n));
}

int mhc_pre(int64_t T, int n, int64_t C, int dtype, const void* X, const float* H_pre, void* u,
            void* stream) {
    MHC_TRY(check_shape(T, n, C));
    MHC_TRY(check_dtype(dtype));
    MHC_TRY(req({X, H_pre, u}));
    const bool chk = mhc::check_finite_on();
    MHC_FINITE_IN(iospan(X, T * n * C, dtype), f32span(H_pre, T * n));
    (void)hipGetLastError();
    const int st = finish(mhc::launch_pre(T, n, C, dtype, X, H_pre, u, S(stream)));
    MHC_FINITE_OUT(st, iospan(u, T * C, dtype));
}

int mhc_post_res(int64_t T, int n, int64_t C, int dtype, const void* X, const void* F_out,
                 const float* H_res, const float* H_post, void* X_out, void* stream) {
    MHC_TRY(check_shape(T, n, C));
    MHC_TRY(check_dtype(dtype));
    MHC_TRY(req({X, F_out, H_res, H_post, X_out}));
    if (X_out == X) return MHC_ERR_SHAPE;
    const bool chk = mhc::check_finite_on();
    MHC_FINITE_IN(iospan(X, T * n * C, dtype), iospan(F_out, T * C, dtype),
                  f32span(H_res, T * n * n), f32span(H_post, T * n));
    (void)hipGetLastError();
    const int st = finish(mhc::launch_post_res(T, n, C, dtype, X, F_out, H_res, H_post, X_out,
                                               S(stream)));
    MHC_FINITE_OUT(st, iospan(X_out, T * n * C, dtype));
}

int mhc_post_res_bwd(int64_t T, int n, int64_t C, int dtype, const void* dX_out, const void* X,
                     const void* F_out, const float* H_res, const float* H_post, float* dF,
                     float* dH_res, float* dH_post, float* dX, void* stream) {
    MHC_TRY(check_shape(T, n, C));
    MHC_TRY(check_dtype(dtype));
    MHC_TRY(req({dX_out, X, F_out, H_res, H_post, dF, dH_res, dH_post}));
    MHC_TRY(opt({dX}));
    const bool chk = mhc::check_finite_on();
    MHC_FINITE_IN(iospan(dX_out, T * n * C, dtype), iospan(X, T * n * C, dtype),
                  iospan(F_out, T * C, dtype), f32span(H_res, T * n * n), f32span(H_post, T * n));
    (void)hipGetLastError();
    const int st = finish(mhc::launch_post_res_bwd(T, n, C, dtype, dX_out, X, F_out, H_res, H_post,
                                                   dF, dH_res, dH_post, dX, S(stream)));
    MHC_FINITE_OUT(st, f32span(dF, T * C), f32span(dH_res, T * n * n), f32span(dH_post, T * n),
                   f32span(dX, T * n * C));
}

int mhc_pre_bwd(int64_t T, int n, int64_t C, int dtype, const void* du, const void* X,
                const float* H_pre, float* dH_pre, float* dX, void* stream) {
    MHC_TRY(check_shape(T, n, C));
    MHC_TRY(check_dtype(dtype));
    MHC_TRY(req({du, X, H_pre, dH_pre}));
    MHC_TRY(opt({dX}));
    const bool chk = mhc::check_finite_on();
    MHC_FINITE_IN(iospan(du, T * C, dtype), iospan(X, T * n * C, dtype), f32span(H_pre, T * n));
    (void)hipGetLastError();
    const int st = finish(mhc::launch_pre_bwd(T, n, C, dtype, du, X, H_pre, dH_pre, dX, S(stream)));
    MHC_FINITE_OUT(st, f32span(dH_pre, T * n), f32span(dX, T * n * C));
}

int mhc_sinkhorn_bwd(int64_t T, int n, const float* z_res, int64_t ld_z, int iters,
                     const float* dH_res, float* dz_res, int64_t ld_dz, void* stream) {
    MHC_TRY(check_shape(T, n, 8));
    MHC_TRY(check_iters(iters));
    if (!z_res || !dH_res || !dz_res) return MHC_ERR_NULL;
    if (ld_z < (int64_t)n * n || ld_dz < (int64_t)n * n) return MHC_ERR_SHAPE;
    if (!aligned4(z_res) || !aligned4(dz_res) || !aligned16(dH_res)) return MHC_ERR_ALIGN;
    const bool chk = mhc::check_finite_on();
    MHC_FINITE_IN(f32rows(z_res, T, n * n, ld_z), f32span(dH_res, T * n * n));
    (void)hipGetLastError();
    const int st = finish(mhc::launch_sinkhorn_bwd(T, n, z_res, ld_z, iters, dH_res, dz_res, ld_dz,
                                                   S(stream)));
    MHC_FINITE_OUT(st, f32rows(dz_res, T, n * n, ld_dz));
}

int mhc_coeffs_bwd(int64_t T, int n, int64_t C, int dtype, const void* X, const float* gamma,
                   const float* W, const float* alpha, const float* z, const float* bias,
                   const float* rms, const float* H_pre, const float* H_post,
                   const float* dH_pre, const float* dH_post, const float* dz_res, float* dX,
                   float* dW, float* dbias, float* dgamma, float* dz, void* workspace,
                   size_t workspace_bytes, void* stream) {
    MHC_TRY(check_shape(T, n, C));
    MHC_TRY(check_dtype(dtype));
    MHC_TRY(check_alpha(alpha));
    MHC_TRY(req({X, gamma, W, z, bias, rms, H_pre, H_post, dH_pre, dH_post, dz_res, dW, dbias}));
    MHC_TRY(opt({dX, dgamma, dz}));
    MHC_TRY(check_ws(workspace, workspace_bytes, mhc::bwd_workspace_bytes(T, n, C, dtype)));
    const bool chk = mhc::check_finite_on();
    MHC_FINITE_IN(iospan(X, T * n * C, dtype), f32span(gamma, n * C), f32span(W, n * C * K_of(n)),
                  f32span(z, T * K_of(n)), f32span(bias, K_of(n)), f32span(rms, T),
                  f32span(H_pre, T * n), f32span(H_post, T * n), f32span(dH_pre, T * n),
                  f32span(dH_post, T * n), f32span(dz_res, T * n * n));
    (void)hipGetLastError();
    const int st = finish(mhc::launch_coeffs_bwd(T, n, C, dtype, X, gamma, W, alpha, z, bias, rms,
                                                 H_pre, H_post, dH_pre, dH_post, dz_res, nullptr, 0,
                                                 nullptr, 20, nullptr, nullptr, nullptr, dX, dW,
                                                 dbias, dgamma, dz, workspace, S(stream)));
    MHC_FINITE_OUT(st, f32span(dX, T * n * C), f32span(dW, n * C * K_of(n)),
                   f32span(dbias, K_of(n)), f32span(dgamma, n * C), f32span(dz, T * K_of(n)));
}

int mhc_fwd_pre(int64_t T, int n, int64_t C, int dtype, const void* X, const float* gamma,
                float eps, const float* W, const float* bias, const float* alpha, int iters,
                const float* z_res_in, float* z, float* rms, float* H_pre, float* H_post,
                float* H_res, void* u, float* proj, void* workspace, size_t workspace_bytes,
                void* stream) {
    MHC_TRY(check_shape(T, n, C));
    MHC_TRY(check_dtype(dtype));
    MHC_TRY(check_iters(iters));
    MHC_TRY(check_alpha(alpha));
    MHC_TRY(req({X, gamma, W, bias, z, rms, H_pre, H_post, H_res, u}));
    MHC_TRY(opt({z_res_in, proj}));
    MHC_TRY(check_ws(workspace, workspace_bytes, mhc::fwd_pre_workspace_bytes(T, n, C, dtype)));
    const bool chk = mhc::check_finite_on();
    MHC_FINITE_IN(iospan(X, T * n * C, dtype), f32span(gamma, n * C), f32span(W, n * C * K_of(n)),
                  f32span(bias, K_of(n)), f32span(z_res_in, T * n * n));
    (void)hipGetLastError();
    // coefficients and gates, then Sinkhorn-Knopp of the res logits (or of the
    // injected ones), then u
    const int st = finish(mhc::launch_fwd_pre(T, n, C, dtype, X, gamma, eps, W, bias, alpha, z, rms,
                                              H_pre, H_post, iters, z_res_in, H_res, u, proj,
                                              workspace, S(stream)));
    MHC_FINITE_OUT(st, f32span(z, T * K_of(n)), f32span(rms, T), f32span(H_pre, T * n),
                   f32span(H_post, T * n), f32span(H_res, T * n * n), iospan(u, T * C, dtype),
                   f32span(proj, T * K_of(n)));
}

int mhc_post_res_fwd_pre(int64_t T, int n, int64_t C, int dtype, const void* X,
                         const void* F_out, const float* H_res, const float* H_post, void* X_out,
                         const float* gamma, float eps, const float* W, const float* bias,
                         const float* alpha, int iters, const float* z_res_in, float* z,
                         float* rms, float* H_pre_next, float* H_post_next, float* H_res_next,
                         void* u, float* proj, void* workspace, size_t workspace_bytes,
                         void* stream) {
    MHC_TRY(check_shape(T, n, C));
    MHC_TRY(check_dtype(dtype));
    MHC_TRY(check_iters(iters));
    MHC_TRY(check_alpha(alpha));
    MHC_TRY(req({X, F_out, H_res, H_post, X_out, gamma, W, bias, z, rms, H_pre_next, H_post_next,
                 H_res_next, u}));
    MHC_TRY(opt({z_res_in, proj}));
    {
        // the pass reads X, F_out and this layer's maps while it writes X_out, u and the
        // next layer's maps: no written buffer may overlap one it reads
        const size_t s = dtype == MHC_BF16 ? 2 : 4;
        const size_t bx = (size_t)(T * n * C) * s, bf = (size_t)(T * C) * s;
        const size_t bhr = sizeof(float) * (size_t)(T * n * n), bhp = sizeof(float) * (size_t)(T * n);
        const std::pair<const void*, size_t> in[] = {{X, bx}, {F_out, bf}, {H_res, bhr}, {H_post, bhp}};
        const std::pair<const void*, size_t> out[] = {{X_out, bx}, {u, bf}, {H_res_next, bhr},
                                                      {H_post_next, bhp}};
        for (const auto& o : out)
            for (const auto& i : in)
                if (overlap(o.first, o.second, i.first, i.second)) return MHC_ERR_SHAPE;
    }
    MHC_TRY(check_ws(workspace, workspace_bytes, mhc::fwd_pre_workspace_bytes(T, n, C, dtype)));
    const bool chk = mhc::check_finite_on();
    MHC_FINITE_IN(iospan(X, T * n * C, dtype), iospan(F_out, T * C, dtype),
                  f32span(H_res, T * n * n), f32span(H_post, T * n), f32span(gamma, n * C),
                  f32span(W, n * C * K_of(n)), f32span(bias, K_of(n)),
                  f32span(z_res_in, T * n * n));
    (void)hipGetLastError();
    const int st = finish(mhc::launch_post_res_fwd_pre(
        T, n, C, dtype, X, F_out, H_res, H_post, X_out, gamma, eps, W, bias, alpha, z, rms,
        H_pre_next, H_post_next, iters, z_res_in, H_res_next, u, proj, workspace, S(stream)));
    MHC_FINITE_OUT(st, iospan(X_out, T * n * C, dtype), f32span(z, T * K_of(n)), f32span(rms, T),
                   f32span(H_pre_next, T * n), f32span(H_post_next, T * n),
                   f32span(H_res_next, T * n * n), iospan(u, T * C, dtype),
                   f32span(proj, T * K_of(n)));
}

int mhc_fwd_pre_noalloc(int64_t T, int n, int64_t C, int dtype, const void* X,
                        const float* gamma, float eps, const float* W, const float* bias,
                        const float* alpha, int iters, const float* z_res_in, float* z,
                        float* rms, float* H_pre, float* H_post, float* H_res, void* u,
                        float* proj, void* stream) {
    MHC_TRY(check_shape(T, n, C));
    MHC_TRY(check_dtype(dtype));
    MHC_TRY(check_iters(iters));
    MHC_TRY(check_alpha(alpha));
    MHC_TRY(req({X, gamma, W, bias, z, rms, H_pre, H_post, H_res, u}));
    MHC_TRY(opt({z_res_in, proj}));
    const size_t need = mhc::fwd_pre_workspace_bytes(T, n, C, dtype);
    if (need > (size_t)MHC_NOALLOC_SCRATCH_BYTES) return MHC_ERR_SCRATCH;
    void* ws = nullptr;
    if (need > 0) {
        hipError_t e = hipSuccess;
        ws = scratch_ptr(&e);
        if (!ws) return MHC_ERR_HIP;
    }
    const bool chk = mhc::check_finite_on();
    MHC_FINITE_IN(iospan(X, T * n * C, dtype), f32span(gamma, n * C), f32span(W, n * C * K_of(n)),
                  f32span(bias, K_of(n)), f32span(z_res_in, T * n * n));
    (void)hipGetLastError();
    // the same launches as mhc_fwd_pre, with the device array as the workspace: the
    // exchange ring's tags are cleared by the first launch of the call, and every other
    // byte the kernels read is written earlier in the same call
    const int st = finish(mhc::launch_fwd_pre(T, n, C, dtype, X, gamma, eps, W, bias, alpha, z, rms,
                                              H_pre, H_post, iters, z_res_in, H_res, u, proj, ws,
                                              S(stream)));
    MHC_FINITE_OUT(st, f32span(z, T * K_of(n)), f32span(rms, T), f32span(H_pre, T * n),
                   f32span(H_post, T * n), f32span(H_res, T * n * n), iospan(u, T * C, dtype),
                   f32span(proj, T * K_of(n)));
}

int mhc_bwd_pre(int64_t T, int n, int64_t C, int dtype, const void* dX_out, const void* du,
                const void* X, const float* gamma, const float* W, const float* alpha,
                const float* z, const float* bias, const float* rms, const float* H_pre,
                const float* H_post, const float* H_res, const float* dH_res,
                const float* dH_post, int iters, const float* z_res_in, float* dX, float* dW,
                float* dbias, float* dH_pre, float* dz, float* dgamma, void* workspace,
                size_t workspace_bytes, void* stream) {
    MHC_TRY(check_shape(T, n, C));
    MHC_TRY(check_dtype(dtype));
    MHC_TRY(check_iters(iters));
    MHC_TRY(check_alpha(alpha));
    MHC_TRY(req({dX_out, du, X, gamma, W, z, bias, rms, H_pre, H_post, H_res, dH_res, dH_post,
                 dX, dW, dbias, dH_pre, dz}));
    MHC_TRY(opt({z_res_in, dgamma}));
    MHC_TRY(check_ws(workspace, workspace_bytes, mhc::bwd_workspace_bytes(T, n, C, dtype)));
    const bool chk = mhc::check_finite_on();
    MHC_FINITE_IN(iospan(dX_out, T * n * C, dtype), iospan(du, T * C, dtype),
                  iospan(X, T * n * C, dtype), f32span(gamma, n * C), f32span(W, n * C * K_of(n)),
                  f32span(z, T * K_of(n)), f32span(bias, K_of(n)), f32span(rms, T),
                  f32span(H_pre, T * n), f32span(H_post, T * n), f32span(H_res, T * n * n),
                  f32span(z_res_in, T * n * n), f32span(dH_res, T * n * n),
                  f32span(dH_post, T * n));
    (void)hipGetLastError();
    const float* zres = z_res_in ? z_res_in : z + 2 * n;
    const int64_t ldz = z_res_in ? (int64_t)n * n : K_of(n);
    // n = 4: the Sinkhorn backward rides in the pre backward's launch, into dz's res columns
    const bool fused = n == 4;
    const hipError_t e =
        fused ? mhc::launch_pre_bwd_sk(T, C, dtype, du, X, H_pre, dH_pre, zres, ldz, iters, dH_res,
                                       dz + 2 * n, K_of(n), S(stream))
              : mhc::launch_pre_bwd(T, n, C, dtype, du, X, H_pre, dH_pre, nullptr, S(stream));
    if (e != hipSuccess) return MHC_ERR_HIP;
    const int st = finish(mhc::launch_coeffs_bwd(T, n, C, dtype, X, gamma, W, alpha, z, bias, rms,
                                                 H_pre, H_post, dH_pre, dH_post, nullptr, zres, ldz,
                                                 dH_res, iters, dX_out, du, H_res, dX, dW, dbias,
                                                 dgamma, dz, workspace, S(stream), false, fused));
    MHC_FINITE_OUT(st, f32span(dX, T * n * C), f32span(dW, n * C * K_of(n)),
                   f32span(dbias, K_of(n)), f32span(dH_pre, T * n), f32span(dz, T * K_of(n)),
                   f32span(dgamma, n * C));
}

int mhc_post_res_bwd_pre(int64_t T, int n, int64_t C, int dtype, const void* dX_out,
                         const void* du, const void* X, const void* F_out, const float* H_res,
                         const float* H_post, float* dF, float* dH_res, float* dH_post,
                         float* dH_pre, void* stream) {
    MHC_TRY(check_shape(T, n, C));
    MHC_TRY(check_dtype(dtype));
    MHC_TRY(req({dX_out, du, X, F_out, H_res, H_post, dF, dH_res, dH_post, dH_pre}));
    const bool chk = mhc::check_finite_on();
    MHC_FINITE_IN(iospan(dX_out, T * n * C, dtype), iospan(du, T * C, dtype),
                  iospan(X, T * n * C, dtype), iospan(F_out, T * C, dtype),
                  f32span(H_res, T * n * n), f32span(H_post, T * n));
    (void)hipGetLastError();
    const int st = finish(mhc::launch_post_res_bwd(T, n, C, dtype, dX_out, X, F_out, H_res, H_post,
                                                   dF, dH_res, dH_post, nullptr, S(stream), du,
                                                   dH_pre));
    MHC_FINITE_OUT(st, f32span(dF, T * C), f32span(dH_res, T * n * n), f32span(dH_post, T * n),
                   f32span(dH_pre, T * n));
}

int mhc_bwd_pre_from_dh(int64_t T, int n, int64_t C, int dtype, const void* dX_out,
                        const void* du, const void* X, const float* gamma, const float* W,
                        const float* alpha, const float* z, const float* bias, const float* rms,
                        const float* H_pre, const float* H_post, const float* H_res,
                        const float* dH_pre, const float* dH_res, const float* dH_post, int iters,
                        const float* z_res_in, float* dX, float* dW, float* dbias, float* dz,
                        float* dgamma, void* workspace, size_t workspace_bytes, void* stream) {
    MHC_TRY(check_shape(T, n, C));
    MHC_TRY(check_dtype(dtype));
    MHC_TRY(check_iters(iters));
    MHC_TRY(check_alpha(alpha));
    MHC_TRY(req({dX_out, du, X, gamma, W, z, bias, rms, H_pre, H_post, H_res, dH_pre, dH_res,
                 dH_post, dX, dW, dbias, dz}));
    MHC_TRY(opt({z_res_in, dgamma}));
    MHC_TRY(check_ws(workspace, workspace_bytes, mhc::bwd_workspace_bytes(T, n, C, dtype)));
    const bool chk = mhc::check_finite_on();
    MHC_FINITE_IN(iospan(dX_out, T * n * C, dtype), iospan(du, T * C, dtype),
                  iospan(X, T * n * C, dtype), f32span(gamma, n * C), f32span(W, n * C * K_of(n)),
                  f32span(z, T * K_of(n)), f32span(bias, K_of(n)), f32span(rms, T),
                  f32span(H_pre, T * n), f32span(H_post, T * n), f32span(H_res, T * n * n),
                  f32span(z_res_in, T * n * n), f32span(dH_pre, T * n), f32span(dH_res, T * n * n),
                  f32span(dH_post, T * n));
    (void)hipGetLastError();
    const float* zres = z_res_in ? z_res_in : z + 2 * n;
    const int64_t ldz = z_res_in ? (int64_t)n * n : K_of(n);
    // the Sinkhorn backward runs on its own (16 lanes per token at n = 4) into dz's res
    // columns; the logit-gradient kernel reads them there
    const int st = finish(mhc::launch_coeffs_bwd(T, n, C, dtype, X, gamma, W, alpha, z, bias, rms,
                                                 H_pre, H_post, dH_pre, dH_post, nullptr, zres, ldz,
                                                 dH_res, iters, dX_out, du, H_res, dX, dW, dbias,
                                                 dgamma, dz, workspace, S(stream), false, false));
    MHC_FINITE_OUT(st, f32span(dX, T * n * C), f32span(dW, n * C * K_of(n)),
                   f32span(dbias, K_of(n)), f32span(dz, T * K_of(n)), f32span(dgamma, n * C));
}

int mhc_post_res_next(int64_t T, int n, int64_t C, int dtype, const void* X,
                      const void* F_out, const float* H_res, const float* H_post,
                      void* X_out, const float* gamma_next, const float* W_next,
                      void* workspace, size_t workspace_bytes, void* stream) {
    MHC_TRY(check_shape(T, n, C));
    MHC_TRY(check_dtype(dtype));
    if (dtype != MHC_BF16) return MHC_ERR_DTYPE;
    if (!mhc::next_shape_ok(n, C, dtype)) return MHC_ERR_SHAPE;
    MHC_TRY(req({X, F_out, H_res, H_post, X_out, gamma_next, W_next}));
    MHC_TRY(check_ws(workspace, workspace_bytes, mhc::next_workspace_bytes(T, C)));
    const bool chk = mhc::check_finite_on();
    MHC_FINITE_IN(iospan(X, T * n * C, dtype), iospan(F_out, T * C, dtype),
                  f32span(H_res, T * n * n), f32span(H_post, T * n), f32span(gamma_next, n * C),
                  f32span(W_next, n * C * K_of(n)));
    (void)hipGetLastError();
    const int st = finish(mhc::launch_post_res_next(T, C, X, F_out, H_res, H_post, X_out,
                                                    gamma_next, W_next, workspace, S(stream)));
    MHC_FINITE_OUT(st, iospan(X_out, T * n * C, dtype));
}

int mhc_fwd_pre_next(int64_t T, int n, int64_t C, int dtype, const void* X, float eps,
                     const float* bias, const float* alpha, int iters,
                     const float* z_res_in, float* z, float* rms, float* H_pre,
                     float* H_post, float* H_res, void* u, float* proj, void* workspace,
                     size_t workspace_bytes, void* stream) {
    MHC_TRY(check_shape(T, n, C));
    MHC_TRY(check_dtype(dtype));
    if (dtype != MHC_BF16) return MHC_ERR_DTYPE;
    if (!mhc::next_shape_ok(n, C, dtype)) return MHC_ERR_SHAPE;
    MHC_TRY(check_iters(iters));
    MHC_TRY(check_alpha(alpha));
    MHC_TRY(req({X, bias, z, rms, H_pre, H_post, H_res, u}));
    MHC_TRY(opt({z_res_in, proj}));
    MHC_TRY(check_ws(workspace, workspace_bytes, mhc::next_workspace_bytes(T, C)));
    const bool chk = mhc::check_finite_on();
    MHC_FINITE_IN(iospan(X, T * n * C, dtype), f32span(bias, K_of(n)),
                  f32span(z_res_in, T * n * n));
    (void)hipGetLastError();
    const int st = finish(mhc::launch_fwd_pre_from_next(T, C, eps, bias, alpha, z, rms, H_pre,
                                                        H_post, iters, z_res_in, H_res, X, u, proj,
                                                        workspace, S(stream)));
    MHC_FINITE_OUT(st, f32span(z, T * K_of(n)), f32span(rms, T), f32span(H_pre, T * n),
                   f32span(H_post, T * n), f32span(H_res, T * n * n), iospan(u, T * C, dtype),
                   f32span(proj, T * K_of(n)));
}

int mhc_alpha_bwd(int64_t T, int n, const float* proj, const float* dz, float* dalpha,
                  void* workspace, size_t workspace_bytes, void* stream) {
    MHC_TRY(check_shape(T, n, 8));
    MHC_TRY(req({proj, dz, dalpha}));
    MHC_TRY(check_ws(workspace, workspace_bytes, mhc::alpha_bwd_workspace_bytes()));
    const bool chk = mhc::check_finite_on();
    MHC_FINITE_IN(f32span(proj, T * K_of(n)), f32span(dz, T * K_of(n)));
    (void)hipGetLastError();
    const int st = finish(mhc::launch_alpha_bwd(T, n, proj, dz, dalpha, workspace, S(stream)));
    MHC_FINITE_OUT(st, f32span(dalpha, 3));
}


int mhc_stack_block_size(int L) { return (L < 1 || L > kStackMaxL) ? 0 : mhc::stack_block_size(L); }

size_t mhc_stack_workspace_size(int L, int B, int64_t T, int n, int64_t C, int dtype) {
    if (check_stack(L, B) != MHC_OK || check_shape(T, n, C) != MHC_OK || check_dtype(dtype) != MHC_OK)
        return 0;
    return mhc::stack_workspace_bytes(L, B, T, n, C, dtype);
}

int mhc_stack_forward(int L, int B, int64_t T, int n, int64_t C, int dtype, const void* X0,
                      const float* const* gamma, const float* const* W, const float* const* bias,
                      const float* alpha, const void* const* F_out, void* const* u, float eps,
                      int iters, void* const* X_save, void* X_L, void* workspace,
                      size_t workspace_bytes, void* stream) {
    MHC_TRY(check_stack(L, B));
    MHC_TRY(check_shape(T, n, C));
    MHC_TRY(check_dtype(dtype));
    MHC_TRY(check_iters(iters));
    MHC_TRY(req({X0, X_L}));
    MHC_TRY(req_array(gamma, L));
    MHC_TRY(req_array(W, L));
    MHC_TRY(req_array(bias, L));
    MHC_TRY(req_array(F_out, L));
    MHC_TRY(req_array(X_save, (L + B - 1) / B));
    if (u) MHC_TRY(req_array(u, L));
    MHC_TRY(check_alpha(alpha, L));
    for (int i = 0; i < (L + B - 1) / B; ++i)
        if (X_save[i] == X_L) return MHC_ERR_SHAPE;
    MHC_TRY(check_ws(workspace, workspace_bytes, mhc::stack_workspace_bytes(L, B, T, n, C, dtype)));
    (void)hipGetLastError();
    return finish(mhc::stack_forward(L, B, T, n, C, dtype, X0, gamma, W, bias, alpha, F_out, u, eps,
                                     iters, X_save, X_L, workspace, S(stream)));
}

int mhc_stack_backward(int L, int B, int64_t T, int n, int64_t C, int dtype,
                       const void* const* X_save, const float* const* gamma, const float* const* W,
                       const float* const* bias, const float* alpha, const void* const* F_out,
                       const void* const* du, int iters, const void* dX_L, float* dX0,
                       float* const* dW, float* const* dbias, float* const* dF,
                       void* workspace, size_t workspace_bytes, void* stream) {
    MHC_TRY(check_stack(L, B));
    MHC_TRY(check_shape(T, n, C));
    MHC_TRY(check_dtype(dtype));
    MHC_TRY(check_iters(iters));
    MHC_TRY(req({dX_L, dX0}));
    MHC_TRY(req_array(X_save, (L + B - 1) / B));
    MHC_TRY(req_array(gamma, L));
    MHC_TRY(req_array(W, L));
    MHC_TRY(req_array(bias, L));
    MHC_TRY(req_array(F_out, L));
    MHC_TRY(req_array(du, L));
    MHC_TRY(req_array(dW, L));
    MHC_TRY(req_array(dbias, L));
    if (dF) MHC_TRY(req_array(dF, L));
    MHC_TRY(check_alpha(alpha, L));
    MHC_TRY(check_ws(workspace, workspace_bytes, mhc::stack_workspace_bytes(L, B, T, n, C, dtype)));
    (void)hipGetLastError();
    return finish(mhc::stack_backward(L, B, T, n, C, dtype, X_save, gamma, W, bias, alpha, F_out, du,
                                      iters, dX_L, dX0, dW, dbias, dF, workspace, S(stream)));
}

int mhc_composite(int64_t T, int n, const float* H_res, float* P, float* gain_row,
                  float* gain_col, void* stream) {
    MHC_TRY(check_shape(T, n, 8));
    MHC_TRY(req({H_res, P}));
    MHC_TRY(opt({gain_row, gain_col}));
    (void)hipGetLastError();
    return finish(mhc::launch_composite(T, n, H_res, P, gain_row, gain_col, S(stream)));
}

}  // extern "C"
