// mhc_stack.hip -- layer-block recomputation over a stack of L mHC layers
// (staging.reportify.cn, "高效基础设施设计" notes [21], [22]: the mHC operators'
// intermediate activations are dropped after the forward and recomputed in the
// backward, in blocks whose size is chosen to minimise memory).
//
// The forward keeps, for every layer, its logits, rms and maps (K + 1 + 2n + n^2
// floats per token, under 1 % of the layer's n-stream buffer) in the workspace, and
// the n-stream buffer X itself only at block boundaries (every B layers, in caller
// buffers).  The backward walks the blocks top-down: it re-runs the post + residual
// pass of the block's layers from the boundary to get their X back (bitwise the
// forward's: the same kernels on the same inputs), then runs the block's layer
// backwards top-down.  B = 1 keeps every X (no recomputation).
#include "mhc_device.hpp"
#include "mhc_internal.hpp"
#include "../../include/mhc.h"

namespace mhc {

namespace {

struct Coef {
    float *z, *r, *hpre, *hpost, *hres;
};

size_t coef_bytes(int64_t T, int n)
{
    return align256(sizeof(float) * (size_t)T * K_of(n)) + align256(sizeof(float) * (size_t)T) +
           2 * align256(sizeof(float) * (size_t)T * n) + align256(sizeof(float) * (size_t)T * n * n);
}

Coef coef_at(void* ws, int l, int64_t T, int n)
{
    char* p = static_cast<char*>(ws) + (size_t)l * coef_bytes(T, n);
    Coef c;
    c.z = reinterpret_cast<float*>(p);     p += align256(sizeof(float) * (size_t)T * K_of(n));
    c.r = reinterpret_cast<float*>(p);     p += align256(sizeof(float) * (size_t)T);
    c.hpre = reinterpret_cast<float*>(p);  p += align256(sizeof(float) * (size_t)T * n);
    c.hpost = reinterpret_cast<float*>(p); p += align256(sizeof(float) * (size_t)T * n);
    c.hres = reinterpret_cast<float*>(p);
    return c;
}

size_t x_bytes(int64_t T, int n, int64_t C, int dtype)
{
    return (size_t)T * n * C * (dtype == MHC_BF16 ? 2 : 4);
}

// Scratch after the coefficient store: the forward's and the backward's regions
// overlap (the forward's are dead once it returns).  nws: the cross-layer pair's
// partials (bf16, n = 4, C % 64 == 0 only).
struct FwdScratch {
    void *xa, *xb, *u, *cws, *nws;
};
struct BwdScratch {
    void* slot0;              // B - 1 block buffers of X, x_bytes apart (aligned)
    void *g, *gb;             // dX_out of the next layer down in the storage dtype, alternating
    float *df, *dhres, *dhpost, *dhpre, *dz;
    void* bws;
};

size_t fwd_scratch_bytes(int64_t T, int n, int64_t C, int dtype)
{
    const size_t sx = align256(x_bytes(T, n, C, dtype));
    const size_t su = align256((size_t)T * C * (dtype == MHC_BF16 ? 2 : 4));
    const size_t sn = next_shape_ok(n, C, dtype) ? align256(next_workspace_bytes(T, C)) : 0;
    return 2 * sx + su + align256(fwd_pre_workspace_bytes(T, n, C, dtype)) + sn;
}

size_t bwd_scratch_bytes(int B, int64_t T, int n, int64_t C, int dtype)
{
    const size_t sx = align256(x_bytes(T, n, C, dtype));
    return (size_t)(B + 1) * sx + align256(sizeof(float) * (size_t)T * C) +
           align256(sizeof(float) * (size_t)T * n * n) + 2 * align256(sizeof(float) * (size_t)T * n) +
           align256(sizeof(float) * (size_t)T * K_of(n)) + align256(bwd_workspace_bytes(T, n, C, dtype));
}

FwdScratch fwd_carve(void* ws, int L, int64_t T, int n, int64_t C, int dtype)
{
    char* p = static_cast<char*>(ws) + (size_t)L * coef_bytes(T, n);
    const size_t sx = align256(x_bytes(T, n, C, dtype));
    FwdScratch f;
    f.xa = p;  p += sx;
    f.xb = p;  p += sx;
    f.u = p;   p += align256((size_t)T * C * (dtype == MHC_BF16 ? 2 : 4));
    f.cws = p; p += align256(fwd_pre_workspace_bytes(T, n, C, dtype));
    f.nws = next_shape_ok(n, C, dtype) ? p : nullptr;
    return f;
}

BwdScratch bwd_carve(void* ws, int L, int B, int64_t T, int n, int64_t C, int dtype)
{
    char* p = static_cast<char*>(ws) + (size_t)L * coef_bytes(T, n);
    const size_t sx = align256(x_bytes(T, n, C, dtype));
    BwdScratch b;
    b.slot0 = p;                               p += (size_t)(B - 1) * sx;
    b.g = p;                                   p += sx;
    b.gb = p;                                  p += sx;
    b.df = reinterpret_cast<float*>(p);        p += align256(sizeof(float) * (size_t)T * C);
    b.dhres = reinterpret_cast<float*>(p);     p += align256(sizeof(float) * (size_t)T * n * n);
    b.dhpost = reinterpret_cast<float*>(p);    p += align256(sizeof(float) * (size_t)T * n);
    b.dhpre = reinterpret_cast<float*>(p);     p += align256(sizeof(float) * (size_t)T * n);
    b.dz = reinterpret_cast<float*>(p);        p += align256(sizeof(float) * (size_t)T * K_of(n));
    b.bws = p;
    return b;
}

}  // namespace

int stack_block_size(int L)
{
    // buffers of X alive during the backward: ceil(L / B) boundaries + (B - 1) slots
    int best = 1;
    int64_t cost = L;
    for (int B = 2; B <= L; ++B) {
        const int64_t c = (L + B - 1) / B + (B - 1);
        if (c < cost) { cost = c; best = B; }
    }
    return best;
}

size_t stack_workspace_bytes(int L, int B, int64_t T, int n, int64_t C, int dtype)
{
    const size_t f = fwd_scratch_bytes(T, n, C, dtype), b = bwd_scratch_bytes(B, T, n, C, dtype);
    return (size_t)L * coef_bytes(T, n) + (f > b ? f : b);
}

hipError_t stack_forward(int L, int B, int64_t T, int n, int64_t C, int dtype, const void* X0,
                         const float* const* gamma, const float* const* W,
                         const float* const* bias, const float* alpha, const void* const* F,
                         void* const* u, float eps, int iters, void* const* Xsave, void* XL,
                         void* ws, hipStream_t s)
{
    const FwdScratch fs = fwd_carve(ws, L, T, n, C, dtype);
    if (Xsave[0] != X0) {
        const hipError_t e = hipMemcpyAsync(Xsave[0], X0, x_bytes(T, n, C, dtype),
                                            hipMemcpyDeviceToDevice, s);
        if (e != hipSuccess) return e;
    }
    // Where the read side runs in one pass (fwd_sr_available), layer l's post + residual
    // pass and layer l + 1's read side are one launch that reads X_l and F_l once and
    // projects X_{l+1} as it forms it.  Elsewhere, with the cross-layer pair (bf16,
    // n = 4, C % 64 == 0), each post + residual pass but the last also projects the next
    // layer's logits from the X' it writes, and that layer's read side reads X' once.
    // Every X' has the bits of the plain pass.
    const bool fused = fwd_sr_available(T, n, C, dtype);
    const bool next = !fused && fs.nws != nullptr;
    const void* x = X0;
    if (fused) {
        const Coef c = coef_at(ws, 0, T, n);
        const hipError_t e = launch_fwd_pre(T, n, C, dtype, x, gamma[0], eps, W[0], bias[0], alpha,
                                            c.z, c.r, c.hpre, c.hpost, iters, nullptr, c.hres,
                                            u ? u[0] : fs.u, nullptr, fs.cws, s);
        if (e != hipSuccess) return e;
    }
    for (int l = 0; l < L; ++l) {
        const Coef c = coef_at(ws, l, T, n);
        hipError_t e = hipSuccess;
        if (!fused) {
            void* ul = u ? u[l] : fs.u;
            e = (next && l > 0)
                ? launch_fwd_pre_from_next(T, C, eps, bias[l], alpha + 3 * l, c.z, c.r, c.hpre,
                                           c.hpost, iters, nullptr, c.hres, x, ul, nullptr, fs.nws, s)
                : launch_fwd_pre(T, n, C, dtype, x, gamma[l], eps, W[l], bias[l], alpha + 3 * l,
                                 c.z, c.r, c.hpre, c.hpost, iters, nullptr, c.hres, ul, nullptr,
                                 fs.cws, s);
            if (e != hipSuccess) return e;
        }
        void* out;
        if (l + 1 == L) out = XL;
        else if ((l + 1) % B == 0) out = Xsave[(l + 1) / B];
        else out = (x == fs.xa) ? fs.xb : fs.xa;
        if (fused && l + 1 < L) {
            const Coef cn = coef_at(ws, l + 1, T, n);
            e = launch_post_res_fwd_pre(T, n, C, dtype, x, F[l], c.hres, c.hpost, out, gamma[l + 1],
                                        eps, W[l + 1], bias[l + 1], alpha + 3 * (l + 1), cn.z, cn.r,
                                        cn.hpre, cn.hpost, iters, nullptr, cn.hres,
                                        u ? u[l + 1] : fs.u, nullptr, fs.cws, s);
        } else if (next && l + 1 < L) {
            e = launch_post_res_next(T, C, x, F[l], c.hres, c.hpost, out, gamma[l + 1], W[l + 1],
                                     fs.nws, s);
        } else {
            e = launch_post_res(T, n, C, dtype, x, F[l], c.hres, c.hpost, out, s);
        }
        if (e != hipSuccess) return e;
        x = out;
    }
    return hipSuccess;
}

hipError_t stack_backward(int L, int B, int64_t T, int n, int64_t C, int dtype,
                          const void* const* Xsave, const float* const* gamma,
                          const float* const* W, const float* const* bias, const float* alpha,
                          const void* const* F, const void* const* du, int iters, const void* GL,
                          float* dX0, float* const* dW, float* const* dbias, float* const* dF,
                          void* ws, hipStream_t s)
{
    const BwdScratch bs = bwd_carve(ws, L, B, T, n, C, dtype);
    const size_t sx = align256(x_bytes(T, n, C, dtype));
    const int K = K_of(n);
    const int nb = (L + B - 1) / B;
    const void* G = GL;
    bool flip = false;
    const void* xs[1024];     // X of the block's layers (B <= 1024 is checked by the caller)
    for (int kb = nb - 1; kb >= 0; --kb) {
        const int l0 = kb * B, l1 = (l0 + B) < L ? (l0 + B) : L;
        xs[0] = Xsave[kb];
        for (int l = l0; l + 1 < l1; ++l) {
            const Coef c = coef_at(ws, l, T, n);
            void* out = static_cast<char*>(bs.slot0) + (size_t)(l - l0) * sx;
            const hipError_t e = launch_post_res(T, n, C, dtype, xs[l - l0], F[l], c.hres, c.hpost,
                                                 out, s);
            if (e != hipSuccess) return e;
            xs[l - l0 + 1] = out;
        }
        for (int l = l1 - 1; l >= l0; --l) {
            const Coef c = coef_at(ws, l, T, n);
            const void* xl = xs[l - l0];
            // a layer's order: dF, dH_res and dH_post first (a sublayer forms du from dF),
            // then the read map's gradient dH_pre = <du, X_k> (at n = 4 with the Sinkhorn
            // backward in the same launch, into dz's res columns), then the coefficient
            // backward
            hipError_t e = launch_post_res_bwd(T, n, C, dtype, G, xl, F[l], c.hres, c.hpost,
                                               dF ? dF[l] : bs.df, bs.dhres, bs.dhpost, nullptr, s);
            if (e != hipSuccess) return e;
            const bool sk = n == 4;
            e = sk ? launch_pre_bwd_sk(T, C, dtype, du[l], xl, c.hpre, bs.dhpre, c.z + 2 * n, K,
                                       iters, bs.dhres, bs.dz + 2 * n, K, s)
                   : launch_pre_bwd(T, n, C, dtype, du[l], xl, c.hpre, bs.dhpre, nullptr, s);
            if (e != hipSuccess) return e;
            // above layer 0, dX goes straight to the next layer down as its dX_out, in the
            // storage dtype (bf16 rounded by the backward kernel itself); two buffers
            // alternate so that no layer reads the buffer it writes
            const bool pass_on = l > 0;
            float* dxo = pass_on ? static_cast<float*>(flip ? bs.gb : bs.g) : dX0;
            e = launch_coeffs_bwd(T, n, C, dtype, xl, gamma[l], W[l], alpha + 3 * l, c.z, bias[l],
                                  c.r, c.hpre, c.hpost, bs.dhpre, bs.dhpost, nullptr, c.z + 2 * n, K,
                                  bs.dhres, iters, G, du[l], c.hres, dxo, dW[l], dbias[l], nullptr,
                                  bs.dz, bs.bws, s, pass_on, sk);
            if (e != hipSuccess) return e;
            if (pass_on) {
                G = dxo;
                flip = !flip;
            }
        }
    }
    return hipGetLastError();
}

}  // namespace mhc
