/*
 * mhc.h -- C ABI of libmhc.so, the MI355X (gfx950) implementation of the per-layer
 * mHC (Manifold-Constrained Hyper-Connections) residual operator, forward and
 * backward.
 *
 * The operator (chatgpz.de, "Von Residualverbindungen zu Hyperverbindungen"): each
 * token keeps an n-stream residual buffer X in R^{n x C}; a layer reads
 * u = H_pre X, runs its sublayer F(u), and writes X' = H_res X + H_post^T F(u).
 * The maps are per-token: logits z come from RMSNorm(vec X) through one projection
 * (same page, "Systemarbeit und Schulungsaufwand": fused RMSNorm, projections and
 * gating); H_pre and H_post are sigmoid(z) (non-negative: "Vielfaeltig
 * eingeschraenkte Hyperverbindungen"; staging.reportify.cn "mHC方法原理" note
 * [12]); H_res is Sinkhorn-Knopp(exp z) with `iters` iterations of a row
 * normalisation followed by a column normalisation (same sections; note [16]:
 * t_max = 20).  F itself is the caller's: its output F_out (forward) and the
 * gradient of the loss w.r.t. u, du (backward), are passed in as tensors.
 *
 * Conventions for every call
 *   Pointers   Tensor pointers are DEVICE pointers owned by the caller.  The library
 *              keeps no state between calls and allocates no device memory: scratch
 *              comes from a caller-provided workspace of mhc_workspace_size() bytes.
 *              `alpha` is a HOST pointer to 3 floats (scales of the pre, post and
 *              res logit groups), read during the call.
 *   Stream     `stream` is a hipStream_t (NULL = the default stream).  Every call
 *              only enqueues work on it and returns; inputs must stay alive and
 *              outputs untouched until the stream reaches that point.  Concurrent
 *              calls that share a workspace race.
 *   Shapes     T >= 1 tokens, n in {1, 2, 4, 8} streams, C >= 8 channels with C % 8 == 0,
 *              K = n*n + 2n logits per token (24 at n = 4).
 *   Dtypes     `dtype` (MHC_F32 or MHC_BF16) is the storage type of X, F_out, u,
 *              X_out, dX_out and du.  Logits, maps, rms and every gradient are fp32.
 *              Arithmetic accumulates in fp32; bf16 outputs are rounded to nearest
 *              even once.
 *   Layouts    Row-major and contiguous.  X, X_out, dX_out, dX: [T][n][C].
 *              u, F_out, du, dF: [T][C].  z, dz: [T][K], columns pre 0..n-1,
 *              post n..2n-1, res 2n + i*n + j.  H_pre, H_post, dH_pre, dH_post:
 *              [T][n].  H_res, dH_res: [T][n][n]; H_res[i][j] feeds stream j into
 *              output stream i.  gamma: [n*C].  W, dW: [n*C][K], row index
 *              k*C + c for stream k, channel c.  bias: [K].  rms: [T].
 *   Alignment  Every tensor pointer must be 16-byte aligned.
 *   Outputs    "write" outputs are overwritten; "+=" outputs are accumulated into
 *              (the caller zeroes them or passes an earlier result).  A NULL
 *              optional output skips its work.
 *   Errors     All arguments are validated on the host before anything is
 *              enqueued; a call that returns an error enqueued nothing and wrote
 *              nothing.  MHC_ERR_HIP reports a failed launch (the stream state is
 *              then the caller's to inspect).  Nothing throws or aborts across the
 *              ABI.  mhc_status_str() names a status.
 *   Determinism  Reductions over tokens (dW, dbias, dgamma) use a fixed order:
 *              identical inputs give bitwise identical outputs.
 */
#ifndef MHC_H
#define MHC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define MHC_OK             0
#define MHC_ERR_NULL      -1   /* a required pointer is NULL */
#define MHC_ERR_SHAPE     -2   /* T < 1, n not in {1,2,4,8}, C < 8 or C % 8 != 0, bad ld */
#define MHC_ERR_ALIGN     -3   /* a tensor pointer is not 16-byte aligned */
#define MHC_ERR_DTYPE     -4   /* dtype not MHC_F32 / MHC_BF16 */
#define MHC_ERR_ITERS     -5   /* iters < 1 or iters > 10000 */
#define MHC_ERR_WORKSPACE -6   /* workspace NULL or smaller than mhc_workspace_size() */
#define MHC_ERR_HIP       -7   /* a kernel launch failed */
#define MHC_ERR_VALUE     -8   /* alpha has a non-finite entry */
#define MHC_ERR_SCRATCH   -9   /* mhc_fwd_pre_noalloc: more scratch than MHC_NOALLOC_SCRATCH_BYTES */
#define MHC_ERR_NONFINITE -10  /* MHC_CHECK_FINITE: a NaN or Inf in an input or an output */

/* Environment switches (read on every call):
 *   MHC_CHECK_FINITE  set to anything but "" or "0": every call that takes floating-point
 *                     tensors (all but the stack calls) scans its inputs before it
 *                     enqueues anything -- a NaN or Inf returns MHC_ERR_NONFINITE and
 *                     nothing is computed -- and its outputs after its kernels -- a NaN
 *                     or Inf there returns MHC_ERR_NONFINITE with the outputs written.
 *                     Each scan synchronises the stream: a debugging aid, not for code
 *                     under graph capture.  Off, the calls never look at values (NaN and
 *                     Inf propagate through the arithmetic as usual).
 *   MHC_FORCE_PATH    "vector": the plain vector kernels of the projections (forward
 *                     and backward) instead of the MFMA ones; "twopass": the forward read
 *                     side reads X twice (projection pass, then the finishing pass with
 *                     u) instead of once.  For measurement and cross-checks; every path
 *                     meets the same tolerances. */

/* storage dtypes */
#define MHC_F32  0
#define MHC_BF16 1

/* workspace queries */
#define MHC_OP_COEFFS     0
#define MHC_OP_COEFFS_BWD 1
#define MHC_OP_FWD_PRE    2
#define MHC_OP_BWD_PRE    3
#define MHC_OP_NEXT       4   /* shared by mhc_post_res_next and mhc_fwd_pre_next */
#define MHC_OP_ALPHA_BWD  5   /* mhc_alpha_bwd (size independent of T, n, C, dtype) */

/* Human-readable name of a status code (static string, never NULL). */
const char* mhc_status_str(int status);

/* ABI revision of this header; bumped on any incompatible change. */
int mhc_abi_version(void);

/* Bytes of device workspace the call `op` needs for these sizes (0 = none; the
 * workspace pointer may then be NULL).  Returns 0 for invalid arguments too. */
size_t mhc_workspace_size(int op, int64_t T, int n, int64_t C, int dtype);

/* Coefficients and gating (steps 1-2 of the layer), per token t:
 *   v = vec(X_t) (stream-major), r = sqrt(mean(v^2) + eps),
 *   proj_k = ((v .* gamma) . W[:,k]) / r,   z_k = alpha_g(k) * proj_k + bias_k,
 *   H_pre = sigmoid(z[0:n]), H_post = sigmoid(z[n:2n]).
 * chatgpz.de "Systemarbeit und Schulungsaufwand" (fused RMSNorm, projection,
 * gating); staging.reportify.cn "高效基础设施设计" note [17] (RMSNorm reordered:
 * the kernel divides the projection by r after the dot products, an exact
 * identity).  Writes z [T][K], rms [T], H_pre, H_post [T][n] and proj [T][K] (the
 * unscaled normalised projection, which mhc_alpha_bwd takes); rms, H_pre, H_post
 * and proj may be NULL.  alpha: three finite floats (else MHC_ERR_VALUE). */
int mhc_coeffs(int64_t T, int n, int64_t C, int dtype,
               const void* X, const float* gamma, float eps, const float* W,
               const float* bias, const float* alpha,
               float* z, float* rms, float* H_pre, float* H_post, float* proj,
               void* workspace, size_t workspace_bytes, void* stream);

/* Sinkhorn-Knopp projection of H_res (step 3): M = exp(Z) with
 * Z[i][j] = z_res[t*ld_z + i*n + j]; `iters` times divide each row by its sum,
 * then each column by its sum; H_res = M.  chatgpz.de "Vielfaeltig
 * eingeschraenkte Hyperverbindungen"; staging.reportify.cn "mHC方法原理" notes
 * [10], [16].  The kernel subtracts each row's maximum before exp (every iteration
 * starts with a row normalisation, so the shift cancels).  ld_z >= n*n.
 * Writes H_res [T][n][n]. */
int mhc_sinkhorn(int64_t T, int n, const float* z_res, int64_t ld_z, int iters,
                 float* H_res, void* stream);

/* Read map (step 4): u[t][c] = sum_k H_pre[t][k] X[t][k][c]
 * (chatgpz.de "Von Residualverbindungen zu Hyperverbindungen").  Writes u. */
int mhc_pre(int64_t T, int n, int64_t C, int dtype, const void* X, const float* H_pre,
            void* u, void* stream);

/* Write map and residual merge (step 5):
 *   X_out[t][i][c] = sum_j H_res[t][i][j] X[t][j][c] + H_post[t][i] F_out[t][c]
 * (chatgpz.de update rule; staging.reportify.cn "高效基础设施设计" note [20]:
 * maps applied together with the residual merge).  X_out must not alias X. */
int mhc_post_res(int64_t T, int n, int64_t C, int dtype, const void* X, const void* F_out,
                 const float* H_res, const float* H_post, void* X_out, void* stream);

/* Backward of step 5 with F_out held as an input, G = dX_out:
 *   dF[t][c] = sum_i H_post[t][i] G[t][i][c]            (write)
 *   dH_post[t][i] = <G[t][i], F_out[t]>                  (write)
 *   dH_res[t][i][j] = <G[t][i], X[t][j]>                 (write)
 *   dX[t][j][c] = sum_i H_res[t][i][j] G[t][i][c]        (write; may be NULL) */
int mhc_post_res_bwd(int64_t T, int n, int64_t C, int dtype, const void* dX_out,
                     const void* X, const void* F_out, const float* H_res,
                     const float* H_post, float* dF, float* dH_res, float* dH_post,
                     float* dX, void* stream);

/* Backward of step 4, with du the gradient w.r.t. u:
 *   dH_pre[t][k] = <du[t], X[t][k]>                      (write)
 *   dX[t][k][c] += H_pre[t][k] du[t][c]                  (+=; may be NULL) */
int mhc_pre_bwd(int64_t T, int n, int64_t C, int dtype, const void* du, const void* X,
                const float* H_pre, float* dH_pre, float* dX, void* stream);

/* Backward of step 3 (staging.reportify.cn "高效基础设施设计" note [19]: the
 * iterations get their own backward; note [21]: recomputed, not stored).  Re-runs
 * the `iters` iterations from the logits, then differentiates the 2*iters
 * normalisations in reverse: for Y = M/colsum, dM_ij = (dY_ij - sum_m dY_mj Y_mj)
 * / colsum_j; for Y = M/rowsum likewise by rows; dz = dM .* exp(Z).
 * Writes dz_res[t*ld_dz + i*n + j]; ld_z, ld_dz >= n*n. */
int mhc_sinkhorn_bwd(int64_t T, int n, const float* z_res, int64_t ld_z, int iters,
                     const float* dH_res, float* dz_res, int64_t ld_dz, void* stream);

/* Backward of steps 1-2.  dz_pre = dH_pre H_pre (1 - H_pre), dz_post likewise,
 * dz_res given ([T][n*n]); with q_k = alpha_g(k) dz_k, dy = W q (per token),
 * y = gamma .* v / r:
 *   dX[t] += gamma .* dy / r - v * (sum_k dz_k (z_k - bias_k)) / (N r^2)   (+=)
 *   dW = sum_t y_t q_t^T, dbias = sum_t dz_t, dgamma = sum_t v .* dy / r (write)
 * (the middle term uses sum_m gamma_m v_m dy_m = r sum_k dz_k (z_k - b_k), exact for
 * the projection's z).  dX, dgamma and dz (the assembled [T][K] logit gradient,
 * write) may be NULL. */
int mhc_coeffs_bwd(int64_t T, int n, int64_t C, int dtype,
                   const void* X, const float* gamma, const float* W, const float* alpha,
                   const float* z, const float* bias, const float* rms,
                   const float* H_pre, const float* H_post,
                   const float* dH_pre, const float* dH_post, const float* dz_res,
                   float* dX, float* dW, float* dbias, float* dgamma, float* dz,
                   void* workspace, size_t workspace_bytes, void* stream);

/* Fused forward read side: steps 1-4 in one call (staging.reportify.cn
 * "高效基础设施设计" note [18]: one operator for the scans and matmuls).  Equal to
 * mhc_coeffs -> mhc_sinkhorn -> mhc_pre.  z_res_in (nullable, [T][n*n]) replaces
 * the projected res logits at the Sinkhorn input; z still returns the
 * projection's logits.  Writes z, rms, H_pre, H_post, H_res, u, and proj when it
 * is not NULL (as mhc_coeffs).
 * At bf16, n = 4 and C = 1024 k (k = 1..8), on a device with 256 CUs, it reads X once:
 * one block per CU, and the CUs of each XCD exchange per-token partial sums, so the
 * call needs its blocks resident together (work running beside it on other streams can
 * delay that).  A block that waits more than 0.5 s for another's sums gives up: the u
 * of the tokens concerned is NaN (z, rms, H and proj stay exact) -- wrong values do
 * not pass silently.  MHC_FORCE_PATH=twopass takes the two-pass path instead. */
int mhc_fwd_pre(int64_t T, int n, int64_t C, int dtype,
                const void* X, const float* gamma, float eps, const float* W,
                const float* bias, const float* alpha, int iters, const float* z_res_in,
                float* z, float* rms, float* H_pre, float* H_post, float* H_res, void* u,
                float* proj, void* workspace, size_t workspace_bytes, void* stream);

/* mhc_fwd_pre for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same arguments,
 * kernels and results (bitwise) as mhc_fwd_pre, without the workspace.  Its scratch
 * (the split projection, the partial logits, the exchange ring of the single-read pass:
 * mhc_workspace_size(MHC_OP_FWD_PRE, ...) bytes) lives in a device array of
 * MHC_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on until the
 * process ends; the call allocates nothing (no hipMalloc, no allocating library
 * routine).  Sizes whose scratch exceeds that array return MHC_ERR_SCRATCH before
 * anything is enqueued: n = 4 bf16 fits every T up to 149744 at C = 1024, 74048 at
 * C = 2048, 36208 at C = 4096 and 20032 at C = 7168; the fp32 and n != 4 paths need no
 * scratch and take any size.  The parts of the scratch that must start cleared (the
 * exchange ring's tags) are cleared by a fill kernel at the start of every call.  Every
 * call on one GPU uses that GPU's one array: calls that overlap on a GPU (different
 * streams or host threads without ordering between them) race.  MHC_ERR_HIP also
 * reports a failure to look up the array's device address. */
#define MHC_NOALLOC_SCRATCH_BYTES (64u << 20)
int mhc_fwd_pre_noalloc(int64_t T, int n, int64_t C, int dtype,
                        const void* X, const float* gamma, float eps, const float* W,
                        const float* bias, const float* alpha, int iters, const float* z_res_in,
                        float* z, float* rms, float* H_pre, float* H_post, float* H_res, void* u,
                        float* proj, void* stream);

/* Fused backward read side: mhc_pre_bwd + mhc_sinkhorn_bwd + mhc_coeffs_bwd plus
 * the direct term H_res^T dX_out, in one call; pairs with an mhc_post_res_bwd that
 * passed dX = NULL.  The Sinkhorn is recomputed from z_res_in when given (the
 * injected logits are read as the projected ones plus a constant offset, so the
 * gradient still flows through the projection), else from z[:, 2n:].
 *   dX = H_res^T dX_out + H_pre^T du + (coefficient path)   (write)
 *   dW, dbias (write), dH_pre (write), dz [T][K] (write), dgamma (write, nullable) */
int mhc_bwd_pre(int64_t T, int n, int64_t C, int dtype,
                const void* dX_out, const void* du, const void* X,
                const float* gamma, const float* W, const float* alpha,
                const float* z, const float* bias, const float* rms,
                const float* H_pre, const float* H_post, const float* H_res,
                const float* dH_res, const float* dH_post, int iters,
                const float* z_res_in,
                float* dX, float* dW, float* dbias, float* dH_pre, float* dz,
                float* dgamma, void* workspace, size_t workspace_bytes, void* stream);

/* Backward read side in two calls, with X streamed once for both reductions of a
 * token over the channels (chatgpz.de update rule: dH_res, dH_post and dH_pre all
 * contract X or X-shaped rows over c):
 *
 * mhc_post_res_bwd_pre: mhc_post_res_bwd with dX = NULL, plus the read map's
 *   dH_pre[t][k] = <du[t], X[t][k]>                      (write; bitwise the value
 *   mhc_pre_bwd and mhc_bwd_pre form)
 *
 * The pair needs du when dF is formed.  Inside one layer a sublayer forms du from dF,
 * so there the pair only serves callers that know du in advance; the order a layer
 * runs is mhc_post_res_bwd, the sublayer's backward, then mhc_bwd_pre (which reads X
 * once more than this pair).
 *
 * mhc_bwd_pre_from_dh: mhc_bwd_pre with dH_pre an input instead of an output
 *   (mhc_sinkhorn_bwd + mhc_coeffs_bwd + the direct terms H_res^T dX_out and
 *   H_pre^T du); the same workspace (MHC_OP_BWD_PRE).  Its outputs are bitwise those
 *   of mhc_bwd_pre on the same inputs. */
int mhc_post_res_bwd_pre(int64_t T, int n, int64_t C, int dtype, const void* dX_out,
                         const void* du, const void* X, const void* F_out,
                         const float* H_res, const float* H_post, float* dF,
                         float* dH_res, float* dH_post, float* dH_pre, void* stream);
int mhc_bwd_pre_from_dh(int64_t T, int n, int64_t C, int dtype,
                        const void* dX_out, const void* du, const void* X,
                        const float* gamma, const float* W, const float* alpha,
                        const float* z, const float* bias, const float* rms,
                        const float* H_pre, const float* H_post, const float* H_res,
                        const float* dH_pre, const float* dH_res, const float* dH_post,
                        int iters, const float* z_res_in,
                        float* dX, float* dW, float* dbias, float* dz, float* dgamma,
                        void* workspace, size_t workspace_bytes, void* stream);

/* Cross-layer fusion (bf16 storage, n = 4, C % 64 == 0; otherwise MHC_ERR_DTYPE or
 * MHC_ERR_SHAPE).  In a stack, layer l's write map and layer l+1's coefficient
 * projection both stream X' = X_{l+1}; this pair of calls does the projection while
 * X' is being written (staging.reportify.cn "高效基础设施设计" notes [18], [20]:
 * fused scans/matmuls, maps applied with the residual merge), so the next layer's
 * read side reads X' once.
 *
 * mhc_post_res_next: X_out exactly as mhc_post_res, plus the partial projection of
 * the bf16 X_out with the NEXT layer's gamma_next and W_next (sums of
 * (x .* gamma_next) . W_next[:,k] and of x^2 over channel ranges), left in
 * `workspace` (mhc_workspace_size(MHC_OP_NEXT, ...) bytes).
 *
 * mhc_fwd_pre_next: the next layer's read side from those partials: the same
 * outputs as mhc_fwd_pre on X = that X_out (z, rms, H_pre, H_post, H_res from the
 * logits or z_res_in, u), given the same workspace, untouched in between.  eps,
 * bias and alpha are the next layer's.  The two calls must see the same T and C. */
int mhc_post_res_next(int64_t T, int n, int64_t C, int dtype, const void* X,
                      const void* F_out, const float* H_res, const float* H_post,
                      void* X_out, const float* gamma_next, const float* W_next,
                      void* workspace, size_t workspace_bytes, void* stream);

int mhc_fwd_pre_next(int64_t T, int n, int64_t C, int dtype, const void* X, float eps,
                     const float* bias, const float* alpha, int iters,
                     const float* z_res_in, float* z, float* rms, float* H_pre,
                     float* H_post, float* H_res, void* u, float* proj, void* workspace,
                     size_t workspace_bytes, void* stream);

/* Cross-layer fusion in one call: layer l's write map and residual merge and layer l+1's
 * read side (the same notes: maps applied with the residual merge, fused scans).
 *   X_out = H_res X + H_post^T F_out            exactly as mhc_post_res (write)
 * then, on X_out, everything mhc_fwd_pre writes with the next layer's parameters
 * (gamma, eps, W, bias, alpha, iters, z_res_in): z, rms, H_pre_next, H_post_next,
 * H_res_next, u and proj (nullable), bitwise the values of mhc_post_res followed by
 * mhc_fwd_pre.  H_res / H_post are layer l's maps (inputs), *_next layer l+1's
 * (outputs).  No output (X_out, u, H_res_next, H_post_next) may overlap an input (X,
 * F_out, H_res, H_post): MHC_ERR_SHAPE.  The workspace is
 * mhc_workspace_size(MHC_OP_FWD_PRE, ...) bytes.
 * Where mhc_fwd_pre reads X once (bf16, n = 4, C = 1024 k, a 256-CU device), this call
 * reads X and F_out once and forms X_out tile by tile in the same pass, projecting the
 * tile it formed: 20 C bytes of HBM traffic per token (X, F_out in; X_out, u out) instead
 * of 28 C for the two calls, with the single-read pass's co-residency and timeout
 * behaviour (a timeout poisons u only; X_out is always written).  Elsewhere it runs the
 * two calls in turn. */
int mhc_post_res_fwd_pre(int64_t T, int n, int64_t C, int dtype, const void* X,
                         const void* F_out, const float* H_res, const float* H_post, void* X_out,
                         const float* gamma, float eps, const float* W, const float* bias,
                         const float* alpha, int iters, const float* z_res_in, float* z,
                         float* rms, float* H_pre_next, float* H_post_next, float* H_res_next,
                         void* u, float* proj, void* workspace, size_t workspace_bytes,
                         void* stream);

/* Gradient of the three logit scales, for callers that train alpha (the maps' gating
 * scales; the definition of z above).  z_k = alpha_g(k) proj_k + bias_k, so
 *   dalpha[g] = sum_t sum_{k in group g} dz[t][k] proj[t][k]
 * (write, fp32 [3], device pointer).  proj: the unscaled normalised projection [T][K]
 * that mhc_coeffs / mhc_fwd_pre / mhc_fwd_pre_next wrote (also when z_res_in was
 * injected); dz: the logit gradient [T][K] of mhc_bwd_pre, mhc_bwd_pre_from_dh or
 * mhc_coeffs_bwd.  Products and sums run in fp64 in a fixed order; the result is
 * rounded to fp32 once.  alpha itself is not needed (zero is a valid scale).
 * `workspace` is mhc_workspace_size(MHC_OP_ALPHA_BWD, ...) bytes (any valid T, n, C,
 * dtype). */
int mhc_alpha_bwd(int64_t T, int n, const float* proj, const float* dz, float* dalpha,
                  void* workspace, size_t workspace_bytes, void* stream);

/* Layer-block recomputation over a stack of L layers (staging.reportify.cn
 * "高效基础设施设计" notes [21], [22]: the mHC operators' intermediate activations
 * are dropped after the forward and recomputed in the backward, in blocks sized to
 * minimise memory).  Layer l (0-based) maps X_l to X_{l+1} as mhc_fwd_pre +
 * mhc_post_res do, with its own gamma[l], W[l], bias[l] (device pointers in host
 * arrays of L entries), alpha[3 l .. 3 l + 2] (one HOST array of 3 L floats, finite)
 * and sublayer output F_out[l].  The sublayer is the caller's: F_out[l] and, in the
 * backward, du[l] (the gradient its backward returns) are given per layer.
 *
 * Blocks of B layers (1 <= B <= min(L, 1024)): the forward keeps X_l only for
 * l = 0, B, 2B, ... in X_save[l / B] (ceil(L / B) caller buffers [T][n][C]; X_save[0]
 * may be X0 itself, else X0 is copied there) and every layer's logits, rms and
 * maps (K + 1 + 2n + n^2 floats per token) in `workspace`.  The backward, given the
 * same X_save and the workspace untouched since the forward, walks the blocks from
 * the top: it re-runs the post + residual pass of the block's layers from X_save to
 * get their X back (bitwise the forward's), then runs each layer's backward
 * (mhc_post_res_bwd, then mhc_bwd_pre with du[l]) top-down.  Since du[l] is taken up
 * front, the runner serves stacks whose sublayer gradients are known before the
 * backward starts (synthetic or precomputed ones); a network whose sublayer forms du
 * from dF runs the per-layer calls itself, with its sublayer backward between them.  B = 1 keeps every X (no
 * recomputation); X buffers alive during the backward: ceil(L / B) + B - 1.  Where
 * the cross-layer pair applies (bf16, n = 4, C % 64 == 0) the forward runs layer l's
 * post + residual pass as mhc_post_res_next with layer l + 1's gamma and W, and layer
 * l + 1's read side as mhc_fwd_pre_next (layer 0: mhc_fwd_pre; the last layer:
 * mhc_post_res).
 *
 * mhc_stack_block_size(L): the B that minimises ceil(L / B) + B - 1 (the smallest such
 * B), about sqrt(L); 0 for L < 1.
 * mhc_stack_workspace_size: bytes of the workspace shared by the two calls (0 for
 * invalid arguments).
 * mhc_stack_forward: writes X_save (entries 1 ..), X_L = X_{L} and, when `u` is not
 * NULL, u[l] = H_pre,l X_l.  X_L must not be one of X_save.
 * mhc_stack_backward: dX_L (storage dtype) is the loss gradient w.r.t. X_L.  Writes
 * dX0 (fp32 [T][n][C]), dW[l], dbias[l] (write), and dF[l] when dF is not NULL.
 * Between layers, layer l's dX goes to layer l-1 as its dX_out in the storage dtype
 * (bf16: rounded to nearest even once, by the backward kernel that forms it). */
int mhc_stack_block_size(int L);
size_t mhc_stack_workspace_size(int L, int B, int64_t T, int n, int64_t C, int dtype);
int mhc_stack_forward(int L, int B, int64_t T, int n, int64_t C, int dtype, const void* X0,
                      const float* const* gamma, const float* const* W, const float* const* bias,
                      const float* alpha, const void* const* F_out, void* const* u, float eps,
                      int iters, void* const* X_save, void* X_L, void* workspace,
                      size_t workspace_bytes, void* stream);
int mhc_stack_backward(int L, int B, int64_t T, int n, int64_t C, int dtype,
                       const void* const* X_save, const float* const* gamma, const float* const* W,
                       const float* const* bias, const float* alpha, const void* const* F_out,
                       const void* const* du, int iters, const void* dX_L, float* dX0,
                       float* const* dW, float* const* dbias, float* const* dF,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Composite residual mapping over depth (chatgpz.de "Warum Hyperverbindungen
 * instabil werden"): P[t] <- H_res[t] P[t] (later layers on the left), then
 * gain_row[t] = max_i sum_j |P_ij|, gain_col[t] = max_j sum_i |P_ij| (write;
 * either may be NULL).  P is [T][n][n], updated in place. */
int mhc_composite(int64_t T, int n, const float* H_res, float* P, float* gain_row,
                  float* gain_col, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MHC_H */
