"""ctypes binding of libmhc.so (C ABI in include/mhc.h).

Argument marshalling only: every step of the operator runs in the HIP kernels of
libmhc.so.  Functions carry the C names; they take torch tensors on the GPU,
derive T, n, C and the storage dtype from their shapes, allocate outputs and
workspaces with torch when the caller passes none, and enqueue on torch's current
stream.  A non-zero status raises MhcError.  Importing this module fails loudly
when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmhc.so")

MHC_F32, MHC_BF16 = 0, 1
MHC_OP_COEFFS, MHC_OP_COEFFS_BWD, MHC_OP_FWD_PRE, MHC_OP_BWD_PRE, MHC_OP_NEXT = 0, 1, 2, 3, 4
MHC_OP_ALPHA_BWD = 5


class MhcError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is not built; run `python -m "
                          "manifold_constrained_residuals_amd.build` (hipcc, gfx950)")
    L = ctypes.CDLL(_LIB_PATH)
    vp, fp, i64, i32, f32, sz = (ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                 ctypes.c_float, ctypes.c_size_t)
    L.mhc_status_str.argtypes = [i32]; L.mhc_status_str.restype = ctypes.c_char_p
    L.mhc_abi_version.argtypes = []; L.mhc_abi_version.restype = i32
    L.mhc_workspace_size.argtypes = [i32, i64, i32, i64, i32]; L.mhc_workspace_size.restype = sz
    sigs = {
        "mhc_coeffs": [i64, i32, i64, i32, vp, fp, f32, fp, fp, fp, fp, fp, fp, fp, fp, vp, sz, vp],
        "mhc_sinkhorn": [i64, i32, fp, i64, i32, fp, vp],
        "mhc_pre": [i64, i32, i64, i32, vp, fp, vp, vp],
        "mhc_post_res": [i64, i32, i64, i32, vp, vp, fp, fp, vp, vp],
        "mhc_post_res_bwd": [i64, i32, i64, i32, vp, vp, vp, fp, fp, fp, fp, fp, fp, vp],
        "mhc_pre_bwd": [i64, i32, i64, i32, vp, vp, fp, fp, fp, vp],
        "mhc_sinkhorn_bwd": [i64, i32, fp, i64, i32, fp, fp, i64, vp],
        "mhc_coeffs_bwd": [i64, i32, i64, i32, vp, fp, fp, fp, fp, fp, fp, fp, fp, fp, fp, fp,
                           fp, fp, fp, fp, fp, vp, sz, vp],
        "mhc_fwd_pre": [i64, i32, i64, i32, vp, fp, f32, fp, fp, fp, i32, fp, fp, fp, fp, fp, fp,
                        vp, fp, vp, sz, vp],
        "mhc_post_res_fwd_pre": [i64, i32, i64, i32, vp, vp, fp, fp, vp, fp, f32, fp, fp, fp, i32,
                                 fp, fp, fp, fp, fp, fp, vp, fp, vp, sz, vp],
        "mhc_fwd_pre_noalloc": [i64, i32, i64, i32, vp, fp, f32, fp, fp, fp, i32, fp, fp, fp, fp,
                                fp, fp, vp, fp, vp],
        "mhc_bwd_pre": [i64, i32, i64, i32, vp, vp, vp, fp, fp, fp, fp, fp, fp, fp, fp, fp, fp, fp,
                        i32, fp, fp, fp, fp, fp, fp, fp, vp, sz, vp],
        "mhc_post_res_bwd_pre": [i64, i32, i64, i32, vp, vp, vp, vp, fp, fp, fp, fp, fp, fp, vp],
        "mhc_bwd_pre_from_dh": [i64, i32, i64, i32, vp, vp, vp, fp, fp, fp, fp, fp, fp, fp, fp, fp,
                                fp, fp, fp, i32, fp, fp, fp, fp, fp, fp, vp, sz, vp],
        "mhc_composite": [i64, i32, fp, fp, fp, fp, vp],
        "mhc_alpha_bwd": [i64, i32, fp, fp, fp, vp, sz, vp],
        "mhc_stack_forward": [i32, i32, i64, i32, i64, i32, vp, vp, vp, vp, fp, vp, vp, f32, i32,
                              vp, vp, vp, sz, vp],
        "mhc_stack_backward": [i32, i32, i64, i32, i64, i32, vp, vp, vp, vp, fp, vp, vp, i32, vp,
                               vp, vp, vp, vp, vp, sz, vp],
        "mhc_post_res_next": [i64, i32, i64, i32, vp, vp, fp, fp, vp, fp, fp, vp, sz, vp],
        "mhc_fwd_pre_next": [i64, i32, i64, i32, vp, f32, fp, fp, i32, fp, fp, fp, fp, fp, fp,
                             vp, fp, vp, sz, vp],
    }
    L.mhc_stack_block_size.argtypes = [i32]; L.mhc_stack_block_size.restype = i32
    L.mhc_stack_workspace_size.argtypes = [i32, i32, i64, i32, i64, i32]
    L.mhc_stack_workspace_size.restype = sz
    for name, args in sigs.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = i32
    return L


lib = _load()
LIB_PATH = _LIB_PATH


# ------------------------------------------------------------------ marshalling
def _p(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libmhc must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MHC_BF16
    if t.dtype == torch.float32:
        return MHC_F32
    raise ValueError(f"unsupported storage dtype {t.dtype}")


def _alpha(alpha) -> ctypes.Array:
    vals = [float(a) for a in (alpha.tolist() if hasattr(alpha, "tolist") else alpha)]
    if len(vals) != 3:
        raise ValueError("alpha needs 3 values (pre, post, res)")
    return (ctypes.c_float * 3)(*vals)


def _check(st: int):
    if st != 0:
        raise MhcError(st, lib.mhc_status_str(st).decode())


def _f32(shape, like: torch.Tensor):
    return torch.empty(shape, dtype=torch.float32, device=like.device)


def _shape3(X: torch.Tensor):
    if X.dim() != 3:
        raise ValueError("X must be [T, n, C]")
    return X.shape[0], X.shape[1], X.shape[2]


def K_of(n: int) -> int:
    return n * n + 2 * n


def mhc_workspace_size(op: int, T: int, n: int, C: int, dtype: int) -> int:
    return int(lib.mhc_workspace_size(op, T, n, C, dtype))


def workspace(op: int, T: int, n: int, C: int, dtype: int, device) -> Optional[torch.Tensor]:
    b = mhc_workspace_size(op, T, n, C, dtype)
    return torch.empty(b, dtype=torch.uint8, device=device) if b else None


def _ws(ws, op, T, n, C, dt, dev):
    if ws is None:
        ws = workspace(op, T, n, C, dt, dev)
    return ws, (_p(ws), ws.numel() if ws is not None else 0)


# ------------------------------------------------------------------ calls
def mhc_coeffs(X, gamma, eps, W, bias, alpha, z=None, rms=None, H_pre=None, H_post=None,
               proj=None, want_proj=False, workspace=None):
    T, n, C = _shape3(X); dt = _dt(X)
    z = _f32((T, K_of(n)), X) if z is None else z
    rms = _f32((T,), X) if rms is None else rms
    H_pre = _f32((T, n), X) if H_pre is None else H_pre
    H_post = _f32((T, n), X) if H_post is None else H_post
    if want_proj and proj is None:
        proj = _f32((T, K_of(n)), X)
    workspace, (wp, wb) = _ws(workspace, MHC_OP_COEFFS, T, n, C, dt, X.device)
    _check(lib.mhc_coeffs(T, n, C, dt, _p(X), _p(gamma), float(eps), _p(W), _p(bias),
                          _alpha(alpha), _p(z), _p(rms), _p(H_pre), _p(H_post), _p(proj), wp, wb,
                          _stream()))
    return dict(z=z, rms=rms, H_pre=H_pre, H_post=H_post, proj=proj)


def mhc_sinkhorn(z_res, n, iters=20, H_res=None):
    """z_res: [T, ld] fp32 with unit column stride (a column slice of z works)."""
    if z_res.dim() != 2 or z_res.stride(1) != 1:
        raise ValueError("z_res must be 2-D with unit column stride")
    T, ld = z_res.shape[0], z_res.stride(0)
    H_res = _f32((T, n, n), z_res) if H_res is None else H_res
    _check(lib.mhc_sinkhorn(T, n, ctypes.c_void_p(z_res.data_ptr()), ld, int(iters), _p(H_res),
                            _stream()))
    return H_res


def mhc_pre(X, H_pre, u=None):
    T, n, C = _shape3(X)
    u = torch.empty((T, C), dtype=X.dtype, device=X.device) if u is None else u
    _check(lib.mhc_pre(T, n, C, _dt(X), _p(X), _p(H_pre), _p(u), _stream()))
    return u


def mhc_post_res(X, F_out, H_res, H_post, X_out=None):
    T, n, C = _shape3(X)
    X_out = torch.empty_like(X) if X_out is None else X_out
    _check(lib.mhc_post_res(T, n, C, _dt(X), _p(X), _p(F_out), _p(H_res), _p(H_post), _p(X_out),
                            _stream()))
    return X_out


def mhc_post_res_bwd(dX_out, X, F_out, H_res, H_post, want_dx=False, dF=None, dH_res=None,
                     dH_post=None, dX=None):
    T, n, C = _shape3(X)
    dF = _f32((T, C), X) if dF is None else dF
    dH_res = _f32((T, n, n), X) if dH_res is None else dH_res
    dH_post = _f32((T, n), X) if dH_post is None else dH_post
    if want_dx and dX is None:
        dX = _f32((T, n, C), X)
    _check(lib.mhc_post_res_bwd(T, n, C, _dt(X), _p(dX_out), _p(X), _p(F_out), _p(H_res),
                                _p(H_post), _p(dF), _p(dH_res), _p(dH_post), _p(dX), _stream()))
    return dict(dF=dF, dH_res=dH_res, dH_post=dH_post, dX=dX)


def mhc_pre_bwd(du, X, H_pre, dH_pre=None, dX=None):
    """dX (fp32 [T,n,C]) is accumulated into when given."""
    T, n, C = _shape3(X)
    dH_pre = _f32((T, n), X) if dH_pre is None else dH_pre
    _check(lib.mhc_pre_bwd(T, n, C, _dt(X), _p(du), _p(X), _p(H_pre), _p(dH_pre), _p(dX),
                           _stream()))
    return dict(dH_pre=dH_pre, dX=dX)


def mhc_sinkhorn_bwd(z_res, dH_res, n, iters=20, dz_res=None):
    if z_res.dim() != 2 or z_res.stride(1) != 1:
        raise ValueError("z_res must be 2-D with unit column stride")
    T, ld = z_res.shape[0], z_res.stride(0)
    dz_res = _f32((T, n * n), z_res) if dz_res is None else dz_res
    if dz_res.dim() != 2 or dz_res.stride(1) != 1:
        raise ValueError("dz_res must be 2-D with unit column stride")
    _check(lib.mhc_sinkhorn_bwd(T, n, ctypes.c_void_p(z_res.data_ptr()), ld, int(iters),
                                _p(dH_res), ctypes.c_void_p(dz_res.data_ptr()), dz_res.stride(0),
                                _stream()))
    return dz_res


def mhc_coeffs_bwd(X, gamma, W, alpha, z, bias, rms, H_pre, H_post, dH_pre, dH_post, dz_res,
                   dX=None, dW=None, dbias=None, dgamma=None, dz=None, want_dgamma=True,
                   want_dz=True, workspace=None):
    """dX (fp32 [T,n,C]) is accumulated into when given."""
    T, n, C = _shape3(X); dt = _dt(X); K = K_of(n)
    dW = _f32((n * C, K), X) if dW is None else dW
    dbias = _f32((K,), X) if dbias is None else dbias
    if want_dgamma and dgamma is None:
        dgamma = _f32((n * C,), X)
    if want_dz and dz is None:
        dz = _f32((T, K), X)
    workspace, (wp, wb) = _ws(workspace, MHC_OP_COEFFS_BWD, T, n, C, dt, X.device)
    _check(lib.mhc_coeffs_bwd(T, n, C, dt, _p(X), _p(gamma), _p(W), _alpha(alpha), _p(z), _p(bias),
                              _p(rms), _p(H_pre), _p(H_post), _p(dH_pre), _p(dH_post), _p(dz_res),
                              _p(dX), _p(dW), _p(dbias), _p(dgamma), _p(dz), wp, wb, _stream()))
    return dict(dX=dX, dW=dW, dbias=dbias, dgamma=dgamma, dz=dz)


def mhc_fwd_pre(X, gamma, eps, W, bias, alpha, iters=20, z_res_in=None, z=None, rms=None,
                H_pre=None, H_post=None, H_res=None, u=None, proj=None, want_proj=False,
                workspace=None):
    T, n, C = _shape3(X); dt = _dt(X)
    z = _f32((T, K_of(n)), X) if z is None else z
    rms = _f32((T,), X) if rms is None else rms
    H_pre = _f32((T, n), X) if H_pre is None else H_pre
    H_post = _f32((T, n), X) if H_post is None else H_post
    H_res = _f32((T, n, n), X) if H_res is None else H_res
    u = torch.empty((T, C), dtype=X.dtype, device=X.device) if u is None else u
    if want_proj and proj is None:
        proj = _f32((T, K_of(n)), X)
    workspace, (wp, wb) = _ws(workspace, MHC_OP_FWD_PRE, T, n, C, dt, X.device)
    _check(lib.mhc_fwd_pre(T, n, C, dt, _p(X), _p(gamma), float(eps), _p(W), _p(bias),
                           _alpha(alpha), int(iters), _p(z_res_in), _p(z), _p(rms), _p(H_pre),
                           _p(H_post), _p(H_res), _p(u), _p(proj), wp, wb, _stream()))
    return dict(z=z, rms=rms, H_pre=H_pre, H_post=H_post, H_res=H_res, u=u, proj=proj)


def mhc_post_res_fwd_pre(X, F_out, H_res, H_post, gamma, eps, W, bias, alpha, iters=20,
                         z_res_in=None, X_out=None, z=None, rms=None, H_pre=None, H_post_next=None,
                         H_res_next=None, u=None, proj=None, want_proj=False, workspace=None):
    """Layer l's mhc_post_res and layer l+1's mhc_fwd_pre in one call: X_out = H_res X +
    H_post^T F_out, then the read side of X_out with the next layer's gamma, eps, W, bias,
    alpha.  Returns the mhc_fwd_pre outputs (H_post, H_res: the next layer's) plus X_out."""
    T, n, C = _shape3(X); dt = _dt(X)
    X_out = torch.empty_like(X) if X_out is None else X_out
    z = _f32((T, K_of(n)), X) if z is None else z
    rms = _f32((T,), X) if rms is None else rms
    H_pre = _f32((T, n), X) if H_pre is None else H_pre
    H_post_next = _f32((T, n), X) if H_post_next is None else H_post_next
    H_res_next = _f32((T, n, n), X) if H_res_next is None else H_res_next
    u = torch.empty((T, C), dtype=X.dtype, device=X.device) if u is None else u
    if want_proj and proj is None:
        proj = _f32((T, K_of(n)), X)
    workspace, (wp, wb) = _ws(workspace, MHC_OP_FWD_PRE, T, n, C, dt, X.device)
    _check(lib.mhc_post_res_fwd_pre(T, n, C, dt, _p(X), _p(F_out), _p(H_res), _p(H_post),
                                    _p(X_out), _p(gamma), float(eps), _p(W), _p(bias),
                                    _alpha(alpha), int(iters), _p(z_res_in), _p(z), _p(rms),
                                    _p(H_pre), _p(H_post_next), _p(H_res_next), _p(u), _p(proj),
                                    wp, wb, _stream()))
    return dict(X_out=X_out, z=z, rms=rms, H_pre=H_pre, H_post=H_post_next, H_res=H_res_next,
                u=u, proj=proj)


def mhc_fwd_pre_noalloc(X, gamma, eps, W, bias, alpha, iters=20, z_res_in=None, z=None,
                        rms=None, H_pre=None, H_post=None, H_res=None, u=None, proj=None,
                        want_proj=False):
    """mhc_fwd_pre without a workspace: the library's device-resident scratch array is
    used (outputs the caller does not pass are still allocated here, by torch)."""
    T, n, C = _shape3(X); dt = _dt(X)
    z = _f32((T, K_of(n)), X) if z is None else z
    rms = _f32((T,), X) if rms is None else rms
    H_pre = _f32((T, n), X) if H_pre is None else H_pre
    H_post = _f32((T, n), X) if H_post is None else H_post
    H_res = _f32((T, n, n), X) if H_res is None else H_res
    u = torch.empty((T, C), dtype=X.dtype, device=X.device) if u is None else u
    if want_proj and proj is None:
        proj = _f32((T, K_of(n)), X)
    _check(lib.mhc_fwd_pre_noalloc(T, n, C, dt, _p(X), _p(gamma), float(eps), _p(W), _p(bias),
                                   _alpha(alpha), int(iters), _p(z_res_in), _p(z), _p(rms),
                                   _p(H_pre), _p(H_post), _p(H_res), _p(u), _p(proj), _stream()))
    return dict(z=z, rms=rms, H_pre=H_pre, H_post=H_post, H_res=H_res, u=u, proj=proj)


def mhc_bwd_pre(dX_out, du, X, gamma, W, alpha, z, bias, rms, H_pre, H_post, H_res, dH_res,
                dH_post, iters=20, z_res_in=None, dX=None, dW=None, dbias=None, dH_pre=None,
                dz=None, dgamma=None, want_dgamma=True, workspace=None):
    T, n, C = _shape3(X); dt = _dt(X); K = K_of(n)
    dX = _f32((T, n, C), X) if dX is None else dX
    dW = _f32((n * C, K), X) if dW is None else dW
    dbias = _f32((K,), X) if dbias is None else dbias
    dH_pre = _f32((T, n), X) if dH_pre is None else dH_pre
    dz = _f32((T, K), X) if dz is None else dz
    if want_dgamma and dgamma is None:
        dgamma = _f32((n * C,), X)
    workspace, (wp, wb) = _ws(workspace, MHC_OP_BWD_PRE, T, n, C, dt, X.device)
    _check(lib.mhc_bwd_pre(T, n, C, dt, _p(dX_out), _p(du), _p(X), _p(gamma), _p(W),
                           _alpha(alpha), _p(z), _p(bias), _p(rms), _p(H_pre), _p(H_post),
                           _p(H_res), _p(dH_res), _p(dH_post), int(iters), _p(z_res_in), _p(dX),
                           _p(dW), _p(dbias), _p(dH_pre), _p(dz), _p(dgamma), wp, wb, _stream()))
    return dict(dX=dX, dW=dW, dbias=dbias, dH_pre=dH_pre, dz=dz, dgamma=dgamma)


def mhc_post_res_bwd_pre(dX_out, du, X, F_out, H_res, H_post, dF=None, dH_res=None,
                         dH_post=None, dH_pre=None):
    """mhc_post_res_bwd (no dX) plus dH_pre = <du, X_k>, from one pass over X."""
    T, n, C = _shape3(X)
    dF = _f32((T, C), X) if dF is None else dF
    dH_res = _f32((T, n, n), X) if dH_res is None else dH_res
    dH_post = _f32((T, n), X) if dH_post is None else dH_post
    dH_pre = _f32((T, n), X) if dH_pre is None else dH_pre
    _check(lib.mhc_post_res_bwd_pre(T, n, C, _dt(X), _p(dX_out), _p(du), _p(X), _p(F_out),
                                    _p(H_res), _p(H_post), _p(dF), _p(dH_res), _p(dH_post),
                                    _p(dH_pre), _stream()))
    return dict(dF=dF, dH_res=dH_res, dH_post=dH_post, dH_pre=dH_pre)


def mhc_bwd_pre_from_dh(dX_out, du, X, gamma, W, alpha, z, bias, rms, H_pre, H_post, H_res,
                        dH_pre, dH_res, dH_post, iters=20, z_res_in=None, dX=None, dW=None,
                        dbias=None, dz=None, dgamma=None, want_dgamma=True, workspace=None):
    """mhc_bwd_pre with dH_pre given (from mhc_post_res_bwd_pre)."""
    T, n, C = _shape3(X); dt = _dt(X); K = K_of(n)
    dX = _f32((T, n, C), X) if dX is None else dX
    dW = _f32((n * C, K), X) if dW is None else dW
    dbias = _f32((K,), X) if dbias is None else dbias
    dz = _f32((T, K), X) if dz is None else dz
    if want_dgamma and dgamma is None:
        dgamma = _f32((n * C,), X)
    workspace, (wp, wb) = _ws(workspace, MHC_OP_BWD_PRE, T, n, C, dt, X.device)
    _check(lib.mhc_bwd_pre_from_dh(T, n, C, dt, _p(dX_out), _p(du), _p(X), _p(gamma), _p(W),
                                   _alpha(alpha), _p(z), _p(bias), _p(rms), _p(H_pre),
                                   _p(H_post), _p(H_res), _p(dH_pre), _p(dH_res), _p(dH_post),
                                   int(iters), _p(z_res_in), _p(dX), _p(dW), _p(dbias), _p(dz),
                                   _p(dgamma), wp, wb, _stream()))
    return dict(dX=dX, dW=dW, dbias=dbias, dz=dz, dgamma=dgamma)


def mhc_post_res_next(X, F_out, H_res, H_post, gamma_next, W_next, workspace, X_out=None):
    """X_out as mhc_post_res, plus the next layer's partial logits left in `workspace`
    (mhc_workspace_size(MHC_OP_NEXT, ...) bytes) for mhc_fwd_pre_next."""
    T, n, C = _shape3(X)
    X_out = torch.empty_like(X) if X_out is None else X_out
    _check(lib.mhc_post_res_next(T, n, C, _dt(X), _p(X), _p(F_out), _p(H_res), _p(H_post),
                                 _p(X_out), _p(gamma_next), _p(W_next), _p(workspace),
                                 workspace.numel(), _stream()))
    return X_out


def mhc_fwd_pre_next(X, eps, bias, alpha, workspace, iters=20, z_res_in=None, z=None, rms=None,
                     H_pre=None, H_post=None, H_res=None, u=None, proj=None, want_proj=False):
    """mhc_fwd_pre's outputs for X = the X_out of the mhc_post_res_next call that filled
    `workspace`."""
    T, n, C = _shape3(X); dt = _dt(X)
    z = _f32((T, K_of(n)), X) if z is None else z
    rms = _f32((T,), X) if rms is None else rms
    H_pre = _f32((T, n), X) if H_pre is None else H_pre
    H_post = _f32((T, n), X) if H_post is None else H_post
    H_res = _f32((T, n, n), X) if H_res is None else H_res
    u = torch.empty((T, C), dtype=X.dtype, device=X.device) if u is None else u
    if want_proj and proj is None:
        proj = _f32((T, K_of(n)), X)
    _check(lib.mhc_fwd_pre_next(T, n, C, dt, _p(X), float(eps), _p(bias), _alpha(alpha),
                                int(iters), _p(z_res_in), _p(z), _p(rms), _p(H_pre), _p(H_post),
                                _p(H_res), _p(u), _p(proj), _p(workspace), workspace.numel(),
                                _stream()))
    return dict(z=z, rms=rms, H_pre=H_pre, H_post=H_post, H_res=H_res, u=u, proj=proj)


def mhc_alpha_bwd(proj, dz, dalpha=None, workspace=None):
    """d loss / d alpha [3] (fp32, on the device) from the forward's unscaled normalised
    projection (the `proj` output of mhc_fwd_pre / mhc_coeffs) and the backward's dz."""
    T, K = proj.shape
    n = {K_of(m): m for m in (1, 2, 4, 8)}.get(K)
    if n is None:
        raise ValueError("proj must be [T, n*n + 2n]")
    dalpha = _f32((3,), proj) if dalpha is None else dalpha
    workspace, (wp, wb) = _ws(workspace, MHC_OP_ALPHA_BWD, T, n, 8, MHC_F32, proj.device)
    _check(lib.mhc_alpha_bwd(T, n, _p(proj), _p(dz), _p(dalpha), wp, wb, _stream()))
    return dalpha


def mhc_composite(H_res, P, gain_row=None, gain_col=None):
    T, n, _ = H_res.shape
    gain_row = _f32((T,), H_res) if gain_row is None else gain_row
    gain_col = _f32((T,), H_res) if gain_col is None else gain_col
    _check(lib.mhc_composite(T, n, _p(H_res), _p(P), _p(gain_row), _p(gain_col), _stream()))
    return gain_row, gain_col


# ------------------------------------------------------------------ stacks
def _ptrs(ts):
    """host array of device pointers (None stays NULL)"""
    if ts is None:
        return None
    return (ctypes.c_void_p * len(ts))(*[t.data_ptr() for t in ts])


def _alphas(layers):
    vals = []
    for p in layers:
        a = p["alpha"]
        vals += [float(v) for v in (a.tolist() if hasattr(a, "tolist") else a)]
    return (ctypes.c_float * len(vals))(*vals)


def mhc_stack_block_size(L: int) -> int:
    return int(lib.mhc_stack_block_size(L))


def mhc_stack_workspace_size(L, B, T, n, C, dtype) -> int:
    return int(lib.mhc_stack_workspace_size(L, B, T, n, C, dtype))


def mhc_stack_forward(X0, layers, F_out, B, eps=1e-6, iters=20, X_save=None, X_L=None, u=None,
                      workspace=None):
    """Forward of a stack of len(layers) layers (dicts with device gamma, W, bias and a
    host alpha triple), keeping X only every B layers.  Returns dict(X_L, X_save,
    workspace); the backward needs X_save and the workspace as the forward left them."""
    T, n, C = _shape3(X0); dt = _dt(X0); L = len(layers)
    nb = (L + B - 1) // B
    if X_save is None:
        X_save = [X0] + [torch.empty_like(X0) for _ in range(nb - 1)]
    X_L = torch.empty_like(X0) if X_L is None else X_L
    if workspace is None:
        workspace = torch.empty(mhc_stack_workspace_size(L, B, T, n, C, dt), dtype=torch.uint8,
                                device=X0.device)
    keep = (_ptrs([p["gamma"] for p in layers]), _ptrs([p["W"] for p in layers]),
            _ptrs([p["bias"] for p in layers]), _ptrs(F_out), _ptrs(u), _ptrs(X_save))
    _check(lib.mhc_stack_forward(L, B, T, n, C, dt, _p(X0), keep[0], keep[1], keep[2],
                                 _alphas(layers), keep[3], keep[4], float(eps), int(iters), keep[5],
                                 _p(X_L), _p(workspace), workspace.numel(), _stream()))
    return dict(X_L=X_L, X_save=X_save, workspace=workspace)


def mhc_stack_backward(X_save, layers, F_out, du, dX_L, B, workspace, iters=20, dX0=None, dW=None,
                       dbias=None, dF=None):
    """Backward of the stack whose forward filled X_save and workspace.  Returns
    dict(dX0, dW, dbias, dF) (dF only when given)."""
    T, n, C = _shape3(X_save[0]); dt = _dt(X_save[0]); L = len(layers); K = K_of(n)
    dX0 = _f32((T, n, C), dX_L) if dX0 is None else dX0
    dW = [_f32((n * C, K), dX_L) for _ in range(L)] if dW is None else dW
    dbias = [_f32((K,), dX_L) for _ in range(L)] if dbias is None else dbias
    keep = (_ptrs(X_save), _ptrs([p["gamma"] for p in layers]), _ptrs([p["W"] for p in layers]),
            _ptrs([p["bias"] for p in layers]), _ptrs(F_out), _ptrs(du), _ptrs(dW), _ptrs(dbias),
            _ptrs(dF))
    _check(lib.mhc_stack_backward(L, B, T, n, C, dt, keep[0], keep[1], keep[2], keep[3],
                                  _alphas(layers), keep[4], keep[5], int(iters), _p(dX_L), _p(dX0),
                                  keep[6], keep[7], keep[8], _p(workspace), workspace.numel(),
                                  _stream()))
    return dict(dX0=dX0, dW=dW, dbias=dbias, dF=dF)

