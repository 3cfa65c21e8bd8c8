"""fp64 CPU oracle for the per-layer mHC operator -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and its
binding) never imports, links or calls it, and this package imports nothing from
the product path.

The arithmetic lives in ``mhc_oracle.c`` (plain C, fp64, OpenMP over tokens); this
module only builds it, marshals numpy arrays through ctypes and chains the steps
in the order the update rule of the mHC pages fixes (chatgpz.de, "Von
Residualverbindungen zu Hyperverbindungen": X' = H_res X + H_post^T F(H_pre X)).
The only arithmetic done here is assembling the per-step outputs into one dict.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mhc_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (fp64, no fast-math, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
             _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        i64, i32, dbl = ctypes.c_int64, ctypes.c_int, ctypes.c_double
        sig = {
            "orc_coeffs": [i64, i32, i64, dp, dp, dbl, dp, dp, dp, dp, dp, dp, dp],
            "orc_sinkhorn_one": [i32, dp, i32, dp, dp, dp, dp, dp],
            "orc_sinkhorn": [i64, i32, dp, i64, i32, dp],
            "orc_pre": [i64, i32, i64, dp, dp, dp],
            "orc_post_res": [i64, i32, i64, dp, dp, dp, dp, dp],
            "orc_post_res_bwd": [i64, i32, i64, dp, dp, dp, dp, dp, dp, dp, dp, dp],
            "orc_pre_bwd": [i64, i32, i64, dp, dp, dp, dp, dp],
            "orc_sinkhorn_bwd_one": [i32, dp, i32, dp, dp],
            "orc_sinkhorn_bwd": [i64, i32, dp, i64, i32, dp, dp],
            "orc_gating_bwd": [i64, i32, dp, dp, dp, dp],
            "orc_coeffs_bwd": [i64, i32, i64, dp, dp, dbl, dp, dp, dp, dp, dp, dp, dp],
            "orc_composite": [i64, i32, dp, dp, dp, dp],
            "orc_alpha_bwd": [i64, i32, i64, dp, dp, dbl, dp, dp, dp],
        }
        for name, args in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = None
        _lib = L
    return _lib


def _d(a):
    """fp64 C-contiguous view/copy (exact widening of fp32 / bf16-as-fp32)."""
    return np.ascontiguousarray(a, dtype=np.float64)


def _p(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def K_of(n: int) -> int:
    return n * n + 2 * n


# ---------------------------------------------------------------- single steps
def coeffs(X, gamma, eps, W, bias, alpha):
    X = _d(X)
    T, n, C = X.shape
    K = K_of(n)
    gamma, W, bias, alpha = _d(gamma), _d(W), _d(bias), _d(alpha)
    z = np.empty((T, K)); r = np.empty(T)
    Hpre = np.empty((T, n)); Hpost = np.empty((T, n))
    lib().orc_coeffs(T, n, C, _p(X), _p(gamma), float(eps), _p(W), _p(bias), _p(alpha),
                     _p(z), _p(r), _p(Hpre), _p(Hpost))
    return dict(z=z, r=r, Hpre=Hpre, Hpost=Hpost)


def sinkhorn(zres, n, iters=20):
    zres = _d(zres).reshape(-1, n * n)
    T = zres.shape[0]
    H = np.empty((T, n, n))
    lib().orc_sinkhorn(T, n, _p(zres), n * n, int(iters), _p(H))
    return H


def sinkhorn_trace(zres, n, iters=20):
    """One matrix: H plus every row/column divisor and intermediate matrix."""
    zres = _d(zres).reshape(n * n)
    H = np.empty((n, n)); rho = np.empty((iters, n)); kap = np.empty((iters, n))
    Yr = np.empty((iters, n, n)); Yc = np.empty((iters, n, n))
    lib().orc_sinkhorn_one(n, _p(zres), int(iters), _p(H), _p(rho), _p(kap), _p(Yr), _p(Yc))
    return dict(H=H, rho=rho, kap=kap, Yrow=Yr, Ycol=Yc)


def pre(X, Hpre):
    X = _d(X); T, n, C = X.shape
    Hpre = _d(Hpre)
    u = np.empty((T, C))
    lib().orc_pre(T, n, C, _p(X), _p(Hpre), _p(u))
    return u


def post_res(X, F, Hres, Hpost):
    X = _d(X); T, n, C = X.shape
    F, Hres, Hpost = _d(F), _d(Hres), _d(Hpost)
    Xo = np.empty((T, n, C))
    lib().orc_post_res(T, n, C, _p(X), _p(F), _p(Hres), _p(Hpost), _p(Xo))
    return Xo


def post_res_bwd(G, X, F, Hres, Hpost, want_dx=True):
    X = _d(X); T, n, C = X.shape
    G, F, Hres, Hpost = _d(G), _d(F), _d(Hres), _d(Hpost)
    dF = np.empty((T, C)); dHres = np.empty((T, n, n)); dHpost = np.empty((T, n))
    dXd = np.empty((T, n, C)) if want_dx else None
    lib().orc_post_res_bwd(T, n, C, _p(G), _p(X), _p(F), _p(Hres), _p(Hpost),
                           _p(dF), _p(dHres), _p(dHpost), _p(dXd))
    return dict(dF=dF, dHres=dHres, dHpost=dHpost, dXdir=dXd)


def pre_bwd(g, X, Hpre, dX=None):
    """dH_pre, and dX += H_pre (x) g when dX (fp64, modified in place) is given."""
    X = _d(X); T, n, C = X.shape
    g, Hpre = _d(g), _d(Hpre)
    dHpre = np.empty((T, n))
    if dX is not None:
        assert dX.dtype == np.float64 and dX.flags.c_contiguous
    lib().orc_pre_bwd(T, n, C, _p(g), _p(X), _p(Hpre), _p(dHpre), _p(dX))
    return dHpre


def sinkhorn_bwd(zres, dHres, n, iters=20):
    zres = _d(zres).reshape(-1, n * n)
    T = zres.shape[0]
    dH = _d(dHres).reshape(T, n * n)
    dz = np.empty((T, n * n))
    lib().orc_sinkhorn_bwd(T, n, _p(zres), n * n, int(iters), _p(dH), _p(dz))
    return dz


def gating_bwd(z, dHpre, dHpost, n):
    z = _d(z); T = z.shape[0]
    dz = np.zeros((T, K_of(n)))
    lib().orc_gating_bwd(T, n, _p(z), _p(_d(dHpre)), _p(_d(dHpost)), _p(dz))
    return dz


def coeffs_bwd(X, gamma, eps, W, alpha, dz, dX=None, want_dgamma=True):
    X = _d(X); T, n, C = X.shape
    N, K = n * C, K_of(n)
    dW = np.empty((N, K)); db = np.empty(K)
    dg = np.empty(N) if want_dgamma else None
    if dX is not None:
        assert dX.dtype == np.float64 and dX.flags.c_contiguous
    lib().orc_coeffs_bwd(T, n, C, _p(X), _p(_d(gamma)), float(eps), _p(_d(W)), _p(_d(alpha)),
                         _p(_d(dz)), _p(dX), _p(dW), _p(db), _p(dg))
    return dict(dW=dW, db=db, dgamma=dg)


def alpha_bwd(X, gamma, eps, W, dz):
    """d loss / d alpha (3 groups: pre, post, res) given the logit gradient dz."""
    X = _d(X); T, n, C = X.shape
    out = np.empty(3)
    lib().orc_alpha_bwd(T, n, C, _p(X), _p(_d(gamma)), float(eps), _p(_d(W)), _p(_d(dz)), _p(out))
    return out


def composite(Hres, P):
    """P <- H_res P in place (fp64 [T,n,n]); returns (gain_row, gain_col)."""
    T, n, _ = Hres.shape
    Hres = _d(Hres)
    assert P.dtype == np.float64 and P.flags.c_contiguous
    gr = np.empty(T); gc = np.empty(T)
    lib().orc_composite(T, n, _p(Hres), _p(P), _p(gr), _p(gc))
    return gr, gc


# ---------------------------------------------------------------- chained layer
def forward(X, F, gamma, eps, W, bias, alpha, iters=20, zres_in=None):
    """One mHC layer forward.  zres_in (optional [T, n*n]) replaces the projected
    res logits at the Sinkhorn input (the projection's z is still returned)."""
    X = _d(X); n = X.shape[1]
    c = coeffs(X, gamma, eps, W, bias, alpha)
    zres = c["z"][:, 2 * n:] if zres_in is None else _d(zres_in)
    Hres = sinkhorn(zres, n, iters)
    u = pre(X, c["Hpre"])
    Xo = post_res(X, F, Hres, c["Hpost"])
    return dict(z=c["z"], r=c["r"], Hpre=c["Hpre"], Hpost=c["Hpost"], Hres=Hres, u=u, Xout=Xo)


def forward_unconstrained(X, F, gamma, eps, W, bias, alpha):
    """One layer of plain hyper-connections (the comparison the mHC pages draw in
    "Warum Hyperverbindungen instabil werden" on chatgpz.de): the same coefficients and
    gates, but the residual mixer is the raw res logit block Z (no exp, no Sinkhorn
    projection), X' = Z X + H_post^T F."""
    X = _d(X); n = X.shape[1]
    c = coeffs(X, gamma, eps, W, bias, alpha)
    Hres = np.ascontiguousarray(c["z"][:, 2 * n:]).reshape(-1, n, n)
    Xo = post_res(X, F, Hres, c["Hpost"])
    return dict(z=c["z"], r=c["r"], Hpre=c["Hpre"], Hpost=c["Hpost"], Hres=Hres, Xout=Xo)


def backward(X, F, gamma, eps, W, bias, alpha, G, g, fwd, iters=20, zres_in=None,
             learn_alpha=False):
    """Gradient of L = <G, X'> + <g, u> with F's output held fixed.  Returns dX, dF,
    dW, db, dgamma, dz and the per-map gradients; with learn_alpha also dalpha [3]."""
    X = _d(X); T, n, C = X.shape
    pb = post_res_bwd(G, X, F, fwd["Hres"], fwd["Hpost"], want_dx=True)
    dX = pb["dXdir"]
    dHpre = pre_bwd(g, X, fwd["Hpre"], dX=dX)
    dz = gating_bwd(fwd["z"], dHpre, pb["dHpost"], n)
    zres = fwd["z"][:, 2 * n:] if zres_in is None else _d(zres_in)
    dz[:, 2 * n:] = sinkhorn_bwd(zres, pb["dHres"], n, iters)
    cb = coeffs_bwd(X, gamma, eps, W, alpha, dz, dX=dX)
    return dict(dX=dX, dF=pb["dF"], dW=cb["dW"], db=cb["db"], dgamma=cb["dgamma"], dz=dz,
                dHpre=dHpre, dHpost=pb["dHpost"], dHres=pb["dHres"],
                dalpha=alpha_bwd(X, gamma, eps, W, dz) if learn_alpha else None)


def loss(X, F, gamma, eps, W, bias, alpha, G, g, iters=20, zres_in=None):
    """The scalar whose gradient ``backward`` returns."""
    f = forward(X, F, gamma, eps, W, bias, alpha, iters, zres_in)
    return float(np.sum(_d(G) * f["Xout"]) + np.sum(_d(g) * f["u"]))
