"""mhc_fwd_pre_noalloc (the forward read side without a workspace, on the library's
device-resident scratch array) against mhc_fwd_pre: two calls in a row on the same
GPU, the second with a smaller input, each bitwise equal to mhc_fwd_pre on the same
inputs (the same kernels on the same partition) and within the tolerances of the
fp64 oracle."""
import numpy as np
import pytest

from manifold_constrained_residuals_amd import inputs as I
from tests._util import TOL, assert_close, proj_ref, to_dev, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def M():
    from manifold_constrained_residuals_amd import mhc
    assert torch.cuda.is_available()
    return mhc


KEYS = ("z", "rms", "H_pre", "H_post", "H_res", "u", "proj")


def _case(M, T, C, seed, rows=None):
    """rows: the tokens the oracle checks (all by default)."""
    import oracle
    wl = I.Workload("noalloc", T=T, n=4, C=C, dtype="bf16", seed=seed, alpha=1 / np.sqrt(4 * C),
                    backward=False)
    p = I.layer_params(wl)
    tk = I.layer_tokens(wl)
    X = to_dev(tk["X"], torch)
    g, W, b = (torch.from_numpy(p[k]).cuda() for k in ("gamma", "W", "bias"))
    # outputs poisoned so that an unwritten element shows
    out = {k: v.fill_(float("nan")) for k, v in
           M.mhc_fwd_pre(X, g, wl.eps, W, b, p["alpha"], wl.iters, want_proj=True).items()}
    torch.cuda.synchronize()
    na = M.mhc_fwd_pre_noalloc(X, g, wl.eps, W, b, p["alpha"], wl.iters, **out)
    ref = M.mhc_fwd_pre(X, g, wl.eps, W, b, p["alpha"], wl.iters, want_proj=True)
    torch.cuda.synchronize()
    for k in KEYS:
        a, r = na[k], ref[k]
        if a.dtype == torch.bfloat16:
            a, r = a.view(torch.int16), r.view(torch.int16)
        assert torch.equal(a, r), f"{k}: no-alloc result differs from mhc_fwd_pre (T={T}, C={C})"
    rs = np.arange(T) if rows is None else np.asarray(rows)
    f = oracle.forward(I.widen(tk["X"][rs]), I.widen(tk["F"][rs]), p["gamma"], wl.eps, p["W"],
                       p["bias"], p["alpha"], wl.iters)
    h = lambda k: to_host(na[k], torch)[rs]
    tol = TOL["f32"]
    assert_close("z", h("z"), f["z"], tol)
    assert_close("rms", h("rms"), f["r"], tol)
    assert_close("H_pre", h("H_pre"), f["Hpre"], tol)
    assert_close("H_post", h("H_post"), f["Hpost"], tol)
    assert_close("H_res", h("H_res"), f["Hres"], tol)
    assert_close("u", h("u"), f["u"], TOL["bf16"])
    assert_close("proj", h("proj"), proj_ref(f["z"], p["bias"], p["alpha"], 4), tol)


def test_noalloc_forward_two_calls_second_smaller(M):
    # the first three run the single-read pass (C = 256 G, G in {16, 8, 4}: its exchange
    # ring in the scratch keeps the previous call's tags), the last the two-pass path; the
    # first is the benchmark's layer size, its oracle check on the first and last tiles
    # and a middle stretch
    T0 = 16384
    rows = np.r_[0:48, 8000:8048, T0 - 48:T0]
    for T, C, seed, rs in ((T0, 4096, 60, rows), (1000, 2048, 61, None), (300, 1024, 62, None),
                           (77, 512, 63, None)):
        print(f"[noalloc] T={T} C={C}", flush=True)
        _case(M, T, C, seed, rs)


def test_noalloc_rejects_oversized_scratch(M):
    X = torch.empty((8, 4, 8), dtype=torch.bfloat16, device="cuda")
    T, n, C = 262144, 4, 4096       # needs more than MHC_NOALLOC_SCRATCH_BYTES
    assert M.mhc_workspace_size(M.MHC_OP_FWD_PRE, T, n, C, M.MHC_BF16) > 64 << 20
    import ctypes
    A = ctypes.c_void_p(X.data_ptr())
    al = (ctypes.c_float * 3)(1, 1, 1)
    st = M.lib.mhc_fwd_pre_noalloc(T, n, C, M.MHC_BF16, A, A, 1e-6, A, A, al, 20, None, A, A, A, A,
                                   A, A, None, None)
    assert st == -9
