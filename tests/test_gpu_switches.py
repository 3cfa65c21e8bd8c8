"""The environment switches of include/mhc.h on the GPU.

MHC_FORCE_PATH: the whole layer (forward read side, post + residual, both backward
calls, the scale gradient) on each path -- the default (single-read forward and MFMA
projections where the shape allows), "twopass" (the forward read side in two passes over
X) and "vector" (the vector kernels of the projections) -- against the oracle at the
parity tolerances, and the paths against each other.

MHC_CHECK_FINITE: finite inputs give the unchecked results bitwise; a NaN or Inf input
returns MHC_ERR_NONFINITE before anything is written; an output that overflows returns
MHC_ERR_NONFINITE with the output written; without the switch a NaN input is computed
through (no status)."""
import os

import numpy as np
import pytest

from tests._util import TOL, to_dev
from tests.test_gpu_parity import _compare, _make, _oracle, _run_fused

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def M():
    from manifold_constrained_residuals_amd import mhc
    assert torch.cuda.is_available()
    return mhc


class _env:
    """Set an environment variable for the duration of a block (the library reads it on
    every call)."""

    def __init__(self, key, value):
        self.key, self.value = key, value

    def __enter__(self):
        self.old = os.environ.get(self.key)
        if self.value is None:
            os.environ.pop(self.key, None)
        else:
            os.environ[self.key] = self.value

    def __exit__(self, *a):
        if self.old is None:
            os.environ.pop(self.key, None)
        else:
            os.environ[self.key] = self.old


# (dtype, n, T, C, alpha): the single-read shape (C = 256 G, G = 16 and 4), an n = 4 bf16
# shape that only the two-pass path takes (C = 384), and fp32
PATH_CASES = [
    ("bf16", 4, 300, 4096, 1 / 128),
    ("bf16", 4, 77, 1024, 1 / 64),
    ("bf16", 4, 45, 384, 1 / np.sqrt(4 * 384)),
    ("f32", 4, 33, 256, 1.0),
]
PATHS = [None, "twopass", "vector"]


@pytest.mark.parametrize("case", PATH_CASES, ids=[f"{c[0]}-T{c[2]}-C{c[3]}" for c in PATH_CASES])
def test_force_path_every_path_matches_oracle(M, case):
    wl, p, tk = _make(*case, seed=41)
    f, b = _oracle(wl, p, tk)
    outs = {}
    for path in PATHS:
        print(f"[force path] {case} {path or 'default'}", flush=True)
        with _env("MHC_FORCE_PATH", path):
            g = _run_fused(M, wl, p, tk)
        _compare(wl, f, b, g, case)
        outs[path] = g
    # the paths agree with each other within the same tolerances (relative to the oracle's
    # scale)
    tol = TOL["f32"]
    for path in PATHS[1:]:
        for k in ("z", "rms", "H_pre", "H_post", "H_res", "dX", "dW", "dbias", "dz"):
            a, r = np.asarray(outs[path][k], np.float64), np.asarray(outs[None][k], np.float64)
            e = np.abs(a - r).max() / max(np.abs(r).max(), 1e-30)
            assert e <= 2 * tol, f"{k}: path {path} vs default {e:.2e}"


def _fwd_inputs(M, T=64, C=512, seed=5):
    wl, p, tk = _make("bf16", 4, T, C, 1 / np.sqrt(4 * C), seed=seed)
    X = to_dev(tk["X"], torch)
    g, W, b = (torch.from_numpy(p[k]).cuda() for k in ("gamma", "W", "bias"))
    return wl, p, X, g, W, b


def test_check_finite_passes_finite_inputs_bitwise(M):
    wl, p, X, g, W, b = _fwd_inputs(M)
    ref = M.mhc_fwd_pre(X, g, wl.eps, W, b, p["alpha"], wl.iters, want_proj=True)
    with _env("MHC_CHECK_FINITE", "1"):
        got = M.mhc_fwd_pre(X, g, wl.eps, W, b, p["alpha"], wl.iters, want_proj=True)
    torch.cuda.synchronize()
    for k in ref:
        a, r = got[k], ref[k]
        if a.dtype == torch.bfloat16:
            a, r = a.view(torch.int16), r.view(torch.int16)
        assert torch.equal(a, r), k


@pytest.mark.parametrize("bad", [float("nan"), float("inf")])
def test_check_finite_rejects_nonfinite_input_before_writing(M, bad):
    wl, p, X, g, W, b = _fwd_inputs(M)
    X[3, 1, 7] = bad
    T, n, C = X.shape
    out = {k: v.fill_(-7.0) for k, v in
           M.mhc_fwd_pre(X, g, wl.eps, W, b, p["alpha"], wl.iters, want_proj=True).items()}
    torch.cuda.synchronize()
    with _env("MHC_CHECK_FINITE", "1"):
        with pytest.raises(M.MhcError) as ei:
            M.mhc_fwd_pre(X, g, wl.eps, W, b, p["alpha"], wl.iters, **out)
    assert ei.value.status == -10
    torch.cuda.synchronize()
    for k, v in out.items():
        assert bool((v.float() == -7.0).all()), f"{k} was written"
    # a NaN in the backward's incoming gradient is caught by the backward calls too
    Gx = torch.zeros((T, n, C), dtype=torch.bfloat16, device="cuda")
    Gx[0, 0, 0] = bad
    with _env("MHC_CHECK_FINITE", "1"):
        with pytest.raises(M.MhcError) as ei:
            M.mhc_post_res_bwd(Gx, X, X[:, 0].contiguous(), out["H_res"], out["H_post"])
    assert ei.value.status == -10


def test_check_finite_reports_output_overflow_with_output_written(M):
    T, n, C = 16, 4, 256
    X = torch.full((T, n, C), 3.0e38, dtype=torch.bfloat16, device="cuda")
    H = torch.full((T, n), 1.0, dtype=torch.float32, device="cuda")     # u = 4 * 3e38 -> Inf
    u = torch.zeros((T, C), dtype=torch.bfloat16, device="cuda")
    with _env("MHC_CHECK_FINITE", "1"):
        with pytest.raises(M.MhcError) as ei:
            M.mhc_pre(X, H, u)
    assert ei.value.status == -10
    torch.cuda.synchronize()
    assert bool(torch.isinf(u.float()).all()), "the output was not written"


def test_without_check_nan_input_flows_through(M):
    wl, p, X, g, W, b = _fwd_inputs(M)
    X[5, 2, 9] = float("nan")
    with _env("MHC_CHECK_FINITE", None):
        got = M.mhc_fwd_pre(X, g, wl.eps, W, b, p["alpha"], wl.iters)
    torch.cuda.synchronize()
    assert bool(torch.isnan(got["z"][5]).all())
    assert bool(torch.isfinite(got["z"][:5]).all())


def test_single_read_timeout_poisons_u_and_exits(M):
    """The single-read pass's bounded wait, forced from the host: MHC_SR_TEST_TIMEOUT makes
    every reader expect tags that never come and wait 20 us for them.  The kernel gives up
    and exits normally; u is NaN on every token, the outputs that come from the finishing
    pass (z, rms, H, proj) are bitwise those of a normal call, and the next normal call is
    exact again (the exchange ring starts cleared)."""
    wl, p, tk = _make("bf16", 4, 300, 4096, 1 / 128, seed=17)
    X = to_dev(tk["X"], torch)
    g, W, b = (torch.from_numpy(p[k]).cuda() for k in ("gamma", "W", "bias"))
    ref = M.mhc_fwd_pre(X, g, wl.eps, W, b, p["alpha"], wl.iters, want_proj=True)
    torch.cuda.synchronize()
    with _env("MHC_SR_TEST_TIMEOUT", "1"):
        bad = M.mhc_fwd_pre(X, g, wl.eps, W, b, p["alpha"], wl.iters, want_proj=True)
        torch.cuda.synchronize()
    assert bool(torch.isnan(bad["u"].float()).all()), "u not poisoned"
    for k in ("z", "rms", "H_pre", "H_post", "H_res", "proj"):
        assert torch.equal(bad[k], ref[k]), k
    again = M.mhc_fwd_pre(X, g, wl.eps, W, b, p["alpha"], wl.iters, want_proj=True)
    torch.cuda.synchronize()
    assert torch.equal(again["u"].view(torch.int16), ref["u"].view(torch.int16))
