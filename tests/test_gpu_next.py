"""GPU parity of the cross-layer pair mhc_post_res_next -> mhc_fwd_pre_next.

Layer l's maps come from the oracle on X; layer l+1 has its own seeded params.
Expected values are the oracle's: X_{l+1} = H_res X + H_post^T F in fp64, then
(stored in bf16, as the next layer sees it) the next layer's forward on it.

- X_out of mhc_post_res_next is bitwise the X_out of mhc_post_res, and within one
  bf16 rounding of the exact value;
- z, r, H_pre, H_post, H_res (fp32, 1e-5) and u (bf16, 1e-2) of mhc_fwd_pre_next
  match the oracle's next-layer forward; with injected res logits too.
Shapes span several token tiles, ragged tails, channel splits down to one 64-channel
chunk, and T = 1."""
import numpy as np
import pytest

from manifold_constrained_residuals_amd import inputs as I
from tests._util import proj_ref, TOL, assert_close, to_dev, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

CASES = [(300, 4096), (77, 1024), (129, 192), (1, 64), (1000, 2048)]


@pytest.fixture(scope="module")
def M():
    from manifold_constrained_residuals_amd import mhc
    assert torch.cuda.is_available()
    return mhc


def _one_rounding(name, gpu, ref):
    slack = 1e-6 * np.abs(ref).max()
    ulp_half = np.ldexp(1.0, np.frexp(np.abs(ref))[1] - 9)
    bad = np.abs(gpu - ref) > ulp_half + slack
    assert not bad.any(), f"{name}: {bad.sum()} elements beyond one bf16 rounding"


def _pair(T, C, seed, zsplit=None):
    wl = I.Workload("next", T=T, n=4, C=C, dtype="bf16", seed=seed, alpha=1 / np.sqrt(4 * C),
                    backward=False, zres_split=zsplit)
    return wl, I.layer_params(wl, 0), I.layer_params(wl, 1), I.layer_tokens(wl, layer=0)


@pytest.mark.parametrize("T,C", CASES, ids=[f"T{t}-C{c}" for t, c in CASES])
def test_post_res_next_then_fwd_pre_next(M, T, C):
    import oracle
    print(f"[next] T={T} C={C}", flush=True)
    wl, p0, p1, tk = _pair(T, C, seed=50 + T % 7)
    X, F = I.widen(tk["X"]), I.widen(tk["F"])
    f0 = oracle.forward(X, F, p0["gamma"], wl.eps, p0["W"], p0["bias"], p0["alpha"], wl.iters)
    X1 = f0["Xout"]                                         # exact next-layer input

    Xd, Fd = to_dev(tk["X"], torch), to_dev(tk["F"], torch)
    Hres = torch.from_numpy(f0["Hres"].astype(np.float32)).cuda()
    Hpost = torch.from_numpy(f0["Hpost"].astype(np.float32)).cuda()
    g1, W1, b1 = (torch.from_numpy(p1[k]).cuda() for k in ("gamma", "W", "bias"))
    ws = M.workspace(M.MHC_OP_NEXT, T, 4, C, M.MHC_BF16, "cuda")
    Xn = M.mhc_post_res_next(Xd, Fd, Hres, Hpost, g1, W1, ws)
    Xp = M.mhc_post_res(Xd, Fd, Hres, Hpost)
    g = M.mhc_fwd_pre_next(Xn, wl.eps, b1, p1["alpha"], ws, wl.iters, want_proj=True)
    torch.cuda.synchronize()
    assert torch.equal(Xn.view(torch.int16), Xp.view(torch.int16)), "X_out differs from mhc_post_res"
    xo = to_host(Xn, torch)
    assert_close("X_out", xo, X1, TOL["bf16"])
    _one_rounding("X_out", xo, X1)
    # the next layer against the oracle run on the X' the GPU wrote (bf16 values, exact
    # in fp64): a correctly rounded X' may differ from the oracle's own rounding by one
    # bf16 ulp in an element, which the unscaled projection would show
    f1 = oracle.forward(xo, np.zeros((T, C)), p1["gamma"], wl.eps, p1["W"], p1["bias"],
                        p1["alpha"], wl.iters)
    tol = TOL["f32"]
    assert_close("z", to_host(g["z"], torch), f1["z"], tol)
    assert_close("rms", to_host(g["rms"], torch), f1["r"], tol)
    assert_close("H_pre", to_host(g["H_pre"], torch), f1["Hpre"], tol)
    assert_close("H_post", to_host(g["H_post"], torch), f1["Hpost"], tol)
    assert_close("H_res", to_host(g["H_res"], torch), f1["Hres"], tol)
    assert_close("u", to_host(g["u"], torch), f1["u"], TOL["bf16"])
    assert_close("proj", to_host(g["proj"], torch), proj_ref(f1["z"], p1["bias"], p1["alpha"], 4),
                 tol)


def test_fwd_pre_next_with_injected_res_logits(M):
    import oracle
    T, C = 130, 512
    wl, p0, p1, tk = _pair(T, C, seed=71, zsplit=(4.0, 0.01))
    zin = tk.pop("ZRES")
    X, F = I.widen(tk["X"]), I.widen(tk["F"])
    f0 = oracle.forward(X, F, p0["gamma"], wl.eps, p0["W"], p0["bias"], p0["alpha"], wl.iters)
    Xd, Fd = to_dev(tk["X"], torch), to_dev(tk["F"], torch)
    Hres = torch.from_numpy(f0["Hres"].astype(np.float32)).cuda()
    Hpost = torch.from_numpy(f0["Hpost"].astype(np.float32)).cuda()
    g1, W1, b1 = (torch.from_numpy(p1[k]).cuda() for k in ("gamma", "W", "bias"))
    ws = M.workspace(M.MHC_OP_NEXT, T, 4, C, M.MHC_BF16, "cuda")
    Xn = M.mhc_post_res_next(Xd, Fd, Hres, Hpost, g1, W1, ws)
    g = M.mhc_fwd_pre_next(Xn, wl.eps, b1, p1["alpha"], ws, wl.iters,
                           z_res_in=torch.from_numpy(zin).cuda())
    torch.cuda.synchronize()
    f1 = oracle.forward(to_host(Xn, torch), np.zeros((T, C)), p1["gamma"], wl.eps, p1["W"],
                        p1["bias"], p1["alpha"], wl.iters, zin)
    assert_close("z", to_host(g["z"], torch), f1["z"], TOL["f32"])
    assert_close("H_res", to_host(g["H_res"], torch), f1["Hres"], TOL["f32"])
    assert_close("u", to_host(g["u"], torch), f1["u"], TOL["bf16"])
