"""GPU checks of layer-block recomputation over a stack of layers.

- fp32, 4 layers, n = 4 and n = 2: X_L, dX0, every layer's dW, db and dF against the
  fp64 oracle run layer by layer over the whole stack (forward, then backward with
  each layer's dX as the next layer down's dX_out), for block sizes 1 (every X
  kept), 2 and 4.
- bf16, 5 layers on the MFMA paths: for block sizes 1, 2, 3 and 5 the results are
  bitwise those of the single-layer entry points chained with every X kept and dX
  rounded to bf16 between layers (the recomputed X are the forward's bits); the
  chain's forward goes through the cross-layer pair like the runner's, its backward
  through mhc_post_res_bwd + mhc_bwd_pre (bitwise the runner's split backward).
"""
import numpy as np
import pytest

from manifold_constrained_residuals_amd import inputs as I
from tests._util import TOL, assert_close, to_dev, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def M():
    from manifold_constrained_residuals_amd import mhc
    assert torch.cuda.is_available()
    return mhc


def _stack_inputs(wl, L):
    params = [I.layer_params(wl, layer=l) for l in range(L)]
    toks = [I.layer_tokens(wl, layer=l, which=("X", "F", "GX", "GU")) for l in range(L)]
    return params, toks


def _dev_layers(params):
    return [dict(gamma=torch.from_numpy(p["gamma"]).cuda(), W=torch.from_numpy(p["W"]).cuda(),
                 bias=torch.from_numpy(p["bias"]).cuda(), alpha=p["alpha"]) for p in params]


def _run_stack(M, wl, params, toks, L, B, copy_x0=False):
    X0 = to_dev(toks[0]["X"], torch)
    F = [to_dev(t["F"], torch) for t in toks]
    du = [to_dev(t["GU"], torch) for t in toks]
    GL = to_dev(toks[L - 1]["GX"], torch)
    layers = _dev_layers(params)
    X_save = None
    if copy_x0:
        X_save = [torch.empty_like(X0) for _ in range((L + B - 1) // B)]
    f = M.mhc_stack_forward(X0, layers, F, B, wl.eps, wl.iters, X_save=X_save)
    dF = [torch.empty((wl.T, wl.C), dtype=torch.float32, device="cuda") for _ in range(L)]
    b = M.mhc_stack_backward(f["X_save"], layers, F, du, GL, B, f["workspace"], wl.iters, dF=dF)
    torch.cuda.synchronize()
    return f["X_L"], b


@pytest.mark.parametrize("n", [4, 2])
def test_stack_fp32_matches_oracle_chain(M, n):
    import oracle
    L = 4
    wl = I.Workload("stack", T=70, n=n, C=264, dtype="f32", seed=9, alpha=1.0, backward=True,
                    f_scale=0.1)
    params, toks = _stack_inputs(wl, L)
    # oracle: forward through the stack, then backward layer by layer
    X = [I.widen(toks[0]["X"]).astype(np.float64)]
    fw = []
    for l in range(L):
        p = params[l]
        f = oracle.forward(X[l], I.widen(toks[l]["F"]), p["gamma"], wl.eps, p["W"], p["bias"],
                           p["alpha"], wl.iters)
        fw.append(f)
        X.append(f["Xout"])
    G = I.widen(toks[L - 1]["GX"]).astype(np.float64)
    ref = [None] * L
    for l in reversed(range(L)):
        p = params[l]
        b = oracle.backward(X[l], I.widen(toks[l]["F"]), p["gamma"], wl.eps, p["W"], p["bias"],
                            p["alpha"], G, I.widen(toks[l]["GU"]), fw[l], wl.iters)
        ref[l] = b
        G = b["dX"]
    tol = TOL["f32"]
    for B in (1, 2, 4):
        print(f"[stack fp32] n={n} L={L} B={B}", flush=True)
        XL, g = _run_stack(M, wl, params, toks, L, B, copy_x0=(B == 2))
        assert_close(f"X_L B={B}", to_host(XL, torch), X[L], tol)
        assert_close(f"dX0 B={B}", to_host(g["dX0"], torch), ref[0]["dX"], tol)
        for l in range(L):
            assert_close(f"dW[{l}] B={B}", to_host(g["dW"][l], torch), ref[l]["dW"], tol)
            assert_close(f"db[{l}] B={B}", to_host(g["dbias"][l], torch), ref[l]["db"], tol)
            assert_close(f"dF[{l}] B={B}", to_host(g["dF"][l], torch), ref[l]["dF"], tol)


def _chain_reference(M, wl, params, toks, L):
    """Single-layer entry points, every X kept, dX rounded to bf16 between layers; the
    forward through the cross-layer pair (mhc_post_res_next / mhc_fwd_pre_next), as
    the stack runner does for this shape."""
    layers = _dev_layers(params)
    X = [to_dev(toks[0]["X"], torch)]
    fw = []
    nws = M.workspace(M.MHC_OP_NEXT, wl.T, wl.n, wl.C, M._dt(X[0]), X[0].device)
    for l in range(L):
        p = layers[l]
        if l == 0:
            f = M.mhc_fwd_pre(X[l], p["gamma"], wl.eps, p["W"], p["bias"], p["alpha"], wl.iters)
        else:
            f = M.mhc_fwd_pre_next(X[l], wl.eps, p["bias"], p["alpha"], nws, wl.iters)
        fw.append(f)
        Fl = to_dev(toks[l]["F"], torch)
        if l + 1 < L:
            q = layers[l + 1]
            X.append(M.mhc_post_res_next(X[l], Fl, f["H_res"], f["H_post"], q["gamma"], q["W"], nws))
        else:
            X.append(M.mhc_post_res(X[l], Fl, f["H_res"], f["H_post"]))
    G = to_dev(toks[L - 1]["GX"], torch)
    out = [None] * L
    for l in reversed(range(L)):
        p, f = layers[l], fw[l]
        Fl, dul = to_dev(toks[l]["F"], torch), to_dev(toks[l]["GU"], torch)
        pb = M.mhc_post_res_bwd(G, X[l], Fl, f["H_res"], f["H_post"])
        bb = M.mhc_bwd_pre(G, dul, X[l], p["gamma"], p["W"], p["alpha"], f["z"], p["bias"],
                           f["rms"], f["H_pre"], f["H_post"], f["H_res"], pb["dH_res"],
                           pb["dH_post"], wl.iters, want_dgamma=False)
        out[l] = dict(dW=bb["dW"], db=bb["dbias"], dF=pb["dF"], dX=bb["dX"])
        G = bb["dX"].to(torch.bfloat16)
    torch.cuda.synchronize()
    return X[L], out


@pytest.mark.parametrize("B", [1, 2, 3, 5])
def test_stack_bf16_recompute_is_bitwise(M, B):
    L = 5
    wl = I.Workload("stack", T=300, n=4, C=512, dtype="bf16", seed=12, alpha=1 / np.sqrt(2048),
                    backward=True)
    params, toks = _stack_inputs(wl, L)
    print(f"[stack bf16] L={L} B={B}", flush=True)
    XL_ref, ref = _chain_reference(M, wl, params, toks, L)
    XL, g = _run_stack(M, wl, params, toks, L, B)
    assert torch.equal(XL.view(torch.int16), XL_ref.view(torch.int16)), "X_L"
    assert torch.equal(g["dX0"], ref[0]["dX"]), "dX0"
    for l in range(L):
        assert torch.equal(g["dW"][l], ref[l]["dW"]), f"dW[{l}]"
        assert torch.equal(g["dbias"][l], ref[l]["db"]), f"db[{l}]"
        assert torch.equal(g["dF"][l], ref[l]["dF"]), f"dF[{l}]"
