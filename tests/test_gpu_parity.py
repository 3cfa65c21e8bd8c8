"""GPU parity of every libmhc entry point against the fp64 oracle, element by
element, on seeded inputs small enough for the oracle yet spanning several
tiles and ragged tails (tokens and channels).  Tolerance: inf-norm relative
error per tensor, 1e-5 for fp32 outputs and 1e-2 for bf16 outputs; bf16 outputs
are also checked to be within one bf16 rounding of the exact value."""
import numpy as np
import pytest

from manifold_constrained_residuals_amd import inputs as I
from tests._util import TOL, assert_close, proj_ref, to_dev, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

CASES = [
    # (dtype, n, T, C, alpha)
    ("bf16", 4, 300, 4096, 1 / 128),
    ("bf16", 4, 77, 264, 1 / np.sqrt(4 * 264)),
    ("bf16", 4, 45, 384, 1 / np.sqrt(4 * 384)),
    ("bf16", 4, 1, 1024, 1 / 64),
    ("bf16", 4, 17, 640, 1 / np.sqrt(4 * 640)),
    ("f32", 4, 64, 256, 1.0),
    ("f32", 4, 19, 1032, 1.0),
    ("f32", 1, 50, 40, 1.0),
    ("bf16", 1, 33, 64, 0.3),
    ("f32", 2, 70, 264, 1.0),
    ("bf16", 2, 45, 512, 0.2),
    ("f32", 8, 33, 128, 1.0),
    ("bf16", 8, 20, 64, 0.5),
    # coefficient-backward work chunks that cross slices, and slices with fewer pieces
    # than the partial slots (zero-filled), on a full 256-block grid and on a small one
    ("bf16", 4, 1000, 1280, 1 / np.sqrt(4 * 1280)),
    ("bf16", 4, 100, 384, 1 / np.sqrt(4 * 384)),
    # the stress width: 56 slices, chunks of about two steps, most crossing slices
    ("bf16", 4, 100, 7168, 1 / np.sqrt(4 * 7168)),
]


@pytest.fixture(scope="module")
def M():
    from manifold_constrained_residuals_amd import mhc
    assert torch.cuda.is_available()
    return mhc


def _make(dtype, n, T, C, alpha, seed=11, zsplit=None):
    wl = I.Workload("t", T=T, n=n, C=C, dtype=dtype, seed=seed, alpha=alpha, backward=True,
                    zres_split=zsplit)
    return wl, I.layer_params(wl), I.layer_tokens(wl)


def _oracle(wl, p, tk, zres_in=None):
    import oracle
    X, F = I.widen(tk["X"]), I.widen(tk["F"])
    G, g = I.widen(tk["GX"]), I.widen(tk["GU"])
    f = oracle.forward(X, F, p["gamma"], wl.eps, p["W"], p["bias"], p["alpha"], wl.iters, zres_in)
    b = oracle.backward(X, F, p["gamma"], wl.eps, p["W"], p["bias"], p["alpha"], G, g, f,
                        wl.iters, zres_in, learn_alpha=True)
    return f, b


def _bf16_one_rounding(name, gpu, ref):
    # |gpu - ref| <= half a bf16 ulp of ref (rounding) + fp32 accumulation slack
    slack = 1e-6 * np.abs(ref).max()
    ulp_half = np.ldexp(1.0, np.frexp(np.abs(ref))[1] - 9)
    bad = np.abs(gpu - ref) > ulp_half + slack
    assert not bad.any(), f"{name}: {bad.sum()} elements beyond one bf16 rounding"


def _run_fused(M, wl, p, tk, zres_in=None):
    d = {k: to_dev(v, torch) for k, v in tk.items()}
    gam, W, b = (torch.from_numpy(p[k]).cuda() for k in ("gamma", "W", "bias"))
    zi = torch.from_numpy(zres_in).float().cuda().contiguous() if zres_in is not None else None
    f = M.mhc_fwd_pre(d["X"], gam, wl.eps, W, b, p["alpha"], wl.iters, z_res_in=zi,
                      want_proj=True)
    Xo = M.mhc_post_res(d["X"], d["F"], f["H_res"], f["H_post"])
    pb = M.mhc_post_res_bwd(d["GX"], d["X"], d["F"], f["H_res"], f["H_post"])
    bb = M.mhc_bwd_pre(d["GX"], d["GU"], d["X"], gam, W, p["alpha"], f["z"], b, f["rms"],
                       f["H_pre"], f["H_post"], f["H_res"], pb["dH_res"], pb["dH_post"], wl.iters,
                       z_res_in=zi)
    bb["dalpha"] = M.mhc_alpha_bwd(f["proj"], bb["dz"])
    torch.cuda.synchronize()
    out = {k: to_host(v, torch) for k, v in f.items()}
    out["Xout"] = to_host(Xo, torch)
    out.update({k: to_host(v, torch) for k, v in pb.items() if v is not None})
    out.update({k: to_host(v, torch) for k, v in bb.items() if v is not None})
    return out


def _compare(wl, f, b, g, sd):
    tol, tb = TOL["f32"], TOL[wl.dtype]
    n = wl.n
    assert_close("z", g["z"], f["z"], tol)
    assert_close("rms", g["rms"], f["r"], tol)
    assert_close("H_pre", g["H_pre"], f["Hpre"], tol)
    assert_close("H_post", g["H_post"], f["Hpost"], tol)
    assert_close("H_res", g["H_res"], f["Hres"], tol)
    assert_close("u", g["u"], f["u"], tb)
    assert_close("X_out", g["Xout"], f["Xout"], tb)
    if wl.dtype == "bf16":
        _bf16_one_rounding("u", g["u"], f["u"])
        _bf16_one_rounding("X_out", g["Xout"], f["Xout"])
    else:
        assert_close("u(f32)", g["u"], f["u"], tol)
    assert_close("dF", g["dF"], b["dF"], tol)
    assert_close("dH_post", g["dH_post"], b["dHpost"], tol)
    assert_close("dH_res", g["dH_res"], b["dHres"], tol)
    assert_close("dH_pre", g["dH_pre"], b["dHpre"], tol)
    assert_close("dz", g["dz"], b["dz"], tol)
    assert_close("dX", g["dX"], b["dX"], tol)
    assert_close("dW", g["dW"], b["dW"], tol)
    assert_close("dbias", g["dbias"], b["db"], tol)
    assert_close("dgamma", g["dgamma"], b["dgamma"], tol)
    p = I.layer_params(wl)
    assert_close("proj", g["proj"], proj_ref(f["z"], p["bias"], p["alpha"], n), tol)
    assert_close("dalpha", g["dalpha"], b["dalpha"], tol)


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-n{c[1]}-T{c[2]}-C{c[3]}" for c in CASES])
def test_fused_layer_matches_oracle(M, case):
    wl, p, tk = _make(*case)
    print(f"[parity fused] {case}", flush=True)
    f, b = _oracle(wl, p, tk)
    g = _run_fused(M, wl, p, tk)
    _compare(wl, f, b, g, case)


def _run_split(M, wl, p, tk):
    """The layer with the split backward: mhc_post_res_bwd_pre -> mhc_bwd_pre_from_dh."""
    d = {k: to_dev(v, torch) for k, v in tk.items()}
    gam, W, b = (torch.from_numpy(p[k]).cuda() for k in ("gamma", "W", "bias"))
    f = M.mhc_fwd_pre(d["X"], gam, wl.eps, W, b, p["alpha"], wl.iters, want_proj=True)
    Xo = M.mhc_post_res(d["X"], d["F"], f["H_res"], f["H_post"])
    pb = M.mhc_post_res_bwd_pre(d["GX"], d["GU"], d["X"], d["F"], f["H_res"], f["H_post"])
    bb = M.mhc_bwd_pre_from_dh(d["GX"], d["GU"], d["X"], gam, W, p["alpha"], f["z"], b, f["rms"],
                               f["H_pre"], f["H_post"], f["H_res"], pb["dH_pre"], pb["dH_res"],
                               pb["dH_post"], wl.iters)
    bb["dalpha"] = M.mhc_alpha_bwd(f["proj"], bb["dz"])
    torch.cuda.synchronize()
    out = {k: to_host(v, torch) for k, v in f.items()}
    out["Xout"] = to_host(Xo, torch)
    out.update({k: to_host(v, torch) for k, v in pb.items() if v is not None})
    out.update({k: to_host(v, torch) for k, v in bb.items() if v is not None})
    return out


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-n{c[1]}-T{c[2]}-C{c[3]}" for c in CASES])
def test_split_backward_matches_oracle_and_fused(M, case):
    """The split backward against the oracle, and bitwise against mhc_post_res_bwd +
    mhc_bwd_pre (the same reductions in the same order)."""
    wl, p, tk = _make(*case, seed=31)
    print(f"[parity split] {case}", flush=True)
    f, b = _oracle(wl, p, tk)
    g = _run_split(M, wl, p, tk)
    _compare(wl, f, b, g, case)
    h = _run_fused(M, wl, p, tk)
    for k in ("dF", "dH_res", "dH_post", "dH_pre", "dz", "dX", "dW", "dbias", "dgamma", "dalpha"):
        assert np.array_equal(np.asarray(g[k]), np.asarray(h[k])), f"{k} differs from the fused pair"


UNFUSED = CASES[:7] + CASES[9:]


@pytest.mark.parametrize("case", UNFUSED, ids=[f"{c[0]}-n{c[1]}-T{c[2]}-C{c[3]}" for c in UNFUSED])
def test_unfused_calls_match_oracle(M, case):
    import oracle
    wl, p, tk = _make(*case, seed=23)
    print(f"[parity unfused] {case}", flush=True)
    f, b = _oracle(wl, p, tk)
    d = {k: to_dev(v, torch) for k, v in tk.items()}
    gam, W, bias = (torch.from_numpy(p[k]).cuda() for k in ("gamma", "W", "bias"))
    n, tol = wl.n, TOL["f32"]
    c = M.mhc_coeffs(d["X"], gam, wl.eps, W, bias, p["alpha"], want_proj=True)
    Hres = M.mhc_sinkhorn(c["z"][:, 2 * n:], n, wl.iters)
    u = M.mhc_pre(d["X"], c["H_pre"])
    Xo = M.mhc_post_res(d["X"], d["F"], Hres, c["H_post"])
    pb = M.mhc_post_res_bwd(d["GX"], d["X"], d["F"], Hres, c["H_post"], want_dx=True)
    dX = pb["dX"]
    pr = M.mhc_pre_bwd(d["GU"], d["X"], c["H_pre"], dX=dX)
    dzr = M.mhc_sinkhorn_bwd(c["z"][:, 2 * n:], pb["dH_res"], n, wl.iters)
    cb = M.mhc_coeffs_bwd(d["X"], gam, W, p["alpha"], c["z"], bias, c["rms"], c["H_pre"],
                          c["H_post"], pr["dH_pre"], pb["dH_post"], dzr, dX=dX)
    da = M.mhc_alpha_bwd(c["proj"], cb["dz"])
    torch.cuda.synchronize()
    h = lambda t: to_host(t, torch)
    assert_close("z", h(c["z"]), f["z"], tol)
    assert_close("H_res", h(Hres), f["Hres"], tol)
    assert_close("u", h(u), f["u"], TOL[wl.dtype])
    assert_close("X_out", h(Xo), f["Xout"], TOL[wl.dtype])
    assert_close("dz_res", h(dzr), b["dz"][:, 2 * n:], tol)
    assert_close("dz", h(cb["dz"]), b["dz"], tol)
    assert_close("dX", h(dX), b["dX"], tol)
    assert_close("dW", h(cb["dW"]), b["dW"], tol)
    assert_close("dbias", h(cb["dbias"]), b["db"], tol)
    assert_close("dgamma", h(cb["dgamma"]), b["dgamma"], tol)
    assert_close("proj", h(c["proj"]), proj_ref(f["z"], p["bias"], p["alpha"], n), tol)
    assert_close("dalpha", h(da), b["dalpha"], tol)


def test_injected_res_logits_match_oracle(M):
    # sharp (std 4) and near-uniform (std 0.01) res logits on alternating tokens
    wl, p, tk = _make("bf16", 4, 130, 512, 1 / np.sqrt(2048), seed=31, zsplit=(4.0, 0.01))
    print("[parity injected]", flush=True)
    zin = tk.pop("ZRES")
    f, b = _oracle(wl, p, tk, zres_in=zin)
    g = _run_fused(M, wl, p, tk, zres_in=zin)
    _compare(wl, f, b, g, "injected")


@pytest.mark.parametrize("n", [4, 1, 2, 8])
@pytest.mark.parametrize("iters", [1, 7, 20, 21, 200])
def test_sinkhorn_fwd_bwd_iters(M, n, iters):
    import oracle
    rng = np.random.default_rng(iters * 7 + n)
    T = 193
    scales = np.where(np.arange(T) % 3 == 0, 4.0, np.where(np.arange(T) % 3 == 1, 1.0, 0.01))
    z = (rng.normal(size=(T, n * n)) * scales[:, None]).astype(np.float32)
    dH = rng.normal(size=(T, n, n)).astype(np.float32)
    zt, dHt = torch.from_numpy(z).cuda(), torch.from_numpy(dH).cuda()
    H = M.mhc_sinkhorn(zt, n, iters)
    dz = M.mhc_sinkhorn_bwd(zt, dHt, n, iters)
    torch.cuda.synchronize()
    Hr = oracle.sinkhorn(z, n, iters)
    dzr = oracle.sinkhorn_bwd(z, dH, n, iters)
    assert_close("H_res", to_host(H, torch), Hr, 1e-5)
    if n > 1:
        # Per token as well (gradients of sharp tokens dwarf the others).  A saturated
        # token's gradient is a difference of terms of the size of dH, so fp32
        # leaves an absolute error that scales with |dH|, not with the (tiny) result:
        # the per-token error is measured against max(|dz_t|, 1e-2 |dH_t|).
        g = to_host(dz, torch)
        for t in range(T):
            tol = 1e-4 if scales[t] == 4.0 else 1e-5
            den = max(np.abs(dzr[t]).max(), 1e-2 * np.abs(dH[t]).max())
            err = np.abs(g[t] - dzr[t]).max() / den
            assert err <= tol, f"dz_res[{t}]: {err:.3e} > {tol:.0e}"
        assert_close("dz_res", g, dzr, 1e-5)
    else:
        assert np.all(to_host(dz, torch) == 0.0)


def test_composite_matches_oracle(M):
    import oracle
    rng = np.random.default_rng(3)
    T, n = 300, 4
    P = np.broadcast_to(np.eye(n), (T, n, n)).astype(np.float64).copy()
    Pt = torch.from_numpy(P.astype(np.float32)).cuda()
    for layer in range(10):
        H = oracle.sinkhorn(rng.normal(size=(T, n * n)), n).astype(np.float32)
        gr, gc = M.mhc_composite(torch.from_numpy(H).cuda(), Pt)
        r, c = oracle.composite(H.astype(np.float64), P)
    torch.cuda.synchronize()
    assert_close("P", to_host(Pt, torch), P, 1e-5)
    assert_close("gain_row", to_host(gr, torch), r, 1e-5)
    assert_close("gain_col", to_host(gc, torch), c, 1e-5)


def test_n1_unit_maps_are_standard_residual_bitwise(M):
    rng = np.random.default_rng(4)
    T, C = 40, 264
    x = torch.from_numpy(rng.normal(size=(T, 1, C)).astype(np.float32)).cuda()
    F = torch.from_numpy(rng.normal(size=(T, C)).astype(np.float32)).cuda()
    one = torch.ones((T, 1), device="cuda")
    u = M.mhc_pre(x, one)
    Xo = M.mhc_post_res(x, F, torch.ones((T, 1, 1), device="cuda"), one)
    torch.cuda.synchronize()
    assert torch.equal(u, x[:, 0])
    assert torch.equal(Xo[:, 0], x[:, 0] + F)


def test_bf16_output_rounding_is_rne(M):
    # u = h x with x bf16 and h = 1 + 2^-9: the exact fp32 product needs rounding;
    # the kernel must round to nearest even, as the input generator does
    rng = np.random.default_rng(5)
    T, C = 64, 512
    xb = I.f32_to_bf16_bits(rng.normal(size=(T, 1, C)).astype(np.float32))
    h = np.float32(1 + 2.0 ** -9)
    X = to_dev(xb, torch)
    u = M.mhc_pre(X, torch.full((T, 1), float(h), device="cuda"))
    torch.cuda.synchronize()
    want = I.f32_to_bf16_bits((I.bf16_bits_to_f32(xb)[:, 0] * h).astype(np.float32))
    got = u.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, want)


def test_gpu_invariants_and_determinism(M):
    wl, p, tk = _make("bf16", 4, 256, 1024, 1 / 64, seed=41)
    g1 = _run_fused(M, wl, p, tk)
    g2 = _run_fused(M, wl, p, tk)
    for k in ("dW", "dbias", "dgamma", "dalpha", "dX", "z", "H_res"):
        assert np.array_equal(g1[k], g2[k]), k
    H = g1["H_res"]
    assert (H >= 0).all()
    assert np.abs(H.sum(1) - 1).max() < 1e-6          # column sums after the last column step
    assert np.abs(H.sum(2) - 1).max() < 1e-2          # rows near 1
    dzr = g1["dz"][:, 8:].reshape(-1, 4, 4)
    assert np.abs(dzr.sum(2)).max() <= 1e-5 * np.abs(dzr).max()
    X = I.widen(tk["X"]).astype(np.float64); F = I.widen(tk["F"]).astype(np.float64)
    # feature mass: sum_i X'_i = sum_j colsum_j(H_res) X_j + (sum_i H_post_i) F
    lhs = g1["Xout"].sum(1)
    rhs = np.einsum("tj,tjc->tc", H.sum(1), X) + g1["H_post"].sum(1)[:, None] * F
    assert np.abs(lhs - rhs).max() <= 0.02 * np.abs(rhs).max()
