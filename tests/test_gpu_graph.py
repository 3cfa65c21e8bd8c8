"""A layer step (mhc_fwd_pre -> mhc_post_res -> mhc_post_res_bwd -> mhc_bwd_pre) captured
as a HIP graph: every replay, with eager work of the program and synchronisations
between replays, gives bitwise the outputs of the eager step (the kernels are
deterministic and none of the step's launches is a memset).  The same for the
steady-state stack step through mhc_post_res_fwd_pre."""
import numpy as np
import pytest

from manifold_constrained_residuals_amd import inputs as I
from tests._util import to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def M():
    from manifold_constrained_residuals_amd import mhc
    assert torch.cuda.is_available()
    return mhc


def _buffers(M, wl, X):
    T, n, C, K = wl.T, wl.n, wl.C, wl.K
    f32 = lambda *sh: torch.empty(sh, dtype=torch.float32, device="cuda")
    return dict(
        fo=dict(z=f32(T, K), rms=f32(T), H_pre=f32(T, n), H_post=f32(T, n), H_res=f32(T, n, n),
                u=torch.empty((T, C), dtype=X.dtype, device="cuda")),
        Xo=torch.empty_like(X),
        po=dict(dF=f32(T, C), dH_res=f32(T, n, n), dH_post=f32(T, n), dH_pre=f32(T, n)),
        bo=dict(dX=f32(T, n, C), dW=f32(n * C, K), dbias=f32(K), dz=f32(T, K)),
        wsf=M.workspace(M.MHC_OP_FWD_PRE, T, n, C, M._dt(X), "cuda"),
        wsb=M.workspace(M.MHC_OP_BWD_PRE, T, n, C, M._dt(X), "cuda"))


def _step(M, wl, d, p, b):
    fo, po, bo = b["fo"], b["po"], b["bo"]
    M.mhc_fwd_pre(d["X"], p["gamma"], wl.eps, p["W"], p["bias"], p["alpha"], wl.iters,
                  workspace=b["wsf"], **fo)
    M.mhc_post_res(d["X"], d["F"], fo["H_res"], fo["H_post"], X_out=b["Xo"])
    M.mhc_post_res_bwd(d["GX"], d["X"], d["F"], fo["H_res"], fo["H_post"], dF=po["dF"],
                       dH_res=po["dH_res"], dH_post=po["dH_post"])
    M.mhc_bwd_pre(d["GX"], d["GU"], d["X"], p["gamma"], p["W"], p["alpha"], fo["z"], p["bias"],
                  fo["rms"], fo["H_pre"], fo["H_post"], fo["H_res"], po["dH_res"], po["dH_post"],
                  wl.iters, dH_pre=po["dH_pre"], want_dgamma=False, workspace=b["wsb"], **bo)


def _flat(b):
    out = dict(b["fo"])
    out["Xo"] = b["Xo"]
    out.update(b["po"])
    out.update(b["bo"])
    return out


@pytest.mark.parametrize("dtype,n,T,C", [("bf16", 4, 300, 4096), ("f32", 2, 70, 264)])
def test_graph_replays_match_eager(M, dtype, n, T, C):
    print(f"[graph] {dtype} n={n} T={T} C={C}", flush=True)
    wl = I.Workload("g", T=T, n=n, C=C, dtype=dtype, seed=5, alpha=1 / np.sqrt(n * C), backward=True)
    pr = I.layer_params(wl)
    p = dict(gamma=torch.from_numpy(pr["gamma"]).cuda(), W=torch.from_numpy(pr["W"]).cuda(),
             bias=torch.from_numpy(pr["bias"]).cuda(), alpha=pr["alpha"])
    d = {k: to_dev(v, torch) for k, v in I.layer_tokens(wl).items()}
    ref = _buffers(M, wl, d["X"])
    _step(M, wl, d, p, ref)
    torch.cuda.synchronize()
    ref_out = {k: v.clone() for k, v in _flat(ref).items()}

    cap = _buffers(M, wl, d["X"])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _step(M, wl, d, p, cap)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for t in _flat(cap).values():
        t.zero_()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _step(M, wl, d, p, cap)
    for rep in range(3):
        for t in _flat(cap).values():            # stale results must be overwritten
            t.fill_(float("nan")) if t.dtype.is_floating_point else t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _flat(cap)
        for k, v in ref_out.items():
            assert torch.equal(got[k].view(torch.int16) if got[k].dtype == torch.bfloat16 else got[k],
                               v.view(torch.int16) if v.dtype == torch.bfloat16 else v), (rep, k)
        _step(M, wl, d, p, ref)                   # eager work between replays
        torch.cuda.synchronize()
    del g


def test_graph_replays_fused_steady_step(M):
    """The steady-state layer step of a stack -- mhc_post_res_fwd_pre (the previous
    layer's post + residual pass and this layer's read side) then the backward on the X
    it formed -- captured and replayed three times, eager work between replays: every
    replay bitwise the eager step."""
    T, C = 300, 4096
    wl = I.Workload("gs", T=T, n=4, C=C, dtype="bf16", seed=9, alpha=1 / np.sqrt(4 * C),
                    backward=True)
    pr = I.layer_params(wl)
    p = dict(gamma=torch.from_numpy(pr["gamma"]).cuda(), W=torch.from_numpy(pr["W"]).cuda(),
             bias=torch.from_numpy(pr["bias"]).cuda(), alpha=pr["alpha"])
    d = {k: to_dev(v, torch) for k, v in I.layer_tokens(wl).items()}
    prev = M.mhc_fwd_pre(d["X"], p["gamma"], wl.eps, p["W"], p["bias"], p["alpha"], wl.iters)
    torch.cuda.synchronize()

    def step(b):
        fo, po, bo = b["fo"], b["po"], b["bo"]
        M.mhc_post_res_fwd_pre(d["X"], d["F"], prev["H_res"], prev["H_post"], p["gamma"], wl.eps,
                               p["W"], p["bias"], p["alpha"], wl.iters, X_out=b["Xo"], z=fo["z"],
                               rms=fo["rms"], H_pre=fo["H_pre"], H_post_next=fo["H_post"],
                               H_res_next=fo["H_res"], u=fo["u"], workspace=b["wsf"])
        M.mhc_post_res_bwd(d["GX"], b["Xo"], d["F"], fo["H_res"], fo["H_post"], dF=po["dF"],
                           dH_res=po["dH_res"], dH_post=po["dH_post"])
        M.mhc_bwd_pre(d["GX"], d["GU"], b["Xo"], p["gamma"], p["W"], p["alpha"], fo["z"],
                      p["bias"], fo["rms"], fo["H_pre"], fo["H_post"], fo["H_res"], po["dH_res"],
                      po["dH_post"], wl.iters, dH_pre=po["dH_pre"], want_dgamma=False,
                      workspace=b["wsb"], **bo)

    ref = _buffers(M, wl, d["X"])
    step(ref)
    torch.cuda.synchronize()
    ref_out = {k: v.clone() for k, v in _flat(ref).items()}
    cap = _buffers(M, wl, d["X"])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(cap)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(cap)
    for rep in range(3):
        for t in _flat(cap).values():
            t.fill_(float("nan")) if t.dtype.is_floating_point else t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _flat(cap)
        for k, v in ref_out.items():
            assert torch.equal(got[k].view(torch.int16) if got[k].dtype == torch.bfloat16 else got[k],
                               v.view(torch.int16) if v.dtype == torch.bfloat16 else v), (rep, k)
        step(ref)
        torch.cuda.synchronize()
    del g
