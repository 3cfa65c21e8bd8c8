"""Benchmark of the mHC layer forward + backward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

One step = one pass of the whole layer over one batch of synthetic tokens, in the
order a layer of a network runs it:
    mhc_fwd_pre -> [F] -> mhc_post_res -> mhc_post_res_bwd -> [F_bwd] -> mhc_bwd_pre
The sublayer F and its backward are the caller's; their tensors (F's output, and du,
the gradient F_bwd returns from dF) are given.  du is read only after the call that
writes dF, since a real sublayer forms du from dF.  Inputs are resident in HBM before
the timed region.  Prints one JSON line.

Metric: tokens/s of the layer fwd+bwd at n = 4, C = 4096, bf16 storage, with the
fraction of the HBM peak that the algorithmic traffic implies.  Algorithmic bytes
per token and call (s = storage bytes, fp32 gradients):
  fwd_pre            s*C*(n+1)               read X, write u
  post_res           s*C*(2n+1)              read X, F, write X'
  post_res_bwd       s*C*(2n+1) + 4*C        read dX', X, F, write dF
  bwd_pre            s*C*(2n+1) + 4*n*C      read du, X, dX', write dX
Each tensor counts once per call.  mhc_bwd_pre reads X twice: the read map's gradient
dH_pre = <du, X_k> is a reduction over all of a token's channels that the coefficient
backward's dX needs first, so its HBM bytes exceed its algorithmic ones.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0

# The timed step's calls in order, with what each reads and writes among the tensors
# that carry the layer's data dependencies; du (written by the caller's sublayer
# backward from dF) may only be read after the call that writes dF.
STEP = (
    ("mhc_fwd_pre", ("X",), ("z", "H", "u")),
    ("mhc_post_res", ("X", "F", "H"), ("X_out",)),
    ("mhc_post_res_bwd", ("dX_out", "X", "F", "H"), ("dF", "dH_res", "dH_post")),
    ("mhc_bwd_pre", ("dX_out", "du", "X", "z", "H", "dH_res", "dH_post"),
     ("dX", "dW", "dbias", "dz", "dH_pre")),
)


def algo_bytes_per_token(n, C, s):
    return {
        "mhc_fwd_pre": s * C * (n + 1),
        "mhc_post_res": s * C * (2 * n + 1),
        "mhc_post_res_bwd": s * C * (2 * n + 1) + 4 * C,
        "mhc_bwd_pre": s * C * (2 * n + 1) + 4 * n * C,
    }


def fused_algo_bytes_per_token(n, C, s):
    """mhc_post_res_fwd_pre (a previous layer's post + residual pass and this layer's read
    side in one call): read X_prev, F, write X, u."""
    return {"mhc_post_res_fwd_pre": s * C * (2 * n + 2)}


def step_bytes_per_token(n, C, s):
    """Algorithmic bytes of one layer step per token: the calls' sum."""
    return sum(algo_bytes_per_token(n, C, s).values())


def _traffic(workload, entry):
    """HBM bytes per launch of one pass from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE, copy-calibrated), or None when there is none for
    this workload or the kernel sources changed since it was taken."""
    from manifold_constrained_residuals_amd import profiling
    t = profiling.load_traffic(os.path.join(ROOT, "profiles", f"{workload}_traffic.json"))
    if t is None or entry not in t["passes"]:
        return None
    return t["passes"][entry]["hbm_bytes"]


def _gen_device(wl, torch):
    """Seeded synthetic inputs (chunked generator), moved to the GPU."""
    from manifold_constrained_residuals_amd import inputs as I
    dev = "cuda"
    p = I.layer_params(wl)
    out = {k: torch.from_numpy(p[k]).to(dev) for k in ("gamma", "W", "bias")}
    out["alpha"] = p["alpha"]
    step = 2048
    for key, shape in (("X", (wl.n, wl.C)), ("F", (wl.C,)), ("GX", (wl.n, wl.C)), ("GU", (wl.C,))):
        tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
        buf = torch.empty((wl.T,) + shape, dtype=tdt, device=dev)
        for t0 in range(0, wl.T, step):
            t1 = min(wl.T, t0 + step)
            a = I.layer_tokens(wl, t0, t1, which=(key,))[key]
            h = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if a.dtype == np.uint16 \
                else torch.from_numpy(a)
            buf[t0:t1].copy_(h)
        out[key] = buf
    return out


def _time_steps(torch, calls, stream, steps, warmup):
    """Warm up, then time `steps` steps of the call sequence with HIP events recorded
    on the stream the kernels run on: per-call and per-step averages (ms)."""
    for _ in range(warmup):
        for _, c in calls:
            c()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)]
          for _ in range(steps)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for k in range(steps):
        ev[k][0].record(stream)
        for j, (_, c) in enumerate(calls):
            c()
            ev[k][j + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    per_call = {name: 0.0 for name, _ in calls}
    step_ms = []
    for k in range(steps):
        for j, (name, _) in enumerate(calls):
            per_call[name] += ev[k][j].elapsed_time(ev[k][j + 1])
        step_ms.append(ev[k][0].elapsed_time(ev[k][-1]))
    return {k: v / steps for k, v in per_call.items()}, step_ms, wall


def _graph_replay(torch, calls, steps, warmup):
    """The same step (same kernels, buffers and workspaces) captured once as a HIP
    graph and replayed; per-step time from HIP events around each replay."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _, c in calls:
            c()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _, c in calls:
            c()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(st)
    for k in range(steps):
        g.replay()
        ev[k + 1].record(st)
    torch.cuda.synchronize()
    ms = float(np.mean([ev[k].elapsed_time(ev[k + 1]) for k in range(steps)]))
    del g
    return ms


def _steady_state(torch, mhc, wl, d, fo, po, bo, wsb, stream, args):
    """One layer of a stack in steady state: the previous layer's post + residual pass
    and this layer's read side in one call (mhc_post_res_fwd_pre: X_{l-1} and F read
    once, X_l formed tile by tile and projected as it is formed), then this layer's
    backward on X_l in the headline's order.  X and the maps ping-pong between two sets of
    buffers, so no call reads what it writes."""
    T, n, C = wl.T, wl.n, wl.C
    a = d["alpha"]
    XA, XB = torch.empty_like(d["X"]), torch.empty_like(d["X"])
    maps = [dict(fo), {k: (torch.empty_like(v) if v is not None else None) for k, v in fo.items()}]
    wsf = mhc.workspace(mhc.MHC_OP_FWD_PRE, T, n, C, mhc._dt(d["X"]), d["X"].device)
    # prologue: the previous layer's maps (on the input X) and its output X_A
    mhc.mhc_fwd_pre(d["X"], d["gamma"], wl.eps, d["W"], d["bias"], a, wl.iters, **maps[0])
    mhc.mhc_post_res(d["X"], d["F"], maps[0]["H_res"], maps[0]["H_post"], X_out=XA)
    cur = [XA, XB]

    def fused():
        m0, m1 = maps
        mhc.mhc_post_res_fwd_pre(cur[0], d["F"], m0["H_res"], m0["H_post"], d["gamma"], wl.eps,
                                 d["W"], d["bias"], a, wl.iters, X_out=cur[1], z=m1["z"],
                                 rms=m1["rms"], H_pre=m1["H_pre"], H_post_next=m1["H_post"],
                                 H_res_next=m1["H_res"], u=m1["u"], workspace=wsf)

    def bwd_a():
        m1 = maps[1]
        mhc.mhc_post_res_bwd(d["GX"], cur[1], d["F"], m1["H_res"], m1["H_post"], dF=po["dF"],
                             dH_res=po["dH_res"], dH_post=po["dH_post"])

    def bwd_b():
        m1 = maps[1]
        mhc.mhc_bwd_pre(d["GX"], d["GU"], cur[1], d["gamma"], d["W"], a, m1["z"], d["bias"],
                        m1["rms"], m1["H_pre"], m1["H_post"], m1["H_res"], po["dH_res"],
                        po["dH_post"], wl.iters, dH_pre=po["dH_pre"], want_dgamma=False,
                        workspace=wsb, **bo)
        cur.reverse()
        maps.reverse()

    calls = [("mhc_post_res_fwd_pre", fused), ("mhc_post_res_bwd", bwd_a),
             ("mhc_bwd_pre", bwd_b)]
    per_call, step_ms, _ = _time_steps(torch, calls, stream, args.steps, args.warmup)
    ms = float(np.mean(step_ms))
    s = 2 if wl.dtype == "bf16" else 4
    total = step_bytes_per_token(n, C, s) * T
    return {"value": T / (ms * 1e-3), "unit": "tokens/s", "ms_per_step": ms,
            "median_ms": float(np.median(step_ms)),
            "hbm_frac_of_peak": total / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9),
            "per_call_ms": per_call,
            "note": "layer of a stack in steady state: the previous layer's post + residual "
                    "pass and this layer's read side in one call (X_{l-1} and F read once); "
                    "same work per step as the headline sequence, fraction against its "
                    "algorithmic bytes"}


def _block_recompute(torch, mhc, wl, d, stream, args, L=16):
    """A stack of L layers through the stack runner (every layer reuses the headline
    layer's parameters and sublayer tensors), forward then backward: B = 1 keeps every
    layer's X; B = mhc_stack_block_size(L) keeps X every B layers and re-runs the post +
    residual pass of each block in the backward.  Reports time per layer and the X
    buffers alive during the backward for both."""
    T, n, C = wl.T, wl.n, wl.C
    dt = mhc._dt(d["X"])
    layers = [dict(gamma=d["gamma"], W=d["W"], bias=d["bias"], alpha=d["alpha"])] * L
    F, du = [d["F"]] * L, [d["GU"]] * L
    xbytes = d["X"].numel() * d["X"].element_size()
    out = {"layers": L}
    for B in (1, mhc.mhc_stack_block_size(L)):
        nb = (L + B - 1) // B
        X_save = [d["X"]] + [torch.empty_like(d["X"]) for _ in range(nb - 1)]
        XL = torch.empty_like(d["X"])
        ws = torch.empty(mhc.mhc_stack_workspace_size(L, B, T, n, C, dt), dtype=torch.uint8,
                         device=d["X"].device)
        dX0 = torch.empty(d["X"].shape, dtype=torch.float32, device=d["X"].device)
        dW = [torch.empty_like(d["W"]) for _ in range(L)]
        db = [torch.empty_like(d["bias"]) for _ in range(L)]

        def fwd():
            mhc.mhc_stack_forward(d["X"], layers, F, B, wl.eps, wl.iters, X_save=X_save, X_L=XL,
                                  workspace=ws)

        def bwd():
            mhc.mhc_stack_backward(X_save, layers, F, du, d["GX"], B, ws, wl.iters, dX0=dX0, dW=dW,
                                   dbias=db)

        per_call, step_ms, _ = _time_steps(torch, [("forward", fwd), ("backward", bwd)], stream,
                                           max(2, args.steps // 5), 1)
        out[f"B{B}"] = {"block": B, "ms_per_layer": float(np.mean(step_ms)) / L,
                        "forward_ms": per_call["forward"], "backward_ms": per_call["backward"],
                        "x_buffers_in_backward": nb + B - 1,
                        "x_save_bytes": nb * xbytes, "workspace_bytes": ws.numel(),
                        "total_bytes": nb * xbytes + ws.numel()}
        del X_save, XL, ws, dX0, dW, db
        torch.cuda.empty_cache()
    out["note"] = ("stack runner, fwd+bwd per layer; between layers dX goes to the layer below "
                   "in the storage dtype; total_bytes = kept X (X_save, with X0) + workspace")
    return out


def copy_ceiling(torch, reps=10):
    """The box's device-to-device copy rate in this run: 1 GiB read + 1 GiB written per
    copy, HIP events around `reps` copies on the current stream (GB/s counts both)."""
    src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    st = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    torch.cuda.synchronize()
    ev[0].record(st)
    for k in range(reps):
        dst.copy_(src)
        ev[k + 1].record(st)
    torch.cuda.synchronize()
    ms = [ev[k].elapsed_time(ev[k + 1]) for k in range(reps)]
    nbytes = 2 * src.numel() * src.element_size()
    del src, dst
    torch.cuda.empty_cache()
    return {"gbs_median": nbytes / (float(np.median(ms)) * 1e-3) / 1e9,
            "gbs_best": nbytes / (min(ms) * 1e-3) / 1e9,
            "bytes_per_copy": nbytes, "copies": reps,
            "note": "torch device-to-device copy of 1 GiB fp32 (read + write counted)"}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, budget_s=15.0):
    """The fp64 oracle (as it stands) on a bounded token sample of the same
    workload; returns tokens/s and the thread count it used."""
    import oracle
    from manifold_constrained_residuals_amd import inputs as I
    threads = len(os.sched_getaffinity(0))
    os.environ.setdefault("OMP_NUM_THREADS", str(threads))
    p = I.layer_params(wl)
    tot_tok, tot_s, t0 = 0, 0.0, 0
    sample = 256
    while tot_s < budget_s and t0 + sample <= wl.T:
        tk = I.layer_tokens(wl, t0, t0 + sample)
        X, F, G, g = (I.widen(tk[k]) for k in ("X", "F", "GX", "GU"))
        X, F, G, g = (a.astype(np.float64) for a in (X, F, G, g))
        c0 = time.perf_counter()
        f = oracle.forward(X, F, p["gamma"], wl.eps, p["W"], p["bias"], p["alpha"], wl.iters)
        oracle.backward(X, F, p["gamma"], wl.eps, p["W"], p["bias"], p["alpha"], G, g, f, wl.iters)
        tot_s += time.perf_counter() - c0
        tot_tok += sample
        t0 += sample
    return {"value": tot_tok / tot_s, "unit": "tokens/s", "cores": int(os.environ.get("OMP_NUM_THREADS", threads)),
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"{tot_tok} tokens of {wl.name} (T={wl.T}, n={wl.n}, C={wl.C}) in {sample}-token "
                      f"batches, fp64 forward+backward, {tot_s:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="layer_bf16_fwdbwd")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-steady-state", action="store_true",
                    help="skip the steady-state stack-layer and block-recompute measurements "
                         "(profiling runs)")
    ap.add_argument("--steady-only", action="store_true",
                    help="time only the steady-state stack layer and print its line (profiling "
                         "runs of the fused post + residual / read-side call)")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain 1 GiB device-to-device copy (known bytes) so that "
                         "hardware byte counters can be scaled")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only (asked for --gpus {args.gpus}); the operator is "
              "per-token and would shard by tokens across GPUs", file=sys.stderr)
        sys.exit(2)

    import torch
    from manifold_constrained_residuals_amd import inputs as I
    from manifold_constrained_residuals_amd import mhc

    wl = I.workload(args.workload)
    T, n, C = wl.T, wl.n, wl.C
    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")   # 1 GiB
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    s = 2 if wl.dtype == "bf16" else 4
    K = n * n + 2 * n
    d = _gen_device(wl, torch)
    dev = d["X"].device
    f32 = lambda *sh: torch.empty(sh, dtype=torch.float32, device=dev)
    # outputs and workspaces allocated once, outside the timed region
    fo = dict(z=f32(T, K), rms=f32(T), H_pre=f32(T, n), H_post=f32(T, n), H_res=f32(T, n, n),
              u=torch.empty((T, C), dtype=d["X"].dtype, device=dev))
    Xo = torch.empty_like(d["X"])
    po = dict(dF=f32(T, C), dH_res=f32(T, n, n), dH_post=f32(T, n), dH_pre=f32(T, n))
    bo = dict(dX=f32(T, n, C), dW=f32(n * C, K), dbias=f32(K), dz=f32(T, K))
    wsf = mhc.workspace(mhc.MHC_OP_FWD_PRE, T, n, C, mhc._dt(d["X"]), dev)
    wsb = mhc.workspace(mhc.MHC_OP_BWD_PRE, T, n, C, mhc._dt(d["X"]), dev)
    alpha = d["alpha"]

    calls = [
        ("mhc_fwd_pre", lambda: mhc.mhc_fwd_pre(d["X"], d["gamma"], wl.eps, d["W"], d["bias"], alpha,
                                                wl.iters, workspace=wsf, **fo)),
        ("mhc_post_res", lambda: mhc.mhc_post_res(d["X"], d["F"], fo["H_res"], fo["H_post"], X_out=Xo)),
        ("mhc_post_res_bwd", lambda: mhc.mhc_post_res_bwd(d["GX"], d["X"], d["F"], fo["H_res"],
                                                          fo["H_post"], dF=po["dF"],
                                                          dH_res=po["dH_res"],
                                                          dH_post=po["dH_post"])),
        ("mhc_bwd_pre", lambda: mhc.mhc_bwd_pre(
            d["GX"], d["GU"], d["X"], d["gamma"], d["W"], alpha, fo["z"], d["bias"], fo["rms"],
            fo["H_pre"], fo["H_post"], fo["H_res"], po["dH_res"], po["dH_post"], wl.iters,
            dH_pre=po["dH_pre"], want_dgamma=False, workspace=wsb, **bo)),
    ]
    assert [c[0] for c in calls] == [c[0] for c in STEP]
    stream = torch.cuda.current_stream()
    if args.steady_only:
        st = _steady_state(torch, mhc, wl, d, fo, po, bo, wsb, stream, args)
        st.update({"metric": f"steady-state stack layer fwd+bwd tokens/s (n={n}, C={C}, {wl.dtype})",
                   "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                   "higher_is_better": True, "dtype": wl.dtype, "data": "synthetic",
                   "config": {"workload": wl.name, "T": T, "n": n, "C": C, "storage": wl.dtype,
                              "accumulate": "f32", "sinkhorn_iters": wl.iters,
                              "parallelism": "single GPU", "step": "steady_state_layer"}})
        print(json.dumps(st), flush=True)
        return
    ceiling = copy_ceiling(torch)
    per_call, step_ms, wall = _time_steps(torch, calls, stream, args.steps, args.warmup)
    ms = float(np.mean(step_ms))
    tok_s = T / (ms * 1e-3)
    ab = algo_bytes_per_token(n, C, s)
    total_bytes = step_bytes_per_token(n, C, s) * T
    from manifold_constrained_residuals_amd.profiling import PASS_KERNELS
    dom = max(per_call, key=per_call.get)
    dom_gbs = ab[dom] * T / (per_call[dom] * 1e-3) / 1e9
    out = {
        "metric": f"mHC layer fwd+bwd tokens/sec (n={n}, C={C}, {wl.dtype}) and % of HBM peak",
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "T": T, "n": n, "C": C, "storage": wl.dtype,
                   "accumulate": "f32", "sinkhorn_iters": wl.iters, "parallelism": "single GPU"},
        "hbm_frac_of_peak": total_bytes / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9),
        "algorithmic_bytes_per_step": total_bytes,
        "step_ms_stats": {"mean": ms, "median": float(np.median(step_ms)),
                          "min": float(np.min(step_ms)), "p90": float(np.percentile(step_ms, 90))},
        "hbm_copy_ceiling_gbs": ceiling["gbs_median"],
        "hbm_copy_ceiling": ceiling,
        "per_call_ms": per_call,
        "wall_s_timed": wall,
        "roofline": {"bound": "hbm", "kernel": f"{dom}: {', '.join(PASS_KERNELS[dom])}",
                     "achieved": dom_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": dom_gbs / HBM_PEAK_GBS, "traffic": _traffic(wl.name, dom),
                     "algorithmic_bytes_per_launch": ab[dom] * T,
                     "avg_launch_ms": per_call[dom]},
    }
    if not args.no_steady_state:
        out["steady_state_layer"] = _steady_state(torch, mhc, wl, d, fo, po, bo, wsb, stream, args)
    if not args.no_steady_state:
        gms = _graph_replay(torch, calls, args.steps, args.warmup)
        out["graph_replay"] = {"value": T / (gms * 1e-3), "unit": "tokens/s", "ms_per_step": gms,
                               "hbm_frac_of_peak": total_bytes / (gms * 1e-3) / (HBM_PEAK_GBS * 1e9),
                               "note": "the headline step's launches captured once as a HIP graph "
                                       "and replayed (same kernels and buffers, fewer launch gaps)"}
        out["block_recompute"] = _block_recompute(torch, mhc, wl, d, stream, args)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
