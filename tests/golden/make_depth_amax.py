"""Writes depth_amax.txt: the per-depth Amax gain of the composite residual mixer for
the 60-layer depth workload (T = 4096, n = 4, C = 2048, fp32 inputs, seed 4), in the
fp64 oracle, for two stacks that share W_l, b_l, gamma_l, F_l and X_0:

  mhc            H_res = Sinkhorn-Knopp(exp z_res), 20 iterations (the method);
  unconstrained  H_res = the raw res logit block z_res (plain hyper-connections).

Amax at depth l = max over tokens of max(max row abs-sum, max column abs-sum) of
P_l = H_res^(l) ... H_res^(1) (chatgpz.de, "Warum Hyperverbindungen instabil werden":
the composite mapping's gain from its maximal row and column sums).  Each stack runs
on its own trajectory of X.  Only the oracle and the seeded input generator are used.

    python tests/golden/make_depth_amax.py
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from manifold_constrained_residuals_amd import inputs as I  # noqa: E402

OUT = os.path.join(HERE, "depth_amax.txt")


def run_stacks(layers=None):
    """Per-depth (log10 Amax of the unconstrained stack, Amax of the mHC stack)."""
    wl = I.workload("depth_f32_fwd")
    L = wl.layers if layers is None else layers
    n = wl.n
    X0 = I.widen(I.layer_tokens(wl, layer=0, which=("X",))["X"]).astype(np.float64)
    Xu, Xm = X0.copy(), X0.copy()
    Pu = np.broadcast_to(np.eye(n), (wl.T, n, n)).copy()
    Pm = Pu.copy()
    rows = []
    for layer in range(L):
        p = I.layer_params(wl, layer)
        F = I.widen(I.layer_tokens(wl, layer=layer, which=("F",))["F"])
        ou = oracle.forward_unconstrained(Xu, F, p["gamma"], wl.eps, p["W"], p["bias"], p["alpha"])
        gr, gc = oracle.composite(ou["Hres"], Pu)
        amax_u = max(gr.max(), gc.max())
        om = oracle.forward(Xm, F, p["gamma"], wl.eps, p["W"], p["bias"], p["alpha"], wl.iters)
        gr, gc = oracle.composite(om["Hres"], Pm)
        amax_m = max(gr.max(), gc.max())
        Xu, Xm = ou["Xout"], om["Xout"]
        rows.append((layer + 1, float(np.log10(amax_u)), float(amax_m)))
    return rows


def main():
    rows = run_stacks()
    with open(OUT, "w") as f:
        f.write("# depth_f32_fwd (T=4096, n=4, C=2048, seed 4), fp64 oracle; written by "
                "make_depth_amax.py\n")
        f.write("# depth  log10_amax_unconstrained  amax_mhc\n")
        for d, lu, am in rows:
            f.write(f"{d:3d} {lu:.12f} {am:.15f}\n")
    print(f"wrote {OUT}")


if __name__ == "__main__":
    main()
