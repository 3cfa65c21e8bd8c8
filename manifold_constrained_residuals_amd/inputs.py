"""Seeded synthetic inputs for the mHC layer operator.

This module holds no arithmetic of the method: it only draws random tensors,
rounds them to their storage dtype and describes the five workloads.  It is the
one piece shared by the HIP path's tests/benchmark and by the fp64 oracle, so
that both sides see bit-identical inputs.

Draws use NumPy's PCG64 seeded with ``[seed, tensor_id, chunk]`` so that any
1024-token chunk can be regenerated alone (large workloads stream; sampled
parity checks regenerate only the chunks they need).  Values are drawn in fp32
and, for bf16 workloads, rounded to nearest-even bf16 once.

The pages give no operator-level shapes (their models are 3B/9B/27B MoE training
runs); the workloads below stand in for those activations: N(0,1) activations,
a projection W ~ N(0, 0.02), biases N(0, 0.1) with +3 on the H_res diagonal so
the residual mixer starts near the identity, RMSNorm scale ~ U(0.9, 1.1),
eps = 1e-6.
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import math
import os
from typing import Optional

import numpy as np

CHUNK = 1024

# tensor ids of the seeded streams
TID_X, TID_F, TID_W, TID_B, TID_GAMMA, TID_GX, TID_GU, TID_ZRES = range(8)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    n: int
    C: int
    dtype: str            # "f32" or "bf16" storage of X, F, u, X', dX', du
    seed: int
    alpha: float          # fixed logit scale (same for pre, post, res)
    backward: bool
    zres_split: Optional[tuple] = None   # (std even tokens, std odd tokens) injected res logits
    layers: int = 1
    f_scale: float = 1.0
    eps: float = 1e-6
    iters: int = 20

    @property
    def N(self):
        return self.n * self.C

    @property
    def K(self):
        return self.n * self.n + 2 * self.n


def _alpha_scaled(n, C):
    return 1.0 / math.sqrt(n * C)


WORKLOADS = {
    "tiny_f32_fwd": Workload("tiny_f32_fwd", T=64, n=4, C=256, dtype="f32", seed=0,
                             alpha=1.0, backward=False),
    "layer_bf16_fwd": Workload("layer_bf16_fwd", T=16384, n=4, C=4096, dtype="bf16", seed=1,
                               alpha=_alpha_scaled(4, 4096), backward=False),
    "layer_bf16_fwdbwd": Workload("layer_bf16_fwdbwd", T=16384, n=4, C=4096, dtype="bf16",
                                  seed=2, alpha=_alpha_scaled(4, 4096), backward=True),
    "stress_bf16_fwdbwd": Workload("stress_bf16_fwdbwd", T=65536, n=4, C=7168, dtype="bf16",
                                   seed=3, alpha=_alpha_scaled(4, 7168), backward=True,
                                   zres_split=(4.0, 0.01)),
    "depth_f32_fwd": Workload("depth_f32_fwd", T=4096, n=4, C=2048, dtype="f32", seed=4,
                              alpha=1.0, backward=False, layers=60, f_scale=0.1),
}


def workload(name: str, **over) -> Workload:
    return dataclasses.replace(WORKLOADS[name], **over)


# ------------------------------------------------------------------ rounding
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern (uint16), round to nearest even (inputs are finite)."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rb = ((b >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((b + rb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def store(a32: np.ndarray, dtype: str) -> np.ndarray:
    """Round an fp32 draw to the storage dtype: fp32 array, or uint16 bf16 bits."""
    return f32_to_bf16_bits(a32) if dtype == "bf16" else np.ascontiguousarray(a32, np.float32)


def widen(a: np.ndarray) -> np.ndarray:
    """Storage array (fp32, or uint16 bf16 bits) -> exact fp32 values."""
    return bf16_bits_to_f32(a) if a.dtype == np.uint16 else np.asarray(a, np.float32)


# ------------------------------------------------------------------ draws
def _rng(seed, tid, chunk):
    return np.random.default_rng([int(seed), int(tid), int(chunk)])


_POOL = None


def _pool():
    global _POOL
    if _POOL is None:
        workers = max(1, min(16, len(os.sched_getaffinity(0))))
        _POOL = concurrent.futures.ThreadPoolExecutor(max_workers=workers)
    return _POOL


def token_normal(seed, tid, t0, t1, row_shape, std=1.0, dtype="f32"):
    """N(0, std^2) rows for tokens [t0, t1), chunk-seeded, drawn in fp32 and
    returned in storage dtype (fp32, or uint16 bf16 bits).  Chunks are drawn and
    rounded in parallel threads (each chunk has its own generator, so the result
    does not depend on the thread count)."""
    row_shape = tuple(row_shape)
    out = np.empty((t1 - t0,) + row_shape, np.uint16 if dtype == "bf16" else np.float32)

    def one(c):
        a, b = c * CHUNK, (c + 1) * CHUNK
        blk = _rng(seed, tid, c).standard_normal((CHUNK,) + row_shape, dtype=np.float32)
        lo, hi = max(a, t0), min(b, t1)
        v = blk[lo - a:hi - a]
        if std != 1.0:
            v *= np.float32(std)
        out[lo - t0:hi - t0] = store(v, dtype)

    chunks = range(t0 // CHUNK, (t1 + CHUNK - 1) // CHUNK)
    if len(chunks) == 1:
        one(chunks[0])
    else:
        list(_pool().map(one, chunks))
    return out


def layer_params(wl: Workload, layer: int = 0):
    """W [N,K] ~ N(0,0.02), bias [K] ~ N(0,0.1) (+3 on the H_res diagonal),
    gamma [N] ~ U(0.9,1.1), alpha [3]; all fp32."""
    off = 100 * layer
    n, N, K = wl.n, wl.N, wl.K
    W = (_rng(wl.seed, off + TID_W, 0).standard_normal((N, K), dtype=np.float32)
         * np.float32(0.02))
    b = _rng(wl.seed, off + TID_B, 0).standard_normal(K, dtype=np.float32) * np.float32(0.1)
    for i in range(n):
        b[2 * n + i * n + i] += np.float32(3.0)
    gamma = _rng(wl.seed, off + TID_GAMMA, 0).uniform(0.9, 1.1, N).astype(np.float32)
    alpha = np.full(3, wl.alpha, np.float32)
    return dict(W=np.ascontiguousarray(W), bias=b, gamma=gamma, alpha=alpha)


def layer_tokens(wl: Workload, t0: int = 0, t1: Optional[int] = None, layer: int = 0,
                 which=("X", "F", "GX", "GU", "ZRES")):
    """Token tensors for [t0, t1) in storage dtype (bf16 as uint16 bits).
    X [T,n,C]; F [T,C] (F's output); GX = dX' [T,n,C]; GU = du [T,C];
    ZRES [T,n*n] fp32 (only for workloads with injected res logits)."""
    t1 = wl.T if t1 is None else t1
    off = 100 * layer
    out = {}
    if "X" in which:
        out["X"] = token_normal(wl.seed, off + TID_X, t0, t1, (wl.n, wl.C), dtype=wl.dtype)
    if "F" in which:
        out["F"] = token_normal(wl.seed, off + TID_F, t0, t1, (wl.C,), std=wl.f_scale,
                                dtype=wl.dtype)
    if wl.backward and "GX" in which:
        out["GX"] = token_normal(wl.seed, off + TID_GX, t0, t1, (wl.n, wl.C), dtype=wl.dtype)
    if wl.backward and "GU" in which:
        out["GU"] = token_normal(wl.seed, off + TID_GU, t0, t1, (wl.C,), dtype=wl.dtype)
    if wl.zres_split is not None and "ZRES" in which:
        z = token_normal(wl.seed, off + TID_ZRES, t0, t1, (wl.n * wl.n,))
        even = (np.arange(t0, t1) % 2) == 0
        z[even] *= np.float32(wl.zres_split[0])
        z[~even] *= np.float32(wl.zres_split[1])
        out["ZRES"] = z
    return out
