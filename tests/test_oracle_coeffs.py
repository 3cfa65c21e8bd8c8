"""Pins of the oracle's coefficient step: RMSNorm of vec(X), projection to
n*n + 2n logits, per-group scale, bias and sigmoid gating (chatgpz.de,
"Systemarbeit und Schulungsaufwand": RMSNorm, projections and gating fused into
the mHC maps; "Vielfaeltig eingeschraenkte Hyperverbindungen" and
staging.reportify.cn "mHC方法原理" note [12]: non-negative pre/post maps).

Closed forms and invariants only: each one fails on a plausible mistake (a
wrong flatten order, a transposed W, a missing 1/r or eps, a wrong group).
"""
import math

import numpy as np
import pytest

import oracle


def _params(n, C, seed=0):
    rng = np.random.default_rng(seed)
    N, K = n * C, n * n + 2 * n
    return dict(gamma=rng.uniform(0.9, 1.1, N), W=rng.normal(0, 0.02, (N, K)),
                bias=rng.normal(0, 0.1, K), alpha=np.array([0.7, 1.3, 0.4]))


def test_rms_closed_form():
    # X constant c: mean(v^2) = c^2, so r = sqrt(c^2 + eps) (RMSNorm over all n*C values)
    n, C, eps = 4, 12, 1e-3
    p = _params(n, C)
    for c in (0.5, 3.0):
        X = np.full((3, n, C), c)
        out = oracle.coeffs(X, p["gamma"], eps, p["W"], p["bias"], p["alpha"])
        np.testing.assert_allclose(out["r"], math.sqrt(c * c + eps), rtol=1e-15)
    # a single non-zero among N values: mean(v^2) = v^2 / N
    X = np.zeros((1, n, C)); X[0, 2, 5] = 2.0
    out = oracle.coeffs(X, p["gamma"], 0.0, p["W"], p["bias"], p["alpha"])
    assert math.isclose(out["r"][0], 2.0 / math.sqrt(n * C), rel_tol=1e-15)


def test_onehot_projection_selects_stream_major_element():
    # W[:, k] = e_{idx_k}: logit k reads the single element v[idx_k] with
    # v = vec(X) stream-major (idx = stream * C + channel).  X entries are +-1, so
    # r = sqrt(1 + eps) exactly and z_k = alpha_g gamma_idx X[s, c] / r + b_k.
    n, C, eps = 4, 8, 1e-6
    N, K = n * C, n * n + 2 * n
    rng = np.random.default_rng(1)
    X = rng.choice([-1.0, 1.0], size=(5, n, C))
    idx = rng.choice(N, size=K, replace=False)
    W = np.zeros((N, K)); W[idx, np.arange(K)] = 1.0
    gamma = rng.uniform(0.9, 1.1, N)
    bias = rng.normal(size=K)
    alpha = np.array([0.5, 2.0, -1.5])
    out = oracle.coeffs(X, gamma, eps, W, bias, alpha)
    r = math.sqrt(1.0 + eps)
    for k in range(K):
        g = 0 if k < n else (1 if k < 2 * n else 2)
        s, c = divmod(int(idx[k]), C)
        want = alpha[g] * gamma[idx[k]] * X[:, s, c] / r + bias[k]
        np.testing.assert_allclose(out["z"][:, k], want, rtol=1e-14, atol=1e-14)


def test_scale_invariance_without_eps():
    n, C = 4, 16
    p = _params(n, C, 2)
    X = np.random.default_rng(2).normal(size=(4, n, C))
    a = oracle.coeffs(X, p["gamma"], 0.0, p["W"], p["bias"], p["alpha"])
    b = oracle.coeffs(37.5 * X, p["gamma"], 0.0, p["W"], p["bias"], p["alpha"])
    np.testing.assert_allclose(a["z"], b["z"], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(37.5 * a["r"], b["r"], rtol=1e-14)


def test_linear_in_W_and_bias_only_offsets():
    n, C = 4, 16
    p = _params(n, C, 3)
    X = np.random.default_rng(3).normal(size=(4, n, C))
    W2 = np.random.default_rng(4).normal(0, 0.05, p["W"].shape)
    f = lambda W, b: oracle.coeffs(X, p["gamma"], 1e-6, W, b, p["alpha"])["z"]
    zero = np.zeros_like(p["bias"])
    np.testing.assert_allclose(f(p["W"] + W2, zero), f(p["W"], zero) + f(W2, zero),
                               rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(f(p["W"], p["bias"]) - f(p["W"], zero),
                               np.broadcast_to(p["bias"], (4, p["bias"].size)), atol=1e-14)
    np.testing.assert_allclose(f(np.zeros_like(p["W"]), p["bias"]),
                               np.broadcast_to(p["bias"], (4, p["bias"].size)), atol=0)


def test_alpha_scales_its_group_only():
    n, C = 4, 16
    p = _params(n, C, 5)
    X = np.random.default_rng(5).normal(size=(3, n, C))
    zero = np.zeros_like(p["bias"])
    base = oracle.coeffs(X, p["gamma"], 1e-6, p["W"], zero, np.ones(3))["z"]
    for g, sl in enumerate([slice(0, n), slice(n, 2 * n), slice(2 * n, None)]):
        al = np.ones(3); al[g] = 3.0
        z = oracle.coeffs(X, p["gamma"], 1e-6, p["W"], zero, al)["z"]
        want = base.copy(); want[:, sl] *= 3.0
        np.testing.assert_allclose(z, want, rtol=1e-14, atol=1e-15)


def test_sigmoid_gating_closed_forms():
    # W = 0: logits are the biases; sigmoid(0) = 1/2, sigmoid(log 3) = 3/4,
    # sigmoid(-log 3) = 1/4, sigmoid(log 9) = 9/10
    n, C = 4, 8
    K = n * n + 2 * n
    bias = np.zeros(K)
    bias[:2 * n] = [0.0, math.log(3), -math.log(3), math.log(9), math.log(9), 0.0, -math.log(3), math.log(3)]
    X = np.random.default_rng(6).normal(size=(2, n, C))
    out = oracle.coeffs(X, np.ones(n * C), 1e-6, np.zeros((n * C, K)), bias, np.ones(3))
    np.testing.assert_allclose(out["Hpre"], [[0.5, 0.75, 0.25, 0.9]] * 2, rtol=1e-15)
    np.testing.assert_allclose(out["Hpost"], [[0.9, 0.5, 0.25, 0.75]] * 2, rtol=1e-15)
    assert ((out["Hpre"] > 0) & (out["Hpre"] < 1)).all()


def test_n1_three_logits():
    # n = 1: K = 1 + 2 = 3 logits (pre, post, one res logit)
    X = np.random.default_rng(7).normal(size=(3, 1, 8))
    out = oracle.coeffs(X, np.ones(8), 1e-6, np.zeros((8, 3)), np.array([0.0, 0.0, 5.0]), np.ones(3))
    assert out["z"].shape == (3, 3)
    H = oracle.sinkhorn(out["z"][:, 2:], 1)
    np.testing.assert_array_equal(H, 1.0)
