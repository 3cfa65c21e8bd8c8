"""Pins of the oracle's read map u = H_pre X and write X' = H_res X + H_post^T F
(chatgpz.de, "Von Residualverbindungen zu Hyperverbindungen": the update rule;
"Vielfaeltig eingeschraenkte Hyperverbindungen": convex combination of streams,
feature mass preserved).  Special cases reduce to the standard residual
x + F(x) (same page; staging.reportify.cn, the x + F(x) structure)."""
import numpy as np

import oracle


def test_n1_unit_maps_reduce_to_standard_residual():
    rng = np.random.default_rng(0)
    T, C = 5, 33
    x = rng.normal(size=(T, 1, C)); F = rng.normal(size=(T, C))
    one = np.ones((T, 1))
    u = oracle.pre(x, one)
    np.testing.assert_array_equal(u, x[:, 0])
    Xo = oracle.post_res(x, F, np.ones((T, 1, 1)), one)
    np.testing.assert_array_equal(Xo[:, 0], x[:, 0] + F)


def test_pre_selects_stream():
    rng = np.random.default_rng(1)
    T, n, C = 3, 4, 16
    X = rng.normal(size=(T, n, C))
    for k in range(n):
        H = np.zeros((T, n)); H[:, k] = 1.0
        np.testing.assert_array_equal(oracle.pre(X, H), X[:, k])


def test_res_orientation_with_permutation():
    # H_res[i][j] feeds input stream j into output stream i
    rng = np.random.default_rng(2)
    T, n, C = 2, 4, 8
    X = rng.normal(size=(T, n, C)); F = rng.normal(size=(T, C))
    perm = [2, 0, 3, 1]
    P = np.broadcast_to(np.eye(n)[perm], (T, n, n)).copy()
    Xo = oracle.post_res(X, F, P, np.zeros((T, n)))
    for i in range(n):
        np.testing.assert_array_equal(Xo[:, i], X[:, perm[i]])
    e = np.zeros((T, n)); e[:, 3] = 1.0
    Xo = oracle.post_res(X, F, np.zeros((T, n, n)), e)
    np.testing.assert_array_equal(Xo[:, 3], F)
    np.testing.assert_array_equal(Xo[:, :3], 0.0)


def test_mass_conservation_and_convexity():
    rng = np.random.default_rng(3)
    T, n, C = 6, 4, 40
    X = rng.normal(size=(T, n, C)); F = rng.normal(size=(T, C))
    H = oracle.sinkhorn(rng.normal(size=(T, n * n)), n, iters=400)
    Hp = rng.uniform(0, 1, (T, n))
    Xo = oracle.post_res(X, F, H, Hp)
    np.testing.assert_allclose(Xo.sum(1), X.sum(1) + Hp.sum(1)[:, None] * F, atol=1e-12)
    Xr = oracle.post_res(X, F, H, np.zeros((T, n)))
    lo, hi = X.min(1, keepdims=True), X.max(1, keepdims=True)
    assert (Xr >= lo - 1e-12).all() and (Xr <= hi + 1e-12).all()
