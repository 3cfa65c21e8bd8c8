"""Pins of the composite residual mapping over depth and its Amax gain
(chatgpz.de, "Warum Hyperverbindungen instabil werden": product of the residual
mixers over many layers, gain from maximal row and column sums; staging.
reportify.cn, "mHC方法原理" note [15]: products of doubly stochastic matrices
stay doubly stochastic)."""
import numpy as np

import oracle


def _gain(H):
    P = np.broadcast_to(np.eye(H.shape[-1]), H.shape).copy()
    return oracle.composite(H, P)


def test_gain_closed_forms():
    cases = [
        (np.eye(4), 1.0, 1.0),
        (np.eye(4)[[1, 2, 3, 0]], 1.0, 1.0),
        (np.full((4, 4), 0.25), 1.0, 1.0),
        (np.diag([2.0, 1.0, 0.5, 1.0]), 2.0, 2.0),
        (np.array([[1.0, 2.0], [0.0, 0.0]]), 3.0, 2.0),
        (np.array([[1.0, -2.0], [3.0, 0.5]]), 3.5, 4.0),
    ]
    for H, gr, gc in cases:
        r, c = _gain(H[None].copy())
        assert r[0] == gr and c[0] == gc


def test_later_layers_multiply_on_the_left():
    rng = np.random.default_rng(0)
    H1, H2 = rng.normal(size=(1, 4, 4)), rng.normal(size=(1, 4, 4))
    P = np.eye(4)[None].copy()
    oracle.composite(H1, P)
    oracle.composite(H2, P)
    np.testing.assert_allclose(P[0], H2[0] @ H1[0], rtol=1e-14)


def test_stack_gain_bounded_vs_unconstrained_growth():
    # 60-layer toy stack, random weights: doubly stochastic mixers keep the gain
    # near 1; unconstrained mixers (raw logits) grow geometrically with depth
    rng = np.random.default_rng(1)
    T, n, C, L = 4, 4, 16, 60
    P_m = np.broadcast_to(np.eye(n), (T, n, n)).copy()
    P_u = P_m.copy()
    g_m, g_u = [], []
    for _ in range(L):
        z = rng.normal(scale=1.0, size=(T, n * n)) + 3.0 * np.eye(n).ravel()
        r, c = oracle.composite(oracle.sinkhorn(z, n), P_m)
        g_m.append(max(r.max(), c.max()))
        r, c = oracle.composite(z.reshape(T, n, n), P_u)
        g_u.append(max(r.max(), c.max()))
    # columns sum to 1 after every column step, so only the small row residual of
    # 20 iterations accumulates: the gain stays within a few percent of 1
    assert max(g_m) < 1.1 and min(g_m) >= 1.0 - 1e-12
    assert np.log10(g_u[-1]) > 20 and np.log10(g_u[-1]) > 1.5 * np.log10(g_u[L // 2])
