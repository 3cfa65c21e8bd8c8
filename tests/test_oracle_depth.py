"""The depth workload's two stacks in the fp64 oracle (60 layers, T = 4096, n = 4,
C = 2048, seed 4): the mHC stack, whose residual mixers are Sinkhorn projections,
and the unconstrained hyper-connection stack with the raw res logit block as the
mixer (chatgpz.de, "Warum Hyperverbindungen instabil werden": the composite of
unconstrained mixers is unbounded, peaking near 3000 in the trained model;
"Vielfaeltig eingeschraenkte Hyperverbindungen": about 1.6 with the constraint).

Pins:
- the mHC composite stays doubly stochastic up to the row residual of 20 Sinkhorn
  iterations: its Amax gain is at least 1 (columns sum to 1, so rows average 1)
  and below 1.1 at every depth;
- the unconstrained composite is a product of independent random matrices, so
  log Amax grows linearly with depth (the Furstenberg-Kesten limit
  log ||P_L|| / L -> a constant): the growth rates over depths 20-40 and 40-60
  agree within 15 %, and the gain passes 1e30 by depth 60;
- both stacks reproduce tests/golden/depth_amax.txt (written by the committed
  make_depth_amax.py from the oracle), which the GPU depth test prints beside the
  GPU's own mHC gains."""
import os

import numpy as np
import pytest

from tests.golden.make_depth_amax import OUT, run_stacks

pytestmark = pytest.mark.slow


def _golden():
    a = np.loadtxt(OUT, comments="#")
    return a[:, 0].astype(int), a[:, 1], a[:, 2]


@pytest.fixture(scope="module")
def stacks():
    rows = run_stacks()
    return (np.array([r[0] for r in rows]), np.array([r[1] for r in rows]),
            np.array([r[2] for r in rows]))


def test_mhc_gain_stays_near_one(stacks):
    _, _, am = stacks
    assert (am >= 1.0 - 1e-9).all() and (am < 1.1).all()


def test_unconstrained_gain_grows_linearly_in_log(stacks):
    d, lu, _ = stacks
    assert len(d) == 60 and np.isfinite(lu).all()
    assert lu[-1] > 30
    assert (np.diff(lu[::10]) > 0).all()
    r1 = (lu[39] - lu[19]) / 20
    r2 = (lu[59] - lu[39]) / 20
    assert r1 > 0.3 and r2 > 0.3
    assert abs(r1 - r2) <= 0.15 * max(r1, r2)


def test_golden_table_reproduces(stacks):
    assert os.path.exists(OUT)
    d, lu, am = stacks
    gd, glu, gam = _golden()
    assert np.array_equal(d, gd)
    np.testing.assert_allclose(lu, glu, rtol=1e-9, atol=0)
    np.testing.assert_allclose(am, gam, rtol=1e-12, atol=0)
