"""The fp64 oracle against exact values: a hand-worked example and the
exact-rational fixtures under tests/golden/ (written by make_golden.py from
oracle/exact.py).  Formulas: gist.science technical summary of "OSDN:
Improving Delta Rule with Provable Online Preconditioning in Linear Attention",
§1 (delta rule), §2.1 (preconditioned key), §2.2 (closed-form surrogate),
§2.3 (APF), §3 (residual ratio)."""
import glob
import json
import os
from fractions import Fraction as Fr

import numpy as np
import pytest

from oracle import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def _arr(x):
    if x is None:
        return None
    if isinstance(x, list):
        return np.array([_arr(y) for y in x], dtype=np.float64)
    return float(Fr(x))


def test_hand_worked_two_tokens():
    """dk = dv = 2, d0 = 1, S0 = 0, eta = 1/2, no retention.
    t=0: k=(3/5,4/5) (n=1, a=1), beta=1/2, v=(1,2), q=(1,0)
         S1 = 1/2 (1,2)^T (3/5,4/5) = [[3/10, 2/5], [3/5, 4/5]];  o0 = (3/10, 3/5)
         rho0 = (1 - 1/2)^2 = 1/4;  c = 1/2*1/2*(1-1/2)/1 = 1/8
         d1 = 1 + (1/8)(9/25, 16/25) = (209/200, 27/25)
    t=1: k=(0,1) (n=1, a=27/25), beta=1, v=(0,1), q=(0,1)
         k~ = (0, 27/25);  u = v - S1 k = (-2/5, 1/5)
         S2 = S1 + u k~^T = [[3/10, -4/125], [3/5, 127/125]];  o1 = (-4/125, 127/125)
         rho1 = (1 - 27/25)^2 = 4/625;  c = 1/2*(1-27/25) = -1/25
         d2 = (209/200, 26/25)
    """
    k = np.array([[0.6, 0.8], [0.0, 1.0]])[None, None]
    v = np.array([[1.0, 2.0], [0.0, 1.0]])[None, None]
    q = np.array([[1.0, 0.0], [0.0, 1.0]])[None, None]
    beta = np.array([[[0.5, 1.0]]])
    out = oracle.forward(q=q, k=k, v=v, beta=beta, eta=0.5, want=("o", "S", "d", "rho", "k_tilde"))
    tol = 1e-15
    assert np.allclose(out["o"][0, 0], [[0.3, 0.6], [-4 / 125, 127 / 125]], rtol=0, atol=tol)
    assert np.allclose(out["S"][0, 0], [[0.3, -4 / 125], [0.6, 127 / 125]], rtol=0, atol=tol)
    assert np.allclose(out["d"][0, 0], [209 / 200, 26 / 25], rtol=0, atol=tol)
    assert np.allclose(out["rho"][0, 0], [0.25, 4 / 625], rtol=0, atol=tol)
    assert np.allclose(out["k_tilde"][0, 0], [[0.6, 0.8], [0.0, 27 / 25]], rtol=0, atol=tol)


@pytest.mark.parametrize("path", sorted(glob.glob(os.path.join(HERE, "golden", "*.json"))))
def test_exact_rational_fixture(path):
    rec = json.load(open(path))
    i = rec["inputs"]
    out = oracle.forward(q=_arr(i["q"])[None, None], k=_arr(i["k"])[None, None],
                         v=_arr(i["v"])[None, None], beta=_arr(i["beta"])[None, None],
                         r=None if i["r"] is None else _arr(i["r"])[None, None],
                         d0=None if i["d0"] is None else _arr(i["d0"])[None, None],
                         S0=None if i["S0"] is None else _arr(i["S0"])[None, None],
                         eta=float(Fr(i["eta"])))
    for name, key in (("o", "o"), ("S", "S"), ("d", "d"), ("k_tilde", "k_tilde"), ("rho", "rho")):
        want = _arr(rec["outputs"][key])
        got = out[name][0, 0]
        assert np.max(np.abs(got - want)) <= 1e-14 * (1 + np.max(np.abs(want))), name
