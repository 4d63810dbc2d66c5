"""Pins of the oracle's per-channel state gate (Kimi Delta Attention backbone).

The pages evaluate OSDN on KDA but print no formula for it ([summary §4] lists
the backbones).  The reading implemented generalises the scalar gate to one
gate per key dimension:
    S_t = S_{t-1} D_t + beta_t (v_t - S_{t-1} D_t k_t) kt_t^T,   D_t = diag(alpha_t),
with the preconditioner walk unchanged.  These tests pin the oracle's
per-channel recurrence against an exact-rational run (oracle/exact.py,
written separately), closed forms (a basis key, in which the channels
decouple), invariances (a zero channel gate forgets that column; equal
channels are the scalar gate), and the chunked algebra with per-channel
cumulative decays that the GPU kernels implement.
"""
from fractions import Fraction as Fr

import numpy as np
import pytest

from oracle import exact, oracle


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _case(T=24, dk=6, dv=5, seed=0, apf=True, lo=2.0):
    """Inputs of one head and per-channel gates sigmoid(lo + N(0,1))."""
    g = np.random.default_rng(seed)
    c = dict(q=_unit(g.standard_normal((1, 1, T, dk))), k=_unit(g.standard_normal((1, 1, T, dk))),
             v=g.standard_normal((1, 1, T, dv)),
             beta=1 / (1 + np.exp(-g.standard_normal((1, 1, T)))),
             r=1 / (1 + np.exp(-(2 + g.standard_normal((1, 1, T))))) if apf else None,
             d0=0.5 + g.random((1, 1, dk)), S0=0.3 * g.standard_normal((1, 1, dv, dk)))
    al = 1 / (1 + np.exp(-(lo + g.standard_normal((1, 1, T, dk)))))
    return c, al


def test_equal_channels_are_the_scalar_gate_bitwise():
    c, al = _case(seed=1)
    scalar = al[..., 0]
    a = oracle.forward(**c, eta=0.2, alpha=scalar)
    b = oracle.forward(**c, eta=0.2, alpha=np.repeat(scalar[..., None], 6, axis=-1))
    for name in ("o", "S", "d", "k_tilde", "rho"):
        assert np.array_equal(a[name], b[name]), name


@pytest.mark.parametrize("seed,T,dk,dv,apf,deltanet", [(5, 5, 3, 2, True, False),
                                                      (6, 6, 2, 3, False, False),
                                                      (7, 4, 3, 3, True, True)])
def test_per_channel_exact_rational(seed, T, dk, dv, apf, deltanet):
    g = np.random.default_rng(seed)
    R = lambda lo, hi: Fr(int(g.integers(lo, hi)), int(g.integers(1, 9)))
    q = [[R(-8, 9) for _ in range(dk)] for _ in range(T)]
    k = [[R(-8, 9) for _ in range(dk)] for _ in range(T)]
    v = [[R(-8, 9) for _ in range(dv)] for _ in range(T)]
    beta = [Fr(int(g.integers(1, 8)), 8) for _ in range(T)]
    r = [Fr(int(g.integers(5, 9)), 8) for _ in range(T)] if apf else None
    alpha = [[Fr(int(g.integers(0, 9)), 8) for _ in range(dk)] for _ in range(T)]
    d0 = [Fr(int(g.integers(4, 12)), 8) for _ in range(dk)]
    S0 = [[Fr(int(g.integers(-4, 5)), 4) for _ in range(dk)] for _ in range(dv)]
    eta = Fr(3, 10)
    ex = exact.run(q, k, v, beta, r, d0, S0, eta, deltanet=deltanet, alpha=alpha)
    f = lambda x: np.array(x, dtype=np.float64)
    out = oracle.forward(q=f(q)[None, None], k=f(k)[None, None], v=f(v)[None, None],
                         beta=f(beta)[None, None], r=None if r is None else f(r)[None, None],
                         d0=f(d0)[None, None], S0=f(S0)[None, None], eta=float(eta),
                         mode="deltanet" if deltanet else "osdn", alpha=f(alpha)[None, None])
    for key in ("o", "S", "rho") + (() if deltanet else ("d",)):
        want = f([[float(x) for x in row] for row in ex[key]] if isinstance(ex[key][0], list)
                 else [float(x) for x in ex[key]])
        got = out[key][0, 0]
        assert np.max(np.abs(got - want)) <= 1e-13 * (1 + np.max(np.abs(want))), key


def test_zero_channel_gate_forgets_that_column():
    """alpha_0[i] = 0: column i of the entry state is gone before token 0 reads
    it, so no output depends on it (bit for bit); with the gate open it does."""
    c, al = _case(T=12, seed=2)
    al[0, 0, 0, 3] = 0.0
    base = oracle.forward(**c, eta=0.2, alpha=al, want=("o", "S"))
    S0 = c["S0"].copy()
    S0[0, 0, :, 3] += np.arange(1.0, 6.0)
    moved = oracle.forward(**{**c, "S0": S0}, eta=0.2, alpha=al, want=("o", "S"))
    assert np.array_equal(base["o"], moved["o"]) and np.array_equal(base["S"], moved["S"])
    al[0, 0, 0, 3] = 0.5
    a = oracle.forward(**c, eta=0.2, alpha=al, want=("o",))
    b = oracle.forward(**{**c, "S0": S0}, eta=0.2, alpha=al, want=("o",))
    assert np.max(np.abs(a["o"] - b["o"])) > 1e-3


@pytest.mark.parametrize("i,b_const", [(0, 0.5), (4, 0.3)])
def test_basis_key_channels_decouple(i, b_const):
    """k_t = q_t = e_i, eta = 0 (kt = k), constant per-channel gates a, beta and
    value: column i obeys s_t = a_i (1 - beta) s_{t-1} + beta v, so
    o_t = beta v (1 - lam^(t+1)) / (1 - lam) + lam^(t+1) S0[:, i], lam = a_i (1 - beta);
    every other column j only decays: S_T[:, j] = a_j^T S0[:, j]."""
    T, dk, dv = 30, 6, 3
    g = np.random.default_rng(10 + i)
    a = 0.55 + 0.4 * g.random(dk)
    vv = g.standard_normal(dv)
    S0 = g.standard_normal((1, 1, dv, dk))
    e = np.zeros(dk)
    e[i] = 1.0
    k = np.broadcast_to(e, (1, 1, T, dk)).copy()
    v = np.broadcast_to(vv, (1, 1, T, dv)).copy()
    out = oracle.forward(q=k, k=k, v=v, beta=np.full((1, 1, T), b_const), S0=S0, eta=0.0,
                         alpha=np.broadcast_to(a, (1, 1, T, dk)).copy(), want=("o", "S"))
    lam = a[i] * (1 - b_const)
    t = np.arange(T)[:, None]
    want = (b_const * vv[None, :] * (1 - lam ** (t + 1)) / (1 - lam)
            + lam ** (t + 1) * S0[0, 0, :, i][None, :])
    assert np.max(np.abs(out["o"][0, 0] - want)) <= 1e-13
    for j in range(dk):
        if j != i:
            assert np.max(np.abs(out["S"][0, 0, :, j] - a[j] ** T * S0[0, 0, :, j])) <= 1e-14


@pytest.mark.parametrize("T", [1, 9, 30])
def test_per_channel_chunked_form_equals_sequential_every_chunk(T):
    """The chunked algebra with per-channel cumulative decays."""
    c, al = _case(T=T, seed=40 + T)
    seq = oracle.forward(**c, eta=0.2, alpha=al, want=("o", "S", "k_tilde"))
    for C in range(1, T + 1):
        o, S = oracle.chunked_state_pass(c["q"][0, 0], c["k"][0, 0], seq["k_tilde"][0, 0],
                                         c["v"][0, 0], c["beta"][0, 0], c["S0"][0, 0], C,
                                         alpha=al[0, 0])
        assert np.max(np.abs(o - seq["o"][0, 0])) <= 1e-11 * (1 + np.max(np.abs(seq["o"])))
        assert np.max(np.abs(S - seq["S"][0, 0])) <= 1e-11 * (1 + np.max(np.abs(seq["S"])))


def test_per_channel_chunked_form_fails_with_a_scalar_decay():
    """Replacing the per-channel decays by their mean breaks the chunk form (the
    pin can fail)."""
    c, al = _case(T=12, seed=9, lo=0.0)
    seq = oracle.forward(**c, eta=0.2, alpha=al, want=("o", "k_tilde"))
    o_bad, _ = oracle.chunked_state_pass(c["q"][0, 0], c["k"][0, 0], seq["k_tilde"][0, 0],
                                         c["v"][0, 0], c["beta"][0, 0], c["S0"][0, 0], 4,
                                         alpha=al[0, 0].mean(axis=-1))
    assert np.max(np.abs(o_bad - seq["o"][0, 0])) > 1e-4
