"""Pins of the oracle's optional state gate alpha (Gated DeltaNet backbone).

The pages evaluate OSDN on Gated DeltaNet but print no formula for it
([summary §4] lists the backbones); the reading implemented is
    S_t = alpha_t S_{t-1} + beta_t (v_t - alpha_t S_{t-1} k_t) kt_t^T,
with the preconditioner walk unchanged.  These tests pin the oracle's gated
recurrence against an exact-rational run (oracle/exact.py, written
separately), closed forms (a state reset, one repeated key), the ungated
special case, and the chunked (WY) algebra with cumulative decays that the
GPU kernels implement.
"""
from fractions import Fraction as Fr

import numpy as np
import pytest

from oracle import exact, oracle


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _case(T=24, dk=6, dv=5, seed=0, apf=True):
    g = np.random.default_rng(seed)
    return dict(q=_unit(g.standard_normal((1, 1, T, dk))), k=_unit(g.standard_normal((1, 1, T, dk))),
                v=g.standard_normal((1, 1, T, dv)),
                beta=1 / (1 + np.exp(-g.standard_normal((1, 1, T)))),
                r=1 / (1 + np.exp(-(2 + g.standard_normal((1, 1, T))))) if apf else None,
                d0=0.5 + g.random((1, 1, dk)), S0=0.3 * g.standard_normal((1, 1, dv, dk))), \
        1 / (1 + np.exp(-(2.5 + g.standard_normal((1, 1, T)))))


def test_alpha_one_is_ungated_bitwise():
    c, _ = _case(seed=1)
    a = oracle.forward(**c, eta=0.2)
    b = oracle.forward(**c, eta=0.2, alpha=np.ones((1, 1, 24)))
    for name in ("o", "S", "d", "k_tilde", "rho"):
        assert np.array_equal(a[name], b[name]), name


@pytest.mark.parametrize("seed,T,dk,dv,apf", [(5, 5, 2, 3, True), (6, 6, 3, 2, False)])
def test_gated_exact_rational(seed, T, dk, dv, apf):
    g = np.random.default_rng(seed)
    R = lambda lo, hi: Fr(int(g.integers(lo, hi)), int(g.integers(1, 9)))
    q = [[R(-8, 9) for _ in range(dk)] for _ in range(T)]
    k = [[R(-8, 9) for _ in range(dk)] for _ in range(T)]
    v = [[R(-8, 9) for _ in range(dv)] for _ in range(T)]
    beta = [Fr(int(g.integers(1, 8)), 8) for _ in range(T)]
    r = [Fr(int(g.integers(5, 9)), 8) for _ in range(T)] if apf else None
    alpha = [Fr(int(g.integers(3, 9)), 8) for _ in range(T)]
    d0 = [Fr(int(g.integers(4, 12)), 8) for _ in range(dk)]
    S0 = [[Fr(int(g.integers(-4, 5)), 4) for _ in range(dk)] for _ in range(dv)]
    eta = Fr(3, 10)
    ex = exact.run(q, k, v, beta, r, d0, S0, eta, alpha=alpha)
    f = lambda x: np.array(x, dtype=np.float64)
    out = oracle.forward(q=f(q)[None, None], k=f(k)[None, None], v=f(v)[None, None],
                         beta=f(beta)[None, None], r=None if r is None else f(r)[None, None],
                         d0=f(d0)[None, None], S0=f(S0)[None, None], eta=float(eta),
                         alpha=f(alpha)[None, None])
    for key in ("o", "S", "d", "rho"):
        want = f([[float(x) for x in row] for row in ex[key]] if isinstance(ex[key][0], list)
                 else [float(x) for x in ex[key]])
        got = out[key][0, 0]
        assert np.max(np.abs(got - want)) <= 1e-13 * (1 + np.max(np.abs(want))), key


def test_zero_gate_resets_the_state():
    """alpha_t = 0 forgets everything before t: S_t = beta_t v_t kt_t^T and
    o_t = beta_t (kt_t . q_t) v_t, whatever came before."""
    c, al = _case(T=10, seed=2)
    al[0, 0, 6] = 0.0
    out = oracle.forward(**c, eta=0.2, alpha=al, want=("o", "S", "k_tilde"))
    kt = out["k_tilde"][0, 0, 6]
    S6 = c["beta"][0, 0, 6] * np.outer(c["v"][0, 0, 6], kt)  # the definition, zero prior
    o6 = S6 @ c["q"][0, 0, 6]
    assert np.max(np.abs(out["o"][0, 0, 6] - o6)) <= 1e-14 * (1 + np.max(np.abs(o6)))
    # the run from token 6 on equals a fresh run started there with S0 = 0
    tail = {k_: (v_[:, :, 6:] if (v_ is not None and v_.ndim >= 3 and k_ not in ("d0", "S0")) else v_)
            for k_, v_ in c.items()}
    rest = oracle.forward(**{**tail, "S0": None, "d0": None}, eta=0.0, mode="given",
                          k_given=out["k_tilde"][:, :, 6:], alpha=al[:, :, 6:], want=("o", "S"))
    assert np.max(np.abs(rest["o"] - out["o"][:, :, 6:])) <= 1e-13 * (1 + np.max(np.abs(rest["o"])))
    assert np.max(np.abs(rest["S"] - out["S"])) <= 1e-13 * (1 + np.max(np.abs(rest["S"])))


@pytest.mark.parametrize("a_const,b_const", [(0.9, 0.5), (0.97, 0.3)])
def test_repeated_key_geometric_closed_form(a_const, b_const):
    """One unit key k (= q), constant alpha, beta, eta = 0 (kt = k), S0 = 0 and a
    constant value: s_t = S_t k obeys s_t = alpha (1 - beta) s_{t-1} + beta v, so
    o_t = s_t = beta v (1 - lam^(t+1)) / (1 - lam) with lam = alpha (1 - beta)."""
    T, dk, dv = 40, 6, 3
    g = np.random.default_rng(3)
    kv = _unit(g.standard_normal(dk))
    vv = g.standard_normal(dv)
    k = np.broadcast_to(kv, (1, 1, T, dk)).copy()
    v = np.broadcast_to(vv, (1, 1, T, dv)).copy()
    out = oracle.forward(q=k, k=k, v=v, beta=np.full((1, 1, T), b_const), eta=0.0,
                         alpha=np.full((1, 1, T), a_const), want=("o",))
    lam = a_const * (1 - b_const)
    t = np.arange(T)[:, None]
    want = b_const * vv[None, :] * (1 - lam ** (t + 1)) / (1 - lam)
    assert np.max(np.abs(out["o"][0, 0] - want)) <= 1e-13


@pytest.mark.parametrize("T", [1, 9, 30])
def test_gated_chunked_form_equals_sequential_every_chunk(T):
    """The chunked algebra with cumulative decays (what the kernels compute)."""
    c, al = _case(T=T, seed=40 + T)
    seq = oracle.forward(**c, eta=0.2, alpha=al, want=("o", "S", "k_tilde"))
    for C in range(1, T + 1):
        o, S = oracle.chunked_state_pass(c["q"][0, 0], c["k"][0, 0], seq["k_tilde"][0, 0],
                                         c["v"][0, 0], c["beta"][0, 0], c["S0"][0, 0], C,
                                         alpha=al[0, 0])
        assert np.max(np.abs(o - seq["o"][0, 0])) <= 1e-11 * (1 + np.max(np.abs(seq["o"])))
        assert np.max(np.abs(S - seq["S"][0, 0])) <= 1e-11 * (1 + np.max(np.abs(seq["S"])))


def test_gated_chunked_form_fails_without_the_decay_on_the_read_side():
    """Dropping gamma from the K S^T term breaks the chunk form (the pin can fail)."""
    c, al = _case(T=12, seed=9)
    seq = oracle.forward(**c, eta=0.2, alpha=al, want=("o", "k_tilde"))
    o_bad, _ = oracle.chunked_state_pass(c["q"][0, 0], c["k"][0, 0], seq["k_tilde"][0, 0],
                                         c["v"][0, 0], c["beta"][0, 0], c["S0"][0, 0], 4,
                                         alpha=None)
    assert np.max(np.abs(o_bad - seq["o"][0, 0])) > 1e-4
