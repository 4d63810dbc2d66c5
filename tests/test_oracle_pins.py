"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Source: gist.science technical summary of "OSDN: Improving Delta Rule with
Provable Online Preconditioning in Linear Attention" (arXiv 2605.13473),
cited as [summary §N].  None of these tests retypes the oracle's recurrence
and compares it with itself: each checks it against a closed form, a special
case with a hand-derived answer, an independent formulation (explicit dense
preconditioner, explicit gradient, chunk form), an exact-rational run, or a
finite-difference derivative of the surrogate's definition.
"""
from fractions import Fraction as Fr

import numpy as np
import pytest

from oracle import exact, oracle

RNG = np.random.default_rng(20260513)


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _rand_case(B=1, H=1, T=24, dk=6, dv=5, apf=True, seed=0, S0=True, d0=True):
    g = np.random.default_rng(seed)
    q = _unit(g.standard_normal((B, H, T, dk)))
    k = _unit(g.standard_normal((B, H, T, dk)))
    v = g.standard_normal((B, H, T, dv))
    beta = 1 / (1 + np.exp(-g.standard_normal((B, H, T))))
    r = 1 / (1 + np.exp(-(2 + g.standard_normal((B, H, T))))) if apf else None
    d0a = 0.5 + g.random((B, H, dk)) if d0 else None
    S0a = 0.3 * g.standard_normal((B, H, dv, dk)) if S0 else None
    return dict(q=q, k=k, v=v, beta=beta, r=r, d0=d0a, S0=S0a)


# --------------------------------------------------------------------------
# (a) the closed-form surrogate equals its ratio definition  [summary §2.2]
# --------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(8))
def test_surrogate_closed_form_equals_direct_ratio(seed):
    g = np.random.default_rng(100 + seed)
    dk, dv = 7, 5
    S = g.standard_normal((dv, dk))
    v = g.standard_normal(dv)
    k = g.standard_normal(dk)
    d = 0.2 + 2 * g.random(dk)
    beta = float(g.random())
    h_direct = oracle.surrogate_direct(S, k, v, d, beta)
    h_closed = oracle.surrogate_closed(d, k, beta)
    # both sides are O(1/||k||^2); absolute tolerance scaled by it
    assert abs(h_direct - h_closed) <= 1e-10 * (1 + abs(h_closed)) / min(1.0, float(k @ k))


@pytest.mark.parametrize("seed", range(6))
def test_surrogate_gradient_matches_finite_differences_of_definition(seed):
    """The gradient that drives the d step, against central differences of the
    *ratio definition* (explicit S update), which never sees the closed form."""
    g = np.random.default_rng(200 + seed)
    dk, dv = 6, 4
    S = g.standard_normal((dv, dk))
    v = g.standard_normal(dv)
    k = g.standard_normal(dk)
    d = 0.5 + g.random(dk)
    beta = 0.3 + 0.6 * float(g.random())
    eps = 1e-5
    fd = np.zeros(dk)
    for i in range(dk):
        e = np.zeros(dk)
        e[i] = eps
        fd[i] = (oracle.surrogate_direct(S, k, v, d + e, beta)
                 - oracle.surrogate_direct(S, k, v, d - e, beta)) / (2 * eps)
    grad = oracle.surrogate_grad(d, k, beta)
    assert np.max(np.abs(fd - grad)) <= 1e-7 * (1 + np.max(np.abs(grad)))


@pytest.mark.parametrize("apf", [False, True])
def test_oracle_d_step_is_descent_on_the_definition(apf):
    """One token of the C oracle: d_1 = r d_0 - eta * grad h (grad by finite
    differences of the ratio definition).  An ascent step (the '+' printed in the
    APF equation of [summary §2.3]) fails this."""
    g = np.random.default_rng(7)
    dk, dv = 5, 3
    c = _rand_case(T=1, dk=dk, dv=dv, apf=apf, seed=11)
    eta = 0.37
    out = oracle.forward(**c, eta=eta)
    k = c["k"][0, 0, 0]
    v = c["v"][0, 0, 0]
    S = c["S0"][0, 0]
    d = c["d0"][0, 0]
    beta = float(c["beta"][0, 0, 0])
    rt = float(c["r"][0, 0, 0]) if apf else 1.0
    eps = 1e-5
    fd = np.array([(oracle.surrogate_direct(S, k, v, d + eps * e, beta)
                    - oracle.surrogate_direct(S, k, v, d - eps * e, beta)) / (2 * eps)
                   for e in np.eye(dk)])
    expect = rt * d - eta * fd
    assert np.max(np.abs(out["d"][0, 0] - expect)) <= 1e-8
    # and it is a real descent step: h decreases for small eta (no retention)
    if not apf:
        h0 = oracle.surrogate_closed(d, k, beta)
        h1 = oracle.surrogate_closed(out["d"][0, 0], k, beta)
        assert h1 <= h0 + 1e-15


# --------------------------------------------------------------------------
# (b) token-local residual ratio  [summary §3]
# --------------------------------------------------------------------------

@pytest.mark.parametrize("apf", [False, True])
def test_residual_ratio_and_vector_identity(apf):
    T, dk, dv = 12, 6, 4
    c = _rand_case(T=T, dk=dk, dv=dv, apf=apf, seed=21)
    eta = 0.3
    full = oracle.forward(**c, eta=eta, want=("rho", "d_all", "k_tilde"))
    # states after each prefix: run the oracle on prefixes
    states = [c["S0"][0, 0]]
    for t in range(1, T + 1):
        pre = {kk: (vv[:, :, :t] if (vv is not None and vv.ndim >= 3 and kk not in ("d0", "S0"))
                    else vv) for kk, vv in c.items()}
        states.append(oracle.forward(**pre, eta=eta, want=("S",))["S"][0, 0])
    for t in range(T):
        k = c["k"][0, 0, t]
        v = c["v"][0, 0, t]
        S_prev, S_new = states[t], states[t + 1]
        f_prev = 0.5 * np.sum((S_prev @ k - v) ** 2)
        f_new = 0.5 * np.sum((S_new @ k - v) ** 2)
        rho = full["rho"][0, 0, t]
        assert abs(f_new / f_prev - rho) <= 1e-11 * max(1.0, rho)
        # S_t k - v = -(1 - beta a) (v - S_{t-1} k) with a = <d_t, k^2>
        a = float(full["d_all"][0, 0, t] @ (k * k))
        beta = c["beta"][0, 0, t]
        lhs = S_new @ k - v
        rhs = -(1 - beta * a) * (v - S_prev @ k)
        assert np.max(np.abs(lhs - rhs)) <= 1e-12 * (1 + np.max(np.abs(rhs)))
        assert abs((1 - beta * a) ** 2 - rho) <= 1e-13


# --------------------------------------------------------------------------
# (c) eta = 0, d0 = 1 reduces to the plain delta rule  [summary §1, §2.1]
# --------------------------------------------------------------------------

def test_eta_zero_is_deltanet_bitwise():
    c = _rand_case(B=2, H=2, T=40, dk=8, dv=6, apf=False, seed=31, d0=False)
    osdn = oracle.forward(**c, eta=0.0, mode="osdn", want=("o", "S", "d", "k_tilde", "rho"))
    dn = oracle.forward(**c, eta=0.0, mode="deltanet", want=("o", "S", "k_tilde", "rho"))
    assert np.array_equal(osdn["o"], dn["o"])
    assert np.array_equal(osdn["S"], dn["S"])
    assert np.array_equal(osdn["k_tilde"], c["k"])
    assert np.all(osdn["d"] == 1.0)
    # DeltaNet's residual ratio with unit keys is (1 - beta)^2
    assert np.allclose(dn["rho"], (1 - c["beta"]) ** 2, rtol=1e-13, atol=1e-15)


def test_eta_zero_with_retention_only_decays():
    """With APF and eta = 0 the preconditioner only decays: d_T = prod_t r_t * d_0."""
    c = _rand_case(B=2, H=2, T=40, dk=8, dv=6, apf=True, seed=32, d0=False)
    out = oracle.forward(**c, eta=0.0, want=("d",))
    assert np.allclose(out["d"], np.prod(c["r"], axis=-1)[..., None] * np.ones(8), rtol=1e-13)


def test_deltanet_orthonormal_keys_store_exactly():
    """Textbook delta-rule fact: with orthonormal keys, beta = 1 and no
    preconditioning, each write makes S k_t = v_t exactly and leaves earlier
    keys' memories intact; queries equal to keys read back the values."""
    dk = dv = 6
    Qm, _ = np.linalg.qr(RNG.standard_normal((dk, dk)))
    K = Qm.T[None, None]              # rows are orthonormal keys
    V = RNG.standard_normal((1, 1, dk, dv))
    beta = np.ones((1, 1, dk))
    out = oracle.forward(q=K, k=K, v=V, beta=beta, eta=0.0, mode="deltanet", want=("o", "S"))
    assert np.max(np.abs(out["o"] - V)) < 1e-12
    S = out["S"][0, 0]
    assert np.max(np.abs(S @ K[0, 0].T - V[0, 0].T)) < 1e-12


# --------------------------------------------------------------------------
# explicit dense preconditioner: right-preconditioned gradient step equals the
# write-key scaling  [summary §2.1]
# --------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(4))
def test_dense_right_preconditioning_equals_key_scaling(seed):
    g = np.random.default_rng(300 + seed)
    dk, dv = 7, 5
    S = g.standard_normal((dv, dk))
    k = g.standard_normal(dk)
    v = g.standard_normal(dv)
    d = 0.5 + g.random(dk)
    beta = float(g.random())
    grad = np.outer(S @ k - v, k)                  # grad f_t(S) [summary §1]
    S_dense = S - beta * grad @ np.diag(d)          # S - beta grad f D
    out = oracle.forward(q=k[None, None, None], k=k[None, None, None], v=v[None, None, None],
                         beta=np.array([[[beta]]]), d0=d[None, None], S0=S[None, None],
                         eta=0.0, want=("S",))
    assert np.max(np.abs(out["S"][0, 0] - S_dense)) <= 1e-13 * (1 + np.max(np.abs(S_dense)))


# --------------------------------------------------------------------------
# (d) chunkwise form == sequential at every chunk size  [summary §2.1]
# --------------------------------------------------------------------------

@pytest.mark.parametrize("T", [1, 7, 33])
def test_chunked_state_pass_equals_sequential_every_chunk(T):
    dk, dv = 5, 4
    c = _rand_case(T=T, dk=dk, dv=dv, apf=True, seed=40 + T)
    seq = oracle.forward(**c, eta=0.2, want=("o", "S", "k_tilde"))
    for C in range(1, T + 1):
        o, S = oracle.chunked_state_pass(c["q"][0, 0], c["k"][0, 0], seq["k_tilde"][0, 0],
                                         c["v"][0, 0], c["beta"][0, 0], c["S0"][0, 0], C)
        assert np.max(np.abs(o - seq["o"][0, 0])) <= 1e-11 * (1 + np.max(np.abs(seq["o"])))
        assert np.max(np.abs(S - seq["S"][0, 0])) <= 1e-11 * (1 + np.max(np.abs(seq["S"])))


def test_chunked_form_uses_mixed_keys():
    """The chunk form must put K (not K~) on the read side: using K~ in the
    residual fails against the sequential recurrence."""
    T, dk, dv = 16, 5, 4
    c = _rand_case(T=T, dk=dk, dv=dv, apf=False, seed=55, S0=False)
    seq = oracle.forward(**c, eta=0.5, want=("o", "S", "k_tilde"))
    kt = seq["k_tilde"][0, 0]
    assert np.max(np.abs(kt - c["k"][0, 0])) > 1e-3   # preconditioner really moved
    o_bad, _ = oracle.chunked_state_pass(c["q"][0, 0], kt, kt, c["v"][0, 0], c["beta"][0, 0],
                                         None, 4)
    assert np.max(np.abs(o_bad - seq["o"][0, 0])) > 1e-6


# --------------------------------------------------------------------------
# P5: exact-rational brute force
# --------------------------------------------------------------------------

def _rat_case(seed, T, dk, dv, apf):
    g = np.random.default_rng(seed)
    R = lambda lo, hi: Fr(int(g.integers(lo, hi)), int(g.integers(1, 9)))
    q = [[R(-8, 9) for _ in range(dk)] for _ in range(T)]
    k = [[R(-8, 9) for _ in range(dk)] for _ in range(T)]
    v = [[R(-8, 9) for _ in range(dv)] for _ in range(T)]
    beta = [Fr(int(g.integers(1, 8)), 8) for _ in range(T)]
    r = [Fr(int(g.integers(5, 9)), 8) for _ in range(T)] if apf else None
    d0 = [Fr(int(g.integers(4, 12)), 8) for _ in range(dk)]
    S0 = [[Fr(int(g.integers(-4, 5)), 4) for _ in range(dk)] for _ in range(dv)]
    return q, k, v, beta, r, d0, S0


@pytest.mark.parametrize("seed,T,dk,dv,apf", [(1, 5, 2, 3, False), (2, 6, 3, 3, True),
                                              (3, 4, 3, 2, True), (4, 6, 2, 2, False)])
def test_exact_rational_brute_force(seed, T, dk, dv, apf):
    q, k, v, beta, r, d0, S0 = _rat_case(seed, T, dk, dv, apf)
    eta = Fr(3, 10)
    ex = exact.run(q, k, v, beta, r, d0, S0, eta)
    f = lambda x: np.array(x, dtype=np.float64)
    out = oracle.forward(q=f(q)[None, None], k=f(k)[None, None], v=f(v)[None, None],
                         beta=f(beta)[None, None], r=None if r is None else f(r)[None, None],
                         d0=f(d0)[None, None], S0=f(S0)[None, None], eta=float(eta))
    for name, key in (("o", "o"), ("S", "S"), ("d", "d"), ("k_tilde", "k_tilde"), ("rho", "rho")):
        want = f([[float(x) for x in row] for row in ex[key]] if isinstance(ex[key][0], list)
                 else [float(x) for x in ex[key]])
        got = out[name][0, 0]
        assert np.max(np.abs(got - want)) <= 1e-13 * (1 + np.max(np.abs(want))), name


# --------------------------------------------------------------------------
# P6: one repeated key -- scalar affine recurrence, gated Newton fixed point
# [summary §3: beta <d*, k^2> = 1]
# --------------------------------------------------------------------------

@pytest.mark.parametrize("r_const", [1.0, 0.93])
def test_repeated_key_closed_form(r_const):
    T, dk, dv = 200, 8, 5
    g = np.random.default_rng(61)
    k = g.standard_normal(dk)
    k *= 0.9 / np.linalg.norm(k)
    v = g.standard_normal(dv)
    beta, eta = 0.6, 0.4
    K = np.tile(k, (T, 1))[None, None]
    out = oracle.forward(q=K, k=K, v=np.tile(v, (T, 1))[None, None],
                         beta=np.full((1, 1, T), beta),
                         r=np.full((1, 1, T), r_const) if r_const != 1.0 else None,
                         eta=eta, want=("o", "d_all", "rho"))
    p = k * k
    n = p.sum()
    pp = p @ p
    lam = r_const - eta * beta ** 2 * pp / n
    mu = eta * beta * pp / n
    a_star = mu / (1 - lam)
    t = np.arange(T)
    a_closed = lam ** t * (n - a_star) + a_star          # a_0 = <1, p> = n
    a_oracle = out["d_all"][0, 0] @ p
    assert np.max(np.abs(a_oracle - a_closed)) <= 1e-12
    if r_const == 1.0:
        # gated Newton: beta a -> 1, with 1 - beta a_t = (1 - beta n) lam^t
        assert abs(a_star - 1 / beta) < 1e-14
        assert np.max(np.abs((1 - beta * a_oracle) - (1 - beta * n) * lam ** t)) <= 1e-12
    # readout: o_t = (1 - prod_{s<=t} (1 - beta a_s)) v  (S_0 = 0, q = k)
    prod = np.cumprod(1 - beta * a_closed)
    assert np.max(np.abs(out["o"][0, 0] - (1 - prod)[:, None] * v[None])) <= 1e-12
    assert np.max(np.abs(out["rho"][0, 0] - (1 - beta * a_closed) ** 2)) <= 1e-12


# --------------------------------------------------------------------------
# P7: basis keys -- per-column gated EMA, hand-derived
# --------------------------------------------------------------------------

@pytest.mark.parametrize("apf", [False, True])
def test_basis_keys_closed_form(apf):
    T, dk, dv = 50, 4, 3
    g = np.random.default_rng(71)
    j = g.integers(0, dk, size=T)
    K = np.eye(dk)[j]
    Q = g.standard_normal((T, dk))
    V = g.standard_normal((T, dv))
    beta = g.random(T)
    r = 0.8 + 0.2 * g.random(T) if apf else np.ones(T)
    eta = 0.7
    out = oracle.forward(q=Q[None, None], k=K[None, None], v=V[None, None],
                         beta=beta[None, None], r=r[None, None] if apf else None, eta=eta,
                         want=("o", "S", "d", "d_all"))
    # hand-derived: write key = d_j e_j ; column j of S is an EMA towards v
    d = np.ones(dk)
    S = np.zeros((dv, dk))
    for t in range(T):
        jj = j[t]
        assert np.allclose(out["d_all"][0, 0, t], d, rtol=0, atol=1e-13)
        w = beta[t] * d[jj]
        S[:, jj] = (1 - w) * S[:, jj] + w * V[t]
        assert np.allclose(out["o"][0, 0, t], S @ Q[t], rtol=0, atol=1e-12)
        step = eta * beta[t] * (1 - beta[t] * d[jj])
        d = r[t] * d
        d[jj] += step
    assert np.allclose(out["S"][0, 0], S, rtol=0, atol=1e-12)
    assert np.allclose(out["d"][0, 0], d, rtol=0, atol=1e-13)


# --------------------------------------------------------------------------
# P8: continuation through the persistent state (S, d)  [summary §4.3]
# --------------------------------------------------------------------------

@pytest.mark.parametrize("split", [1, 17, 39])
def test_continuation_bitwise(split):
    T = 40
    c = _rand_case(B=1, H=2, T=T, dk=6, dv=5, apf=True, seed=81)
    whole = oracle.forward(**c, eta=0.3, want=("o", "S", "d"))
    cut = lambda sl: {kk: (vv[:, :, sl] if (vv is not None and kk not in ("d0", "S0")) else vv)
                      for kk, vv in c.items()}
    first = oracle.forward(**cut(slice(0, split)), eta=0.3, want=("o", "S", "d"))
    c2 = cut(slice(split, T))
    c2["S0"], c2["d0"] = first["S"], first["d"]
    second = oracle.forward(**c2, eta=0.3, want=("o", "S", "d"))
    assert np.array_equal(np.concatenate([first["o"], second["o"]], axis=2), whole["o"])
    assert np.array_equal(second["S"], whole["S"])
    assert np.array_equal(second["d"], whole["d"])


# --------------------------------------------------------------------------
# P9: the preconditioner recurrence unrolled per chunk  [summary §2.3, affine]
# --------------------------------------------------------------------------

@pytest.mark.parametrize("apf", [False, True])
def test_chunked_dwalk_equals_serial(apf):
    T, dk = 37, 6
    c = _rand_case(T=T, dk=dk, dv=2, apf=apf, seed=91)
    ser = oracle.forward(**c, eta=0.45, want=("d_all", "d"))
    for C in (1, 2, 5, 8, 16, 37):
        d_all, d_fin = oracle.chunked_dwalk(c["k"][0, 0], c["beta"][0, 0],
                                            None if c["r"] is None else c["r"][0, 0],
                                            c["d0"][0, 0], 0.45, C)
        assert np.max(np.abs(d_all - ser["d_all"][0, 0])) <= 1e-12
        assert np.max(np.abs(d_fin - ser["d"][0, 0])) <= 1e-12


# --------------------------------------------------------------------------
# degenerate inputs
# --------------------------------------------------------------------------

def test_zero_key_leaves_d_untouched_except_retention():
    dk, dv = 4, 3
    k = np.zeros((1, 1, 3, dk))
    k[0, 0, 1] = [0.5, -0.5, 0.5, 0.5]
    out = oracle.forward(q=k, k=k, v=np.ones((1, 1, 3, dv)), beta=np.full((1, 1, 3), 0.5),
                         r=np.full((1, 1, 3), 0.9), eta=0.3, want=("d_all", "d", "o", "S"))
    da = out["d_all"][0, 0]
    assert np.allclose(da[1], 0.9 * da[0]) and np.all(np.isfinite(out["S"]))


def test_empty_sequence_returns_initial_state():
    c = _rand_case(T=0, dk=4, dv=3, seed=5)
    out = oracle.forward(**c, eta=0.1)
    assert out["o"].shape == (1, 1, 0, 3)
    assert np.array_equal(out["S"], c["S0"]) and np.array_equal(out["d"], c["d0"])


def test_head_subset_matches_full_run():
    c = _rand_case(B=2, H=3, T=20, dk=5, dv=4, seed=12)
    full = oracle.forward(**c, eta=0.2)
    sub = oracle.forward(**c, eta=0.2, heads=[4, 1])
    for bh in (1, 4):
        b, h = divmod(bh, 3)
        assert np.array_equal(sub["o"][b, h], full["o"][b, h])
        assert np.array_equal(sub["S"][b, h], full["S"][b, h])


def test_q_geo_definition():
    rho = np.array([0.25, 1.0, 0.5, 2.0])
    assert abs(oracle.q_geo(rho) - (0.25 * 1.0 * 0.5 * 2.0) ** 0.25) < 1e-15
