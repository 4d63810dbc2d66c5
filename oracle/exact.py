"""Exact-rational OSDN recurrence (fractions.Fraction) -- TEST INFRASTRUCTURE ONLY.

A second, independently written statement of the token-serial recurrence of
the OSDN technical summary (gist.science, "OSDN: Improving Delta Rule with
Provable Online Preconditioning in Linear Attention", §1 delta rule, §2.1
preconditioned key, §2.2 closed-form surrogate, §2.3 APF), in exact rational
arithmetic.  The recurrence needs only + - * /, so for rational inputs every
quantity is exact and the fp64 C oracle must agree to rounding.  Pure Python
loops: tiny cases only (T <= 8, dk, dv <= 4).
"""
from __future__ import annotations

from fractions import Fraction as F


def run(q, k, v, beta, r=None, d0=None, S0=None, eta=F(0), deltanet=False, alpha=None):
    """Sequences of rationals: q,k [T][dk], v [T][dv], beta,r [T], d0 [dk],
    S0 [dv][dk].  alpha is the optional state gate (the state is scaled by
    alpha_t before token t reads and writes it): [T] scalars, or [T][dk] with one
    gate per key dimension, which scales column i of the state by alpha_t[i].
    Returns dict(o [T][dv], S [dv][dk], d [dk], k_tilde [T][dk], rho [T])."""
    T = len(k)
    dk = len(k[0]) if T else (len(d0) if d0 is not None else 0)
    dv = len(v[0]) if T else (len(S0) if S0 is not None else 0)
    S = [[F(x) for x in row] for row in S0] if S0 is not None else [[F(0)] * dk for _ in range(dv)]
    d = [F(x) for x in d0] if d0 is not None else [F(1)] * dk
    eta = F(eta)
    outs, kts, rhos = [], [], []
    for t in range(T):
        kt_vec = [F(x) for x in k[t]]
        b = F(beta[t])
        rt = F(r[t]) if r is not None else F(1)
        sq = [x * x for x in kt_vec]
        n = sum(sq, F(0))
        a = sum((di * si for di, si in zip(d, sq)), F(0))
        w = list(kt_vec) if deltanet else [di * ki for di, ki in zip(d, kt_vec)]
        kts.append(w)
        if alpha is not None and isinstance(alpha[t], (list, tuple)):
            ag = [F(x) for x in alpha[t]]
            S = [[ag[i] * row[i] for i in range(dk)] for row in S]
        elif alpha is not None:
            at = F(alpha[t])
            S = [[at * x for x in row] for row in S]
        # state read with (the gated) S_{t-1}, then rank-one write
        resid = [F(v[t][j]) - sum((S[j][i] * kt_vec[i] for i in range(dk)), F(0)) for j in range(dv)]
        for j in range(dv):
            for i in range(dk):
                S[j][i] += b * resid[j] * w[i]
        qt = [F(x) for x in q[t]]
        outs.append([sum((S[j][i] * qt[i] for i in range(dk)), F(0)) for j in range(dv)])
        kk = n if deltanet else a
        rhos.append((1 - b * kk) ** 2)
        if not deltanet:
            step = (eta * b * (1 - b * a) / n) if n != 0 else F(0)
            d = [rt * di + step * si for di, si in zip(d, sq)]
    return {"o": outs, "S": S, "d": d, "k_tilde": kts, "rho": rhos}
