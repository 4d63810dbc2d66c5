"""OSDN forward oracle (fp64, CPU) -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this module.  The GPU library never does; the two share no code.

Sources (cited as in the C file): the gist.science technical summary of
"OSDN: Improving Delta Rule with Provable Online Preconditioning in Linear
Attention" (arXiv 2605.13473) -- [summary §N] -- and its arXiv abstract.

Contents
--------
forward            token-serial recurrence, C (osdn_oracle.c) driven through ctypes
surrogate_closed   closed-form hypergradient surrogate h_t(d)         [summary §2.2]
surrogate_direct   the ratio definition of h_t, from an explicit S update [summary §2.2]
surrogate_grad     gradient in d of the closed form (derived, see its docstring)
chunked_state_pass the chunkwise (WY/UT) form of the state pass with K~ in
                   place of K in the gram and the scores           [summary §2.1]
chunked_dwalk      the preconditioner recurrence unrolled over a chunk
                   (affine in d, as the APF section notes)          [summary §2.3]
q_geo              geometric mean of the token-local residual ratios [summary §3, §4.2]
prepare_inputs     L2 normalisation of q and k per token and the logistic sigmoid
                   of gate logits, the input transforms the measured workloads
                   apply before the recurrence (plain definitions, fp64)

Every function here is pinned by tests/test_oracle_*.py against closed forms,
special cases, an exact-rational brute force or an independent formulation.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "osdn_oracle.c")
# OSDN_ORACLE_LIB names a prebuilt oracle library to load instead (the
# sanitizer test builds one with AddressSanitizer and UndefinedBehaviorSanitizer)
_LIB_ENV = os.environ.get("OSDN_ORACLE_LIB")
_LIB_PATH = _LIB_ENV or os.path.join(_HERE, "liboracle.so")
_lib = None
_lib_lock = threading.Lock()

MODES = {"osdn": 0, "deltanet": 1, "given": 2}


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (plain IEEE fp64: no fast-math, no contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
               "-ffp-contract=off", "-fno-fast-math", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lib_lock:
        if _lib is None:
            if not _LIB_ENV and (not os.path.exists(_LIB_PATH) or (
                    os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC))):
                build(force=True)
            lib = ctypes.CDLL(_LIB_PATH)
            P = ctypes.c_void_p
            lib.oracle_forward.restype = ctypes.c_int
            lib.oracle_forward.argtypes = [
                ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                ctypes.c_int, ctypes.c_double,
                P, P, P, P, P, P, P, P, P, P,  # q k v beta r d0 S0 k_given alpha alpha_k
                P, P, P, P, P, P,         # o S_final d_final k_tilde d_all rho
                P, ctypes.c_long, ctypes.c_int]
            _lib = lib
    return _lib


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor: exact widening of the stored bits
        x = x.detach().cpu().double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def prepare_inputs(q, k, beta, r=None, norm_qk=True, gate_logits=True):
    """The input transforms on the stored values, in fp64.

    norm_qk: q_t <- q_t / ||q_t||_2 and k_t <- k_t / ||k_t||_2 per token (a zero
    vector stays zero).  gate_logits: beta_t <- 1 / (1 + exp(-beta_t)), and the
    same for r_t.  Returns (q, k, beta, r) as fp64 arrays (r None if absent).
    """
    q, k, beta, r = _f64(q), _f64(k), _f64(beta), _f64(r)
    if norm_qk:
        def unit(x):
            n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
            return np.where(n > 0, x / np.where(n > 0, n, 1.0), 0.0)
        q, k = unit(q), unit(k)
    if gate_logits:
        def sig(x):
            if x is None:
                return None
            with np.errstate(over="ignore"):  # exp(-x) = inf gives 0 exactly
                return 1.0 / (1.0 + np.exp(-x))
        beta, r = sig(beta), sig(r)
    return q, k, beta, r


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def forward(q, k, v, beta, r=None, d0=None, S0=None, eta=0.0, mode="osdn",
            k_given=None, heads=None, want=("o", "S", "d", "k_tilde", "rho"),
            threads=None, alpha=None):
    """Token-serial fp64 OSDN forward.

    ``alpha`` [B,H,T] is the optional state gate (Gated DeltaNet backbone):
    S_t = alpha_t S_{t-1} + beta_t (v_t - alpha_t S_{t-1} k_t) kt_t^T.
    ``alpha`` [B,H,T,dk] is the per-channel gate (Kimi Delta Attention
    backbone): S_t = S_{t-1} D_t + beta_t (v_t - S_{t-1} D_t k_t) kt_t^T with
    D_t = diag(alpha_t), which scales the key columns of S.

    Arrays are [B,H,T,dk] (q, k, k_given), [B,H,T,dv] (v), [B,H,T] (beta, r),
    [B,H,dk] (d0), [B,H,dv,dk] (S0); anything convertible (numpy, torch CPU)
    is widened to fp64 exactly.  ``heads`` restricts the run to a list of
    flattened b*H+h indices (outputs of other heads stay zero).  ``want``
    selects outputs among o, S, d, k_tilde, d_all, rho.  Returns a dict of
    fp64 arrays.
    """
    lib = _load()
    k = _f64(k)
    B, H, T, dk = k.shape
    v = _f64(v)
    dv = v.shape[-1]
    q = _f64(q) if q is not None else None
    beta = _f64(beta)
    r = _f64(r)
    d0 = _f64(d0)
    S0 = _f64(S0)
    k_given = _f64(k_given)
    alpha = _f64(alpha)
    assert v.shape == (B, H, T, dv) and beta.shape == (B, H, T)
    alpha_k = None
    if alpha is not None and alpha.ndim == 4:
        assert alpha.shape == (B, H, T, dk)
        alpha, alpha_k = None, alpha
    if alpha is not None:
        assert alpha.shape == (B, H, T)
    if q is not None:
        assert q.shape == (B, H, T, dk)
    if r is not None:
        assert r.shape == (B, H, T)
    if d0 is not None:
        assert d0.shape == (B, H, dk)
    if S0 is not None:
        assert S0.shape == (B, H, dv, dk)
    if mode == "given":
        assert k_given is not None and k_given.shape == (B, H, T, dk)
    out = {}
    o = np.zeros((B, H, T, dv)) if ("o" in want and q is not None) else None
    Sf = np.zeros((B, H, dv, dk)) if "S" in want else None
    df = np.zeros((B, H, dk)) if "d" in want else None
    kt = np.zeros((B, H, T, dk)) if "k_tilde" in want else None
    da = np.zeros((B, H, T, dk)) if "d_all" in want else None
    rho = np.zeros((B, H, T)) if "rho" in want else None
    if heads is not None:
        hv = np.ascontiguousarray(np.asarray(heads, dtype=np.int64))
        assert hv.ndim == 1 and (hv.size == 0 or (hv.min() >= 0 and hv.max() < B * H))
        n_heads = hv.size
    else:
        hv = None
        n_heads = B * H
    nthr = threads if threads is not None else min(default_threads(), max(1, n_heads))
    rc = lib.oracle_forward(B, H, T, dk, dv, MODES[mode], float(eta),
                            _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(r), _ptr(d0),
                            _ptr(S0), _ptr(k_given), _ptr(alpha), _ptr(alpha_k),
                            _ptr(o), _ptr(Sf), _ptr(df), _ptr(kt), _ptr(da), _ptr(rho),
                            _ptr(hv), n_heads, int(nthr))
    if rc != 0:
        raise RuntimeError("oracle_forward failed (rc=%d)" % rc)
    for name, arr in (("o", o), ("S", Sf), ("d", df), ("k_tilde", kt), ("d_all", da),
                      ("rho", rho)):
        if arr is not None:
            out[name] = arr
    out["threads"] = nthr
    return out


# ---------------------------------------------------------------------------
# The hypergradient surrogate  [summary §2.2]
# ---------------------------------------------------------------------------

def inner_loss(S, k, v):
    """f_t(S) = 1/2 ||S k - v||^2, the per-token regression loss [summary §1]."""
    e = S @ k - v
    return 0.5 * float(e @ e)


def surrogate_direct(S, k, v, d, beta):
    """h_t by its definition: (f_t(S_t) - f_t(S_{t-1})) / ||grad f_t(S_{t-1})||_F^2,
    where S_t is the preconditioned write S_{t-1} + beta (v - S_{t-1} k)(d*k)^T
    [summary §2.1-2.2].  grad f_t(S) = (S k - v) k^T [summary §1]."""
    u = v - S @ k
    S_new = S + beta * np.outer(u, d * k)
    grad = np.outer(S @ k - v, k)
    return (inner_loss(S_new, k, v) - inner_loss(S, k, v)) / float(np.sum(grad * grad))


def surrogate_closed(d, k, beta):
    """h_t(d) = ((1 - beta <d, k^2>)^2 - 1) / (2 ||k||^2)  [summary §2.2]."""
    a = float(d @ (k * k))
    n = float(k @ k)
    return ((1.0 - beta * a) ** 2 - 1.0) / (2.0 * n)


def surrogate_grad(d, k, beta):
    """grad_d h_t = -beta (1 - beta <d,k^2>) k^2 / ||k||^2 (differentiating the
    closed form: d/dd of (1-beta a)^2 is -2 beta (1-beta a) k^2)."""
    a = float(d @ (k * k))
    n = float(k @ k)
    return -beta * (1.0 - beta * a) * (k * k) / n


# ---------------------------------------------------------------------------
# Chunkwise form of the state pass with K~  [summary §2.1]
# ---------------------------------------------------------------------------

def chunked_state_pass(q, k, k_tilde, v, beta, S0=None, C=64, alpha=None):
    """One (b,h) sequence, fp64, chunk length C (last chunk may be short).

    The summary states that the only change to DeltaNet's chunkwise pipeline is
    K -> K~ in the chunk gram and the intra-chunk scores.  Within a chunk with
    entry state S and rows t (pseudo-values x_t = beta_t (v_t - S_{t-1} k_t)):
        S_t = S + sum_{s<=t} x_s k~_s^T
    so  x_t + beta_t sum_{s<t} (k_t . k~_s) x_s = beta_t (v_t - S k_t), i.e.
        (I + A) X = diag(beta) (V - K S^T),   A = strict_lower(diag(beta) K K~^T)
        O  = Q S^T + lower_incl_diag(Q K~^T) X
        S' = S + X^T K~
    With the state gate alpha (S_t = alpha_t S_{t-1} + x_t k~_t^T, x_t =
    beta_t (v_t - alpha_t S_{t-1} k_t)) and gamma_t = prod_{m<=t} alpha_m within
    the chunk, S_t = gamma_t S + sum_{s<=t} (gamma_t / gamma_s) x_s k~_s^T, so
        A_ts = beta_t (gamma_t/gamma_s) k_t . k~_s (s < t),
        (I + A) X = diag(beta) (V - diag(gamma) K S^T),
        O_t = gamma_t S q_t + sum_{s<=t} (gamma_t/gamma_s) (q_t . k~_s) x_s,
        S' = gamma_L S + sum_s (gamma_L/gamma_s) x_s k~_s^T.
    With a per-channel gate (alpha [T,dk], S_t = S_{t-1} D_t + x_t k~_t^T,
    D_t = diag(alpha_t)) the decays are vectors g_t = prod_{m<=t} alpha_m, and
    S_{t-1} D_t = S diag(g_t) + sum_{s<t} x_s (k~_s (.) g_t / g_s)^T gives
        A_ts = beta_t <k_t (.) g_t, k~_s / g_s> (s < t),
        (I + A) X = diag(beta) (V - (K (.) G) S^T),
        O = (Q (.) G) S^T + lower_incl_diag((Q (.) G) (K~ / G)^T) X,
        S' = S diag(g_L) + X^T (K~ (.) g_L / G).
    (Plain fp64 division by g: for gates bounded away from zero.)
    Inputs: q, k, k_tilde [T,dk]; v [T,dv]; beta [T]; alpha [T] or [T,dk];
    S0 [dv,dk].  Returns (o [T,dv], S_final [dv,dk]).
    """
    q, k, kt, v, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, k_tilde, v, beta))
    T, dk = k.shape
    dv = v.shape[1]
    al = np.ones(T) if alpha is None else np.asarray(alpha, dtype=np.float64)
    S = np.zeros((dv, dk)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.zeros((T, dv))
    for c0 in range(0, T, C):
        sl = slice(c0, min(T, c0 + C))
        Q, K, Kt, V, bt = q[sl], k[sl], kt[sl], v[sl], beta[sl]
        if al.ndim == 2:  # one gate per key dimension
            G = np.cumprod(al[sl], axis=0)
            KG, QG, KtG = K * G, Q * G, Kt / G
            A = np.tril(bt[:, None] * (KG @ KtG.T), k=-1)
            rhs = bt[:, None] * (V - KG @ S.T)
            X = np.linalg.solve(np.eye(len(bt)) + A, rhs)
            o[sl] = QG @ S.T + np.tril(QG @ KtG.T) @ X
            S = S * G[-1][None, :] + X.T @ (Kt * (G[-1][None, :] / G))
            continue
        gam = np.cumprod(al[sl])
        ratio = gam[:, None] / gam[None, :]          # gamma_t / gamma_s
        A = np.tril(bt[:, None] * ratio * (K @ Kt.T), k=-1)
        rhs = bt[:, None] * (V - gam[:, None] * (K @ S.T))
        X = np.linalg.solve(np.eye(len(bt)) + A, rhs)
        o[sl] = gam[:, None] * (Q @ S.T) + np.tril(ratio * (Q @ Kt.T)) @ X
        S = gam[-1] * S + (X * (gam[-1] / gam)[:, None]).T @ Kt
    return o, S


# ---------------------------------------------------------------------------
# Chunked preconditioner walk  [summary §2.3: the recurrence in d is affine]
# ---------------------------------------------------------------------------

def chunked_dwalk(k, beta, r=None, d0=None, eta=0.0, C=64):
    """One (b,h) sequence, fp64.  Returns (d_all [T,dk] = d used at each token, d_final).

    Within a chunk (local index j = 0..L-1, entry vector d_0):
        d_{j+1} = r_j d_j + c_j p_j,     p_j = k_j*k_j,  n_j = ||k_j||^2,
        c_j = alpha_j (1 - beta_j a_j),  a_j = <d_j, p_j>,  alpha_j = eta beta_j / n_j (0 if n_j=0)
    Unrolling, with Gamma_j = prod_{m<j} r_m and R_{j,i} = prod_{i<m<j} r_m:
        d_j = Gamma_j d_0 + sum_{i<j} R_{j,i} c_i p_i
        a_j = Gamma_j <d_0,p_j> + sum_{i<j} R_{j,i} <p_i,p_j> c_i
    so c solves the unit lower-triangular system
        c_j + alpha_j beta_j sum_{i<j} R_{j,i} <p_i,p_j> c_i = alpha_j (1 - beta_j Gamma_j <d_0,p_j>).
    """
    k = np.asarray(k, dtype=np.float64)
    T, dk = k.shape
    beta = np.asarray(beta, dtype=np.float64)
    r = np.ones(T) if r is None else np.asarray(r, dtype=np.float64)
    d = np.ones(dk) if d0 is None else np.array(d0, dtype=np.float64)
    d_all = np.zeros((T, dk))
    for c0 in range(0, T, C):
        sl = slice(c0, min(T, c0 + C))
        K, bt, rt = k[sl], beta[sl], r[sl]
        L = len(bt)
        P = K * K
        n = P.sum(axis=1)
        alpha = np.where(n > 0, eta * bt / np.where(n > 0, n, 1.0), 0.0)
        # Gamma[j] = prod_{m<j} r_m  (j = 0..L);  R[j,i] = prod_{i<m<j} r_m  (i<j<=L)
        Gamma = np.ones(L + 1)
        for j in range(1, L + 1):
            Gamma[j] = Gamma[j - 1] * rt[j - 1]
        R = np.zeros((L + 1, L))
        for j in range(L + 1):
            for i in range(min(j, L)):
                R[j, i] = np.prod(rt[i + 1:j])
        G = P @ P.T
        M = np.zeros((L, L))
        for j in range(L):
            for i in range(j):
                M[j, i] = alpha[j] * bt[j] * R[j, i] * G[j, i]
        rhs = alpha * (1.0 - bt * Gamma[:L] * (P @ d))
        c = np.linalg.solve(np.eye(L) + M, rhs)
        for j in range(L):
            d_all[c0 + j] = Gamma[j] * d + (R[j, :j] * c[:j]) @ P[:j]
        d = Gamma[L] * d + (R[L, :] * c) @ P
    return d_all, d


def q_geo(rho):
    """Geometric mean of token-local residual ratios rho_t = f_t(S_t)/f_t(S_{t-1})
    [summary §3 defines the product, §4.2 reports its geometric mean]."""
    rho = np.asarray(rho, dtype=np.float64).ravel()
    if rho.size == 0:
        return float("nan")
    with np.errstate(divide="ignore"):
        return float(np.exp(np.mean(np.log(rho))))
