"""GPU parity of the state gate alpha (OSDN on the Gated DeltaNet backbone)
against the fp64 oracle, through the C ABI.

The pages evaluate OSDN on Gated DeltaNet [summary §4] without printing its
update; both sides implement the reading
    S_t = alpha_t S_{t-1} + beta_t (v_t - alpha_t S_{t-1} k_t) kt_t^T
with the preconditioner walk unchanged.  The kernels use the chunk form with
cumulative decays gamma_t / gamma_s = 2^(lg_t - lg_s); the oracle runs the
token recurrence.  Tolerances are the ungated ones (the decays are <= 1 and
only shrink the terms they touch): fp32 data o, S 1e-4 and d 1e-5; bf16 data
o, S 2e-2 and d 1e-5.  Inputs come from the seeded generators; expected values
from the oracle only.  The matrix-core shapes run both paths: the multi-launch
pipeline (the default workspace) and the single fused kernel (workspace=None).
"""
import dataclasses

import numpy as np
import pytest
import torch

import delta_rule_recurrent_precond_amd as osdn
from delta_rule_recurrent_precond_amd import workloads as W
from oracle import oracle

from _helpers import as_f64, matrix_rel, rowwise_rel

pytestmark = pytest.mark.gpu

TOL = {"f32": dict(d=1e-5, o=1e-4, S=1e-4), "bf16": dict(d=1e-5, o=2e-2, S=2e-2)}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    osdn.load()
    torch.cuda.init()


def _log(msg):
    print(msg, flush=True)


def _gated(B, H, T, dk, dv, chunk, dtype, apf=True, seed=0, **kw):
    return W.custom(B, H, T, dk, dv, chunk, dtype=dtype, eta=0.1, apf=apf, seed=seed,
                    gated=True, **kw)


def _heads(w, n):
    total = w.B * w.H
    if n >= total:
        return list(range(total))
    g = np.random.default_rng(w.seed + 17)
    return sorted(g.choice(total, size=n, replace=False).tolist())


def _select(x, heads, w):
    x = as_f64(x)
    return x.reshape((w.B * w.H,) + x.shape[2:])[heads]


def _check(w, inp, precond=True, S0=None, heads=None, alpha=None, ws=True):
    alpha = inp.alpha if alpha is None else alpha
    heads = heads if heads is not None else list(range(w.B * w.H))
    dev = inp.to("cuda")
    _log("gated forward %s precond=%s heads=%d workspace=%s" % (w.name, precond, len(heads), ws))
    out = osdn.forward(dev.q, dev.k, dev.v, dev.beta, dev.r, None,
                       None if S0 is None else S0.cuda(), eta=inp.eta, chunk=w.chunk,
                       precond=precond, alpha=alpha.cuda(), workspace=ws)
    torch.cuda.synchronize()
    ref = oracle.forward(inp.q, inp.k, inp.v, inp.beta, inp.r, None, S0, eta=inp.eta,
                         mode="osdn" if precond else "deltanet", heads=heads,
                         want=("o", "S", "d"), alpha=alpha)
    tol = TOL[w.dtype]
    errs = {"o": rowwise_rel(_select(out["o"], heads, w), _select(ref["o"], heads, w)),
            "S": matrix_rel(_select(out["S_final"], heads, w), _select(ref["S"], heads, w))}
    if precond:
        errs["d"] = rowwise_rel(_select(out["d_final"], heads, w), _select(ref["d"], heads, w))
    _log("  errors %s" % {k: "%.3g" % v for k, v in errs.items()})
    for name, e in errs.items():
        assert e <= tol[name], errs
    return out


@pytest.mark.parametrize("dtype,dk,dv,chunk,T", [
    ("bf16", 128, 128, 64, 300),   # matrix-core kernel, ragged last chunk
    ("bf16", 128, 128, 64, 65),
    ("bf16", 64, 32, 16, 150),     # vector-ALU chunk kernel
    ("f32", 16, 16, 16, 100),
    ("f32", 32, 64, 32, 77),
    ("f32", 128, 128, 64, 130),
])
@pytest.mark.parametrize("precond", [True, False])
@pytest.mark.parametrize("ws", [True, None])
def test_forward_gated_parity(dtype, dk, dv, chunk, T, precond, ws):
    if ws is None and dk != 128:
        pytest.skip("only the matrix-core shapes have a second path")
    w = _gated(2, 2, T, dk, dv, chunk, dtype, seed=900 + dk + dv + T)
    inp = W.generate(w)
    S0 = 0.1 * torch.randn(w.B, w.H, dv, dk, generator=torch.Generator().manual_seed(4))
    _check(w, inp, precond, S0=S0, ws=ws)


@pytest.mark.parametrize("T", [1, 63, 64, 129])
@pytest.mark.parametrize("ws", [True, None])
def test_forward_gated_chunk_boundaries(T, ws):
    w = _gated(1, 2, T, 128, 128, 64, "bf16", seed=950 + T)
    _check(w, W.generate(w), ws=ws)


@pytest.mark.parametrize("ws", [True, None])
def test_strong_decay_and_zero_gates(ws):
    """Gates spread over (0, 1) with some exact zeros (a state reset: the state
    before such a token is forgotten)."""
    w = _gated(2, 2, 200, 128, 128, 64, "bf16", seed=961, alpha_mu=0.0, alpha_sigma=2.0)
    inp = W.generate(w)
    alpha = inp.alpha.clone()
    alpha[:, :, 5] = 0.0
    alpha[:, :, 64] = 0.0     # first token of a chunk
    alpha[:, :, 127] = 0.0    # last token of a chunk
    S0 = torch.randn(w.B, w.H, 128, 128, generator=torch.Generator().manual_seed(5))
    _check(w, inp, S0=S0, alpha=alpha, ws=ws)
    # every token resets the state: o_t = beta_t (q_t . kt_t) v_t.  With q = k the
    # factor is sum_i d_i k_i^2 > 0, so no row of o is a cancelling dot product
    # (whose row-relative error would measure one fp16 rounding, not the pass)
    rec = dataclasses.replace(inp, q=inp.k)
    for p in (True, False):
        _check(w, rec, precond=p, S0=S0, alpha=torch.zeros_like(alpha), ws=ws)
    wf = _gated(1, 2, 90, 32, 32, 16, "f32", seed=962, alpha_mu=0.0, alpha_sigma=2.0)
    inpf = W.generate(wf)
    af = inpf.alpha.clone()
    af[:, :, 0] = 0.0
    af[:, :, 40] = 0.0
    _check(wf, inpf, alpha=af)


@pytest.mark.parametrize("dtype,dk,chunk", [("bf16", 128, 64), ("f32", 32, 16)])
@pytest.mark.parametrize("precond", [True, False])
@pytest.mark.parametrize("ws", [True, None])
def test_unit_gate_equals_ungated_bitwise(dtype, dk, chunk, precond, ws):
    """alpha = 1 gives decays of exactly 1, so the gated kernels reproduce the
    ungated results of the same path bit for bit."""
    if ws is None and dtype == "f32":
        pytest.skip("the fp32 path needs its workspace")
    w = W.custom(2, 2, 150, dk, dk, chunk, dtype=dtype, eta=0.1, apf=True, seed=970 + dk)
    inp = W.generate(w)
    dev = inp.to("cuda")
    ones = torch.ones(w.B, w.H, w.T, device="cuda")
    a = osdn.forward(dev.q, dev.k, dev.v, dev.beta, dev.r, eta=inp.eta, chunk=chunk,
                     precond=precond, workspace=ws)
    b = osdn.forward(dev.q, dev.k, dev.v, dev.beta, dev.r, eta=inp.eta, chunk=chunk,
                     precond=precond, alpha=ones, workspace=ws)
    torch.cuda.synchronize()
    for name in ("o", "S_final", "d_final", "log_ratio_sum"):
        if a.get(name) is not None:
            assert torch.equal(a[name], b[name]), name


@pytest.mark.parametrize("dtype,dk,dv,chunk,T", [("bf16", 128, 128, 64, 300),
                                                 ("bf16", 128, 128, 64, 64),
                                                 ("f32", 64, 32, 32, 97)])
@pytest.mark.parametrize("ws", [True, None])
def test_chunk_fwd_gated_given_ktilde(dtype, dk, dv, chunk, T, ws):
    w = _gated(2, 2, T, dk, dv, chunk, dtype, seed=980 + T)
    inp = W.generate(w)
    S0 = 0.1 * torch.randn(w.B, w.H, dv, dk, generator=torch.Generator().manual_seed(6))
    kt_ref = oracle.forward(inp.q, inp.k, inp.v, inp.beta, inp.r, eta=inp.eta,
                            want=("k_tilde",))["k_tilde"]
    kt = torch.from_numpy(kt_ref).to(inp.k.dtype)
    dev = inp.to("cuda")
    _log("gated chunk %s" % w.name)
    o, S = osdn.chunk_fwd(dev.q, dev.k, kt.cuda(), dev.v, dev.beta, S0.cuda(), chunk,
                          alpha=dev.alpha, workspace=ws)
    torch.cuda.synchronize()
    ref = oracle.forward(inp.q, inp.k, inp.v, inp.beta, None, None, S0, mode="given",
                         k_given=kt, want=("o", "S"), alpha=inp.alpha)
    tol = TOL[dtype]
    assert rowwise_rel(o, ref["o"]) <= tol["o"]
    assert matrix_rel(S, ref["S"]) <= tol["S"]


def test_chunk_fwd_gated_unit_gate_bitwise():
    """The chunk-parallel pass with alpha = 1 reproduces its ungated results bit
    for bit (given keys and kt = k alike)."""
    w = _gated(1, 2, 200, 128, 128, 64, "bf16", seed=985)
    inp = W.generate(w)
    dev = inp.to("cuda")
    n = osdn.chunk_fwd_workspace_bytes(w.B, w.H, w.T, 128, 128, 64, 0)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    ones = torch.ones(w.B, w.H, w.T, device="cuda")
    for kt in (dev.k, dev.q):
        a = osdn.chunk_fwd(dev.q, dev.k, kt, dev.v, dev.beta, None, 64, alpha=ones, workspace=ws)
        b = osdn.chunk_fwd(dev.q, dev.k, kt, dev.v, dev.beta, None, 64, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("dtype,dk,dv", [("f32", 32, 64), ("bf16", 128, 128)])
def test_gated_steps_match_oracle(dtype, dk, dv):
    T = 12
    w = _gated(2, 3, T, dk, dv, 16, dtype, seed=990 + dk)
    inp = W.generate(w)
    g = torch.Generator().manual_seed(13)
    S0 = 0.1 * torch.randn(w.B, w.H, dv, dk, generator=g)
    d0 = 0.5 + torch.rand(w.B, w.H, dk, generator=g)
    ref = oracle.forward(inp.q, inp.k, inp.v, inp.beta, inp.r, d0, S0, eta=inp.eta,
                         want=("o", "S", "d"), alpha=inp.alpha)
    dev = inp.to("cuda")
    S, d = S0.clone().cuda(), d0.clone().cuda()
    _log("gated steps %s" % w.name)
    tok = lambda x, t: x[:, :, t].contiguous()
    os_ = []
    for t in range(T):
        os_.append(osdn.step(tok(dev.q, t), tok(dev.k, t), tok(dev.v, t), tok(dev.beta, t), S, d,
                             tok(dev.r, t), eta=inp.eta, alpha=tok(dev.alpha, t))["o"])
    o = torch.stack(os_, dim=2)
    torch.cuda.synchronize()
    assert rowwise_rel(o, ref["o"]) <= (1e-5 if dtype == "f32" else 2.0 ** -8)
    assert matrix_rel(S, ref["S"]) <= 1e-5
    assert rowwise_rel(d, ref["d"]) <= 1e-5


def test_gated_steps_continue_a_gated_forward():
    w = _gated(2, 2, 70, 128, 128, 64, "bf16", seed=995)
    inp = W.generate(w)
    dev = inp.to("cuda")
    cut = lambda x: x[:, :, :64].contiguous()
    out = osdn.forward(cut(dev.q), cut(dev.k), cut(dev.v), cut(dev.beta), cut(dev.r),
                       eta=inp.eta, chunk=64, alpha=cut(dev.alpha))
    S, d = out["S_final"], out["d_final"]
    tok = lambda x, t: x[:, :, t].contiguous()
    for t in range(64, 70):
        osdn.step(tok(dev.q, t), tok(dev.k, t), tok(dev.v, t), tok(dev.beta, t), S, d,
                  tok(dev.r, t), eta=inp.eta, alpha=tok(dev.alpha, t))
    torch.cuda.synchronize()
    ref = oracle.forward(inp.q, inp.k, inp.v, inp.beta, inp.r, eta=inp.eta, want=("S", "d"),
                         alpha=inp.alpha)
    assert matrix_rel(S, ref["S"]) <= 2e-2
    assert rowwise_rel(d, ref["d"]) <= 1e-5


@pytest.mark.slow
@pytest.mark.parametrize("ws", [True, None])
def test_gated_workload_full_size(ws):
    """The gated 1.3B-style layer at full size, every (b,h) compared."""
    w = W.CONFIGS["1.3b-apf-gated"]
    inp = W.generate(w)
    _check(w, inp, heads=_heads(w, w.B * w.H), ws=ws)
