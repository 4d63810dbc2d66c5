"""GPU parity of the per-channel state gate (OSDN on the Kimi Delta Attention
backbone) against the fp64 oracle, through the C ABI.

The pages evaluate OSDN on KDA without printing its update; both sides
implement the reading
    S_t = S_{t-1} D_t + beta_t (v_t - S_{t-1} D_t k_t) kt_t^T,  D_t = diag(alpha_t),
with the preconditioner walk unchanged.  On the matrix-core shapes
osdn_forward runs the multi-launch pipeline given its workspace (tiles below
the diagonal factored through block boundaries, diagonal blocks term by term)
and the two-phase path given less scratch than that pipeline needs; on other shapes the
two-phase path (the vector chunk kernel applies the per-channel decays term by
term).  osdn_step scales each column of S.  Tolerances are the gated ones:
fp32 data o, S 1e-4 and d 1e-5; bf16 data o, S 2e-2 and d 1e-5.  Inputs come from the seeded generators;
expected values from the oracle only.
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


def _kda(B, H, T, dk, dv, chunk, dtype, seed, **kw):
    return W.custom(B, H, T, dk, dv, chunk, dtype=dtype, eta=0.1, apf=True, seed=seed,
                    gated=True, gate_channels=True, **kw)


def _heads(w, n):
    total = w.B * w.H
    if n >= total:
        return list(range(total))
    g = np.random.default_rng(w.seed + 17)
    return sorted(g.choice(total, size=n, replace=False).tolist())


def _select(x, heads, w):
    x = as_f64(x)
    return x.reshape((w.B * w.H,) + x.shape[2:])[heads]


def _check(w, inp, precond=True, S0=None, heads=None, alpha=None, q=None, norm_qk=False,
           gate_logits=False, ws=True):
    alpha = inp.alpha if alpha is None else alpha
    q = inp.q if q is None else q
    heads = heads if heads is not None else list(range(w.B * w.H))
    dev = inp.to("cuda")
    code = 0 if w.dtype == "bf16" else 1
    if ws == "two-phase":  # one byte short of the split pipeline's scratch: the two-phase path
        n = osdn.forward_workspace_bytes(w.B, w.H, w.T, w.dk, w.dv, w.chunk, code, precond,
                                         per_channel=True)
        ws = torch.empty(max(n - 1, 1), dtype=torch.uint8, device="cuda")
    nbytes = (osdn.forward_workspace_bytes(w.B, w.H, w.T, w.dk, w.dv, w.chunk, code, precond,
                                           per_channel=True) if ws is True else ws.numel())
    _log("per-channel forward %s precond=%s heads=%d path=%s" % (
        w.name, precond, len(heads),
        osdn.forward_path(w.B, w.H, w.T, w.dk, w.dv, w.chunk, code, precond,
                          workspace_bytes=nbytes, per_channel=True)))
    out = osdn.forward(q.cuda(), dev.k, dev.v, dev.beta, dev.r, None,
                       None if S0 is None else S0.cuda(), eta=inp.eta, chunk=w.chunk,
                       precond=precond, alpha=alpha.cuda(), norm_qk=norm_qk,
                       gate_logits=gate_logits, workspace=ws)
    torch.cuda.synchronize()
    qq, kk, bb, rr = oracle.prepare_inputs(q, inp.k, inp.beta, inp.r, norm_qk, gate_logits)
    ref = oracle.forward(qq, kk, inp.v, bb, rr, None, S0, eta=inp.eta,
                         mode="osdn" if precond else "deltanet", heads=heads,
                         want=("o", "S", "d", "rho"), alpha=alpha)
    tol = TOL[w.dtype]
    errs = {"o": rowwise_rel(_select(out["o"], heads, w), _select(ref["o"], heads, w)),
            "S": matrix_rel(_select(out["S_final"], heads, w), _select(ref["S"], heads, w))}
    if precond:
        errs["d"] = rowwise_rel(_select(out["d_final"], heads, w), _select(ref["d"], heads, w))
    lrs_ref = np.log(_select(ref["rho"], heads, w)).sum(axis=-1)
    lrs = _select(out["log_ratio_sum"], heads, w)
    errs["lrs"] = float(np.max(np.abs(lrs - lrs_ref) / (1e-3 + 1e-4 * np.abs(lrs_ref))))
    _log("  errors %s" % {k: "%.3g" % v for k, v in errs.items()})
    for name in ("o", "S", "d"):
        if name in errs:
            assert errs[name] <= tol[name], errs
    assert errs["lrs"] <= 1.0, errs
    return out


@pytest.mark.parametrize("dtype,dk,dv,chunk,T", [
    ("bf16", 128, 128, 64, 300),   # the layer shape, ragged last chunk
    ("bf16", 64, 32, 16, 150),
    ("f32", 16, 16, 16, 100),
    ("f32", 32, 64, 32, 77),
    ("f32", 128, 128, 64, 130),
])
@pytest.mark.parametrize("precond", [True, False])
@pytest.mark.parametrize("ws", [True, "two-phase"])
def test_forward_per_channel_parity(dtype, dk, dv, chunk, T, precond, ws):
    if ws != True and not (dtype == "bf16" and dk == 128):  # noqa: E712
        pytest.skip("only the matrix-core shapes have a second path")
    w = _kda(2, 2, T, dk, dv, chunk, dtype, seed=1200 + dk + dv + T)
    S0 = 0.1 * torch.randn(w.B, w.H, dv, dk, generator=torch.Generator().manual_seed(4))
    _check(w, W.generate(w), precond, S0=S0, ws=ws)


@pytest.mark.parametrize("T", [1, 63, 64, 129])
@pytest.mark.parametrize("ws", [True, "two-phase"])
def test_forward_per_channel_chunk_boundaries(T, ws):
    w = _kda(1, 2, T, 128, 128, 64, "bf16", seed=1250 + T)
    _check(w, W.generate(w), ws=ws)


def test_strong_decay_and_zero_channel_gates():
    """Gates spread over (0, 1), some channels closed at single tokens (a column
    reset), and every channel closed at chunk edges."""
    w = _kda(2, 2, 200, 64, 64, 64, "f32", seed=1261, alpha_mu=0.0, alpha_sigma=2.0)
    inp = W.generate(w)
    alpha = inp.alpha.clone()
    alpha[:, :, 5, :7] = 0.0
    alpha[:, :, 64, 10:] = 0.0    # first token of a chunk
    alpha[:, :, 127] = 0.0        # last token of a chunk, every channel
    S0 = torch.randn(w.B, w.H, 64, 64, generator=torch.Generator().manual_seed(5))
    for p in (True, False):
        _check(w, inp, precond=p, S0=S0, alpha=alpha)
    wb = _kda(1, 2, 150, 128, 128, 64, "bf16", seed=1262, alpha_mu=0.0, alpha_sigma=2.0)
    inpb = W.generate(wb)
    ab = inpb.alpha.clone()
    ab[:, :, 70, ::3] = 0.0       # some channels closed inside a 16-token block
    ab[:, :, 80, 1::3] = 0.0      # first token of a block
    ab[:, :, 127, :] = 0.0        # last token of a chunk, every channel
    for ws in (True, "two-phase"):
        for p in (True, False):
            _check(wb, inpb, precond=p, alpha=ab, ws=ws)


@pytest.mark.parametrize("dtype,dk", [("f32", 32), ("bf16", 128)])
def test_equal_channels_match_the_scalar_gate(dtype, dk):
    """Per-channel gates equal across channels are the scalar gate: the
    per-channel forward matches the oracle's scalar-gated run."""
    w = W.custom(2, 2, 140, dk, dk, 32 if dtype == "f32" else 64, dtype=dtype, eta=0.1, apf=True,
                 seed=1270 + dk, gated=True)
    inp = W.generate(w)
    wide = inp.alpha[..., None].expand(-1, -1, -1, dk).contiguous()
    dev = inp.to("cuda")
    out = osdn.forward(dev.q, dev.k, dev.v, dev.beta, dev.r, eta=inp.eta, chunk=w.chunk,
                       alpha=wide.cuda())
    torch.cuda.synchronize()
    ref = oracle.forward(inp.q, inp.k, inp.v, inp.beta, inp.r, eta=inp.eta, want=("o", "S", "d"),
                         alpha=inp.alpha)
    tol = TOL[dtype]
    assert rowwise_rel(out["o"], ref["o"]) <= tol["o"]
    assert matrix_rel(out["S_final"], ref["S"]) <= tol["S"]
    assert rowwise_rel(out["d_final"], ref["d"]) <= tol["d"]


@pytest.mark.parametrize("precond", [True, False])
@pytest.mark.parametrize("ws", [True, "two-phase"])
def test_per_channel_raw_inputs(precond, ws):
    """Per-channel gate with the in-kernel input transforms."""
    w = dataclasses.replace(_kda(2, 2, 170, 128, 128, 64, "bf16", seed=1280), raw=True)
    _check(w, W.generate(w), precond, norm_qk=True, gate_logits=True, ws=ws)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("precond", [True, False])
def test_unit_channel_gates_equal_ungated_bitwise(dtype, precond):
    """alpha = 1 in every channel: every decay product is exactly 1, so the
    per-channel kernels agree with the ungated run of the same path up to
    their own rounding (they sum the products in another order: fp32 rounding
    on the vector path, fp16-operand rounding on the multi-launch pipeline),
    and the preconditioner walk, which the gate does not reach, is bitwise
    the same."""
    dk = 128 if dtype == "bf16" else 32
    w = W.custom(2, 2, 150, dk, dk, 64 if dtype == "bf16" else 32, dtype=dtype, eta=0.1,
                 apf=True, seed=1285)
    inp = W.generate(w)
    dev = inp.to("cuda")
    ones = torch.ones(w.B, w.H, w.T, dk, device="cuda")
    a = osdn.forward(dev.q, dev.k, dev.v, dev.beta, dev.r, eta=inp.eta, chunk=w.chunk,
                     precond=precond)
    b = osdn.forward(dev.q, dev.k, dev.v, dev.beta, dev.r, eta=inp.eta, chunk=w.chunk,
                     precond=precond, alpha=ones)
    torch.cuda.synchronize()
    tol = 1e-5 if dtype == "f32" else 1e-2
    assert rowwise_rel(b["o"], a["o"]) <= tol
    assert matrix_rel(b["S_final"], a["S_final"]) <= tol
    if precond:
        assert torch.equal(a["d_final"], b["d_final"])
    assert torch.equal(a["log_ratio_sum"], b["log_ratio_sum"])


@pytest.mark.parametrize("dtype,dk,dv,chunk,T", [("bf16", 128, 128, 64, 300),
                                                 ("bf16", 128, 128, 64, 64),
                                                 ("f32", 64, 32, 32, 97)])
@pytest.mark.parametrize("ws", [True, None])
def test_chunk_fwd_per_channel_given_ktilde(dtype, dk, dv, chunk, T, ws):
    """osdn_chunk_fwd with the per-channel gate: the two-kernel pass given its
    workspace, the vector chunk kernel without."""
    w = _kda(2, 2, T, dk, dv, chunk, dtype, seed=1300 + T)
    inp = W.generate(w)
    S0 = 0.1 * torch.randn(w.B, w.H, dv, dk, generator=torch.Generator().manual_seed(6))
    kt_ref = oracle.forward(inp.q, inp.k, inp.v, inp.beta, inp.r, eta=inp.eta,
                            want=("k_tilde",))["k_tilde"]
    kt = torch.from_numpy(kt_ref).to(inp.k.dtype)
    dev = inp.to("cuda")
    _log("per-channel chunk %s workspace=%s" % (w.name, ws))
    o, S = osdn.chunk_fwd(dev.q, dev.k, kt.cuda(), dev.v, dev.beta, S0.cuda(), chunk,
                          alpha=dev.alpha, workspace=ws)
    torch.cuda.synchronize()
    ref = oracle.forward(inp.q, inp.k, inp.v, inp.beta, None, None, S0, mode="given",
                         k_given=kt, want=("o", "S"), alpha=inp.alpha)
    tol = TOL[dtype]
    assert rowwise_rel(o, ref["o"]) <= tol["o"]
    assert matrix_rel(S, ref["S"]) <= tol["S"]


@pytest.mark.parametrize("dtype,dk,dv", [("f32", 32, 64), ("bf16", 128, 128)])
def test_per_channel_steps_match_oracle(dtype, dk, dv):
    T = 12
    w = _kda(2, 3, T, dk, dv, 16, dtype, seed=1290 + dk)
    inp = W.generate(w)
    g = torch.Generator().manual_seed(13)
    S0 = 0.1 * torch.randn(w.B, w.H, dv, dk, generator=g)
    d0 = 0.5 + torch.rand(w.B, w.H, dk, generator=g)
    ref = oracle.forward(inp.q, inp.k, inp.v, inp.beta, inp.r, d0, S0, eta=inp.eta,
                         want=("o", "S", "d"), alpha=inp.alpha)
    dev = inp.to("cuda")
    S, d = S0.clone().cuda(), d0.clone().cuda()
    _log("per-channel steps %s" % w.name)
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


def test_per_channel_steps_continue_a_forward():
    w = _kda(2, 2, 70, 128, 128, 64, "bf16", seed=1295)
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
@pytest.mark.parametrize("ws", [True, "two-phase"])
def test_per_channel_workload_full_size(ws):
    """The 1.3B-style layer with per-channel gates at full size, every (b,h) compared."""
    w = W.CONFIGS["1.3b-apf-kda"]
    inp = W.generate(w)
    _check(w, inp, heads=_heads(w, w.B * w.H), ws=ws)
