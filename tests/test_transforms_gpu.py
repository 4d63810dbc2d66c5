"""GPU parity of the in-kernel input transforms (OSDN_NORM_QK, OSDN_GATE_LOGITS):
the forward and the decoding step on raw inputs -- q, k unnormalised, beta and r
as logits -- against the fp64 oracle run on the oracle's own transforms of the
same stored values (oracle.prepare_inputs).  Tolerances are the plain ones: bf16
data o, S 2e-2 and d 1e-5; fp32 data o, S 1e-4 and d 1e-5.  Inputs come from
the seeded generators (raw draws); expected values from the oracle only.
"""
import dataclasses

import numpy as np
import pytest
import torch

import delta_rule_recurrent_precond_amd as osdn
from delta_rule_recurrent_precond_amd import _lib
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


def _heads(w, n):
    total = w.B * w.H
    if n >= total:
        return list(range(total))
    g = np.random.default_rng(w.seed + 17)
    return sorted(g.choice(total, size=n, replace=False).tolist())


def _select(x, heads, w):
    x = as_f64(x)
    return x.reshape((w.B * w.H,) + x.shape[2:])[heads]


def _check(w, inp, precond=True, heads=None, S0=None, norm_qk=True, gate_logits=True,
           gated=False):
    heads = heads if heads is not None else list(range(w.B * w.H))
    dev = inp.to("cuda")
    code = 0 if w.dtype == "bf16" else 1
    ws_n = osdn.forward_workspace_bytes(w.B, w.H, w.T, w.dk, w.dv, w.chunk, code, precond)
    _log("raw-input forward %s precond=%s path=%s" % (
        w.name, precond, osdn.forward_path(w.B, w.H, w.T, w.dk, w.dv, w.chunk, code, precond,
                                           workspace_bytes=ws_n)))
    out = osdn.forward(dev.q, dev.k, dev.v, dev.beta, dev.r, None,
                       None if S0 is None else S0.cuda(), eta=inp.eta, chunk=w.chunk,
                       precond=precond, norm_qk=norm_qk, gate_logits=gate_logits,
                       alpha=dev.alpha if gated else None)
    torch.cuda.synchronize()
    q, k, b, r = oracle.prepare_inputs(inp.q, inp.k, inp.beta, inp.r, norm_qk, gate_logits)
    ref = oracle.forward(q, k, inp.v, b, r, None, S0, eta=inp.eta,
                         mode="osdn" if precond else "deltanet", heads=heads,
                         want=("o", "S", "d", "rho"), alpha=inp.alpha if gated else None)
    tol = TOL[w.dtype]
    errs = {"o": rowwise_rel(_select(out["o"], heads, w), _select(ref["o"], heads, w)),
            "S": matrix_rel(_select(out["S_final"], heads, w), _select(ref["S"], heads, w))}
    if precond:
        errs["d"] = rowwise_rel(_select(out["d_final"], heads, w), _select(ref["d"], heads, w))
    lrs_ref = np.log(_select(ref["rho"], heads, w)).sum(axis=-1)
    lrs = _select(out["log_ratio_sum"], heads, w)
    errs["lrs"] = float(np.max(np.abs(lrs - lrs_ref) / (1e-3 + 1e-4 * np.abs(lrs_ref))))
    _log("  errors %s" % {k_: "%.3g" % v for k_, v in errs.items()})
    for name in ("o", "S", "d"):
        if name in errs:
            assert errs[name] <= tol[name], errs
    assert errs["lrs"] <= 1.0, errs


def _raw(B, H, T, dk, dv, chunk, dtype, seed, apf=True, gated=False):
    return dataclasses.replace(W.custom(B, H, T, dk, dv, chunk, dtype=dtype, eta=0.1, apf=apf,
                                        seed=seed, gated=gated), raw=True)


@pytest.mark.parametrize("precond", [True, False])
@pytest.mark.parametrize("dtype,dk,dv,chunk,T", [
    ("bf16", 128, 128, 64, 300),   # multi-launch pipeline, ragged last chunk
    ("bf16", 128, 128, 64, 64),
    ("bf16", 64, 32, 16, 150),     # two-phase path
    ("f32", 32, 64, 32, 77),
    ("f32", 128, 128, 64, 130),
])
def test_forward_raw_inputs(dtype, dk, dv, chunk, T, precond):
    w = _raw(2, 2, T, dk, dv, chunk, dtype, seed=1100 + dk + T)
    S0 = 0.1 * torch.randn(2, 2, dv, dk, generator=torch.Generator().manual_seed(8))
    _check(w, W.generate(w), precond, S0=S0)


@pytest.mark.parametrize("precond", [True, False])
@pytest.mark.parametrize("dtype,dk,dv,chunk,T", [
    ("bf16", 128, 128, 64, 300),   # multi-launch pipeline with the state gate
    ("bf16", 128, 128, 64, 2048),  # the same, 30 of 32 chunks prepared in the walk's launch
    ("f32", 32, 64, 32, 77),       # two-phase path
])
def test_gated_forward_raw_inputs(dtype, dk, dv, chunk, T, precond):
    """Raw inputs with the state gate (OSDN on Gated DeltaNet; Gated DeltaNet
    itself without the preconditioner)."""
    w = _raw(2, 2, T, dk, dv, chunk, dtype, seed=1190 + dk + T, gated=True)
    S0 = 0.1 * torch.randn(2, 2, dv, dk, generator=torch.Generator().manual_seed(9))
    _check(w, W.generate(w), precond, S0=S0, gated=True)


@pytest.mark.parametrize("norm_qk,gate_logits", [(True, False), (False, True)])
def test_each_transform_alone(norm_qk, gate_logits):
    w = _raw(1, 2, 200, 128, 128, 64, "bf16", seed=1150)
    inp = W.generate(w)
    if not norm_qk:   # keys given normalised, gates given as logits
        q, k, _, _ = oracle.prepare_inputs(inp.q, inp.k, inp.beta, inp.r, True, False)
        inp = dataclasses.replace(inp, q=torch.from_numpy(q).to(torch.bfloat16),
                                  k=torch.from_numpy(k).to(torch.bfloat16))
    else:             # gates given as values
        _, _, b, r = oracle.prepare_inputs(inp.q, inp.k, inp.beta, inp.r, False, True)
        inp = dataclasses.replace(inp, beta=torch.from_numpy(b).float(),
                                  r=torch.from_numpy(r).float())
    _check(w, inp, norm_qk=norm_qk, gate_logits=gate_logits)


def test_zero_key_rows_stay_zero():
    w = _raw(1, 2, 130, 128, 128, 64, "bf16", seed=1160)
    inp = W.generate(w)
    k = inp.k.clone()
    k[:, :, 7] = 0
    k[:, :, 64] = 0
    _check(w, dataclasses.replace(inp, k=k))


def test_fused_only_shapes_refuse_transforms():
    w = _raw(1, 1, 64, 128, 128, 64, "bf16", seed=1170)
    dev = W.generate(w).to("cuda")
    with pytest.raises(osdn.OsdnError) as e:
        osdn.forward(dev.q, dev.k, dev.v, dev.beta, dev.r, eta=0.1, chunk=64, workspace=None,
                     norm_qk=True)
    assert e.value.status == _lib.OSDN_ERR_UNSUPPORTED
    assert osdn.forward_path(1, 1, 64, 128, 128, 64, 0) == "fused"


@pytest.mark.parametrize("dtype,dk,dv", [("f32", 32, 64), ("bf16", 128, 128)])
def test_step_raw_inputs(dtype, dk, dv):
    T = 10
    w = _raw(2, 3, T, dk, dv, 16, dtype, seed=1180 + dk)
    inp = W.generate(w)
    g = torch.Generator().manual_seed(14)
    S0 = 0.1 * torch.randn(w.B, w.H, dv, dk, generator=g)
    d0 = 0.5 + torch.rand(w.B, w.H, dk, generator=g)
    q, k, b, r = oracle.prepare_inputs(inp.q, inp.k, inp.beta, inp.r)
    ref = oracle.forward(q, k, inp.v, b, r, d0, S0, eta=inp.eta, want=("o", "S", "d"))
    dev = inp.to("cuda")
    S, d = S0.clone().cuda(), d0.clone().cuda()
    tok = lambda x, t: x[:, :, t].contiguous()
    os_ = [osdn.step(tok(dev.q, t), tok(dev.k, t), tok(dev.v, t), tok(dev.beta, t), S, d,
                     tok(dev.r, t), eta=inp.eta, norm_qk=True, gate_logits=True)["o"]
           for t in range(T)]
    o = torch.stack(os_, dim=2)
    torch.cuda.synchronize()
    assert rowwise_rel(o, ref["o"]) <= (1e-5 if dtype == "f32" else 2.0 ** -8)
    assert matrix_rel(S, ref["S"]) <= 1e-5
    assert rowwise_rel(d, ref["d"]) <= 1e-5


@pytest.mark.slow
def test_raw_workload_full_size():
    """The 1.3B-style layer drawn raw, at full size, every (b,h) compared."""
    w = dataclasses.replace(W.CONFIGS["1.3b-apf"], raw=True)
    _check(w, W.generate(w), heads=_heads(w, w.B * w.H))
