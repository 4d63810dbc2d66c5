"""Inputs far from unit scale, on every path that uses the matrix cores.

The matrix cores take fp16 operands (range about 6e-5 .. 6.5e4).  The kernels
keep every operand inside that range whatever the inputs' scale: values are
staged in bf16 (exact) and the pseudo-values and the fp16 copy of the state are
divided by per-chunk powers of two; raw q and k (OSDN_NORM_QK) are staged
divided by a power of two per chunk and normalised in fp32; the walk's key
gram is formed from keys divided by a power of two.  Dividing by a power of
two keeps the significand, so none of this changes how anything rounds.

  - v scaled by 2^-20 and 2^17 (about 1e-6 and 1.3e5; the scaled bf16 values are
    exact): the recurrence is linear in (v, S), so o and S scale with v and the
    relative errors must stay at the bar.
  - raw q and k scaled by 2^10 and 2^-17 with OSDN_NORM_QK: the normalisation
    makes the method independent of their scale.

Every case is checked against the fp64 oracle on the same stored inputs, at
the bf16 bar (o, S 2e-2; d 1e-5).
"""
import numpy as np
import pytest
import torch

import delta_rule_recurrent_precond_amd as osdn
from delta_rule_recurrent_precond_amd import workloads as W
from oracle import oracle

from _helpers import matrix_rel, rowwise_rel

pytestmark = pytest.mark.gpu

TOL = dict(o=2e-2, S=2e-2, d=1e-5)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    osdn.load()


def _log(msg):
    print(msg, flush=True)


def _scaled(x, scale):
    """x times a power of two, stored in x's dtype (exact while in range)."""
    y = (x.double() * scale).to(x.dtype)
    assert torch.equal(y.double() / scale, x.double()), "scaling must be exact"
    return y


def _errors(out, ref, precond=True):
    errs = {"o": rowwise_rel(out["o"], ref["o"]), "S": matrix_rel(out["S_final"], ref["S"])}
    if precond:
        errs["d"] = rowwise_rel(out["d_final"], ref["d"])
    return errs


@pytest.mark.parametrize("scale", [2.0 ** -20, 2.0 ** 17])
@pytest.mark.parametrize("ws", [True, None])  # the split pipeline, the single fused kernel
@pytest.mark.parametrize("precond", [True, False])
def test_forward_value_scale(scale, ws, precond):
    w = W.custom(1, 2, 200, 128, 128, 64, dtype="bf16", eta=0.05, apf=True, seed=2201)
    inp = W.generate(w)
    v = _scaled(inp.v, scale)
    S0 = (0.05 * scale) * torch.randn(w.B, w.H, w.dv, w.dk,
                                      generator=torch.Generator().manual_seed(3))
    dev = inp.to("cuda")
    code = 0
    n = osdn.forward_workspace_bytes(w.B, w.H, w.T, w.dk, w.dv, w.chunk, code, precond)
    _log("value scale %g path=%s precond=%s" % (
        scale, osdn.forward_path(w.B, w.H, w.T, w.dk, w.dv, w.chunk, code, precond,
                                 workspace_bytes=n if ws else 0), precond))
    out = osdn.forward(dev.q, dev.k, v.cuda(), dev.beta, dev.r, None, S0.cuda(), eta=inp.eta,
                       chunk=w.chunk, precond=precond, workspace=ws)
    torch.cuda.synchronize()
    ref = oracle.forward(inp.q, inp.k, v, inp.beta, inp.r, None, S0, eta=inp.eta,
                         mode="osdn" if precond else "deltanet", want=("o", "S", "d"))
    errs = _errors(out, ref, precond)
    _log("  errors %s" % {k: "%.3g" % x for k, x in errs.items()})
    for name, e in errs.items():
        assert e <= TOL[name], errs


@pytest.mark.parametrize("scale", [2.0 ** -20, 2.0 ** 17])
@pytest.mark.parametrize("ws", [True, None])  # chunk_prep + chunk_state, the single kernel
def test_chunk_fwd_value_scale(scale, ws):
    w = W.custom(2, 2, 150, 128, 128, 64, dtype="bf16", eta=0.1, apf=True, seed=2202)
    inp = W.generate(w)
    v = _scaled(inp.v, scale)
    ref_kt = oracle.forward(inp.q, inp.k, inp.v, inp.beta, inp.r, eta=inp.eta,
                            want=("k_tilde",))["k_tilde"]
    kt = torch.from_numpy(ref_kt).to(torch.bfloat16)
    dev = inp.to("cuda")
    o, S = osdn.chunk_fwd(dev.q, dev.k, kt.cuda(), v.cuda(), dev.beta, None, 64,
                          workspace=True if ws else None)
    torch.cuda.synchronize()
    ref = oracle.forward(inp.q, inp.k, v, inp.beta, None, eta=0.0, mode="given", k_given=kt,
                         want=("o", "S"))
    errs = {"o": rowwise_rel(o, ref["o"]), "S": matrix_rel(S, ref["S"])}
    _log("chunk_fwd value scale %g ws=%s errors %s" % (scale, ws, errs))
    assert errs["o"] <= TOL["o"] and errs["S"] <= TOL["S"], errs


@pytest.mark.parametrize("scale", [2.0 ** 10, 2.0 ** -17])
@pytest.mark.parametrize("shape", [(128, 128, 64), (64, 32, 16)])  # split, two-phase
@pytest.mark.parametrize("precond", [True, False])
def test_raw_query_key_scale(scale, shape, precond):
    dk, dv, chunk = shape
    w = W.custom(2, 2, 190, dk, dv, chunk, dtype="bf16", eta=0.05, apf=True, seed=2203 + dk,
                 raw=True)
    inp = W.generate(w)
    q, k = _scaled(inp.q, scale), _scaled(inp.k, scale)
    dev = inp.to("cuda")
    code = 0
    n = osdn.forward_workspace_bytes(w.B, w.H, w.T, w.dk, w.dv, w.chunk, code, precond)
    _log("raw q, k scale %g dk=%d path=%s precond=%s" % (
        scale, dk, osdn.forward_path(w.B, w.H, w.T, w.dk, w.dv, w.chunk, code, precond,
                                     workspace_bytes=n), precond))
    out = osdn.forward(q.cuda(), k.cuda(), dev.v, dev.beta, dev.r, eta=inp.eta, chunk=chunk,
                       precond=precond, norm_qk=True, gate_logits=True)
    torch.cuda.synchronize()
    qq, kk, bb, rr = oracle.prepare_inputs(q, k, inp.beta, inp.r)
    ref = oracle.forward(qq, kk, inp.v, bb, rr, eta=inp.eta,
                         mode="osdn" if precond else "deltanet", want=("o", "S", "d"))
    errs = _errors(out, ref, precond)
    _log("  errors %s" % {k_: "%.3g" % x for k_, x in errs.items()})
    for name, e in errs.items():
        assert e <= TOL[name], errs
    assert np.all(np.isfinite(out["o"].float().cpu().numpy()))
