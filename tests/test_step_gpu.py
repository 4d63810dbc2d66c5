"""GPU parity of osdn_step (one decoding step with persistent S and d)
against the fp64 oracle run over the same tokens (through the C ABI).

fp32 data: o, S and d within 1e-5 (fp32 arithmetic over a dozen tokens).
bf16 data: the same for S and d (the step computes in fp32 on the stored
bits); o is rounded to bf16 once, so within 2^-8.  log rho is compared with
the conditioning-aware bound of the scan tests.  Inputs come from the seeded
generators; expected values from the oracle only.
"""
import numpy as np
import pytest
import torch

import delta_rule_recurrent_precond_amd as osdn
from delta_rule_recurrent_precond_amd import workloads as W
from oracle import oracle

from _helpers import as_f64, matrix_rel, rowwise_rel

pytestmark = pytest.mark.gpu


def _log_ratio_tol(rho, eps_a=2e-5):
    g = np.sqrt(np.maximum(rho, 1e-300))
    return 2.0 * eps_a / g + 1e-6


def _token(x, t):
    return None if x is None else x[:, :, t].contiguous()


def _run_steps(dev, S, d, eta, t0, t1):
    os_, lrs = [], []
    for t in range(t0, t1):
        out = osdn.step(_token(dev.q, t), _token(dev.k, t), _token(dev.v, t), _token(dev.beta, t),
                        S, d, _token(dev.r, t), eta=eta, want_log_ratio=True)
        os_.append(out["o"])
        lrs.append(out["log_ratio"])
    return torch.stack(os_, dim=2), torch.stack(lrs, dim=2)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (64, 32), (128, 128)])
@pytest.mark.parametrize("apf", [False, True])
def test_steps_match_oracle(dtype, dk, dv, apf):
    T = 12
    w = W.custom(2, 3, T, dk, dv, 16, dtype=dtype, eta=0.1, apf=apf, seed=700 + dk + dv)
    inp = W.generate(w)
    g = torch.Generator().manual_seed(11)
    S0 = 0.1 * torch.randn(w.B, w.H, dv, dk, generator=g)
    d0 = 0.5 + torch.rand(w.B, w.H, dk, generator=g)
    ref = oracle.forward(inp.q, inp.k, inp.v, inp.beta, inp.r, d0, S0, eta=inp.eta,
                         want=("o", "S", "d", "rho"))
    dev = inp.to("cuda")
    S, d = S0.clone().cuda(), d0.clone().cuda()
    print("steps %s" % w.name, flush=True)
    o, lr = _run_steps(dev, S, d, inp.eta, 0, T)
    torch.cuda.synchronize()
    tol_o = 1e-5 if dtype == "f32" else 2.0 ** -8
    assert rowwise_rel(o, ref["o"]) <= tol_o
    assert matrix_rel(S, ref["S"]) <= 1e-5
    assert rowwise_rel(d, ref["d"]) <= 1e-5
    assert np.all(np.abs(as_f64(lr) - np.log(ref["rho"])) <= _log_ratio_tol(ref["rho"]))


def test_steps_continue_a_forward():
    """A chunked forward over the first 64 tokens, then single steps: the state
    and preconditioner at the end match the oracle over all 70 tokens."""
    w = W.custom(2, 2, 70, 128, 128, 64, dtype="bf16", eta=0.05, apf=True, seed=71)
    inp = W.generate(w)
    dev = inp.to("cuda")
    out = osdn.forward(dev.q[:, :, :64].contiguous(), dev.k[:, :, :64].contiguous(),
                       dev.v[:, :, :64].contiguous(), dev.beta[:, :, :64].contiguous(),
                       dev.r[:, :, :64].contiguous(), eta=inp.eta, chunk=64)
    S, d = out["S_final"], out["d_final"]
    o, _ = _run_steps(dev, S, d, inp.eta, 64, 70)
    torch.cuda.synchronize()
    ref = oracle.forward(inp.q, inp.k, inp.v, inp.beta, inp.r, eta=inp.eta, want=("o", "S", "d"))
    assert matrix_rel(S, ref["S"]) <= 2e-2
    assert rowwise_rel(d, ref["d"]) <= 1e-5
    assert rowwise_rel(o, ref["o"][:, :, 64:]) <= 2e-2


def test_step_decode_batch_full_size():
    """The decode batch the benchmark times (64 x 16 heads, dk = dv = 128)."""
    w = W.DECODE
    inp = W.generate(w)
    g = torch.Generator().manual_seed(12)
    S0 = 0.1 * torch.randn(w.B, w.H, 128, 128, generator=g)
    d0 = 0.5 + torch.rand(w.B, w.H, 128, generator=g)
    ref = oracle.forward(inp.q, inp.k, inp.v, inp.beta, inp.r, d0, S0, eta=inp.eta,
                         want=("o", "S", "d"))
    dev = inp.to("cuda")
    S, d = S0.clone().cuda(), d0.clone().cuda()
    o, _ = _run_steps(dev, S, d, inp.eta, 0, 1)
    torch.cuda.synchronize()
    assert rowwise_rel(o, ref["o"]) <= 2.0 ** -8
    assert matrix_rel(S, ref["S"]) <= 1e-5
    assert rowwise_rel(d, ref["d"]) <= 1e-5
