"""osdn_forward_noalloc against osdn_forward, through the C ABI.

The no-allocation entry point runs the same kernels with the library's fixed
scratch array in place of a workspace, so its outputs must equal those of
osdn_forward given the workspace osdn_forward_workspace_bytes reports, bit for
bit.  Two calls in a row, the second on a smaller problem (the array keeps the
first call's contents), then the plain delta rule and raw inputs on the same
array.  Inputs come from the seeded generators; nothing is compared against a
value the HIP path produced except the other entry point's output.
"""
import pytest
import torch

import delta_rule_recurrent_precond_amd as osdn
from delta_rule_recurrent_precond_amd import _lib
from delta_rule_recurrent_precond_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    osdn.load()


def _equal(a, b):
    for key in ("o", "S_final", "d_final", "log_ratio_sum"):
        x, y = a.get(key), b.get(key)
        if x is None and y is None:
            continue
        assert torch.equal(x, y), key


def _both(w, precond=True, raw=False):
    inp = W.generate(w)
    dev = inp.to("cuda")
    kw = dict(eta=inp.eta, chunk=w.chunk, precond=precond, norm_qk=raw, gate_logits=raw)
    code = 0 if w.dtype == "bf16" else 1
    n = osdn.forward_workspace_bytes(w.B, w.H, w.T, w.dk, w.dv, w.chunk, code, precond)
    assert 0 < n <= _lib.OSDN_NOALLOC_MAX_BYTES
    ref = osdn.forward(dev.q, dev.k, dev.v, dev.beta, dev.r, **kw)
    got = osdn.forward_noalloc(dev.q, dev.k, dev.v, dev.beta, dev.r, **kw)
    torch.cuda.synchronize()
    print("noalloc %s precond=%s raw=%s path=%s scratch=%d B" % (
        w.name, precond, raw, osdn.forward_path(w.B, w.H, w.T, w.dk, w.dv, w.chunk, code, precond,
                                                workspace_bytes=n), n), flush=True)
    _equal(got, ref)


def test_noalloc_equals_forward_on_two_calls_the_second_smaller():
    _both(W.custom(2, 4, 330, 128, 128, 64, dtype="bf16", eta=0.05, apf=True, seed=3301))
    _both(W.custom(1, 2, 130, 128, 128, 64, dtype="bf16", eta=0.05, apf=True, seed=3302))


def test_noalloc_other_modes_on_the_same_array():
    _both(W.custom(2, 3, 200, 128, 128, 64, dtype="bf16", eta=0.05, apf=True, seed=3303),
          precond=False)
    _both(W.custom(2, 3, 190, 128, 128, 64, dtype="bf16", eta=0.05, apf=True, seed=3304, raw=True),
          raw=True)
    # a two-phase shape: the write-key buffer lives in the same array
    _both(W.custom(2, 2, 150, 64, 32, 16, dtype="bf16", eta=0.1, apf=True, seed=3305))
