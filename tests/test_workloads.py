"""The seeded input generators (host only): the gated workloads add a state
gate without changing any other draw."""
from dataclasses import replace

import numpy as np
import torch

from delta_rule_recurrent_precond_amd import workloads as W


def test_gate_draw_leaves_other_inputs_unchanged():
    w = W.custom(2, 3, 50, 16, 8, 16, dtype="bf16", apf=True, seed=42)
    a = W.generate(w)
    b = W.generate(replace(w, gated=True))
    assert a.alpha is None and b.alpha is not None
    for name in ("q", "k", "v", "beta", "r"):
        assert torch.equal(getattr(a, name), getattr(b, name)), name
    al = b.alpha.numpy()
    assert al.shape == (2, 3, 50) and al.dtype == np.float32
    assert np.all((al > 0) & (al < 1))


def test_gated_layer_workload_matches_ungated_draws():
    g = W.CONFIGS["1.3b-apf-gated"]
    assert g.gated and replace(g, gated=False, name=W.L13B_APF.name) == W.L13B_APF


def test_raw_draw_transforms_to_the_plain_draw():
    """Raw inputs are the plain workload's draws before its normalisation and
    sigmoids: transforming them (in fp64, before rounding) reaches the same
    values up to the one rounding to the stored type."""
    from oracle import oracle
    w = W.custom(1, 2, 20, 16, 8, 16, dtype="f32", apf=True, seed=9)
    plain = W.generate(w)
    raw = W.generate(replace(w, raw=True))
    q, k, b, r = oracle.prepare_inputs(raw.q, raw.k, raw.beta, raw.r)
    assert torch.equal(plain.v, raw.v)
    assert np.allclose(q, plain.q.double().numpy(), rtol=0, atol=1e-6)
    assert np.allclose(k, plain.k.double().numpy(), rtol=0, atol=1e-6)
    assert np.allclose(b, plain.beta.double().numpy(), rtol=0, atol=1e-6)
    assert np.allclose(r, plain.r.double().numpy(), rtol=0, atol=1e-6)
