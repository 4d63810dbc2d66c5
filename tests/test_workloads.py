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
