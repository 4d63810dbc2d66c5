"""Pins of the oracle's input transforms (L2 normalisation of q and k per token,
logistic sigmoid of the gate logits): the properties that define them."""
import math

import numpy as np

from oracle import oracle


def test_rows_become_unit_vectors_along_the_input():
    g = np.random.default_rng(3)
    x = 3.0 * g.standard_normal((2, 3, 17, 32))
    q, k, _, _ = oracle.prepare_inputs(x, 0.5 * x, np.zeros((2, 3, 17)), gate_logits=False)
    n = np.linalg.norm(x, axis=-1, keepdims=True)
    assert np.allclose(np.linalg.norm(q, axis=-1), 1.0, rtol=0, atol=1e-15)
    assert np.allclose(q * n, x, rtol=1e-14, atol=0)        # same direction, positive scale
    assert np.array_equal(q, k)                            # scale-invariant


def test_zero_and_axis_rows():
    x = np.zeros((1, 1, 3, 4))
    x[0, 0, 1, 2] = -0.125
    x[0, 0, 2] = [3.0, 4.0, 0.0, 0.0]
    q, _, _, _ = oracle.prepare_inputs(x, x, np.zeros((1, 1, 3)), gate_logits=False)
    assert np.array_equal(q[0, 0, 0], np.zeros(4))
    assert np.array_equal(q[0, 0, 1], np.array([0.0, 0.0, -1.0, 0.0]))
    assert np.allclose(q[0, 0, 2], [0.6, 0.8, 0.0, 0.0], rtol=0, atol=1e-16)


def test_sigmoid_of_logits():
    z = np.array([0.0, math.log(3.0), -math.log(3.0), 40.0, -40.0, 745.0, -745.0])
    _, _, b, r = oracle.prepare_inputs(np.ones((1, 1, 7, 2)), np.ones((1, 1, 7, 2)),
                                       z.reshape(1, 1, 7), -z.reshape(1, 1, 7), norm_qk=False)
    b, r = b.ravel(), r.ravel()
    assert b[0] == 0.5
    assert abs(b[1] - 0.75) < 1e-15 and abs(b[2] - 0.25) < 1e-15
    assert np.all(np.abs(b + r - 1.0) < 1e-15)             # sigmoid(x) + sigmoid(-x) = 1
    assert b[5] == 1.0 and b[6] >= 0.0 and np.all(np.isfinite(b))
    assert np.all(np.diff(b[[6, 4, 2, 0, 1, 3, 5]]) >= 0)  # monotone


def test_transforms_are_optional():
    g = np.random.default_rng(4)
    x = g.standard_normal((1, 2, 5, 8))
    bl = g.standard_normal((1, 2, 5))
    q, k, b, r = oracle.prepare_inputs(x, x, bl, None, norm_qk=False, gate_logits=False)
    assert np.array_equal(q, x) and np.array_equal(b, bl) and r is None
