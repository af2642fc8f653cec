"""The sorted-order fp32 evaluation (oracle/sorted_f32.py) computes the same
definition as the fp64 oracle: on small workloads it agrees with it to fp32
accuracy on every output, and it differs from the C oracle's own fp32
evaluation only by rounding (it is used to measure the fp32 floor only)."""
import numpy as np
import pytest

import oracle
import synthetic
from oracle import sorted_f32


def _check(w):
    ref = oracle.run(w.src, w.dst, w.num_nodes, w.input_nodes, w.edge_values, w.leak, w.bias,
                     w.drives, w.state0, w.microsteps, grad_out=w.grad_out)
    alt = sorted_f32.run(w.src, w.dst, w.num_nodes, w.input_nodes, w.edge_values, w.leak, w.bias,
                         w.drives, w.state0, w.microsteps, w.grad_out)
    for k in ("out", "g_edge_values", "g_leak", "g_bias", "g_drives", "g_state0"):
        a, b = alt[k], ref[k]
        assert a.shape == b.shape, k
        scale = max(float(np.abs(b).max()), 1e-30)
        assert float(np.abs(a - b).max()) <= 2e-5 * scale, (k, float(np.abs(a - b).max()), scale)


def test_sorted_f32_matches_oracle_tiny():
    _check(synthetic.make("tiny"))


@pytest.mark.parametrize("B,M", [(3, 1), (5, 3)])
def test_sorted_f32_matches_oracle_other_shapes(B, M):
    _check(synthetic.make("tiny", B=B, T=5, M=M))


def test_sorted_f32_detects_a_planted_mistake():
    """A wrong leak (the check must not pass on a different definition)."""
    w = synthetic.make("tiny")
    ref = oracle.run(w.src, w.dst, w.num_nodes, w.input_nodes, w.edge_values, w.leak, w.bias,
                     w.drives, w.state0, w.microsteps, grad_out=w.grad_out)
    alt = sorted_f32.run(w.src, w.dst, w.num_nodes, w.input_nodes, w.edge_values, w.leak * 0.99,
                         w.bias, w.drives, w.state0, w.microsteps, w.grad_out)
    assert float(np.abs(alt["out"] - ref["out"]).max()) > 1e-4
