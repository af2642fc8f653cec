"""The oracle's summation-order option (oracle.run(order=...)) and its fp32
build, which the GPU parity tests use as the fp32 reference where the stated
per-element bound is missed: a different edge order changes only the rounding
of the same definition (fp64 results agree to ~1e-12, the edge gradient comes
back in the caller's order), and the fp32 build agrees with the fp64 oracle to
fp32 accuracy and sees a planted change of definition."""
import numpy as np
import pytest

import oracle
import synthetic

KEYS = ("out", "g_edge_values", "g_leak", "g_bias", "g_drives", "g_state0")


def _run(w, **kw):
    return oracle.run(w.src, w.dst, w.num_nodes, w.input_nodes, w.edge_values, w.leak, w.bias,
                      w.drives, w.state0, w.microsteps, grad_out=w.grad_out, **kw)


@pytest.mark.parametrize("order", ["sorted", 3])
def test_edge_order_changes_only_rounding(order):
    w = synthetic.make("tiny")
    a, b = _run(w), _run(w, order=order)
    for k in KEYS:
        scale = max(float(np.abs(a[k]).max()), 1e-30)
        assert float(np.abs(a[k] - b[k]).max()) <= 1e-12 * scale, k


def test_edge_order_permutations():
    src = np.array([3, 1, 2, 1, 0])
    dst = np.array([0, 2, 0, 0, 2])
    np.testing.assert_array_equal(oracle.edge_order(src, dst, None), np.arange(5))
    # by (dst, src, caller index): (0,1,#3) (0,2,#2) (0,3,#0) (2,0,#4) (2,1,#1)
    np.testing.assert_array_equal(oracle.edge_order(src, dst, "sorted"), [3, 2, 0, 4, 1])
    p = oracle.edge_order(src, dst, 7)
    np.testing.assert_array_equal(np.sort(p), np.arange(5))


def test_edge_gradient_comes_back_in_caller_order():
    """Duplicating one edge's value into a planted spike: its gradient lands
    on the same caller index whatever the order."""
    w = synthetic.make("tiny", T=2)
    for order in (None, "sorted", 5):
        g = _run(w, order=order)["g_edge_values"]
        g2 = oracle.run(w.src, w.dst, w.num_nodes, w.input_nodes, w.edge_values, w.leak, w.bias,
                        w.drives, w.state0, w.microsteps, grad_out=w.grad_out * 2.0,
                        order=order)["g_edge_values"]
        np.testing.assert_allclose(g2, 2.0 * g, rtol=1e-12, atol=1e-300)
        np.testing.assert_allclose(g, _run(w)["g_edge_values"], rtol=1e-10, atol=1e-14)


@pytest.mark.parametrize("order", [None, "sorted", 11])
def test_fp32_build_matches_oracle(order):
    w = synthetic.make("tiny", B=5, T=5, M=3)
    ref, f32 = _run(w), _run(w, precision="f32", order=order)
    for k in KEYS:
        scale = max(float(np.abs(ref[k]).max()), 1e-30)
        assert float(np.abs(f32[k] - ref[k]).max()) <= 2e-5 * scale, k


def test_fp32_build_detects_a_planted_mistake():
    w = synthetic.make("tiny")
    ref = _run(w)
    w.leak = (w.leak * 0.99).astype(np.float32)
    alt = _run(w, precision="f32", order="sorted")
    assert float(np.abs(alt["out"] - ref["out"]).max()) > 1e-4
