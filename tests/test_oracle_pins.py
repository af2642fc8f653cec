"""Pins of the CPU oracle against what the pages and mathematics fix.

The oracle (oracle/ck_oracle.c) is checked against:
  * a hand-derived worked example (tests/golden/worked_example.json);
  * a dense brute-force recurrence (numpy, dense W) on tiny graphs with
    duplicates, self-loops, empty rows, E=0 and n_in=0, for M in 1..3;
  * the textbook tanh Elman RNN (torch.nn.RNN) at leak=1, M=1, forward and
    gradients through torch autograd;
  * torch autograd on a dense fp64 formulation for general leak and M;
  * central finite differences of L = sum(out * G), every coordinate of all
    five inputs, plus a directional test on the tiny workload;
  * closed forms (leak=0; a single node without edges);
  * exact invariants (batch-column independence, microstep composition,
    linearity in G, caller edge order) and the graph builder's total order.
Each of these fails on a dropped term, a wrong sign or index or a transposed
operand somewhere in the oracle.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synthetic
from dense_ref import dense_forward, torch_dense_grads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
GRAD_KEYS = ("g_edge_values", "g_leak", "g_bias", "g_drives", "g_state0")


def _run(w, G=None, **kw):
    return oracle.run(w.src, w.dst, w.num_nodes, w.input_nodes, w.edge_values, w.leak, w.bias,
                      w.drives, w.state0, w.microsteps, grad_out=G, **kw)


def _small(seed, N=7, E=20, n_in=2, B=3, T=3, M=2, **kw):
    return synthetic.random_graph(np.random.default_rng(seed), N, E, n_in, B, T, M, **kw)


# ---------------------------------------------------------------- worked example
def test_worked_example_by_hand():
    with open(os.path.join(GOLDEN, "worked_example.json")) as f:
        fx = json.load(f)
    x = fx["inputs"]
    v = x["edge_values"][0]
    res = oracle.run(x["src"], x["dst"], x["num_nodes"], x["input_nodes"], x["edge_values"],
                     x["leak"], x["bias"], x["drives"], x["state0"], x["microsteps"],
                     grad_out=x["grad_out"])
    for key, exp in fx["expected"].items():
        want = np.vectorize(lambda d: d["c0"] + d["c1"] * v, otypes=[float])(np.array(exp, dtype=object))
        np.testing.assert_allclose(res[key], want, rtol=0, atol=1e-13, err_msg=key)


# ---------------------------------------------------------------- dense brute force
CASES = [
    dict(N=7, E=20, n_in=2, B=3, T=3, M=1),
    dict(N=7, E=20, n_in=2, B=3, T=3, M=2),
    dict(N=9, E=40, n_in=3, B=5, T=4, M=3),
    dict(N=32, E=200, n_in=4, B=4, T=2, M=2),
    dict(N=12, E=0, n_in=3, B=2, T=3, M=2),       # no edges
    dict(N=12, E=30, n_in=0, B=2, T=3, M=2),      # no input nodes
    dict(N=1, E=3, n_in=1, B=2, T=2, M=3),        # one node, self-loops only
]


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("seed", [11, 12])
def test_forward_matches_dense_bruteforce(case, seed):
    w = _small(seed, **case)
    res = _run(w)
    ref = dense_forward(w.num_nodes, w.src, w.dst, w.input_nodes, w.edge_values, w.leak, w.bias,
                        w.drives, w.state0, w.microsteps)
    np.testing.assert_allclose(res["out"], ref, rtol=0, atol=1e-12)


def test_forward_empty_rows_and_parallel_edges_dense():
    rng = np.random.default_rng(5)
    N = 10
    # node 9 and node 4 get no in-edges; (1 -> 2) appears three times; 3 -> 3 self-loop
    src = np.array([1, 1, 1, 3, 0, 5, 6, 7, 8, 2, 2], np.int64)
    dst = np.array([2, 2, 2, 3, 1, 0, 0, 5, 6, 7, 8], np.int64)
    w = _small(1, N=N, E=11, n_in=3, B=2, T=3, M=2)
    w.src, w.dst = src, dst
    w.edge_values = rng.standard_normal(11).astype(np.float32)
    res = _run(w, G=w.grad_out)
    ref = torch_dense_grads(N, src, dst, w.input_nodes, w.edge_values, w.leak, w.bias, w.drives,
                            w.state0, 2, w.grad_out)
    np.testing.assert_allclose(res["out"], ref["out"], rtol=0, atol=1e-12)
    for k in GRAD_KEYS:
        np.testing.assert_allclose(res[k], ref[k], rtol=1e-10, atol=1e-12, err_msg=k)
    # the three parallel copies of 1 -> 2 each receive the full dL/dW[2, 1]
    assert res["g_edge_values"][0] == res["g_edge_values"][1] == res["g_edge_values"][2]


# ---------------------------------------------------------------- textbook Elman RNN
@pytest.mark.parametrize("seed", [3, 4])
def test_leak_one_single_microstep_is_elman_rnn(seed):
    """leak = 1, M = 1:  h_t = tanh(W h_{t-1} + S d_t + bias), torch.nn.RNN(tanh)."""
    w = _small(seed, N=8, E=25, n_in=3, B=4, T=5, M=1, duplicates=False)
    w.leak = np.ones(w.num_nodes, np.float32)
    N, n_in = w.num_nodes, w.n_in
    rnn = torch.nn.RNN(n_in, N, nonlinearity="tanh", bias=True, dtype=torch.float64)
    W = np.zeros((N, N))
    np.add.at(W, (w.dst, w.src), w.edge_values.astype(np.float64))
    Sel = np.zeros((N, n_in))
    Sel[w.input_nodes, np.arange(n_in)] = 1.0
    with torch.no_grad():
        rnn.weight_hh_l0.copy_(torch.from_numpy(W))
        rnn.weight_ih_l0.copy_(torch.from_numpy(Sel))
        rnn.bias_ih_l0.copy_(torch.from_numpy(w.bias.astype(np.float64)))
        rnn.bias_hh_l0.zero_()
    x = torch.tensor(np.transpose(w.drives, (0, 2, 1)).astype(np.float64), requires_grad=True)
    h0 = torch.tensor(w.state0.astype(np.float64)[None], requires_grad=True)
    y, _ = rnn(x, h0)
    G = w.grad_out.astype(np.float64)
    (y * torch.from_numpy(G)).sum().backward()
    res = _run(w, G=w.grad_out)
    np.testing.assert_allclose(res["out"], y.detach().numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(res["g_state0"], h0.grad.numpy()[0], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(res["g_drives"], np.transpose(x.grad.numpy(), (0, 2, 1)),
                               rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(res["g_bias"], rnn.bias_ih_l0.grad.numpy(), rtol=1e-10, atol=1e-12)
    gW = rnn.weight_hh_l0.grad.numpy()
    np.testing.assert_allclose(res["g_edge_values"], gW[w.dst, w.src], rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------- autograd (dense)
@pytest.mark.parametrize("case", CASES)
def test_gradients_match_dense_autograd(case):
    w = _small(21, **case)
    res = _run(w, G=w.grad_out)
    ref = torch_dense_grads(w.num_nodes, w.src, w.dst, w.input_nodes, w.edge_values, w.leak,
                            w.bias, w.drives, w.state0, w.microsteps, w.grad_out)
    np.testing.assert_allclose(res["out"], ref["out"], rtol=0, atol=1e-12)
    for k in GRAD_KEYS:
        np.testing.assert_allclose(res[k], ref[k], rtol=1e-10, atol=1e-12, err_msg=k)


# ---------------------------------------------------------------- finite differences
def _loss(w, G, **over):
    args = dict(edge_values=w.edge_values, leak=w.leak, bias=w.bias, drives=w.drives,
                state0=w.state0)
    args.update(over)
    r = oracle.run(w.src, w.dst, w.num_nodes, w.input_nodes, args["edge_values"], args["leak"],
                   args["bias"], args["drives"], args["state0"], w.microsteps)
    return float(np.sum(r["out"] * G))


@pytest.mark.parametrize("seed,M", [(31, 1), (32, 2), (33, 3)])
def test_gradients_match_central_differences_every_coordinate(seed, M):
    w = _small(seed, N=6, E=14, n_in=2, B=2, T=3, M=M)
    w.src[0], w.dst[0] = 2, 2          # a self-loop
    w.src[1], w.dst[1] = w.src[2], w.dst[2]  # a parallel edge
    G = w.grad_out.astype(np.float64)
    res = _run(w, G=G)
    names = {"edge_values": "g_edge_values", "leak": "g_leak", "bias": "g_bias",
             "drives": "g_drives", "state0": "g_state0"}
    for arg, gkey in names.items():
        base = getattr(w, arg).astype(np.float64)
        fd = np.zeros(base.shape)
        for idx in np.ndindex(base.shape):
            eps = 1e-6 * max(1.0, abs(base[idx]))
            xp, xm = base.copy(), base.copy()
            xp[idx] += eps
            xm[idx] -= eps
            fd[idx] = (_loss(w, G, **{arg: xp}) - _loss(w, G, **{arg: xm})) / (2 * eps)
        np.testing.assert_allclose(res[gkey], fd, rtol=1e-6, atol=1e-8, err_msg=gkey)


def test_directional_derivative_on_tiny_workload():
    w = synthetic.make("tiny")
    G = w.grad_out.astype(np.float64)
    res = _run(w, G=G)
    rng = np.random.default_rng(7)
    dirs = {k: rng.standard_normal(getattr(w, k).shape)
            for k in ("edge_values", "leak", "bias", "drives", "state0")}
    pred = sum(float(np.sum(res["g_" + k] * d)) for k, d in dirs.items())
    eps = 1e-5

    def at(sign):
        over = {k: getattr(w, k).astype(np.float64) + sign * eps * d for k, d in dirs.items()}
        return _loss(w, G, **over)
    fd = (at(+1) - at(-1)) / (2 * eps)
    assert abs(fd - pred) <= 1e-6 * max(1.0, abs(pred)), (fd, pred)


# ---------------------------------------------------------------- closed forms
def test_leak_zero_closed_form():
    w = _small(41, N=9, E=30, n_in=3, B=3, T=4, M=3)
    w.leak = np.zeros(w.num_nodes, np.float32)
    G = w.grad_out.astype(np.float64)
    res = _run(w, G=G)
    h0 = w.state0.astype(np.float64)
    T = w.T
    for t in range(T):
        np.testing.assert_array_equal(res["out"][t], h0)
    np.testing.assert_allclose(res["g_state0"], G.sum(axis=0), rtol=0, atol=1e-13)
    for k in ("g_edge_values", "g_bias", "g_drives"):
        assert np.all(res[k] == 0.0), k
    # g_leak_i = M * sum_t sum_b (sum_{t' >= t} G[t'])_{b,i} * (tanh(W h0 + d_t + bias) - h0)_{b,i}
    N = w.num_nodes
    W = np.zeros((N, N))
    np.add.at(W, (w.dst, w.src), w.edge_values.astype(np.float64))
    tail = np.cumsum(G[::-1], axis=0)[::-1]
    gl = np.zeros(N)
    for t in range(T):
        d = np.zeros((w.B, N))
        d[:, w.input_nodes] = w.drives[t].T
        p = np.tanh(h0 @ W.T + d + w.bias.astype(np.float64))
        gl += w.microsteps * np.sum(tail[t] * (p - h0), axis=0)
    np.testing.assert_allclose(res["g_leak"], gl, rtol=1e-12, atol=1e-13)


def test_single_node_without_edges_closed_form():
    lam, h0, d, b = 0.3, 0.25, 0.7, -0.2
    res = oracle.run([], [], 1, [0], np.zeros(0), [lam], [b], [[[d]]], [[h0]], 1,
                     grad_out=[[[1.0]]])
    p = math.tanh(d + b)
    assert abs(res["out"][0, 0, 0] - ((1 - lam) * h0 + lam * p)) < 1e-15
    sech2 = 1.0 / math.cosh(d + b) ** 2
    assert abs(res["g_state0"][0, 0] - (1 - lam)) < 1e-15
    assert abs(res["g_leak"][0] - (p - h0)) < 1e-15
    assert abs(res["g_bias"][0] - lam * sech2) < 1e-15
    assert abs(res["g_drives"][0, 0, 0] - lam * sech2) < 1e-15


def test_saturated_preactivation_gradient_is_finite_and_small():
    # |a| ~ 400: tanh = +-1 exactly in fp64, sech^2 underflows to 0 without NaN
    lam = 0.5
    res = oracle.run([], [], 1, [0], np.zeros(0), [lam], [0.0], [[[400.0]]], [[0.1]], 1,
                     grad_out=[[[1.0]]])
    assert res["g_bias"][0] == 0.0 and res["g_drives"][0, 0, 0] == 0.0
    assert abs(res["out"][0, 0, 0] - (0.5 * 0.1 + 0.5)) < 1e-15


# ---------------------------------------------------------------- invariants
def test_batch_columns_are_independent_bitwise():
    w = _small(51, N=20, E=80, n_in=4, B=4, T=3, M=2)
    full = _run(w, G=w.grad_out)
    for b in range(w.B):
        wb = _small(51, N=20, E=80, n_in=4, B=4, T=3, M=2)
        wb.state0 = w.state0[b:b + 1]
        wb.drives = w.drives[:, :, b:b + 1]
        one = _run(wb, G=w.grad_out[:, b:b + 1])
        np.testing.assert_array_equal(full["out"][:, b], one["out"][:, 0])
        np.testing.assert_array_equal(full["g_state0"][b], one["g_state0"][0])
        np.testing.assert_array_equal(full["g_drives"][:, :, b], one["g_drives"][:, :, 0])


def test_microsteps_compose_as_repeated_steps():
    M = 3
    w = _small(61, N=15, E=60, n_in=3, B=2, T=4, M=M)
    res = _run(w, G=w.grad_out)
    w1 = _small(61, N=15, E=60, n_in=3, B=2, T=4, M=M)
    w1.microsteps = 1
    w1.drives = np.repeat(w.drives, M, axis=0)
    G1 = np.zeros((w.T * M, w.B, w.num_nodes))
    G1[M - 1::M] = w.grad_out
    r1 = _run(w1, G=G1)
    np.testing.assert_array_equal(res["out"], r1["out"][M - 1::M])
    np.testing.assert_allclose(res["g_drives"], r1["g_drives"].reshape(w.T, M, w.n_in, w.B).sum(1),
                               rtol=1e-13, atol=1e-15)
    for k in ("g_edge_values", "g_leak", "g_bias", "g_state0"):
        np.testing.assert_allclose(res[k], r1[k], rtol=1e-13, atol=1e-15, err_msg=k)


def test_gradients_are_linear_in_upstream_gradient():
    w = _small(71, N=12, E=50, n_in=3, B=3, T=3, M=2)
    rng = np.random.default_rng(0)
    G1 = rng.standard_normal(w.grad_out.shape)
    G2 = rng.standard_normal(w.grad_out.shape)
    r1, r2, r12 = _run(w, G=G1), _run(w, G=G2), _run(w, G=G1 - 2.5 * G2)
    for k in GRAD_KEYS:
        np.testing.assert_allclose(r12[k], r1[k] - 2.5 * r2[k], rtol=1e-11, atol=1e-13, err_msg=k)


def test_caller_edge_order_is_invisible():
    w = _small(81, N=30, E=150, n_in=4, B=2, T=3, M=2, duplicates=False)
    res = _run(w, G=w.grad_out)
    p = np.random.default_rng(1).permutation(w.num_edges)
    w2 = _small(81, N=30, E=150, n_in=4, B=2, T=3, M=2, duplicates=False)
    w2.src, w2.dst, w2.edge_values = w.src[p], w.dst[p], w.edge_values[p]
    r2 = _run(w2, G=w.grad_out)
    np.testing.assert_allclose(r2["out"], res["out"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(r2["g_edge_values"], res["g_edge_values"][p], rtol=1e-12, atol=1e-14)


def test_thread_count_does_not_change_results():
    w = _small(91, N=40, E=300, n_in=5, B=6, T=3, M=2)
    a = _run(w, G=w.grad_out, nthreads=1)
    b = _run(w, G=w.grad_out, nthreads=5)
    for k in ("out",) + GRAD_KEYS:
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)


# ---------------------------------------------------------------- graph build
@pytest.mark.parametrize("seed", [1, 2])
def test_graph_build_total_order(seed):
    w = _small(seed, N=50, E=600, n_in=7, B=1, T=1, M=1)  # many parallel edges
    g = oracle.build_graph(w.src, w.dst, w.num_nodes, w.input_nodes)
    E, N = w.num_edges, w.num_nodes
    e = np.arange(E)
    # independent construction: numpy lexsort by (dst, src, e) and (src, dst, e)
    csr = np.lexsort((e, w.src, w.dst))
    csc = np.lexsort((e, w.dst, w.src))
    np.testing.assert_array_equal(g["perm"], csr)
    np.testing.assert_array_equal(g["col_idx"], w.src[csr])
    np.testing.assert_array_equal(g["t_perm"], csc)
    np.testing.assert_array_equal(g["t_col_idx"], w.dst[csc])
    np.testing.assert_array_equal(g["row_ptr"], np.concatenate([[0], np.cumsum(np.bincount(w.dst, minlength=N))]))
    np.testing.assert_array_equal(g["t_row_ptr"], np.concatenate([[0], np.cumsum(np.bincount(w.src, minlength=N))]))
    slot = np.full(N, -1)
    slot[w.input_nodes] = np.arange(w.n_in)
    np.testing.assert_array_equal(g["input_slot"], slot)
    # structural: rows ascending by (src, caller index)
    for i in range(N):
        r = slice(g["row_ptr"][i], g["row_ptr"][i + 1])
        key = g["col_idx"][r].astype(np.int64) * E + g["perm"][r]
        assert np.all(np.diff(key) > 0)


@pytest.mark.parametrize("src,dst,N,inputs,code", [
    ([0, 1], [1, 2], 2, [0], 3),          # dst out of range
    ([-1], [0], 2, [0], 3),               # negative src
    ([0], [1], 2, [2], 3),                # input out of range
    ([0], [1], 3, [1, 1], 4),             # duplicate input
    ([0], [1], 0, [], 2),                 # no nodes
    ([], [], 4, [], 0),                   # empty graph is legal
])
def test_validation_rules(src, dst, N, inputs, code):
    assert oracle.validate(src, dst, N, inputs) == code
