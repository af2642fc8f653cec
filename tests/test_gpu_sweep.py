"""Seeded random sweeps through the C ABI: many small graphs and shapes, each
on a randomly chosen kernel family, against the oracle.

Recurrence: 120 random graphs (N log-uniform in 1..12,000, mean in-degree
0.5..200, uniform sources, a hub row or many empty rows, 1 <= B <= 70,
T <= 4, M <= 3).  Summation order is not fixed by the definition, so a
tensor whose GPU result misses the stated bound somewhere is held to the
spread of fp32 evaluations of the same definition in several orders (the
CSR rows, the caller's order, two random orders): it may miss the bound on
at most two more elements than the worst of them does with its errors
doubled, and its largest and 99th-percentile errors may be at most twice the
worst of theirs.  (In a long run of such sweeps, about one case in 150 has
one or two gradient entries of a sum over many batch columns, with a value
near zero, past the bound where the CSR-order evaluation happens not to be.)

LIF: 120 random runs (delays up to 24, both spike lookups), bit-exact."""
import os

import numpy as np
import pytest
import torch

import oracle
import sparse_graph_recurrent_amd as sgr
import synthetic
from gpu_helpers import GRAD_ATOL, GRAD_KEYS, GRAD_RTOL, STATE_ATOL, STATE_RTOL, log, to_dev

pytestmark = pytest.mark.gpu
PATH_ENV = {"per_microstep": {"CK_RESIDENT": "0", "CK_BLOCKED": "0"},
            "resident": {"CK_RESIDENT": "1", "CK_BLOCKED": "0"},
            "blocked": {"CK_RESIDENT": "0", "CK_BLOCKED": "1"},
            "blocked_both": {"CK_RESIDENT": "0", "CK_BLOCKED": "2"}}


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sgr.lib()


def _graph(w, env):
    saved = {k: os.environ.get(k) for k in env}
    os.environ.update(env)
    try:
        return sgr.SparseGraph(to_dev(w.src), to_dev(w.dst), w.num_nodes, to_dev(w.input_nodes))
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


def _recurrence_case(i):
    rng = np.random.default_rng([20261, i])
    N = max(1, int(np.exp(rng.uniform(0, np.log(12000)))))
    deg = float(np.exp(rng.uniform(np.log(0.5), np.log(200))))
    E = int(min(400_000, N * deg))
    n_in = int(rng.integers(0, N + 1)) if rng.random() < 0.8 else 0
    B, T, M = int(rng.integers(1, 71)), int(rng.integers(1, 5)), int(rng.integers(1, 4))
    kind = str(rng.choice(["uniform", "hub", "empty rows"]))
    w = synthetic.random_graph(rng, N, E, n_in, B, T, M, v_scale=float(1 / np.sqrt(deg + 1)))
    if kind == "hub" and N > 2 and E > 0:
        k = int(min(E // 2, 20000))
        w.dst = np.concatenate([w.dst[:E - k], np.full(k, int(rng.integers(0, N)))])
    if kind == "empty rows" and N > 4:
        keep = w.dst % 7 != 3
        w.src, w.dst = w.src[keep], w.dst[keep]
    w.edge_values = (rng.standard_normal(w.src.size) / np.sqrt(deg + 1)).astype(np.float32)
    paths = ["per_microstep"] + (["resident"] if N <= 9184 else []) + \
            (["blocked", "blocked_both"] if 5 <= B <= 64 else [])
    return w, str(rng.choice(paths)), kind


def _oracle(w, precision="f64", order=None):
    return oracle.run(w.src, w.dst, w.num_nodes, w.input_nodes, w.edge_values, w.leak, w.bias,
                      w.drives, w.state0, w.microsteps, grad_out=w.grad_out, precision=precision,
                      order=order)


def _within_fp32_spread(w, got, ref):
    evals = None
    for k in ("out",) + GRAD_KEYS:
        rt, at = (STATE_RTOL, STATE_ATOL) if k == "out" else (GRAD_RTOL, GRAD_ATOL)
        if ref[k].size == 0:
            continue
        bound = at + rt * np.abs(ref[k])
        err = np.abs(np.asarray(got[k], np.float64) - ref[k])
        bad = int(np.sum(err > bound))
        if bad == 0:
            continue
        if evals is None:
            evals = [_oracle(w, "f32", o) for o in ("sorted", None, 1, 2)]
        e32 = [np.abs(ev[k] - ref[k]) for ev in evals]
        lim = max(int(np.sum(2 * e > bound)) for e in e32) + 2
        mx32 = max(float(e.max()) for e in e32)
        p9932 = max(float(np.quantile(e, 0.99)) for e in e32)
        log(f"  {k}: {bad} outside the bound (allowed {lim}); max {err.max():.3e} "
            f"(fp32 orders {mx32:.3e}); p99 {np.quantile(err, 0.99):.3e} (fp32 orders {p9932:.3e})")
        assert bad <= lim, (k, bad, lim)
        assert err.max() <= 2 * mx32, (k, float(err.max()), mx32)
        assert np.quantile(err, 0.99) <= 2 * p9932, (k, float(np.quantile(err, 0.99)), p9932)


@pytest.mark.parametrize("block", range(4))
def test_random_recurrence_sweep(block):
    for i in range(block * 30, block * 30 + 30):
        w, path, kind = _recurrence_case(i)
        g = _graph(w, PATH_ENV[path])
        taken = sgr.recurrence_path(g, w.B)
        log(f"sweep {i}: N={w.num_nodes} E={w.src.size} n_in={w.input_nodes.size} B={w.B} "
            f"T={w.T} M={w.microsteps} {kind}, {path} requested, {taken} taken")
        ev, lk, bs = to_dev(w.edge_values), to_dev(w.leak), to_dev(w.bias)
        dr, st = to_dev(w.drives), to_dev(w.state0)
        out, saved, ws = sgr.recurrence_forward(g, ev, lk, bs, dr, st, w.microsteps)
        grads = sgr.recurrence_backward(g, ev, lk, st, w.microsteps, saved,
                                        to_dev(w.grad_out, torch.float32), workspace=ws)
        torch.cuda.synchronize()
        got = {"out": out.cpu().numpy(), **{k: v.cpu().numpy() for k, v in grads.items()}}
        _within_fp32_spread(w, got, _oracle(w))
        g.destroy()


@pytest.mark.parametrize("block", range(4))
def test_random_lif_sweep(block, monkeypatch):
    for i in range(block * 30, block * 30 + 30):
        rng = np.random.default_rng([20262, i])
        N = max(1, int(np.exp(rng.uniform(0, np.log(50000)))))
        E = int(min(500_000, N * np.exp(rng.uniform(np.log(0.5), np.log(150)))))
        md, T = int(rng.integers(1, 25)), int(rng.integers(1, 41))
        src, dst = rng.integers(0, N, E), rng.integers(0, N, E)
        w = (np.where(rng.random(E) < 0.75, 1, -1) * rng.integers(1, 200, E)).astype(np.int16)
        d = rng.integers(1, md + 1, E).astype(np.int32)
        v0 = rng.integers(-300, 700, N).astype(np.int32)
        thr, reset, refr = int(rng.integers(20, 300)), int(rng.integers(-60, 1)), int(rng.integers(0, 4))
        shifts = [int(x) for x in rng.integers(1, 9, int(rng.integers(0, 3)))]
        lds = "1" if rng.random() < 0.8 else "0"
        monkeypatch.setenv("CK_LIF_LDS", lds)
        log(f"LIF sweep {i}: N={N} E={E} delays<={md} T={T} lookups={'lds' if lds == '1' else 'bytes'}")
        g = sgr.SparseGraph(to_dev(np.asarray(src, np.int64)), to_dev(np.asarray(dst, np.int64)), N,
                            to_dev(np.zeros(0, np.int64)))
        s, p = sgr.lif_forward(g, to_dev(w), to_dev(d), to_dev(v0), T, thr, reset, refr, shifts)
        s2, p2 = oracle.lif_run(src, dst, N, w, d, v0, T, thr, reset, refr, shifts)
        np.testing.assert_array_equal(s.cpu().numpy(), s2, err_msg=f"case {i}")
        np.testing.assert_array_equal(p.cpu().numpy(), p2, err_msg=f"case {i}")
        g.destroy()
