"""Shared helpers of the GPU parity tests: run the HIP path through the Python
binding (which calls the C ABI), run the oracle on the same seeded inputs, and
compare element by element with the stated tolerances."""
from __future__ import annotations

import os

import numpy as np
import torch

import oracle
import sparse_graph_recurrent_amd as sgr

# Tolerances, per element, as stated: |gpu - oracle| <= atol + rtol * |oracle|
# with rtol/atol 1e-5 / 1e-6 for the outputs (states) and 1e-4 / 1e-6 for the
# five gradients.  Where an element misses that bound, the GPU is held to the
# same definition evaluated in fp32 by the oracle's fp32 build, summing each
# node's edge terms in the order the kernels do (the rows of the CSR by
# destination, and of the transposed CSR): per tensor, the GPU's errors may be
# at most twice that evaluation's -- it may miss the bound on no more elements
# than twice that evaluation's errors do, and its 99th-percentile and largest
# errors may be at most twice that evaluation's.  (On workloads whose
# gradients amplify fp32 rounding -- long rows of mostly positive weights --
# fp32 evaluations of the definition themselves miss the bound on some
# elements, by amounts that depend several-fold on summation order alone; and
# which few elements of a tensor cross the bound is chance, so the count is
# taken at the same factor as the error quantiles.)
STATE_RTOL, STATE_ATOL = 1e-5, 1e-6     # outputs (states)
GRAD_RTOL, GRAD_ATOL = 1e-4, 1e-6       # the five gradients
GRAD_KEYS = ("g_edge_values", "g_leak", "g_bias", "g_drives", "g_state0")


def log(msg: str):
    print(msg, flush=True)


def to_dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


PATHS = ("resident", "per_microstep", "blocked", "blocked_both")
BLOCKED = ("blocked", "blocked_both")  # paths that need 5 <= B <= 64


def make_graph(w, path=None, env=None) -> sgr.SparseGraph:
    """The workload's graph.  path: None for the library's choice, or
    "resident" / "per_microstep" / "blocked" / "blocked_both" to pin the
    kernels (CK_RESIDENT and CK_BLOCKED at creation; the requested path must be the one taken at
    the workload's B).  env: extra environment variables set while the graph
    is created."""
    set_env = dict(env or {})
    if path == "per_microstep":
        set_env.update(CK_RESIDENT="0", CK_BLOCKED="0")
    elif path == "resident":
        set_env["CK_RESIDENT"] = "1"
    elif path == "blocked":
        set_env.update(CK_RESIDENT="0", CK_BLOCKED="1")
    elif path == "blocked_both":
        set_env.update(CK_RESIDENT="0", CK_BLOCKED="2")
    saved = {k: os.environ.get(k) for k in set_env}
    os.environ.update(set_env)
    try:
        g = sgr.SparseGraph(to_dev(w.src), to_dev(w.dst), w.num_nodes, to_dev(w.input_nodes))
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    if path is not None:
        assert sgr.recurrence_path(g, w.B) == path, f"requested {path} kernels are not taken"
    return g


def run_gpu(w, G=None, graph=None, backward=True, path=None):
    """Forward (+ backward with grad_out G, default w.grad_out) on the GPU."""
    g = make_graph(w, path) if graph is None else graph
    ev, lk, bs = to_dev(w.edge_values), to_dev(w.leak), to_dev(w.bias)
    dr, st = to_dev(w.drives), to_dev(w.state0)
    out, saved, ws = sgr.recurrence_forward(g, ev, lk, bs, dr, st, w.microsteps)
    res = {"out": out}
    if backward:
        Gd = to_dev(w.grad_out if G is None else G, torch.float32)
        res.update(sgr.recurrence_backward(g, ev, lk, st, w.microsteps, saved, Gd, workspace=ws))
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in res.items()}


def run_oracle(w, G=None, cols=None, backward=True, nthreads=0, precision="f64", order=None):
    """Oracle on all batch columns, or only on `cols` (columns are independent).
    precision="f32" with order="sorted" is the fp32 evaluation in the kernels'
    summation order."""
    dr, st = w.drives, w.state0
    Gx = w.grad_out if G is None else G
    if cols is not None:
        cols = np.asarray(cols)
        dr, st, Gx = dr[:, :, cols], st[cols], Gx[:, cols]
    return oracle.run(w.src, w.dst, w.num_nodes, w.input_nodes, w.edge_values, w.leak, w.bias,
                      dr, st, w.microsteps, grad_out=Gx if backward else None, nthreads=nthreads,
                      precision=precision, order=order)


def compare(name, got, want, rtol, atol, want32=None):
    """Per-element parity of `got` against the fp64 oracle `want`; see the
    criterion at the top.  want32: the fp32 evaluation in the kernels'
    summation order (required only if some element misses the bound)."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (name, got.shape, want.shape)
    if got.size == 0:
        return
    bound = atol + rtol * np.abs(want)
    err = np.abs(got - want)
    bad = int(np.sum(err > bound))
    mx, p99 = float(err.max()), float(np.quantile(err, 0.99))
    msg = f"  {name:14s} n={got.size:>10d} outside_bound={bad} max_abs={mx:.3e} p99_abs={p99:.3e}"
    if want32 is not None:
        e32 = np.abs(np.asarray(want32, np.float64) - want)
        bad32, bad32x2 = int(np.sum(e32 > bound)), int(np.sum(2 * e32 > bound))
        mx32, p9932 = float(e32.max()), float(np.quantile(e32, 0.99))
        msg += (f" | fp32 evaluation: outside_bound={bad32} (errors doubled: {bad32x2}) "
                f"max_abs={mx32:.3e} p99_abs={p9932:.3e}")
    log(msg)
    if bad == 0:
        return
    i = np.unravel_index(np.argmax(err - bound), err.shape)
    where = f"worst at {i}: got {got[i]!r} want {want[i]!r}"
    assert want32 is not None, f"{name}: {bad} of {got.size} elements outside atol={atol} rtol={rtol}; {where}"
    assert bad <= bad32x2, (f"{name}: {bad} elements outside the bound, the fp32 evaluation "
                            f"{bad32} ({bad32x2} with its errors doubled); {where}")
    assert p99 <= 2 * p9932, f"{name}: p99 error {p99:.3e} above twice the fp32 evaluation's {p9932:.3e}"
    assert mx <= 2 * mx32, f"{name}: max error {mx:.3e} above twice the fp32 evaluation's {mx32:.3e}"


def _sampled(gpu, k, cols):
    g = gpu[k]
    if cols is not None:
        if k == "out":
            g = g[:, cols]
        elif k == "g_drives":
            g = g[:, :, cols]
        elif k == "g_state0":
            g = g[cols]
    return g


def check_parity(gpu, w, G=None, cols=None, backward=True):
    """Outputs (and the five gradients) of a GPU run against the oracle on
    the same inputs, on all batch columns or the sampled `cols`; the fp32
    evaluation in the kernels' summation order is computed only if some
    element misses the stated bound."""
    ref = run_oracle(w, G=G, cols=cols, backward=backward)
    keys = ("out",) + (GRAD_KEYS if backward else ())
    tol = {k: (STATE_RTOL, STATE_ATOL) if k == "out" else (GRAD_RTOL, GRAD_ATOL) for k in keys}

    def misses(k):
        rt, at = tol[k]
        g = np.asarray(_sampled(gpu, k, cols), np.float64)
        return g.size and bool(np.any(np.abs(g - ref[k]) > at + rt * np.abs(ref[k])))

    ref32 = None
    if any(misses(k) for k in keys):
        ref32 = run_oracle(w, G=G, cols=cols, backward=backward, precision="f32", order="sorted")
    for k in keys:
        compare(k, _sampled(gpu, k, cols), ref[k], *tol[k],
                want32=None if ref32 is None else ref32[k])


def check_outputs_all_columns(gpu_out, w):
    """`out` of a GPU run against a forward-only oracle run on every batch column."""
    ref = run_oracle(w, backward=False)
    ref32 = None
    if np.any(np.abs(gpu_out - ref["out"]) > STATE_ATOL + STATE_RTOL * np.abs(ref["out"])):
        ref32 = run_oracle(w, backward=False, precision="f32", order="sorted")
    compare("out (all cols)", gpu_out, ref["out"], STATE_RTOL, STATE_ATOL,
            want32=None if ref32 is None else ref32["out"])


def column_masked_grad(w, cols):
    """grad_out that is zero outside batch columns `cols` (the gradient then
    only depends on those columns, so a column-sampled oracle is exact)."""
    G = np.zeros_like(w.grad_out)
    G[:, cols] = w.grad_out[:, cols]
    return G
