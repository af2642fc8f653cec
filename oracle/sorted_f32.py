"""A second fp32 evaluation of the recurrence, in a different summation order.

TEST INFRASTRUCTURE ONLY, used to measure the fp32 rounding floor, never as a
parity reference.  It evaluates the same definition as ``ck_oracle.c``
(connectome-kernels README, introduction: the proposal and the leaky update,
repeated `microsteps` times per input step; the gradient of
L = sum(out * G) with respect to edge values, leak, bias, drives and initial
state), entirely in float32, with scipy's sparse matrix products: each node's
incoming (forward) and outgoing (transposed product) terms are summed in
sorted index order, where the C oracle sums them in the caller's edge order.
Two fp32 evaluations that differ only in summation order bracket how far fp32
arithmetic alone can move a result; on ill-conditioned workloads (large
hubs, mostly positive weights) that spread is several-fold.
"""
from __future__ import annotations

import numpy as np
import scipy.sparse as sp


def run(src, dst, num_nodes, input_nodes, edge_values, leak, bias, drives, state0, microsteps,
        grad_out):
    """Forward and gradient in float32.  Layouts as the C oracle: drives
    [T][n_in][B], state0 [B][N], grad_out [T][B][N]; returns a dict with
    out [T][B][N], g_edge_values [E] (caller order), g_leak [N], g_bias [N],
    g_drives [T][n_in][B], g_state0 [B][N] (float64 copies of fp32 values)."""
    f = np.float32
    N = int(num_nodes)
    src = np.asarray(src, np.int64)
    dst = np.asarray(dst, np.int64)
    src32, dst32 = src.astype(np.int32), dst.astype(np.int32)
    inputs = np.asarray(input_nodes, np.int64)
    v = np.asarray(edge_values, f)
    T, n_in, B = np.asarray(drives).shape
    M = int(microsteps)
    S = T * M
    # W[dst, src] = v (parallel edges add); its transpose for the state gradient
    W = sp.csr_matrix((v, (dst, src)), shape=(N, N), dtype=f)
    WT = sp.csr_matrix(W.T, dtype=f)
    lam = np.asarray(leak, f)[:, None]
    beta = np.asarray(bias, f)[:, None]
    drv = np.asarray(drives, f)
    G = np.asarray(grad_out, f)

    # forward: a = W h + drive + bias; h' = (1 - leak) h + leak tanh(a)
    h = [np.asarray(state0, f).T.copy()]  # [N][B]
    a = []
    out = np.empty((T, B, N), f)
    for s in range(1, S + 1):
        t = (s - 1) // M
        d = np.zeros((N, B), f)
        d[inputs] = drv[t]
        x = (W @ h[-1]).astype(f) + d + beta
        a.append(x)
        h.append(((f(1) - lam) * h[-1] + lam * np.tanh(x)).astype(f))
        if s % M == 0:
            out[t] = h[-1].T

    # reverse pass over the microsteps
    g = np.zeros((N, B), f)
    gv = np.zeros(len(v), f)
    gl = np.zeros(N, f)
    gb = np.zeros(N, f)
    gd = np.zeros((T, n_in, B), f)
    for s in range(S, 0, -1):
        t = (s - 1) // M
        if s % M == 0:
            g = (g + G[t].T).astype(f)
        x, q = a[s - 1], h[s - 1]
        p = np.tanh(x).astype(f)
        gl += (g * (p - q)).sum(axis=1, dtype=f)
        with np.errstate(over="ignore"):  # cosh -> inf gives sech^2 = 0, as it should
            c = np.cosh(x.astype(np.float64))
            ga = (g * lam * (1.0 / (c * c)).astype(f)).astype(f)
        gb += ga.sum(axis=1, dtype=f)
        gd[t] += ga[inputs]
        # edge terms sum over the batch columns in ascending order
        d = np.zeros(len(v), f)
        for b in range(B):
            d += np.take(np.ascontiguousarray(ga[:, b]), dst32) * np.take(np.ascontiguousarray(q[:, b]), src32)
        gv += d
        g = ((f(1) - lam) * g + (WT @ ga).astype(f)).astype(f)
    d64 = lambda x: np.asarray(x, np.float64)
    return {"out": d64(out), "g_edge_values": d64(gv), "g_leak": d64(gl), "g_bias": d64(gb),
            "g_drives": d64(gd), "g_state0": d64(g.T)}
