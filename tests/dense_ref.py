"""Dense brute-force formulations used to pin the CPU oracle.

Independent of the oracle's edge-loop code: the sparse weight matrix is
materialised as a dense [N, N] array (an edge src -> dst adds its value to
W[dst, src]; connectome-kernels README, "Use") and every microstep is a dense
matrix product in the [B, N] layout, following the README's two update
equations (introduction).  The gradient comes from torch autograd on the same
dense formulation, not from a hand derivation.
"""
from __future__ import annotations

import numpy as np
import torch


def dense_forward(N, src, dst, input_nodes, v, leak, bias, drives, state0, M):
    src = np.asarray(src, np.int64)
    dst = np.asarray(dst, np.int64)
    inp = np.asarray(input_nodes, np.int64)
    W = np.zeros((N, N))
    np.add.at(W, (dst, src), np.asarray(v, np.float64))
    leak = np.asarray(leak, np.float64)
    bias = np.asarray(bias, np.float64)
    drives = np.asarray(drives, np.float64)
    h = np.array(state0, np.float64)
    T, B = drives.shape[0], h.shape[0]
    out = np.zeros((T, B, N))
    for t in range(T):
        d = np.zeros((B, N))
        d[:, inp] = drives[t].T
        for _ in range(M):
            a = h @ W.T + d + bias
            h = (1.0 - leak) * h + leak * np.tanh(a)
        out[t] = h
    return out


def torch_dense_grads(N, src, dst, input_nodes, v, leak, bias, drives, state0, M, G):
    """Loss sum(out * G) and its gradient wrt all five inputs, via autograd (fp64, CPU)."""
    f64 = torch.float64
    src_t = torch.as_tensor(np.asarray(src, np.int64))
    dst_t = torch.as_tensor(np.asarray(dst, np.int64))
    inp = torch.as_tensor(np.asarray(input_nodes, np.int64))
    v_t = torch.tensor(np.asarray(v, np.float64), dtype=f64, requires_grad=True)
    lk = torch.tensor(np.asarray(leak, np.float64), dtype=f64, requires_grad=True)
    bs = torch.tensor(np.asarray(bias, np.float64), dtype=f64, requires_grad=True)
    dr = torch.tensor(np.asarray(drives, np.float64), dtype=f64, requires_grad=True)
    h0 = torch.tensor(np.asarray(state0, np.float64), dtype=f64, requires_grad=True)
    W = torch.zeros((N, N), dtype=f64).index_put((dst_t, src_t), v_t, accumulate=True)
    T, B = dr.shape[0], h0.shape[0]
    h = h0
    outs = []
    for t in range(T):
        d = torch.zeros((B, N), dtype=f64).index_put((torch.arange(B).repeat_interleave(inp.numel()),
                                                       inp.repeat(B)), dr[t].T.reshape(-1))
        for _ in range(M):
            a = h @ W.T + d + bs
            h = (1.0 - lk) * h + lk * torch.tanh(a)
        outs.append(h)
    out = torch.stack(outs)
    loss = (out * torch.as_tensor(np.asarray(G, np.float64))).sum()
    loss.backward()
    def grad(x):
        return x.grad.numpy() if x.grad is not None else np.zeros(tuple(x.shape))
    return {
        "out": out.detach().numpy(), "loss": float(loss.detach()),
        "g_edge_values": grad(v_t), "g_leak": grad(lk), "g_bias": grad(bs),
        "g_drives": grad(dr), "g_state0": grad(h0),
    }
