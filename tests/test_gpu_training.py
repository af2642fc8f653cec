"""End-to-end use of the autograd wrapper: a small training loop.

The caller-side parametrization the connectome-kernels README leaves to the
caller ("Use": sigmoid leak, signs, scaling) is written here in plain torch:
edge weights are sign * softplus(raw) / sqrt(in-degree of the target), the
leak is sigmoid(raw leak).  A teacher network with fixed random parameters
produces targets on the same graph; a student with its own initial
parameters is fitted to them with Adam through `sparse_recurrence`, whose
backward is the library's fused backward.  The loss must fall substantially,
and every parameter must receive a finite, non-zero gradient.
"""
import numpy as np
import pytest
import torch

import sparse_graph_recurrent_amd as sgr
import synthetic
from gpu_helpers import log, make_graph

pytestmark = pytest.mark.gpu


def _params(N, E, rng):
    raw_v = torch.tensor(rng.standard_normal(E).astype(np.float32) * 0.5, device="cuda")
    raw_l = torch.tensor(rng.standard_normal(N).astype(np.float32) * 0.5, device="cuda")
    bias = torch.tensor(rng.standard_normal(N).astype(np.float32) * 0.1, device="cuda")
    return raw_v, raw_l, bias


def _forward(raw_v, raw_l, bias, drives, state0, graph, sign, inv_sqrt_deg, M):
    v = sign * torch.nn.functional.softplus(raw_v) * inv_sqrt_deg
    return sgr.sparse_recurrence(v, torch.sigmoid(raw_l), bias, drives, state0, graph,
                                 microsteps=M)


def test_training_loop_reduces_loss():
    w = synthetic.make("tiny", T=6)
    N, E, M = w.num_nodes, w.num_edges, w.microsteps
    g = make_graph(w)
    rng = np.random.default_rng(11)
    sign = torch.tensor(np.where(rng.random(E) < 0.8, 1.0, -1.0).astype(np.float32), device="cuda")
    deg = np.bincount(w.dst, minlength=N)[w.dst].astype(np.float32)
    inv_sqrt_deg = torch.tensor(1.0 / np.sqrt(deg), device="cuda")
    drives = torch.tensor(w.drives, device="cuda")
    state0 = torch.tensor(w.state0, device="cuda")
    with torch.no_grad():
        teacher = _params(N, E, np.random.default_rng(12))
        target = _forward(*teacher, drives, state0, g, sign, inv_sqrt_deg, M)
    student = [p.clone().requires_grad_() for p in _params(N, E, rng)]
    opt = torch.optim.Adam(student, lr=0.05)
    losses = []
    for it in range(60):
        opt.zero_grad()
        out = _forward(*student, drives, state0, g, sign, inv_sqrt_deg, M)
        loss = torch.mean((out - target) ** 2)
        loss.backward()
        if it == 0:
            for name, p in zip(("raw edge values", "raw leak", "bias"), student):
                assert torch.isfinite(p.grad).all() and p.grad.abs().sum() > 0, name
        opt.step()
        losses.append(float(loss))
    log(f"training loop: loss {losses[0]:.4e} -> {losses[-1]:.4e} after {len(losses)} Adam steps")
    assert np.all(np.isfinite(losses))
    assert losses[-1] < 0.25 * losses[0]
