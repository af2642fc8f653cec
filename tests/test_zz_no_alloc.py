"""The allocation-free forward (ck_recurrence_forward_noalloc, fixed device
scratch) against the workspace forward (ck_recurrence_forward) through the C
ABI: the same kernels, so outputs and the gradients computed from the two
saved arenas must agree bit for bit,
on two calls in a row (the second with a smaller input, so stale scratch
from the first must not leak into it), on both kernel families; the saved
arena it writes serves the backward unchanged; and a forward that needs more
scratch than the fixed array holds is rejected."""
import numpy as np
import pytest
import torch

import sparse_graph_recurrent_amd as sgr
import synthetic
from gpu_helpers import log, make_graph, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sgr.lib()


def _both(w, g):
    ev, lk, bs, dr, st = (to_dev(x) for x in (w.edge_values, w.leak, w.bias, w.drives, w.state0))
    sb, _ = sgr.recurrence_sizes(g, w.T, w.B, w.microsteps)
    out_a, saved_a, ws = sgr.recurrence_forward(g, ev, lk, bs, dr, st, w.microsteps)
    out_b = torch.full_like(out_a, 5.0)
    saved_b = torch.full((sb,), 7, dtype=torch.uint8, device="cuda")
    sgr.recurrence_forward_noalloc(g, ev, lk, bs, dr, st, w.microsteps, out_b, saved_b)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out_b.cpu().numpy(), out_a.cpu().numpy())
    # (the arenas' padding bytes are never written; the backward below reads
    # every byte that was, from each arena)
    G = to_dev(w.grad_out)
    ga = sgr.recurrence_backward(g, ev, lk, st, w.microsteps, saved_a, G, workspace=ws)
    gb = sgr.recurrence_backward(g, ev, lk, st, w.microsteps, saved_b, G)
    torch.cuda.synchronize()
    for k in ga:
        np.testing.assert_array_equal(gb[k].cpu().numpy(), ga[k].cpu().numpy(), err_msg=k)


@pytest.mark.parametrize("path", ["resident", "per_microstep", "blocked"])
def test_noalloc_forward_matches_workspace_forward(path):
    big = synthetic.make("flygpt", T=6)
    log(f"no-alloc forward: flygpt graph T=6 B=32, {path} kernels")
    _both(big, make_graph(big, path))
    rng = np.random.default_rng(31)
    small = synthetic.random_graph(rng, 700, 9000, 11, B=5, T=3, M=3, v_scale=0.2)
    log(f"no-alloc forward: smaller graph N=700 B=5, {path} kernels")
    _both(small, make_graph(small, path))


def test_noalloc_forward_rejects_oversized_scratch():
    w = synthetic.make("mid_scale", T=1, B=4)
    w.src = np.concatenate([w.src] * 3)
    w.dst = np.concatenate([w.dst] * 3)
    w.edge_values = np.concatenate([w.edge_values] * 3)
    log("no-alloc forward: 15M-edge graph needs more than the fixed scratch")
    g = make_graph(w)
    ev, lk, bs, dr, st = (to_dev(x) for x in (w.edge_values, w.leak, w.bias, w.drives, w.state0))
    sb, _ = sgr.recurrence_sizes(g, w.T, w.B, w.microsteps)
    out = torch.empty((w.T, w.B, w.num_nodes), dtype=torch.float32, device="cuda")
    saved = torch.empty(sb, dtype=torch.uint8, device="cuda")
    with pytest.raises(sgr.CkError) as ei:
        sgr.recurrence_forward_noalloc(g, ev, lk, bs, dr, st, w.microsteps, out, saved)
    assert ei.value.status == 5
