"""GPU checks specific to the XCD-resident kernels (one launch per call, each
XCD computing one group of 4 batch columns): which calls take them, and the
failure path of their bounded waits, forced from the host.

Parity of the resident kernels against the oracle is covered, path by path,
in test_gpu_parity.py."""
import numpy as np
import pytest
import torch

import sparse_graph_recurrent_amd as sgr
import synthetic
from gpu_helpers import check_parity, log, make_graph, run_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_path_selection():
    """Graphs of up to 9184 nodes take the resident kernels at every batch
    width (beyond 32 columns each XCD computes several column groups in
    turn), graphs of 100,000 nodes and more the blocked forward (and the
    per-microstep backward) from 5 to 64 columns, the rest the per-microstep
    kernels; CK_RESIDENT=0 and CK_BLOCKED=0 at creation turn the first two
    off, CK_BLOCKED=2 makes the backward blocked too."""
    w = synthetic.make("flygpt", T=2)
    g = make_graph(w)
    log("path selection: flygpt graph")
    assert [sgr.recurrence_path(g, B) for B in (1, 8, 20, 32, 33, 64, 100)] == ["resident"] * 7
    assert sgr.recurrence_path(make_graph(w, env={"CK_RESIDENT": "0"}), 32) == "per_microstep"
    # the resident kernels address a step's [B][N] and [n_in][B] tensors with
    # 32-bit byte offsets: a batch that puts N * B * 4 past 2^31 (while N * Bp
    # stays below 2^30) takes the per-microstep kernels
    assert 5000 * 110_000 * 4 >= 2**31 and 5000 * 110_000 < 2**30
    assert sgr.recurrence_path(g, 110_000) == "per_microstep"
    big = synthetic.make("mid_scale", T=1)
    log("path selection: mid-scale graph")
    assert sgr.recurrence_path(make_graph(big), 32) == "per_microstep"
    # graphs of 100,000 nodes and more take the blocked kernels from 5 to 64
    # batch columns; CK_BLOCKED=0 at creation turns them off
    huge = synthetic.random_graph(np.random.default_rng(5), 100_000, 200_000, 16, B=8, T=1, M=1)
    log("path selection: 100,000-node graph")
    gh = make_graph(huge)
    assert ([sgr.recurrence_path(gh, B) for B in (4, 5, 32, 64, 65)]
            == ["per_microstep"] + ["blocked"] * 3 + ["per_microstep"])
    assert sgr.recurrence_path(make_graph(huge, env={"CK_BLOCKED": "0"}), 32) == "per_microstep"
    g2 = make_graph(huge, env={"CK_BLOCKED": "2"})
    assert ([sgr.recurrence_path(g2, B) for B in (4, 5, 64, 65)]
            == ["per_microstep", "blocked_both", "blocked_both", "per_microstep"])


def test_largest_resident_graph():
    """At the node limit, 9,184 nodes, a workgroup's LDS holds the state plane
    with its 16 zero rows and the partial sums in all but a few hundred of the
    CU's 160 KiB: the resident kernels still match the oracle there, and one
    node more takes the per-microstep kernels."""
    rng = np.random.default_rng(9184)
    w = synthetic.random_graph(rng, 9184, 120_000, 64, B=8, T=2, M=2, v_scale=0.2)
    g = make_graph(w)
    assert sgr.recurrence_path(g, 8) == "resident"
    log("parity: largest resident graph, N=9184 E=120000 B=8")
    check_parity(run_gpu(w, graph=g), w)
    w2 = synthetic.random_graph(np.random.default_rng(9185), 9185, 1000, 4, B=1, T=1, M=1)
    assert sgr.recurrence_path(make_graph(w2), 8) == "per_microstep"


def test_failed_wait_poisons_every_output():
    """With every wait of the resident kernels forced to give up at once
    (CK_RESIDENT_SPIN_LIMIT=-1 at creation; the kernels still run to their
    end), forward and backward report the failure as NaN in every output and
    as CK_ERR_WAIT from ck_recurrence_status; a backward on a healthy graph
    given the saved arena of the failed forward does too (the arena carries
    the forward's status), and so does the autograd wrapper.  A graph created
    afterwards computes correctly again."""
    w = synthetic.make("tiny")
    log("resident failure path: all waits give up")
    g = make_graph(w, "resident", env={"CK_RESIDENT_SPIN_LIMIT": "-1"})
    bad = run_gpu(w, graph=g)
    for k, v in bad.items():
        assert np.isnan(v).all(), k
    ev, lk, bs, dr, st, G = (to_dev(x) for x in (w.edge_values, w.leak, w.bias, w.drives,
                                                  w.state0, w.grad_out))
    out, saved, ws = sgr.recurrence_forward(g, ev, lk, bs, dr, st, w.microsteps)
    with pytest.raises(sgr.CkError) as ei:
        sgr.recurrence_status(g, w.T, w.B, w.microsteps, ws)
    assert ei.value.status == 10
    log("resident failure path: healthy backward given the failed forward's arena")
    good = make_graph(w, "resident")
    ws2 = torch.empty(sgr.recurrence_sizes(good, w.T, w.B, w.microsteps)[1], dtype=torch.uint8,
                      device="cuda")
    grads = sgr.recurrence_backward(good, ev, lk, st, w.microsteps, saved, G, workspace=ws2)
    for k, v in grads.items():
        assert torch.isnan(v).all().item(), k
    with pytest.raises(sgr.CkError) as ei:
        sgr.recurrence_status(good, w.T, w.B, w.microsteps, ws2)
    assert ei.value.status == 10
    log("resident failure path: autograd wrapper raises")
    ins = [x.clone().requires_grad_() for x in (ev, lk, bs, dr, st)]
    with pytest.raises(sgr.CkError) as ei:
        sgr.sparse_recurrence(*ins, g, microsteps=w.microsteps)
    assert ei.value.status == 10
    log("resident failure path: healthy graph afterwards")
    check_parity(run_gpu(w, graph=good), w)
    out, saved, ws = sgr.recurrence_forward(good, ev, lk, bs, dr, st, w.microsteps)
    sgr.recurrence_status(good, w.T, w.B, w.microsteps, ws)


def test_paths_agree_on_flygpt():
    """The two kernel families compute the same sums in different orders:
    on the FlyGPT launch shape they agree to the state / gradient
    tolerances."""
    w = synthetic.make("flygpt", T=8)
    log("resident vs per-microstep: flygpt shape, T=8")
    a = run_gpu(w, path="resident")
    b = run_gpu(w, path="per_microstep")
    np.testing.assert_allclose(a["out"], b["out"], rtol=1e-5, atol=1e-6)
    for k in ("g_edge_values", "g_leak", "g_bias", "g_drives", "g_state0"):
        scale = np.sqrt(np.mean(b[k].astype(np.float64) ** 2))
        np.testing.assert_allclose(a[k], b[k], rtol=1e-4, atol=1e-6 + 1e-5 * scale, err_msg=k)
