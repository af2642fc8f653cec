"""GPU parity of the fixed-point LIF forward (ck_lif_forward, through the C
ABI) against the LIF oracle (oracle/lif_oracle.c): integer arithmetic, so
spikes and potentials must be bit-exact, and a rejected overflow must be
reported at the same timestep.  Workloads: the hand-worked timeline, small
random graphs with delays up to 9 steps, the soup-connectome page's standard
and stress runs re-read on the synthetic whole-connectome graph, and an
active run on that graph (hubs of in-degree up to 20,000, delays 1..4)."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import sparse_graph_recurrent_amd as sgr
import synthetic
from gpu_helpers import log, to_dev

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))
I32_MAX = 2**31 - 1


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sgr.lib()


def _graph(src, dst, N):
    return sgr.SparseGraph(to_dev(np.asarray(src, np.int64)), to_dev(np.asarray(dst, np.int64)), N,
                           to_dev(np.zeros(0, np.int64)))


def _both(src, dst, N, w, d, v0, T, thr, reset, refr, shifts, graph=None):
    g = _graph(src, dst, N) if graph is None else graph
    s, p = sgr.lif_forward(g, to_dev(np.asarray(w, np.int16)), to_dev(np.asarray(d, np.int32)),
                           to_dev(np.asarray(v0, np.int32)), T, thr, reset, refr, shifts)
    s, p = s.cpu().numpy(), p.cpu().numpy()
    s2, p2 = oracle.lif_run(src, dst, N, w, d, v0, T, thr, reset, refr, shifts)
    np.testing.assert_array_equal(s, s2)
    np.testing.assert_array_equal(p, p2)
    return s


def test_hand_worked_timeline():
    g = json.load(open(os.path.join(HERE, "golden", "lif_timeline.json")))
    log("LIF: hand-worked timeline")
    s = _both(g["src"], g["dst"], g["num_nodes"], g["impulse"], g["delay"], g["v0"], g["T"],
              g["threshold"], g["reset"], g["refractory_steps"], g["decay_shifts"])
    np.testing.assert_array_equal(s, np.array(g["spikes"], np.uint8))


@pytest.mark.parametrize("seed,N,E,max_delay,refr,shifts,active", [
    (1, 50, 900, 1, 0, [2], True), (2, 300, 9000, 9, 2, [1, 4], True),
    (3, 1000, 4000, 3, 1, [], True), (4, 129, 5000, 5, 3, [0], False),
    (5, 2000, 60000, 7, 2, [3, 31], True)])
def test_random_graphs(seed, N, E, max_delay, refr, shifts, active):
    """(shift 0 zeroes every potential before the impulses arrive: no neuron
    ever reaches the threshold there.)"""
    rng = np.random.default_rng(seed)
    src, dst = rng.integers(0, N, E), rng.integers(0, N, E)   # parallel edges, self-loops
    w = (np.where(rng.random(E) < 0.8, 1, -1) * rng.integers(1, 120, E)).astype(np.int16)
    d = rng.integers(1, max_delay + 1, E).astype(np.int32)
    v0 = rng.integers(-200, 600, N).astype(np.int32)
    log(f"LIF: random graph N={N} E={E} delays<={max_delay}")
    s = _both(src, dst, N, w, d, v0, 20, 100, -20, refr, shifts)
    assert (s[10:].sum() > 0) == active


def _random_case(seed, N, E, max_delay, T=20, refr=2, shifts=(2,)):
    rng = np.random.default_rng(seed)
    src, dst = rng.integers(0, N, E), rng.integers(0, N, E)
    w = (np.where(rng.random(E) < 0.8, 1, -1) * rng.integers(1, 120, E)).astype(np.int16)
    d = rng.integers(1, max_delay + 1, E).astype(np.int32)
    v0 = rng.integers(-200, 600, N).astype(np.int32)
    return _both(src, dst, N, w, d, v0, T, 100, -20, refr, list(shifts))


@pytest.mark.parametrize("seed,N,E,max_delay", [
    (11, 33, 700, 2), (12, 65, 2000, 16), (13, 300, 9000, 9), (14, 2000, 60000, 7)])
def test_byte_lookups_match(seed, N, E, max_delay, monkeypatch):
    """The same runs with the spike lookups forced to one byte read of the
    spike history per edge (CK_LIF_LDS=0) instead of LDS bit rows."""
    monkeypatch.setenv("CK_LIF_LDS", "0")
    log(f"LIF: byte lookups, N={N} E={E} delays<={max_delay}")
    s = _random_case(seed, N, E, max_delay)
    assert s[10:].sum() > 0


@pytest.mark.parametrize("seed,N,E,max_delay,T", [
    (21, 33, 700, 2, 20),          # ragged last ballot word (N = 32 + 1)
    (22, 65, 2000, 16, 40),        # the longest delay the bit ring holds
    (23, 400, 8000, 17, 40),       # one step past it: byte lookups
    (24, 600, 9000, 40, 60),       # delays far past it
    (25, 262144, 1000000, 4, 8),   # 4 bit rows of 8,192 words: exactly 128 KB of LDS
    (26, 262176, 1000000, 4, 8)])  # one word more per row: byte lookups
def test_lookup_boundaries(seed, N, E, max_delay, T):
    """Cases on both sides of the limits that pick the spike lookup (largest
    delay 16, 128 KB of bit rows), bit-exact against the oracle."""
    log(f"LIF: lookup boundary N={N} E={E} delays<={max_delay} T={T}")
    s = _random_case(seed, N, E, max_delay, T=T)
    assert s[1:].sum() > 0


@pytest.mark.parametrize("E", [1, 2, 3, 5, 127, 129, 255, 257, 4095, 4097, 6145, 8193, 12289])
def test_odd_and_ragged_edge_counts(E):
    """The LDS-lookup gather reads four positions per lane in two 16-byte
    loads and walks the positions in chunks of 4,096: edge counts that leave
    the last group of four partly past the records, and counts just around a
    group, a wave's 256 positions and a chunk, bit-exact against the
    oracle."""
    log(f"LIF: edge count {E}")
    N = 64 if E < 100 else 300
    rng = np.random.default_rng(E)
    src, dst = rng.integers(0, N, E), rng.integers(0, N, E)
    w = rng.integers(30, 120, E).astype(np.int16)
    d = rng.integers(1, 4, E).astype(np.int32)
    v0 = rng.integers(0, 100, N).astype(np.int32)
    _both(src, dst, N, w, d, v0, 12, 100, 0, 1, [3])


@pytest.mark.parametrize("gap", [2, 63, 4096])
def test_empty_row_gaps(gap):
    """In-edges into rows 0, gap, 2 gap, 2 gap + 2 and 3 gap + 2 only: long
    runs of rows without edges between the rows whose runs a wave sums."""
    rng = np.random.default_rng(gap)
    rows = np.array([0, gap, 2 * gap, 2 * gap + 2, 3 * gap + 2], np.int64)
    N = int(rows[-1]) + 10
    E = 5000
    dst = rows[rng.integers(0, rows.size, E)]
    src = np.concatenate([rows, rng.integers(0, N, E - rows.size)])
    w = (np.where(rng.random(E) < 0.8, 1, -1) * rng.integers(1, 120, E)).astype(np.int16)
    d = rng.integers(1, 5, E).astype(np.int32)
    v0 = rng.integers(-200, 600, N).astype(np.int32)
    v0[rows] = 500
    log(f"LIF: empty-row gap {gap}")
    s = _both(src, dst, N, w, d, v0, 12, 100, -20, 1, [2])
    assert s[1:, rows].sum() > 0


@pytest.fixture(scope="module")
def connectome():
    w = synthetic.make_lif("connectome")
    g = _graph(w.src, w.dst, w.num_nodes)
    return w, g


def test_pages_standard_run_on_connectome(connectome):
    """threshold 20000, reset 0, decay_shifts [2], refractory 2, 4 steps,
    neuron 0 seeded at 30000 (soup-connectome, "Full-scale benchmark")."""
    w, g = connectome
    v0 = np.zeros(w.num_nodes, np.int32)
    v0[0] = 30000
    log("LIF: the page's standard run on the synthetic connectome")
    s = _both(w.src, w.dst, w.num_nodes, w.impulses, w.delays, v0, 4, 20000, 0, 2, [2], graph=g)
    assert s.sum(axis=1).tolist() == [1, 0, 0, 0]


def test_pages_stress_run_on_connectome(connectome):
    """threshold 1, reset 0, decay_shifts [31], refractory 0, 2 steps (the
    page's active stress configuration)."""
    w, g = connectome
    v0 = np.zeros(w.num_nodes, np.int32)
    v0[0] = 30000
    log("LIF: the page's stress run on the synthetic connectome")
    s = _both(w.src, w.dst, w.num_nodes, w.impulses, w.delays, v0, 2, 1, 0, 0, [31], graph=g)
    log(f"  spike counts {s.sum(axis=1).tolist()}")
    assert s[0].sum() == 1 and s[1].sum() > 0


def test_active_run_on_connectome():
    """A run that stays active: 12-48 % of the 211,577 neurons spike per step,
    delays 1..4, hubs of in-degree up to 20,000."""
    w = synthetic.make_lif("connectome", max_delay=4, v0_range=(0, 60))
    log("LIF: active run on the synthetic connectome, 16 steps")
    s = _both(w.src, w.dst, w.num_nodes, w.impulses, w.delays, w.v0, 16, 40, 0, 2, [2])
    log(f"  spike counts {s.sum(axis=1).tolist()}")
    assert (s.sum(axis=1) > 1000).all()


@pytest.mark.parametrize("lookups", ["lds", "bytes"])
def test_prepare_then_runs(lookups, monkeypatch):
    """ck_lif_prepare once, then ck_lif_run several times from different
    initial potentials and parameters: each run equals the oracle bit for
    bit, with either spike lookup."""
    if lookups == "bytes":
        monkeypatch.setenv("CK_LIF_LDS", "0")
    rng = np.random.default_rng(61)
    N, E = 3000, 80000
    src, dst = rng.integers(0, N, E), rng.integers(0, N, E)
    w = (np.where(rng.random(E) < 0.8, 1, -1) * rng.integers(1, 120, E)).astype(np.int16)
    d = rng.integers(1, 6, E).astype(np.int32)
    g = _graph(src, dst, N)
    log(f"LIF: prepare once, three runs ({lookups} lookups)")
    ws = sgr.lif_prepare(g, to_dev(w), to_dev(d))
    for k, (thr, refr, shifts) in enumerate(((100, 2, [2]), (60, 0, [1, 3]), (150, 3, []))):
        v0 = rng.integers(-200, 600, N).astype(np.int32)
        s, p = sgr.lif_run(g, ws, to_dev(v0), 12, thr, -20, refr, shifts)
        s2, p2 = oracle.lif_run(src, dst, N, w, d, v0, 12, thr, -20, refr, shifts)
        np.testing.assert_array_equal(s.cpu().numpy(), s2, err_msg=f"run {k}")
        np.testing.assert_array_equal(p.cpu().numpy(), p2, err_msg=f"run {k}")
        assert s2[6:].sum() > 0


def test_run_needs_prepared_synapses_of_the_graph():
    rng = np.random.default_rng(62)
    src, dst = rng.integers(0, 500, 4000), rng.integers(0, 500, 4000)
    g, g2 = _graph(src, dst, 500), _graph(src, dst, 500)
    w = to_dev(np.full(4000, 7, np.int16))
    d = to_dev(np.ones(4000, np.int32))
    v0 = to_dev(np.zeros(500, np.int32))
    fresh = sgr.lif_workspace(g)
    fresh.zero_()
    with pytest.raises(sgr.CkError) as ei:
        sgr.lif_run(g, fresh, v0, 3, 10, 0, 0, [])
    assert ei.value.status == 12
    ws = sgr.lif_prepare(g, w, d)
    sgr.lif_run(g, ws, v0, 3, 10, 0, 0, [])
    with pytest.raises(sgr.CkError) as ei:   # prepared for another graph of the same size
        sgr.lif_run(g2, ws, v0, 3, 10, 0, 0, [])
    assert ei.value.status == 12
    with pytest.raises(sgr.CkError) as ei:   # a failed prepare leaves no synapses behind
        sgr.lif_prepare(g, w, to_dev(np.zeros(4000, np.int32)), workspace=ws)
    assert ei.value.status == 12
    with pytest.raises(sgr.CkError) as ei:
        sgr.lif_run(g, ws, v0, 3, 10, 0, 0, [])
    assert ei.value.status == 12


@pytest.mark.parametrize("sign", [1, -1])
def test_overflow_is_rejected_at_the_same_step(sign):
    v0 = [I32_MAX, sign * (I32_MAX - 500), 5]
    src, dst, w, d = [0, 0], [1, 2], [sign * 1000, 3], [3, 1]
    with pytest.raises(oracle.LifOverflow) as eo:
        oracle.lif_run(src, dst, 3, w, d, v0, 6, I32_MAX, 0, 0, [])
    log(f"LIF: overflow ({'up' if sign > 0 else 'down'}) at step {eo.value.step}")
    g = _graph(src, dst, 3)
    with pytest.raises(sgr.CkError) as ei:
        sgr.lif_forward(g, to_dev(np.asarray(w, np.int16)), to_dev(np.asarray(d, np.int32)),
                        to_dev(np.asarray(v0, np.int32)), 6, I32_MAX, 0, 0, [])
    assert ei.value.status == 11 and ei.value.step == eo.value.step == 3


def test_invalid_values_are_rejected():
    g = _graph([0, 1], [1, 0], 2)
    w = to_dev(np.array([5, 5], np.int16))
    v0 = to_dev(np.zeros(2, np.int32))
    for d, shifts, refr in (([0, 1], [2], 0), ([1, 40000], [2], 0), ([1, 1], [32], 0),
                            ([1, 1], [2], -1), ([1, 1], list(range(9)), 0)):
        with pytest.raises((sgr.CkError, ValueError)) as ei:
            sgr.lif_forward(g, w, to_dev(np.asarray(d, np.int32)), v0, 3, 10, 0, refr, shifts)
        if isinstance(ei.value, sgr.CkError):
            assert ei.value.status == 12


def test_misaligned_workspace_is_rejected():
    """A workspace 16 bytes into an allocation (not on a 256-byte boundary)
    is rejected with CK_ERR_BAD_VALUE before any work is queued."""
    g = _graph([0, 1], [1, 0], 2)
    w = to_dev(np.array([5, 5], np.int16))
    d = to_dev(np.array([1, 1], np.int32))
    v0 = to_dev(np.zeros(2, np.int32))
    ws = sgr.lif_workspace(g)
    big = torch.empty(ws.numel() + 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(sgr.CkError) as ei:
        sgr.lif_forward(g, w, d, v0, 3, 10, 0, 0, [2], workspace=big[16:])
    assert ei.value.status == 12


def test_graph_without_edges():
    log("LIF: graph without edges")
    _both([], [], 7, [], [], [0, 5, 10, 15, 20, -3, 99], 5, 12, 1, 1, [1])
