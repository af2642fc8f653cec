"""Host-side checks of the row schedule the per-microstep kernels walk.

The planner (csrc/schedule.cpp, plain C++) is compiled with g++ together with
a small driver and run on synthetic graphs of the benchmark shapes and on
degenerate ones.  Each table is then replayed the way the kernels read it:
segments accumulate edge batches, pieces of split rows go to numbered LDS
slots and the wave holding a row's last piece adds them after the workgroup
barrier.  The replay must reproduce every row sum exactly once, and the table
must stay inside the limits the kernels rely on.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import synthetic

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_graph_recurrent_amd", "csrc")
FIRST, LAST, PIECE, GROUP, COMBINE = 1 << 18, 1 << 19, 1 << 17, 1 << 16, 1 << 12
SLOT_MASK, COUNT_SHIFT, BATCH = 63, 6, 64


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("sched") / "schedule_driver")
    subprocess.run([gxx, "-std=c++17", "-O2", "-Wall", "-Werror", "-I", CSRC, "-o", exe,
                    os.path.join(ROOT, "tests", "schedule_driver.cpp"),
                    os.path.join(CSRC, "schedule.cpp")], check=True)
    return exe


def plan(driver, ptr, cus, waves):
    N = len(ptr) - 1
    text = f"{N} {cus} {waves}\n" + " ".join(map(str, ptr)) + "\n"
    out = subprocess.run([driver], input=text, capture_output=True, text=True, check=True).stdout
    lines = out.split("\n")
    num_wgs, w, KB = map(int, lines[0].split())
    assert w == waves
    tab = np.array(" ".join(lines[1:]).split(), dtype=np.int64).reshape(num_wgs * waves, KB, 4)
    return num_wgs, KB, tab


def replay(driver, major, N, waves, cus=256):
    """Walk the table like the kernels; return (num_wgs, KB, busiest wave's batches)."""
    major = np.asarray(major, dtype=np.int64)
    deg = np.bincount(major, minlength=N).astype(np.int64) if len(major) else np.zeros(N, np.int64)
    ptr = np.concatenate([[0], np.cumsum(deg)])
    num_wgs, KB, tab = plan(driver, ptr.tolist(), cus, waves)
    E = len(major)
    val = np.random.default_rng(0).integers(-1000, 1000, E)  # exact integer sums
    csum = np.concatenate([[0], np.cumsum(val)])
    want = csum[ptr[1:]] - csum[ptr[:-1]]
    got = np.full(N, np.iinfo(np.int64).min)
    cover = np.zeros(E, np.int64)
    owner = np.full(N, -1)
    busiest = 0
    for g in range(num_wgs):
        slots, combiners, has_piece = {}, [], False
        lists = [tab[g * waves + w] for w in range(waves)]
        for w, lst in enumerate(lists):
            acc, nb = 0, 0
            for row, kb, cnt, info in lst.tolist():
                if row < 0:
                    break
                nb += 1
                assert 0 <= row < N and 0 <= cnt <= BATCH
                assert owner[row] in (-1, g), "a row spans workgroups"
                owner[row] = g
                assert ptr[row] <= kb and kb + cnt <= ptr[row + 1]
                if info & FIRST:
                    acc = 0
                acc += int(val[kb:kb + cnt].sum())
                cover[kb:kb + cnt] += 1
                if info & LAST:
                    if info & PIECE:
                        has_piece = True
                        q = info & SLOT_MASK
                        assert q < 2 * waves and q not in slots
                        slots[q] = (row, acc)
                    else:
                        assert got[row] == np.iinfo(np.int64).min, "row finished twice"
                        got[row] = acc
            busiest = max(busiest, nb)
            if lst[0][0] >= 0 and lst[0][3] & COMBINE:
                combiners.append(lst[0].tolist())
        if has_piece:  # every wave must reach the workgroup barrier
            assert all(lst[0][3] & GROUP for lst in lists)
        used = set()
        for row, _, _, info in combiners:
            q1 = info & SLOT_MASK
            n = (info >> COUNT_SHIFT) & SLOT_MASK
            assert 2 <= n <= waves and q1 - n + 1 >= 0
            total = 0
            for q in range(q1 - n + 1, q1 + 1):
                assert slots[q][0] == row, "slot range holds another row"
                total += slots[q][1]
                used.add(q)
            assert got[row] == np.iinfo(np.int64).min, "row finished twice"
            got[row] = total
        assert used == set(slots), "a piece is never combined"
    assert (cover == 1).all(), "every edge exactly once"
    assert (got != np.iinfo(np.int64).min).all(), "every row finished"
    np.testing.assert_array_equal(got, want)
    return num_wgs, KB, busiest


@pytest.mark.parametrize("waves", [8, 16])
@pytest.mark.parametrize("name", ["tiny", "flygpt", "edge_cases"])
def test_workload_schedules(driver, name, waves):
    w = synthetic.make(name, synthetic.DEFAULT_SEEDS[name])
    for major in (w.dst, w.src):
        replay(driver, major, w.num_nodes, waves)


def test_flygpt_balance(driver):
    """FlyGPT shape, 16-wave workgroups: no wave walks more than 3 batches
    (the graph has 2.63 batches per wave on average by destination)."""
    w = synthetic.make("flygpt", synthetic.DEFAULT_SEEDS["flygpt"])
    for major in (w.dst, w.src):
        num_wgs, KB, busiest = replay(driver, major, w.num_nodes, 16)
        assert num_wgs == 256 and busiest <= 3


@pytest.mark.parametrize("waves", [8, 16])
@pytest.mark.parametrize("cus", [256, 8, 1])
@pytest.mark.parametrize("case", ["empty", "one_node", "single_edge", "one_row", "hub", "isolated"])
def test_degenerate_schedules(driver, case, cus, waves):
    rng = np.random.default_rng(1)
    major, N = {
        "empty": ([], 7),
        "one_node": ([], 1),
        "single_edge": ([0], 1),
        "one_row": ([3] * 5000, 10),
        "hub": (list(rng.integers(0, 50, 3000)) + [7] * 20000, 50),  # hub beyond a workgroup's share
        "isolated": ([1, 1, 999], 1000),
    }[case]
    replay(driver, major, N, waves, cus)


def test_random_schedules(driver):
    rng = np.random.default_rng(2)
    for _ in range(12):
        N = int(rng.integers(1, 3000))
        E = int(rng.integers(0, 40000))
        p = np.arange(1, N + 1, dtype=np.float64) ** -float(rng.choice([0.0, 1.0, 2.0]))
        major = rng.choice(N, size=E, p=p / p.sum())
        replay(driver, major, N, int(rng.choice([8, 16])), int(rng.choice([256, 64, 8, 1])))
