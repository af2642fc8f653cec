"""Host-side checks of the blocked plan (csrc/schedule.cpp, plain C++): the
work items of the per-microstep kernels for graphs whose state plane is far
larger than the L2 caches.  The gathered nodes are cut into 8 contiguous
blocks, one per XCD; a row's edges into one block are cut into items of at
most 64 edges, each leaving one partial row that a second kernel adds up in
item order.

The plan is built with g++ and a small driver, then replayed: the blocked edge
order is a permutation of the edges in which each wave's items follow one
another in groups, every edge lies in exactly one item (a run of one row's
edges in compressed order), item ids follow the same layout and
row_items / item_ids list each row's
items with blocks and chunks ascending, every item's
edges lie in the block its workgroup serves, each wave's list is a prefix of
items sorted largest first, the dealing is balanced, and adding each row's
item sums in id order gives the row sums exactly (integer weights).
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import synthetic

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_graph_recurrent_amd", "csrc")
BLOCKS, CHUNK, WAVES, ITEM_COST, PAD, GROUP = 8, 64, 16, 8, 64, 8


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("blk") / "blocked_driver")
    subprocess.run([gxx, "-std=c++17", "-O2", "-Wall", "-Werror", "-I", CSRC, "-o", exe,
                    os.path.join(ROOT, "tests", "blocked_driver.cpp"),
                    os.path.join(CSRC, "schedule.cpp")], check=True)
    return exe


def plan(driver, ptr, col, cus):
    N = len(ptr) - 1
    text = f"{N} {cus}\n" + " ".join(map(str, ptr)) + "\n" + " ".join(map(str, col)) + "\n"
    out = subprocess.run([driver], input=text, capture_output=True, text=True, check=True).stdout
    lines = out.strip("\n").split("\n")
    if lines[0] == "none":
        return None
    wgs, KB, items = map(int, lines[0].split())
    row_items = np.array(lines[1].split(), dtype=np.int64)
    # each wave's list is followed by PAD padding entries
    table = np.array(lines[2].split(), dtype=np.int64).reshape(wgs * WAVES, KB + PAD, 4)
    assert (table[:, KB:, 0] == -1).all(), "padding after a wave's list"
    table = table[:, :KB]
    order = np.array(lines[3].split() if len(lines) > 3 else [], dtype=np.int64)
    ids = np.array(lines[4].split() if len(lines) > 4 else [], dtype=np.int64)
    return dict(wgs=wgs, KB=KB, items=items, row_items=row_items, table=table, order=order,
                ids=ids)


def replay(driver, major, minor, N, cus=256):
    """Plan the rows `major` (with gathered nodes `minor`) and replay the plan."""
    major = np.asarray(major, dtype=np.int64)
    minor = np.asarray(minor, dtype=np.int64)
    order = np.lexsort((minor, major))
    col = minor[order]
    deg = np.bincount(major, minlength=N) if len(major) else np.zeros(N, np.int64)
    ptr = np.concatenate([[0], np.cumsum(deg)]).astype(np.int64)
    p = plan(driver, ptr.tolist(), col.tolist(), cus)
    if p is None:
        return None
    E = int(ptr[-1])
    bs = max(1, -(-N // BLOCKS))
    ri = p["row_items"]
    assert len(ri) == N + 1 and ri[0] == 0 and ri[-1] == p["items"] and (np.diff(ri) >= 0).all()
    t = p["table"]
    real = t[:, :, 0] >= 0
    # each wave's list: a prefix of items, largest first
    for v in range(t.shape[0]):
        n = int(real[v].sum())
        assert real[v, :n].all() and not real[v, n:].any(), "items are not a prefix"
        assert (np.diff(t[v, :n, 2]) <= 0).all(), "a wave's items are not largest first"
    # the blocked edge order: a permutation laid out group by group (8 items
    # of one wave's list side by side; every wave's first group, then every
    # wave's second group, ...), item ids in the same order
    order = p["order"]
    assert np.array_equal(np.sort(order), np.arange(E)), "edge order is not a permutation"
    pos, walk = 0, 0
    for g0 in range(0, t.shape[1], GROUP):
        for v in range(t.shape[0]):
            for row, kb, cnt, iid in t[v, g0:g0 + GROUP][real[v, g0:g0 + GROUP]]:
                assert kb == pos and iid == walk, "items are not laid out group by group"
                pos += cnt
                walk += 1
    assert pos == E and walk == p["items"]
    # from here on, kbeg is the item's first edge in compressed order
    t = t.copy()
    if E:
        t[:, :, 1] = np.where(real, order[np.minimum(t[:, :, 1], E - 1)], t[:, :, 1])
        for v in range(t.shape[0]):
            for q in np.nonzero(real[v])[0]:
                kb, cnt = p["table"][v, q, 1], t[v, q, 2]
                run = order[kb:kb + cnt]
                assert np.array_equal(run, np.arange(run[0], run[0] + cnt)), "item is not one run"
    items = t[real]
    assert len(items) == p["items"]
    assert np.array_equal(np.sort(items[:, 3]), np.arange(p["items"])), "ids are not 0 .. items-1"
    assert ((items[:, 2] >= 1) & (items[:, 2] <= CHUNK)).all()
    # every edge in exactly one item, inside the item's row and one block
    cover = np.zeros(E, np.int64)
    by_id = items[np.argsort(items[:, 3])]
    for row, kb, cnt, _ in by_id:
        assert ptr[row] <= kb and kb + cnt <= ptr[row + 1], "item outside its row"
        cover[kb:kb + cnt] += 1
        assert len(set((col[kb:kb + cnt] // bs).tolist())) == 1, "item spans two blocks"
    assert (cover == 1).all(), "every edge in exactly one item"
    # row i's items: item_ids[row_items[i] .. row_items[i+1]), in edge order
    ids = p["ids"]
    assert np.array_equal(np.sort(ids), np.arange(p["items"])), "item_ids is not a permutation"
    for i in range(N):
        mine = by_id[ids[ri[i]:ri[i + 1]]]
        assert (mine[:, 0] == i).all(), "row_items range holds another row's items"
        assert (np.diff(mine[:, 1]) > 0).all(), "a row's items are not in edge order"
    # the block of every item is the one its workgroup serves
    wave_block = (np.arange(t.shape[0]) // WAVES) % BLOCKS
    for v in range(t.shape[0]):
        for row, kb, cnt, _ in t[v][real[v]]:
            assert col[kb] // bs == wave_block[v], "item on another block's XCD"
    # balance: the dealing leaves no wave above the block's average by more than one item
    cost = np.where(real, t[:, :, 2] + ITEM_COST, 0).sum(axis=1)
    for x in range(BLOCKS):
        c = cost[wave_block == x]
        assert c.max() <= c.mean() + CHUNK + ITEM_COST
    # row sums: items' sums added in id order
    val = np.random.default_rng(0).integers(-1000, 1000, E)
    csum = np.concatenate([[0], np.cumsum(val)])
    part = csum[by_id[:, 1] + by_id[:, 2]] - csum[by_id[:, 1]]
    got = np.array([part[ids[ri[i]:ri[i + 1]]].sum() for i in range(N)], dtype=np.int64)
    np.testing.assert_array_equal(got, csum[ptr[1:]] - csum[ptr[:-1]])
    return p


@pytest.mark.parametrize("name", ["tiny", "edge_cases"])
def test_workload_plans(driver, name):
    w = synthetic.make(name, synthetic.DEFAULT_SEEDS[name])
    for major, minor in ((w.dst, w.src), (w.src, w.dst)):
        assert replay(driver, major, minor, w.num_nodes) is not None


def test_random_plans(driver):
    rng = np.random.default_rng(3)
    for _ in range(6):
        N = int(rng.integers(1, 20000))
        E = int(rng.integers(0, 100000))
        p = np.arange(1, N + 1, dtype=np.float64) ** -float(rng.choice([0.0, 1.0, 2.0]))
        major = rng.choice(N, size=E, p=p / p.sum())
        minor = rng.integers(0, N, size=E)
        assert replay(driver, major, minor, N, cus=int(rng.choice([256, 64, 8]))) is not None


@pytest.mark.parametrize("case", ["empty", "one_node", "fewer_nodes_than_blocks", "hub"])
def test_degenerate_plans(driver, case):
    rng = np.random.default_rng(1)
    major, minor, N = {
        "empty": ([], [], 7),
        "one_node": ([0, 0, 0], [0, 0, 0], 1),
        "fewer_nodes_than_blocks": ([0, 1, 2, 2], [2, 1, 0, 2], 3),
        "hub": ([5] * 3000 + list(rng.integers(0, 40, 500)), list(rng.integers(0, 40, 3500)), 40),
    }[case]
    assert replay(driver, major, minor, N) is not None


def test_device_shapes(driver):
    """No plan unless the workgroups split evenly over the 8 XCDs."""
    assert plan(driver, [0, 0], [], 12) is None
    assert plan(driver, [0, 0], [], 0) is None
    assert plan(driver, [0, 0], [], 16) is not None
