"""The resident planner's assignment solver (csrc/schedule.cpp,
assign_min_cost: the Hungarian method), which picks each wave-slot's
permutation of bank groups.  Pinned to brute force over every permutation
for n <= 7 and to scipy's linear_sum_assignment at the planner's size,
n = 16, on random, tied and degenerate cost matrices: the result must be a
permutation whose total cost is the minimum."""
import itertools
import os
import shutil
import subprocess

import numpy as np
import pytest
from scipy.optimize import linear_sum_assignment

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_graph_recurrent_amd", "csrc")


@pytest.fixture(scope="module")
def solve(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("assign") / "assign_driver")
    subprocess.run([gxx, "-std=c++17", "-O2", "-Wall", "-Werror", "-I", CSRC, "-o", exe,
                    os.path.join(ROOT, "tests", "assign_driver.cpp"),
                    os.path.join(CSRC, "schedule.cpp")], check=True)

    def run(mats):
        text = "".join(f"{len(m)} " + " ".join(map(str, np.asarray(m).ravel())) + "\n" for m in mats)
        out = subprocess.run([exe], input=text, capture_output=True, text=True, check=True).stdout
        return [np.array(ln.split(), dtype=np.int64) for ln in out.strip().split("\n")]
    return run


def cases(rng, n, k):
    mats = [rng.integers(0, 100, (n, n)) for _ in range(k)]       # random
    mats += [rng.integers(0, 3, (n, n)) for _ in range(k)]        # many ties
    mats.append(np.zeros((n, n), np.int64))                       # all equal
    mats.append(np.full((n, n), 40) - 10 * np.eye(n, dtype=np.int64)[::-1])  # anti-diagonal best
    return mats


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 6, 7])
def test_matches_brute_force(solve, n):
    mats = cases(np.random.default_rng(n), n, 20)
    for m, col in zip(mats, solve(mats)):
        assert sorted(col.tolist()) == list(range(n)), "not a permutation"
        best = min(sum(m[i, p[i]] for i in range(n)) for p in itertools.permutations(range(n)))
        assert m[np.arange(n), col].sum() == best


def test_matches_scipy_at_16(solve):
    """The planner's case: 16 lane classes by 16 bank groups, costs 0..40 in
    steps that mimic its offers (4 lanes, 10 per edge left, 9 per empty slot)."""
    rng = np.random.default_rng(16)
    mats = cases(rng, 16, 30)
    offer = rng.integers(0, 2, (40, 16, 16, 4)) * rng.choice([10, 9], (40, 16, 16, 4))
    mats += list(40 - offer.sum(axis=3))
    for m, col in zip(mats, solve(mats)):
        assert sorted(col.tolist()) == list(range(16)), "not a permutation"
        r, c = linear_sum_assignment(m)
        assert m[np.arange(16), col].sum() == m[r, c].sum()
