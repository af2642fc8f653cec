"""Pins of the fixed-point LIF oracle (oracle/lif_oracle.c; soup-connectome
page, "Runtime contract" and "Full-scale benchmark"), none of which calls the
HIP path: a hand-worked timeline (tests/golden/lif_timeline.json), hand-derived
leak sequences (floor shifts of positive and negative potentials, several
shifts, k = 0 and 31), the threshold edge case, overflow rejection in both
directions, the page's two published runs re-read on a small graph, the delay
line checked against a direct gather over the spike history on random graphs,
and planted mistakes in a copy of the oracle, each caught by a pin."""
import json
import os
import subprocess
import tempfile

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
I32_MAX, I32_MIN = 2**31 - 1, -2**31


def _run(src, dst, N, w, d, v0, T, thr, reset, refr, shifts):
    return oracle.lif_run(np.asarray(src, np.int64), np.asarray(dst, np.int64), N, w, d, v0, T,
                          thr, reset, refr, shifts)


def test_hand_worked_timeline():
    g = json.load(open(os.path.join(HERE, "golden", "lif_timeline.json")))
    s, p = _run(g["src"], g["dst"], g["num_nodes"], g["impulse"], g["delay"], g["v0"], g["T"],
                g["threshold"], g["reset"], g["refractory_steps"], g["decay_shifts"])
    np.testing.assert_array_equal(s, np.array(g["spikes"], np.uint8))
    np.testing.assert_array_equal(p, np.array(g["potentials"], np.int32))


@pytest.mark.parametrize("v0,shifts,want", [
    (1000, [2], [750, 563, 423, 318, 239]),          # floor(750/4) = 187, ...
    (-1000, [2], [-750, -562, -421, -315, -236]),    # floor(-187.5) = -188, ...
    (800, [1, 3], [350, 154, 68]),                   # shifts applied in order
    (7, [31], [7, 7, 7]),                            # floor(7 / 2^31) = 0
    (-7, [31], [-6, -5, -4]),                        # floor(-7 / 2^31) = -1
    (5, [0], [0, 0]),                                # V - V
    (1234, [], [1234, 1234]),                        # no leak
])
def test_leak_sequences_by_hand(v0, shifts, want):
    s, p = _run([], [], 1, [], [], [v0], len(want), I32_MAX, 0, 0, shifts)
    assert not s.any()
    np.testing.assert_array_equal(p[:, 0], want)


def test_reaching_the_threshold_exactly_spikes():
    s, p = _run([], [], 2, [], [], [100, 99], 1, 100, -3, 0, [])
    np.testing.assert_array_equal(s[0], [1, 0])
    np.testing.assert_array_equal(p[0], [-3, 99])


@pytest.mark.parametrize("sign", [1, -1])
def test_overflow_is_rejected_at_its_step(sign):
    """Node 0 spikes at step 0 (it starts at the threshold), its impulse
    reaches node 1 at step 3, whose potential then leaves the int32 range."""
    v1 = sign * (I32_MAX - 500)
    with pytest.raises(oracle.LifOverflow) as ei:
        _run([0], [1], 2, [sign * 1000], [3], [I32_MAX, v1], 6, I32_MAX, 0, 0, [])
    assert ei.value.step == 3
    # reaching +-(2^31 - 1) exactly stays inside the range (and, upwards, is
    # the threshold here: a spike, then the reset)
    s, p = _run([0], [1], 2, [sign * 500], [3], [I32_MAX, v1], 6, I32_MAX, 0, 0, [])
    if sign > 0:
        assert s[3, 1] == 1 and p[3, 1] == 0
    else:
        assert s[3, 1] == 0 and p[3, 1] == -I32_MAX


def test_invalid_values_are_rejected():
    for d, shifts, refr in (([0], [2], 0), ([40000], [2], 0), ([1], [32], 0), ([1], [-1], 0),
                            ([1], [2], -1)):
        with pytest.raises(oracle.OracleError) as ei:
            _run([0], [1], 2, [5], d, [0, 0], 2, 10, 0, refr, shifts)
        assert ei.value.code == oracle.LIF_BAD_VALUE
    with pytest.raises(oracle.OracleError) as ei:
        _run([0], [2], 2, [5], [1], [0, 0], 2, 10, 0, 0, [])
    assert ei.value.code == 3


def _small_connectome(seed, N=400, E=6000, delay_max=1, wmax=60):
    rng = np.random.default_rng(seed)
    src, dst = rng.integers(0, N, E), rng.integers(0, N, E)
    w = (np.where(rng.random(E) < 0.8, 1, -1) * rng.integers(1, wmax, E)).astype(np.int16)
    d = rng.integers(1, delay_max + 1, E).astype(np.int32)
    return src, dst, w, d


def test_pages_standard_run_reread():
    """threshold 20000, reset 0, decay_shifts [2], refractory 2, 4 steps, the
    seed neuron at 30000 and impulses far below the threshold: the seed spikes
    once at step 0 and nothing else does (the page's counts [1, 0, 0, 0])."""
    src, dst, w, d = _small_connectome(1)
    v0 = np.zeros(400, np.int32)
    v0[0] = 30000
    s, _ = _run(src, dst, 400, w, d, v0, 4, 20000, 0, 2, [2])
    assert s.sum(axis=1).tolist() == [1, 0, 0, 0]


def test_pages_stress_run_reread():
    """threshold 1, reset 0, decay_shifts [31], refractory 0, 2 steps: at step
    1 exactly the neurons whose summed impulse from the seed is positive
    spike (the page's counts [1, 319] on its own graph)."""
    src, dst, w, d = _small_connectome(2)
    v0 = np.zeros(400, np.int32)
    v0[0] = 30000
    s, _ = _run(src, dst, 400, w, d, v0, 2, 1, 0, 0, [31])
    from_seed = np.zeros(400, np.int64)
    np.add.at(from_seed, dst[src == 0], w[src == 0].astype(np.int64))
    assert s[0].sum() == 1 and s[0, 0] == 1
    np.testing.assert_array_equal(s[1].astype(bool), from_seed > 0)


def _direct_gather(src, dst, N, w, d, v0, T, thr, reset, refr, shifts):
    """The same update with the arriving impulses gathered directly from the
    spike history (impulse of edge e arrives at t iff src[e] spiked at t - d[e])."""
    V = np.asarray(v0, np.int64).copy()
    r = np.zeros(N, np.int64)
    S = np.zeros((T, N), np.uint8)
    P = np.zeros((T, N), np.int64)
    for t in range(T):
        inc = np.zeros(N, np.int64)
        for e in range(len(src)):
            if t - d[e] >= 0 and S[t - d[e], src[e]]:
                inc[dst[e]] += int(w[e])
        for i in range(N):
            if r[i] > 0:
                r[i] -= 1
            else:
                v = int(V[i])
                for k in shifts:
                    v -= v // (1 << k)   # Python // floors
                v += int(inc[i])
                if v >= thr:
                    S[t, i], v, r[i] = 1, reset, refr
                V[i] = v
            P[t, i] = V[i]
    return S, P


@pytest.mark.parametrize("seed,delay_max,refr,shifts", [(3, 1, 0, [2]), (4, 5, 2, [1, 4]),
                                                         (5, 9, 1, [3])])
def test_delay_line_matches_direct_gather(seed, delay_max, refr, shifts):
    N = 60
    src, dst, w, d = _small_connectome(seed, N=N, E=700, delay_max=delay_max, wmax=120)
    rng = np.random.default_rng(seed + 100)
    v0 = rng.integers(0, 600, N).astype(np.int32)
    s, p = _run(src, dst, N, w, d, v0, 12, 100, -20, refr, shifts)
    s2, p2 = _direct_gather(src, dst, N, w, d, v0, 12, 100, -20, refr, shifts)
    assert (s[6:].sum(axis=1) > 5).all()  # the run stays active
    np.testing.assert_array_equal(s, s2)
    np.testing.assert_array_equal(p, p2)


# ------------------------------------------------------------ planted mistakes
SRC = os.path.join(os.path.dirname(oracle.__file__), "lif_oracle.c")
MUTANTS = {
    "shift_truncates": ("if (v % d != 0 && v < 0) q -= 1;", ""),
    "arrives_a_step_early": ("line[((t + delay[e]) % H) * N + dst[e]]", "line[((t + delay[e] - 1) % H) * N + dst[e]]"),
    "refractory_keeps_input": ("        r[i] -= 1;\n", "        r[i] -= 1;\n        V[i] += (int32_t)in;\n"),
    "leak_after_input": ("        for (int32_t j = 0; j < num_shifts; ++j) v = v - lor_floor_shift(v, shifts[j]);\n        v += in;",
                         "        v += in;\n        for (int32_t j = 0; j < num_shifts; ++j) v = v - lor_floor_shift(v, shifts[j]);"),
    "strict_threshold": ("if (v >= threshold) {", "if (v > threshold) {"),
    "no_reset": ("          v = reset;\n", ""),
    "no_overflow_check": ("if (v < INT32_MIN || v > INT32_MAX) {", "if (0) {"),
    "refractory_one_short": ("r[i] = refractory_steps;", "r[i] = refractory_steps - 1;"),
}
PINS = [
    lambda: test_hand_worked_timeline(),
    lambda: test_leak_sequences_by_hand(-1000, [2], [-750, -562, -421, -315, -236]),
    lambda: test_reaching_the_threshold_exactly_spikes(),
    lambda: test_overflow_is_rejected_at_its_step(1),
    lambda: test_delay_line_matches_direct_gather(4, 5, 2, [1, 4]),
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_every_planted_mistake_fails_a_pin(name, monkeypatch):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation anchor not unique: {old!r}"
    with tempfile.TemporaryDirectory() as tmp:
        path = os.path.join(tmp, "mut.c")
        open(path, "w").write(text.replace(old, new))
        lib = os.path.join(tmp, "libmut.so")
        subprocess.run(["gcc", "-std=c11", "-O1", "-fPIC", "-shared", "-o", lib, path], check=True)
        monkeypatch.setattr(oracle, "_LIF_PATH", lib)
        monkeypatch.setattr(oracle, "_lif", None)
        failed = 0
        for pin in PINS:
            try:
                pin()
            except (AssertionError, oracle.OracleError, pytest.fail.Exception):
                failed += 1
        monkeypatch.setattr(oracle, "_lif", None)
    assert failed > 0, f"mutant {name} passed every pin"
