"""Seeded synthetic workloads shaped like the published ones.

This module only draws random inputs: graphs as caller-ordered (src, dst) int64
lists plus fp32 parameter, drive, state and upstream-gradient arrays.  It holds
none of the recurrence's arithmetic and is the one module that both the HIP
path's tests/benchmark and the CPU oracle consume.

The connectome-kernels README ("Why": the FlyGPT launch-shape table) gives the
reference workload N=5,000 nodes, E=524,324 edges, batch 32, 64 input steps x 2
microsteps; the MaleCNS connectome it was built for (211,577 neurons,
24,678,466 edges, soup-connectome page, "Status at a glance") is not available,
so the graphs below are synthetic stand-ins with the stated degree
distributions:

  tiny        N=256, 4,096 unique non-self pairs drawn uniformly, inputs 0..15,
              B=8, T=8, M=2; v~N(0,1)/4, leak=0.5, bias~N(0,0.1),
              drives~N(0,1), state0~N(0,0.1), G~N(0,1).
  flygpt      N=5,000, E=524,324 unique; in-degree lognormal(4.3, 1.0) rescaled
              to sum E (largest remainder, ties to the lower id); distinct
              uniform sources; inputs 0..255; B=32, T=64, M=2.
  edge_cases  N=5,000, E=600,000; 50 hubs with in-degree U{6000..9000} whose
              sources are drawn with replacement (parallel edges), 500 nodes of
              in-degree 0, the rest lognormal(4.3,1) with distinct sources;
              inputs 0..127; B=20, T=16, M=3.
  mid_scale   N=50,000, E=5,000,000; in-degree lognormal(4.4, 1.2); each source
              is (dst + U{-500..500}) mod N with p=0.7, else uniform (parallel
              edges allowed); inputs 0..1023; B=64, T=32, M=2.
  connectome  N=211,577, E=24,678,466 unique; in-degree from a continuous power
              law k^-2.2 on [k_min, 20000] with k_min chosen so the mean is E/N;
              distinct uniform sources; v = sign * |N(0,1)| / sqrt(E/N) with
              sign +1 (p=0.8) / -1 (p=0.2); inputs 0..2047; B=32, T=32, M=2.

Unless stated: v ~ N(0,1)/sqrt(E/N), leak = sigmoid(N(0, 0.5)),
bias ~ N(0, 0.1), drives ~ N(0,1), state0 = 0, G ~ N(0,1).  N(0, s) takes s as
the standard deviation.  The edge list is randomly permuted before it is
returned, so the caller's edge order differs from any sorted order.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

CONFIGS = ("tiny", "flygpt", "edge_cases", "mid_scale", "connectome")
DEFAULT_SEEDS = {"tiny": 1, "flygpt": 2, "edge_cases": 3, "mid_scale": 4, "connectome": 5}
SHAPES = {  # name: (N, E, n_in, B, T, M)
    "tiny": (256, 4096, 16, 8, 8, 2),
    "flygpt": (5000, 524324, 256, 32, 64, 2),
    "edge_cases": (5000, 600000, 128, 20, 16, 3),
    "mid_scale": (50000, 5000000, 1024, 64, 32, 2),
    "connectome": (211577, 24678466, 2048, 32, 32, 2),
}


@dataclasses.dataclass
class Workload:
    name: str
    seed: int
    num_nodes: int
    src: np.ndarray          # int64 [E], caller order
    dst: np.ndarray          # int64 [E]
    input_nodes: np.ndarray  # int64 [n_in]
    edge_values: np.ndarray  # float32 [E]
    leak: np.ndarray         # float32 [N]
    bias: np.ndarray         # float32 [N]
    drives: np.ndarray       # float32 [T, n_in, B]
    state0: np.ndarray       # float32 [B, N]
    grad_out: np.ndarray     # float32 [T, B, N]
    microsteps: int

    @property
    def num_edges(self) -> int:
        return int(self.src.size)

    @property
    def T(self) -> int:
        return int(self.drives.shape[0])

    @property
    def B(self) -> int:
        return int(self.state0.shape[0])

    @property
    def n_in(self) -> int:
        return int(self.input_nodes.size)


def _largest_remainder(x: np.ndarray, total: int, cap: int) -> np.ndarray:
    """Integers proportional to x summing to total, none above cap.

    Floors of the scaled values, then +1 for the largest fractional parts
    (ties to the lower index); nodes that would exceed cap are pinned at cap
    and the rest re-apportioned.
    """
    x = np.asarray(x, np.float64)
    d = np.zeros(x.size, np.int64)
    free = np.ones(x.size, bool)
    remaining = int(total)
    while True:
        idx = np.nonzero(free)[0]
        scaled = x[idx] * (remaining / x[idx].sum())
        fl = np.floor(scaled).astype(np.int64)
        short = remaining - int(fl.sum())
        frac = scaled - fl
        order = np.lexsort((idx, -frac))  # largest fraction first, ties -> lower id
        fl[order[:short]] += 1
        over = fl > cap
        if not over.any():
            d[idx] = fl
            return d
        pin = idx[over]
        d[pin] = cap
        free[pin] = False
        remaining -= cap * pin.size


def _distinct_sources(rng: np.random.Generator, deg: np.ndarray, N: int):
    """For every node i, deg[i] distinct sources uniform over [0, N)."""
    deg = np.asarray(deg, np.int64)
    E = int(deg.sum())
    dst = np.repeat(np.arange(N, dtype=np.int64), deg)
    src = np.empty(E, np.int64)
    starts = np.concatenate([[0], np.cumsum(deg)])
    big = deg > N // 4
    for i in np.nonzero(big)[0]:
        src[starts[i]:starts[i + 1]] = rng.permutation(N)[: deg[i]]
    idx = np.nonzero(~big[dst])[0]
    src[idx] = rng.integers(0, N, idx.size)
    todo = idx
    while todo.size:
        # re-draw every later copy of a (dst, src) pair inside the small rows
        key = dst[idx] * N + src[idx]
        order = np.argsort(key, kind="stable")
        ks = key[order]
        dup = np.zeros(idx.size, bool)
        dup[order[1:][ks[1:] == ks[:-1]]] = True
        todo = idx[dup]
        src[todo] = rng.integers(0, N, todo.size)
    return src, dst


def _powerlaw_kmin(alpha: float, kmax: float, mean: float) -> float:
    def m(kmin):
        a1, a2 = 1.0 - alpha, 2.0 - alpha
        num = (kmax ** a2 - kmin ** a2) / a2
        den = (kmax ** a1 - kmin ** a1) / a1
        return num / den
    lo, hi = 1.0, mean
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if m(mid) < mean:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def _graph(name: str, rng: np.random.Generator):
    N, E, n_in = SHAPES[name][:3]
    if name == "tiny":
        p = rng.choice(N * (N - 1), size=E, replace=False).astype(np.int64)
        src = p // (N - 1)
        r = p % (N - 1)
        dst = r + (r >= src)
    elif name == "flygpt":
        deg = _largest_remainder(rng.lognormal(4.3, 1.0, N), E, N)
        src, dst = _distinct_sources(rng, deg, N)
    elif name == "edge_cases":
        ids = rng.permutation(N)
        hubs, empty, rest = ids[:50], ids[50:550], ids[550:]
        deg = np.zeros(N, np.int64)
        deg[hubs] = rng.integers(6000, 9001, hubs.size)
        deg[rest] = _largest_remainder(rng.lognormal(4.3, 1.0, rest.size),
                                       E - int(deg[hubs].sum()), N)
        is_hub = np.zeros(N, bool)
        is_hub[hubs] = True
        d_rest = np.where(is_hub, 0, deg)
        src_r, dst_r = _distinct_sources(rng, d_rest, N)
        dst_h = np.repeat(np.arange(N, dtype=np.int64), np.where(is_hub, deg, 0))
        src_h = rng.integers(0, N, dst_h.size)
        src, dst = np.concatenate([src_r, src_h]), np.concatenate([dst_r, dst_h])
        del empty
    elif name == "mid_scale":
        deg = _largest_remainder(rng.lognormal(4.4, 1.2, N), E, E)
        dst = np.repeat(np.arange(N, dtype=np.int64), deg)
        local = rng.random(E) < 0.7
        off = rng.integers(-500, 501, E)
        uni = rng.integers(0, N, E)
        src = np.where(local, (dst + off) % N, uni).astype(np.int64)
    elif name == "connectome":
        alpha, kmax = 2.2, 20000.0
        kmin = _powerlaw_kmin(alpha, kmax, E / N)
        u = rng.random(N)
        a1 = 1.0 - alpha
        x = (kmin ** a1 + u * (kmax ** a1 - kmin ** a1)) ** (1.0 / a1)
        deg = _largest_remainder(x, E, int(kmax))
        src, dst = _distinct_sources(rng, deg, N)
    else:
        raise ValueError(f"unknown workload {name!r}")
    perm = rng.permutation(src.size)
    return src[perm].astype(np.int64), dst[perm].astype(np.int64), np.arange(n_in, dtype=np.int64)


def make(name: str, seed: int | None = None, B: int | None = None, T: int | None = None,
         M: int | None = None) -> Workload:
    """Seeded workload ``name``; B, T, M may be overridden (the graph is unchanged)."""
    if name not in SHAPES:
        raise ValueError(f"unknown workload {name!r}; expected one of {CONFIGS}")
    seed = DEFAULT_SEEDS[name] if seed is None else int(seed)
    N, E, n_in, B0, T0, M0 = SHAPES[name]
    B = B0 if B is None else int(B)
    T = T0 if T is None else int(T)
    M = M0 if M is None else int(M)
    g_rng = np.random.default_rng([seed, 0])
    v_rng = np.random.default_rng([seed, 1])
    src, dst, inputs = _graph(name, g_rng)
    E = src.size
    f32 = np.float32
    if name == "tiny":
        v = (v_rng.standard_normal(E) / 4.0).astype(f32)
        leak = np.full(N, 0.5, f32)
    elif name == "connectome":
        sign = np.where(v_rng.random(E) < 0.8, 1.0, -1.0)
        v = (sign * np.abs(v_rng.standard_normal(E)) / math.sqrt(E / N)).astype(f32)
        leak = (1.0 / (1.0 + np.exp(-0.5 * v_rng.standard_normal(N)))).astype(f32)
    else:
        v = (v_rng.standard_normal(E) / math.sqrt(E / N)).astype(f32)
        leak = (1.0 / (1.0 + np.exp(-0.5 * v_rng.standard_normal(N)))).astype(f32)
    bias = (0.1 * v_rng.standard_normal(N)).astype(f32)
    drives = v_rng.standard_normal((T, n_in, B), dtype=f32)
    if name == "tiny":
        state0 = (0.1 * v_rng.standard_normal((B, N))).astype(f32)
    else:
        state0 = np.zeros((B, N), f32)
    grad_out = v_rng.standard_normal((T, B, N), dtype=f32)
    return Workload(name, seed, N, src, dst, inputs, v, leak, bias, drives, state0, grad_out, M)


def random_graph(rng: np.random.Generator, N: int, E: int, n_in: int, B: int, T: int, M: int,
                 self_loops: bool = True, duplicates: bool = True, v_scale: float = 0.5,
                 leak_range=(0.2, 0.9)) -> Workload:
    """Small unstructured workload for edge-case tests (uniform src and dst)."""
    f32 = np.float32
    if duplicates:
        src = rng.integers(0, N, E)
        dst = rng.integers(0, N, E)
        if not self_loops:
            clash = src == dst
            dst[clash] = (dst[clash] + 1) % N
    else:
        pool = N * N if self_loops else N * (N - 1)
        p = rng.choice(pool, size=E, replace=False).astype(np.int64)
        if self_loops:
            src, dst = p // N, p % N
        else:
            src = p // (N - 1)
            r = p % (N - 1)
            dst = r + (r >= src)
    inputs = rng.permutation(N)[:n_in].astype(np.int64)
    v = (v_scale * rng.standard_normal(E)).astype(f32)
    leak = rng.uniform(leak_range[0], leak_range[1], N).astype(f32)
    bias = (0.1 * rng.standard_normal(N)).astype(f32)
    drives = rng.standard_normal((T, n_in, B)).astype(f32)
    state0 = (0.3 * rng.standard_normal((B, N))).astype(f32)
    grad_out = rng.standard_normal((T, B, N)).astype(f32)
    return Workload("random", -1, N, src.astype(np.int64), dst.astype(np.int64), inputs, v, leak,
                    bias, drives, state0, grad_out, M)


@dataclasses.dataclass
class LifWorkload:
    """Inputs of the fixed-point LIF forward on a workload's graph."""
    name: str
    num_nodes: int
    src: np.ndarray        # int64 [E], caller order
    dst: np.ndarray        # int64 [E]
    input_nodes: np.ndarray
    impulses: np.ndarray   # int16 [E]
    delays: np.ndarray     # int32 [E]
    v0: np.ndarray         # int32 [N]


def make_lif(name: str = "connectome", seed: int = 7, max_delay: int = 1,
             v0_range=(0, 1)) -> LifWorkload:
    """The graph of workload `name` with integer LIF inputs: each edge's
    impulse is sign * synapse count, sign +1 with p=0.8 (else -1) and count
    = 1 + floor(lognormal(1.5, 1.0)) capped at 32767; delays uniform in
    1..max_delay (the soup-connectome page's runs fix none; 1 reproduces a
    one-step delay line); initial potentials uniform in v0_range."""
    w = make(name, B=1, T=1)
    rng = np.random.default_rng([seed, 2])
    E = w.num_edges
    count = np.minimum(1 + np.floor(rng.lognormal(1.5, 1.0, E)), 32767).astype(np.int64)
    sign = np.where(rng.random(E) < 0.8, 1, -1)
    impulses = (sign * count).astype(np.int16)
    delays = rng.integers(1, max_delay + 1, E).astype(np.int32)
    v0 = rng.integers(v0_range[0], v0_range[1], w.num_nodes).astype(np.int32)
    return LifWorkload(name, w.num_nodes, w.src, w.dst, w.input_nodes, impulses, delays, v0)
