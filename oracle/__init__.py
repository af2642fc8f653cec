"""CPU oracle of the leaky-tanh sparse-graph recurrence (fp64, plain C + OpenMP).

TEST INFRASTRUCTURE ONLY: imported by the test suite, by the smoke check and by
the benchmark's CPU-baseline leg, never by the product package.  It shares no
code with the HIP library.  What it computes is stated in ``ck_oracle.c``,
following the connectome-kernels README (introduction: the proposal/update
equations; "Use": argument shapes and edge order; "Design notes": the saved
state and pre-activation).

Parity: the forward is pinned by a dense brute-force recurrence, by the tanh
Elman RNN special case (torch.nn.RNN) and by closed forms; the gradient is
pinned by central finite differences, by torch autograd on dense fp64
formulations and by closed forms (see tests/test_oracle_pins.py).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# "f64" is the oracle; "f32" is the same code evaluated in fp32: the rounding
# floor of the method, to which the GPU parity tests hold a tensor only where
# some element misses the stated bound against the fp64 oracle.
_LIB_PATHS = {"f64": os.path.join(_HERE, "libckoracle.so"),
              "f32": os.path.join(_HERE, "libckoracle_f32.so")}
_libs = {}

# Status values of the documented error convention (restated, not shared).
STATUS = {0: "ok", 1: "null_arg", 2: "bad_size", 3: "index_range", 4: "dup_input",
          5: "too_large", 7: "nomem"}


class OracleError(RuntimeError):
    def __init__(self, code: int):
        super().__init__(f"oracle status {code} ({STATUS.get(code, '?')})")
        self.code = code


def _load(precision: str = "f64"):
    path = _LIB_PATHS[precision]
    if path not in _libs:
        if not os.path.exists(path):
            from . import build as _b
            _b.build()
        lib = ctypes.CDLL(path)
        i64, p = ctypes.c_int64, ctypes.c_void_p
        lib.ckor_validate.restype = ctypes.c_int
        lib.ckor_validate.argtypes = [i64, i64, p, p, i64, p]
        lib.ckor_build.restype = ctypes.c_int
        lib.ckor_build.argtypes = [i64, i64, p, p, i64, p] + [p] * 7
        lib.ckor_run.restype = ctypes.c_int
        lib.ckor_run.argtypes = [i64, i64, p, p, i64, p, p, p, p, p, p, i64, i64, i64,
                                 p, p, p, p, p, p, p, ctypes.c_int]
        _libs[path] = lib
    return _libs[path]


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _i64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.int64))


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def validate(src, dst, num_nodes, input_nodes) -> int:
    """Status code the documented validation rules give for this graph."""
    src, dst, inp = _i64(src), _i64(dst), _i64(input_nodes)
    if src.shape != dst.shape:
        return 2
    return int(_load().ckor_validate(num_nodes, src.size, _ptr(src), _ptr(dst), inp.size, _ptr(inp)))


def build_graph(src, dst, num_nodes: int, input_nodes):
    """CSR by destination and transposed CSR by source, ties by caller index.

    Returns a dict of int32 arrays: row_ptr, col_idx, perm, t_row_ptr,
    t_col_idx, t_perm, input_slot.
    """
    src, dst, inp = _i64(src), _i64(dst), _i64(input_nodes)
    if src.shape != dst.shape:
        raise OracleError(2)
    N, E = int(num_nodes), src.size
    n = max(N, 0)
    res = {
        "row_ptr": np.zeros(n + 1, np.int32), "col_idx": np.zeros(E, np.int32),
        "perm": np.zeros(E, np.int32), "t_row_ptr": np.zeros(n + 1, np.int32),
        "t_col_idx": np.zeros(E, np.int32), "t_perm": np.zeros(E, np.int32),
        "input_slot": np.zeros(n, np.int32),
    }
    rc = _load().ckor_build(N, E, _ptr(src), _ptr(dst), inp.size, _ptr(inp),
                            *[_ptr(res[k]) for k in ("row_ptr", "col_idx", "perm", "t_row_ptr",
                                                     "t_col_idx", "t_perm", "input_slot")])
    if rc:
        raise OracleError(rc)
    return res


def edge_order(src, dst, order):
    """Permutation p of the caller's edges giving the order in which the
    oracle visits them: None = caller order, "sorted" = by (dst, src, caller
    index) (the order of the rows of the CSR by destination), an int = a
    random order drawn with that seed."""
    src, dst = _i64(src), _i64(dst)
    if order is None:
        return np.arange(src.size)
    if order == "sorted":
        return np.lexsort((np.arange(src.size), src, dst))
    return np.random.default_rng(int(order)).permutation(src.size)


def run(src, dst, num_nodes: int, input_nodes, edge_values, leak, bias, drives, state0,
        microsteps: int, grad_out=None, nthreads: int = 0, precision: str = "f64", order=None):
    """Forward (and, with grad_out, the gradient of sum(out * grad_out)).

    Shapes: edge_values[E] (caller order), leak[N], bias[N], drives[T, n_in, B],
    state0[B, N], grad_out[T, B, N].  Returns a dict with ``out`` [T, B, N] and,
    with grad_out, ``g_edge_values``, ``g_leak``, ``g_bias``, ``g_drives``,
    ``g_state0`` -- all float64.  precision="f32" evaluates the same steps in
    fp32 (rounding-floor measurement only).  order (see edge_order) sets the
    order in which each node's incoming and outgoing edge terms are summed;
    the result is the same definition whatever the order (only its rounding
    differs), and g_edge_values is returned in the caller's edge order.
    """
    if order is not None:
        p = edge_order(src, dst, order)
        res = run(_i64(src)[p], _i64(dst)[p], num_nodes, input_nodes, _f64(edge_values)[p], leak,
                  bias, drives, state0, microsteps, grad_out=grad_out, nthreads=nthreads,
                  precision=precision)
        if "g_edge_values" in res:
            gv = np.empty_like(res["g_edge_values"])
            gv[p] = res["g_edge_values"]
            res["g_edge_values"] = gv
        return res
    src, dst, inp = _i64(src), _i64(dst), _i64(input_nodes)
    v, lk, bs = _f64(edge_values), _f64(leak), _f64(bias)
    st0 = _f64(state0)
    N, E, n_in = int(num_nodes), src.size, inp.size
    B = st0.shape[0]
    dr = _f64(drives)
    T = dr.shape[0]
    if dr.shape != (T, n_in, B) or st0.shape != (B, N) or v.shape != (E,) \
            or lk.shape != (N,) or bs.shape != (N,):
        raise OracleError(2)
    out = np.zeros((T, B, N), np.float64)
    res = {"out": out}
    G = None
    args_g = [None] * 5
    if grad_out is not None:
        G = _f64(grad_out)
        if G.shape != (T, B, N):
            raise OracleError(2)
        res.update(g_edge_values=np.zeros(E), g_leak=np.zeros(N), g_bias=np.zeros(N),
                   g_drives=np.zeros((T, n_in, B)), g_state0=np.zeros((B, N)))
        args_g = [res[k] for k in ("g_edge_values", "g_leak", "g_bias", "g_drives", "g_state0")]
    rc = _load(precision).ckor_run(N, E, _ptr(src), _ptr(dst), n_in, _ptr(inp), _ptr(v), _ptr(lk), _ptr(bs),
                          _ptr(dr), _ptr(st0), T, B, int(microsteps), _ptr(G), _ptr(out),
                          *[_ptr(a) for a in args_g], int(nthreads))
    if rc:
        raise OracleError(rc)
    return res


# ---------------------------------------------------------------- LIF forward
# Integer fixed-point leaky integrate-and-fire forward (lif_oracle.c; soup-connectome
# page, "Runtime contract").
_LIF_PATH = os.path.join(_HERE, "libliforacle.so")
_lif = None
LIF_OVERFLOW = 11   # the run was rejected: a potential left the int32 range
LIF_BAD_VALUE = 12  # a delay, decay shift or refractory count out of range


def _load_lif():
    global _lif
    if _lif is None:
        if not os.path.exists(_LIF_PATH):
            from . import build as _b
            _b.build()
        lib = ctypes.CDLL(_LIF_PATH)
        i64, i32, p = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
        lib.lifor_run.restype = ctypes.c_int
        lib.lifor_run.argtypes = [i64, i64, p, p, p, p, i32, i32, i32, i32, p, p, i64, p, p, p]
        _lif = lib
    return _lif


class LifOverflow(OracleError):
    def __init__(self, step: int):
        super().__init__(LIF_OVERFLOW)
        self.step = step


def lif_run(src, dst, num_nodes: int, impulses, delays, v0, T: int, threshold: int, reset: int,
            refractory_steps: int, decay_shifts):
    """Spikes uint8 [T, N] and potentials int32 [T, N] (after each step) of the
    fixed-point LIF forward.  impulses int16 [E] and delays int32 [E] are in the
    caller's edge order.  Raises LifOverflow (with .step) if a potential leaves
    the int32 range, OracleError for invalid arguments."""
    src, dst = _i64(src), _i64(dst)
    w = np.ascontiguousarray(np.asarray(impulses, np.int16))
    d = np.ascontiguousarray(np.asarray(delays, np.int32))
    v = np.ascontiguousarray(np.asarray(v0, np.int32))
    sh = np.ascontiguousarray(np.asarray(list(decay_shifts), np.int32))
    N, E = int(num_nodes), src.size
    if dst.size != E or w.size != E or d.size != E or v.size != N:
        raise OracleError(2)
    spikes = np.zeros((int(T), N), np.uint8)
    pot = np.zeros((int(T), N), np.int32)
    step = ctypes.c_int64(-1)
    rc = _load_lif().lifor_run(N, E, _ptr(src), _ptr(dst), _ptr(w), _ptr(d), int(threshold),
                               int(reset), int(refractory_steps), sh.size, _ptr(sh) if sh.size else None,
                               _ptr(v), int(T), _ptr(spikes), _ptr(pot), ctypes.byref(step))
    if rc == LIF_OVERFLOW:
        raise LifOverflow(step.value)
    if rc:
        raise OracleError(rc)
    return spikes, pot
