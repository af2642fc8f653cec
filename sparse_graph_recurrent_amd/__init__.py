"""MI355X (gfx950) leaky-tanh recurrence on a fixed sparse graph: Python binding.

A thin ctypes layer over the C ABI of ``libck_hip.so`` (declared in
``include/ck.h``).  Every step of the computation runs in the library's HIP
kernels; this module only checks tensor shapes/dtypes and passes device
pointers and the current HIP stream.  PyTorch provides device memory and
streams.

API after the connectome-kernels README ("Use"):

    graph = SparseGraph(src, dst, num_nodes=N, input_nodes=input_nodes)
    out = sparse_recurrence(edge_values, leak, bias, drives, state0, graph, microsteps=2)

with src/dst int64 [E] (edge e: src[e] -> dst[e]), input_nodes int64 [n_in],
edge_values fp32 [E] in the caller's edge order, leak/bias fp32 [N],
drives fp32 [T, n_in, B], state0 fp32 [B, N] and out fp32 [T, B, N].
``sparse_recurrence`` is differentiable in all five tensor arguments.

The library is required: importing works without it, but every call raises
``CkLibraryMissing`` if ``libck_hip.so`` has not been built
(``python -m sparse_graph_recurrent_amd.build``).  There is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libck_hip.so")

STATUS_NAMES = {
    0: "CK_OK", 1: "CK_ERR_NULL_ARG", 2: "CK_ERR_BAD_SIZE", 3: "CK_ERR_INDEX_RANGE",
    4: "CK_ERR_DUP_INPUT", 5: "CK_ERR_TOO_LARGE", 6: "CK_ERR_WORKSPACE", 7: "CK_ERR_NOMEM",
    8: "CK_ERR_HIP", 9: "CK_ERR_BAD_HANDLE", 10: "CK_ERR_WAIT", 11: "CK_ERR_OVERFLOW",
    12: "CK_ERR_BAD_VALUE",
}

EXPORTED = ("ck_graph_create", "ck_graph_destroy", "ck_graph_sizes", "ck_graph_export",
            "ck_recurrence_sizes", "ck_recurrence_path", "ck_recurrence_forward",
            "ck_recurrence_backward", "ck_recurrence_status", "ck_recurrence_forward_noalloc",
            "ck_lif_workspace_size", "ck_lif_forward", "ck_lif_prepare", "ck_lif_run",
            "ck_profile_collect_lif",
            "ck_profile_enable", "ck_profile_collect", "ck_status_string", "ck_last_error")


class CkLibraryMissing(RuntimeError):
    pass


class LifParams(ctypes.Structure):
    """ck_lif_params of include/ck.h."""
    _fields_ = [("threshold", ctypes.c_int32), ("reset", ctypes.c_int32),
                ("refractory_steps", ctypes.c_int32), ("num_decay_shifts", ctypes.c_int32),
                ("decay_shifts", ctypes.c_int32 * 8)]


class CkError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {detail}")
        self.status = status
        self.detail = detail


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded C-ABI library (raises CkLibraryMissing if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise CkLibraryMissing(
                f"{LIB_PATH} is missing; build it with `python -m sparse_graph_recurrent_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        i64, p, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
        L.ck_graph_create.argtypes = [p, p, i64, i64, p, i64, p, ctypes.POINTER(p)]
        L.ck_graph_destroy.argtypes = [p]
        L.ck_graph_sizes.argtypes = [p, ctypes.POINTER(i64), ctypes.POINTER(i64), ctypes.POINTER(i64)]
        L.ck_graph_export.argtypes = [p] * 9
        L.ck_recurrence_sizes.argtypes = [p, i64, i64, i64, ctypes.POINTER(sz), ctypes.POINTER(sz)]
        L.ck_recurrence_path.argtypes = [p, i64, ctypes.POINTER(ctypes.c_int)]
        L.ck_recurrence_forward.argtypes = [p, p, p, p, p, p, i64, i64, i64, p, p, p, sz, p]
        L.ck_recurrence_backward.argtypes = [p, p, p, p, i64, i64, i64, p, p, p, p, p, p, p, p, sz, p]
        L.ck_recurrence_status.argtypes = [p, i64, i64, i64, p, sz, p]
        L.ck_recurrence_forward_noalloc.argtypes = [p, p, p, p, p, p, i64, i64, i64, p, p, p]
        L.ck_lif_workspace_size.argtypes = [p, ctypes.POINTER(sz)]
        L.ck_lif_forward.argtypes = [p, p, p, ctypes.POINTER(LifParams), p, i64, p, p,
                                     ctypes.POINTER(i64), p, sz, p]
        L.ck_lif_prepare.argtypes = [p, p, p, p, sz, p]
        L.ck_lif_run.argtypes = [p, ctypes.POINTER(LifParams), p, i64, p, p, ctypes.POINTER(i64),
                                 p, sz, p]
        L.ck_profile_enable.argtypes = [ctypes.c_int]
        dp = ctypes.POINTER(ctypes.c_double)
        ip = ctypes.POINTER(i64)
        L.ck_profile_collect.argtypes = [dp, ip, dp, ip]
        L.ck_profile_collect_lif.argtypes = [dp, ip, dp, ip]
        for name in EXPORTED[:-2]:
            getattr(L, name).restype = ctypes.c_int
        L.ck_status_string.argtypes = [ctypes.c_int]
        L.ck_status_string.restype = ctypes.c_char_p
        L.ck_last_error.argtypes = []
        L.ck_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        raise CkError(status, lib().ck_last_error().decode())


def _ptr(t: torch.Tensor | None):
    if t is None or t.numel() == 0:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t: torch.Tensor, name: str, dtype: torch.dtype, shape=None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


class SparseGraph:
    """Device graph: CSR by destination, transposed CSR, edge permutations,
    input-slot map and row schedules, built by ``ck_graph_create``."""

    def __init__(self, src: torch.Tensor, dst: torch.Tensor, num_nodes: int,
                 input_nodes: torch.Tensor, stream=None):
        E = src.numel()
        _dev(src, "src", torch.int64, (E,))
        _dev(dst, "dst", torch.int64, (E,))
        _dev(input_nodes, "input_nodes", torch.int64, (input_nodes.numel(),))
        h = ctypes.c_void_p()
        self._lib = lib()
        self.device = src.device
        _check(self._lib.ck_graph_create(_ptr(src), _ptr(dst), E, int(num_nodes),
                                         _ptr(input_nodes), input_nodes.numel(), _stream(stream),
                                         ctypes.byref(h)))
        self._h = h
        self.num_nodes = int(num_nodes)
        self.num_edges = int(E)
        self.num_inputs = int(input_nodes.numel())

    @property
    def handle(self) -> ctypes.c_void_p:
        if self._h is None:
            raise CkError(9, "graph was destroyed")
        return self._h

    def sizes(self):
        n, e, k = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
        _check(self._lib.ck_graph_sizes(self.handle, ctypes.byref(n), ctypes.byref(e), ctypes.byref(k)))
        return n.value, e.value, k.value

    def export(self, stream=None) -> dict:
        N, E = self.num_nodes, self.num_edges
        kw = dict(dtype=torch.int32, device=self.device)
        res = {"row_ptr": torch.empty(N + 1, **kw), "col_idx": torch.empty(E, **kw),
               "perm": torch.empty(E, **kw), "t_row_ptr": torch.empty(N + 1, **kw),
               "t_col_idx": torch.empty(E, **kw), "t_perm": torch.empty(E, **kw),
               "input_slot": torch.empty(N, **kw)}
        _check(self._lib.ck_graph_export(
            self.handle, *[_ptr(res[k]) for k in ("row_ptr", "col_idx", "perm", "t_row_ptr",
                                                  "t_col_idx", "t_perm", "input_slot")],
            _stream(stream)))
        return res

    def destroy(self):
        if getattr(self, "_h", None) is not None:
            _check(self._lib.ck_graph_destroy(self._h))
            self._h = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def recurrence_sizes(graph: SparseGraph, T: int, B: int, microsteps: int):
    """(saved_bytes, workspace_bytes) for a window of T steps, batch B."""
    s, w = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().ck_recurrence_sizes(graph.handle, int(T), int(B), int(microsteps),
                                     ctypes.byref(s), ctypes.byref(w)))
    return s.value, w.value


PATH_NAMES = {0: "per_microstep", 1: "resident", 2: "blocked", 3: "blocked_both"}


def recurrence_path(graph: SparseGraph, B: int) -> str:
    """Kernels a call with batch B runs on this graph: "resident" (one launch
    per call, each XCD computing one group of 4 batch columns), "blocked" (a
    forward of two launches per microstep, each XCD gathering from its own
    block of nodes, and the per-microstep backward), "blocked_both" (blocked
    kernels in both directions) or "per_microstep" (one launch per microstep
    in both directions)."""
    r = ctypes.c_int()
    _check(lib().ck_recurrence_path(graph.handle, int(B), ctypes.byref(r)))
    return PATH_NAMES[r.value]


def _byte_buffer(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def recurrence_forward(graph: SparseGraph, edge_values, leak, bias, drives, state0,
                       microsteps: int, out=None, saved=None, workspace=None, stream=None):
    """Run ``ck_recurrence_forward``; returns (out, saved, workspace)."""
    N, E, n_in = graph.num_nodes, graph.num_edges, graph.num_inputs
    B = state0.shape[0]
    T = drives.shape[0]
    _dev(edge_values, "edge_values", torch.float32, (E,))
    _dev(leak, "leak", torch.float32, (N,))
    _dev(bias, "bias", torch.float32, (N,))
    _dev(drives, "drives", torch.float32, (T, n_in, B))
    _dev(state0, "state0", torch.float32, (B, N))
    sb, wb = recurrence_sizes(graph, T, B, microsteps)
    dev = state0.device
    out = torch.empty((T, B, N), dtype=torch.float32, device=dev) if out is None else \
        _dev(out, "out", torch.float32, (T, B, N))
    saved = _byte_buffer(sb, dev) if saved is None else saved
    workspace = _byte_buffer(wb, dev) if workspace is None else workspace
    if saved.numel() * saved.element_size() < sb:
        raise ValueError("saved buffer too small")
    _check(lib().ck_recurrence_forward(
        graph.handle, _ptr(edge_values), _ptr(leak), _ptr(bias), _ptr(drives), _ptr(state0),
        T, B, int(microsteps), _ptr(out), _ptr(saved), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return out, saved, workspace


def recurrence_forward_noalloc(graph: SparseGraph, edge_values, leak, bias, drives, state0,
                               microsteps: int, out, saved, stream=None):
    """Run ``ck_recurrence_forward_noalloc`` into the caller's `out` and `saved`
    (no workspace: the library's fixed device scratch is used)."""
    N, E, n_in = graph.num_nodes, graph.num_edges, graph.num_inputs
    B = state0.shape[0]
    T = drives.shape[0]
    _dev(edge_values, "edge_values", torch.float32, (E,))
    _dev(leak, "leak", torch.float32, (N,))
    _dev(bias, "bias", torch.float32, (N,))
    _dev(drives, "drives", torch.float32, (T, n_in, B))
    _dev(state0, "state0", torch.float32, (B, N))
    _dev(out, "out", torch.float32, (T, B, N))
    sb, _ = recurrence_sizes(graph, T, B, microsteps)
    if saved.numel() * saved.element_size() < sb:
        raise ValueError("saved buffer too small")
    _check(lib().ck_recurrence_forward_noalloc(
        graph.handle, _ptr(edge_values), _ptr(leak), _ptr(bias), _ptr(drives), _ptr(state0),
        T, B, int(microsteps), _ptr(out), _ptr(saved), _stream(stream)))
    return out, saved


def recurrence_backward(graph: SparseGraph, edge_values, leak, state0, microsteps: int, saved,
                        grad_out, workspace=None, grads=None, stream=None) -> dict:
    """Run ``ck_recurrence_backward``; returns the five gradients (overwritten)."""
    N, E, n_in = graph.num_nodes, graph.num_edges, graph.num_inputs
    T, B = grad_out.shape[0], grad_out.shape[1]
    _dev(edge_values, "edge_values", torch.float32, (E,))
    _dev(leak, "leak", torch.float32, (N,))
    _dev(state0, "state0", torch.float32, (B, N))
    _dev(grad_out, "grad_out", torch.float32, (T, B, N))
    sb, wb = recurrence_sizes(graph, T, B, microsteps)
    dev = grad_out.device
    if saved.numel() * saved.element_size() < sb:
        raise ValueError("saved buffer too small")
    workspace = _byte_buffer(wb, dev) if workspace is None else workspace
    if grads is None:
        f = dict(dtype=torch.float32, device=dev)
        grads = {"g_edge_values": torch.empty(E, **f), "g_leak": torch.empty(N, **f),
                 "g_bias": torch.empty(N, **f), "g_drives": torch.empty((T, n_in, B), **f),
                 "g_state0": torch.empty((B, N), **f)}
    _check(lib().ck_recurrence_backward(
        graph.handle, _ptr(edge_values), _ptr(leak), _ptr(state0), T, B, int(microsteps),
        _ptr(saved), _ptr(grad_out), _ptr(grads["g_edge_values"]), _ptr(grads["g_leak"]),
        _ptr(grads["g_bias"]), _ptr(grads["g_drives"]), _ptr(grads["g_state0"]),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))
    return grads


def recurrence_status(graph: SparseGraph, T: int, B: int, microsteps: int, workspace,
                      stream=None):
    """Synchronise the stream and raise CkError (CK_ERR_WAIT) if the last call
    that used `workspace` failed inside the XCD-resident kernels (its outputs
    were then set to NaN); see ``ck_recurrence_status``."""
    _check(lib().ck_recurrence_status(graph.handle, int(T), int(B), int(microsteps),
                                      _ptr(workspace), workspace.numel() * workspace.element_size(),
                                      _stream(stream)))


def profile_enable(enable: bool = True):
    """Turn the library's per-launch HIP-event timing on or off (process-wide)."""
    _check(lib().ck_profile_enable(1 if enable else 0))


def profile_collect() -> dict:
    """Kernel-only milliseconds and launch counts recorded since the last collect:
    {"fwd_ms", "fwd_launches", "bwd_ms", "bwd_launches"}."""
    fm, bm = ctypes.c_double(), ctypes.c_double()
    fn, bn = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().ck_profile_collect(ctypes.byref(fm), ctypes.byref(fn), ctypes.byref(bm),
                                    ctypes.byref(bn)))
    return {"fwd_ms": fm.value, "fwd_launches": fn.value, "bwd_ms": bm.value,
            "bwd_launches": bn.value}


def _lif_params(threshold, reset, refractory_steps, decay_shifts):
    shifts = list(decay_shifts)
    if len(shifts) > 8:
        raise ValueError("at most 8 decay shifts")
    return LifParams(int(threshold), int(reset), int(refractory_steps), len(shifts),
                     (ctypes.c_int32 * 8)(*shifts))


def lif_workspace(graph: SparseGraph, device="cuda") -> torch.Tensor:
    """A workspace of ``ck_lif_workspace_size`` bytes for this graph."""
    wb = ctypes.c_size_t()
    _check(lib().ck_lif_workspace_size(graph.handle, ctypes.byref(wb)))
    return _byte_buffer(wb.value, device)


def _lif_outputs(N, T, device):
    return (torch.empty((int(T), N), dtype=torch.uint8, device=device),
            torch.empty((int(T), N), dtype=torch.int32, device=device))


def _lif_raise(st, step):
    err = CkError(st, lib().ck_last_error().decode())
    err.step = step.value
    raise err


def lif_forward(graph: SparseGraph, impulses, delays, v0, T: int, threshold: int, reset: int,
                refractory_steps: int, decay_shifts=(), workspace=None, stream=None):
    """Run ``ck_lif_forward`` (fixed-point leaky integrate-and-fire on the
    graph): impulses int16 [E] and delays int32 [E] in the caller's edge
    order, v0 int32 [N].  Returns (spikes uint8 [T, N], potentials int32
    [T, N]).  Synchronises the stream; raises CkError with status
    CK_ERR_OVERFLOW (and .step, the first overflowing timestep) if a
    potential left the int32 range."""
    N, E = graph.num_nodes, graph.num_edges
    _dev(impulses, "impulses", torch.int16, (E,))
    _dev(delays, "delays", torch.int32, (E,))
    _dev(v0, "v0", torch.int32, (N,))
    prm = _lif_params(threshold, reset, refractory_steps, decay_shifts)
    workspace = lif_workspace(graph, v0.device) if workspace is None else workspace
    spikes, pot = _lif_outputs(N, T, v0.device)
    step = ctypes.c_int64(-1)
    st = lib().ck_lif_forward(graph.handle, _ptr(impulses), _ptr(delays), ctypes.byref(prm),
                              _ptr(v0), int(T), _ptr(spikes), _ptr(pot), ctypes.byref(step),
                              _ptr(workspace), workspace.numel() * workspace.element_size(),
                              _stream(stream))
    if st != 0:
        _lif_raise(st, step)
    return spikes, pot


def lif_prepare(graph: SparseGraph, impulses, delays, workspace=None, stream=None) -> torch.Tensor:
    """``ck_lif_prepare``: validate the delays and pack the synapses into a
    workspace (allocated when None), returned for ``lif_run``."""
    E = graph.num_edges
    _dev(impulses, "impulses", torch.int16, (E,))
    _dev(delays, "delays", torch.int32, (E,))
    workspace = lif_workspace(graph, impulses.device) if workspace is None else workspace
    _check(lib().ck_lif_prepare(graph.handle, _ptr(impulses), _ptr(delays), _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream(stream)))
    return workspace


def lif_run(graph: SparseGraph, workspace, v0, T: int, threshold: int, reset: int,
            refractory_steps: int, decay_shifts=(), stream=None):
    """``ck_lif_run``: T steps from v0 on the synapses ``lif_prepare`` left in
    ``workspace``; returns and raises as ``lif_forward``."""
    N = graph.num_nodes
    _dev(v0, "v0", torch.int32, (N,))
    prm = _lif_params(threshold, reset, refractory_steps, decay_shifts)
    spikes, pot = _lif_outputs(N, T, v0.device)
    step = ctypes.c_int64(-1)
    st = lib().ck_lif_run(graph.handle, ctypes.byref(prm), _ptr(v0), int(T), _ptr(spikes),
                          _ptr(pot), ctypes.byref(step), _ptr(workspace),
                          workspace.numel() * workspace.element_size(), _stream(stream))
    if st != 0:
        _lif_raise(st, step)
    return spikes, pot


def profile_collect_lif() -> dict:
    """LIF kernel milliseconds and launch counts recorded since the last collect."""
    gm, um = ctypes.c_double(), ctypes.c_double()
    gn, un = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().ck_profile_collect_lif(ctypes.byref(gm), ctypes.byref(gn), ctypes.byref(um),
                                        ctypes.byref(un)))
    return {"gather_ms": gm.value, "gather_launches": gn.value, "update_ms": um.value,
            "update_launches": un.value}


class _SparseRecurrence(torch.autograd.Function):
    @staticmethod
    def forward(ctx, edge_values, leak, bias, drives, state0, graph, microsteps, check):
        ev, lk, bs = edge_values.contiguous(), leak.contiguous(), bias.contiguous()
        dr, st = drives.contiguous(), state0.contiguous()
        out, saved, ws = recurrence_forward(graph, ev, lk, bs, dr, st, microsteps)
        if check:
            recurrence_status(graph, dr.shape[0], st.shape[0], microsteps, ws)
        ctx.graph, ctx.microsteps, ctx.check = graph, microsteps, check
        ctx.save_for_backward(ev, lk, st, saved)
        return out

    @staticmethod
    def backward(ctx, grad_out):
        ev, lk, st, saved = ctx.saved_tensors
        G = grad_out.contiguous().float()
        T, B = G.shape[0], G.shape[1]
        sb, wb = recurrence_sizes(ctx.graph, T, B, ctx.microsteps)
        ws = _byte_buffer(wb, G.device)
        g = recurrence_backward(ctx.graph, ev, lk, st, ctx.microsteps, saved, G, workspace=ws)
        if ctx.check:
            recurrence_status(ctx.graph, T, B, ctx.microsteps, ws)
        return (g["g_edge_values"], g["g_leak"], g["g_bias"], g["g_drives"], g["g_state0"],
                None, None, None)


def sparse_recurrence(edge_values, leak, bias, drives, state0, graph: SparseGraph,
                      microsteps: int = 2, check: bool = True) -> torch.Tensor:
    """Run the recurrence over the whole window as one autograd node
    (connectome-kernels README, "Use": argument names and shapes).

    Returns the node states at the end of every input step, shaped
    [T, B, N]; gradients reach all five tensor arguments.  With check=True
    (the default) the forward and the backward each synchronise their stream
    once and raise CkError (CK_ERR_WAIT) if the XCD-resident kernels failed
    (their outputs are then NaN); check=False skips that synchronisation, e.g.
    under HIP graph capture."""
    return _SparseRecurrence.apply(edge_values, leak, bias, drives, state0, graph,
                                   int(microsteps), bool(check))


__all__ = ["SparseGraph", "sparse_recurrence", "recurrence_forward", "recurrence_backward",
           "recurrence_forward_noalloc", "lif_forward", "profile_collect_lif", "LifParams",
           "recurrence_sizes", "recurrence_status", "recurrence_path", "profile_enable", "profile_collect", "CkError", "CkLibraryMissing",
           "lib", "LIB_PATH", "EXPORTED"]
