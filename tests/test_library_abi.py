"""CPU-side checks of the C-ABI library: it loads, exports every symbol that
include/ck.h declares, and its host-side argument validation (which runs
before any HIP call) returns the documented status codes, agreeing with the
oracle's validation rules.  No compute call is made here."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import sparse_graph_recurrent_amd as sgr

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "ck.h")


def _declared():
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(ck_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(sgr.LIB_PATH):
        from sparse_graph_recurrent_amd import build
        build.build()
    return sgr.lib()


def test_every_declared_symbol_is_exported(L):
    names = _declared()
    assert set(names) == set(sgr.EXPORTED)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    for code, name in sgr.STATUS_NAMES.items():
        assert L.ck_status_string(code).decode() == name
    assert L.ck_status_string(77).decode() == "CK_ERR_UNKNOWN"


def _create(L, src, dst, E, N, inputs, n_in, out=True):
    h = ctypes.c_void_p()
    return L.ck_graph_create(src, dst, E, N, inputs, n_in, None, ctypes.byref(h) if out else None)


def test_host_side_validation_codes_match_oracle(L):
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails before any device work
    # num_nodes <= 0 -> BAD_SIZE, same as the oracle
    assert _create(L, fake, fake, 1, 0, None, 0) == 2 == oracle.validate([0], [0], 0, [])
    assert _create(L, fake, fake, -1, 5, None, 0) == 2
    assert _create(L, fake, fake, 1, 5, fake, -3) == 2
    # 2^31 nodes or edges -> TOO_LARGE
    assert _create(L, fake, fake, 1, 2**31, None, 0) == 5
    assert _create(L, fake, fake, 2**31, 5, None, 0) == 5
    # NULL edge list with edges, NULL input list with inputs -> NULL_ARG
    assert _create(L, None, fake, 3, 5, None, 0) == 1
    assert _create(L, fake, None, 3, 5, None, 0) == 1
    assert _create(L, fake, fake, 3, 5, None, 2) == 1
    # NULL output handle pointer
    assert _create(L, fake, fake, 3, 5, None, 0, out=False) == 1
    assert "NULL" in L.ck_last_error().decode()


def test_null_handles_are_rejected(L):
    assert L.ck_graph_destroy(None) == 0
    n = ctypes.c_int64()
    assert L.ck_graph_sizes(None, ctypes.byref(n), None, None) == 9
    s = ctypes.c_size_t()
    assert L.ck_recurrence_sizes(None, 1, 1, 1, ctypes.byref(s), ctypes.byref(s)) == 9
    assert L.ck_recurrence_status(None, 1, 1, 1, None, 0, None) == 9
    assert L.ck_recurrence_forward(None, *([None] * 5), 1, 1, 1, None, None, None, 0, None) == 9
    assert L.ck_recurrence_backward(None, None, None, None, 1, 1, 1, *([None] * 8), 0, None) == 9
    assert "handle" in L.ck_last_error().decode()
    assert L.ck_lif_workspace_size(None, ctypes.byref(s)) == 9
    assert L.ck_lif_forward(None, None, None, None, None, 1, None, None, None, None, 0, None) == 9
    assert L.ck_lif_prepare(None, None, None, None, 0, None) == 9
    assert L.ck_lif_run(None, None, None, 1, None, None, None, None, 0, None) == 9
    assert "handle" in L.ck_last_error().decode()


def test_oracle_and_header_agree_on_status_values():
    with open(HEADER) as f:
        text = f.read()
    codes = dict((m[0], int(m[1])) for m in re.findall(r"(CK_[A-Z_]+)\s*=\s*(\d+)", text))
    assert codes == {v: k for k, v in sgr.STATUS_NAMES.items()}
    for code, name in oracle.STATUS.items():
        assert sgr.STATUS_NAMES[code].lower().endswith(name)
