"""The oracle's pins are sharp: plant plausible mistakes in a copy of the
oracle's C source, build it, and check that at least one pin fails for each.

Mistakes are planted only in a temporary copy of the oracle, on the CPU.
"""
import os
import subprocess
import tempfile

import pytest

import oracle
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "ck_oracle.c")

MUTANTS = {
    "transposed_W_forward": ("acc[dst[e]] += v[e] * hb[src[e]];", "acc[src[e]] += v[e] * hb[dst[e]];"),
    "bias_dropped": ("real x = acc[i] + drive + bias[i];", "real x = acc[i] + drive;"),
    "leak_mix_swapped": ("hn[b * N + i] = ((real)1 - leak[i]) * hb[i] + leak[i] * tanh(x);",
                         "hn[b * N + i] = leak[i] * hb[i] + ((real)1 - leak[i]) * tanh(x);"),
    "drive_column_fixed": ("drives[(t * n_in + slot[i]) * B + b]", "drives[(t * n_in + slot[i]) * B]"),
    "output_first_microstep": ("if (s % M == 0)\n      for (int64_t x = 0; x < BN; ++x) out[",
                               "if (s % M == 1 % M)\n      for (int64_t x = 0; x < BN; ++x) out["),
    "carry_leak_dropped": ("gnb[j] = ((real)1 - leak[j]) * gb_row[j];", "gnb[j] = gb_row[j];"),
    "transposed_W_backward": ("gnb[src[e]] += v[e] * gab[dst[e]];", "gnb[dst[e]] += v[e] * gab[src[e]];"),
    "edge_grad_swapped": ("ga[b * N + dst[e]] * q[b * N + src[e]]", "ga[b * N + src[e]] * q[b * N + dst[e]]"),
    "leak_grad_sign": ("gl += g[x] * (p - q[x]);", "gl += g[x] * (q[x] - p);"),
    "ga_without_leak": ("ga[x] = g[x] * leak[i] * or_sech2(a[x]);", "ga[x] = g[x] * or_sech2(a[x]);"),
    "drive_grad_wrong_node": ("+= ga[b * N + inputs[k]];", "+= ga[b * N + k];"),
    "upstream_grad_wrong_step": ("if (s % M == 0)\n        for (int64_t x = 0; x < BN; ++x) g[x] +=",
                                 "if (s % M == 1 % M)\n        for (int64_t x = 0; x < BN; ++x) g[x] +="),
    "leak_grad_uses_new_state": ("const real* q = hs + (s - 1) * BN;", "const real* q = hs + s * BN;"),
    "sech2_is_sech": ("return (real)1 / (c * c);", "return (real)1 / c;"),
}

PIN_CALLS = [
    ("worked_example", lambda: pins.test_worked_example_by_hand()),
    ("dense_fwd_M2", lambda: pins.test_forward_matches_dense_bruteforce(pins.CASES[2], 11)),
    ("autograd_M3", lambda: pins.test_gradients_match_dense_autograd(pins.CASES[2])),
    ("autograd_M1", lambda: pins.test_gradients_match_dense_autograd(pins.CASES[0])),
    ("closed_form_leak0", lambda: pins.test_leak_zero_closed_form()),
]


def _build_mutant(tmp, old, new):
    with open(SRC) as f:
        text = f.read()
    assert text.count(old) == 1, f"mutation anchor not unique: {old!r}"
    path = os.path.join(tmp, "mut.c")
    with open(path, "w") as f:
        f.write(text.replace(old, new))
    lib = os.path.join(tmp, "libmut.so")
    subprocess.run(["gcc", "-std=c11", "-O1", "-fopenmp", "-fPIC", "-shared", "-o", lib, path, "-lm"],
                   check=True)
    return lib


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_every_planted_mistake_fails_a_pin(name, monkeypatch):
    old, new = MUTANTS[name]
    with tempfile.TemporaryDirectory() as tmp:
        lib = _build_mutant(tmp, old, new)
        monkeypatch.setitem(oracle._LIB_PATHS, "f64", lib)
        monkeypatch.setattr(oracle, "_libs", {})
        failed = []
        for pin_name, call in PIN_CALLS:
            try:
                call()
            except AssertionError:
                failed.append(pin_name)
        assert failed, f"mutant {name} passed every pin"
    monkeypatch.setattr(oracle, "_libs", {})
