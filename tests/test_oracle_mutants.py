"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a private copy of the C oracle (on the CPU,
compiled to a temporary library), swaps it in, and checks that the
independent pins of test_oracle.py reject it.
"""
import ctypes
import json
import os
import subprocess

import numpy as np
import pytest

import oracle
from synth import random_slice

SRC = os.path.join(os.path.dirname(oracle.__file__), "wkv_oracle.c")
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked_d2_t3.json")

MUTANTS = {
    "bonus_dropped": ("acc += rt[i] * (S[i * D + j] + ud[i] * kt[i] * vt[j]);",
                      "acc += rt[i] * (S[i * D + j]);"),
    "decay_on_value_axis": ("S[i * D + j] = wt[i] * S[i * D + j] + kt[i] * vt[j];",
                            "S[i * D + j] = wt[j] * S[i * D + j] + kt[i] * vt[j];"),
    "state_transposed_in_readout": ("acc += rt[i] * (S[i * D + j] + ud[i]",
                                    "acc += rt[i] * (S[j * D + i] + ud[i]"),
    "decay_applied_before_readout": ("acc += rt[i] * (S[i * D + j] + ud[i]",
                                     "acc += rt[i] * (wt[i] * S[i * D + j] + ud[i]"),
    "carried_state_ignored": ("memcpy(S, s0, (size_t)D * D * sizeof(double));",
                              "(void)s0;"),
    "bonus_on_value_channel": ("ud[i] * kt[i] * vt[j]", "ud[j] * kt[i] * vt[j]"),
}


def _build_mutant(tmp_path, name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert old in src, name
    path_c = tmp_path / ("%s.c" % name)
    path_c.write_text(src.replace(old, new))
    path_so = tmp_path / ("lib%s.so" % name)
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                    "-o", str(path_so), str(path_c)], check=True)
    lib = ctypes.CDLL(str(path_so))
    lib.oracle_wkv_f64.restype = ctypes.c_int
    lib.oracle_wkv_f64.argtypes = oracle._load().oracle_wkv_f64.argtypes
    lib.oracle_max_threads.restype = ctypes.c_int
    return lib


def _pins_pass():
    """True when the mutant still passes every pin below."""
    T, D = 20, 6
    for seed in (1, 2):
        r, k, v, w, u, s0 = random_slice(seed, T, D, state_sigma=0.5)
        add = lambda a: a.reshape(1, T, 1, D)
        o, s = oracle.wkv_scan(add(r), add(k), add(v), add(w), u.reshape(1, D),
                               s0.astype(np.float64).reshape(1, 1, D, D))
        ob, sb = oracle.wkv_sum_form(r, k, v, w, u, s0)
        if not (np.allclose(o.reshape(T, D), ob, rtol=1e-10, atol=1e-10)
                and np.allclose(s.reshape(D, D), sb, rtol=1e-10, atol=1e-10)):
            return False
    g = json.load(open(GOLDEN))
    f = lambda key: np.array(g[key], dtype=np.float32)
    add = lambda a: a.reshape(1, 3, 1, 2)
    o, s = oracle.wkv_scan(add(f("r")), add(f("k")), add(f("v")), add(f("w")),
                           f("u").reshape(1, 2), f("state0").astype(np.float64).reshape(1, 1, 2, 2))
    return bool(np.array_equal(o.reshape(3, 2), np.array(g["o"]))
                and np.array_equal(s.reshape(2, 2), np.array(g["state_final"])))


def test_unmutated_oracle_passes_pins():
    assert _pins_pass()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_mutant(tmp_path, monkeypatch, name):
    lib = _build_mutant(tmp_path, name)
    monkeypatch.setattr(oracle, "_lib", lib)
    assert not _pins_pass(), "planted mistake %r was not detected" % name
