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

# mistakes in the log-decay and Finch-C2 forms, caught by the pins of
# test_oracle_variants.py (replayed in _variant_pins_pass)
VARIANT_MUTANTS = {
    "c2_key_scaled_by_w": ("kt[i] = kt[i] * (1.0 - wt[i]);", "kt[i] = kt[i] * wt[i];"),
    "c2_key_not_scaled": ("kt[i] = kt[i] * (1.0 - wt[i]);", "kt[i] = kt[i];"),
    "c2_reads_current_token": ("acc += rt[i] * S[i * D + j];",
                               "acc += rt[i] * (S[i * D + j] + kt[i] * vt[j]);"),
    "c2_second_value_dropped": ("if (u2) acc += load_value(kind, u2, base + j);", "(void)u2;"),
    "c2_second_value_on_wrong_token": ("if (u2) acc += load_value(kind, u2, base + j);",
                                       "if (u2 && t > t0) acc += load_value(kind, u2, base - (int64_t)H * D + j);"),
    "log_decay_sign": ("wt[i] = exp(-exp(wt[i]));", "wt[i] = exp(-exp(-wt[i]));"),
    "log_decay_single_exponential": ("wt[i] = exp(-exp(wt[i]));", "wt[i] = exp(wt[i]);"),
}
ALL_MUTANTS = dict(MUTANTS, **VARIANT_MUTANTS)


def _build_mutant(tmp_path, name):
    old, new = ALL_MUTANTS[name]
    src = open(SRC).read()
    assert old in src, name
    path_c = tmp_path / ("%s.c" % name)
    path_c.write_text(src.replace(old, new))
    path_so = tmp_path / ("lib%s.so" % name)
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                    "-o", str(path_so), str(path_c), "-lm"], check=True)
    lib = ctypes.CDLL(str(path_so))
    lib.oracle_wkv_f64.restype = ctypes.c_int
    lib.oracle_wkv_f64.argtypes = oracle._load().oracle_wkv_f64.argtypes
    lib.oracle_wkv_f64_ex.restype = ctypes.c_int
    lib.oracle_wkv_f64_ex.argtypes = oracle._load().oracle_wkv_f64_ex.argtypes
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


def _variant_pins_pass():
    """True when the mutant passes every pin of the log-decay and C2 forms."""
    import test_oracle_variants as tv
    checks = [tv.test_c2_hand_worked_fixture,
              tv.test_c2_second_value_is_additive_and_keeps_the_state,
              tv.test_c2_is_finch_with_prescaled_keys_and_no_bonus,
              lambda: tv.test_c2_normalisation_closed_form("w"),
              lambda: tv.test_c2_normalisation_closed_form("log"),
              lambda: tv.test_log_decay_extremes_in_closed_form("finch"),
              lambda: tv.test_log_decay_extremes_in_closed_form("c2"),
              tv.test_constant_log_decay_is_a_recursive_filter]
    for decay in ("w", "log"):
        for variant in ("finch", "c2"):
            checks.append(lambda d=decay, v=variant: tv.test_forms_match_brute_force_sum(d, v, 4, 33, 2))
    for check in checks:
        try:
            check()
        except AssertionError:
            return False
    return True


def test_unmutated_oracle_passes_pins():
    assert _pins_pass()
    assert _variant_pins_pass()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_mutant(tmp_path, monkeypatch, name):
    lib = _build_mutant(tmp_path, name)
    monkeypatch.setattr(oracle, "_lib", lib)
    assert not _pins_pass(), "planted mistake %r was not detected" % name


@pytest.mark.parametrize("name", sorted(VARIANT_MUTANTS))
def test_variant_pins_reject_mutant(tmp_path, monkeypatch, name):
    lib = _build_mutant(tmp_path, name)
    monkeypatch.setattr(oracle, "_lib", lib)
    assert _pins_pass(), "the base Finch form must be untouched by %r" % name
    assert not _variant_pins_pass(), "planted mistake %r was not detected" % name
