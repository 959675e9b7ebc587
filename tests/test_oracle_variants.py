"""Pins of the oracle's two further forms: the decay given as d_t with
w_t = exp(-exp(d_t)) (GoldFinch architecture summary, section 3.4, paragraph
"Data-dependent decay") and the Finch-C2 time mixer (same section: keys scaled
by 1 - w_t, no static bonus, second value u'_t added to the read-out).

Facts that do not come from the oracle:

* a hand-worked Finch-C2 fixture (tests/golden/hand_worked_c2_d2_t3.json),
* the brute-force closed sum of the state equation with the C2 keys,
* the normalisation property the key factor is introduced for: with constant
  w = c and constant k, v every state row relaxes geometrically onto k^T v,
  S_t = c^t S_0 + (1 - c^t) k^T v (closed form),
* d -> -inf gives w = 1 (causal linear attention) and d -> +inf gives w = 0
  (every token forgets everything before it), both in closed form,
* constant d per channel: first-order recursive filter with w = exp(-exp(d))
  (scipy.signal.lfilter),
* C2 equals base Finch with the keys pre-scaled and no bonus, on inputs whose
  scaled keys are exact in fp32, and u'_t enters additively.
"""
import json
import os

import numpy as np
import pytest

import oracle
from synth import random_slice, f32_to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def scan1(r, k, v, w, u, s0=None, **kw):
    """Oracle on one [T, D] slice (adds B=1, H=1 axes)."""
    T, D = r.shape
    add = lambda a: None if a is None else np.asarray(a).reshape(1, T, 1, D)
    st = None if s0 is None else np.asarray(s0, dtype=np.float64).reshape(1, 1, D, D)
    if "second_value" in kw:
        kw["second_value"] = add(kw["second_value"])
    uu = None if u is None else np.asarray(u).reshape(1, D)
    o, s = oracle.wkv_scan(add(r), add(k), add(v), add(w), uu, st, **kw)
    return o.reshape(T, D), s.reshape(D, D)


def test_c2_hand_worked_fixture():
    g = json.load(open(os.path.join(GOLDEN, "hand_worked_c2_d2_t3.json")))
    f = lambda key: np.array(g[key], dtype=np.float32)
    o, s = scan1(f("r"), f("k"), f("v"), f("w"), None, f("state0"), variant="c2",
                 second_value=f("u2"))
    np.testing.assert_array_equal(o, np.array(g["o"]))
    np.testing.assert_array_equal(s, np.array(g["state_final"]))
    o2, s2 = oracle.wkv_sum_form(f("r"), f("k"), f("v"), f("w"), None, f("state0"),
                                 variant="c2", second_value=f("u2"))
    np.testing.assert_array_equal(o2, np.array(g["o"]))
    np.testing.assert_array_equal(s2, np.array(g["state_final"]))


def _u2(seed, T, D, dtype="f32"):
    a = np.random.default_rng(seed).normal(0.0, 0.5, size=(T, D)).astype(np.float32)
    return f32_to_bf16_bits(a) if dtype == "bf16" else a


def _as_d(w):
    """d with exp(-exp(d)) = w (float64), stored as float32."""
    return np.log(-np.log(np.asarray(w, dtype=np.float64))).astype(np.float32)


@pytest.mark.parametrize("decay", ["w", "log"])
@pytest.mark.parametrize("variant", ["finch", "c2"])
@pytest.mark.parametrize("D,T,seed", [(4, 1, 1), (4, 33, 2), (64, 20, 3)])
def test_forms_match_brute_force_sum(decay, variant, D, T, seed):
    r, k, v, w, u, s0 = random_slice(seed, T, D, state_sigma=0.5)
    dec = _as_d(w) if decay == "log" else w
    kw = dict(decay=decay, variant=variant)
    if variant == "c2":
        kw["second_value"] = _u2(seed, T, D)
        u = None
    o, s = scan1(r, k, v, dec, u, s0, **dict(kw))
    ob, sb = oracle.wkv_sum_form(r, k, v, dec, u, s0, **kw)
    np.testing.assert_allclose(o, ob, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(s, sb, rtol=1e-12, atol=1e-12)


def test_forms_match_brute_force_on_bf16_inputs():
    r, k, v, w, u, s0 = random_slice(8, 29, 8, dtype="bf16", state_sigma=0.3)
    d = f32_to_bf16_bits(np.random.default_rng(9).uniform(-6, 0.5, size=(29, 8)).astype(np.float32))
    u2 = _u2(10, 29, 8, "bf16")
    for kw in (dict(decay="log"), dict(variant="c2", second_value=u2),
               dict(decay="log", variant="c2", second_value=u2)):
        dec = d if kw.get("decay") == "log" else w
        uu = None if kw.get("variant") == "c2" else u
        o, s = scan1(r, k, v, dec, uu, s0, **dict(kw))
        ob, sb = oracle.wkv_sum_form(r, k, v, dec, uu, s0, **kw)
        np.testing.assert_allclose(o, ob, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(s, sb, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("decay", ["w", "log"])
def test_c2_normalisation_closed_form(decay):
    """Constant per-channel c and constant k, v: S_t = c^t S_0 + (1 - c^t) k^T v."""
    T, D = 300, 8
    g = np.random.default_rng(5)
    c = np.array([0.5, 0.75, 0.9, 0.99, 0.999, 1.0, 0.25, 0.6])
    kv_k = g.normal(size=D).astype(np.float32)
    kv_v = g.normal(size=D).astype(np.float32)
    r = g.normal(size=(T, D)).astype(np.float32)
    s0 = g.normal(size=(D, D)).astype(np.float32)
    k = np.tile(kv_k, (T, 1))
    v = np.tile(kv_v, (T, 1))
    if decay == "w":
        w = np.tile(c.astype(np.float32), (T, 1))
        cc = w[0].astype(np.float64)
    else:
        d = np.full((T, D), -np.inf, dtype=np.float32)
        d[:, :5] = _as_d(c[:5])
        d[:, 6:] = _as_d(c[6:])
        w = d
        cc = np.exp(-np.exp(d[0].astype(np.float64)))
    o, s = scan1(r, k, v, w, None, s0, decay=decay, variant="c2")
    KV = np.outer(kv_k.astype(np.float64), kv_v.astype(np.float64))
    S0 = s0.astype(np.float64)
    expect_o = np.empty((T, D))
    for t in range(T):
        ct = cc ** t
        S_prev = ct[:, None] * S0 + (1.0 - ct)[:, None] * KV
        expect_o[t] = r[t].astype(np.float64) @ S_prev
    cT = cc ** T
    np.testing.assert_allclose(o, expect_o, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(s, cT[:, None] * S0 + (1.0 - cT)[:, None] * KV, rtol=1e-10, atol=1e-10)


def test_c2_second_value_is_additive_and_keeps_the_state():
    r, k, v, w, _, s0 = random_slice(12, 40, 16, state_sigma=0.4)
    u2 = _u2(13, 40, 16)
    o1, s1 = scan1(r, k, v, w, None, s0, variant="c2", second_value=u2)
    o0, s0_ = scan1(r, k, v, w, None, s0, variant="c2")
    np.testing.assert_allclose(o1 - o0, u2.astype(np.float64), rtol=0, atol=1e-14)
    np.testing.assert_array_equal(s1, s0_)


def test_c2_is_finch_with_prescaled_keys_and_no_bonus():
    """w in {0.5, 0.75, 0.875, 1} and 8-bit keys: k (1 - w) is exact in fp32."""
    T, D = 50, 16
    g = np.random.default_rng(14)
    w = g.choice(np.array([0.5, 0.75, 0.875, 1.0], dtype=np.float32), size=(T, D))
    k = (g.integers(-128, 128, size=(T, D)) / 64.0).astype(np.float32)
    r, v = (g.normal(size=(T, D)).astype(np.float32) for _ in range(2))
    s0 = g.normal(size=(D, D)).astype(np.float32)
    u2 = _u2(15, T, D)
    kscaled = (k.astype(np.float64) * (1.0 - w.astype(np.float64))).astype(np.float32)
    assert np.array_equal(kscaled.astype(np.float64), k.astype(np.float64) * (1.0 - w.astype(np.float64)))
    o_c2, s_c2 = scan1(r, k, v, w, None, s0, variant="c2", second_value=u2)
    o_f, s_f = scan1(r, kscaled, v, w, np.zeros(D, dtype=np.float32), s0)
    np.testing.assert_allclose(o_c2, o_f + u2.astype(np.float64), rtol=0, atol=1e-13)
    np.testing.assert_allclose(s_c2, s_f, rtol=0, atol=1e-13)


@pytest.mark.parametrize("variant", ["finch", "c2"])
def test_log_decay_extremes_in_closed_form(variant):
    """d = -inf: w = 1 (causal linear attention); d = +inf: w = 0 (only the
    previous token survives in the state read by token t)."""
    T, D = 60, 8
    r, k, v, _, u, s0 = random_slice(16, T, D, state_sigma=0.3)
    R, K, V, U, S0 = (a.astype(np.float64) for a in (r, k, v, u, s0))
    uu = None if variant == "c2" else u
    bonus = np.zeros((T, D)) if variant == "c2" else ((R * U * K).sum(1))[:, None] * V
    # d = -inf: no decay; C2 keys are multiplied by 1 - 1 = 0
    d = np.full((T, D), -np.inf, dtype=np.float32)
    o, s = scan1(r, k, v, d, uu, s0, decay="log", variant=variant)
    Keff = np.zeros_like(K) if variant == "c2" else K
    expect = np.tril(R @ Keff.T, -1) @ V + R @ S0 + bonus
    np.testing.assert_allclose(o, expect, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(s, S0 + Keff.T @ V, rtol=1e-11, atol=1e-11)
    # d = +inf: w = 0, C2 keys unscaled (1 - 0)
    d = np.full((T, D), np.inf, dtype=np.float32)
    o, s = scan1(r, k, v, d, uu, s0, decay="log", variant=variant)
    prev = np.vstack([R[:1] @ S0, ((R[1:] * K[:-1]).sum(1))[:, None] * V[:-1]])
    np.testing.assert_allclose(o, prev + bonus, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(s, np.outer(K[-1], V[-1]), rtol=1e-12, atol=1e-12)


def test_constant_log_decay_is_a_recursive_filter():
    """Constant d per channel, base Finch: each state entry is a first-order IIR
    filter with pole exp(-exp(d)) driven by k_t v_t."""
    signal = pytest.importorskip("scipy.signal")
    T, D = 400, 6
    r, k, v, _, u, s0 = random_slice(17, T, D, state_sigma=0.2)
    dch = np.array([-6.0, -3.0, -1.0, 0.0, 0.5, 1.5], dtype=np.float32)
    d = np.tile(dch, (T, 1))
    o, s = scan1(r, k, v, d, u, s0, decay="log")
    c = np.exp(-np.exp(dch.astype(np.float64)))
    K, V, R, U = (a.astype(np.float64) for a in (k, v, r, u))
    S_hist = np.empty((T + 1, D, D))
    S_hist[0] = s0
    for i in range(D):
        for j in range(D):
            x = K[:, i] * V[:, j]
            y, _ = signal.lfilter([1.0], [1.0, -c[i]], x, zi=[c[i] * s0[i, j]])
            S_hist[1:, i, j] = y
    expect = np.einsum("ti,tij->tj", R, S_hist[:-1]) + ((R * U * K).sum(1))[:, None] * V
    np.testing.assert_allclose(o, expect, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(s, S_hist[-1], rtol=1e-10, atol=1e-10)


def test_log_decay_agrees_with_w_form_on_the_same_weights():
    """d given vs w = exp(-exp(d)) given (rounded to fp32): equal within the
    fp32 rounding of w."""
    T, D = 80, 16
    r, k, v, w, u, s0 = random_slice(18, T, D, state_sigma=0.3)
    d = _as_d(w)
    wd = np.exp(-np.exp(d.astype(np.float64))).astype(np.float32)
    for variant in ("finch", "c2"):
        uu = None if variant == "c2" else u
        o_d, s_d = scan1(r, k, v, d, uu, s0, decay="log", variant=variant)
        o_w, s_w = scan1(r, k, v, wd, uu, s0, variant=variant)
        scale = max(np.abs(o_w).max(), 1e-30)
        assert np.abs(o_d - o_w).max() / scale < 1e-5
        assert np.abs(s_d - s_w).max() / np.abs(s_w).max() < 1e-5
