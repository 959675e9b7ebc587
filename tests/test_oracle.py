"""Pins of the fp64 oracle against facts that do not come from the oracle.

Each check is chosen so that a plausible mistake in the oracle (dropped bonus,
decay applied one token early or late, decay on the value axis instead of the
key axis, transposed state, carried-in state not decayed, offsets off by one)
fails at least one of them:

* a hand-worked fixture (tests/golden/hand_worked_d2_t3.json),
* the brute-force closed sum of the GoldFinch architecture summary (section
  3.4, state equation), formed pair by pair,
* the no-decay special case, which is causal linear attention written in its
  masked quadratic form (the "Transformers are RNNs" form the pages build on),
* constant decay per channel, where every state entry is a first-order
  recursive filter evaluated by scipy.signal.lfilter,
* split-and-carry, ragged packing, linearity, permutation and independence
  invariants, T = 1 by hand, bonus isolation.
"""
import json
import os

import numpy as np
import pytest

import oracle
from synth import random_slice, make_workload, f32_to_bf16_bits, bf16_bits_to_f32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def scan1(r, k, v, w, u, s0=None, **kw):
    """Oracle on a single [T, D] slice (adds B=1, H=1 axes)."""
    T, D = r.shape
    add = lambda a: a.reshape(1, T, 1, D)
    st = None if s0 is None else np.asarray(s0, dtype=np.float64).reshape(1, 1, D, D)
    o, s = oracle.wkv_scan(add(r), add(k), add(v), add(w), np.asarray(u).reshape(1, D), st, **kw)
    return o.reshape(T, D), s.reshape(D, D)


def test_hand_worked_fixture():
    g = json.load(open(os.path.join(GOLDEN, "hand_worked_d2_t3.json")))
    f = lambda key: np.array(g[key], dtype=np.float32)
    o, s = scan1(f("r"), f("k"), f("v"), f("w"), f("u"), f("state0"))
    np.testing.assert_array_equal(o, np.array(g["o"]))
    np.testing.assert_array_equal(s, np.array(g["state_final"]))
    o2, s2 = oracle.wkv_sum_form(f("r"), f("k"), f("v"), f("w"), f("u"), f("state0"))
    np.testing.assert_array_equal(o2, np.array(g["o"]))
    np.testing.assert_array_equal(s2, np.array(g["state_final"]))


@pytest.mark.parametrize("D,T,seed", [(4, 1, 1), (4, 17, 2), (4, 64, 3), (64, 24, 4)])
@pytest.mark.parametrize("with_state", [False, True])
def test_recurrence_matches_brute_force_sum(D, T, seed, with_state):
    r, k, v, w, u, s0 = random_slice(seed, T, D, state_sigma=0.5 if with_state else None)
    o, s = scan1(r, k, v, w, u, s0)
    ob, sb = oracle.wkv_sum_form(r, k, v, w, u, s0)
    np.testing.assert_allclose(o, ob, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(s, sb, rtol=1e-12, atol=1e-12)


def test_brute_force_on_bf16_inputs():
    r, k, v, w, u, s0 = random_slice(7, 33, 8, dtype="bf16", state_sigma=0.3)
    o, s = scan1(r, k, v, w, u, s0)
    ob, sb = oracle.wkv_sum_form(r, k, v, w, u, s0)
    np.testing.assert_allclose(o, ob, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(s, sb, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("T,D", [(50, 8), (300, 64)])
def test_no_decay_is_causal_linear_attention(T, D):
    """w == 1: o = (strictly causal (r k^T)) v + r S_0 + (r.u.k) v."""
    r, k, v, _, u, s0 = random_slice(11, T, D, state_sigma=0.2)
    w = np.ones((T, D), dtype=np.float32)
    o, s = scan1(r, k, v, w, u, s0)
    R, K, V, U = (a.astype(np.float64) for a in (r, k, v, u))
    scores = np.tril(R @ K.T, -1)
    expect = scores @ V + R @ s0.astype(np.float64) + ((R * U * K).sum(1))[:, None] * V
    np.testing.assert_allclose(o, expect, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(s, s0 + K.T @ V, rtol=1e-11, atol=1e-11)


def test_constant_decay_is_first_order_iir():
    """w_t = c (per key channel): S[i, j] is y[t] = c_i y[t-1] + k_t[i] v_t[j]."""
    from scipy.signal import lfilter
    T, D = 120, 6
    r, k, v, _, u, s0 = random_slice(13, T, D, state_sigma=0.4)
    c = np.linspace(0.3, 0.97, D).astype(np.float32)
    w = np.tile(c, (T, 1))
    o, s = scan1(r, k, v, w, u, s0)
    K, V, R, U = (a.astype(np.float64) for a in (k, v, r, u))
    S0 = s0.astype(np.float64)
    states = np.zeros((T + 1, D, D))        # states[t] = state before token t
    states[0] = S0
    for i in range(D):
        ci = float(c[i])
        for j in range(D):
            y, _ = lfilter([1.0], [1.0, -ci], K[:, i] * V[:, j], zi=[ci * S0[i, j]])
            states[1:, i, j] = y
    expect = np.einsum("ti,tij->tj", R, states[:-1]) + ((R * U * K).sum(1))[:, None] * V
    np.testing.assert_allclose(o, expect, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(s, states[-1], rtol=1e-10, atol=1e-10)


def test_single_token_by_hand():
    D = 5
    r, k, v, w, u, s0 = random_slice(17, 1, D, state_sigma=1.0)
    o, s = scan1(r, k, v, w, u, s0)
    R, K, V, W, U = (a[0].astype(np.float64) for a in (r, k, v, w, np.asarray(u)[None]))
    S0 = s0.astype(np.float64)
    expect_o = np.array([sum(R[i] * (S0[i, j] + U[i] * K[i] * V[j]) for i in range(D)) for j in range(D)])
    expect_s = np.array([[W[i] * S0[i, j] + K[i] * V[j] for j in range(D)] for i in range(D)])
    np.testing.assert_allclose(o[0], expect_o, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(s, expect_s, rtol=1e-14, atol=1e-14)


def test_bonus_isolation():
    r, k, v, w, u, s0 = random_slice(19, 40, 16, state_sigma=0.3)
    o_u, s_u = scan1(r, k, v, w, u, s0)
    o_0, s_0 = scan1(r, k, v, w, np.zeros_like(u), s0)
    R, K, V, U = (a.astype(np.float64) for a in (r, k, v, u))
    np.testing.assert_allclose(o_u - o_0, ((R * U * K).sum(1))[:, None] * V, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(s_u, s_0)       # the bonus never enters the state


@pytest.mark.parametrize("split", [1, 37, 64, 99])
def test_split_and_carry_invariant(split):
    T, D = 100, 16
    r, k, v, w, u, s0 = random_slice(23, T, D, state_sigma=0.3)
    o, s = scan1(r, k, v, w, u, s0)
    oa, sa = scan1(r[:split], k[:split], v[:split], w[:split], u, s0)
    ob, sb = scan1(r[split:], k[split:], v[split:], w[split:], u, sa)
    np.testing.assert_allclose(np.concatenate([oa, ob]), o, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(sb, s, rtol=1e-13, atol=1e-14)


def test_ragged_equals_separate_sequences():
    wl = make_workload(4, lengths=[5, 0, 17, 1, 9], H=3)
    o, s = oracle.wkv_scan(wl.r, wl.k, wl.v, wl.w, wl.u, wl.state0, wl.cu_seqlens)
    cu = wl.cu_seqlens
    for n in range(5):
        a, z = int(cu[n]), int(cu[n + 1])
        sl = lambda x: x[a:z][None]
        on, sn = oracle.wkv_scan(sl(wl.r), sl(wl.k), sl(wl.v), sl(wl.w), wl.u, wl.state0[n:n + 1])
        np.testing.assert_array_equal(o[a:z], on[0])
        np.testing.assert_array_equal(s[n], sn[0])
    # the empty sequence hands its state through unchanged
    np.testing.assert_array_equal(s[1], wl.state0[1].astype(np.float64))


def test_linearity_in_values_and_state_and_receptance():
    T, D = 30, 8
    r, k, _, w, u, _ = random_slice(29, T, D)
    # small-integer values and states keep the combination exact in float32
    g = np.random.default_rng(31)
    v1, v2 = (g.integers(-8, 9, size=(T, D)).astype(np.float32) for _ in range(2))
    s1, s2 = (g.integers(-8, 9, size=(D, D)).astype(np.float32) for _ in range(2))
    a, b = 0.75, -1.5
    o1, t1 = scan1(r, k, v1, w, u, s1)
    o2, t2 = scan1(r, k, v2, w, u, s2)
    o12, t12 = scan1(r, k, a * v1 + b * v2, w, u, a * s1.astype(np.float64) + b * s2.astype(np.float64))
    np.testing.assert_allclose(o12, a * o1 + b * o2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(t12, a * t1 + b * t2, rtol=1e-12, atol=1e-12)
    o3, _ = scan1(2.0 * r, k, v1, w, u, s1)
    np.testing.assert_allclose(o3, 2.0 * o1, rtol=1e-14, atol=1e-14)


def test_key_channel_permutation_and_value_column_permutation():
    T, D = 25, 8
    r, k, v, w, u, s0 = random_slice(37, T, D, state_sigma=0.5)
    o, s = scan1(r, k, v, w, u, s0)
    p = np.random.default_rng(0).permutation(D)
    # permute key channels consistently: r, k, w, u and rows of S_0
    op, sp = scan1(r[:, p], k[:, p], v, w[:, p], u[p], s0[p, :])
    np.testing.assert_allclose(op, o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(sp, s[p, :], rtol=1e-12, atol=1e-13)
    # permute value channels: v and columns of S_0; o and state columns follow
    oq, sq = scan1(r, k, v[:, p], w, u, s0[:, p])
    np.testing.assert_allclose(oq, o[:, p], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(sq, s[:, p], rtol=1e-12, atol=1e-13)
    # value columns are independent: changing column 0 of v leaves others alone
    v2 = v.copy()
    v2[:, 0] += 1.0
    o2, _ = scan1(r, k, v2, w, u, s0)
    np.testing.assert_array_equal(o2[:, 1:], o[:, 1:])


def test_heads_and_sequences_are_independent():
    wl = make_workload(1, B=2, T=40, H=3)
    o, s = oracle.wkv_scan(wl.r, wl.k, wl.v, wl.w, wl.u)
    for b in range(2):
        for h in range(3):
            sl = lambda x: x[b:b + 1, :, h:h + 1]
            oh, sh = oracle.wkv_scan(sl(wl.r), sl(wl.k), sl(wl.v), sl(wl.w), wl.u[h:h + 1])
            np.testing.assert_array_equal(oh[0, :, 0], o[b, :, h])
            np.testing.assert_array_equal(sh[0, 0], s[b, h])


def test_slice_mask_and_threads_do_not_change_results():
    wl = make_workload(1, B=1, T=70, H=4)
    o, s = oracle.wkv_scan(wl.r, wl.k, wl.v, wl.w, wl.u, threads=1)
    o4, s4 = oracle.wkv_scan(wl.r, wl.k, wl.v, wl.w, wl.u, threads=4)
    np.testing.assert_array_equal(o, o4)
    np.testing.assert_array_equal(s, s4)
    mask = np.array([0, 1, 0, 1], dtype=np.uint8)
    om, sm = oracle.wkv_scan(wl.r, wl.k, wl.v, wl.w, wl.u, slice_mask=mask)
    np.testing.assert_array_equal(om[:, :, 1], o[:, :, 1])
    np.testing.assert_array_equal(om[:, :, 0], 0.0)
    np.testing.assert_array_equal(sm[0, 3], s[0, 3])


def test_oracle_rejects_bad_offsets():
    wl = make_workload(4, lengths=[3, 4], H=1)
    bad = np.array([0, 5, 4], dtype=np.int64)
    with pytest.raises(ValueError):
        oracle.wkv_scan(wl.r, wl.k, wl.v, wl.w, wl.u, None, bad)


# ---- input generator ------------------------------------------------------

def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    x = np.random.default_rng(5).normal(0, 3, size=100000).astype(np.float32)
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 3.0e38]   # ties and overflow
    mine = f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(mine, ref)
    np.testing.assert_array_equal(bf16_bits_to_f32(mine),
                                  torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_generator_is_deterministic_and_head_stable():
    a = make_workload(1, T=32, H=4)
    b = make_workload(1, T=32, H=4)
    for name in ("r", "k", "v", "w", "u"):
        np.testing.assert_array_equal(getattr(a, name), getattr(b, name))
    c = make_workload(1, T=32, H=2)
    np.testing.assert_array_equal(a.r[:, :, :2], c.r)
    np.testing.assert_array_equal(a.w[:, :, :2], c.w)


def test_generator_distributions():
    wl = make_workload(1, T=512, H=4)
    w = bf16_bits_to_f32(wl.w)
    assert w.min() >= np.exp(-np.exp(-0.5)) - 1e-2 and w.max() <= 1.0
    rr = bf16_bits_to_f32(wl.r)
    assert abs(rr.std() - 0.125) < 0.01
    assert wl.state0 is None
    from synth.gen import ragged_lengths
    from synth import get_config
    L = ragged_lengths(get_config(4))
    assert len(L) == 16 and L.min() >= 1024 and L.max() <= 32768
    wl4 = make_workload(4, lengths=[3, 5], H=2)
    assert wl4.state0.shape == (2, 2, 64, 64) and wl4.r.shape == (8, 2, 64)


# ---- bf16 input decoding ----------------------------------------------------
# Every bf16 value the oracle sees passes through its decoders (the C one in
# wkv_oracle.c and oracle.bf16_bits_to_f64).  They are pinned here against
# torch's own bfloat16 -> float64 conversion on all 65536 bit patterns.

def _torch_bf16_table():
    torch = pytest.importorskip("torch")
    bits = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    return bits.view(torch.bfloat16).to(torch.float64).numpy()


def _same_values(got, ref, signed_zero=True, rtol=0.0):
    got = np.asarray(got, dtype=np.float64)
    nan = np.isnan(ref)
    np.testing.assert_array_equal(np.isnan(got), nan)
    if rtol:
        np.testing.assert_allclose(got[~nan], ref[~nan], rtol=rtol, atol=0)
    else:
        np.testing.assert_array_equal(got[~nan], ref[~nan])
    if signed_zero:                     # the table holds +0 and -0
        zero = ref == 0
        np.testing.assert_array_equal(np.signbit(got[zero]), np.signbit(ref[zero]))


def test_python_bf16_decoder_all_patterns():
    ref = _torch_bf16_table()
    _same_values(oracle.bf16_bits_to_f64(np.arange(65536, dtype=np.uint32).astype(np.uint16)), ref)


@pytest.mark.parametrize("role", ["r", "k", "v", "w", "d", "u2"])
def test_c_oracle_decodes_every_bf16_pattern(role):
    """One token, D = 1, one head per bit pattern, so that o (or the state)
    equals the decoded value of the pattern under test in the given role:
      r, k, v: o = r (S_0 + u k v) with the other two = 1, u = 1, S_0 = 0;
      w:       state = w S_0 + k v with S_0 = 1, k = 0;
      d:       the same with w = exp(-exp(d)) (decay given as d);
      u2:      Finch-C2 o = r S_0 + u' with r = 0."""
    ref = _torch_bf16_table()
    H = 65536
    pat = np.arange(H, dtype=np.uint32).astype(np.uint16).reshape(1, 1, H, 1)
    one = np.full_like(pat, 0x3F80)
    zero = np.zeros_like(pat)
    u = np.ones((H, 1), dtype=np.float32)
    args = dict(r=one, k=one, v=one, w=one)
    s0 = None
    kw = {}
    if role in ("r", "k", "v"):
        args[role] = pat
    elif role in ("w", "d"):
        args["w"], args["k"] = pat, zero
        s0 = np.ones((1, H, 1, 1))
        if role == "d":
            kw["decay"] = "log"
    else:
        args["r"] = zero
        kw.update(variant="c2", second_value=pat)
    o, s = oracle.wkv_scan(args["r"], args["k"], args["v"], args["w"], u, s0, **kw)
    if role in ("w", "d"):
        got = s.reshape(H)
        if role == "d":
            with np.errstate(over="ignore", invalid="ignore"):
                ref = np.exp(-np.exp(ref))
        # exp() of the C library and of numpy may differ in the last bit, and
        # exp(-x) multiplies the relative error of x = exp(d) by x
        _same_values(got, ref, signed_zero=False, rtol=1e-12 if role == "d" else 0.0)
    else:
        # the read-out sums onto +0, so the sign of a zero is not observable
        _same_values(o.reshape(H), ref, signed_zero=False)


def _bf16_fixture(name):
    """A hand-worked fixture whose values are all exact in bf16, as bf16 bit
    patterns (the encoding round-trips exactly, which is checked)."""
    g = json.load(open(os.path.join(GOLDEN, name)))
    enc = {}
    for key in ("r", "k", "v", "w", "u2"):
        if key in g:
            x = np.array(g[key], dtype=np.float32)
            bits = f32_to_bf16_bits(x)
            np.testing.assert_array_equal(bf16_bits_to_f32(bits), x)
            enc[key] = bits
    return g, enc


def test_hand_worked_fixture_in_bf16():
    g, b = _bf16_fixture("hand_worked_d2_t3.json")
    f = lambda key: np.array(g[key], dtype=np.float32)
    o, s = scan1(b["r"], b["k"], b["v"], b["w"], f("u"), f("state0"))
    np.testing.assert_array_equal(o, np.array(g["o"]))
    np.testing.assert_array_equal(s, np.array(g["state_final"]))
    o2, s2 = oracle.wkv_sum_form(b["r"], b["k"], b["v"], b["w"], f("u"), f("state0"))
    np.testing.assert_array_equal(o2, np.array(g["o"]))
    np.testing.assert_array_equal(s2, np.array(g["state_final"]))


def test_c2_hand_worked_fixture_in_bf16():
    g, b = _bf16_fixture("hand_worked_c2_d2_t3.json")
    D = 2
    T = len(g["r"])
    add = lambda a: a.reshape(1, T, 1, D)
    s0 = np.array(g["state0"], dtype=np.float64).reshape(1, 1, D, D)
    o, s = oracle.wkv_scan(add(b["r"]), add(b["k"]), add(b["v"]), add(b["w"]), None, s0,
                           variant="c2", second_value=add(b["u2"]))
    np.testing.assert_array_equal(o.reshape(T, D), np.array(g["o"]))
    np.testing.assert_array_equal(s.reshape(D, D), np.array(g["state_final"]))
