"""The chunked scan's bf16 hi/lo splits, emulated on the CPU
(tests/split_emulation.py): with every split product the kernel's arithmetic
stays far inside the 2e-3 bar against the fp64 oracle, and leaving out any one
product puts the worst token row above it.  This is why the kernel keeps all
of them."""
import numpy as np
import pytest

import oracle
import split_emulation as se
from synth import make_workload

torch = pytest.importorskip("torch")

BAR = 2e-3


def test_rounding_helpers_match_torch():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-30, 30, 100000))).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(se.rne_bf16(x), want)
    hi = se.trunc_bf16(x)
    assert (np.abs(hi) <= np.abs(x)).all() and np.array_equal(se.trunc_bf16(hi), hi)
    for hi_rne in (False, True):
        h, lo = se.split(x, hi_rne)
        # hi + lo carries x to 16 significant bits
        assert (np.abs(h.astype(np.float64) + lo - x) <= np.abs(x) * 2.0 ** -16).all()


@pytest.fixture(scope="module")
def layer_slice():
    wl = make_workload(1, T=1024, H=8)          # the 1.5B-class layer's distributions, 16 chunks, 8 heads
    o_ref, s_ref = oracle.wkv_scan(wl.r, wl.k, wl.v, wl.w, wl.u, wl.state0)
    return se.workload_arrays(wl), o_ref[0], s_ref[0]


def test_all_splits_stay_far_inside_the_bar(layer_slice):
    (r, k, v, w, u, s0), o_ref, s_ref = layer_slice
    o, s = se.chunked_scan(r, k, v, w, u, s0)
    block, row, state = se.errors(o, o_ref, s, s_ref)
    assert block < 1e-4 and row < 2e-4 and state < 1e-4, (block, row, state)


def test_nearest_rounded_hi_parts_halve_the_error(layer_slice):
    (r, k, v, w, u, s0), o_ref, s_ref = layer_slice
    o, s = se.chunked_scan(r, k, v, w, u, s0)
    o_t, s_t = se.chunked_scan(r, k, v, w, u, s0, dict(hi_trunc=True))
    near, trunc = se.errors(o, o_ref, s, s_ref), se.errors(o_t, o_ref, s_t, s_ref)
    assert all(a <= 0.6 * b for a, b in zip(near, trunc)), (near, trunc)


@pytest.mark.parametrize("name", [n for n in se.VARIANTS if n.startswith(("A's", "k~", "S's", "r~", "no "))])
def test_dropping_any_product_fails_the_row_bar(layer_slice, name):
    (r, k, v, w, u, s0), o_ref, s_ref = layer_slice
    o, s = se.chunked_scan(r, k, v, w, u, s0, se.VARIANTS[name])
    block, row, state = se.errors(o, o_ref, s, s_ref)
    assert row > BAR, (name, block, row, state)
