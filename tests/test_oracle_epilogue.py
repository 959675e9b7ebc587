"""Pins of the epilogue oracle (oracle/epilogue.py) against facts that do not
come from it: hand-worked LayerNorm rows, a constant row, shift and scale
invariance, the first two moments of the output, brute-force products and
selection matrices for the GOLD compression.  Planted mistakes in a copy of
the LayerNorm must each fail one of them."""
import numpy as np
import pytest

import oracle
from oracle import epilogue
from synth import f32_to_bf16_bits


def test_layernorm_hand_worked_rows():
    # x = [0, 0, 4, 4]: mean 2, deviations [-2, -2, 2, 2], variance 4, eps 0
    # -> normalised [-1, -1, 1, 1]; scale [1, 2, 0.5, 1], shift [0, 1, 0, -1]
    y = epilogue.layernorm_heads(np.array([[0.0, 0.0, 4.0, 4.0]], np.float32),
                                 np.array([1.0, 2.0, 0.5, 1.0], np.float32),
                                 np.array([0.0, 1.0, 0.0, -1.0], np.float32), eps=0.0)
    np.testing.assert_array_equal(y, [[-1.0, -1.0, 0.5, 0.0]])
    # x = [1, 1, 1, 5]: mean 2, variance 3, eps 1 -> sqrt(4) = 2
    # -> normalised [-0.5, -0.5, -0.5, 1.5]
    y = epilogue.layernorm_heads(np.array([[1.0, 1.0, 1.0, 5.0]], np.float32),
                                 np.ones(4, np.float32), np.zeros(4, np.float32), eps=1.0)
    np.testing.assert_array_equal(y, [[-0.5, -0.5, -0.5, 1.5]])


def _pins_layernorm(ln):
    """Every LayerNorm pin on a function with the oracle's signature."""
    g = np.random.default_rng(1)
    W = 2048
    x = g.normal(0, 0.3, size=(6, W)).astype(np.float32)
    gamma = (1 + g.normal(0, 0.1, size=W)).astype(np.float32)
    beta = g.normal(0, 0.1, size=W).astype(np.float32)
    # hand-worked row
    if not np.array_equal(ln(np.array([[0.0, 0.0, 4.0, 4.0]], np.float32),
                             np.array([1.0, 2.0, 0.5, 1.0], np.float32),
                             np.array([0.0, 1.0, 0.0, -1.0], np.float32), eps=0.0),
                          [[-1.0, -1.0, 0.5, 0.0]]):
        return False
    # constant row -> the shift
    c = np.full((1, W), 3.25, np.float32)
    if not np.allclose(ln(c, gamma, beta, eps=1e-5), beta[None].astype(np.float64), rtol=0, atol=1e-12):
        return False
    # shift and scale invariance (eps = 0)
    if not np.allclose(ln(x, gamma, beta, eps=0.0),
                       ln((x.astype(np.float64) * 7.5 - 2.0), gamma, beta, eps=0.0), rtol=1e-11, atol=1e-11):
        return False
    # moments with unit scale and zero shift (eps = 0): mean 0, mean square 1
    y = ln(x, np.ones(W, np.float32), np.zeros(W, np.float32), eps=0.0)
    if not (np.allclose(y.mean(-1), 0, atol=1e-12) and np.allclose((y * y).mean(-1), 1, atol=1e-12)):
        return False
    # with eps: mean square = var / (var + eps), per row
    v = x.astype(np.float64).var(-1)
    y = ln(x, np.ones(W, np.float32), np.zeros(W, np.float32), eps=0.05)
    return bool(np.allclose((y * y).mean(-1), v / (v + 0.05), rtol=1e-12))


def test_layernorm_pins():
    assert _pins_layernorm(epilogue.layernorm_heads)


def _ln_ddof1(x, gamma, beta, eps=1e-5):
    x = oracle.as_f64(x)
    m = x.mean(-1, keepdims=True)
    return (x - m) / np.sqrt(x.var(-1, ddof=1, keepdims=True) + eps) * gamma + beta


def _ln_eps_outside(x, gamma, beta, eps=1e-5):
    x = oracle.as_f64(x)
    m = x.mean(-1, keepdims=True)
    return (x - m) / (np.sqrt(((x - m) ** 2).mean(-1, keepdims=True)) + eps) * gamma + beta


def _ln_no_centering(x, gamma, beta, eps=1e-5):
    x = oracle.as_f64(x)
    return x / np.sqrt((x * x).mean(-1, keepdims=True) + eps) * gamma + beta


def _ln_swapped_affine(x, gamma, beta, eps=1e-5):
    return epilogue.layernorm_heads(x, beta, gamma, eps)


@pytest.mark.parametrize("wrong", [_ln_ddof1, _ln_eps_outside, _ln_no_centering, _ln_swapped_affine])
def test_layernorm_pins_reject_planted_mistakes(wrong):
    assert not _pins_layernorm(wrong)


def _brute(x, w):
    x, w = oracle.as_f64(x), oracle.as_f64(w)
    M, D = x.shape
    N = w.shape[0]
    c = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for d in range(D):
                acc += x[m, d] * w[n, d]
            c[m, n] = acc
    return c


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_compress_matches_brute_force(dtype):
    g = np.random.default_rng(2)
    x = g.normal(size=(5, 64)).astype(np.float32)
    w = g.normal(size=(4, 64)).astype(np.float32)
    if dtype == "bf16":
        x, w = f32_to_bf16_bits(x), f32_to_bf16_bits(w)
    np.testing.assert_allclose(epilogue.gold_compress(x, w), _brute(x, w), rtol=1e-12, atol=1e-12)


def test_compress_selection_matrix_picks_columns():
    """Rows of the [D/16, D] weight that are unit vectors select columns of x."""
    g = np.random.default_rng(3)
    D = 256
    x = f32_to_bf16_bits(g.normal(size=(9, D)).astype(np.float32))
    pick = g.permutation(D)[: D // 16]
    w = np.zeros((D // 16, D), np.float32)
    w[np.arange(D // 16), pick] = 1.0
    c = epilogue.gold_compress(x, f32_to_bf16_bits(w))
    np.testing.assert_array_equal(c, oracle.as_f64(x)[:, pick])
    # and it is linear: a doubled weight doubles c exactly
    np.testing.assert_array_equal(epilogue.gold_compress(x, f32_to_bf16_bits(2 * w)), 2 * c)
