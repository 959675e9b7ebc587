"""Oracle for the two steps that follow the scan in Finch-C2 pre-fill -- plain
fp64 numpy.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  It
shares no code with the GPU library and never imports it.

* ``layernorm_heads`` -- the LayerNorm over the concatenated heads of the
  Finch-C2 output equation (GoldFinch architecture summary page, section 3.4,
  "Finch-C2 Time Mixing", output equation: LayerNorm(concat(r_t wkv_t +
  u'_t)) W_O; the norm spans all heads of a token, replacing base Finch's
  per-head GroupNorm).  Standard LayerNorm: population mean and variance over
  the row, (x - mean) / sqrt(var + eps), then the learned per-channel scale
  and shift.
* ``gold_compress`` -- the GOLD key compression (same page, "GOLD Key
  Compression and TokenCat Decompression", compression step): c_t = x_t W_KD
  with W_KD of shape [D, D/16], x_t the output of the last Finch-C2 layer.
  The weight is passed in the [D/16, D] (output-major) layout, i.e. W_KD
  transposed; c = x @ w_out_major.T.

Parity status: pinned by ``tests/test_oracle_epilogue.py`` (hand-worked
LayerNorm row, constant rows, shift and scale invariance, moments of the
output, brute-force products, selection matrices).
"""
from __future__ import annotations

import numpy as np

from . import as_f64


def layernorm_heads(x, gamma, beta, eps=1e-5):
    """x: [..., W] (float32 or bf16 bits); gamma, beta: [W] float32.
    Returns the normalised rows in float64."""
    x = as_f64(x)
    g = np.asarray(gamma, dtype=np.float64)
    b = np.asarray(beta, dtype=np.float64)
    mean = x.mean(axis=-1, keepdims=True)
    var = ((x - mean) ** 2).mean(axis=-1, keepdims=True)
    return (x - mean) / np.sqrt(var + eps) * g + b


def gold_compress(x, w_out_major):
    """x: [M, D] (bf16 bits or float32); w_out_major: [D/16, D] (bf16 bits or
    float32), the transposed W_KD.  Returns c = x W_KD [M, D/16] in float64."""
    x = as_f64(x)
    w = as_f64(w_out_major)
    return x @ w.T
