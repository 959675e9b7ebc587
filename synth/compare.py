"""Normwise per-block error used for every GPU-vs-oracle comparison.

A block is one (sequence, head) slice of ``o`` ([L, D]) or of the final state
([D, D]).  Its error is max|g - ref| / max|ref|; the reported figure is the
maximum over blocks.  A block whose reference is identically zero reports the
absolute max|g|.  Element-wise |g - ref| / |ref| is ill-posed where the
reference crosses zero, which is why the norm is taken per block.
"""
from __future__ import annotations

import numpy as np


def _blocks_o(o, cu_seqlens):
    """Yield [L, D] blocks of o ([B,T,H,D] or packed [tokens,H,D])."""
    if cu_seqlens is None:
        B, T, H, D = o.shape
        for b in range(B):
            for h in range(H):
                yield (b, h), o[b, :, h, :]
    else:
        _, H, D = o.shape
        for n in range(len(cu_seqlens) - 1):
            a, z = int(cu_seqlens[n]), int(cu_seqlens[n + 1])
            for h in range(H):
                yield (n, h), o[a:z, h, :]


def block_errors(got, ref, cu_seqlens=None, *, kind="o"):
    """Dict {(seq, head): error} for o (kind="o") or states (kind="state")."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if got.shape != ref.shape:
        raise ValueError("shape mismatch %s vs %s" % (got.shape, ref.shape))
    out = {}
    if kind == "state":
        N, H = ref.shape[:2]
        pairs = (((n, h), got[n, h], ref[n, h]) for n in range(N) for h in range(H))
    else:
        pairs = ((key, g, r) for (key, g), (_, r) in
                 zip(_blocks_o(got, cu_seqlens), _blocks_o(ref, cu_seqlens)))
    for key, g, r in pairs:
        if g.size == 0:
            out[key] = 0.0
            continue
        den = float(np.max(np.abs(r)))
        num = float(np.max(np.abs(g - r)))
        if not np.isfinite(num):
            out[key] = float("inf")
        else:
            out[key] = num / den if den > 0 else num
    return out


def max_block_error(got, ref, cu_seqlens=None, *, kind="o") -> float:
    errs = block_errors(got, ref, cu_seqlens, kind=kind)
    return max(errs.values()) if errs else 0.0
