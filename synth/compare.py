"""Error measures for every GPU-vs-oracle comparison.

A block is one (sequence, head) slice of ``o`` ([L, D]) or of the final state
([D, D]).

* Normwise block error (the pass rule): max|g - ref| / max|ref| over the
  block; the reported figure is the maximum over blocks.  A block whose
  reference is identically zero reports the absolute max|g|.
* Per-row error: for every token row t of an o block (every key row of a
  state), max_j |g - ref| / max(max_j |ref|, floor), floor = 1e-3 rms(block).
  It catches an error confined to a few rows (early rows of a long block whose
  outputs grow over time, say) that the block maximum would hide.
* Floored element-wise error: |g - ref| / max(|ref|, floor), same floor.  The
  plain element-wise ratio is ill-posed where the reference crosses zero; the
  floor keeps it finite.  It is reported as a diagnostic only.
"""
from __future__ import annotations

import numpy as np

FLOOR = 1e-3      # floor of the per-row and element-wise denominators, relative to rms(block)


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


def _pairs(got, ref, cu_seqlens, kind):
    got = np.asarray(got)
    ref = np.asarray(ref)
    if got.shape != ref.shape:
        raise ValueError("shape mismatch %s vs %s" % (got.shape, ref.shape))
    if kind == "state":
        N, H = ref.shape[:2]
        return (((n, h), got[n, h], ref[n, h]) for n in range(N) for h in range(H))
    return ((key, g, r) for (key, g), (_, r) in
            zip(_blocks_o(got, cu_seqlens), _blocks_o(ref, cu_seqlens)))


def _block_measures(g, r):
    """(normwise, worst row, worst row index, floored element-wise) of one block."""
    g = np.asarray(g, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    if g.size == 0:
        return 0.0, 0.0, -1, 0.0
    diff = np.abs(g - r)
    num = float(diff.max())
    if not np.isfinite(num):
        return float("inf"), float("inf"), int(np.argmax(~np.isfinite(diff).all(axis=-1))), float("inf")
    absr = np.abs(r)
    den = float(absr.max())
    block = num / den if den > 0 else num
    floor = FLOOR * float(np.sqrt(np.mean(r * r)))
    if floor == 0.0:
        floor = 1.0                      # all-zero reference: absolute errors
    row_err = diff.max(axis=-1) / np.maximum(absr.max(axis=-1), floor)
    worst = int(np.argmax(row_err))
    elem = float((diff / np.maximum(absr, floor)).max())
    return block, float(row_err[worst]), worst, elem


def block_errors(got, ref, cu_seqlens=None, *, kind="o"):
    """Dict {(seq, head): normwise error} for o (kind="o") or states (kind="state")."""
    return {key: _block_measures(g, r)[0] for key, g, r in _pairs(got, ref, cu_seqlens, kind)}


def max_block_error(got, ref, cu_seqlens=None, *, kind="o") -> float:
    errs = block_errors(got, ref, cu_seqlens, kind=kind)
    return max(errs.values()) if errs else 0.0


def error_report(got, ref, cu_seqlens=None, *, kind="o", heads=None) -> dict:
    """All three measures, each maximised over the blocks, with the block (and
    row) where the worst per-row error sits.  ``heads`` maps the head axis of
    the arrays to the head numbers they hold (for the report only)."""
    rep = {"block": 0.0, "row": 0.0, "elem_floored": 0.0, "worst_row": None}
    for key, g, r in _pairs(got, ref, cu_seqlens, kind):
        b, rw, idx, el = _block_measures(g, r)
        rep["block"] = max(rep["block"], b)
        rep["elem_floored"] = max(rep["elem_floored"], el)
        if rw >= rep["row"] and idx >= 0:
            seq, h = key
            rep["row"] = rw
            rep["worst_row"] = {"seq": seq, "head": heads[h] if heads is not None else h, "row": idx}
    return rep
