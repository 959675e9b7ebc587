"""CPU emulation of the chunked scan's arithmetic, to measure which bf16 hi/lo
split products the matrix-core evaluation needs.

The chunked form (64-token chunks; [Summary] section 3.4, "Training and
Inference Procedures": pre-fill in parallel chunks of the recurrence) feeds
the matrix cores bf16 operands.  An fp32 operand x is carried as
hi = x rounded to nearest-even bf16 and lo = x - hi rounded the same way, and
a product of two such operands as hi*hi + hi*lo + lo*hi.  This module repeats the
kernel's chunk arithmetic on the CPU with every operand rounded as the kernel
rounds it, and can leave out any of the split products:

- per chunk, prefix products P_t of the decays (fp32), r~_t = r_t P_{t-1} and
  k~_s = k_s / P_s (fp32), the bonus sum_i r u k on the diagonal;
- A[t][s] = r~_t . k~_s for s < t (from the split r~ and k~), then A split;
- o = r~ S (split r~, split S) + A v (split A, bf16 v);
- S <- diag(P_63) (S + k~^T v) (split k~).

The hi parts may also be truncated instead (the kernel's earlier form, one
byte permute per two values in place of one packing convert): the remainder
is then up to a whole bf16 ulp, and the errors are about twice as large.

A matrix-core instruction is emulated as exact products of its bf16 inputs
summed in fp64 over its 32-wide contraction slice, added to the fp32
accumulator and rounded to fp32 once; the instructions follow the kernel's
order.  Chunks whose decay product falls below 2^-96 take an exact
token-serial path in the kernel; the workloads here have none (checked).

Test infrastructure only: this models the GPU kernel's rounding; it shares no
code with the oracle, and nothing in the library imports it.

    python tests/split_emulation.py [config]     # the table for a workload
"""
from __future__ import annotations

import os
import sys

import numpy as np

CHUNK = 64
MIN_CHUNK_DECAY = 2.0 ** -96

# products kept, by name: (A tile, read-out, state update, in-chunk pairs)
FULL = dict(a_hl=True, a_lh=True, ro_rl=True, ro_sl=True, st_kl=True, pr_al=True)
VARIANTS = {
    "all splits (the kernel)": {},
    "all splits, hi truncated (the earlier kernel)": dict(hi_trunc=True),
    "A's lo part dropped in the in-chunk pairs": dict(pr_al=False),
    "k~'s lo part dropped in the state update": dict(st_kl=False),
    "S's lo part dropped in the read-out": dict(ro_sl=False),
    "r~'s lo part dropped in the read-out": dict(ro_rl=False),
    "no split in the read-out": dict(ro_rl=False, ro_sl=False),
    "r~ and k~ unsplit inside the A tiles": dict(a_hl=False, a_lh=False),
    "no splits at all": dict(a_hl=False, a_lh=False, ro_rl=False, ro_sl=False, st_kl=False, pr_al=False),
}


def bf16_bits_to_f32(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def trunc_bf16(x):
    """x (fp32) with its low 16 bits cleared."""
    return (np.asarray(x, dtype=np.float32).view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)


def rne_bf16(x):
    """x (fp32, finite) rounded to the nearest bf16, ties to even."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def split(x, hi_rne=False):
    """(hi, lo) with hi + lo = x to about 16 bits: hi truncated (the kernel's
    split) or rounded to nearest, lo the rounded remainder."""
    hi = rne_bf16(x) if hi_rne else trunc_bf16(x)
    lo = rne_bf16((x - hi).astype(np.float32))       # x - hi is exact in fp32
    return hi, lo


def mfma_chain(acc, pairs):
    """acc (fp32, [..., M, N]) plus sum of a @ b over `pairs`, one 32-wide
    contraction slice at a time, products of a slice in the given order,
    each instruction rounded to fp32 once."""
    K = pairs[0][0].shape[-1]
    for k0 in range(0, K, 32):
        for a, b in pairs:
            p = np.matmul(a[..., k0:k0 + 32].astype(np.float64), b[..., k0:k0 + 32, :].astype(np.float64))
            acc = (acc.astype(np.float64) + p).astype(np.float32)
    return acc


def chunked_scan(r, k, v, w, u, state0=None, keep=None):
    """One sequence: r, k, v, w fp32 [T, H, D] (bf16 values), u fp32 [H, D],
    state0 fp32 [H, D, D] or None.  Returns o fp32 [T, H, D] and the final
    state fp32 [H, D, D].  `keep` names products to leave out (False) and
    hi_trunc=True truncates the hi parts."""
    keep = {**FULL, "hi_trunc": False, **(keep or {})}
    hi_rne = not keep.pop("hi_trunc")
    split_ = lambda x: split(x, hi_rne)
    T, H, D = r.shape
    S = np.zeros((H, D, D), np.float32) if state0 is None else state0.astype(np.float32).copy()
    o = np.zeros((T, H, D), np.float32)
    for t0 in range(0, T, CHUNK):
        n = min(CHUNK, T - t0)
        # [H, token, channel], padding tokens: r = k = v = 0, w = 1
        def take(x, pad):
            out = np.full((H, CHUNK, D), pad, np.float32)
            out[:, :n] = np.transpose(x[t0:t0 + n], (1, 0, 2))
            return out
        rr, kk, vv, ww = take(r, 0.0), take(k, 0.0), take(v, 0.0), take(w, 1.0)
        P = np.cumprod(ww, axis=1, dtype=np.float32)                     # P_t, inclusive
        P_prev = np.concatenate([np.ones((H, 1, D), np.float32), P[:, :-1]], axis=1)
        if not (P[:, -1] >= MIN_CHUNK_DECAY).all():
            raise ValueError("stiff chunk at token %d: not modelled" % t0)
        rt = (rr * P_prev).astype(np.float32)
        kt = (kk * (np.float32(1.0) / P).astype(np.float32)).astype(np.float32)
        bonus = np.sum(rr * u[:, None, :] * kk, axis=2, dtype=np.float32)   # [H, token]
        rt_hi, rt_lo = split_(rt)
        kt_hi, kt_lo = split_(kt)
        ktT_hi, ktT_lo = np.swapaxes(kt_hi, 1, 2), np.swapaxes(kt_lo, 1, 2)
        # in-chunk matrix A[t][s] = r~_t . k~_s, masked: s < t kept, bonus on s = t
        pairs = [(rt_hi, ktT_hi)]
        if keep["a_hl"]:
            pairs.append((rt_hi, ktT_lo))
        if keep["a_lh"]:
            pairs.append((rt_lo, ktT_hi))
        A = mfma_chain(np.zeros((H, CHUNK, CHUNK), np.float32), pairs)
        tri = np.tril(np.ones((CHUNK, CHUNK), bool), -1)
        A = np.where(tri, A, np.float32(0.0))
        idx = np.arange(CHUNK)
        A[:, idx, idx] = bonus
        a_hi, a_lo = split_(A)
        # read-out of the carried state
        s_hi, s_lo = split_(S)
        pairs = [(rt_hi, s_hi)]
        if keep["ro_rl"]:
            pairs.append((rt_lo, s_hi))
        if keep["ro_sl"]:
            pairs.append((rt_hi, s_lo))
        acc = mfma_chain(np.zeros((H, CHUNK, D), np.float32), pairs)
        # state update S = diag(P_63) (S + k~^T v)
        pairs = [(ktT_hi, vv)]
        if keep["st_kl"]:
            pairs.append((ktT_lo, vv))
        p = mfma_chain(np.zeros((H, D, D), np.float32), pairs)
        S = (P[:, -1][:, :, None] * (S + p).astype(np.float32)).astype(np.float32)
        # in-chunk pairs o += A v
        pairs = [(a_hi, vv)]
        if keep["pr_al"]:
            pairs.append((a_lo, vv))
        acc = mfma_chain(acc, pairs)
        o[t0:t0 + n] = np.transpose(acc[:, :n], (1, 0, 2))
    return o, S


def errors(o, o_ref, s, s_ref):
    """Normwise block errors (max |g - ref| / max |ref| over a head's block)
    and the worst per-row error (max over j of |g - ref| / max over j of |ref|)."""
    eo = np.abs(o - o_ref).max(axis=(0, 2)) / np.abs(o_ref).max(axis=(0, 2))
    es = np.abs(s - s_ref).max(axis=(1, 2)) / np.abs(s_ref).max(axis=(1, 2))
    den = np.abs(o_ref).max(axis=2)
    row = np.abs(o - o_ref).max(axis=2)[den > 0] / den[den > 0]
    return float(eo.max()), float(row.max()), float(es.max())


def workload_arrays(wl, seq=0):
    """fp32 views of one sequence of a synthetic workload ([T, H, D])."""
    f = lambda x: bf16_bits_to_f32(x[seq]) if x.dtype == np.uint16 else x[seq].astype(np.float32)
    s0 = None if wl.state0 is None else wl.state0[seq]
    return f(wl.r), f(wl.k), f(wl.v), f(wl.w), wl.u.astype(np.float32), s0


def main(argv):
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    sys.path.insert(0, root)
    from synth import make_workload
    import oracle
    cfg = argv[1] if len(argv) > 1 else "1"
    wl = make_workload(int(cfg) if cfg.isdigit() else cfg)
    if wl.packed:
        raise SystemExit("fixed-length workloads only")
    r, k, v, w, u, s0 = workload_arrays(wl)
    o_ref, s_ref = oracle.wkv_scan(wl.r, wl.k, wl.v, wl.w, wl.u, wl.state0)
    o_ref, s_ref = o_ref[0], s_ref[0]
    print("| Products kept | block err (o) | worst row (o) | state |")
    print("|---|---|---|---|")
    for name, keep in VARIANTS.items():
        o, s = chunked_scan(r, k, v, w, u, s0, keep)
        eo, er, es = errors(o, o_ref, s, s_ref)
        print("| %s | %.1e | %.1e | %.1e |" % (name, eo, er, es), flush=True)


if __name__ == "__main__":
    main(sys.argv)
