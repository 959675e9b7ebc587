"""Seeded input generation (numpy PCG64, one substream per (tensor, head)).

Only random draws and storage rounding happen here.  bf16 values are produced
from float32 by round-to-nearest-even on the bit pattern and are returned as
uint16 bit patterns; the GPU receives exactly these bits and the oracle widens
exactly these bits.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

from .configs import WorkloadConfig, get_config

# substream tags
_R, _K, _V, _X, _U, _S0, _LEN, _U2 = 1, 2, 3, 4, 5, 6, 7, 8


def f32_to_bf16_bits(x) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest, ties to even.

    In uint32 arithmetic: add 0x7FFF plus the lowest kept bit, keep the top
    16 bits.  Only NaN patterns can wrap; they are replaced by a quiet NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    acc = u >> 16
    acc &= 1
    acc += 0x7FFF
    acc += u
    acc >>= 16
    out = acc.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=key)))


@dataclass
class Workload:
    config: WorkloadConfig
    r: np.ndarray                 # [B, T, H, D] or packed [tokens, H, D]
    k: np.ndarray
    v: np.ndarray
    w: np.ndarray
    u: np.ndarray                 # [H, D] float32
    state0: Optional[np.ndarray]  # [N, H, D, D] float32 or None
    cu_seqlens: Optional[np.ndarray] = None   # [N + 1] int64 (packed only)
    meta: dict = field(default_factory=dict)
    decay: str = "w"              # "w": the w array holds w; "log": it holds d (w = exp(-exp(d)))
    variant: str = "finch"        # "finch" (bonus u) or "c2" (k scaled by 1 - w, second value u2)
    u2: Optional[np.ndarray] = None   # Finch-C2 second value, like r (None: absent)

    @property
    def packed(self) -> bool:
        return self.cu_seqlens is not None

    @property
    def n_seq(self) -> int:
        return len(self.cu_seqlens) - 1 if self.packed else self.r.shape[0]

    @property
    def tokens(self) -> int:
        return int(self.cu_seqlens[-1]) if self.packed else self.r.shape[0] * self.r.shape[1]


def ragged_lengths(cfg: WorkloadConfig) -> np.ndarray:
    lo, hi = cfg.ragged_lengths
    return _rng(cfg.seed, _LEN).integers(lo, hi, size=cfg.B, endpoint=True).astype(np.int64)


def _default_workers() -> int:
    n = len(os.sched_getaffinity(0))
    return max(1, min(16, n))


def make_workload(cfg, *, T: Optional[int] = None, B: Optional[int] = None,
                  H: Optional[int] = None, lengths=None, heads=None,
                  seed: Optional[int] = None, workers: Optional[int] = None,
                  decay: str = "w", variant: str = "finch") -> Workload:
    """Draw the inputs of ``cfg`` (an index, a name or a WorkloadConfig).

    ``T``, ``B``, ``H``, ``lengths`` and ``seed`` override the config's sizes
    (same distributions) for reduced parity cases.  ``lengths`` (a list of
    sequence lengths) makes a packed ragged workload.  Every (tensor, head)
    pair draws from its own substream, so a head's values do not depend on H,
    nor on ``workers`` (threads filling the (tensor, head) pairs in parallel;
    numpy releases the GIL while it draws).

    ``decay="log"`` stores the decay draw x itself (the d of w = exp(-exp(d)))
    instead of w; ``variant="c2"`` adds the second value u2 ~ N(0, rkv_sigma)
    from its own substream.  Neither changes any other tensor's values.
    """
    if decay not in ("w", "log") or variant not in ("finch", "c2"):
        raise ValueError("decay must be 'w' or 'log', variant 'finch' or 'c2'")
    cfg = get_config(cfg)
    over = {}
    if T is not None:
        over["T"] = T
    if B is not None:
        over["B"] = B
    if H is not None:
        over["H"] = H
    if seed is not None:
        over["seed"] = seed
    if over:
        cfg = replace(cfg, **over)
    if lengths is None and cfg.ragged_lengths is not None:
        lengths = ragged_lengths(cfg)
    Hh, D = cfg.H, cfg.D
    bf16 = cfg.dtype == "bf16"
    store = np.uint16 if bf16 else np.float32

    if lengths is not None:
        lengths = np.asarray(lengths, dtype=np.int64)
        cu = np.zeros(len(lengths) + 1, dtype=np.int64)
        cu[1:] = np.cumsum(lengths)
        shape = (int(cu[-1]), Hh, D)
        n_seq = len(lengths)
    else:
        cu = None
        shape = (cfg.B, cfg.T, Hh, D)
        n_seq = cfg.B
    per_head = shape[:-2] + (D,)

    def draw(tag, h, fn):
        vals = fn(_rng(cfg.seed, tag, h), per_head)
        vals = np.asarray(vals, dtype=np.float32)
        return f32_to_bf16_bits(vals) if bf16 else vals

    def fn_w(g, s, lo=cfg.x_range[0], hi=cfg.x_range[1]):
        x = g.uniform(lo, hi, size=s)
        return x if decay == "log" else np.exp(-np.exp(x))

    def fn_rkv(g, s, sigma=cfg.rkv_sigma):
        return g.normal(0.0, sigma, size=s)

    tensors = (("r", _R), ("k", _K), ("v", _V), ("w", _X))
    if variant == "c2":
        tensors += (("u2", _U2),)
    out = {name: np.empty(shape, dtype=store) for name, _ in tensors}

    def fill(job):
        name, tag, h = job
        out[name][..., h, :] = draw(tag, h, fn_w if name == "w" else fn_rkv)

    jobs = [(name, tag, h) for name, tag in tensors for h in range(Hh)]
    n_workers = workers if workers is not None else _default_workers()
    if n_workers > 1 and len(jobs) > 1 and shape[0] * (shape[1] if len(shape) == 4 else 1) >= 4096:
        with ThreadPoolExecutor(max_workers=n_workers) as ex:
            list(ex.map(fill, jobs))
    else:
        for job in jobs:
            fill(job)

    u = np.stack([_rng(cfg.seed, _U, h).normal(0.0, cfg.u_sigma, size=D)
                  for h in range(Hh)]).astype(np.float32)
    state0 = None
    if cfg.state_sigma is not None:
        state0 = np.empty((n_seq, Hh, D, D), dtype=np.float32)
        for h in range(Hh):
            state0[:, h] = _rng(cfg.seed, _S0, h).normal(
                0.0, cfg.state_sigma, size=(n_seq, D, D)).astype(np.float32)

    wl = Workload(cfg, out["r"], out["k"], out["v"], out["w"], u, state0, cu,
                  decay=decay, variant=variant, u2=out.get("u2"))
    if heads is not None:
        wl = select_heads(wl, heads)
    return wl


def select_heads(wl: Workload, heads) -> Workload:
    heads = list(heads)
    sl = (Ellipsis, heads, slice(None))
    s0 = None if wl.state0 is None else np.ascontiguousarray(wl.state0[:, heads])
    u2 = None if wl.u2 is None else np.ascontiguousarray(wl.u2[sl])
    return Workload(replace(wl.config, H=len(heads)),
                    *(np.ascontiguousarray(a[sl]) for a in (wl.r, wl.k, wl.v, wl.w)),
                    np.ascontiguousarray(wl.u[heads]), s0, wl.cu_seqlens,
                    dict(wl.meta, heads=heads), decay=wl.decay, variant=wl.variant, u2=u2)


def random_slice(seed: int, T: int, D: int, *, dtype="f32", rkv_sigma=1.0,
                 x_range=(-6.0, -1.0), u_sigma=0.5, state_sigma=None):
    """A single (sequence, head) slice [T, D] for small oracle pins."""
    g = _rng(seed, 99)
    r, k, v = (g.normal(0.0, rkv_sigma, size=(T, D)).astype(np.float32) for _ in range(3))
    w = np.exp(-np.exp(g.uniform(x_range[0], x_range[1], size=(T, D)))).astype(np.float32)
    u = g.normal(0.0, u_sigma, size=D).astype(np.float32)
    s0 = None if state_sigma is None else g.normal(0.0, state_sigma, size=(D, D)).astype(np.float32)
    if dtype == "bf16":
        r, k, v, w = (f32_to_bf16_bits(a) for a in (r, k, v, w))
    return r, k, v, w, u, s0


def make_norm_inputs(tokens: int, width: int, seed: int = 7001):
    """Rows for the LayerNorm over heads: each row has its own offset
    mu ~ N(0, 0.5) and scale sigma ~ U(0.05, 1) (x = mu + sigma N(0, 1)), so
    both the centring and the scaling matter; gamma = 1 + N(0, 0.1),
    beta ~ N(0, 0.1).  All float32."""
    g = _rng(seed, 1)
    mu = g.normal(0.0, 0.5, size=(tokens, 1))
    sd = g.uniform(0.05, 1.0, size=(tokens, 1))
    x = (mu + sd * _rng(seed, 2).normal(size=(tokens, width))).astype(np.float32)
    gamma = (1.0 + _rng(seed, 3).normal(0.0, 0.1, size=width)).astype(np.float32)
    beta = _rng(seed, 4).normal(0.0, 0.1, size=width).astype(np.float32)
    return x, gamma, beta


def make_compress_inputs(tokens: int, d_model: int, seed: int = 7002):
    """Hidden states x ~ N(0, 1) [tokens, d_model] and a compression weight
    W_KD ~ N(0, 1/d_model) stored transposed [d_model/16, d_model], both as
    bf16 bit patterns."""
    x = _rng(seed, 1).normal(size=(tokens, d_model)).astype(np.float32)
    w = _rng(seed, 2).normal(0.0, d_model ** -0.5, size=(d_model // 16, d_model)).astype(np.float32)
    return f32_to_bf16_bits(x), f32_to_bf16_bits(w)
