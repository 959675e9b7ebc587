"""The workloads of the Finch WKV pre-fill, with their input recipes.

Shapes follow the pages' model sizes: the 1.5B-class layer (24 layers,
d_model 2048) of the GoldFinch experiments and the 32-layer, d_model 4096,
256k-context point of the cache-size table; the head size is 64.  The last
two are recurrent generation steps of the 1.5B-class layer: a batch of 128
sequences continuing from pre-filled states (random fp32 here), one and
sixteen tokens per call.  The pages
give no head size and no input distributions: those below are the stated
workload recipes, drawn from fixed seeds.

``sigma`` is a standard deviation.  Decays are w = exp(-exp(x)) with x uniform
on ``x_range``; the bonus u ~ N(0, 0.5) per (head, channel); initial states are
N(0, ``state_sigma``) fp32 or absent (zeros).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Tuple


@dataclass(frozen=True)
class WorkloadConfig:
    index: int
    name: str
    B: int                      # sequences (ragged: number of packed sequences)
    T: int                      # tokens per sequence (ragged: 0, see lengths)
    H: int
    D: int
    dtype: str                  # "f32" or "bf16" for r, k, v, w
    rkv_sigma: float
    x_range: Tuple[float, float]
    u_sigma: float
    state_sigma: Optional[float]
    ragged_lengths: Optional[Tuple[int, int]] = None   # inclusive U{lo..hi}
    tolerance: float = 2e-3
    seed: int = 0

    @property
    def d_model(self) -> int:
        return self.H * self.D


_BASE_SEED = 20240716

CONFIGS = (
    WorkloadConfig(0, "tiny_f32", B=1, T=64, H=1, D=64, dtype="f32",
                   rkv_sigma=1.0, x_range=(-6.0, -1.0), u_sigma=0.5,
                   state_sigma=None, tolerance=1e-5, seed=_BASE_SEED + 0),
    WorkloadConfig(1, "layer_1p5b_t4096", B=1, T=4096, H=32, D=64, dtype="bf16",
                   rkv_sigma=1.0 / 8.0, x_range=(-8.0, -0.5), u_sigma=0.5,
                   state_sigma=None, seed=_BASE_SEED + 1),
    WorkloadConfig(2, "train_batch_b8_t4096", B=8, T=4096, H=32, D=64,
                   dtype="bf16", rkv_sigma=1.0 / 8.0, x_range=(-8.0, -0.5),
                   u_sigma=0.5, state_sigma=None, seed=_BASE_SEED + 2),
    WorkloadConfig(3, "long_context_t262144", B=1, T=262144, H=64, D=64,
                   dtype="bf16", rkv_sigma=1.0 / 8.0, x_range=(-10.0, -1.0),
                   u_sigma=0.5, state_sigma=0.1, seed=_BASE_SEED + 3),
    WorkloadConfig(4, "ragged_16seq", B=16, T=0, H=32, D=64, dtype="bf16",
                   rkv_sigma=1.0 / 8.0, x_range=(-8.0, -0.5), u_sigma=0.5,
                   state_sigma=0.1, ragged_lengths=(1024, 32768),
                   seed=_BASE_SEED + 4),
    WorkloadConfig(5, "step_b128_t1", B=128, T=1, H=32, D=64, dtype="bf16",
                   rkv_sigma=1.0 / 8.0, x_range=(-8.0, -0.5), u_sigma=0.5,
                   state_sigma=0.1, seed=_BASE_SEED + 5),
    WorkloadConfig(6, "step_b128_t16", B=128, T=16, H=32, D=64, dtype="bf16",
                   rkv_sigma=1.0 / 8.0, x_range=(-8.0, -0.5), u_sigma=0.5,
                   state_sigma=0.1, seed=_BASE_SEED + 6),
)


def get_config(key) -> WorkloadConfig:
    if isinstance(key, WorkloadConfig):
        return key
    if isinstance(key, int):
        return CONFIGS[key]
    for c in CONFIGS:
        if c.name == key:
            return c
    raise KeyError(key)
