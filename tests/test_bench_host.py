"""Host-side pieces of bench.py (CPU): the algorithmic bytes it divides by,
its model of the matrix-core instructions a call issues, and its mirror of
the library's whole-sequence rule, each checked against something outside
bench.py (the per-token byte count, the hardware counter in the committed
profile, the library's own plan through the C ABI)."""
import ctypes
import os
import re
from types import SimpleNamespace

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "linear_attention_rnn_finch_amd", "libfinch_wkv.so")


def cfg(H, dtype="bf16", D=64):
    return SimpleNamespace(H=H, D=D, dtype=dtype)


def test_algorithmic_bytes():
    # r, k, v, w in bf16 and o in fp32: 12 bytes per model channel and token,
    # plus the fp32 states out (and in)
    assert bench.algorithmic_bytes(cfg(32), 4096, 1, False) == 4096 * 12 * 2048 + 32 * 64 * 64 * 4
    assert bench.algorithmic_bytes(cfg(32), 8 * 4096, 8, False) == 809_500_672
    assert bench.algorithmic_bytes(cfg(64), 262144, 1, True) == 262144 * 12 * 4096 + 2 * 64 * 64 * 64 * 4
    # Finch-C2 adds the second value (bf16)
    assert bench.algorithmic_bytes(cfg(32), 4096, 1, False, "c2") == 4096 * 14 * 2048 + 32 * 64 * 64 * 4


def test_mfma_model_matches_the_hardware_counter():
    """The bench's instruction count for the layer call equals SQ_INSTS_MFMA
    measured on it (profiles/wkv_kernels_layer_1p5b_t4096_sq.md)."""
    text = open(os.path.join(ROOT, "profiles", "wkv_kernels_layer_1p5b_t4096_sq.md")).read()
    measured = int(re.search(r"\| SQ_INSTS_MFMA \| (\d+) \|", text).group(1))
    main, state, inner = bench.chunk_counts([4096], 32)
    assert (main, state, inner) == (64 * 32, 15 * 4 * 32, 15 * 32)
    model = bench.MAIN_MFMA_PER_CHUNK * main - bench.STATE_MFMA_PER_CHUNK * inner + bench.STATE_MFMA_PER_CHUNK * state
    assert model == measured


@pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")
@pytest.mark.parametrize("B,T,H", [(1, 4096, 32), (8, 4096, 32), (4, 4096, 32), (2, 1500, 128), (1, 262144, 64),
                                   (16, 300, 16), (3, 64, 8)])
def test_whole_sequence_rule_matches_the_library(B, T, H):
    """Whole-sequence plans are the split-free bf16 plans that would otherwise
    be split: they need no workspace, every split plan needs one."""
    lib = ctypes.CDLL(LIB)
    lib.wkv_prefill_workspace_bytes.restype = ctypes.c_size_t
    lib.wkv_prefill_workspace_bytes.argtypes = [ctypes.c_int] * 5
    need = lib.wkv_prefill_workspace_bytes(B, T, H, 64, 1)
    whole = bench.whole_sequence_plan([T] * B, H, packed=False)
    split = -(-T // bench._segment([T] * B, H)) > 1
    assert (need == 0) == (whole or not split), (need, whole, split)
