"""The allocation-free entry point (wkv_prefill_noalloc) against the regular
one (wkv_prefill_ex through the binding), through the C ABI: two calls in a
row, the second smaller, each bit for bit equal to the regular call."""
import ctypes

import numpy as np
import pytest

from synth import make_workload
from gpu_util import log, to_gpu, run_gpu, run_oracle, errors

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _noalloc(lib, g, flags=0):
    B, T, H, D = g["r"].shape
    o = torch.full((B, T, H, D), float("nan"), dtype=torch.float32, device="cuda")
    st = torch.full((B, H, D, D), float("nan"), dtype=torch.float32, device="cuda")
    status = lib.wkv_prefill_noalloc(_p(g["r"]), _p(g["k"]), _p(g["v"]), _p(g["w"]), _p(g["u"]), None,
                                     _p(g["state0"]), _p(o), _p(st), B, T, H, D, 1, flags,
                                     ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert status == 0, lib.wkv_last_error()
    return o, st


def test_noalloc_matches_regular_entry_point():
    from linear_attention_rnn_finch_amd import _binding
    lib = _binding._lib
    lib.wkv_prefill_noalloc.restype = ctypes.c_int
    lib.wkv_prefill_noalloc.argtypes = [ctypes.c_void_p] * 9 + [ctypes.c_int] * 5 + [ctypes.c_uint, ctypes.c_void_p]
    # first the 1.5B layer shape (16 segments per head: the scratch holds 512
    # aggregates and start states), then a smaller split call with states
    for cfg, kw in ((1, {}), (3, dict(B=2, T=1500, H=4))):
        wl = make_workload(cfg, **kw)
        g = to_gpu(wl)
        log("noalloc case %s %s" % (wl.config.name, kw))
        o_ref, s_ref = run_gpu(wl, g)
        o, st = _noalloc(lib, g)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(st, s_ref)
        heads = [0, wl.u.shape[0] - 1]
        o_or, s_or = run_oracle(wl, heads)
        eo, es = errors(wl, o, st, o_or, s_or, heads)
        assert eo <= 2e-3 and es <= 2e-3
    # the static scratch's control records: no bounded wait expired
    import linear_attention_rnn_finch_amd as fw
    assert fw.workspace_errors(None) == 0
