"""The C-ABI boundary on the GPU: the plain entry points called through ctypes
on torch buffers, bf16 outputs, explicit streams, and the binding's argument
checks (which must raise before any launch)."""
import ctypes

import numpy as np
import pytest

from synth import make_workload, bf16_bits_to_f32
from gpu_util import log, to_gpu, run_gpu, run_oracle, errors

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def test_plain_wkv_prefill_through_ctypes():
    """wkv_prefill itself (not the extended call the binding uses), on a
    split sequence with an initial state, against the oracle."""
    import linear_attention_rnn_finch_amd as fw
    from linear_attention_rnn_finch_amd import _binding
    wl = make_workload(3, B=2, T=1500, H=4)
    g = to_gpu(wl)
    B, T, H, D = g["r"].shape
    o = torch.empty((B, T, H, D), dtype=torch.float32, device="cuda")
    st = torch.empty((B, H, D, D), dtype=torch.float32, device="cuda")
    need = fw.workspace_bytes(B, T, H, D)
    ws = fw.new_workspace(need, "cuda")
    lib = _binding._lib
    status = lib.wkv_prefill(_ptr(g["r"]), _ptr(g["k"]), _ptr(g["v"]), _ptr(g["w"]), _ptr(g["u"]),
                             _ptr(g["state0"]), _ptr(o), _ptr(st), B, T, H, D, _binding.WKV_BF16,
                             _ptr(ws), need, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert status == 0, lib.wkv_last_error()
    torch.cuda.synchronize()
    o_ref, s_ref = run_oracle(wl)
    eo, es = errors(wl, o, st, o_ref, s_ref)
    assert eo <= 2e-3 and es <= 2e-3


def test_plain_wkv_prefill_varlen_through_ctypes():
    import linear_attention_rnn_finch_amd as fw
    from linear_attention_rnn_finch_amd import _binding
    wl = make_workload(4, lengths=[700, 0, 64, 2100, 5], H=3)
    g = to_gpu(wl)
    total, H, D = g["r"].shape
    N = len(wl.cu_seqlens) - 1
    o = torch.empty((total, H, D), dtype=torch.float32, device="cuda")
    st = torch.empty((N, H, D, D), dtype=torch.float32, device="cuda")
    cu_host = g["cu_host"].contiguous()
    need = fw.varlen_workspace_bytes(cu_host, H, D)
    ws = fw.new_workspace(need, "cuda")
    lib = _binding._lib
    status = lib.wkv_prefill_varlen(_ptr(g["r"]), _ptr(g["k"]), _ptr(g["v"]), _ptr(g["w"]),
                                    _ptr(g["u"]), _ptr(g["cu"]), ctypes.c_void_p(cu_host.data_ptr()), N,
                                    _ptr(g["state0"]), _ptr(o), _ptr(st), H, D, _binding.WKV_BF16,
                                    _ptr(ws), need,
                                    ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert status == 0, lib.wkv_last_error()
    torch.cuda.synchronize()
    o_ref, s_ref = run_oracle(wl)
    eo, es = errors(wl, o, st, o_ref, s_ref)
    assert eo <= 2e-3 and es <= 2e-3


def _bf16_host(t):
    return bf16_bits_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)


BF16_CASES = [
    ("chunked, split, with states", dict(cfg=3, B=2, T=1000, H=4)),
    ("chunked, Finch-C2 with d", dict(cfg=1, T=333, H=3, decay="log", variant="c2")),
    ("ragged", dict(cfg=4, lengths=[300, 0, 1200, 17], H=2)),
    ("fp32 inputs, serial", dict(cfg=0, T=200, H=2)),
    ("one-token steps", dict(cfg=5, B=5, T=1, H=3)),
    ("9-token steps", dict(cfg=6, B=3, T=9, H=2)),
]


@pytest.mark.parametrize("case,spec", BF16_CASES, ids=[c for c, _ in BF16_CASES])
def test_bf16_output(case, spec):
    """o in bf16 is the path's own fp32 result rounded to nearest even (bit
    for bit), hence within one bf16 ulp of the oracle plus the fp32 result's
    own error; the state stays fp32 and unchanged."""
    spec = dict(spec)
    wl = make_workload(spec.pop("cfg"), **spec)
    g = to_gpu(wl)
    log("case %s: %s tokens=%d" % (case, wl.config.name, wl.tokens))
    o32, s32 = run_gpu(wl, g)
    o16, s16 = run_gpu(wl, g, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert o16.dtype == torch.bfloat16
    assert torch.equal(o16, o32.to(torch.bfloat16))
    assert torch.equal(s16, s32)
    o_ref, _ = run_oracle(wl)
    got = _bf16_host(o16)
    g32 = o32.cpu().numpy().astype(np.float64)
    # bf16 spacing at the larger of |ref| and |g32| (g32 may sit a binade
    # above a tiny ref, and its rounding moves it by its own ulp)
    _, e = np.frexp(np.maximum(np.abs(o_ref), np.abs(g32)))
    ulp = np.ldexp(1.0, e - 8)
    bad = np.abs(got - o_ref) > ulp + np.abs(g32 - o_ref)
    log("  bf16 elements beyond one ulp (+ fp32 error): %d of %d" % (bad.sum(), bad.size))
    assert not bad.any()


def test_explicit_side_stream_with_library_workspace():
    """The kernels run on ``stream=``; the outputs and the workspace the
    binding allocates are tied to that stream, so allocations made meanwhile on
    the current stream (and written there) cannot be given the same memory
    while the call is in flight."""
    import linear_attention_rnn_finch_amd as fw
    wl = make_workload(3, B=1, T=1500, H=4)          # split into segments: workspace in use
    g = to_gpu(wl)
    o_ref, s_ref = run_gpu(wl, g)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    for rep in range(3):
        torch.cuda._sleep(2_000_000)                 # keep the side stream's kernels pending
        o, s = fw.prefill(g["r"], g["k"], g["v"], g["w"], g["u"], g["state0"], stream=side)
        # allocations on the current stream meanwhile, scribbled over
        junk = [torch.full((1 << 20,), float("nan"), device="cuda") for _ in range(8)]
        outs.append((o, s))
        del junk
    side.synchronize()
    torch.cuda.synchronize()
    for o, s in outs:
        assert torch.equal(o, o_ref) and torch.equal(s, s_ref)


def test_binding_rejects_bad_outputs_before_launch():
    """prefill_varlen and prefill check o, state_out and a given workspace
    (device, dtype, shape, contiguity) before the library is called."""
    import linear_attention_rnn_finch_amd as fw
    wl = make_workload(4, lengths=[100, 30], H=2)
    g = to_gpu(wl)
    total, H, D = g["r"].shape
    args = (g["r"], g["k"], g["v"], g["w"], g["u"], g["cu"])
    sentinel = torch.zeros(4 * total * H * D, dtype=torch.float32, device="cuda")
    bad_o = [
        sentinel[: total * H * D].view(total, H, D).to(torch.bfloat16),   # wrong dtype
        sentinel[: (total - 1) * H * D].view(total - 1, H, D),            # too short
        sentinel[: 2 * total * H * D].view(total, H, 2 * D)[:, :, :D],    # not contiguous
    ]
    for o in bad_o:
        with pytest.raises((TypeError, ValueError)):
            fw.prefill_varlen(*args, cu_seqlens_host=g["cu_host"], o=o)
    with pytest.raises(ValueError):
        fw.prefill_varlen(*args, cu_seqlens_host=g["cu_host"],
                          state_out=sentinel[: 3 * H * D * D].view(3, H, D, D))
    with pytest.raises((TypeError, ValueError)):
        fw.prefill_varlen(*args, cu_seqlens_host=g["cu_host"],
                          o=sentinel[: total * H * D].view(total, H, D), out_dtype=torch.bfloat16)
    ws_cpu = torch.zeros(1 << 20, dtype=torch.uint8)
    wb = make_workload(1, T=1000, H=2)
    gb = to_gpu(wb)
    with pytest.raises(ValueError):
        fw.prefill(gb["r"], gb["k"], gb["v"], gb["w"], gb["u"], workspace=ws_cpu)
    ws_strided = torch.zeros(1 << 21, dtype=torch.uint8, device="cuda")[::2]
    with pytest.raises(ValueError):
        fw.prefill(gb["r"], gb["k"], gb["v"], gb["w"], gb["u"], workspace=ws_strided)
    torch.cuda.synchronize()
    assert float(sentinel.abs().max()) == 0.0
