"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Tolerances are the normwise per-(sequence, head) block errors of the
specification: 2e-3 for bf16 inputs (fp32 state and accumulation), 1e-5 for
fp32 inputs.  Reduced sizes keep the oracle at a few seconds while spanning
several chunks and a ragged tail; full-size workloads compare every slice the
oracle can afford and sample the rest.
"""
import numpy as np
import pytest

from dataclasses import replace

from synth import make_workload, get_config, f32_to_bf16_bits
from gpu_util import log, to_gpu, run_gpu, run_oracle, errors, gpu_block_error

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _check(wl, heads=None, tol=None, g=None, **kw):
    tol = tol if tol is not None else wl.config.tolerance
    log("case %s B=%d H=%d tokens=%d heads=%s" % (wl.config.name, wl.n_seq, wl.u.shape[0],
                                                 wl.tokens, heads))
    o, s = run_gpu(wl, g, **kw)
    torch.cuda.synchronize()
    o_ref, s_ref = run_oracle(wl, heads)
    err = errors(wl, o, s, o_ref, s_ref, heads)
    eo, es = err
    log("  err o=%.3e state=%.3e (tol %.0e)" % (eo, es, tol))
    assert np.isfinite(eo) and np.isfinite(es)
    assert eo <= tol and es <= tol, (eo, es)
    # per-row errors (floored denominators) within the same bound: an error
    # confined to a few rows of a long block cannot hide behind its maximum
    assert err.row_o <= tol and err.row_s <= tol, (err.row_o, err.row_s)
    return o, s


def test_tiny_f32_config():
    _check(make_workload(0))


@pytest.mark.parametrize("T", [1, 2, 63, 64, 65, 200, 1000])
def test_bf16_short_sequences(T):
    _check(make_workload(1, T=T, H=4))


def test_bf16_with_initial_state_and_batch():
    wl = make_workload(3, B=3, T=777, H=5)          # long-context distributions, random S_0
    _check(wl)


def test_f32_ragged_and_state():
    wl = make_workload(0, lengths=[70, 1, 0, 130], H=2)
    wl.state0 = np.random.default_rng(3).normal(0, 0.1, size=(4, 2, 64, 64)).astype(np.float32)
    _check(wl)


def test_layer_shape_full_size():
    """T=4096, H=32 (d_model 2048): every slice against the oracle."""
    _check(make_workload(1))


def test_ragged_reduced():
    wl = make_workload(4, lengths=[1024, 3, 0, 2500, 64, 4097], H=4)
    _check(wl)


def test_zero_length_passes_state_through():
    wl = make_workload(3, B=2, T=0, H=3)
    g = to_gpu(wl)
    o, s = run_gpu(wl, g)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(s.cpu().numpy(), wl.state0)
    wl2 = make_workload(1, B=2, T=0, H=3)
    o2, s2 = run_gpu(wl2)
    torch.cuda.synchronize()
    assert float(s2.abs().max()) == 0.0


def test_state_in_aliases_state_out():
    wl = make_workload(3, B=2, T=300, H=3)
    g = to_gpu(wl)
    o_ref, s_ref = run_gpu(wl, g)
    carried = g["state0"].clone()
    o2, s2 = run_gpu(wl, g, state_in=carried, state_out=carried)
    torch.cuda.synchronize()
    assert s2.data_ptr() == carried.data_ptr()
    assert torch.equal(o2, o_ref) and torch.equal(carried, s_ref)


def test_carried_state_chain_equals_single_pass():
    wl = make_workload(1, T=1000, H=4)
    g = to_gpu(wl)
    o_full, s_full = run_gpu(wl, g)
    cuts = [0, 1, 130, 512, 1000]
    state = None
    outs = []
    import linear_attention_rnn_finch_amd as fw
    for a, z in zip(cuts[:-1], cuts[1:]):
        o, state = fw.prefill(g["r"][:, a:z].contiguous(), g["k"][:, a:z].contiguous(),
                              g["v"][:, a:z].contiguous(), g["w"][:, a:z].contiguous(),
                              g["u"], state)
        outs.append(o)
    torch.cuda.synchronize()
    o_chain = torch.cat(outs, dim=1)
    o_ref, s_ref = run_oracle(wl)
    eo, es = errors(wl, o_chain, state, o_ref, s_ref)
    assert eo <= 2e-3 and es <= 2e-3
    eo2, es2 = errors(wl, o_chain, state, o_full.cpu().numpy().astype(np.float64),
                      s_full.cpu().numpy().astype(np.float64))
    assert eo2 <= 2e-3 and es2 <= 2e-3


def test_deterministic():
    wl = make_workload(1, T=700, H=8)
    g = to_gpu(wl)
    o1, s1 = run_gpu(wl, g)
    o2, s2 = run_gpu(wl, g)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_guard_bands_untouched():
    wl = make_workload(1, T=130, H=2)
    g = to_gpu(wl)
    B, T, H, D = 1, 130, 2, 64
    pad = 4096
    o_buf = torch.full((pad + B * T * H * D + pad,), 12345.0, device="cuda")
    s_buf = torch.full((pad + B * H * D * D + pad,), -777.0, device="cuda")
    o = o_buf[pad:pad + B * T * H * D].view(B, T, H, D)
    s = s_buf[pad:pad + B * H * D * D].view(B, H, D, D)
    run_gpu(wl, g, o=o, state_out=s)
    torch.cuda.synchronize()
    assert torch.all(o_buf[:pad] == 12345.0) and torch.all(o_buf[-pad:] == 12345.0)
    assert torch.all(s_buf[:pad] == -777.0) and torch.all(s_buf[-pad:] == -777.0)
    o_ref, s_ref = run_oracle(wl)
    eo, es = errors(wl, o, s, o_ref, s_ref)
    assert eo <= 2e-3 and es <= 2e-3


def test_validation_errors_raise():
    """An output overlapping another buffer is rejected before any launch."""
    import linear_attention_rnn_finch_amd as fw
    wl = make_workload(1, T=64, H=2)
    g = to_gpu(wl)
    B, T, H, D = g["r"].shape
    big = torch.zeros(B * T * H * D, dtype=torch.float32, device="cuda")
    o = big.view(B, T, H, D)
    st = big[: B * H * D * D].view(B, H, D, D)       # state_out inside o
    with pytest.raises(fw.WkvError) as ei:
        fw.prefill(g["r"], g["k"], g["v"], g["w"], g["u"], None, o=o, state_out=st)
    assert ei.value.status == 1
    torch.cuda.synchronize()
    assert float(big.abs().max()) == 0.0              # nothing was written


def test_graph_replays_match_eager():
    """The benchmark replays captured calls: every replay must equal the eager
    result, with eager work and synchronisations between replays."""
    import linear_attention_rnn_finch_amd as fw
    wl = make_workload(3, B=1, T=1500, H=4)          # split into segments, with S_0
    g = to_gpu(wl)
    B, T, H, D = g["r"].shape
    o = torch.empty((B, T, H, D), dtype=torch.float32, device="cuda")
    st = torch.empty((B, H, D, D), dtype=torch.float32, device="cuda")
    ws = fw.new_workspace(fw.workspace_bytes(B, T, H, D), "cuda")
    o_ref, s_ref = run_gpu(wl, g)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        fw.prefill(g["r"], g["k"], g["v"], g["w"], g["u"], g["state0"], o=o, state_out=st, workspace=ws)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=cap):
            fw.prefill(g["r"], g["k"], g["v"], g["w"], g["u"], g["state0"], o=o, state_out=st,
                       workspace=ws)
    torch.cuda.synchronize()
    for rep in range(4):
        o.fill_(float("nan"))
        st.fill_(float("nan"))
        ws[fw.WORKSPACE_CONTROL_BYTES:].fill_(0xAB)      # scratch; the control records are kept
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), rep
        assert torch.equal(st, s_ref), rep


def test_train_batch_full_size():
    """B=8, T=4096, H=32: every one of the 256 slices against the oracle."""
    _check(make_workload(2))


def _check_head_batches(wl, results, batch=8):
    """Every head of a large workload against the oracle, ``batch`` heads at a
    time (the oracle's fp64 outputs of all heads together would not fit the
    host comfortably).  ``results`` maps a label to GPU (o, state_out)."""
    tol = wl.config.tolerance
    H = wl.u.shape[0]
    worst = {label: [0.0, 0.0, 0.0, 0.0] for label in results}
    for h0 in range(0, H, batch):
        heads = list(range(h0, min(H, h0 + batch)))
        o_ref, s_ref = run_oracle(wl, heads)
        for label, (o, s) in results.items():
            log("  %s heads %d..%d" % (label, heads[0], heads[-1]))
            err = errors(wl, o, s, o_ref, s_ref, heads)
            eo, es = err
            worst[label] = [max(a, b) for a, b in zip(worst[label], (eo, es, err.row_o, err.row_s))]
            assert np.isfinite(eo) and np.isfinite(es)
            assert eo <= tol and es <= tol, (label, heads, eo, es)
            assert err.row_o <= tol and err.row_s <= tol, (label, heads, err.row_o, err.row_s)
        del o_ref, s_ref
    for label, (eo, es, ro, rs) in worst.items():
        log("  %s, all %d heads: block o=%.3e state=%.3e row o=%.3e state=%.3e"
            % (label, H, eo, es, ro, rs))


@pytest.mark.timeout(1200)
def test_long_context_full_size_and_8_segment_chain():
    """T=262144, H=64 with random fp32 initial states: every head against the
    oracle (in batches of heads), and the same sequence run as 8 consecutive
    carried-state calls against both the oracle and the single call."""
    import linear_attention_rnn_finch_amd as fw
    wl = make_workload(3)
    g = to_gpu(wl)
    log("case %s single call" % wl.config.name)
    o_full, s_full = run_gpu(wl, g)
    B, T, H, D = g["r"].shape
    o_chain = torch.empty_like(o_full)
    state = g["state0"].clone()
    seg = T // 8
    for p in range(8):
        a, z = p * seg, (p + 1) * seg
        log("  chain segment %d tokens %d..%d" % (p, a, z))
        fw.prefill(g["r"][:, a:z], g["k"][:, a:z], g["v"][:, a:z], g["w"][:, a:z], g["u"],
                   state, o=o_chain[:, a:z], state_out=state)
    torch.cuda.synchronize()
    tol = wl.config.tolerance
    e_o = gpu_block_error(o_chain, o_full, (1, 3))
    e_s = gpu_block_error(state, s_full, (2, 3))
    log("  chain vs single call: o=%.3e state=%.3e" % (e_o, e_s))
    assert e_o <= tol and e_s <= tol
    del g
    _check_head_batches(wl, {"single call": (o_full, s_full), "8-call chain": (o_chain, state)})


@pytest.mark.timeout(900)
def test_ragged_full_size():
    """16 packed sequences of U{1024..32768} tokens, own initial states: every
    sequence and every head against the oracle (in batches of heads)."""
    wl = make_workload(4)
    log("case %s tokens=%d" % (wl.config.name, wl.tokens))
    o, s = run_gpu(wl)
    torch.cuda.synchronize()
    _check_head_batches(wl, {"packed call": (o, s)})


def _stiff_workload(T, H):
    """Decays that vary by many orders of magnitude inside one chunk: a channel
    at w = 1e-3 over 80 tokens, one at 1e-30, one at the smallest subnormal
    bf16, and one head with no decay at all (w = 1 exactly)."""
    wl = make_workload(replace(get_config(1), state_sigma=0.1), T=T, H=H)
    w = wl.w
    bits = lambda x: f32_to_bf16_bits(np.float32(x)).item()
    w[:, 100 % T:180 % T + 1, 1 % H, 5] = bits(1e-3)
    w[:, (T // 3):(T // 3) + 60, 2 % H, 63] = bits(1e-30)
    w[:, T - 20:T - 10, (H - 1), 0] = 0x0001
    w[:, :, 0, 17:30] = bits(1.0)
    return wl


@pytest.mark.parametrize("T,H", [(300, 1), (2000, 4)])
def test_stiff_decays(T, H):
    """Chunks whose decay exceeds the rescaling range take the exact token-serial
    path; with H=4, T=2000 the sequence is also split into segments."""
    _check(_stiff_workload(T, H))


def test_f32_long_sequence():
    wl = make_workload(0, T=3000, H=3, B=2)
    _check(wl)


@pytest.mark.timeout(600)
def test_maximum_head_count():
    """H = 65536, the largest the library accepts (64 rows x H x 256 B per
    chunk must fit 32-bit offsets): T = 65 (a full chunk and a ragged one),
    random states; sampled heads, including the last, against the oracle."""
    wl = make_workload(3, T=65, H=65536)
    heads = [0, 1, 4097, 32768, 65534, 65535]
    _check(wl, heads=heads)
