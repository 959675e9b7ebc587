"""The producer/consumer kernel that runs whole sequences: bf16 calls with at
least 256 (sequence, head) pairs whose sequences the 4-wave kernel would
split into segments (packed calls also need no sequence longer than twice
the mean work per CU).  Every form against the fp64 oracle (all heads), with
and without states, a partial last chunk, bf16 o, stiff decays, carried
chains, graph replays and packed batches with empty and short sequences; the
8 x 4096 x 32 training batch and the 16 ragged sequences run it too
(tests/test_gpu_parity.py)."""
from dataclasses import replace

import numpy as np
import pytest

from synth import make_workload, get_config, f32_to_bf16_bits, bf16_bits_to_f32
from gpu_util import log, to_gpu, run_gpu, run_oracle, errors, gpu_block_error

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

FORMS = [("w", "finch"), ("log", "finch"), ("w", "c2"), ("log", "c2")]
IDS = ["w", "logdecay", "c2", "c2_logdecay"]


def _assert_whole_sequence_plan(B, T, H):
    """These shapes take the whole-sequence kernel: no workspace, although a
    smaller batch of the same sequences is split (and needs one)."""
    import linear_attention_rnn_finch_amd as fw
    assert B * H >= 256 and T > 256
    assert fw.workspace_bytes(B, T, H, 64) == 0
    assert fw.workspace_bytes(1, T, 1, 64) > 0


def _check(wl, g=None, **kw):
    tol = wl.config.tolerance
    log("case %s decay=%s variant=%s B=%d H=%d T=%d state=%s" % (
        wl.config.name, wl.decay, wl.variant, wl.n_seq, wl.u.shape[0], wl.tokens // wl.n_seq,
        wl.state0 is not None))
    o, s = run_gpu(wl, g, **kw)
    torch.cuda.synchronize()
    o_ref, s_ref = run_oracle(wl)
    err = errors(wl, o, s, o_ref, s_ref)
    eo, es = err
    assert np.isfinite(eo) and np.isfinite(es)
    assert eo <= tol and es <= tol, (eo, es)
    assert err.row_o <= tol and err.row_s <= tol, (err.row_o, err.row_s)
    return o, s


@pytest.mark.parametrize("decay,variant", FORMS, ids=IDS)
@pytest.mark.parametrize("with_state", [False, True], ids=["zero_state", "state"])
def test_every_form(decay, variant, with_state):
    """2 x 1000 tokens x 128 heads: a partial last chunk (1000 = 15 x 64 + 40)."""
    B, T, H = 2, 1000, 128
    _assert_whole_sequence_plan(B, T, H)
    cfg = 3 if with_state else 1
    _check(make_workload(cfg, B=B, T=T, H=H, decay=decay, variant=variant))


@pytest.mark.parametrize("decay,variant", FORMS, ids=IDS)
def test_bf16_output(decay, variant):
    """o in bf16 is the fp32 result rounded to nearest even, bit for bit."""
    B, T, H = 4, 333, 64
    _assert_whole_sequence_plan(B, T, H)
    wl = make_workload(3, B=B, T=T, H=H, decay=decay, variant=variant)
    g = to_gpu(wl)
    o32, s32 = run_gpu(wl, g)
    o16, s16 = run_gpu(wl, g, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o16, o32.to(torch.bfloat16))
    assert torch.equal(s16, s32)
    o_ref, _ = run_oracle(wl)
    got = bf16_bits_to_f32(o16.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    g32 = o32.cpu().numpy().astype(np.float64)
    # rounding g32 moves it by at most one bf16 ulp at its own magnitude; take
    # the larger of the two magnitudes (g32 may sit a binade above a tiny ref)
    _, e = np.frexp(np.maximum(np.abs(o_ref), np.abs(g32)))
    assert not (np.abs(got - o_ref) > np.ldexp(1.0, e - 8) + np.abs(g32 - o_ref)).any()


@pytest.mark.parametrize("decay,variant", FORMS, ids=IDS)
def test_stiff_decays(decay, variant):
    """Decays spanning many orders of magnitude inside one chunk (exact
    token-serial path of the consumers), one head without any decay."""
    B, T, H = 2, 300, 128
    _assert_whole_sequence_plan(B, T, H)
    wl = make_workload(replace(get_config(1), state_sigma=0.1), B=B, T=T, H=H, decay=decay,
                       variant=variant)
    bits = lambda x: f32_to_bf16_bits(np.float32(x)).item()
    w = wl.w
    if decay == "log":
        w[:, 100:181, 1, 5] = bits(4.0)
        w[:, 100:160, 2, 63] = bits(2.5)
        w[:, T - 20:T - 10, H - 1, 0] = 0x7F80
        w[:, :, 0, 17:30] = 0xFF80
    else:
        w[:, 100:181, 1, 5] = bits(1e-3)
        w[:, 100:160, 2, 63] = bits(1e-30)
        w[:, T - 20:T - 10, H - 1, 0] = 0x0001
        w[:, :, 0, 17:30] = bits(1.0)
    _check(wl)


def test_carried_chain_equals_single_call():
    """The same 2 x 1000-token batch as three carried calls (each of them a
    whole-sequence call) against the single call and the oracle."""
    import linear_attention_rnn_finch_amd as fw
    B, T, H = 2, 1000, 128
    wl = make_workload(3, B=B, T=T, H=H, decay="log", variant="c2")
    g = to_gpu(wl)
    o_full, s_full = _check(wl, g=g)
    cuts = [0, 333, 700, T]
    state = g["state0"].clone()
    o_chain = torch.empty_like(o_full)
    part = lambda x, a, z: x[:, a:z].contiguous()       # B > 1: time slices are strided views
    for a, z in zip(cuts[:-1], cuts[1:]):
        _assert_whole_sequence_plan(B, z - a, H)
        o_part, _ = fw.prefill(part(g["r"], a, z), part(g["k"], a, z), part(g["v"], a, z),
                               part(g["w"], a, z), None, state, state_out=state, decay="log",
                               variant="c2", second_value=part(g["u2"], a, z))
        o_chain[:, a:z] = o_part
    torch.cuda.synchronize()
    e_o = gpu_block_error(o_chain, o_full, (1, 3))
    e_s = gpu_block_error(state, s_full, (2, 3))
    log("  chain vs single call: o=%.3e state=%.3e" % (e_o, e_s))
    assert e_o <= 2e-3 and e_s <= 2e-3
    o_ref, s_ref = run_oracle(wl)
    eo, es = errors(wl, o_chain, state, o_ref, s_ref)
    assert eo <= 2e-3 and es <= 2e-3


def test_no_state_out_and_deterministic():
    """Without state_out the call still writes o (the last chunk then skips
    the state update); two runs agree bit for bit."""
    import linear_attention_rnn_finch_amd as fw
    B, T, H = 2, 700, 128
    wl = make_workload(3, B=B, T=T, H=H)
    g = to_gpu(wl)
    o1, s1 = run_gpu(wl, g)
    o2, _ = fw.prefill(g["r"], g["k"], g["v"], g["w"], g["u"], g["state0"], want_state=False)
    o3, s3 = run_gpu(wl, g)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(o1, o3) and torch.equal(s1, s3)


def test_graph_replays_match_eager():
    import linear_attention_rnn_finch_amd as fw
    B, T, H = 2, 1000, 128
    wl = make_workload(3, B=B, T=T, H=H)
    g = to_gpu(wl)
    o_ref, s_ref = run_gpu(wl, g)
    torch.cuda.synchronize()
    o = torch.full_like(o_ref, float("nan"))
    st = torch.full_like(s_ref, float("nan"))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            fw.prefill(g["r"], g["k"], g["v"], g["w"], g["u"], g["state0"], o=o, state_out=st)
    torch.cuda.synchronize()
    for rep in range(3):
        o.fill_(float("nan"))
        st.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(st, s_ref), rep


@pytest.mark.parametrize("decay,variant", FORMS, ids=IDS)
def test_packed_whole_sequences(decay, variant):
    """A packed batch of 8 sequences x 64 heads (512 pairs) with an initial
    state, lengths 0 to 1000 (empty, shorter than a step call, exactly one
    chunk, partial chunks): whole sequences on the producer/consumer kernel,
    longest first, no workspace beyond the planner's tables."""
    import linear_attention_rnn_finch_amd as fw
    lengths = [1000, 0, 5, 700, 64, 300, 16, 900]
    H = 64
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    assert fw.varlen_workspace_bytes(torch.from_numpy(cu), H, 64) == 262144 + 3 * 256
    _check(make_workload(4, lengths=lengths, H=H, decay=decay, variant=variant))
