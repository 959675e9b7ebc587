"""Split fixed-length bf16 calls on the producer/consumer kernel: fewer than
256 (sequence, head) pairs whose sequences, cut into about 256 segments, give
segments of at least 2048 tokens.  The state pass (in runs) and the segment
scan hand each segment its start state; the producer/consumer kernel runs the
chunked scan of every segment from it, and only a sequence's last segment
writes state_out.  Every form against the fp64 oracle (all heads), with and
without an initial state, partial last segments and chunks, many segments per
sequence, bf16 o, repeated calls, the three-launch switch (which these plans
ignore) and graph replays; the 262,144-token long-context call runs it too
(tests/test_gpu_parity.py)."""
import numpy as np
import pytest

from synth import make_workload
from gpu_util import log, to_gpu, run_gpu, run_oracle, errors

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

FORMS = [("w", "finch"), ("log", "finch"), ("w", "c2"), ("log", "c2")]
IDS = ["w", "logdecay", "c2", "c2_logdecay"]
CTL, AGG, START = 262144, 16640, 16384


def _up(x, m):
    return -(-x // m) * m


def _pc_split_plan(B, T, H):
    """Segment length and segments per sequence of the producer/consumer
    split, checked against the library's workspace size (control records,
    run aggregates of every segment but the last, start states)."""
    import linear_attention_rnn_finch_amd as fw
    assert B * H < 256
    pcs = max(2, 256 // (B * H))
    seg = _up(-(-T // pcs), 64)
    assert seg >= 2048
    per = -(-T // seg)
    items = B * (per - 1) * H
    r = min(768 // items, seg // 256)
    runs = -(-seg // _up(-(-seg // r), 64)) if r > 1 else 1
    assert fw.workspace_bytes(B, T, H, 64) == (
        CTL + _up(items * runs * AGG, 256) + _up(B * per * H * START, 256))
    return seg, per


def _check(wl, g=None, **kw):
    tol = wl.config.tolerance
    H = wl.u.shape[0]
    B, T = wl.n_seq, wl.tokens // wl.n_seq
    seg, per = _pc_split_plan(B, T, H)
    log("case pc split decay=%s variant=%s B=%d T=%d H=%d seg=%d x %d state=%s" % (
        wl.decay, wl.variant, B, T, H, seg, per, wl.state0 is not None))
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
    """2 x 9000 tokens x 32 heads: four segments of 2304 tokens per sequence,
    the last one 2088 tokens (32 chunks and 40 tokens)."""
    wl = make_workload(3 if with_state else 1, B=2, T=9000, H=32, decay=decay, variant=variant)
    _check(wl)


def test_many_segments_per_sequence():
    """1 x 70,001 tokens x 8 heads: 32 segments of 2240 tokens, the last one
    561 tokens, from an initial state."""
    wl = make_workload(3, B=1, T=70001, H=8, decay="log")
    assert _pc_split_plan(1, 70001, 8) == (2240, 32)
    _check(wl)


def test_two_segments_at_128_pairs():
    """4 x 4100 tokens x 32 heads (128 pairs): two segments of 2112 tokens
    per sequence, the last one 1988 tokens."""
    assert _pc_split_plan(4, 4100, 32) == (2112, 2)
    _check(make_workload(3, B=4, T=4100, H=32, variant="c2"))


def test_bf16_output_and_repeats():
    """o in bf16 is the fp32 result rounded to nearest even, bit for bit;
    calls repeated on one workspace, and with the three-launch switch set,
    give the same bits."""
    import linear_attention_rnn_finch_amd as fw
    wl = make_workload(3, B=2, T=8200, H=32)
    _pc_split_plan(2, 8200, 32)
    g = to_gpu(wl)
    ws = fw.new_workspace(fw.workspace_bytes(2, 8200, 32, 64), "cuda")
    o32, s32 = run_gpu(wl, g, workspace=ws)
    o16, s16 = run_gpu(wl, g, workspace=ws, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o16, o32.to(torch.bfloat16)) and torch.equal(s16, s32)
    for _ in range(3):
        o, s = run_gpu(wl, g, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(o, o32) and torch.equal(s, s32)
    fw.set_split_launches(3)
    try:
        o3, s3 = run_gpu(wl, g, workspace=ws)
        torch.cuda.synchronize()
    finally:
        fw.set_split_launches(1)
    assert torch.equal(o3, o32) and torch.equal(s3, s32)
    o_ref, s_ref = run_oracle(wl)
    eo, es = errors(wl, o32, s32, o_ref, s_ref)
    assert eo <= 2e-3 and es <= 2e-3, (eo, es)


def test_state_in_aliases_state_out():
    """state_out may be state_in: every segment's start state comes from the
    state pass and scan, which read state_in before any segment writes."""
    wl = make_workload(3, B=2, T=9000, H=32, decay="log", variant="c2")
    g = to_gpu(wl)
    o_ref, s_ref = run_oracle(wl)
    s = g["state0"].clone()
    o_sep, s_sep = run_gpu(wl, g)
    o, s_out = run_gpu(wl, g, state_in=s, state_out=s)
    torch.cuda.synchronize()
    assert s_out.data_ptr() == s.data_ptr()
    assert torch.equal(o, o_sep) and torch.equal(s, s_sep)
    eo, es = errors(wl, o, s, o_ref, s_ref)
    assert eo <= 2e-3 and es <= 2e-3, (eo, es)


def test_graph_replays_match_eager():
    """A captured call replayed four times, with the outputs and the
    workspace's scratch part overwritten and an eager call between the
    replays, equals the eager call each time."""
    import linear_attention_rnn_finch_amd as fw
    wl = make_workload(3, B=2, T=9000, H=32)
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
        o_e, s_e = run_gpu(wl, g)
        torch.cuda.synchronize()
        assert torch.equal(o_e, o_ref) and torch.equal(s_e, s_ref), rep
