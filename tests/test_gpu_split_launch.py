"""The one-launch form of split calls (wkv_split_kernel): state pass, segment
combine and chunked scan as workgroup roles of one grid, handing segment
states to each other through the workspace's control records.  When every
(segment, head) item fits on the device at once (512 workgroups on MI355X),
one workgroup per item takes both roles in turn (the relay grid); with more
items the grid has a state workgroup and a main workgroup per item.

Every case runs both launch forms on the same inputs: one launch must equal
the three launches (state pass, segment scan, chunked scan) bit for bit, both
must match the fp64 oracle, and after each call the control records must be
ready for the next one (counters back at zero, the epoch counting the calls,
no expired wait)."""
import numpy as np
import pytest

from synth import make_workload
from gpu_util import log, to_gpu, run_gpu, run_oracle, errors

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

FORMS = [("w", "finch"), ("log", "finch"), ("w", "c2"), ("log", "c2")]
IDS = ["w", "logdecay", "c2", "c2_logdecay"]
# SplitCtl fields (16 ints per (sequence, head) record)
EPOCH, DONE, ARRIVED, SCANNED, ERROR = range(5)


def _records(ws, n):
    import linear_attention_rnn_finch_amd as fw
    assert ws.numel() >= fw.WORKSPACE_CONTROL_BYTES
    return ws[:fw.WORKSPACE_CONTROL_BYTES].view(torch.int32).view(-1, 16)[:n].cpu().numpy()


def _check_records(rec, calls):
    """Records of (sequence, head) pairs that ran `calls` one-launch calls."""
    assert (rec[:, ERROR] == 0).all(), "a bounded wait expired"
    assert (rec[:, [DONE, ARRIVED, SCANNED]] == 0).all(), rec[:4]
    assert (rec[:, EPOCH] == calls).all(), rec[:4, EPOCH]
    assert (rec[:, ERROR + 1:] == 0).all()


def _both_forms(wl, g, ws):
    import linear_attention_rnn_finch_amd as fw
    out = {}
    for launches in (3, 1):
        fw.set_split_launches(launches)
        try:
            out[launches] = run_gpu(wl, g, workspace=ws)
            torch.cuda.synchronize()
        finally:
            fw.set_split_launches(1)
    return out


def _workspace(wl):
    import linear_attention_rnn_finch_amd as fw
    B, T, H, D = (wl.r.shape if not wl.packed else (None, None) + wl.r.shape[1:])
    if wl.packed:
        need = fw.varlen_workspace_bytes(torch.from_numpy(wl.cu_seqlens.astype(np.int32)), H, D)
    else:
        need = fw.workspace_bytes(B, T, H, D)
    return fw.new_workspace(need, "cuda")


@pytest.mark.parametrize("decay,variant", FORMS, ids=IDS)
def test_one_launch_equals_three_launches(decay, variant):
    """2 x 2000 tokens x 8 heads with an initial state: segments of 256 tokens
    (8 per sequence, the last one partial), every form."""
    wl = make_workload(3, B=2, T=2000, H=8, decay=decay, variant=variant)
    g = to_gpu(wl)
    ws = _workspace(wl)
    log("case one/three launches decay=%s variant=%s" % (decay, variant))
    out = _both_forms(wl, g, ws)
    assert torch.equal(out[1][0], out[3][0]) and torch.equal(out[1][1], out[3][1])
    _check_records(_records(ws, 2 * 8), calls=1)
    o_ref, s_ref = run_oracle(wl)
    eo, es = errors(wl, out[1][0], out[1][1], o_ref, s_ref)
    assert eo <= 2e-3 and es <= 2e-3, (eo, es)


def test_layer_workload_records_and_repeats():
    """The 1.5B-class layer (T = 4096, H = 32, 16 segments of 256 tokens):
    five calls in a row on one workspace, each equal to the first and to three
    launches; the records count the calls."""
    import linear_attention_rnn_finch_amd as fw
    wl = make_workload(1)
    g = to_gpu(wl)
    ws = _workspace(wl)
    o1, s1 = run_gpu(wl, g, workspace=ws)
    for _ in range(4):
        o, s = run_gpu(wl, g, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(o, o1) and torch.equal(s, s1)
    _check_records(_records(ws, 32), calls=5)
    fw.set_split_launches(3)
    try:
        o3, s3 = run_gpu(wl, g, workspace=ws)
        torch.cuda.synchronize()
    finally:
        fw.set_split_launches(1)
    assert torch.equal(o3, o1) and torch.equal(s3, s1)
    _check_records(_records(ws, 32), calls=5)          # three launches leave the records alone


@pytest.mark.parametrize("decay,variant", [("w", "finch"), ("log", "c2")], ids=["w", "c2_logdecay"])
def test_ragged_one_launch(decay, variant):
    """Packed sequences of mixed lengths (empty, shorter than a chunk, split
    into many segments) with an initial state."""
    lengths = [1700, 0, 64, 2500, 5, 900, 3]
    wl = make_workload(4, lengths=lengths, H=6, decay=decay, variant=variant)
    g = to_gpu(wl)
    ws = _workspace(wl)
    out = _both_forms(wl, g, ws)
    assert torch.equal(out[1][0], out[3][0]) and torch.equal(out[1][1], out[3][1])
    rec = _records(ws, len(lengths) * 6).reshape(len(lengths), 6, 16)
    split = [n for n, L in enumerate(lengths) if L > 256]
    _check_records(rec[split].reshape(-1, 16), calls=1)
    assert (rec[[n for n in range(len(lengths)) if n not in split]] == 0).all()   # never split: untouched
    o_ref, s_ref = run_oracle(wl)
    eo, es = errors(wl, out[1][0], out[1][1], o_ref, s_ref)
    assert eo <= 2e-3 and es <= 2e-3, (eo, es)


def test_one_workspace_serves_calls_of_other_sizes():
    """A workspace sized for the largest call, shared by calls of other
    geometries in turn (their records overlap differently each time)."""
    import linear_attention_rnn_finch_amd as fw
    shapes = [(1, 4096, 32), (2, 1500, 8), (1, 2000, 16), (3, 700, 4), (1, 4096, 32)]
    need = max(fw.workspace_bytes(B, T, H, 64) for B, T, H in shapes)
    ws = fw.new_workspace(need, "cuda")
    for i, (B, T, H) in enumerate(shapes):
        wl = make_workload(3, B=B, T=T, H=H, decay="log" if i % 2 else "w")
        log("case shared workspace B=%d T=%d H=%d" % (B, T, H))
        g = to_gpu(wl)
        o, s = run_gpu(wl, g, workspace=ws)
        torch.cuda.synchronize()
        assert int(_records(ws, 4096)[:, ERROR].max()) == 0
        o_ref, s_ref = run_oracle(wl)
        eo, es = errors(wl, o, s, o_ref, s_ref)
        assert eo <= 2e-3 and es <= 2e-3, (B, T, H, eo, es)


@pytest.mark.parametrize("B,T,H,decay,variant", [(3, 520, 57, "w", "finch"), (4, 600, 48, "log", "c2")],
                         ids=["513_items", "576_items_c2_logdecay"])
def test_two_role_grid_when_items_exceed_the_device(B, T, H, decay, variant):
    """More (segment, head) items than the device holds at once (three
    segments of 256 tokens per sequence, 513 and 576 items) but every state
    workgroup resident: the two-role grid, with an initial state."""
    import linear_attention_rnn_finch_amd as fw
    assert fw.workspace_bytes(B, T, H, 64) > 0
    wl = make_workload(3, B=B, T=T, H=H, decay=decay, variant=variant)
    g = to_gpu(wl)
    ws = _workspace(wl)
    log("case two-role grid B=%d T=%d H=%d" % (B, T, H))
    out = _both_forms(wl, g, ws)
    assert torch.equal(out[1][0], out[3][0]) and torch.equal(out[1][1], out[3][1])
    _check_records(_records(ws, B * H), calls=1)
    o_ref, s_ref = run_oracle(wl)
    eo, es = errors(wl, out[1][0], out[1][1], o_ref, s_ref)
    assert eo <= 2e-3 and es <= 2e-3, (eo, es)


def test_more_pairs_than_records_take_three_launches():
    """4128 (sequence, head) pairs (129 sequences x 32 heads), one of them
    split: more pairs than the control records hold, so the call takes the
    three launches and leaves the records untouched; 128 sequences (4096
    pairs) take the one launch."""
    import linear_attention_rnn_finch_amd as fw
    for n_short, one in ((128, False), (127, True)):
        lengths = [3000] + [20] * n_short
        wl = make_workload(4, lengths=lengths, H=32)
        g = to_gpu(wl)
        ws = _workspace(wl)
        o, s = run_gpu(wl, g, workspace=ws)
        torch.cuda.synchronize()
        rec = _records(ws, fw.WORKSPACE_CONTROL_BYTES // 64)
        if one:
            _check_records(rec[:32], calls=1)               # sequence 0, all heads
        else:
            assert (rec == 0).all()
        o_ref, s_ref = run_oracle(wl)
        eo, es = errors(wl, o, s, o_ref, s_ref)
        assert eo <= 2e-3 and es <= 2e-3, (n_short, eo, es)


def test_random_shapes():
    """Seeded random fixed and ragged calls in every form (segments of 256
    tokens, 2 to 12 per sequence, 1 to 16 heads, with and without states):
    one launch equals three launches bit for bit, matches the oracle, and
    leaves every record of a split sequence ready for the next call."""
    rng = np.random.default_rng(20261203)
    for case in range(28):
        decay, variant = FORMS[case % 4]
        H = int(rng.integers(1, 17))
        cfg = 3 if case % 3 else 1                          # with an initial state, or without
        if case % 2:
            lengths = [int(x) for x in rng.integers(0, 3000, size=int(rng.integers(2, 6)))]
            wl = make_workload(4, lengths=lengths, H=H, decay=decay, variant=variant)
        else:
            B, T = int(rng.integers(1, 4)), int(rng.integers(300, 3000))
            lengths = [T] * B
            wl = make_workload(cfg, B=B, T=T, H=H, decay=decay, variant=variant)
        log("case random %d lengths=%s H=%d decay=%s variant=%s" % (case, lengths, H, decay, variant))
        g = to_gpu(wl)
        ws = _workspace(wl)
        out = _both_forms(wl, g, ws)
        assert torch.equal(out[1][0], out[3][0]) and torch.equal(out[1][1], out[3][1]), case
        rec = _records(ws, len(lengths) * H).reshape(len(lengths), H, 16)
        split = [n for n, L in enumerate(lengths) if L > 256]
        if split:
            _check_records(rec[split].reshape(-1, 16), calls=1)
        o_ref, s_ref = run_oracle(wl)
        eo, es = errors(wl, out[1][0], out[1][1], o_ref, s_ref)
        assert eo <= 2e-3 and es <= 2e-3, (case, eo, es)


def test_workspace_errors_query():
    """wkv_workspace_errors: no marks after one-launch calls; a mark planted
    from the host (what an expired wait leaves; the kernels only ever write
    that word) is counted, cleared on request, and the workspace then gives
    the same results as before."""
    import linear_attention_rnn_finch_amd as fw
    wl = make_workload(3, B=2, T=2000, H=8)
    g = to_gpu(wl)
    ws = _workspace(wl)
    log("case workspace_errors query")
    o1, s1 = run_gpu(wl, g, workspace=ws)
    assert fw.workspace_errors(ws) == 0
    recs = ws[:fw.WORKSPACE_CONTROL_BYTES].view(torch.int32).view(-1, 16)
    recs[3, ERROR] = 1
    recs[9, ERROR] = 7
    recs[9, ARRIVED] = 5                  # counters out of step, as an expired wait can leave them
    assert fw.workspace_errors(ws) == 2
    assert fw.workspace_errors(ws, clear=True) == 2
    assert fw.workspace_errors(ws) == 0
    rec = _records(ws, 2 * 8)
    assert (rec[[3, 9]] == 0).all()      # marked records zeroed whole
    _check_records(np.delete(rec, [3, 9], axis=0), calls=1)
    o2, s2 = run_gpu(wl, g, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    assert fw.workspace_errors(ws) == 0
    rec = _records(ws, 2 * 8)
    _check_records(rec[[3, 9]], calls=1)
    _check_records(np.delete(rec, [3, 9], axis=0), calls=2)
    # a call that needs no workspace has no records to read
    assert fw.workspace_errors(torch.empty(0, dtype=torch.uint8, device="cuda")) == 0


def test_expired_waits_are_reported_and_the_workspace_recovers():
    """The error path, forced from the host: with a wait bound of one tick
    (10 ns) the one launch's waits expire, the launch still ends, the
    records are marked; after clearing them the same workspace gives the
    results of a normal call again, bit for bit."""
    import linear_attention_rnn_finch_amd as fw
    wl = make_workload(3, B=2, T=2000, H=8)
    g = to_gpu(wl)
    ws = _workspace(wl)
    log("case expired waits")
    o1, s1 = run_gpu(wl, g, workspace=ws)
    torch.cuda.synchronize()
    assert fw.workspace_errors(ws) == 0
    fw.set_wait_bound(1)
    try:
        run_gpu(wl, g, workspace=ws)
        torch.cuda.synchronize()
    finally:
        fw.set_wait_bound(0)
    marked = fw.workspace_errors(ws, clear=True)
    assert 0 < marked <= 2 * 8, marked
    assert fw.workspace_errors(ws) == 0
    for _ in range(2):
        o2, s2 = run_gpu(wl, g, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(s1, s2)
    assert fw.workspace_errors(ws) == 0
