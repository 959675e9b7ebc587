"""Longest-first order of a packed call's chunked scan: when there are more
(segment, head) work items than the 512 the device holds at once, the
planner ranks the segments (every full-length segment first, in index order,
then each sequence's last segment by length, longest first, ties by
sequence) and the chunked scan takes its items in that order.  The table is
read back from the workspace and checked against the order computed here
from the host offsets; the call is checked against the oracle."""
import numpy as np
import pytest

from synth import make_workload
from gpu_util import log, to_gpu, run_gpu, run_oracle, errors

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _up(x, m):
    return -(-x // m) * m


def _plan(lengths, H):
    """Segment length, segments per sequence and the workspace offset of the
    rank table, as the library's host plan lays them out (split packed
    call: control records, run aggregates, start states, segment offsets,
    owners, ranks; each array 256-byte aligned)."""
    tokens, max_len = sum(lengths), max(lengths)
    seg = min(max(_up(max(-(-tokens * H // 512), 1), 64), 256), _up(max(max_len, 1), 64))
    P = [1 if L == 0 else -(-L // seg) for L in lengths]
    n_seg, N = sum(P), len(lengths)
    # state runs per segment: enough for about 768 state items, at least 4 chunks each
    runs, items = 1, (n_seg - N) * H
    r = min(768 // items, seg // 256) if items else 1
    if r > 1:
        run_len = _up(-(-seg // r), 64)
        runs = -(-seg // run_len)
    off = 262144
    off += _up((n_seg - N) * runs * H * (64 * 64 + 64) * 4, 256)
    off += _up(n_seg * H * 64 * 64 * 4, 256)
    off += _up((N + 1) * 4, 256)
    off += _up(n_seg * 4, 256)
    return seg, P, off


def _check_order(lengths, H, whole):
    import linear_attention_rnn_finch_amd as fw
    wl = make_workload(4, lengths=lengths, H=H)
    g = to_gpu(wl)
    need = fw.varlen_workspace_bytes(g["cu_host"], H, 64)
    if whole:                                   # one segment per sequence, no aggregates
        seg, P = _up(max(lengths), 64), [1] * len(lengths)
        rank_off = 262144 + _up((len(lengths) + 1) * 4, 256) + _up(len(lengths) * 4, 256)
    else:
        seg, P, rank_off = _plan(lengths, H)
        assert seg > 1024                       # three launches
    assert sum(P) * H > (256 if whole else 512)  # more items than the device holds at once
    assert need >= rank_off + 4 * sum(P)
    ws = fw.new_workspace(need, "cuda")
    log("case longest-first lengths=%s H=%d whole=%s" % (lengths, H, whole))
    o, s = run_gpu(wl, g, workspace=ws)
    torch.cuda.synchronize()
    table = ws[rank_off:rank_off + 4 * sum(P)].view(torch.int32).cpu().numpy()
    first = np.concatenate([[0], np.cumsum(P)])
    full = [int(first[n]) + p for n in range(len(lengths)) for p in range(P[n] - 1)]
    last_len = [L - (P[n] - 1) * seg for n, L in enumerate(lengths)]
    order = sorted(range(len(lengths)), key=lambda n: (-last_len[n], n))
    expect = full + [int(first[n + 1]) - 1 for n in order]
    assert table.tolist() == expect
    o_ref, s_ref = run_oracle(wl)
    eo, es = errors(wl, o, s, o_ref, s_ref)
    assert eo <= 2e-3 and es <= 2e-3, (eo, es)


def test_split_segments_longest_first():
    """192 (sequence, head) pairs: split into segments of 3968 tokens, 672
    items for the 4-wave kernel."""
    _check_order([30000, 500, 20000, 100, 9000, 4000], 32, whole=False)


def test_whole_sequences_longest_first():
    """512 pairs, no sequence longer than twice the mean work per CU: whole
    sequences on the producer/consumer kernel, longest first."""
    _check_order([3000, 100, 2500, 40, 900, 1800, 7, 1200], 64, whole=True)
