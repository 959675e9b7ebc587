"""C-ABI checks that need no GPU: the library loads, exports every function the
public header declares, and rejects bad arguments before any HIP call.

Fake device addresses are plain integers here; every call below fails
validation, so nothing is ever dereferenced or launched.
"""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "finch_wkv.h")
LIB = os.path.join(ROOT, "linear_attention_rnn_finch_amd", "libfinch_wkv.so")

OK, EINVAL, EUNSUP, EWS, EHIP = range(5)
F32, BF16 = 0, 1


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(wkv_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.skip("library not built")
    L = ctypes.CDLL(LIB)
    vp, sz, i = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    L.wkv_prefill.restype = i
    L.wkv_prefill.argtypes = [vp] * 8 + [i] * 5 + [vp, sz, vp]
    L.wkv_prefill_varlen.restype = i
    L.wkv_prefill_varlen.argtypes = [vp] * 7 + [i, vp, vp, vp, i, i, i, vp, sz, vp]
    L.wkv_prefill_workspace_bytes.restype = sz
    L.wkv_prefill_workspace_bytes.argtypes = [i] * 5
    L.wkv_prefill_varlen_workspace_bytes.restype = sz
    L.wkv_prefill_varlen_workspace_bytes.argtypes = [vp, i, i, i, i]
    L.wkv_layernorm_heads.restype = i
    L.wkv_layernorm_heads.argtypes = [vp, vp, vp, ctypes.c_float, vp, i, ctypes.c_int64, i, vp]
    L.wkv_gold_compress.restype = i
    L.wkv_gold_compress.argtypes = [vp, vp, vp, i, ctypes.c_int64, i, vp]
    L.wkv_prefill_ex.restype = i
    L.wkv_prefill_ex.argtypes = [vp] * 9 + [i] * 5 + [ctypes.c_uint, vp, sz, vp]
    L.wkv_prefill_varlen_ex.restype = i
    L.wkv_prefill_varlen_ex.argtypes = [vp] * 8 + [i, vp, vp, vp, i, i, i, ctypes.c_uint, vp, sz, vp]
    L.wkv_last_error.restype = ctypes.c_char_p
    L.wkv_status_string.restype = ctypes.c_char_p
    L.wkv_status_string.argtypes = [i]
    return L


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert "wkv_prefill" in names and "wkv_prefill_varlen" in names
    for n in names:
        assert hasattr(lib, n), "missing export %s" % n


def test_abi_version_and_status_strings(lib):
    assert lib.wkv_abi_version() == 5
    for s in range(5):
        assert lib.wkv_status_string(s)
    assert lib.wkv_status_string(99) == b"unknown status"


# distinct, aligned fake device addresses, far apart
A = 1 << 40
R, K, V, W, U, S_IN, O, S_OUT, WS = (A * (n + 1) for n in range(9))


def call(lib, B=1, T=128, H=4, D=64, dt=BF16, r=R, k=K, v=V, w=W, u=U, s_in=S_IN, o=O,
         s_out=S_OUT, ws=WS, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = lib.wkv_prefill_workspace_bytes(B, T, H, D, dt)
    st = lib.wkv_prefill(r, k, v, w, u, s_in, o, s_out, B, T, H, D, dt, ws, ws_bytes, None)
    return st, lib.wkv_last_error().decode()


@pytest.mark.parametrize("kw,expect", [
    (dict(D=32), EUNSUP),
    (dict(D=128), EUNSUP),
    (dict(dt=7), EUNSUP),
    (dict(H=0), EINVAL),
    (dict(H=65537), EINVAL),
    (dict(B=0), EINVAL),
    (dict(T=-1), EINVAL),
    (dict(B=70000, T=70000), EINVAL),
    (dict(B=300, T=17, H=65536), EUNSUP),     # 19.7M work items: more than one launch holds
    (dict(B=2048, T=1, H=65536), EUNSUP),     # 134M step slices of one wave each
    (dict(r=None), EINVAL),
    (dict(w=None), EINVAL),
    (dict(u=None), EINVAL),
    (dict(o=None), EINVAL),
    (dict(k=K + 2), EINVAL),                  # misaligned
    (dict(o=O + 4), EINVAL),
    (dict(s_in=S_IN + 8), EINVAL),
    (dict(o=R + 64), EINVAL),                 # output overlaps an input
    (dict(s_out=O + 1024), EINVAL),           # state_out inside o
    (dict(s_out=S_IN + 256), EINVAL),         # partial overlap with state_in
])
def test_fixed_length_validation(lib, kw, expect):
    st, msg = call(lib, **kw)
    assert st == expect, (st, msg)
    assert msg


def test_workspace_checks(lib):
    need = lib.wkv_prefill_workspace_bytes(1, 4096, 32, 64, BF16)
    assert need > 0                                   # a split plan needs scratch
    st, msg = call(lib, T=4096, H=32, ws=None)
    assert st == EWS, msg
    st, msg = call(lib, T=4096, H=32, ws_bytes=need - 1)
    assert st == EWS, msg
    st, msg = call(lib, T=4096, H=32, ws=WS + 128)
    assert st == EINVAL and "aligned" in msg
    st, msg = call(lib, T=4096, H=32, ws=O + 256)     # workspace overlaps o
    assert st == EINVAL, msg
    assert lib.wkv_prefill_workspace_bytes(1, 64, 1, 64, F32) == 0
    assert lib.wkv_prefill_workspace_bytes(1, 64, 1, 32, BF16) == 0    # invalid -> 0
    # the query does not disturb the last error
    call(lib, D=32)
    before = lib.wkv_last_error()
    lib.wkv_prefill_workspace_bytes(1, 64, 1, 32, BF16)
    assert lib.wkv_last_error() == before


def test_workspaces_start_with_the_control_records(lib):
    """Every nonzero workspace holds the 256 KiB of control records first and
    the split plan's scratch after them: the 1.5B-class layer (T = 4096,
    H = 32, 16 segments) needs 15 x 32 aggregates of 16,640 bytes and 16 x 32
    start states of 16,384 bytes behind them, each array 256-byte aligned; a
    packed call that is not split still keeps the records ahead of its
    segment tables (offsets, owners, longest-first ranks)."""
    ctl = 262144
    assert re.search(r"#define WKV_WORKSPACE_CONTROL_BYTES %d\b" % ctl, open(HEADER).read())
    align = lambda x: -(-x // 256) * 256
    assert lib.wkv_prefill_workspace_bytes(1, 4096, 32, 64, BF16) == (
        ctl + align(15 * 32 * 16640) + align(16 * 32 * 16384))
    cu = np.array([0, 100, 200], dtype=np.int32)       # two short sequences: no split
    assert lib.wkv_prefill_varlen_workspace_bytes(cu.ctypes.data, 2, 4, 64, BF16) == ctl + 3 * 256


def test_state_pass_runs(lib):
    """A split whose state items alone would leave the device idle cuts each
    segment's state pass into runs, each with its own aggregate.
    4 x 2048 tokens x 32 heads: segments of 512 tokens, 3 x 128 = 384 state
    items, so two runs of 256 tokens (768 aggregates).  With fewer than 256
    (sequence, head) pairs and long enough sequences, the chunked scan runs on
    the producer/consumer kernel over about 256 segments: 4 x 16384 x 32 has
    two segments of 8192 tokens per sequence (128 state items in six runs of
    1408 tokens), 262,144 tokens x 64 heads has four of 65,536 (192 state
    items in four runs of 16,384).  The 1.5B-class layer (480 state items)
    keeps one run per segment."""
    ctl, agg, start = 262144, 16640, 16384
    align = lambda x: -(-x // 256) * 256
    assert lib.wkv_prefill_workspace_bytes(4, 2048, 32, 64, BF16) == (
        ctl + align(3 * 2 * 128 * agg) + align(4 * 4 * 32 * start))
    assert lib.wkv_prefill_workspace_bytes(4, 16384, 32, 64, BF16) == (
        ctl + align(1 * 6 * 128 * agg) + align(4 * 2 * 32 * start))
    assert lib.wkv_prefill_workspace_bytes(1, 262144, 64, 64, BF16) == (
        ctl + align(3 * 4 * 64 * agg) + align(4 * 64 * start))
    assert lib.wkv_prefill_workspace_bytes(1, 4096, 32, 64, BF16) == (
        ctl + align(15 * 32 * agg) + align(16 * 32 * start))


def test_every_fixed_length_plan_fits_the_static_scratch(lib):
    """wkv_prefill_noalloc runs any fixed-length plan out of its 36 MiB static
    scratch: over a sweep of batch sizes, lengths and head counts (split
    plans of the 4-wave kernel, with and without state runs, and of the
    producer/consumer kernel) the workspace never needs more."""
    f = lib.wkv_prefill_workspace_bytes
    Ts = [17, 257, 300, 513, 1000, 1025, 2000, 2049, 4096, 5000, 8192, 9000, 16384,
          65536, 100000, 262144, 1000000, 2000000]
    worst = 0
    for B in list(range(1, 33)) + [48, 64, 100, 127, 128, 255, 256, 511, 512]:
        for H in [1, 2, 3, 5, 8, 13, 16, 24, 32, 48, 64, 100, 128, 255, 256, 511]:
            for T in Ts:
                if B * T < 2**31:
                    worst = max(worst, f(B, T, H, 64, BF16))
    assert 16 << 20 < worst <= 36 << 20, worst


def test_split_launch_switch(lib):
    lib.wkv_set_split_launches.restype = ctypes.c_int
    lib.wkv_set_split_launches.argtypes = [ctypes.c_int]
    assert lib.wkv_set_split_launches(2) == EINVAL
    assert b"launches" in lib.wkv_last_error()
    assert lib.wkv_set_split_launches(3) == OK
    assert lib.wkv_set_split_launches(1) == OK


def test_whole_sequence_plans_need_no_workspace(lib):
    """The planner's choice, seen through the workspace query: a bf16 call
    that would be split runs whole sequences (no scratch beyond a packed
    call's planner tables) once it has at least 256 (sequence, head) pairs;
    below that, or in fp32 (its own kernel, never split), nothing changes;
    from 512 pairs on a fixed-length call needs no split either."""
    ws = lambda B, T, H, dt=BF16: lib.wkv_prefill_workspace_bytes(B, T, H, 64, dt)
    assert ws(8, 4096, 32) == 0                       # 256 pairs: whole sequences
    assert ws(2, 1000, 128) == 0 and ws(12, 4096, 32) == 0
    assert ws(4, 4096, 32) > 0 and ws(7, 4096, 32) > 0    # 128, 224 pairs: split
    assert ws(1, 4096, 32) > 0                        # the 1.5B layer: split
    assert ws(16, 4096, 32) == 0                      # 512 pairs: no split needed
    assert ws(8, 16, 32) == 0                         # recurrent steps
    assert ws(8, 4096, 32, F32) == 0                  # fp32: token-serial kernel
    # packed calls: whole sequences too (only the control records and the
    # planner's three tables) when no sequence is longer than twice the mean
    # work per CU; a batch dominated by one long sequence keeps its segments
    # (aggregates and start states)
    vws = lambda lens, H: lib.wkv_prefill_varlen_workspace_bytes(
        np.concatenate([[0], np.cumsum(lens)]).astype(np.int32).ctypes.data, len(lens), H, 64, BF16)
    assert vws([4096] * 8, 32) == 262144 + 3 * 256
    assert vws([4096] * 7 + [200000], 32) > 262144 + 3 * 256 + 16640


def varlen(lib, cu, H=4, dt=BF16, ws_bytes=None, cu_dev=A * 20, **ptrs):
    cu = np.asarray(cu, dtype=np.int32)
    N = len(cu) - 1
    p = dict(r=R, k=K, v=V, w=W, u=U, s_in=S_IN, o=O, s_out=S_OUT, ws=WS)
    p.update(ptrs)
    if ws_bytes is None:
        ws_bytes = lib.wkv_prefill_varlen_workspace_bytes(cu.ctypes.data, N, H, 64, dt)
    st = lib.wkv_prefill_varlen(p["r"], p["k"], p["v"], p["w"], p["u"], cu_dev, cu.ctypes.data,
                                N, p["s_in"], p["o"], p["s_out"], H, 64, dt, p["ws"], ws_bytes,
                                None)
    return st, lib.wkv_last_error().decode()


@pytest.mark.parametrize("cu,expect", [
    ([1, 5, 9], EINVAL),          # must start at 0
    ([0, 5, 3], EINVAL),          # decreasing
])
def test_varlen_offset_validation(lib, cu, expect):
    st, msg = varlen(lib, cu)
    assert st == expect, msg
    c = np.asarray(cu, dtype=np.int32)
    assert lib.wkv_prefill_varlen_workspace_bytes(c.ctypes.data, len(c) - 1, 4, 64, BF16) == 0


def test_varlen_pointer_validation(lib):
    st, msg = varlen(lib, [0, 100, 300], cu_dev=None)
    assert st == EINVAL and "cu_seqlens_dev" in msg
    st, msg = varlen(lib, [0, 100, 300], cu_dev=A * 20 + 2)
    assert st == EINVAL
    st, msg = varlen(lib, [0, 100, 300], ws=None)
    assert st == EWS
    st, msg = varlen(lib, [0, 100, 300], o=A * 20)            # o overlaps the offsets
    assert st == EINVAL


def test_varlen_workspace_grows_with_segments(lib):
    small = np.array([0, 100, 300], dtype=np.int32)
    big = np.array([0, 30000, 60000, 200000], dtype=np.int32)
    a = lib.wkv_prefill_varlen_workspace_bytes(small.ctypes.data, 2, 32, 64, BF16)
    b = lib.wkv_prefill_varlen_workspace_bytes(big.ctypes.data, 3, 32, 64, BF16)
    assert 0 < a < b
    assert a % 256 == 0 and b % 256 == 0


U2 = A * 30
LOG, C2, OBF16 = 1, 2, 4


def call_ex(lib, flags, u=U, u2=None, B=1, T=128, H=4, dt=BF16, o=O, ws=WS):
    ws_bytes = lib.wkv_prefill_workspace_bytes(B, T, H, 64, dt)
    st = lib.wkv_prefill_ex(R, K, V, W, u, u2, S_IN, o, S_OUT, B, T, H, 64, dt, flags, ws,
                            ws_bytes, None)
    return st, lib.wkv_last_error().decode()


@pytest.mark.parametrize("kw,expect", [
    (dict(flags=8), EUNSUP),                          # unknown flag bit
    (dict(flags=LOG | 8), EUNSUP),
    (dict(flags=0, u2=U2), EINVAL),                   # second value without C2
    (dict(flags=LOG, u=None), EINVAL),                # base Finch needs its bonus
    (dict(flags=C2, u2=U2 + 8), EINVAL),              # misaligned second value
    (dict(flags=C2, u2=U2, o=U2 + 64), EINVAL),       # o overlaps the second value
    (dict(flags=C2 | LOG, u2=U2, o=None), EINVAL),
    (dict(flags=OBF16, o=O + 8), EINVAL),             # bf16 o: still 16-byte aligned
    (dict(flags=OBF16, o=S_OUT - 128 * 4 * 64 * 2 + 256), EINVAL),   # bf16 o reaching state_out
])
def test_extended_validation(lib, kw, expect):
    st, msg = call_ex(lib, **kw)
    assert st == expect, (st, msg)
    assert msg


def test_extended_varlen_validation(lib):
    cu = np.asarray([0, 100, 300], dtype=np.int32)
    ws_bytes = lib.wkv_prefill_varlen_workspace_bytes(cu.ctypes.data, 2, 4, 64, BF16)
    st = lib.wkv_prefill_varlen_ex(R, K, V, W, U, None, A * 20, cu.ctypes.data, 2, S_IN, O, S_OUT,
                                   4, 64, BF16, 16, WS, ws_bytes, None)
    assert st == EUNSUP
    # a bf16 o of 300 tokens x 4 heads x 64 x 2 B ends 256 B into state_out
    st = lib.wkv_prefill_varlen_ex(R, K, V, W, U, None, A * 20, cu.ctypes.data, 2, S_IN,
                                   S_OUT - 300 * 4 * 64 * 2 + 256, S_OUT, 4, 64, BF16, OBF16, WS,
                                   ws_bytes, None)
    assert st == EINVAL and b"overlaps" in lib.wkv_last_error()
    st = lib.wkv_prefill_varlen_ex(R, K, V, W, U, U2, A * 20, cu.ctypes.data, 2, S_IN, O, S_OUT,
                                   4, 64, BF16, LOG, WS, ws_bytes, None)
    assert st == EINVAL and b"Finch-C2" in lib.wkv_last_error()


@pytest.mark.parametrize("kw,expect", [
    (dict(width=2048 + 512), EUNSUP),
    (dict(width=16384), EUNSUP),
    (dict(out=7), EUNSUP),
    (dict(tokens=-1), EINVAL),
    (dict(eps=-1.0), EINVAL),
    (dict(eps=float("nan")), EINVAL),
    (dict(x=None), EINVAL),
    (dict(y=R + 8), EINVAL),                         # misaligned
    (dict(y=R + 4096), EINVAL),                      # y overlaps x
])
def test_layernorm_validation(lib, kw, expect):
    a = dict(x=R, g=K, b=V, eps=1e-5, y=O, out=BF16, tokens=4096, width=2048)
    a.update(kw)
    st = lib.wkv_layernorm_heads(a["x"], a["g"], a["b"], a["eps"], a["y"], a["out"], a["tokens"],
                                 a["width"], None)
    assert st == expect, lib.wkv_last_error()


@pytest.mark.parametrize("kw,expect", [
    (dict(d=2048 + 64), EUNSUP),
    (dict(d=512), EUNSUP),
    (dict(out=3), EUNSUP),
    (dict(tokens=-5), EINVAL),
    (dict(w=None), EINVAL),
    (dict(c=O + 2), EINVAL),
    (dict(c=W + 64), EINVAL),                        # c overlaps the weight
])
def test_compress_validation(lib, kw, expect):
    a = dict(x=R, w=W, c=O, out=F32, tokens=4096, d=2048)
    a.update(kw)
    st = lib.wkv_gold_compress(a["x"], a["w"], a["c"], a["out"], a["tokens"], a["d"], None)
    assert st == expect, lib.wkv_last_error()


def test_workspace_errors_validates_before_any_hip_call(lib):
    lib.wkv_workspace_errors.restype = ctypes.c_int
    lib.wkv_workspace_errors.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                         ctypes.POINTER(ctypes.c_int), ctypes.c_void_p]
    n = ctypes.c_int(-1)
    assert lib.wkv_workspace_errors(A, 1 << 20, 0, None, None) == EINVAL
    assert lib.wkv_workspace_errors(A, 4096, 1, ctypes.byref(n), None) == EWS and n.value == 0
    n.value = -1
    assert lib.wkv_workspace_errors(A, 0, 0, ctypes.byref(n), None) == OK and n.value == 0
    # no workspace and no allocation-free call made on this device (or no
    # device at all): nothing to read
    n.value = -1
    assert lib.wkv_workspace_errors(None, 0, 0, ctypes.byref(n), None) == OK and n.value == 0


def test_wait_bound_switch(lib):
    lib.wkv_set_wait_bound.restype = ctypes.c_int
    lib.wkv_set_wait_bound.argtypes = [ctypes.c_ulonglong]
    assert lib.wkv_set_wait_bound(1 << 32) == EINVAL
    assert lib.wkv_set_wait_bound(100) == OK
    assert lib.wkv_set_wait_bound(0) == OK          # back to the default


def test_noalloc_entry_point_validates_before_any_hip_call(lib):
    """wkv_prefill_noalloc plans and checks its arguments like wkv_prefill_ex
    before it looks up its static scratch (so these fail without a GPU)."""
    vp, i = ctypes.c_void_p, ctypes.c_int
    f = lib.wkv_prefill_noalloc
    f.restype = i
    f.argtypes = [vp] * 9 + [i] * 5 + [ctypes.c_uint, vp]
    args = lambda **kw: [kw.get("r", R), K, V, W, U, None, S_IN, kw.get("o", O), S_OUT, 1, 4096, 32,
                         kw.get("D", 64), BF16, kw.get("flags", 0), None]
    assert f(*args(D=32)) == EUNSUP
    assert f(*args(r=None)) == EINVAL and b"r is NULL" in lib.wkv_last_error()
    assert f(*args(o=O + 4)) == EINVAL and b"aligned" in lib.wkv_last_error()
    assert f(*args(flags=8)) == EUNSUP
