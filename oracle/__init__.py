"""Finch WKV oracle -- plain fp64 CPU implementations.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  It
shares no code with the GPU library (``linear_attention_rnn_finch_amd``) and
never imports it.

Two implementations of the same definition live here:

* ``wkv_scan`` -- the sequential recurrence in plain C (``wkv_oracle.c``),
  OpenMP across independent (sequence, head) slices.  Used for every parity
  comparison with the GPU.
* ``wkv_sum_form`` -- the closed sum printed on the GoldFinch architecture
  summary page (section 3.4, "Finch-C2 Time Mixing", equation for wkv_t),
  evaluated by brute force in numpy, O(T^2 D^2).  Tiny inputs only; it pins
  the recurrence.

Conventions (readings of the pages where they leave a choice open):
  r, k, v, w : [tokens, H, D] packed rows (a batch is a packed set with
               offsets ``cu_seqlens``); D is the head size.
  u          : [H, D] static per-channel bonus (base Finch).
  state      : [N, H, D, D]; row = key channel i (decayed), column = value
               channel j.
  o_t[j] = sum_i r_t[i] (S_{t-1}[i, j] + u[i] k_t[i] v_t[j]);
  S_t    = diag(w_t) S_{t-1} + k_t^T v_t.

Selectable forms of the same section (keyword arguments of both functions):
  decay="log"   the decay input holds d_t and w_t = exp(-exp(d_t))
                (paragraph "Data-dependent decay");
  variant="c2"  the Finch-C2 time mixer: the state takes k_t (1 - w_t), there
                is no static bonus, and the second value u'_t (``second_value``,
                same layout and type as r; None = absent) is added:
                o_t = r_t S_{t-1} + u'_t.

Parity status: every function here is pinned by the CPU tests in
``tests/test_oracle.py`` (brute force, no-decay closed form, constant-decay
IIR filter, split/carry invariant, hand-worked fixture).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "wkv_oracle.c")
_BUILD_DIR = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_BUILD_DIR, "liboracle_wkv.so")

_lock = threading.Lock()
_lib = None

KIND_F32 = 0
KIND_BF16 = 1


def build(force: bool = True) -> str:
    """Compile ``wkv_oracle.c`` with gcc (fp64, no fast-math, OpenMP)."""
    os.makedirs(_BUILD_DIR, exist_ok=True)
    if not force and os.path.exists(_LIB_PATH) and \
            os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", "-fno-fast-math", "-Wall", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            path = build(force=False)
            lib = ctypes.CDLL(path)
            lib.oracle_wkv_f64.restype = ctypes.c_int
            lib.oracle_wkv_f64.argtypes = [
                ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
            lib.oracle_wkv_f64_ex.restype = ctypes.c_int
            lib.oracle_wkv_f64_ex.argtypes = [
                ctypes.c_int, ctypes.c_int, ctypes.c_int,
                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
            lib.oracle_max_threads.restype = ctypes.c_int
            _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def _ptr(a):
    return None if a is None else a.ctypes.data


DECAY_KINDS = {"w": 0, "log": 1}
VARIANTS = {"finch": 0, "c2": 1}


def wkv_scan(r, k, v, w, u, state_in=None, cu_seqlens=None, *, H=None,
             slice_mask=None, want_o=True, threads=0, decay="w", variant="finch",
             second_value=None):
    """Run the fp64 recurrence.

    ``r, k, v, w`` are numpy arrays of float32, or uint16 holding bf16 bit
    patterns, shaped [B, T, H, D] (fixed length) or [tokens, H, D] with
    ``cu_seqlens`` ([N + 1] offsets).  ``w`` holds w_t, or d_t with
    ``decay="log"``.  With ``variant="c2"``, ``u`` is ignored (may be None)
    and ``second_value`` (like r, or None) is u'_t.  Returns ``(o,
    state_out)`` as float64; ``o`` has the input's shape (rows of slices not
    in ``slice_mask`` stay 0).
    """
    if decay not in DECAY_KINDS or variant not in VARIANTS:
        raise ValueError("decay must be one of %s, variant one of %s" % (list(DECAY_KINDS), list(VARIANTS)))
    if variant != "c2" and second_value is not None:
        raise ValueError("second_value belongs to the Finch-C2 variant")
    shape = r.shape
    if r.dtype == np.uint16:
        kind = KIND_BF16
    elif r.dtype == np.float32:
        kind = KIND_F32
    else:
        raise TypeError("inputs must be float32 or bf16 bit patterns (uint16)")
    for name, a in (("k", k), ("v", v), ("w", w), ("second_value", second_value)):
        if a is not None and (a.shape != shape or a.dtype != r.dtype):
            raise ValueError("%s must match r in shape and dtype" % name)
    if cu_seqlens is None:
        if r.ndim != 4:
            raise ValueError("fixed-length inputs are [B, T, H, D]")
        B, T, H_, D = shape
        cu = np.arange(B + 1, dtype=np.int64) * T
    else:
        if r.ndim != 3:
            raise ValueError("packed inputs are [tokens, H, D]")
        _, H_, D = shape
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
        if cu[-1] != shape[0]:
            raise ValueError("cu_seqlens[-1] must equal the token count")
    N = len(cu) - 1
    r, k, v, w = (np.ascontiguousarray(a) for a in (r, k, v, w))
    u2 = None if second_value is None else np.ascontiguousarray(second_value)
    if variant == "c2" and u is None:
        u = np.zeros((H_, D), dtype=np.float32)
    u = np.ascontiguousarray(u, dtype=np.float32).reshape(H_, D)
    s0 = None
    if state_in is not None:
        s0 = np.ascontiguousarray(state_in, dtype=np.float64).reshape(N, H_, D, D)
    mask = None
    if slice_mask is not None:
        mask = np.ascontiguousarray(slice_mask, dtype=np.uint8).reshape(N * H_)
    o = np.zeros(shape, dtype=np.float64) if want_o else None
    so = np.zeros((N, H_, D, D), dtype=np.float64)
    if decay == "w" and variant == "finch":
        rc = _load().oracle_wkv_f64(kind, _ptr(r), _ptr(k), _ptr(v), _ptr(w),
                                    _ptr(u), _ptr(s0), _ptr(cu), N, H_, D,
                                    _ptr(mask), _ptr(o), _ptr(so), int(threads))
    else:
        rc = _load().oracle_wkv_f64_ex(kind, DECAY_KINDS[decay], VARIANTS[variant],
                                       _ptr(r), _ptr(k), _ptr(v), _ptr(w), _ptr(u),
                                       _ptr(u2), _ptr(s0), _ptr(cu), N, H_, D,
                                       _ptr(mask), _ptr(o), _ptr(so), int(threads))
    if rc != 0:
        raise ValueError("oracle rejected cu_seqlens")
    return o, so


def bf16_bits_to_f64(bits):
    """Exact widening of bf16 bit patterns (uint16) to float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def as_f64(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_bits_to_f64(a)
    return a.astype(np.float64)


def wkv_sum_form(r, k, v, w, u, s0=None, *, decay="w", variant="finch", second_value=None):
    """Brute-force closed sum for ONE (sequence, head) slice, fp64.

    Direct transcription of the definition (GoldFinch architecture summary,
    section 3.4, state equation): the state read by token t is

        wkv_t = diag(prod_{j<t} w_j) S_0
                + sum_{i<t} diag(prod_{j=i+1}^{t-1} w_j) k_i^T v_i

    and o_t = r_t wkv_t + r_t diag(u) k_t^T v_t.  Every product of decays is
    formed explicitly for every (t, i) pair -- no recurrence, no reuse.
    With decay="log" the w argument holds d and w = exp(-exp(d)) (paragraph
    "Data-dependent decay"); with variant="c2" the keys in the sum are
    k_i (1 - w_i) (paragraph "Key computation with normalization property")
    and o_t = r_t wkv_t + u'_t (output equation; u'_t = second_value[t], or
    no term when None).
    r, k, v, w: [T, D]; u: [D]; s0: [D, D] or None.  Returns (o [T, D],
    state after the last token [D, D]).
    """
    r, k, v, w = (as_f64(a) for a in (r, k, v, w))
    T, D = r.shape
    if decay == "log":
        w = np.exp(-np.exp(w))
    if variant == "c2":
        k = k * (1.0 - w)
        u = np.zeros(D)
        u2 = np.zeros((T, D)) if second_value is None else as_f64(second_value)
    else:
        u = as_f64(u)
        u2 = np.zeros((T, D))
    S0 = np.zeros((D, D)) if s0 is None else np.asarray(s0, dtype=np.float64)
    o = np.zeros((T, D))

    def state_seen_by(t):
        # decays of tokens 0..t-1 applied to the carried-in state
        dec0 = np.ones(D)
        for j in range(t):
            dec0 = dec0 * w[j]
        acc = dec0[:, None] * S0
        for i in range(t):
            dec = np.ones(D)
            for j in range(i + 1, t):
                dec = dec * w[j]
            acc = acc + (dec * k[i])[:, None] * v[i][None, :]
        return acc

    for t in range(T):
        wkv = state_seen_by(t)
        o[t] = r[t] @ wkv + (r[t] * u * k[t]).sum() * v[t] + u2[t]
    return o, state_seen_by(T)
