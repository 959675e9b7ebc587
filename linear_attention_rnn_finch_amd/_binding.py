"""ctypes binding of libfinch_wkv.so (argument marshalling only).

Every step of the computation runs in the library's HIP kernels; this module
only checks tensor metadata, allocates outputs/workspace through torch's
caching allocator and passes raw device pointers plus torch's current HIP
stream.  There is no CPU fallback: if the library is missing, importing the
package raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY_PATH = os.path.join(_PKG, "libfinch_wkv.so")

WKV_OK, WKV_EINVAL, WKV_EUNSUPPORTED, WKV_EWORKSPACE, WKV_EHIP = range(5)
WKV_F32, WKV_BF16 = 0, 1
WKV_FLAG_DECAY_LOG, WKV_FLAG_FINCH_C2, WKV_FLAG_OUT_BF16 = 1, 2, 4
HEAD_DIM = 64
# control records at the start of every nonzero workspace: zero before the
# first call that uses the workspace, never written between calls
WORKSPACE_CONTROL_BYTES = 262144
DECAYS = ("w", "log")            # decay argument holds w_t, or d_t with w_t = exp(-exp(d_t))
VARIANTS = ("finch", "c2")       # base Finch (bonus u) or the Finch-C2 time mixer

if not os.path.exists(LIBRARY_PATH):
    raise ImportError(
        "libfinch_wkv.so is not built (%s); run `python "
        "linear_attention_rnn_finch_amd/build_lib.py` or __graft_entry__.build()" % LIBRARY_PATH)

_lib = ctypes.CDLL(LIBRARY_PATH)
_vp, _sz, _i, _i32p = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.POINTER(ctypes.c_int32)

_lib.wkv_abi_version.restype = _i
_lib.wkv_abi_version.argtypes = []
_lib.wkv_status_string.restype = ctypes.c_char_p
_lib.wkv_status_string.argtypes = [_i]
_lib.wkv_last_error.restype = ctypes.c_char_p
_lib.wkv_last_error.argtypes = []
_lib.wkv_prefill_workspace_bytes.restype = _sz
_lib.wkv_prefill_workspace_bytes.argtypes = [_i, _i, _i, _i, _i]
_lib.wkv_prefill_varlen_workspace_bytes.restype = _sz
_lib.wkv_prefill_varlen_workspace_bytes.argtypes = [_vp, _i, _i, _i, _i]
_lib.wkv_prefill.restype = _i
_lib.wkv_prefill.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                             _i, _i, _i, _i, _i, _vp, _sz, _vp]
_lib.wkv_prefill_varlen.restype = _i
_lib.wkv_prefill_varlen.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i,
                                    _vp, _vp, _vp, _i, _i, _i, _vp, _sz, _vp]
_lib.wkv_prefill_ex.restype = _i
_lib.wkv_prefill_ex.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                _i, _i, _i, _i, _i, ctypes.c_uint, _vp, _sz, _vp]
_lib.wkv_layernorm_heads.restype = _i
_lib.wkv_layernorm_heads.argtypes = [_vp, _vp, _vp, ctypes.c_float, _vp, _i, ctypes.c_int64, _i, _vp]
_lib.wkv_gold_compress.restype = _i
_lib.wkv_gold_compress.argtypes = [_vp, _vp, _vp, _i, ctypes.c_int64, _i, _vp]
_lib.wkv_set_split_launches.restype = _i
_lib.wkv_set_split_launches.argtypes = [_i]
_lib.wkv_set_wait_bound.restype = _i
_lib.wkv_set_wait_bound.argtypes = [ctypes.c_ulonglong]
_lib.wkv_workspace_errors.restype = _i
_lib.wkv_workspace_errors.argtypes = [_vp, _sz, _i, ctypes.POINTER(ctypes.c_int), _vp]
_lib.wkv_prefill_varlen_ex.restype = _i
_lib.wkv_prefill_varlen_ex.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i,
                                       _vp, _vp, _vp, _i, _i, _i, ctypes.c_uint, _vp, _sz, _vp]


class WkvError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        msg = _lib.wkv_status_string(status).decode()
        super().__init__("%s (%d): %s" % (msg, status, detail))


def abi_version() -> int:
    return int(_lib.wkv_abi_version())


def set_split_launches(launches: int) -> None:
    """Launch form of split bf16 calls made from this thread: 1 (default) runs
    one launch where it can, 3 always the state pass, the segment scan and the
    chunked scan.  Both give identical results.  The one launch needs its
    workgroups resident together; beside long-running kernels of other
    streams, take 3 (see wkv_set_split_launches in finch_wkv.h)."""
    st = int(_lib.wkv_set_split_launches(int(launches)))
    if st != WKV_OK:
        raise WkvError(st, _lib.wkv_last_error().decode())


def set_wait_bound(ticks: int) -> None:
    """Bound of each wait of the one launch, in ticks of the GPU's 100 MHz
    clock, for tests of the error path (calls made from this thread); 0
    restores the default (2^27 ticks, about 1.3 s).  A bound too short for
    the workgroups to meet voids the call's results, which
    workspace_errors() then reports."""
    _check(int(_lib.wkv_set_wait_bound(int(ticks))))


def new_workspace(nbytes: int, device) -> torch.Tensor:
    """A workspace of nbytes on `device`, its control records zeroed (the
    state a workspace must be in before its first call)."""
    ws = torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)
    ws[:WORKSPACE_CONTROL_BYTES].zero_()
    return ws


def workspace_errors(workspace=None, clear: bool = False, stream=None) -> int:
    """Control records of `workspace` (a tensor from new_workspace, or None
    for the static scratch of the allocation-free entry point on the current
    device) marked by a one-launch call whose bounded wait expired, i.e. whose
    results are void; 0 means every such call kept its results.  Waits for the
    work queued on the stream; clear=True also zeroes each marked record (its
    counters may be out of step after an expired wait: clear before using a
    marked workspace again)."""
    if workspace is None:
        ptr, nbytes = None, 0
    else:
        _device_tensor("workspace", workspace)
        ptr, nbytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
        if nbytes == 0:                  # a call that needed no workspace: no records
            return 0
        _same_device(workspace.device, stream)
    n = ctypes.c_int(0)
    _check(int(_lib.wkv_workspace_errors(ptr, nbytes, 1 if clear else 0, ctypes.byref(n),
                                         _stream_handle(stream))))
    return int(n.value)


def _check(status: int):
    if status != WKV_OK:
        raise WkvError(status, _lib.wkv_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return WKV_BF16
    if t.dtype == torch.float32:
        return WKV_F32
    raise TypeError("r, k, v, w must be bfloat16 or float32, got %s" % t.dtype)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream_handle(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _device_tensor(name, t, dtype=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be on a GPU device" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))


def _same_device(device, stream, **tensors):
    """Every given tensor (and the stream, if any) on `device`: the C ABI takes
    bare pointers and launches on the stream's device, so a tensor of another
    GPU would be read or written by kernels that cannot see it."""
    for name, t in tensors.items():
        if t is not None and t.device != device:
            raise ValueError("%s is on %s, the call's inputs on %s" % (name, t.device, device))
    if stream is not None and stream.device != device:
        raise ValueError("stream belongs to %s, the call's inputs to %s" % (stream.device, device))


def workspace_bytes(B: int, T: int, H: int, D: int = HEAD_DIM, dtype=torch.bfloat16) -> int:
    code = WKV_BF16 if dtype == torch.bfloat16 else WKV_F32
    return int(_lib.wkv_prefill_workspace_bytes(B, T, H, D, code))


def varlen_workspace_bytes(cu_seqlens_host, H: int, D: int = HEAD_DIM, dtype=torch.bfloat16) -> int:
    cu = torch.as_tensor(cu_seqlens_host, dtype=torch.int32).contiguous()
    code = WKV_BF16 if dtype == torch.bfloat16 else WKV_F32
    return int(_lib.wkv_prefill_varlen_workspace_bytes(cu.data_ptr(), cu.numel() - 1, H, D, code))


def _flags(decay, variant, u, second_value, r, out_dtype=torch.float32):
    """Flags word of the extended entry points; checks u / second_value."""
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out_dtype must be torch.float32 or torch.bfloat16")
    if decay not in DECAYS:
        raise ValueError("decay must be one of %s" % (DECAYS,))
    if variant not in VARIANTS:
        raise ValueError("variant must be one of %s" % (VARIANTS,))
    flags = (WKV_FLAG_DECAY_LOG if decay == "log" else 0) | (WKV_FLAG_FINCH_C2 if variant == "c2" else 0)
    if out_dtype == torch.bfloat16:
        flags |= WKV_FLAG_OUT_BF16
    if variant == "c2":
        if second_value is not None:
            _device_tensor("second_value", second_value, r.dtype)
            if second_value.shape != r.shape:
                raise ValueError("second_value must have r's shape")
    else:
        if second_value is not None:
            raise ValueError("second_value belongs to the Finch-C2 variant")
        _device_tensor("u", u, torch.float32)
    return flags


def _on_stream(stream):
    """Context in which the binding allocates: the stream the kernels run on.
    The caching allocator then ties every block it hands out here (outputs,
    workspace) to that stream, so no other work can be given the block while
    the kernels still use it."""
    import contextlib
    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


def _workspace(nbytes, device, given, stream):
    """The caller's workspace (checked; its control records are the caller's
    to keep), or a new one on the kernels' stream with them zeroed."""
    if nbytes == 0:
        return None, 0
    if given is not None:
        _device_tensor("workspace", given)
        if given.device != device:
            raise ValueError("workspace must be on %s, got %s" % (device, given.device))
        return given, given.numel() * given.element_size()
    with _on_stream(stream):
        return new_workspace(nbytes, device), nbytes


def _check_outputs(o, state_out, o_shape, s_shape, out_dtype):
    if o is not None:
        _device_tensor("o", o, out_dtype)
        if tuple(o.shape) != o_shape:
            raise ValueError("o must be %s, got %s" % (o_shape, tuple(o.shape)))
    if state_out is not None:
        _device_tensor("state_out", state_out, torch.float32)
        if tuple(state_out.shape) != s_shape:
            raise ValueError("state_out must be %s, got %s" % (s_shape, tuple(state_out.shape)))


def prefill(r, k, v, w, u, state_in=None, *, o=None, state_out=None, want_state=True,
            workspace=None, stream=None, decay="w", variant="finch", second_value=None,
            out_dtype=torch.float32):
    """Finch WKV pre-fill of a fixed-length batch on the GPU.

    r, k, v, w: [B, T, H, 64] bfloat16 (or float32), contiguous, same device.
    u: [H, 64] float32.  state_in: [B, H, 64, 64] float32 or None (zeros).
    Returns (o [B, T, H, 64] in ``out_dtype`` (float32, or bfloat16 rounded
    to nearest even), state_out [B, H, 64, 64] float32 or None).
    ``state_out`` may be ``state_in`` (carried state, updated in place).
    ``decay="log"``: w holds d with w = exp(-exp(d)).  ``variant="c2"``: the
    Finch-C2 mixer (k is taken before its (1 - w) factor, u is unused and may
    be None, ``second_value`` like r or None).
    """
    for name, t in (("r", r), ("k", k), ("v", v), ("w", w)):
        _device_tensor(name, t, r.dtype)
    if r.dim() != 4:
        raise ValueError("r must be [B, T, H, D]")
    B, T, H, D = r.shape
    for name, t in (("k", k), ("v", v), ("w", w)):
        if t.shape != r.shape:
            raise ValueError("%s shape %s != r shape %s" % (name, tuple(t.shape), tuple(r.shape)))
    flags = _flags(decay, variant, u, second_value, r, out_dtype)
    if variant == "finch" and tuple(u.shape) != (H, D):
        raise ValueError("u must be [H, D] = %s" % ((H, D),))
    if variant == "c2":
        u = None
    if state_in is not None:
        _device_tensor("state_in", state_in, torch.float32)
        if tuple(state_in.shape) != (B, H, D, D):
            raise ValueError("state_in must be [B, H, D, D]")
    code = _dtype_code(r)
    _check_outputs(o, state_out, (B, T, H, D), (B, H, D, D), out_dtype)
    _same_device(r.device, stream, k=k, v=v, w=w, u=u, second_value=second_value, state_in=state_in,
                 o=o, state_out=state_out, workspace=workspace)
    with _on_stream(stream):
        if o is None:
            o = torch.empty((B, T, H, D), dtype=out_dtype, device=r.device)
        if state_out is None and want_state:
            state_out = torch.empty((B, H, D, D), dtype=torch.float32, device=r.device)
    need = int(_lib.wkv_prefill_workspace_bytes(B, T, H, D, code))
    ws, ws_bytes = _workspace(need, r.device, workspace, stream)
    with torch.cuda.device(r.device):
        status = _lib.wkv_prefill_ex(_ptr(r), _ptr(k), _ptr(v), _ptr(w), _ptr(u),
                                     _ptr(second_value), _ptr(state_in), _ptr(o),
                                     _ptr(state_out), B, T, H, D, code, flags, _ptr(ws),
                                     ws_bytes, _stream_handle(stream))
    _check(status)
    return o, state_out


def prefill_varlen(r, k, v, w, u, cu_seqlens, state_in=None, *, cu_seqlens_host=None, o=None,
                   state_out=None, want_state=True, workspace=None, stream=None, decay="w",
                   variant="finch", second_value=None, out_dtype=torch.float32):
    """Finch WKV pre-fill of N packed sequences.

    r, k, v, w: [total_tokens, H, 64]; cu_seqlens: [N + 1] int32 offsets on the
    GPU; cu_seqlens_host: the same offsets on the host (copied from the device,
    with a synchronisation, when omitted).  state_in/state_out: [N, H, 64, 64].
    ``decay``, ``variant``, ``second_value`` and ``out_dtype`` as for
    ``prefill``.
    """
    for name, t in (("r", r), ("k", k), ("v", v), ("w", w)):
        _device_tensor(name, t, r.dtype)
    if r.dim() != 3:
        raise ValueError("packed r must be [tokens, H, D]")
    total, H, D = r.shape
    for name, t in (("k", k), ("v", v), ("w", w)):
        if t.shape != r.shape:
            raise ValueError("%s shape differs from r" % name)
    flags = _flags(decay, variant, u, second_value, r, out_dtype)
    if variant == "finch" and tuple(u.shape) != (H, D):
        raise ValueError("u must be [H, D] = %s" % ((H, D),))
    if variant == "c2":
        u = None
    _device_tensor("cu_seqlens", cu_seqlens, torch.int32)
    N = cu_seqlens.numel() - 1
    if cu_seqlens_host is None:
        cu_seqlens_host = cu_seqlens.cpu()
    cu_host = torch.as_tensor(cu_seqlens_host, dtype=torch.int32).contiguous()
    if cu_host.numel() != N + 1:
        raise ValueError("cu_seqlens_host must have N + 1 entries")
    if int(cu_host[-1]) != total:
        raise ValueError("cu_seqlens[-1]=%d != token count %d" % (int(cu_host[-1]), total))
    if state_in is not None:
        _device_tensor("state_in", state_in, torch.float32)
        if tuple(state_in.shape) != (N, H, D, D):
            raise ValueError("state_in must be [N, H, D, D]")
    code = _dtype_code(r)
    _check_outputs(o, state_out, (total, H, D), (N, H, D, D), out_dtype)
    _same_device(r.device, stream, k=k, v=v, w=w, u=u, second_value=second_value, cu_seqlens=cu_seqlens,
                 state_in=state_in, o=o, state_out=state_out, workspace=workspace)
    with _on_stream(stream):
        if o is None:
            o = torch.empty((total, H, D), dtype=out_dtype, device=r.device)
        if state_out is None and want_state:
            state_out = torch.empty((N, H, D, D), dtype=torch.float32, device=r.device)
    need = int(_lib.wkv_prefill_varlen_workspace_bytes(cu_host.data_ptr(), N, H, D, code))
    ws, ws_bytes = _workspace(need, r.device, workspace, stream)
    with torch.cuda.device(r.device):
        status = _lib.wkv_prefill_varlen_ex(_ptr(r), _ptr(k), _ptr(v), _ptr(w), _ptr(u),
                                            _ptr(second_value), _ptr(cu_seqlens),
                                            cu_host.data_ptr(), N, _ptr(state_in), _ptr(o),
                                            _ptr(state_out), H, D, code, flags, _ptr(ws),
                                            ws_bytes, _stream_handle(stream))
    _check(status)
    return o, state_out


def _out_code(dtype):
    if dtype == torch.bfloat16:
        return WKV_BF16
    if dtype == torch.float32:
        return WKV_F32
    raise TypeError("output dtype must be bfloat16 or float32, got %s" % dtype)


def layernorm_heads(x, gamma, beta, eps=1e-5, *, out_dtype=torch.bfloat16, y=None, stream=None):
    """LayerNorm over the concatenated heads of each token (Finch-C2 output).

    x: [..., W] float32 (e.g. the pre-fill output o viewed as [tokens, H*64]),
    W a multiple of 1024 up to 8192; gamma, beta: [W] float32.  Returns y with
    x's shape in ``out_dtype`` (bfloat16 or float32)."""
    _device_tensor("x", x, torch.float32)
    W = x.shape[-1]
    for name, t in (("gamma", gamma), ("beta", beta)):
        _device_tensor(name, t, torch.float32)
        if tuple(t.shape) != (W,):
            raise ValueError("%s must be [%d]" % (name, W))
    code = _out_code(out_dtype)
    if y is not None:
        _device_tensor("y", y, out_dtype)
        if y.shape != x.shape:
            raise ValueError("y must have x's shape")
    _same_device(x.device, stream, gamma=gamma, beta=beta, y=y)
    if y is None:
        with _on_stream(stream):
            y = torch.empty(x.shape, dtype=out_dtype, device=x.device)
    tokens = x.numel() // W if W else 0
    with torch.cuda.device(x.device):
        status = _lib.wkv_layernorm_heads(_ptr(x), _ptr(gamma), _ptr(beta), float(eps), _ptr(y), code,
                                          tokens, W, _stream_handle(stream))
    _check(status)
    return y


def gold_compress(x, w_kd, *, out_dtype=torch.float32, c=None, stream=None):
    """GOLD key compression c = x W_KD (d_model -> d_model/16).

    x: [tokens, d_model] bfloat16; w_kd: [d_model/16, d_model] bfloat16, i.e.
    W_KD transposed (a linear layer's weight layout).  Returns c
    [tokens, d_model/16] in ``out_dtype`` (float32 or bfloat16)."""
    _device_tensor("x", x, torch.bfloat16)
    _device_tensor("w_kd", w_kd, torch.bfloat16)
    if x.dim() != 2:
        raise ValueError("x must be [tokens, d_model]")
    tokens, D = x.shape
    if tuple(w_kd.shape) != (D // 16, D):
        raise ValueError("w_kd must be [d_model/16, d_model] = %s" % ((D // 16, D),))
    code = _out_code(out_dtype)
    if c is not None:
        _device_tensor("c", c, out_dtype)
        if tuple(c.shape) != (tokens, D // 16):
            raise ValueError("c must be [tokens, d_model/16]")
    _same_device(x.device, stream, w_kd=w_kd, c=c)
    if c is None:
        with _on_stream(stream):
            c = torch.empty((tokens, D // 16), dtype=out_dtype, device=x.device)
    with torch.cuda.device(x.device):
        status = _lib.wkv_gold_compress(_ptr(x), _ptr(w_kd), _ptr(c), code, tokens, D, _stream_handle(stream))
    _check(status)
    return c
