"""Helpers for the GPU parity tests: move a synthetic workload to the GPU, run
the library through its Python binding (which calls the C ABI), run the oracle
on the same bits, and compare."""
from __future__ import annotations

import sys

import numpy as np

import oracle
from synth import error_report, select_heads


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_gpu(wl):
    import torch
    dev = torch.device("cuda", 0)

    def cvt(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    out = {name: cvt(getattr(wl, name)) for name in ("r", "k", "v", "w")}
    out["u"] = torch.from_numpy(wl.u).to(dev)
    out["u2"] = None if wl.u2 is None else cvt(wl.u2)
    out["state0"] = None if wl.state0 is None else torch.from_numpy(wl.state0).to(dev)
    if wl.packed:
        out["cu"] = torch.from_numpy(wl.cu_seqlens.astype(np.int32)).to(dev)
        out["cu_host"] = torch.from_numpy(wl.cu_seqlens.astype(np.int32))
    return out


def run_gpu(wl, g=None, state_in="default", **kw):
    """Run the library on workload ``wl``; returns torch (o, state_out)."""
    import linear_attention_rnn_finch_amd as fw
    g = g or to_gpu(wl)
    s0 = g["state0"] if isinstance(state_in, str) else state_in
    if wl.variant == "c2":
        kw.setdefault("variant", "c2")
        kw.setdefault("second_value", g["u2"])
    if wl.decay == "log":
        kw.setdefault("decay", "log")
    u = None if wl.variant == "c2" else g["u"]
    if wl.packed:
        return fw.prefill_varlen(g["r"], g["k"], g["v"], g["w"], u, g["cu"], s0,
                                 cu_seqlens_host=g["cu_host"], **kw)
    return fw.prefill(g["r"], g["k"], g["v"], g["w"], u, s0, **kw)


def run_oracle(wl, heads=None, want_o=True):
    """fp64 oracle on the same bits.  With ``heads``, only those heads are
    computed and returned (arrays hold just the selected heads, in order)."""
    sub = wl if heads is None else select_heads(wl, heads)
    return oracle.wkv_scan(sub.r, sub.k, sub.v, sub.w, sub.u, sub.state0, sub.cu_seqlens,
                           want_o=want_o, decay=sub.decay, variant=sub.variant,
                           second_value=sub.u2)


def _host(x, heads, axis):
    """Selected heads of a GPU (torch) or host array, as a float64 numpy array;
    the selection happens before the copy to the host."""
    if heads is not None:
        idx = list(heads)
        if hasattr(x, "cpu"):
            import torch
            x = x.index_select(axis % x.dim(), torch.tensor(idx, device=x.device))
        else:
            x = np.take(x, idx, axis=axis)
    if hasattr(x, "cpu"):
        x = x.float().cpu().numpy()
    return x


class Errors(tuple):
    """(normwise o error, normwise state error), the pass measures, with the
    per-row errors (``row_o``, ``row_s``) and both full reports attached."""

    def __new__(cls, rep_o, rep_s):
        self = super().__new__(cls, (rep_o["block"], rep_s["block"]))
        self.rep_o, self.rep_s = rep_o, rep_s
        self.row_o, self.row_s = rep_o["row"], rep_s["row"]
        return self


def errors(wl, o_gpu, s_gpu, o_ref, s_ref, heads=None):
    """Error reports of (o, state) against the oracle (synth.compare): the
    normwise block errors unpack as a pair; per-row and floored element-wise
    errors are logged and attached.  With ``heads``, the references hold only
    those heads and the GPU results are reduced to them."""
    empty = {"block": 0.0, "row": 0.0, "elem_floored": 0.0, "worst_row": None}
    rep_o = empty
    if o_ref is not None:
        rep_o = error_report(_host(o_gpu, heads, -2), o_ref, wl.cu_seqlens, heads=heads)
    rep_s = error_report(_host(s_gpu, heads, 1), s_ref, kind="state", heads=heads)
    log("  o: block %.3e row %.3e elem(floored) %.3e worst row %s | state: block %.3e row %.3e"
        % (rep_o["block"], rep_o["row"], rep_o["elem_floored"], rep_o["worst_row"],
           rep_s["block"], rep_s["row"]))
    return Errors(rep_o, rep_s)


def gpu_block_error(a, b, dims):
    """Normwise error max|a - b| / max|b| over each block of two GPU tensors,
    a block being all elements that differ only along ``dims``; max over the
    blocks.  o [B, T, H, D]: dims (1, 3); state [N, H, D, D]: dims (2, 3)."""
    import torch
    num = (a - b).abs().amax(dim=dims)
    den = b.abs().amax(dim=dims)
    return float(torch.max(num / torch.clamp(den, min=1e-30)))
