"""Helpers for the GPU parity tests: move a synthetic workload to the GPU, run
the library through its Python binding (which calls the C ABI), run the oracle
on the same bits, and compare."""
from __future__ import annotations

import sys

import numpy as np

import oracle
from synth import max_block_error


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
    if wl.packed:
        return fw.prefill_varlen(g["r"], g["k"], g["v"], g["w"], g["u"], g["cu"], s0,
                                 cu_seqlens_host=g["cu_host"], **kw)
    return fw.prefill(g["r"], g["k"], g["v"], g["w"], g["u"], s0, **kw)


def run_oracle(wl, heads=None, want_o=True):
    """fp64 oracle on the same bits; ``heads`` restricts the computed slices."""
    mask = None
    if heads is not None:
        H = wl.u.shape[0]
        sel = np.zeros(H, dtype=np.uint8)
        sel[list(heads)] = 1
        mask = np.tile(sel, wl.n_seq)
    return oracle.wkv_scan(wl.r, wl.k, wl.v, wl.w, wl.u, wl.state0, wl.cu_seqlens,
                           slice_mask=mask, want_o=want_o)


def errors(wl, o_gpu, s_gpu, o_ref, s_ref, heads=None):
    """Max normwise block errors (o, state) over the selected heads."""
    o_np = o_gpu.float().cpu().numpy() if hasattr(o_gpu, "cpu") else o_gpu
    s_np = s_gpu.float().cpu().numpy() if hasattr(s_gpu, "cpu") else s_gpu
    if heads is not None:
        heads = list(heads)
        o_np, o_ref = o_np[..., heads, :], o_ref[..., heads, :]
        s_np, s_ref = s_np[:, heads], s_ref[:, heads]
    eo = max_block_error(o_np, o_ref, wl.cu_seqlens) if o_ref is not None else 0.0
    es = max_block_error(s_np, s_ref, kind="state")
    return eo, es
