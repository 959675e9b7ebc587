#!/usr/bin/env python3
"""Finch WKV pre-fill benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 1]
                    [--decay w|log] [--variant finch|c2]

One step = one complete pre-fill call (segment state pass, segment scan and
the chunked scan: every step of the path) over the synthetic workload, inputs
already resident in HBM.  Successive calls rotate over several independent
copies of the inputs, outputs and states, together larger than 1 GiB (four
times the GPU's 256 MB last-level cache), so that every call reads and writes
HBM rather than what the previous call left in the cache.  The K timed steps are captured once into a HIP graph
and replayed, bracketed by device synchronisations, so host launch overhead is
not part of the figure.  The main chunked-scan kernel is also timed per launch
with HIP events attached to its dispatch (through the library's timing hook),
which gives the roofline figure.  The fp64 CPU oracle is timed on the
host cores over a bounded sample of the same workload (cpu_baseline).
With the default workload (one 4096-token sequence, d_model 2048) the batch
of eight such sequences is timed after it in the same process and reported
beside the headline (``same_metric_other_shape``; ``--also ''`` skips it).
``--decay log`` feeds the decay as d (w = exp(-exp(d))) and ``--variant c2``
runs the Finch-C2 mixer (with its second-value stream); each such form is
its own workload name ("<config>+logdecay", "<config>+c2", ...).

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "WKV pre-fill tokens/s at d_model 2048, T=4096; % of HBM/MFMA roofline"
OTHER_METRIC = "WKV tokens/s (workload in config); % of HBM/MFMA roofline"
STEP_MAX_T = 16                  # calls with no longer sequence run the recurrent-step kernel
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, GB/s


def algorithmic_bytes(cfg, tokens, n_seq, has_state_in, variant="finch"):
    """r, k, v, w (and the Finch-C2 second value) in (bf16 or fp32) + o out
    (fp32) per token and head, plus the fp32 state out (and in, when given)
    per (sequence, head)."""
    elt = 2 if cfg.dtype == "bf16" else 4
    n_in = 5 if variant == "c2" else 4
    per_token = cfg.H * cfg.D * (n_in * elt + 4)
    per_state = cfg.D * cfg.D * 4 * (2 if has_state_in else 1)
    return tokens * per_token + n_seq * cfg.H * per_state


# HBM traffic from rocprofv3 FETCH_SIZE / WRITE_SIZE passes (scaled by a plain
# copy of known size); valid only for the workload and the kernel sources the
# counters were taken on.  Records are kept per family: "wkv_call" (the whole
# chunked pre-fill call: state pass, segment scan and chunked scan, summed),
# "wkv_decode" (the step kernels), "epilogue".
def traffic_family(workload_name, kernel_name):
    if workload_name.startswith(("layernorm_heads", "gold_compress")):
        return "epilogue"
    return "wkv_decode" if kernel_name.startswith(("wkv_decode", "wkv_steps")) else "wkv_call"


def traffic_file(workload_name, kernel_name):
    family = traffic_family(workload_name, kernel_name)
    if family == "epilogue":
        return os.path.join(ROOT, "profiles", "%s_traffic.md" % workload_name)
    return os.path.join(ROOT, "profiles", "%s_%s_traffic.md" % (family, workload_name.replace("+", "_")))


def workload_name(cfg_name, decay, variant):
    return cfg_name + ("+c2" if variant == "c2" else "") + ("+logdecay" if decay == "log" else "")


# sources behind each family of traffic records: the kernel, and for the
# chunked scan the host plan that sizes its segments
KERNEL_SOURCES = {
    "wkv_call": ("linear_attention_rnn_finch_amd/csrc/wkv_chunk.hip",
                 "linear_attention_rnn_finch_amd/csrc/wkv_api.cpp",
                 "linear_attention_rnn_finch_amd/csrc/wkv_plan.hip"),
    "wkv_decode": ("linear_attention_rnn_finch_amd/csrc/wkv_decode.hip",),
    "epilogue": ("linear_attention_rnn_finch_amd/csrc/wkv_epilogue.hip",),
}


def kernel_source_digest(family):
    """SHA-256 over the family's sources (any change voids its records)."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[family]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload_name, kernel_name):
    """HBM bytes per launch of the main kernel recorded for this workload and
    this exact kernel source, else None."""
    try:
        text = open(traffic_file(workload_name, kernel_name)).read()
    except OSError:
        return None
    fields = {}
    for line in text.splitlines():
        if line.startswith("- ") and ": " in line:
            key, val = line[2:].split(": ", 1)
            fields[key.strip()] = val.strip().strip("`")
    if fields.get("workload") != workload_name:
        return None
    if fields.get("kernel_source_sha256") != kernel_source_digest(traffic_family(workload_name, kernel_name)):
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# Matrix-core work issued by the chunked path, counted from the kernels'
# instruction sequence: per workgroup and 64-token chunk the chunked scan
# issues 268 v_mfma_f32_16x16x32_bf16 (A tiles 10 x 2 K-steps x 3 split
# products = 60; read-out 4 waves x 4 x 2 x 3 = 96; state update 4 x 4 x 2 x 2
# = 64; in-chunk pairs 4 x 6 x 2 = 48) and the state pass 64 (4 x 4 x 2 x 2).
# The last chunk of a segment that does not end its sequence skips the state
# update (its end state is not used).
MFMA_FLOPS = 16 * 16 * 32 * 2
MAIN_MFMA_PER_CHUNK = 268
STATE_MFMA_PER_CHUNK = 64
BF16_MFMA_PEAK = 2.5e15          # MI355X dense bf16, FLOP/s


def _segment(lengths, H):
    up = lambda x, m: -(-x // m) * m
    tokens, max_len = sum(lengths), max(lengths) if lengths else 0
    return min(max(up(max(-(-tokens * H // 512), 1), 64), 256), up(max(max_len, 1), 64))


def whole_sequence_plan(lengths, H, packed):
    """Whether the library runs this bf16 call as whole sequences on its
    producer/consumer kernel: longer than 16 tokens, split by the segment
    plan, and at least 256 (sequence, head) pairs; a packed call also needs
    its longest sequence to be at most twice the mean work per CU (256)."""
    if not lengths or max(lengths) <= 16:
        return False
    split = -(-max(lengths) // _segment(lengths, H)) > 1
    if not split or len(lengths) * H < 256:
        return False
    return not packed or max(lengths) * 256 <= 2 * sum(lengths) * H


def pc_split_segment(lengths, H, packed):
    """Segment length when the library runs a split fixed-length bf16 call
    with fewer than 256 (sequence, head) pairs on its producer/consumer
    kernel (about 256 segments, at least 2 per sequence, each at least 2048
    tokens), else None."""
    if packed or not lengths or max(lengths) <= 16 or whole_sequence_plan(lengths, H, packed):
        return None
    T, B = max(lengths), len(lengths)
    if -(-T // _segment(lengths, H)) <= 1:
        return None                                     # not split
    pcs = max(2, 256 // (B * H))
    seg = -(-(-(-T // pcs)) // 64) * 64
    return seg if seg >= 2048 else None


def one_launch_plan(lengths, H, packed, capacity):
    """Whether the library runs this split bf16 call as one launch of its
    split kernel: segments of at most 1024 tokens, at most 4096 (sequence,
    head) pairs, and every state workgroup resident at once (`capacity`
    workgroups: compute units x 2)."""
    if not lengths or max(lengths) <= 16 or whole_sequence_plan(lengths, H, packed):
        return False
    if pc_split_segment(lengths, H, packed):
        return False
    seg = _segment(lengths, H)
    n_seg = sum(1 if L == 0 else -(-L // seg) for L in lengths)
    if n_seg == len(lengths):
        return False                                    # nothing is split
    return seg <= 1024 and len(lengths) * H <= 4096 and (n_seg - len(lengths)) * H <= capacity


def chunk_counts(lengths, H, packed=False):
    """(chunked-scan chunks, state-pass chunks, segments that do not end their
    sequence) of a bf16 call over sequences of these lengths, with the
    library's segment plan: about 512 (segment, head) items, segments a
    multiple of 64 tokens and at least 256, no longer than the longest sequence
    rounded up to 64.  A fixed-length call that this plan would split but that
    has at least 256 (sequence, head) pairs runs whole sequences instead (no
    state pass); one with fewer pairs whose producer/consumer segments would
    be at least 2048 tokens uses those segments."""
    if whole_sequence_plan(lengths, H, packed):
        return sum(-(-L // 64) for L in lengths) * H, 0, 0
    seg = pc_split_segment(lengths, H, packed) or _segment(lengths, H)
    main = state = inner = 0
    for L in lengths:
        P = 1 if L == 0 else -(-L // seg)
        main += -(-L // 64)
        if P > 1:
            state += (P - 1) * seg // 64
            inner += P - 1
    return main * H, state * H, inner * H


def time_calls(call, n, torch):
    """Average duration (ms) of whole calls from events recorded on the launch
    stream before and after each call (queued back to back behind a device
    sleep, so the events measure the GPU work, gaps between its kernels
    included)."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    torch.cuda.synchronize()
    torch.cuda._sleep(50_000_000)
    for a, b in evs:
        a.record()
        call()
        b.record()
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in evs) / n


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def copy_bandwidth(torch, mib=1024, reps=20):
    """Device-to-device copy rate (read + write bytes per second, GB/s)."""
    src = torch.empty(mib << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    del src, dst
    return 2 * (mib << 20) / (ms * 1e-3) / 1e9


def hip_runtime():
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                        ctypes.c_void_p]
    hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return hip


def time_main_kernel(call, n, hip, lib, torch):
    """Average and median duration (ms) of the main scan kernel over n calls,
    from the HIP events the library attaches to that kernel's launch (its own
    start and end timestamps).  A device-side sleep keeps the GPU busy while
    the host enqueues the calls, so they run back to back as in a step."""
    evs = []
    for _ in range(2 * n):
        e = ctypes.c_void_p()
        if hip.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        evs.append(e)
    torch.cuda.synchronize()
    torch.cuda._sleep(50_000_000)
    for i in range(n):
        lib.wkv_set_kernel_timing_events(evs[2 * i], evs[2 * i + 1])
        call()
    lib.wkv_set_kernel_timing_events(None, None)
    torch.cuda.synchronize()
    total = 0.0
    ms = ctypes.c_float()
    durations = []
    for i in range(n):
        hip.hipEventElapsedTime(ctypes.byref(ms), evs[2 * i], evs[2 * i + 1])
        durations.append(ms.value)
        total += ms.value
    for e in evs:
        hip.hipEventDestroy(e)
    durations.sort()
    return total / n, durations[len(durations) // 2]


def _time_oracle(wl, threads, target_seconds):
    import oracle
    passes, t0, out = 0, time.perf_counter(), None
    while True:
        out = oracle.wkv_scan(wl.r, wl.k, wl.v, wl.w, wl.u, wl.state0, wl.cu_seqlens,
                              threads=threads, decay=wl.decay, variant=wl.variant,
                              second_value=wl.u2)
        passes += 1
        el = time.perf_counter() - t0
        if el >= target_seconds or passes >= 100000:
            return passes, el, out


def cpu_baseline(wl, target_seconds):
    """Time the fp64 oracle on the host over whole passes of the workload (all
    slices), repeating until about target_seconds of work, on every thread of
    the process affinity mask and on one thread; returns the record and the
    oracle outputs of the last pass."""
    threads = len(os.sched_getaffinity(0))
    if os.environ.get("OMP_NUM_THREADS", "").isdigit():
        threads = min(threads, int(os.environ["OMP_NUM_THREADS"]))
    passes, el, out = _time_oracle(wl, threads, target_seconds)
    passes1, el1, _ = _time_oracle(wl, 1, target_seconds)
    tokens = wl.tokens * passes
    rec = {"value": tokens / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "sample": "%d full pass(es) of the %s workload (%d tokens x %d heads), fp64 "
                     "sequential recurrence, OpenMP over (sequence, head) slices, %.1f s; "
                     "one thread: %d pass(es) in %.1f s"
                     % (passes, workload_name(wl.config.name, wl.decay, wl.variant), wl.tokens,
                        wl.u.shape[0], el, passes1, el1),
           "value_1thread": wl.tokens * passes1 / el1,
           "cpu_model": cpu_model()}
    return rec, out


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="1", help="workload index or name (default: 1)")
    ap.add_argument("--kernel-samples", type=int, default=100)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="time eager calls instead of a graph replay (for profiler runs)")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="first run a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--decay", choices=("w", "log"), default="w",
                    help="decay input: w itself, or d with w = exp(-exp(d))")
    ap.add_argument("--variant", choices=("finch", "c2"), default="finch",
                    help="base Finch (static bonus) or the Finch-C2 time mixer")
    ap.add_argument("--rotate", type=int, default=0,
                    help="buffer sets the calls cycle through (0: enough for 1 GiB, at most 16)")
    ap.add_argument("--split-launches", type=int, choices=(1, 3), default=1,
                    help="launch form of split calls: 1 (the library's default: one launch where it "
                         "can) or 3 (state pass, segment scan, chunked scan), for comparison")
    ap.add_argument("--also", default="train_batch_b8_t4096",
                    help="with the default workload: also time this one (the metric's batch of "
                         "eight sequences at the same d_model and T) and report it beside the "
                         "headline; '' to skip")
    ap.add_argument("--op", choices=("wkv", "layernorm", "compress"), default="wkv",
                    help="the pre-fill scan (default), or one epilogue step on the 1.5B layer "
                         "shape: LayerNorm over heads, GOLD key compression")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.op != "wkv":
        return bench_epilogue(args)
    rec = bench_wkv(args, args.config)
    # the metric's other workload at d_model 2048, T = 4096 (the batch of
    # eight sequences), measured in the same process after the headline and
    # reported beside it; the headline value stays the one-sequence layer's
    if (args.also and rec["config"]["workload"] == "layer_1p5b_t4096"
            and args.decay == "w" and args.variant == "finch"):
        sub = argparse.Namespace(**vars(args))
        sub.no_cpu_baseline, sub.steps, sub.warmup, sub.rotate = True, 50, 5, 0
        other = bench_wkv(sub, args.also)
        rec["same_metric_other_shape"] = {
            "workload": other["config"]["workload"],
            "B": other["config"]["B"], "T": other["config"]["T"], "H": other["config"]["H"],
            "value": other["value"], "unit": other["unit"], "steps": sub.steps,
            "ms_per_step": other["ms_per_step"],
            "frac": other["roofline"]["frac"], "traffic": other["roofline"]["traffic"],
            "algorithmic_bytes_per_call": other["roofline"]["algorithmic_bytes_per_call"],
            "main_kernel": other["roofline"]["main_kernel"]}
    print(json.dumps(rec), flush=True)


def bench_wkv(args, config):
    """The pre-fill scan on one workload (name or index); returns the record."""
    import numpy as np
    import torch
    import linear_attention_rnn_finch_amd as fw
    from linear_attention_rnn_finch_amd import _binding
    from synth import make_workload, get_config, error_report

    fw.set_split_launches(args.split_launches)
    cfg = get_config(int(config) if config.isdigit() else config)
    wl = make_workload(cfg, decay=args.decay, variant=args.variant)
    name = workload_name(cfg.name, args.decay, args.variant)
    dev = torch.device("cuda", 0)

    def cvt(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    host = {n: getattr(wl, n) for n in ("r", "k", "v", "w", "u2")}
    u = None if args.variant == "c2" else torch.from_numpy(wl.u).to(dev)
    n_seq = wl.n_seq
    in_dtype = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    if wl.packed:
        cu = torch.from_numpy(wl.cu_seqlens.astype(np.int32)).to(dev)
        cu_host = torch.from_numpy(wl.cu_seqlens.astype(np.int32))
        o_shape = (wl.tokens, cfg.H, cfg.D)
        ws_bytes = fw.varlen_workspace_bytes(cu_host, cfg.H, cfg.D, in_dtype)
    else:
        o_shape = (cfg.B, cfg.T, cfg.H, cfg.D)
        ws_bytes = fw.workspace_bytes(cfg.B, cfg.T, cfg.H, cfg.D, in_dtype)
    elt = 2 if cfg.dtype == "bf16" else 4
    n_in = 5 if args.variant == "c2" else 4
    set_bytes = (wl.tokens * cfg.H * cfg.D * (n_in * elt + 4) + ws_bytes +
                 n_seq * cfg.H * cfg.D * cfg.D * 4 * (2 if wl.state0 is not None else 1))
    n_sets = args.rotate if args.rotate > 0 else max(1, min(16, -(-(1 << 30) // set_bytes)))

    def make_set():
        t = {n: (None if a is None else cvt(a)) for n, a in host.items()}
        t["s0"] = None if wl.state0 is None else torch.from_numpy(wl.state0).to(dev)
        t["o"] = torch.empty(o_shape, dtype=torch.float32, device=dev)
        t["st"] = torch.empty((n_seq, cfg.H, cfg.D, cfg.D), dtype=torch.float32, device=dev)
        t["ws"] = fw.new_workspace(ws_bytes, dev)
        return t

    sets = [make_set() for _ in range(n_sets)]
    turn = [0]

    def call():
        t = sets[turn[0] % n_sets]
        turn[0] += 1
        form = dict(decay=args.decay, variant=args.variant, second_value=t["u2"])
        if wl.packed:
            fw.prefill_varlen(t["r"], t["k"], t["v"], t["w"], u, cu, t["s0"], cu_seqlens_host=cu_host,
                              o=t["o"], state_out=t["st"], workspace=t["ws"], **form)
        else:
            fw.prefill(t["r"], t["k"], t["v"], t["w"], u, t["s0"], o=t["o"], state_out=t["st"],
                       workspace=t["ws"], **form)
        return t

    if args.copy_mb > 0:                          # known-size copy for counter scaling
        src = torch.empty(args.copy_mb << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # warm-up (eager)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()

    if args.no_graph:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            call()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    else:
        # capture K steps into one HIP graph on a side stream
        graph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            call()                               # first use on this stream
            torch.cuda.synchronize()
            with torch.cuda.graph(graph, stream=cap):
                for _ in range(args.steps):
                    call()
        torch.cuda.synchronize()
        graph.replay()                           # warm replay
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        graph.replay()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    max_len = int(np.diff(wl.cu_seqlens).max()) if wl.packed else cfg.T
    if max_len <= STEP_MAX_T and cfg.dtype == "bf16" and max_len >= 2:
        kernel_name = "wkv_steps_mfma_kernel"
    elif max_len <= STEP_MAX_T:
        kernel_name = "wkv_decode_kernel"
    elif cfg.dtype != "bf16":
        kernel_name = "wkv_serial_kernel"
    else:
        lens = [int(x) for x in np.diff(wl.cu_seqlens)] if wl.packed else [cfg.T] * cfg.B
        capacity = 2 * torch.cuda.get_device_properties(0).multi_processor_count
        kernel_name = ("wkv_chunk_pc_kernel" if whole_sequence_plan(lens, cfg.H, wl.packed)
                       or pc_split_segment(lens, cfg.H, wl.packed)
                       else "wkv_split_kernel" if args.split_launches == 1
                       and one_launch_plan(lens, cfg.H, wl.packed, capacity)
                       else "wkv_chunk_kernel")
    tokens_per_step = wl.tokens
    value = tokens_per_step / (ms_per_step * 1e-3)

    # durations measured live: the main kernel through the library's timing
    # hook (events attached to its own dispatch), the whole call with events
    # recorded on the launch stream around it
    hip = hip_runtime()
    lib = _binding._lib
    lib.wkv_set_kernel_timing_events.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    k_avg_ms, k_med_ms = time_main_kernel(call, args.kernel_samples, hip, lib, torch)
    c_avg_ms = time_calls(call, args.kernel_samples, torch)
    alg = algorithmic_bytes(cfg, wl.tokens, n_seq, wl.state0 is not None, args.variant)
    step_gbs = alg / (ms_per_step * 1e-3) / 1e9
    kernel_gbs = alg / (k_avg_ms * 1e-3) / 1e9
    copy_gbs = copy_bandwidth(torch)
    chunked = kernel_name in ("wkv_chunk_kernel", "wkv_chunk_pc_kernel", "wkv_split_kernel")
    lengths = [int(x) for x in np.diff(wl.cu_seqlens)] if wl.packed else [cfg.T] * cfg.B
    mfma = None
    if chunked:
        main_chunks, state_chunks, inner = chunk_counts(lengths, cfg.H, packed=wl.packed)
        main_flops = MFMA_FLOPS * (MAIN_MFMA_PER_CHUNK * main_chunks - STATE_MFMA_PER_CHUNK * inner)
        flops = main_flops + MFMA_FLOPS * STATE_MFMA_PER_CHUNK * state_chunks
        mfma = {"issued_flops_per_call": flops,
                "mfma_util": round(flops / (ms_per_step * 1e-3) / BF16_MFMA_PEAK, 4),
                "main_kernel_mfma_util": round(main_flops / (k_avg_ms * 1e-3) / BF16_MFMA_PEAK, 4)}

    rec = {
        "metric": METRIC if cfg.name == "layer_1p5b_t4096" else OTHER_METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": name, "B": cfg.B, "T": cfg.T, "H": cfg.H, "D": cfg.D,
                   "decay": args.decay, "variant": args.variant,
                   "d_model": cfg.H * cfg.D, "tokens": wl.tokens,
                   "timing": ("eager calls" if args.no_graph else
                              "HIP graph of %d captured calls, one replay" % args.steps),
                   "buffer_sets": n_sets,
                   "split_launches": args.split_launches},
        # the headline fraction is the whole pre-fill call's (every kernel of
        # the step, in the step time above); the main kernel's own figure is
        # kept beside it
        "roofline": {"bound": "hbm", "scope": "pre-fill call" + (
                         " (state pass, segment scan, chunked scan)" if kernel_name == "wkv_chunk_kernel"
                         and chunk_counts(lengths, cfg.H, packed=wl.packed)[1] > 0
                         else " (one kernel: state pass, segment scan and chunked scan as workgroup roles)"
                         if kernel_name == "wkv_split_kernel" else " (one kernel)"),
                     "achieved": round(step_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(step_gbs / HBM_PEAK_GBS, 4),
                     # the committed counter profiles cover the library's default launch form
                     "traffic": measured_traffic(name, kernel_name) if args.split_launches == 1 else None,
                     "algorithmic_bytes_per_call": alg,
                     "call_event_avg_us": round(c_avg_ms * 1e3, 2),
                     "measured_copy_GBps": round(copy_gbs, 1),
                     "frac_of_copy": round(step_gbs / copy_gbs, 4),
                     "main_kernel": {"kernel": kernel_name,
                                     "avg_us": round(k_avg_ms * 1e3, 2),
                                     "median_us": round(k_med_ms * 1e3, 2),
                                     "achieved": round(kernel_gbs, 1),
                                     "frac": round(kernel_gbs / HBM_PEAK_GBS, 4)}},
    }
    if mfma:
        rec["roofline"].update(mfma)

    if not args.no_cpu_baseline:
        cpu_rec, (o_ref, s_ref) = cpu_baseline(wl, args.cpu_seconds)
        rec["cpu_baseline"] = cpu_rec
        t = call()
        torch.cuda.synchronize()
        ro = error_report(t["o"].cpu().numpy(), o_ref, wl.cu_seqlens)
        rs = error_report(t["st"].cpu().numpy(), s_ref, kind="state")
        rec["parity"] = {
            "max_block_err_o": ro["block"], "max_block_err_state": rs["block"],
            "max_row_err_o": ro["row"], "max_row_err_state": rs["row"],
            "max_elem_err_floored_o": ro["elem_floored"],
            "tol": cfg.tolerance}
    return rec


def bench_epilogue(args):
    """One epilogue step on the 1.5B-class layer shape (4096 tokens, d_model
    2048): the LayerNorm over heads (fp32 in, bf16 out) or the GOLD key
    compression (bf16 in, fp32 out).  Same timing rules as the scan."""
    import numpy as np
    import torch
    import linear_attention_rnn_finch_amd as fw
    from linear_attention_rnn_finch_amd import _binding
    from synth import make_norm_inputs, make_compress_inputs, bf16_bits_to_f32

    tokens, width = 4096, 2048
    dev = torch.device("cuda", 0)

    def cvt(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    if args.op == "layernorm":
        x, gamma, beta = make_norm_inputs(tokens, width)
        name, kernel = "layernorm_heads_t4096_w2048", "layernorm_rows_kernel<bf16 out>"
        alg = tokens * width * (4 + 2) + 2 * width * 4
        set_bytes = tokens * width * 6
        dtype = "f32 in, bf16 out"
        g_d, b_d = cvt(gamma), cvt(beta)

        def make_set():
            return {"x": cvt(x), "y": torch.empty((tokens, width), dtype=torch.bfloat16, device=dev)}

        def run(t):
            fw.layernorm_heads(t["x"], g_d, b_d, 1e-5, out_dtype=torch.bfloat16, y=t["y"])

        def reference():
            from oracle import epilogue
            return epilogue.layernorm_heads(x, gamma, beta, 1e-5)

        def result(t):
            return bf16_bits_to_f32(t["y"].view(torch.int16).cpu().numpy().view(np.uint16))
    else:
        x, w = make_compress_inputs(tokens, width)
        name, kernel = "gold_compress_t4096_d2048", "gold_compress_kernel<f32 out>"
        n_out = width // 16
        alg = tokens * width * 2 + n_out * width * 2 + tokens * n_out * 4
        set_bytes = tokens * width * 2 + tokens * n_out * 4
        dtype = "bf16 in, fp32 accumulate and out"
        w_d = cvt(w)

        def make_set():
            return {"x": cvt(x), "c": torch.empty((tokens, n_out), dtype=torch.float32, device=dev)}

        def run(t):
            fw.gold_compress(t["x"], w_d, out_dtype=torch.float32, c=t["c"])

        def reference():
            from oracle import epilogue
            return epilogue.gold_compress(x, w)

        def result(t):
            return t["c"].cpu().numpy()

    n_sets = args.rotate if args.rotate > 0 else max(1, min(16, -(-(1 << 30) // set_bytes)))
    sets = [make_set() for _ in range(n_sets)]
    turn = [0]

    def call():
        t = sets[turn[0] % n_sets]
        turn[0] += 1
        run(t)
        return t

    if args.copy_mb > 0:                          # known-size copy for counter scaling
        src = torch.empty(args.copy_mb << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    if args.no_graph:
        t0 = time.perf_counter()
        for _ in range(args.steps):
            call()
        torch.cuda.synchronize()
    else:
        graph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            call()
            torch.cuda.synchronize()
            with torch.cuda.graph(graph, stream=cap):
                for _ in range(args.steps):
                    call()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        graph.replay()
        torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    hip = hip_runtime()
    lib = _binding._lib
    lib.wkv_set_kernel_timing_events.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    k_avg_ms, k_med_ms = time_main_kernel(call, args.kernel_samples, hip, lib, torch)
    achieved = alg / (k_avg_ms * 1e-3) / 1e9
    copy_gbs = copy_bandwidth(torch)
    rec = {
        "metric": OTHER_METRIC,
        "value": round(tokens / (ms_per_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": dtype, "data": "synthetic",
        "config": {"workload": name, "tokens": tokens, "d_model": width, "buffer_sets": n_sets,
                   "timing": ("eager calls" if args.no_graph else
                              "HIP graph of %d captured calls, one replay" % args.steps)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(name, kernel),
                     "kernel": kernel, "kernel_avg_us": round(k_avg_ms * 1e3, 2),
                     "kernel_median_us": round(k_med_ms * 1e3, 2),
                     "algorithmic_bytes_per_launch": alg,
                     "measured_copy_GBps": round(copy_gbs, 1),
                     "kernel_frac_of_copy": round(achieved / copy_gbs, 4)},
    }
    if args.op == "compress":
        flops = 2 * tokens * width * (width // 16)
        rec["roofline"]["flops_per_launch"] = flops
        rec["roofline"]["mfma_frac_bf16"] = round(flops / (k_avg_ms * 1e-3) / 2.5e15, 4)
    if not args.no_cpu_baseline:
        passes, t0, ref = 0, time.perf_counter(), None
        while True:
            ref = reference()
            passes += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds:
                break
        cores = 1
        if args.op == "compress":                 # the fp64 product runs on the BLAS thread pool
            try:
                from threadpoolctl import threadpool_info
                cores = max([p["num_threads"] for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
            except ImportError:
                cores = len(os.sched_getaffinity(0))
        rec["cpu_baseline"] = {"value": tokens * passes / el, "unit": "tokens/s", "cores": cores,
                               "kind": "oracle",
                               "sample": "%d full pass(es) of %s (%d tokens), fp64 numpy, %.1f s"
                                         % (passes, name, tokens, el)}
        t = call()
        torch.cuda.synchronize()
        got = result(t).astype(np.float64)
        rec["parity"] = {"max_row_err": float((np.abs(got - ref).max(-1) /
                                               np.abs(ref).max(-1)).max())}
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
