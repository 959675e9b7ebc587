// C ABI of libfinch_wkv: argument validation, launch planning and kernel
// sequencing for the Finch WKV pre-fill.  See include/finch_wkv.h for the
// contract.
#include "finch_wkv.h"
#include "wkv_internal.h"

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

namespace finch {
namespace {

thread_local std::string g_last_error;
thread_local hipEvent_t g_ev_before = nullptr;   // optional timing of the main kernel
thread_local hipEvent_t g_ev_after = nullptr;
thread_local int g_split_launches = 1;           // 1: one launch where possible; 3: always three
thread_local unsigned g_wait_ticks = kDefaultWaitTicks;   // bound of the one launch's waits

wkv_status_t fail(wkv_status_t st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

wkv_status_t fail_hip(hipError_t e, const char *what) {
    return fail(WKV_EHIP, "%s: %s", what, hipGetErrorString(e));
}

// ---- planning -------------------------------------------------------------

// Work items the planner aims for: two resident 4-wave workgroups on each of
// the 256 compute units of an MI355X.
constexpr int64_t kTargetItems = 512;
// A bf16 call that the 4-wave kernel would split into segments runs whole
// sequences on the producer/consumer kernel (one 512-thread workgroup per
// compute unit) instead once it has this many (sequence, head) pairs.
// Measured at T = 4096, H = 32 per call: 262 -> 200 us at B = 8, 481 -> 344 us
// at B = 12; at B = 4 to 7 (which would still need segments) the 4-wave kernel
// with its state pass is as fast or faster, and from 512 pairs on it needs no
// segments.  A packed call also needs no sequence longer than twice the mean
// work per resident workgroup (16 ragged sequences, H = 32: 2314 -> 1862 us).
constexpr int64_t kWholeSeqItems = 256;
constexpr int64_t kWholeSeqSlots = 256;     // producer/consumer workgroups resident at once
// A fixed-length call with fewer pairs whose sequences are split runs its
// chunked scan on the producer/consumer kernel, with about kWholeSeqSlots
// segments, when those are at least this long (its pipeline needs many
// chunks per item: with 512-token segments at T = 4096, H = 32 it lost to
// the 4-wave kernel, 50.1 against 47.1 us).
constexpr int64_t kPcSplitSegment = 2048;
// the kernels address one 64-token chunk with 32-bit byte offsets:
// 64 rows x H heads x 256 B (fp32 o) must stay below 2^31
constexpr int kMaxHeads = 65536;
constexpr int64_t kMinSegment = 4 * kChunk;

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Segment length for a launch of `work` token-heads whose longest sequence
// has `max_len` tokens.  fp32 inputs are never split (their kernel is serial).
int64_t choose_segment(int64_t work, int64_t max_len, bool bf16) {
    if (!bf16) return std::max<int64_t>(round_up(std::max<int64_t>(max_len, 1), kChunk), kChunk);
    int64_t seg = round_up(std::max<int64_t>((work + kTargetItems - 1) / kTargetItems, 1), kChunk);
    seg = std::max(seg, kMinSegment);
    const int64_t whole = round_up(std::max<int64_t>(max_len, 1), kChunk);
    return std::min(seg, whole);
}

// Runs per segment for the state pass of a three-launch split: as many as
// bring its work items up to about three per compute unit (the state kernel's
// occupancy), with runs of at least four chunks.  Packed calls with a few long
// sequences otherwise leave most of the device idle in the state pass (16
// ragged sequences, 192 items of 333 chunks: 690 us at 2.3 TB/s).
constexpr int64_t kStateTargetItems = 768;
constexpr int64_t kMinRun = 4 * kChunk;
void choose_runs(Geometry &g) {
    g.runs = 1;
    g.run_len = g.seg_len;
    const int64_t items = (int64_t)(g.n_seg - g.n_seq) * g.H;
    if (items <= 0) return;
    int64_t r = std::min<int64_t>(kStateTargetItems / items, g.seg_len / kMinRun);
    if (r <= 1) return;
    const int64_t len = round_up((g.seg_len + r - 1) / r, kChunk);
    g.run_len = (int)len;
    g.runs = (int)((g.seg_len + len - 1) / len);
}

struct Plan {
    Geometry g{};
    int64_t max_len = 0;             // longest sequence of the call
    bool bf16 = false;
    bool split = false;              // some sequence has more than one segment
    size_t off_seg_state = 0, off_seg_start = 0, off_seg_off = 0, off_seg_seq = 0, off_seg_rank = 0;
    size_t bytes = 0;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

void layout_workspace(Plan &p, bool varlen) {
    size_t off = 0;
    const size_t items = (size_t)p.g.n_seg * p.g.H;
    // every nonzero workspace starts with the control records, so that calls
    // of any sizes can share one workspace without disturbing them
    if (p.split || varlen) off = WKV_WORKSPACE_CONTROL_BYTES;
    if (p.split) {
        p.off_seg_state = off;
        // aggregates only for segments that are not the last of their
        // sequence, one per state run
        const size_t aggs = (size_t)(p.g.n_seg - p.g.n_seq) * p.g.runs * p.g.H;
        off = align256(off + aggs * kSegStateFloats * sizeof(float));
        p.off_seg_start = off;
        off = align256(off + items * kSegStartFloats * sizeof(float));
    }
    if (varlen) {
        p.off_seg_off = off;
        off = align256(off + (size_t)(p.g.n_seq + 1) * sizeof(int32_t));
        p.off_seg_seq = off;
        off = align256(off + (size_t)p.g.n_seg * sizeof(int32_t));
        p.off_seg_rank = off;
        off = align256(off + (size_t)p.g.n_seg * sizeof(int32_t));
    }
    p.bytes = off;
}

wkv_status_t check_common(int H, int D, wkv_dtype_t dt) {
    if (dt != WKV_F32 && dt != WKV_BF16) return fail(WKV_EUNSUPPORTED, "unknown in_dtype %d", (int)dt);
    if (D != kHeadDim) return fail(WKV_EUNSUPPORTED, "head size D=%d unsupported (only %d)", D, kHeadDim);
    if (H < 1 || H > kMaxHeads) return fail(WKV_EINVAL, "H=%d must be in [1, %d]", H, kMaxHeads);
    return WKV_OK;
}

wkv_status_t plan_fixed(int B, int T, int H, int D, wkv_dtype_t dt, Plan &p) {
    if (wkv_status_t s = check_common(H, D, dt)) return s;
    if (B < 1) return fail(WKV_EINVAL, "B=%d must be >= 1", B);
    if (T < 0) return fail(WKV_EINVAL, "T=%d must be >= 0", T);
    const int64_t tokens = (int64_t)B * T;
    if (tokens > INT32_MAX) return fail(WKV_EINVAL, "B*T=%lld exceeds 2^31-1 tokens", (long long)tokens);
    p.bf16 = dt == WKV_BF16;
    const int64_t seg = choose_segment(tokens * H, T, p.bf16);
    const int64_t per = T == 0 ? 1 : (T + seg - 1) / seg;
    if ((int64_t)B * per * H > INT32_MAX) return fail(WKV_EINVAL, "too many work items");
    p.g.H = H;
    p.g.n_seq = B;
    p.g.seg_len = (int)seg;
    p.g.n_seg = (int)(B * per);
    p.g.total_tokens = tokens;
    p.g.uniform_T = T;
    p.g.segs_per_seq = (int)per;
    p.g.whole_seqs = 0;
    p.g.pc_split = 0;
    p.max_len = T;
    p.split = per > 1;
    if (p.bf16 && T > kDecodeMaxT && per > 1 && (int64_t)B * H >= kWholeSeqItems) {
        // enough (sequence, head) pairs for one producer/consumer workgroup per
        // CU: each runs a whole sequence, with no state pass and no scan
        p.g.whole_seqs = 1;
        p.split = false;
        p.g.seg_len = (int)round_up(T, kChunk);
        p.g.n_seg = B;
        p.g.segs_per_seq = 1;
    } else if (p.bf16 && T > kDecodeMaxT && per > 1) {
        // fewer pairs: long segments, about one per CU, on the
        // producer/consumer kernel, from the combined start states
        const int64_t pcs = std::max<int64_t>(2, kWholeSeqSlots / ((int64_t)B * H));
        const int64_t seg2 = round_up((T + pcs - 1) / pcs, kChunk);
        if (seg2 >= kPcSplitSegment) {
            const int64_t per2 = (T + seg2 - 1) / seg2;
            p.g.pc_split = 1;
            p.g.seg_len = (int)seg2;
            p.g.n_seg = (int)(B * per2);
            p.g.segs_per_seq = (int)per2;
        }
    }
    choose_runs(p.g);
    layout_workspace(p, false);
    return WKV_OK;
}

wkv_status_t plan_varlen(const int32_t *cu_host, int N, int H, int D, wkv_dtype_t dt, Plan &p) {
    if (wkv_status_t s = check_common(H, D, dt)) return s;
    if (N < 0) return fail(WKV_EINVAL, "N=%d must be >= 0", N);
    if (!cu_host) return fail(WKV_EINVAL, "cu_seqlens_host is NULL");
    if (cu_host[0] != 0) return fail(WKV_EINVAL, "cu_seqlens[0]=%d must be 0", cu_host[0]);
    int64_t max_len = 0;
    for (int n = 0; n < N; ++n) {
        if (cu_host[n + 1] < cu_host[n])
            return fail(WKV_EINVAL, "cu_seqlens decreases at %d (%d -> %d)", n, cu_host[n], cu_host[n + 1]);
        max_len = std::max<int64_t>(max_len, (int64_t)cu_host[n + 1] - cu_host[n]);
    }
    const int64_t tokens = cu_host[N];
    p.bf16 = dt == WKV_BF16;
    const int64_t seg = choose_segment(tokens * H, max_len, p.bf16);
    int64_t n_seg = 0;
    bool split = false;
    for (int n = 0; n < N; ++n) {
        const int64_t L = (int64_t)cu_host[n + 1] - cu_host[n];
        const int64_t P = L == 0 ? 1 : (L + seg - 1) / seg;
        split |= P > 1;
        n_seg += P;
    }
    if (n_seg * H > INT32_MAX) return fail(WKV_EINVAL, "too many work items");
    p.g.H = H;
    p.g.n_seq = N;
    p.g.seg_len = (int)seg;
    p.g.n_seg = (int)n_seg;
    p.g.total_tokens = tokens;
    p.g.uniform_T = -1;
    p.g.segs_per_seq = 0;
    p.g.whole_seqs = 0;
    p.g.pc_split = 0;
    p.max_len = max_len;
    p.split = split;
    if (p.bf16 && max_len > kDecodeMaxT && split && (int64_t)N * H >= kWholeSeqItems &&
        max_len * kWholeSeqSlots <= 2 * tokens * H) {
        // whole sequences on the producer/consumer kernel (one per CU, longest
        // first), as for fixed-length batches, when no sequence is longer
        // than twice the mean work per CU: no state pass and no scan
        p.g.whole_seqs = 1;
        p.split = false;
        p.g.seg_len = (int)round_up(max_len, kChunk);
        p.g.n_seg = N;
    }
    choose_runs(p.g);
    layout_workspace(p, true);
    return WKV_OK;
}

// A launch covers at most 2^32 - 1 work-items per grid dimension: every
// kernel a plan would launch is checked here, before anything is enqueued.
wkv_status_t check_grid(const Plan &p) {
    constexpr int64_t kMaxWorkItems = 0xFFFFFFFFll;
    const int64_t items = (int64_t)p.g.n_seg * p.g.H;           // one workgroup per (segment, head)
    const int64_t slices = (int64_t)p.g.n_seq * p.g.H;
    if (p.max_len <= kDecodeMaxT && !p.split) {                 // one wave per (sequence, head)
        if (slices * 64 > kMaxWorkItems)
            return fail(WKV_EUNSUPPORTED, "%lld (sequence, head) pairs exceed one launch", (long long)slices);
        return WKV_OK;
    }
    if (items * 256 > kMaxWorkItems)
        return fail(WKV_EUNSUPPORTED, "%lld work items exceed one launch", (long long)items);
    if (p.split && items * p.g.runs * 256 > kMaxWorkItems)                // state pass: one per run
        return fail(WKV_EUNSUPPORTED, "%lld state runs exceed one launch", (long long)(items * p.g.runs));
    if ((p.g.whole_seqs || p.g.pc_split) && items * 512 > kMaxWorkItems)   // 512 threads per item
        return fail(WKV_EUNSUPPORTED, "%lld work items exceed one launch", (long long)items);
    if (p.split && slices * kScanGroupThreads > kMaxWorkItems)
        return fail(WKV_EUNSUPPORTED, "%lld (sequence, head) pairs exceed the segment scan's launch",
                    (long long)slices);
    return WKV_OK;
}

// ---- pointer checks ---------------------------------------------------------

struct Range {
    const char *name;
    uintptr_t lo, hi;   // [lo, hi)
};

bool misaligned(const void *p, size_t a) { return p && ((uintptr_t)p % a) != 0; }

Range range_of(const char *name, const void *p, size_t bytes) {
    uintptr_t lo = (uintptr_t)p;
    return Range{name, lo, p ? lo + bytes : lo};
}

bool overlaps(const Range &a, const Range &b) {
    return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi;
}

wkv_status_t check_pointers(const Plan &p, const Variant &var, const void *r, const void *k,
                            const void *v, const void *w, const float *u, const void *u2,
                            const float *state_in, const void *o, const float *state_out,
                            const void *ws, size_t ws_bytes, const int32_t *cu_dev) {
    const int64_t tokens = p.g.total_tokens;
    const size_t elt = p.bf16 ? 2 : 4;
    const size_t in_bytes = (size_t)tokens * p.g.H * kHeadDim * elt;
    const size_t o_bytes = (size_t)tokens * p.g.H * kHeadDim * (var.o_bf16 ? 2 : 4);
    const size_t st_bytes = (size_t)p.g.n_seq * p.g.H * kHeadDim * kHeadDim * sizeof(float);
    if (var.c2) u = nullptr;                           // the bonus is not part of Finch-C2
    else if (u2) return fail(WKV_EINVAL, "second_value is only defined for the Finch-C2 variant");
    if (tokens > 0) {
        const void *need[] = {r, k, v, w, u, o};
        const char *names[] = {"r", "k", "v", "w", "u", "o"};
        for (int i = 0; i < 6; ++i)
            if (!need[i] && !(i == 4 && var.c2)) return fail(WKV_EINVAL, "%s is NULL", names[i]);
    }
    const void *al[] = {r, k, v, w, u, state_in, o, state_out, u2};
    const char *aln[] = {"r", "k", "v", "w", "u", "state_in", "o", "state_out", "second_value"};
    for (int i = 0; i < 9; ++i)
        if (misaligned(al[i], 16)) return fail(WKV_EINVAL, "%s is not 16-byte aligned", aln[i]);
    if (misaligned(cu_dev, 4)) return fail(WKV_EINVAL, "cu_seqlens_dev is not 4-byte aligned");
    if (misaligned(ws, 256)) return fail(WKV_EINVAL, "workspace is not 256-byte aligned");
    if (p.bytes > 0 && (!ws || ws_bytes < p.bytes))
        return fail(WKV_EWORKSPACE, "workspace of %zu bytes given, %zu needed", ws ? ws_bytes : 0,
                    p.bytes);

    const size_t n_cu = cu_dev ? (size_t)(p.g.n_seq + 1) * sizeof(int32_t) : 0;
    Range ins[] = {range_of("r", r, in_bytes), range_of("k", k, in_bytes),
                   range_of("v", v, in_bytes), range_of("w", w, in_bytes),
                   range_of("u", u, (size_t)p.g.H * kHeadDim * sizeof(float)),
                   range_of("second_value", u2, in_bytes),
                   range_of("state_in", state_in, state_in ? st_bytes : 0),
                   range_of("cu_seqlens_dev", cu_dev, n_cu),
                   range_of("workspace", ws, p.bytes)};
    Range outs[] = {range_of("o", o, o ? o_bytes : 0),
                    range_of("state_out", state_out, state_out ? st_bytes : 0)};
    for (const Range &out : outs) {
        for (const Range &in : ins) {
            if (out.name == std::string("state_out") && in.name == std::string("state_in") &&
                out.lo == in.lo)
                continue;                               // exact aliasing: carried state
            if (overlaps(out, in))
                return fail(WKV_EINVAL, "output %s overlaps %s", out.name, in.name);
        }
    }
    if (overlaps(outs[0], outs[1])) return fail(WKV_EINVAL, "o overlaps state_out");
    if (!cu_dev && p.g.uniform_T < 0) return fail(WKV_EINVAL, "cu_seqlens_dev is NULL");
    return WKV_OK;
}

// ---- execution --------------------------------------------------------------

// A split bf16 call with segments of at most kOneLaunchSegment tokens runs as
// one launch (wkv_split_kernel) when its (sequence, head) pairs have control
// records and all its state workgroups fit on the device at once (the
// condition under which its waits are safe); otherwise as the state pass, the
// segment scan and the chunked scan.  Measured per call, three launches -> one:
// segments of 256 tokens (T = 4096, H = 32) 47.4 -> 46.2 us, 512 (B = 2)
// 75.7 -> 73.8 us, 1024 (B = 4) 144.8 -> 138.0 us; 4096 (T = 65536) 543 -> 565
// us and 32768 (T = 262144, H = 64) 3.96 -> 4.45 ms.  With long segments the
// first segments' chunked scans, which start at once, take bandwidth from the
// state pass, and the kernel boundaries they save are a small share.
constexpr int64_t kOneLaunchSegment = 1024;

// The relay form (each workgroup the state role and then the main role of its
// item) needs every item resident at once; the two-role grid only the state
// workgroups.
enum class OneLaunch { kNone, kTwoRoles, kRelay };

wkv_status_t one_launch(const Plan &p, const Variant &var, OneLaunch *form) {
    *form = OneLaunch::kNone;
    if (!p.split || !p.bf16 || g_split_launches != 1) return WKV_OK;
    if (p.g.seg_len > kOneLaunchSegment) return WKV_OK;
    if ((int64_t)p.g.n_seq * p.g.H > kCtlRecords) return WKV_OK;
    const int64_t items = (int64_t)p.g.n_seg * p.g.H;
    if (2 * items * 256 > 0xFFFFFFFFll) return WKV_OK;
    int64_t capacity = 0;
    if (hipError_t e = split_launch_capacity(var, true, &capacity)) return fail_hip(e, "occupancy query");
    if (items <= capacity) {
        *form = OneLaunch::kRelay;
        return WKV_OK;
    }
    if (hipError_t e = split_launch_capacity(var, false, &capacity)) return fail_hip(e, "occupancy query");
    if ((int64_t)(p.g.n_seg - p.g.n_seq) * p.g.H <= capacity) *form = OneLaunch::kTwoRoles;
    return WKV_OK;
}

wkv_status_t run(const Plan &p, const Tensors &t, const Variant &var, void *ws, hipStream_t st) {
    Geometry g = p.g;
    g.wait_ticks = g_wait_ticks;
    char *base = static_cast<char *>(ws);
    hipError_t e;
    OneLaunch form = OneLaunch::kNone;
    if (wkv_status_t s = one_launch(p, var, &form)) return s;
    const bool fused = form != OneLaunch::kNone;
    if (g.uniform_T < 0) {
        if (!g.cu) return fail(WKV_EINVAL, "packed launch without device offsets");
        int32_t *seg_off = reinterpret_cast<int32_t *>(base + p.off_seg_off);
        int32_t *seg_seq = reinterpret_cast<int32_t *>(base + p.off_seg_seq);
        if (g.n_seq == 0) return WKV_OK;
        // longest first when the chunked scan has more work items than the
        // device holds at once (the short ones then fill in at the end)
        int32_t *seg_rank = nullptr;
        const int64_t resident = g.whole_seqs ? kWholeSeqSlots : kTargetItems;
        if (p.bf16 && !fused && p.max_len > kDecodeMaxT && g.n_seq <= kRankMaxSeqs &&
            (int64_t)g.n_seg * g.H > resident)
            seg_rank = reinterpret_cast<int32_t *>(base + p.off_seg_rank);
        if ((e = launch_plan_varlen(g, seg_off, seg_seq, seg_rank, st)) != hipSuccess)
            return fail_hip(e, "planner launch");
        g.seg_off = seg_off;
        g.seg_seq = seg_seq;
        g.seg_rank = seg_rank;
    }
    const KernelTiming tm{g_ev_before, g_ev_after};
    if (p.max_len <= kDecodeMaxT && !p.split) {       // recurrent steps: state-streaming kernel
        if ((e = launch_decode(g, t, p.bf16, var, (int)p.max_len, st, tm)) != hipSuccess) return fail_hip(e, "step launch");
        return WKV_OK;
    }
    if (!p.bf16) {
        if ((e = launch_serial(g, t, false, var, st, tm)) != hipSuccess) return fail_hip(e, "scan launch");
        return WKV_OK;
    }
    Workspace w{};
    if (p.split) {
        w.seg_state = reinterpret_cast<float *>(base + p.off_seg_state);
        w.seg_start = reinterpret_cast<float *>(base + p.off_seg_start);
        if (fused) {
            w.ctl = reinterpret_cast<SplitCtl *>(base);
            g.runs = 1;                                // its state role covers whole segments
            g.run_len = g.seg_len;
            g.relay = form == OneLaunch::kRelay;
        }
    }
    if ((e = launch_chunked(g, t, w, p.split, var, st, tm)) != hipSuccess) return fail_hip(e, "scan launch");
    return WKV_OK;
}

constexpr unsigned kKnownFlags = WKV_FLAG_DECAY_LOG | WKV_FLAG_FINCH_C2 | WKV_FLAG_OUT_BF16;

wkv_status_t variant_of(unsigned flags, Variant &v) {
    if (flags & ~kKnownFlags) return fail(WKV_EUNSUPPORTED, "unknown flags 0x%x", flags & ~kKnownFlags);
    v.log_decay = (flags & WKV_FLAG_DECAY_LOG) != 0;
    v.c2 = (flags & WKV_FLAG_FINCH_C2) != 0;
    v.o_bf16 = (flags & WKV_FLAG_OUT_BF16) != 0;
    return WKV_OK;
}

wkv_status_t prefill_fixed(const void *r, const void *k, const void *v, const void *w,
                           const float *u, const void *u2, const float *state_in, void *o,
                           float *state_out, int B, int T, int H, int D, wkv_dtype_t dt,
                           unsigned flags, void *ws, size_t ws_bytes, void *stream) {
    g_last_error.clear();
    Variant var;
    if (wkv_status_t s = variant_of(flags, var)) return s;
    Plan p;
    if (wkv_status_t s = plan_fixed(B, T, H, D, dt, p)) return s;
    if (wkv_status_t s = check_grid(p)) return s;
    if (wkv_status_t s = check_pointers(p, var, r, k, v, w, u, u2, state_in, o, state_out, ws,
                                        ws_bytes, nullptr))
        return s;
    Tensors t{r, k, v, w, var.c2 ? nullptr : u, state_in, o, state_out, u2, var.o_bf16};
    return run(p, t, var, ws, static_cast<hipStream_t>(stream));
}

wkv_status_t prefill_varlen(const void *r, const void *k, const void *v, const void *w,
                            const float *u, const void *u2, const int32_t *cu_dev,
                            const int32_t *cu_host, int N, const float *state_in, void *o,
                            float *state_out, int H, int D, wkv_dtype_t dt, unsigned flags,
                            void *ws, size_t ws_bytes, void *stream) {
    g_last_error.clear();
    Variant var;
    if (wkv_status_t s = variant_of(flags, var)) return s;
    Plan p;
    if (wkv_status_t s = plan_varlen(cu_host, N, H, D, dt, p)) return s;
    if (wkv_status_t s = check_grid(p)) return s;
    if (N > 0 && !cu_dev) return fail(WKV_EINVAL, "cu_seqlens_dev is NULL");
    if (wkv_status_t s = check_pointers(p, var, r, k, v, w, u, u2, state_in, o, state_out, ws,
                                        ws_bytes, cu_dev))
        return s;
    p.g.cu = cu_dev;
    Tensors t{r, k, v, w, var.c2 ? nullptr : u, state_in, o, state_out, u2, var.o_bf16};
    return run(p, t, var, ws, static_cast<hipStream_t>(stream));
}

}  // namespace

wkv_status_t record_error(wkv_status_t st, const char *what) { return fail(st, "%s", what); }

wkv_status_t prefill_fixed_from(const void *r, const void *k, const void *v, const void *w,
                                const float *u, const void *u2, const float *state_in, void *o,
                                float *state_out, int B, int T, int H, int D, wkv_dtype_t dt,
                                unsigned flags, ScratchSource scratch, void *stream) {
    g_last_error.clear();
    Variant var;
    if (wkv_status_t s = variant_of(flags, var)) return s;
    Plan p;
    if (wkv_status_t s = plan_fixed(B, T, H, D, dt, p)) return s;
    if (wkv_status_t s = check_grid(p)) return s;
    void *ws = nullptr;
    if (p.bytes > 0) {
        // pointers are checked first with a stand-in scratch range that cannot
        // overlap anything, so that no HIP call is made for an invalid call
        if (wkv_status_t s = check_pointers(p, var, r, k, v, w, u, u2, state_in, o, state_out, nullptr,
                                            0, nullptr);
            s != WKV_OK && s != WKV_EWORKSPACE)
            return s;
        g_last_error.clear();
        if (wkv_status_t s = scratch(p.bytes, &ws)) return s;
    }
    if (wkv_status_t s = check_pointers(p, var, r, k, v, w, u, u2, state_in, o, state_out, ws,
                                        p.bytes, nullptr))
        return s;
    Tensors t{r, k, v, w, var.c2 ? nullptr : u, state_in, o, state_out, u2, var.o_bf16};
    return run(p, t, var, ws, static_cast<hipStream_t>(stream));
}

}  // namespace finch

using namespace finch;

extern "C" {

int wkv_abi_version(void) { return FINCH_WKV_ABI_VERSION; }

const char *wkv_status_string(wkv_status_t s) {
    switch (s) {
    case WKV_OK: return "success";
    case WKV_EINVAL: return "invalid argument";
    case WKV_EUNSUPPORTED: return "unsupported size or dtype";
    case WKV_EWORKSPACE: return "workspace missing or too small";
    case WKV_EHIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char *wkv_last_error(void) { return g_last_error.c_str(); }

wkv_status_t wkv_set_kernel_timing_events(void *before, void *after) {
    g_ev_before = static_cast<hipEvent_t>(before);
    g_ev_after = static_cast<hipEvent_t>(after);
    return WKV_OK;
}

wkv_status_t wkv_set_split_launches(int launches) {
    if (launches != 1 && launches != 3) return fail(WKV_EINVAL, "launches=%d must be 1 or 3", launches);
    g_split_launches = launches;
    return WKV_OK;
}

wkv_status_t wkv_set_wait_bound(unsigned long long ticks) {
    if (ticks > 0xFFFFFFFFull) return fail(WKV_EINVAL, "ticks=%llu exceeds 2^32 - 1", ticks);
    g_wait_ticks = ticks == 0 ? kDefaultWaitTicks : (unsigned)ticks;
    return WKV_OK;
}

size_t wkv_prefill_workspace_bytes(int B, int T, int H, int D, wkv_dtype_t dt) {
    Plan p;
    std::string keep = g_last_error;
    size_t bytes = plan_fixed(B, T, H, D, dt, p) == WKV_OK ? p.bytes : 0;
    g_last_error = keep;
    return bytes;
}

size_t wkv_prefill_varlen_workspace_bytes(const int32_t *cu_host, int N, int H, int D,
                                          wkv_dtype_t dt) {
    Plan p;
    std::string keep = g_last_error;
    size_t bytes = plan_varlen(cu_host, N, H, D, dt, p) == WKV_OK ? p.bytes : 0;
    g_last_error = keep;
    return bytes;
}

wkv_status_t wkv_prefill(const void *r, const void *k, const void *v, const void *w,
                         const float *u, const float *state_in, float *o, float *state_out,
                         int B, int T, int H, int D, wkv_dtype_t dt, void *ws, size_t ws_bytes,
                         void *stream) {
    return prefill_fixed(r, k, v, w, u, nullptr, state_in, o, state_out, B, T, H, D, dt, 0u, ws,
                         ws_bytes, stream);
}

wkv_status_t wkv_prefill_ex(const void *r, const void *k, const void *v, const void *w,
                            const float *u, const void *u2, const float *state_in, void *o,
                            float *state_out, int B, int T, int H, int D, wkv_dtype_t dt,
                            unsigned flags, void *ws, size_t ws_bytes, void *stream) {
    return prefill_fixed(r, k, v, w, u, u2, state_in, o, state_out, B, T, H, D, dt, flags, ws,
                         ws_bytes, stream);
}

wkv_status_t wkv_prefill_varlen(const void *r, const void *k, const void *v, const void *w,
                                const float *u, const int32_t *cu_dev, const int32_t *cu_host,
                                int N, const float *state_in, float *o, float *state_out, int H,
                                int D, wkv_dtype_t dt, void *ws, size_t ws_bytes, void *stream) {
    return prefill_varlen(r, k, v, w, u, nullptr, cu_dev, cu_host, N, state_in, o, state_out, H,
                          D, dt, 0u, ws, ws_bytes, stream);
}

wkv_status_t wkv_layernorm_heads(const float *x, const float *gamma, const float *beta, float eps,
                                 void *y, wkv_dtype_t out_dtype, int64_t tokens, int width,
                                 void *stream) {
    g_last_error.clear();
    if (out_dtype != WKV_F32 && out_dtype != WKV_BF16)
        return fail(WKV_EUNSUPPORTED, "unknown out_dtype %d", (int)out_dtype);
    if (width < 1024 || width > kMaxNormWidth || width % 1024 != 0)
        return fail(WKV_EUNSUPPORTED, "width=%d must be a multiple of 1024 in [1024, %d]", width, kMaxNormWidth);
    if (tokens < 0) return fail(WKV_EINVAL, "tokens=%lld must be >= 0", (long long)tokens);
    if (!(eps >= 0.f) || eps > 1e30f) return fail(WKV_EINVAL, "eps must be finite and >= 0");
    if (tokens == 0) return WKV_OK;
    const void *need[] = {x, gamma, beta, y};
    const char *names[] = {"x", "gamma", "beta", "y"};
    for (int i = 0; i < 4; ++i) {
        if (!need[i]) return fail(WKV_EINVAL, "%s is NULL", names[i]);
        if (misaligned(need[i], 16)) return fail(WKV_EINVAL, "%s is not 16-byte aligned", names[i]);
    }
    const size_t n = (size_t)tokens * width;
    const Range out = range_of("y", y, n * (out_dtype == WKV_BF16 ? 2 : 4));
    const Range ins[] = {range_of("x", x, n * 4), range_of("gamma", gamma, (size_t)width * 4),
                         range_of("beta", beta, (size_t)width * 4)};
    for (const Range &in : ins)
        if (overlaps(out, in)) return fail(WKV_EINVAL, "output y overlaps %s", in.name);
    const KernelTiming tm{g_ev_before, g_ev_after};
    if (hipError_t e = launch_layernorm_rows(x, gamma, beta, eps, y, out_dtype == WKV_BF16, tokens, width,
                                             static_cast<hipStream_t>(stream), tm))
        return fail_hip(e, "layernorm launch");
    return WKV_OK;
}

wkv_status_t wkv_gold_compress(const void *x, const void *w_kd, void *c, wkv_dtype_t out_dtype,
                               int64_t tokens, int d_model, void *stream) {
    g_last_error.clear();
    if (out_dtype != WKV_F32 && out_dtype != WKV_BF16)
        return fail(WKV_EUNSUPPORTED, "unknown out_dtype %d", (int)out_dtype);
    if (d_model < 1024 || d_model > 65536 || d_model % 1024 != 0)
        return fail(WKV_EUNSUPPORTED, "d_model=%d must be a multiple of 1024 in [1024, 65536]", d_model);
    if (tokens < 0 || tokens > INT32_MAX) return fail(WKV_EINVAL, "tokens=%lld out of range", (long long)tokens);
    if (tokens == 0) return WKV_OK;
    const void *need[] = {x, w_kd, c};
    const char *names[] = {"x", "w_kd", "c"};
    for (int i = 0; i < 3; ++i) {
        if (!need[i]) return fail(WKV_EINVAL, "%s is NULL", names[i]);
        if (misaligned(need[i], 16)) return fail(WKV_EINVAL, "%s is not 16-byte aligned", names[i]);
    }
    const int n_out = d_model / 16;
    const Range out = range_of("c", c, (size_t)tokens * n_out * (out_dtype == WKV_BF16 ? 2 : 4));
    const Range ins[] = {range_of("x", x, (size_t)tokens * d_model * 2),
                         range_of("w_kd", w_kd, (size_t)n_out * d_model * 2)};
    for (const Range &in : ins)
        if (overlaps(out, in)) return fail(WKV_EINVAL, "output c overlaps %s", in.name);
    const KernelTiming tm{g_ev_before, g_ev_after};
    if (hipError_t e = launch_gold_compress(static_cast<const uint16_t *>(x), static_cast<const uint16_t *>(w_kd),
                                            c, out_dtype == WKV_BF16, tokens, d_model, n_out,
                                            static_cast<hipStream_t>(stream), tm))
        return fail_hip(e, "compression launch");
    return WKV_OK;
}

wkv_status_t wkv_prefill_varlen_ex(const void *r, const void *k, const void *v, const void *w,
                                   const float *u, const void *u2, const int32_t *cu_dev,
                                   const int32_t *cu_host, int N, const float *state_in,
                                   void *o, float *state_out, int H, int D, wkv_dtype_t dt,
                                   unsigned flags, void *ws, size_t ws_bytes, void *stream) {
    return prefill_varlen(r, k, v, w, u, u2, cu_dev, cu_host, N, state_in, o, state_out, H, D,
                          dt, flags, ws, ws_bytes, stream);
}

}  // extern "C"
