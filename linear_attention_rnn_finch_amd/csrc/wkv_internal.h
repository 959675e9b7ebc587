// Internal definitions shared by the host launcher and the gfx950 kernels of
// libfinch_wkv.  Not part of the public ABI (include/finch_wkv.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include "finch_wkv.h"

namespace finch {

constexpr int kHeadDim = 64;     // D: the only head size the kernels are built for
constexpr int kChunk = 64;       // tokens per chunk of the chunked scan
constexpr int kDecodeMaxT = 16;  // calls whose sequences all have at most this many tokens take the step kernel
constexpr int kMaxNormWidth = 8192;   // widest row of the LayerNorm over heads (d_model)

// Geometry of one launch.  A "segment" is a run of at most seg_len tokens of
// one sequence; a work item is one (segment, head) pair and is processed by
// exactly one workgroup.  Items are numbered item = seg * H + h, where seg is
// the global segment index (sequence-major, then position in the sequence).
struct Geometry {
    int H;
    int n_seq;              // B or N
    int seg_len;            // tokens per segment (multiple of kChunk)
    int n_seg;              // global segment count (host-planned)
    int64_t total_tokens;   // rows of the packed token axis (bounds for every access)
    int uniform_T;          // >= 0: fixed-length batch of uniform_T tokens; -1: packed
    int segs_per_seq;       // fixed-length only: ceil(T / seg_len), at least 1
    const int32_t *cu;      // packed only: device offsets [n_seq + 1]
    const int32_t *seg_off; // packed only: device, first global segment of sequence n [n_seq + 1]
    const int32_t *seg_seq; // packed only: device, sequence of global segment s (-1: none) [n_seg]
    const int32_t *seg_rank;// packed only, or null: device, the global segment the chunked scan
                            // takes as its r-th (segment, head) group, longest first [n_seg]
    // fixed-length only: 1 when every (sequence, head) is one work item of
    // the producer/consumer kernel (no segments, no state pass), else 0
    int whole_seqs;
    // fixed-length only: 1 when the chunked scan of a split call runs on the
    // producer/consumer kernel (one workgroup per CU and long segment), else 0
    int pc_split;
    // state pass of the three-launch split: each segment that is not the last
    // of its sequence is covered by `runs` runs of run_len tokens (a multiple
    // of 64; the last run of a segment may be shorter), each a work item with
    // its own aggregate, which the segment scan chains in order
    int runs;
    int run_len;
    // one-launch split only: 1 when each workgroup takes the state role and
    // then the main role of its item (grid of items), 0 for the two-role grid
    // of 2 * items
    int relay;
    // one-launch split only: the bound of each wait, in ticks of the 100 MHz
    // clock (kDefaultWaitTicks unless a test shortens it)
    unsigned wait_ticks;
};
constexpr unsigned kDefaultWaitTicks = 1u << 27;   // ~1.3 s: a safety bound only

// One work item's token range and position inside its sequence.
struct ItemRange {
    int n;          // sequence
    int p;          // segment position in the sequence
    int P;          // segments of this sequence
    int64_t t0, t1; // token rows [t0, t1) of the packed axis
    bool valid;
};

__host__ __device__ inline int64_t clamp64(int64_t x, int64_t lo, int64_t hi) {
    return x < lo ? lo : (x > hi ? hi : x);
}

// Decode global segment `s` (device side).  Every range is clamped to
// [0, total_tokens] so inconsistent offsets can never address outside the
// caller's buffers.
__device__ inline ItemRange decode_segment(const Geometry &g, int s) {
    ItemRange it{};
    it.valid = false;
    if (s < 0 || s >= g.n_seg) return it;
    if (g.uniform_T >= 0) {
        it.n = s / g.segs_per_seq;
        it.p = s - it.n * g.segs_per_seq;
        it.P = g.segs_per_seq;
        int64_t base = (int64_t)it.n * g.uniform_T;
        int64_t a = (int64_t)it.p * g.seg_len;
        int64_t b = a + g.seg_len;
        if (b > g.uniform_T) b = g.uniform_T;
        it.t0 = base + a;
        it.t1 = base + b;
    } else {
        int n = g.seg_seq[s];
        if (n < 0 || n >= g.n_seq) return it;
        it.n = n;
        it.p = s - g.seg_off[n];
        it.P = g.seg_off[n + 1] - g.seg_off[n];
        if (it.p < 0 || it.p >= it.P) return it;
        int64_t c0 = g.cu[n], c1 = g.cu[n + 1];
        it.t0 = c0 + (int64_t)it.p * g.seg_len;
        it.t1 = it.t0 + g.seg_len;
        if (it.t1 > c1) it.t1 = c1;
    }
    it.t0 = clamp64(it.t0, 0, g.total_tokens);
    it.t1 = clamp64(it.t1, it.t0, g.total_tokens);
    it.valid = true;
    return it;
}

// Tensors of one call.  r, k, v, w (and u2) are bf16 bit patterns or fp32.
struct Tensors {
    const void *r, *k, *v, *w;   // w holds w_t, or d_t when the decay is given as d
    const float *u;          // [H, D] static bonus (base Finch; unused by Finch-C2)
    const float *state_in;   // [n_seq, H, D, D] or null
    void *o;                 // [tokens, H, D], fp32 or (o_bf16) bf16
    float *state_out;        // [n_seq, H, D, D] or null
    const void *u2;          // Finch-C2 second value [tokens, H, D], or null
    bool o_bf16;             // o is stored as bf16, rounded to nearest even
};

// Output stores shared by the scan kernels: fp32, or bf16 rounded to nearest
// even (the conversion instruction's rounding), chosen per call.
__device__ inline uint16_t bf16_rne_bits(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}
__device__ inline void store_o1(const Tensors &t, size_t idx, float x) {
    if (t.o_bf16)
        static_cast<uint16_t *>(t.o)[idx] = bf16_rne_bits(x);
    else
        static_cast<float *>(t.o)[idx] = x;
}
// four consecutive outputs starting at idx (a multiple of 4)
__device__ inline void store_o4(const Tensors &t, size_t idx, float4 x) {
    if (t.o_bf16) {
        const uint2 b = make_uint2((uint32_t)bf16_rne_bits(x.x) | ((uint32_t)bf16_rne_bits(x.y) << 16),
                                   (uint32_t)bf16_rne_bits(x.z) | ((uint32_t)bf16_rne_bits(x.w) << 16));
        *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(t.o) + idx) = b;
    } else {
        *reinterpret_cast<float4 *>(static_cast<float *>(t.o) + idx) = x;
    }
}

// Form of the recurrence (compile-time switches of the kernels).
struct Variant {
    bool log_decay = false;  // decay input d_t, w_t = exp(-exp(d_t))
    bool c2 = false;         // Finch-C2: keys times (1 - w_t), no bonus, + u2
    bool o_bf16 = false;     // o stored as bf16 (round to nearest even)
};

// Control record of one (sequence, head) for the one-launch split path: the
// workgroups of a call meet through these counters (agent-scope atomics),
// which waiters poll until they reach the number of workgroups counted.  The
// last main workgroup of the (sequence, head) to finish resets them to zero
// and advances the epoch, so a record is ready for the next call without any
// clearing.  A record must be zero before its first use.
struct SplitCtl {
    int epoch;      // calls that have completed on this record
    int done;       // main workgroups of later segments that have finished
    int arrived;    // state workgroups that have published their aggregate
    int scanned;    // state workgroups that have written their start-state slices
    int error;      // sticky: a bounded wait expired (results of that call are void)
    int pad[11];
};
static_assert(sizeof(SplitCtl) == 64, "one 64-byte record per (sequence, head)");
// records at the head of every split plan's workspace: calls with more
// (sequence, head) pairs take the three-launch path
constexpr int kCtlRecords = WKV_WORKSPACE_CONTROL_BYTES / (int)sizeof(SplitCtl);

// Workspace views (fp32).  seg_state[((s - n) * runs + r) * H + h]: the
// zero-start end state (D*D) of run r of global segment s of sequence n,
// followed by its total log2-decay per key channel (D); only segments that are
// not the last of their sequence have them, and s - n numbers those segments
// (runs = 1 in the one-launch kernel).  seg_start[item]: the state
// entering the segment (D*D).  ctl: the control records (one-launch path only,
// else null), record n * H + h.
struct Workspace {
    float *seg_state;
    float *seg_start;
    int32_t *seg_off;
    int32_t *seg_seq;
    SplitCtl *ctl;
};
constexpr int kSegStateFloats = kHeadDim * kHeadDim + kHeadDim;
constexpr int kSegStartFloats = kHeadDim * kHeadDim;
// threads the segment scan launches per (sequence, head)
constexpr int kScanGroupThreads = 1024;

// Launchers (defined in the .hip files).
// Scan kernels take an optional event pair: when set, the launch records the
// kernel's own start and end timestamps into them (profiling hook).
struct KernelTiming {
    hipEvent_t start = nullptr, stop = nullptr;
};

hipError_t launch_serial(const Geometry &g, const Tensors &t, bool bf16, Variant v, hipStream_t st,
                         KernelTiming tm = {});
// short sequences (at most kDecodeMaxT tokens each, never split; max_len the
// longest): one wave per (sequence, head), fp32 state in registers
hipError_t launch_decode(const Geometry &g, const Tensors &t, bool bf16, Variant v, int max_len, hipStream_t st,
                         KernelTiming tm = {});
// bf16 path: when some sequence is split (split), either one launch of the
// split kernel (ws.ctl set) or the state pass and the segment scan, then the
// chunked scan (the kernel the timing events attach to).
hipError_t launch_chunked(const Geometry &g, const Tensors &t, const Workspace &ws, bool split,
                          Variant v, hipStream_t st, KernelTiming tm = {});
// workgroups of the one-launch split kernel that the current device holds at
// once (compute units x resident workgroups per unit)
hipError_t split_launch_capacity(const Variant &v, bool relay, int64_t *capacity);
// epilogue of Finch-C2 pre-fill: LayerNorm over heads, GOLD key compression
hipError_t launch_layernorm_rows(const float *x, const float *gamma, const float *beta, float eps, void *y,
                                 bool out_bf16, int64_t rows, int width, hipStream_t st, KernelTiming tm = {});
hipError_t launch_gold_compress(const uint16_t *x, const uint16_t *w, void *c, bool out_bf16, int64_t M, int K,
                                int N, hipStream_t st, KernelTiming tm = {});
// packed calls of at most this many sequences can have their segments ranked
// longest first (seg_rank)
constexpr int kRankMaxSeqs = 1024;
hipError_t launch_plan_varlen(const Geometry &g, int32_t *seg_off, int32_t *seg_seq, int32_t *seg_rank,
                              hipStream_t st);

}  // namespace finch

#include "finch_wkv.h"

namespace finch {

// Host-side pieces of the C ABI (wkv_api.cpp) that other entry points share.
// A scratch source sets *out to device memory of at least `bytes` for the
// call and returns WKV_OK, or returns the error after recording why
// (record_error).
using ScratchSource = wkv_status_t (*)(size_t bytes, void **out);
wkv_status_t record_error(wkv_status_t st, const char *what);
// The fixed-length pre-fill of wkv_prefill_ex, with its scratch (if the plan
// needs any) taken from `scratch` once the arguments have been validated.
wkv_status_t prefill_fixed_from(const void *r, const void *k, const void *v, const void *w,
                                const float *u, const void *u2, const float *state_in, void *o,
                                float *state_out, int B, int T, int H, int D, wkv_dtype_t dt,
                                unsigned flags, ScratchSource scratch, void *stream);
// The static scratch of wkv_prefill_noalloc on the current device, or null
// when no such call has set it up there.
void *static_scratch_if_set();

}  // namespace finch
