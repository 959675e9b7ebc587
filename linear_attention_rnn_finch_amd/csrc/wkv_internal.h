// Internal definitions shared by the host launcher and the gfx950 kernels of
// libfinch_wkv.  Not part of the public ABI (include/finch_wkv.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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
};

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
    float *o;                // [tokens, H, D]
    float *state_out;        // [n_seq, H, D, D] or null
    const void *u2;          // Finch-C2 second value [tokens, H, D], or null
};

// Form of the recurrence (compile-time switches of the kernels).
struct Variant {
    bool log_decay = false;  // decay input d_t, w_t = exp(-exp(d_t))
    bool c2 = false;         // Finch-C2: keys times (1 - w_t), no bonus, + u2
};

// Workspace views (fp32).  seg_state[item]: the segment's zero-start end state
// (D*D) followed by its total log2-decay per key channel (D).  seg_start[item]:
// the state entering the segment (D*D).
struct Workspace {
    float *seg_state;
    float *seg_start;
    int32_t *seg_off;
    int32_t *seg_seq;
};
constexpr int kSegStateFloats = kHeadDim * kHeadDim + kHeadDim;
constexpr int kSegStartFloats = kHeadDim * kHeadDim;

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
// bf16 path: state pass + segment scan (only when some sequence is split), then
// the main chunked scan.
hipError_t launch_segment_states(const Geometry &g, const Tensors &t, const Workspace &ws,
                                 Variant v, hipStream_t st);
hipError_t launch_chunked_main(const Geometry &g, const Tensors &t, const Workspace &ws,
                               Variant v, hipStream_t st, KernelTiming tm = {});
// epilogue of Finch-C2 pre-fill: LayerNorm over heads, GOLD key compression
hipError_t launch_layernorm_rows(const float *x, const float *gamma, const float *beta, float eps, void *y,
                                 bool out_bf16, int64_t rows, int width, hipStream_t st, KernelTiming tm = {});
hipError_t launch_gold_compress(const uint16_t *x, const uint16_t *w, void *c, bool out_bf16, int64_t M, int K,
                                int N, hipStream_t st, KernelTiming tm = {});
hipError_t launch_plan_varlen(const Geometry &g, int32_t *seg_off, int32_t *seg_seq,
                              hipStream_t st);

}  // namespace finch
