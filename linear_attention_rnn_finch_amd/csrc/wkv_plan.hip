// Ragged-batch launch planner (gfx950): turns the device copy of cu_seqlens
// into the segment tables the scan kernels decode their work item from.
//
// seg_off[n]  = first global segment of sequence n (exclusive prefix sum of
//               P_n = max(1, ceil(L_n / seg_len)); seg_off[N] = total)
// seg_seq[s]  = sequence owning global segment s, or -1 for every s the host
//               planned but the device offsets do not produce.
// seg_rank[r] = global segment that the chunked scan takes as its r-th
//               (segment, head) group when the host asks for an order (else
//               no table): longest first.  Every segment but the last of its
//               sequence has the full segment length and comes first, in
//               index order; the sequences' last segments follow, sorted by
//               length (longest first, ties by sequence), so that when there
//               are more work items than resident workgroups the long ones
//               start first and the short ones fill in at the end.  The sort
//               is a bitonic sort of at most kRankMaxSeqs keys in LDS.
// Offsets are clamped into [0, total_tokens] before use, so a device copy that
// disagrees with the host copy yields unspecified values but no access outside
// the caller's buffers.
#include "wkv_internal.h"

namespace finch {
namespace {

constexpr int kPlanThreads = 256;

__global__ __launch_bounds__(kPlanThreads) void wkv_plan_varlen_kernel(Geometry g, int32_t *seg_off,
                                                                      int32_t *seg_seq, int32_t *seg_rank) {
    __shared__ int32_t scan[kPlanThreads];
    __shared__ int32_t carry;
    __shared__ uint64_t keys[kRankMaxSeqs];        // last segments: (longest first, sequence) keys
    const int tid = threadIdx.x;
    const bool rank = seg_rank != nullptr && g.n_seq <= kRankMaxSeqs;
    for (int s = tid; s < g.n_seg; s += kPlanThreads) {
        seg_seq[s] = -1;
        if (rank) seg_rank[s] = -1;
    }
    if (rank)
        for (int i = tid; i < kRankMaxSeqs; i += kPlanThreads) keys[i] = ~0ull;
    if (tid == 0) carry = 0;
    __syncthreads();

    for (int base = 0; base < g.n_seq; base += kPlanThreads) {
        const int n = base + tid;
        int32_t P = 0;
        if (n < g.n_seq) {
            const int64_t c0 = clamp64(g.cu[n], 0, g.total_tokens);
            const int64_t c1 = clamp64(g.cu[n + 1], c0, g.total_tokens);
            const int64_t L = c1 - c0;
            P = L == 0 ? 1 : (int32_t)((L + g.seg_len - 1) / g.seg_len);
        }
        scan[tid] = P;
        __syncthreads();
        for (int d = 1; d < kPlanThreads; d <<= 1) {       // inclusive Hillis-Steele scan
            const int32_t add = tid >= d ? scan[tid - d] : 0;
            __syncthreads();
            scan[tid] += add;
            __syncthreads();
        }
        const int32_t first = carry + scan[tid] - P;
        if (n < g.n_seq) {
            seg_off[n] = first;
            for (int32_t p = 0; p < P; ++p)
                if (first + p < g.n_seg) seg_seq[first + p] = n;
            if (rank) {
                // full-length segments: ranks in index order (first - n of
                // them precede this sequence's); the last one gets a key
                for (int32_t p = 0; p + 1 < P; ++p)
                    if (first - n + p < g.n_seg && first + p < g.n_seg) seg_rank[first - n + p] = first + p;
                const int64_t c0 = clamp64(g.cu[n], 0, g.total_tokens);
                const int64_t c1 = clamp64(g.cu[n + 1], c0, g.total_tokens);
                const int64_t last = (c1 - c0) - (int64_t)(P - 1) * g.seg_len;   // in [0, seg_len]
                keys[n] = ((uint64_t)(uint32_t)(0x7FFFFFFF - (int32_t)last) << 32) | (uint32_t)n;
            }
        }
        __syncthreads();
        if (tid == kPlanThreads - 1) {
            carry += scan[tid];
            if (base + kPlanThreads >= g.n_seq) seg_off[g.n_seq] = carry;
        }
        __syncthreads();
    }
    if (!rank) return;

    // bitonic sort of the keys, ascending, over the smallest power of two
    // that holds them (unused slots hold the largest key)
    int width = 2;
    while (width < g.n_seq) width <<= 1;
    for (int k = 2; k <= width; k <<= 1)
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = tid; i < width; i += kPlanThreads) {
                const int l = i ^ j;
                if (l > i) {
                    const uint64_t a = keys[i], b = keys[l];
                    if (((i & k) == 0) == (a > b)) {
                        keys[i] = b;
                        keys[l] = a;
                    }
                }
            }
            __syncthreads();
        }
    // the last segments after every full-length one, in key order
    const int32_t full = carry - g.n_seq;
    for (int i = tid; i < g.n_seq; i += kPlanThreads) {
        const int n = (int)(uint32_t)keys[i];
        if (n < 0 || n >= g.n_seq) continue;
        const int32_t s = seg_off[n + 1] - 1;                // this sequence's last segment
        if (full + i < g.n_seg && s >= 0 && s < g.n_seg) seg_rank[full + i] = s;
    }
}

}  // namespace

hipError_t launch_plan_varlen(const Geometry &g, int32_t *seg_off, int32_t *seg_seq, int32_t *seg_rank,
                              hipStream_t st) {
    hipLaunchKernelGGL(wkv_plan_varlen_kernel, dim3(1), dim3(kPlanThreads), 0, st, g, seg_off,
                       seg_seq, seg_rank);
    return hipGetLastError();
}

}  // namespace finch
