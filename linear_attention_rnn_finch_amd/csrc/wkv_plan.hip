// Ragged-batch launch planner (gfx950): turns the device copy of cu_seqlens
// into the segment tables the scan kernels decode their work item from.
//
// seg_off[n]  = first global segment of sequence n (exclusive prefix sum of
//               P_n = max(1, ceil(L_n / seg_len)); seg_off[N] = total)
// seg_seq[s]  = sequence owning global segment s, or -1 for every s the host
//               planned but the device offsets do not produce.
// Offsets are clamped into [0, total_tokens] before use, so a device copy that
// disagrees with the host copy yields unspecified values but no access outside
// the caller's buffers.
#include "wkv_internal.h"

namespace finch {
namespace {

constexpr int kPlanThreads = 256;

__global__ __launch_bounds__(kPlanThreads) void wkv_plan_varlen_kernel(Geometry g, int32_t *seg_off,
                                                                      int32_t *seg_seq) {
    __shared__ int32_t scan[kPlanThreads];
    __shared__ int32_t carry;
    const int tid = threadIdx.x;
    for (int s = tid; s < g.n_seg; s += kPlanThreads) seg_seq[s] = -1;
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
        }
        __syncthreads();
        if (tid == kPlanThreads - 1) {
            carry += scan[tid];
            if (base + kPlanThreads >= g.n_seq) seg_off[g.n_seq] = carry;
        }
        __syncthreads();
    }
}

}  // namespace

hipError_t launch_plan_varlen(const Geometry &g, int32_t *seg_off, int32_t *seg_seq,
                              hipStream_t st) {
    hipLaunchKernelGGL(wkv_plan_varlen_kernel, dim3(1), dim3(kPlanThreads), 0, st, g, seg_off,
                       seg_seq);
    return hipGetLastError();
}

}  // namespace finch
