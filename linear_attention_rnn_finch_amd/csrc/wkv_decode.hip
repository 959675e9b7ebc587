// Short-sequence (recurrent step) WKV kernel for gfx950: T <= kDecodeMaxT
// tokens per (sequence, head), the generation side of the pre-fill state
// (GoldFinch architecture summary, section 3.4 "Training and Inference
// Procedures": generation continues from the pre-filled recurrent state).
//
// Same recurrence as the other kernels (section 3.4, "Recurrent state update
// and output"), evaluated token by token in fp32:
//   o_t[j]  = sum_i r_t[i] S[i][j] + (r_t . u . k_t) v_t[j]      (base Finch)
//   o_t[j]  = sum_i r_t[i] S[i][j] + u'_t[j]                      (Finch-C2)
//   S[i][j] = w_t[i] S[i][j] + k_t[i] v_t[j]   (C2: k_t[i] (1 - w_t[i]))
// with w_t = exp(-exp(d_t)) when the decay is given as d.
//
// With a few tokens per call the 64x64 fp32 state (16 KB in, 16 KB out per
// (sequence, head)) is nearly all of the traffic, so the kernel is built to
// stream states: one wave per (sequence, head), lane j holding state column j
// in 64 registers (every state row is one coalesced 256-byte access), no
// workgroup barrier, and only 768 bytes of LDS per wave -- the token's r, k, w
// rows, broadcast to all lanes -- so that many waves per CU keep state loads
// in flight.
#include <hip/hip_ext.h>

#include "wkv_internal.h"

namespace finch {
namespace {

constexpr int kWavesPerBlock = 4;

__device__ inline float load_in(const float *p, size_t i) { return p[i]; }
__device__ inline float load_in(const uint16_t *p, size_t i) {
    return __uint_as_float((uint32_t)p[i] << 16);
}

__device__ inline float wave_sum(float x) {
    #pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
    return x;
}

template <typename In, bool LOGD, bool C2>
__global__ __launch_bounds__(256) void wkv_decode_kernel(Geometry g, Tensors t) {
    __shared__ float4 bc[kWavesPerBlock][3][kHeadDim / 4];   // r, k, w of the current token, per wave

    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int64_t item = (int64_t)blockIdx.x * kWavesPerBlock + wave;
    if (item >= (int64_t)g.n_seg * g.H) return;             // whole wave: no barrier below
    const int h = (int)(item % g.H);
    const ItemRange it = decode_segment(g, (int)(item / g.H));
    if (!it.valid) return;

    const In *rp = static_cast<const In *>(t.r);
    const In *kp = static_cast<const In *>(t.k);
    const In *vp = static_cast<const In *>(t.v);
    const In *wp = static_cast<const In *>(t.w);
    const In *u2p = static_cast<const In *>(t.u2);

    // lane = value column j; S[i] = S[i][j]
    float S[kHeadDim];
    const size_t so = ((size_t)it.n * g.H + h) * (kHeadDim * kHeadDim);
    #pragma unroll
    for (int i = 0; i < kHeadDim; ++i) S[i] = t.state_in ? t.state_in[so + i * kHeadDim + lane] : 0.f;
    const float u_lane = C2 ? 0.f : t.u[(size_t)h * kHeadDim + lane];
    float *row = reinterpret_cast<float *>(&bc[wave][0][0]);

    for (int64_t tt = it.t0; tt < it.t1; ++tt) {
        const size_t idx = ((size_t)tt * g.H + h) * kHeadDim + lane;
        // lane loads channel `lane` of each vector (key channel for r, k, w;
        // value channel for v)
        const float r = load_in(rp, idx);
        float k = load_in(kp, idx);
        const float v = load_in(vp, idx);
        const float x = load_in(wp, idx);
        const float e = LOGD ? expf(x) : 0.f;                   // exp(d)
        const float w = LOGD ? expf(-e) : x;
        if (C2) k *= LOGD ? -expm1f(-e) : 1.f - x;
        const float bonus = C2 ? 0.f : wave_sum(r * u_lane * k);
        // broadcast the key-side rows through LDS (one wave: program order is
        // enough; the reads of the previous token completed before these
        // writes were issued)
        row[lane] = r;
        row[kHeadDim + lane] = k;
        row[2 * kHeadDim + lane] = w;
        __builtin_amdgcn_wave_barrier();
        float o = 0.f;
        #pragma unroll
        for (int q = 0; q < kHeadDim / 4; ++q) {
            const float4 r4 = bc[wave][0][q];
            o += r4.x * S[4 * q] + r4.y * S[4 * q + 1] + r4.z * S[4 * q + 2] + r4.w * S[4 * q + 3];
        }
        o += C2 ? (u2p ? load_in(u2p, idx) : 0.f) : bonus * v;
        t.o[idx] = o;
        #pragma unroll
        for (int q = 0; q < kHeadDim / 4; ++q) {
            const float4 k4 = bc[wave][1][q];
            const float4 w4 = bc[wave][2][q];
            S[4 * q] = w4.x * S[4 * q] + k4.x * v;
            S[4 * q + 1] = w4.y * S[4 * q + 1] + k4.y * v;
            S[4 * q + 2] = w4.z * S[4 * q + 2] + k4.z * v;
            S[4 * q + 3] = w4.w * S[4 * q + 3] + k4.w * v;
        }
        __builtin_amdgcn_wave_barrier();
    }
    if (t.state_out && it.p == it.P - 1) {
        #pragma unroll
        for (int i = 0; i < kHeadDim; ++i) t.state_out[so + i * kHeadDim + lane] = S[i];
    }
}

template <typename In>
void (*decode_kernel_for(Variant v))(Geometry, Tensors) {
    if (v.log_decay)
        return v.c2 ? wkv_decode_kernel<In, true, true> : wkv_decode_kernel<In, true, false>;
    return v.c2 ? wkv_decode_kernel<In, false, true> : wkv_decode_kernel<In, false, false>;
}

}  // namespace

hipError_t launch_decode(const Geometry &g, const Tensors &t, bool bf16, Variant v, hipStream_t st,
                         KernelTiming tm) {
    const int64_t items = (int64_t)g.n_seg * g.H;
    if (items <= 0) return hipSuccess;
    const dim3 grid((unsigned)((items + kWavesPerBlock - 1) / kWavesPerBlock)), block(64 * kWavesPerBlock);
    if (bf16)
        hipExtLaunchKernelGGL(decode_kernel_for<uint16_t>(v), grid, block, 0, st, tm.start, tm.stop, 0, g, t);
    else
        hipExtLaunchKernelGGL(decode_kernel_for<float>(v), grid, block, 0, st, tm.start, tm.stop, 0, g, t);
    return hipGetLastError();
}

}  // namespace finch
