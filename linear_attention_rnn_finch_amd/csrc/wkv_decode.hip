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
// stream states: one wave per (sequence, head), no LDS and no workgroup
// barrier.  Lane (g, c) = 16 g + c holds the 16 x 4 state tile S[16g..16g+15]
// [4c..4c+3] in 64 registers, so each state row of the tile is a 16-byte
// access and every state access of the wave covers whole 256-byte rows.  The
// key-side values r_t[i], k_t[i], w_t[i] arrive with lane = channel i; lane
// 16g + m holds key channel 16g + m, so the values a tile row needs are DPP
// broadcasts inside the lane's own 16-lane row.  The readout's partial sums
// over the four row groups are reduced with the row-swapping permutes, leaving
// output column 4c + g in lane 16g + c.  Token inputs are fetched a few tokens
// ahead of the arithmetic.
#include <hip/hip_ext.h>

#include "wkv_internal.h"

namespace finch {
namespace {

constexpr int kWavesPerBlock = 4;
constexpr int kAhead = 4;   // tokens whose inputs are in flight ahead of the one computed

__device__ inline float to_f32(float x) { return x; }
__device__ inline float to_f32(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }

// Inputs of one token for this lane: channel `lane` of r, k and the decay
// input; value channels 4c..4c+3 of v; the second value (Finch-C2) at the
// lane's output channel.
template <typename In>
struct Tok {
    In r, k, x, u2 = In(0);
    In v[4];
};

template <typename In, bool C2>
__device__ __forceinline__ Tok<In> load_tok(const Tensors &t, size_t row, int lane, int col, int jo) {
    Tok<In> a;
    a.r = static_cast<const In *>(t.r)[row + lane];
    a.k = static_cast<const In *>(t.k)[row + lane];
    a.x = static_cast<const In *>(t.w)[row + lane];
    const In *vp = static_cast<const In *>(t.v) + row + 4 * col;
    if constexpr (sizeof(In) == 2) {
        const uint2 q = *reinterpret_cast<const uint2 *>(vp);
        a.v[0] = (uint16_t)(q.x & 0xffffu);
        a.v[1] = (uint16_t)(q.x >> 16);
        a.v[2] = (uint16_t)(q.y & 0xffffu);
        a.v[3] = (uint16_t)(q.y >> 16);
    } else {
        const float4 q = *reinterpret_cast<const float4 *>(vp);
        a.v[0] = q.x; a.v[1] = q.y; a.v[2] = q.z; a.v[3] = q.w;
    }
    // without a second value the load reads v instead (same row, always in
    // bounds) and the caller scales it by zero: no branch in the load stream
    if constexpr (C2) a.u2 = static_cast<const In *>(t.u2 ? t.u2 : t.v)[row + jo];
    return a;
}

// Value of lane N of this lane's 16-lane row (DPP row_newbcast; every lane
// has a source, so no fallback value is needed and the move can fold into its
// consumer).
template <int N>
__device__ __forceinline__ float row_bcast(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x150 + N, 0xF, 0xF, true));
}

// Sum over all 64 lanes, in every lane: prefix sums inside each 16-lane row
// (DPP row shifts), the row total broadcast from the row's last lane, then the
// row-swapping permutes across the four rows.
__device__ __forceinline__ float wave_sum(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x111, 0xF, 0xF, true));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x112, 0xF, 0xF, true));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x114, 0xF, 0xF, true));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x118, 0xF, 0xF, true));
    x = row_bcast<15>(x);
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Pairwise reduce-scatter across lane and lane ^ 32 (permlane32_swap): lanes
// 0..31 return the sum of `a`, lanes 32..63 the sum of `b`.  Same across lane
// and lane ^ 16 with permlane16_swap (even rows: `a`, odd rows: `b`).
__device__ __forceinline__ float split32(float a, float b) {
    const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}
__device__ __forceinline__ float split16(float a, float b) {
    const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// Readout partials p[e] += sum over the tile's 16 rows m of r[16g+m] S[m][e].
template <int M>
__device__ __forceinline__ void readout_rows(const float4 (&S)[16], float r, float (&p)[4]) {
    if constexpr (M < 16) {
        const float rb = row_bcast<M>(r);
        p[0] += rb * S[M].x;
        p[1] += rb * S[M].y;
        p[2] += rb * S[M].z;
        p[3] += rb * S[M].w;
        readout_rows<M + 1>(S, r, p);
    }
}

// S[m][e] = w[16g+m] S[m][e] + k[16g+m] v[e] over the tile's 16 rows.
template <int M>
__device__ __forceinline__ void update_rows(float4 (&S)[16], float w, float k, const float (&v)[4]) {
    if constexpr (M < 16) {
        // in place (scale, then accumulate) so that the state never changes
        // registers and both operations take the broadcast as a DPP operand
        const float wb = row_bcast<M>(w);
        const float kb = row_bcast<M>(k);
        S[M].x = fmaf(kb, v[0], S[M].x * wb);
        S[M].y = fmaf(kb, v[1], S[M].y * wb);
        S[M].z = fmaf(kb, v[2], S[M].z * wb);
        S[M].w = fmaf(kb, v[3], S[M].w * wb);
        update_rows<M + 1>(S, w, k, v);
    }
}

// One (sequence, head) item of a wave: its token range, head, token count and
// the offset of this lane's state tile.
struct Item {
    ItemRange it;
    int h = 0;
    int nt = 0;        // tokens (0: an empty sequence)
    bool ok = false;   // a real item (its state is read and written)
    size_t tile = 0;
};

__device__ __forceinline__ Item item_at(const Geometry &g, int64_t item, int grp, int col) {
    Item a;
    if (item < (int64_t)g.n_seg * g.H) {
        a.h = (int)(item % g.H);
        a.it = decode_segment(g, (int)(item / g.H));
        a.ok = a.it.valid;
        if (a.ok) {
            a.nt = (int)(a.it.t1 - a.it.t0);
            a.tile = ((size_t)a.it.n * g.H + a.h) * (kHeadDim * kHeadDim) + (size_t)(16 * grp) * kHeadDim + 4 * col;
        }
    }
    return a;
}

__device__ __forceinline__ void load_state(const Tensors &t, const Item &a, float4 (&S)[16]) {
    if (t.state_in && a.ok) {
        #pragma unroll
        for (int m = 0; m < 16; ++m) S[m] = *reinterpret_cast<const float4 *>(t.state_in + a.tile + m * kHeadDim);
    } else {
        #pragma unroll
        for (int m = 0; m < 16; ++m) S[m] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
}

__device__ __forceinline__ void store_state(const Tensors &t, const Item &a, const float4 (&S)[16]) {
    if (t.state_out && a.ok && a.it.p == a.it.P - 1) {
        #pragma unroll
        for (int m = 0; m < 16; ++m) *reinterpret_cast<float4 *>(t.state_out + a.tile + m * kHeadDim) = S[m];
    }
}

// Row (token, head) offset of token q of item a (a.nt > 0).  Past the item's
// last token the row is clamped to it: look-ahead loads never leave the item.
__device__ __forceinline__ size_t token_row(const Geometry &g, const Item &a, int q) {
    return ((size_t)(a.it.t0 + (q < a.nt ? q : a.nt - 1)) * g.H + a.h) * kHeadDim;
}

// One token of item a (state S): output row and state update.
template <typename In, bool LOGD, bool C2>
__device__ __forceinline__ void step_token(const Tensors &t, const Tok<In> &cur, size_t row, float u_lane,
                                           float u2_scale, int grp, int jo, float4 (&S)[16]) {
    const float r = to_f32(cur.r), x = to_f32(cur.x);
    float k = to_f32(cur.k);
    const float v[4] = {to_f32(cur.v[0]), to_f32(cur.v[1]), to_f32(cur.v[2]), to_f32(cur.v[3])};
    const float e = LOGD ? expf(x) : 0.f;           // exp(d)
    const float w = LOGD ? expf(-e) : x;
    if (C2) k *= LOGD ? -expm1f(-e) : 1.f - x;
    float p[4] = {0.f, 0.f, 0.f, 0.f};
    readout_rows<0>(S, r, p);
    if (!C2) {
        // bonus (r . u . k) v: added once, by the lanes of row group 0
        const float b = wave_sum(r * u_lane * k);
        const float bg = grp == 0 ? b : 0.f;
        #pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) p[e4] += bg * v[e4];
    }
    // lanes of groups 0,1 keep columns e = 0,1, groups 2,3 keep e = 2,3; then
    // even groups keep the first of the two: column 4c + g
    const float q0 = split32(p[0], p[2]);
    const float q1 = split32(p[1], p[3]);
    float o = split16(q0, q1);
    if (C2) o += u2_scale * to_f32(cur.u2);
    t.o[row + jo] = o;
    update_rows<0>(S, w, k, v);
}

// MaxT: the most tokens any item of the launch has (1 or kDecodeMaxT).  The
// token look-ahead covers up to kAhead tokens.
template <typename In, bool LOGD, bool C2, int MaxT>
__global__ __launch_bounds__(64 * kWavesPerBlock, 4) void wkv_decode_kernel(Geometry g, Tensors t) {
    constexpr int Ahead = MaxT < kAhead ? MaxT : kAhead;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: item math on the scalar unit
    const int lane = threadIdx.x & 63;
    const int grp = lane >> 4, col = lane & 15;
    const int jo = 4 * col + grp;                            // output channel of this lane
    const int64_t item = (int64_t)blockIdx.x * kWavesPerBlock + wave;
    if (item >= (int64_t)g.n_seg * g.H) return;             // whole wave: no barrier below
    const Item a = item_at(g, item, grp, col);
    if (!a.ok) return;

    float4 S[16];
    load_state(t, a, S);
    if (a.nt > 0) {
        const float u_lane = C2 ? 0.f : t.u[(size_t)a.h * kHeadDim + lane];
        const float u2_scale = t.u2 ? 1.f : 0.f;
        Tok<In> win[Ahead];
        #pragma unroll
        for (int q = 0; q < Ahead; ++q) win[q] = load_tok<In, C2>(t, token_row(g, a, q), lane, col, jo);
        #pragma unroll
        for (int q = 0; q < MaxT; ++q) {
            const Tok<In> cur = win[q % Ahead];
            if (q + Ahead < MaxT) win[q % Ahead] = load_tok<In, C2>(t, token_row(g, a, q + Ahead), lane, col, jo);
            if (q < a.nt) step_token<In, LOGD, C2>(t, cur, token_row(g, a, q), u_lane, u2_scale, grp, jo, S);
        }
    }
    store_state(t, a, S);
}

template <typename In, int MaxT>
void (*decode_kernel_for(Variant v))(Geometry, Tensors) {
    if (v.log_decay)
        return v.c2 ? wkv_decode_kernel<In, true, true, MaxT> : wkv_decode_kernel<In, true, false, MaxT>;
    return v.c2 ? wkv_decode_kernel<In, false, true, MaxT> : wkv_decode_kernel<In, false, false, MaxT>;
}

template <typename In>
void (*decode_kernel_for(Variant v, int max_len))(Geometry, Tensors) {
    return max_len <= 1 ? decode_kernel_for<In, 1>(v) : decode_kernel_for<In, kDecodeMaxT>(v);
}

}  // namespace

hipError_t launch_decode(const Geometry &g, const Tensors &t, bool bf16, Variant v, int max_len, hipStream_t st,
                         KernelTiming tm) {
    const int64_t items = (int64_t)g.n_seg * g.H;
    if (items <= 0) return hipSuccess;
    if (max_len > kDecodeMaxT) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((items + kWavesPerBlock - 1) / kWavesPerBlock)), block(64 * kWavesPerBlock);
    if (bf16)
        hipExtLaunchKernelGGL(decode_kernel_for<uint16_t>(v, max_len), grid, block, 0, st, tm.start, tm.stop, 0, g,
                              t);
    else
        hipExtLaunchKernelGGL(decode_kernel_for<float>(v, max_len), grid, block, 0, st, tm.start, tm.stop, 0, g, t);
    return hipGetLastError();
}

}  // namespace finch
