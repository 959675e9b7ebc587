// Short-sequence (recurrent step) WKV kernels for gfx950: T <= kDecodeMaxT
// tokens per (sequence, head), the generation side of the pre-fill state
// (GoldFinch architecture summary, section 3.4 "Training and Inference
// Procedures": generation continues from the pre-filled recurrent state).
//
// Same recurrence as the other kernels (section 3.4, "Recurrent state update
// and output"), with fp32 state and accumulation:
//   o_t[j]  = sum_i r_t[i] S[i][j] + (r_t . u . k_t) v_t[j]      (base Finch)
//   o_t[j]  = sum_i r_t[i] S[i][j] + u'_t[j]                      (Finch-C2)
//   S[i][j] = w_t[i] S[i][j] + k_t[i] v_t[j]   (C2: k_t[i] (1 - w_t[i]))
// with w_t = exp(-exp(d_t)) when the decay is given as d.
//
// With a few tokens per call the 64x64 fp32 state (16 KB in, 16 KB out per
// (sequence, head)) is most of the traffic.  Two kernels, one wave per
// (sequence, head) each:
//   - wkv_steps_mfma_kernel (bf16 inputs, 2..16 tokens): the call's tokens as
//     one chunk on the matrix cores (described further down);
//   - wkv_decode_kernel (one token, or fp32 inputs), token-serial on the VALU,
//     also the fallback of the first for calls whose decays are stiff.
// The token-serial kernel streams states with no LDS and no workgroup
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

constexpr int kWavesPerBlock = 1;   // token-serial kernel: one wave per workgroup (no barrier, no LDS)
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
    store_o1(t, row + jo, o);
    update_rows<0>(S, w, k, v);
}

// One (sequence, head) item token by token on the VALU (lane layout above).
// MaxT: the most tokens any item of the launch has (1 or kDecodeMaxT); the
// token look-ahead covers up to kAhead tokens.
template <typename In, bool LOGD, bool C2, int MaxT>
__device__ __forceinline__ void serial_item(const Geometry &g, const Tensors &t, const Item &a, int lane) {
    constexpr int Ahead = MaxT < kAhead ? MaxT : kAhead;
    const int grp = lane >> 4, col = lane & 15;
    const int jo = 4 * col + grp;                            // output channel of this lane
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

template <typename In, bool LOGD, bool C2, int MaxT>
__global__ __launch_bounds__(64 * kWavesPerBlock, 4) void wkv_decode_kernel(Geometry g, Tensors t) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: item math on the scalar unit
    const int lane = threadIdx.x & 63;
    const int64_t item = (int64_t)blockIdx.x * kWavesPerBlock + wave;
    if (item >= (int64_t)g.n_seg * g.H) return;             // whole wave: no barrier below
    const Item a = item_at(g, item, lane >> 4, lane & 15);
    if (!a.ok) return;
    serial_item<In, LOGD, C2, MaxT>(g, t, a, lane);
}

// ---- 2..16 tokens per item on the matrix cores (bf16 inputs) --------------------
// The same recurrence as one chunk of the chunked scan, with the chunk being
// the call's (at most 16) tokens: with P_t = w_0 ... w_t per key channel,
//   r~_t = r_t P_{t-1},  k^_s = k_s / P_s,  A[t][s] = r~_t . k^_s (s < t),
//   A[t][t] = r_t . u . k_t (base Finch; 0 for Finch-C2),
//   o_t = r~_t S + sum_s A[t][s] v_s (+ u'_t),   S' = diag(P_15) (S + k^^T v).
// One wave per (sequence, head) on v_mfma_f32_32x32x16_bf16 (lane l: A[l%32]
// [8(l/32)..+7], B[8(l/32)..+7][l%32], accumulator register 4q+e = row
// 8q + 4(l/32) + e, column l%32).  The state is four 32 x 32 accumulator tiles:
// lane (i32, h) holds S[32mc + 8q + 4h + e][32nj + i32], so each state access
// of the wave covers two whole 128-byte rows.  The outputs are formed
// transposed, o^T = S^T r~^T + V^T A^T: the state operand is then the
// accumulator registers themselves, with the contraction index permuted to
// match (lane half h, slot 4b + e <-> channel 16kk + 8b + 4h + e, or token
// 8b + 4h + e).  The token rows pass through a per-wave LDS tile, read back
// token-major (r~, k^ for the in-chunk product and the read-out) and, with
// ds_read_b64_tr_b16, channel-major (k^, v for the state update).  fp32
// operands enter as bf16 hi + lo pairs (three products per contraction).  A
// call whose decay products fall below 2^-96 within its tokens is evaluated by
// the token-serial path.

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
using lds_i16x4 = __attribute__((address_space(3))) i16x4;

constexpr float kMinStepDecay = 0x1p-96f;   // smaller decay products take the token-serial path
constexpr int kStageTiles = 5;               // r, k, w (or d), v, u'
// One wave per workgroup: the kernel has no workgroup barrier, and a lone
// wave's slot is released as soon as it ends (eight per CU, two per SIMD).
constexpr int kStepWaves = 1;

struct StepSmem {
    uint16_t tile[kStepWaves][kStageTiles][kDecodeMaxT * kHeadDim];   // per wave: 16 token rows per input
    float dec[kStepWaves][kHeadDim];                                  // P_15 per key channel
    float u[kStepWaves][kHeadDim];                                    // bonus u of the item's head
};

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Staging tile: 16 rows of 128 bytes; 16-byte piece p of row r is stored at
// piece p ^ f(r), f(r) = (r1, r2, r1 ^ r3) (bits from low to high), which keeps
// the row writes, the token-major reads and the transposed reads on distinct
// banks.  `unit` is an 8-byte unit (4 channels) of the row.
__device__ __forceinline__ int stage_off(int r, int unit) {
    const int f = ((r >> 1) & 1) | (((r >> 2) & 1) << 1) | ((((r >> 1) ^ (r >> 3)) & 1) << 2);
    return r * kHeadDim + ((((unit >> 1) ^ f) & 7) << 3) + ((unit & 1) << 2);
}

// x = hi + lo, hi = x rounded to the nearest bf16 (ties to even), lo the
// remainder (exact in fp32) rounded the same way; eight values -> two
// operands.  A nearest-rounded hi leaves at most half a bf16 ulp for lo, one
// bit more than a truncated hi, for the same instruction count.
__device__ __forceinline__ void split8(const float (&x)[8], bf16x8 &hi, bf16x8 &lo) {
    u32x4 h4, l4;
    #pragma unroll
    for (int i = 0; i < 4; ++i) {
        const f32x2 v = {x[2 * i], x[2 * i + 1]};
        h4[i] = __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2));
        const f32x2 l = {x[2 * i] - __uint_as_float(h4[i] << 16), x[2 * i + 1] - __uint_as_float(h4[i] & 0xFFFF0000u)};
        l4[i] = __builtin_bit_cast(unsigned, __builtin_convertvector(l, bf16x2));
    }
    hi = __builtin_bit_cast(bf16x8, h4);
    lo = __builtin_bit_cast(bf16x8, l4);
}

__device__ __forceinline__ float bf_lo(unsigned pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf_hi(unsigned pair) { return __uint_as_float(pair & 0xFFFF0000u); }

// Inclusive product over the 16 lanes of each DPP row (lanes without a source
// keep the old value, 1).
__device__ __forceinline__ float row_prod16(float x) {
    const int one = __float_as_int(1.f);
    x *= __int_as_float(__builtin_amdgcn_update_dpp(one, __float_as_int(x), 0x111, 0xF, 0xF, false));
    x *= __int_as_float(__builtin_amdgcn_update_dpp(one, __float_as_int(x), 0x112, 0xF, 0xF, false));
    x *= __int_as_float(__builtin_amdgcn_update_dpp(one, __float_as_int(x), 0x114, 0xF, 0xF, false));
    x *= __int_as_float(__builtin_amdgcn_update_dpp(one, __float_as_int(x), 0x118, 0xF, 0xF, false));
    return x;
}
// Value of the previous lane of the 16-lane row; 1 in its first lane.
__device__ __forceinline__ float row_prev(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(1.f), __float_as_int(x), 0x111, 0xF, 0xF, false));
}
// The same register of lane l ^ 32.
__device__ __forceinline__ float other_half(float x) {
    const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float((threadIdx.x & 32) ? s[0] : s[1]);
}

// w from the decay input, and the key factor of Finch-C2.
template <bool LOGD, bool C2>
__device__ __forceinline__ void decay_and_key(float x, float &w, float &k) {
    const float e = LOGD ? expf(x) : 0.f;                    // exp(d)
    w = LOGD ? expf(-e) : x;
    if (C2) k *= LOGD ? -expm1f(-e) : 1.f - x;
}

template <bool LOGD, bool C2>
__global__ __launch_bounds__(64 * kStepWaves, 2) void wkv_steps_mfma_kernel(Geometry g, Tensors t) {
    __shared__ StepSmem sm;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int i32 = lane & 31, h = lane >> 5;
    const int64_t item = (int64_t)blockIdx.x * kStepWaves + wave;
    if (item >= (int64_t)g.n_seg * g.H) return;             // whole wave: no barrier below
    const Item a = item_at(g, item, lane >> 4, lane & 15);
    if (!a.ok) return;
    const int nt = a.nt;                                      // 0 .. 16
    const size_t head_off = (size_t)a.h * kHeadDim;

    // ---- token rows: requested first, then the state (below), then written to
    // the staging tiles (rows past the item's tokens: r, k, v, u' = 0, w = 1);
    // the writes then wait for the token rows only
    uint16_t *const tiles = &sm.tile[wave][0][0];
    const float u_lane = C2 ? 0.f : t.u[head_off + lane];   // bonus, written to LDS below
    // Every load is unconditional (a row past the item's tokens reads its last
    // token, or row 0 of the tensor for an empty sequence: this kernel only
    // runs for calls with tokens) and the padding is selected at the write, so
    // that no branch joins make the compiler wait for the loads early.
    u32x4 rows[kStageTiles][2];
    {
        const void *src[kStageTiles] = {t.r, t.k, t.w, t.v, t.u2 ? t.u2 : t.v};
        #pragma unroll
        for (int x = 0; x < kStageTiles; ++x) {
            if (!C2 && x == 4) continue;
            #pragma unroll
            for (int m = 0; m < 2; ++m) {
                const int row = (lane >> 3) + 8 * m, piece = lane & 7;
                const int64_t grow = nt > 0 ? a.it.t0 + (row < nt ? row : nt - 1) : 0;
                const size_t off = ((size_t)grow * g.H + a.h) * kHeadDim + 8 * piece;
                rows[x][m] = *reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(src[x]) + off);
            }
        }
    }
    // ---- state, 32 x 32 accumulator tiles: S[mc][nj][4q+e] = S[32mc+8q+4h+e][32nj+i32]
    const size_t sbase = ((size_t)a.it.n * g.H + a.h) * (kHeadDim * kHeadDim);
    // (rows 0-31 now, rows 32-63 after the staging writes, so that the wait
    // before those writes names the token loads exactly). The loads go
    // through a buffer resource over this head's state: with no input state
    // its size is zero and every load reads zero, so no branch is needed
    // (a branch around loads makes every later wait a full drain).
    f32x16 S[2][2];
    const __amdgpu_buffer_rsrc_t s_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void *>(t.state_in ? static_cast<const void *>(t.state_in + sbase) : t.r), (short)0,
        t.state_in ? kHeadDim * kHeadDim * (int)sizeof(float) : 0, 0x00020000);
    const int s_lane = (4 * h * kHeadDim + i32) * (int)sizeof(float);
    auto load_rows = [&](int mc) {
        #pragma unroll
        for (int nj = 0; nj < 2; ++nj)
            #pragma unroll
            for (int r = 0; r < 16; ++r)
                S[mc][nj][r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                    s_rsrc, s_lane + ((32 * mc + 8 * (r >> 2) + (r & 3)) * kHeadDim + 32 * nj) * (int)sizeof(float),
                    0, 0));
    };
    __builtin_amdgcn_sched_barrier(0);   // keep every token load ahead of the state loads
    load_rows(0);

    {
        constexpr unsigned kPadW = LOGD ? 0xFF80FF80u : 0x3F803F80u;   // bf16 pairs: d = -inf, or w = 1
        #pragma unroll
        for (int x = 0; x < kStageTiles; ++x) {
            if (!C2 && x == 4) continue;
            const unsigned pad = x == 2 ? kPadW : 0u;
            const bool present = x != 4 || t.u2 != nullptr;
            #pragma unroll
            for (int m = 0; m < 2; ++m) {
                const int row = (lane >> 3) + 8 * m, piece = lane & 7;
                const u32x4 val = present && row < nt ? rows[x][m] : u32x4{pad, pad, pad, pad};
                *reinterpret_cast<u32x4 *>(tiles + x * (kDecodeMaxT * kHeadDim) + stage_off(row, 2 * piece)) = val;
            }
        }
    }
    load_rows(1);
    if (!C2) sm.u[wave][lane] = u_lane;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- channel-major operands: lane (i32, h) is channel 32mc + i32 (key) or
    // 32nj + i32 (value); slot 4b + e is token 8b + 4h + e
    bool stiff = false;
    bf16x8 kc_hi[2], kc_lo[2], vop[2];
    {
        const int grp16 = lane >> 4, i16 = lane & 15;
        // transposed read of rows 8b + 4h .. +3, columns 16-block (2*blk + (grp16 & 1)) of a tile
        auto tr_read = [&](int x, int blk, int b) {
            const int row = 8 * b + 4 * h + (i16 >> 2);
            const int unit = 8 * blk + 4 * (grp16 & 1) + (i16 & 3);
            const i16x4 v4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4 *)(tiles + x * (kDecodeMaxT * kHeadDim) + stage_off(row, unit)));
            return __builtin_bit_cast(u32x2, v4);
        };
        #pragma unroll
        for (int nj = 0; nj < 2; ++nj) {
            const u32x2 v0 = tr_read(3, nj, 0), v1 = tr_read(3, nj, 1);
            const u32x4 v = {v0.x, v0.y, v1.x, v1.y};
            vop[nj] = __builtin_bit_cast(bf16x8, v);
        }
        #pragma unroll
        for (int mc = 0; mc < 2; ++mc) {
            float kv[2][4], wv[2][4];
            #pragma unroll
            for (int b = 0; b < 2; ++b) {
                const u32x2 pk = tr_read(1, mc, b), pw = tr_read(2, mc, b);
                const float k4[4] = {bf_lo(pk.x), bf_hi(pk.x), bf_lo(pk.y), bf_hi(pk.y)};
                const float x4[4] = {bf_lo(pw.x), bf_hi(pw.x), bf_lo(pw.y), bf_hi(pw.y)};
                #pragma unroll
                for (int e = 0; e < 4; ++e) {
                    kv[b][e] = k4[e];
                    decay_and_key<LOGD, C2>(x4[e], wv[b][e], kv[b][e]);
                }
            }
            // in-lane products over each 4-token block, then the block totals of
            // the other half (blocks alternate between the halves: tokens 0-3 and
            // 8-11 in h = 0, 4-7 and 12-15 in h = 1)
            #pragma unroll
            for (int b = 0; b < 2; ++b) {
                wv[b][1] *= wv[b][0];
                wv[b][2] *= wv[b][1];
                wv[b][3] *= wv[b][2];
            }
            const float mine0 = wv[0][3], mine1 = wv[1][3];
            const float oth0 = other_half(mine0), oth1 = other_half(mine1);
            const float before0 = h ? oth0 : 1.f;                       // product of all earlier blocks
            const float before1 = h ? oth0 * mine0 * oth1 : mine0 * oth0;
            const float total = mine0 * mine1 * oth0 * oth1;            // P_15
            stiff |= !(total >= kMinStepDecay);
            if (h == 0) sm.dec[wave][32 * mc + i32] = total;
            float ks[8];
            #pragma unroll
            for (int e = 0; e < 4; ++e) {
                ks[e] = kv[0][e] * __builtin_amdgcn_rcpf(before0 * wv[0][e]);
                ks[4 + e] = kv[1][e] * __builtin_amdgcn_rcpf(before1 * wv[1][e]);
            }
            split8(ks, kc_hi[mc], kc_lo[mc]);
        }
    }
    if (__any(stiff)) {
        serial_item<uint16_t, LOGD, C2, kDecodeMaxT>(g, t, a, lane);
        return;
    }

    // ---- bonus r_t . u . k_t (base Finch), token-major like the operands below
    const int tt = i32 & 15;
    const bool tpad = i32 >= 16;
    float bonus = 0.f;
    if (!C2) {
        #pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            #pragma unroll
            for (int b = 0; b < 2; ++b) {
                const int o = stage_off(tt, 4 * kk + 2 * b + h);
                const u32x2 pr = *reinterpret_cast<const u32x2 *>(tiles + 0 * (kDecodeMaxT * kHeadDim) + o);
                const u32x2 pk = *reinterpret_cast<const u32x2 *>(tiles + 1 * (kDecodeMaxT * kHeadDim) + o);
                const float4 u4 = *reinterpret_cast<const float4 *>(&sm.u[wave][16 * kk + 8 * b + 4 * h]);
                bonus += bf_lo(pr.x) * u4.x * bf_lo(pk.x) + bf_hi(pr.x) * u4.y * bf_hi(pk.x) +
                         bf_lo(pr.y) * u4.z * bf_lo(pk.y) + bf_hi(pr.y) * u4.w * bf_hi(pk.y);
            }
        bonus = tpad ? 0.f : bonus;
        bonus += other_half(bonus);                          // over all 64 channels
    }

    // ---- token-major operands, one K step (16 channels) at a time: lane (i32, h)
    // is token tt = i32 % 16 (lanes with i32 >= 16 are padding rows of the
    // 32-row tiles), slot 4b + e is channel 16kk + 8b + 4h + e.  Each step feeds
    // A^T = k^ r~^T (rows s, columns t) and the read-out o^T += S^T r~^T (rows
    // j, columns t).
    f32x16 aT = {}, oT[2] = {f32x16{}, f32x16{}};
    #pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        float rs[8], ks[8];
        #pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int o = stage_off(tt, 4 * kk + 2 * b + h);
            const u32x2 pr = *reinterpret_cast<const u32x2 *>(tiles + 0 * (kDecodeMaxT * kHeadDim) + o);
            const u32x2 pk = *reinterpret_cast<const u32x2 *>(tiles + 1 * (kDecodeMaxT * kHeadDim) + o);
            const u32x2 pw = *reinterpret_cast<const u32x2 *>(tiles + 2 * (kDecodeMaxT * kHeadDim) + o);
            const float rv[4] = {bf_lo(pr.x), bf_hi(pr.x), bf_lo(pr.y), bf_hi(pr.y)};
            const float kv[4] = {bf_lo(pk.x), bf_hi(pk.x), bf_lo(pk.y), bf_hi(pk.y)};
            const float xv[4] = {bf_lo(pw.x), bf_hi(pw.x), bf_lo(pw.y), bf_hi(pw.y)};
            #pragma unroll
            for (int e = 0; e < 4; ++e) {
                float w, k = kv[e];
                decay_and_key<LOGD, C2>(xv[e], w, k);
                const float r = tpad ? 0.f : rv[e];
                if (tpad) { k = 0.f; w = 1.f; }
                const float p = row_prod16(w);                  // P_t
                const float pp = row_prev(p);                   // P_{t-1}
                rs[4 * b + e] = r * pp;
                ks[4 * b + e] = k * __builtin_amdgcn_rcpf(p);
            }
        }
        bf16x8 r_hi, r_lo, k_hi, k_lo;
        split8(rs, r_hi, r_lo);
        split8(ks, k_hi, k_lo);
        aT = mfma32(k_hi, r_hi, aT);
        aT = mfma32(k_hi, r_lo, aT);
        aT = mfma32(k_lo, r_hi, aT);
        const int mc = kk >> 1, q0 = 2 * (kk & 1);
        #pragma unroll
        for (int nj = 0; nj < 2; ++nj) {
            float sv[8];
            #pragma unroll
            for (int e = 0; e < 4; ++e) {
                sv[e] = S[mc][nj][4 * q0 + e];
                sv[4 + e] = S[mc][nj][4 * (q0 + 1) + e];
            }
            bf16x8 s_hi, s_lo;
            split8(sv, s_hi, s_lo);
            oT[nj] = mfma32(s_hi, r_hi, oT[nj]);
            oT[nj] = mfma32(s_hi, r_lo, oT[nj]);
            oT[nj] = mfma32(s_lo, r_hi, oT[nj]);
        }
    }

    // ---- in-chunk part: lane (t, h) holds aT[4q+e] = A[t][8q+4h+e]; o^T += V^T A^T
    {
        float av[8];
        #pragma unroll
        for (int q = 0; q < 2; ++q)
            #pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int s = 8 * q + 4 * h + e;
                const float x = s < tt ? aT[4 * q + e] : (s == tt && !C2 ? bonus : 0.f);
                av[4 * q + e] = tpad ? 0.f : x;
            }
        bf16x8 ab_hi, ab_lo;
        split8(av, ab_hi, ab_lo);
        #pragma unroll
        for (int nj = 0; nj < 2; ++nj) {
            oT[nj] = mfma32(vop[nj], ab_hi, oT[nj]);
            oT[nj] = mfma32(vop[nj], ab_lo, oT[nj]);
        }
    }
    // lane (t, h): oT[nj][4q+e] = o_t[32nj + 8q + 4h + e]
    if (!tpad && tt < nt) {
        const size_t orow = ((size_t)(a.it.t0 + tt) * g.H + a.h) * kHeadDim;
        const float u2_scale = t.u2 ? 1.f : 0.f;
        #pragma unroll
        for (int nj = 0; nj < 2; ++nj)
            #pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int j0 = 32 * nj + 8 * q + 4 * h;
                float4 o4 = make_float4(oT[nj][4 * q], oT[nj][4 * q + 1], oT[nj][4 * q + 2], oT[nj][4 * q + 3]);
                if (C2) {
                    const u32x2 pu = *reinterpret_cast<const u32x2 *>(tiles + 4 * (kDecodeMaxT * kHeadDim) +
                                                                      stage_off(tt, j0 >> 2));
                    o4.x += u2_scale * bf_lo(pu.x);
                    o4.y += u2_scale * bf_hi(pu.x);
                    o4.z += u2_scale * bf_lo(pu.y);
                    o4.w += u2_scale * bf_hi(pu.y);
                }
                store_o4(t, orow + j0, o4);
            }
    }

    // ---- S = diag(P_15) (S + k^^T v)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    #pragma unroll
    for (int mc = 0; mc < 2; ++mc)
        #pragma unroll
        for (int nj = 0; nj < 2; ++nj) {
            f32x16 pS = mfma32(kc_hi[mc], vop[nj], f32x16{});
            pS = mfma32(kc_lo[mc], vop[nj], pS);
            #pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 d4 = *reinterpret_cast<const float4 *>(&sm.dec[wave][32 * mc + 8 * q + 4 * h]);
                const float dv[4] = {d4.x, d4.y, d4.z, d4.w};
                #pragma unroll
                for (int e = 0; e < 4; ++e) S[mc][nj][4 * q + e] = dv[e] * (S[mc][nj][4 * q + e] + pS[4 * q + e]);
            }
        }
    if (t.state_out && a.it.p == a.it.P - 1) {
        float *dst = t.state_out + sbase + 4 * h * kHeadDim + i32;
        #pragma unroll
        for (int mc = 0; mc < 2; ++mc)
            #pragma unroll
            for (int nj = 0; nj < 2; ++nj)
                #pragma unroll
                for (int r = 0; r < 16; ++r) dst[(32 * mc + 8 * (r >> 2) + (r & 3)) * kHeadDim + 32 * nj] = S[mc][nj][r];
    }
}

template <bool LOGD>
void (*steps_kernel_for(bool c2))(Geometry, Tensors) {
    return c2 ? wkv_steps_mfma_kernel<LOGD, true> : wkv_steps_mfma_kernel<LOGD, false>;
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
    if (bf16 && max_len >= 2) {
        auto kern = v.log_decay ? steps_kernel_for<true>(v.c2) : steps_kernel_for<false>(v.c2);
        const dim3 sgrid((unsigned)((items + kStepWaves - 1) / kStepWaves)), sblock(64 * kStepWaves);
        hipExtLaunchKernelGGL(kern, sgrid, sblock, 0, st, tm.start, tm.stop, 0, g, t);
    } else if (bf16)
        hipExtLaunchKernelGGL(decode_kernel_for<uint16_t>(v, max_len), grid, block, 0, st, tm.start, tm.stop, 0, g,
                              t);
    else
        hipExtLaunchKernelGGL(decode_kernel_for<float>(v, max_len), grid, block, 0, st, tm.start, tm.stop, 0, g, t);
    return hipGetLastError();
}

}  // namespace finch
