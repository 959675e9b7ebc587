// Chunked Finch WKV scan for bf16 inputs on gfx950 matrix cores.
//
// The recurrence of the GoldFinch architecture summary (section 3.4,
// "Recurrent state update and output") is evaluated 64 tokens at a time.
// Within a chunk, with P_t = w_0 w_1 ... w_t (per key channel, from the chunk
// start; P_{-1} = 1):
//
//   o_t   = sum_i r~_t[i] S[i,:]                                     read-out of the carried state
//         + sum_{s<t} A_ts v_s,  A_ts = sum_i r~_t[i] k~_s[i]        in-chunk pairs
//         + (r_t . u . k_t) v_t                                       bonus
//   S_end = diag(P_63) (S + sum_s k~_s^T v_s)
//
// with r~_t = r_t P_{t-1} and k~_s = k_s / P_s: their product is exactly the
// decay product of the pages' state equation, w_{s+1}...w_{t-1}.  The
// products come from an in-lane and a cross-lane (DPP) scan; only k~ needs a
// reciprocal, no logarithm or exponential is taken.
// All four contractions run on v_mfma_f32_16x16x32_bf16 with fp32
// accumulation; every fp32 operand is split into bf16 hi + lo parts (three
// products, or two when the other operand is an exact bf16 input), which keeps
// about 16 significant bits per product.  The 64x64 fp32 state stays in
// registers for the whole segment.
//
// Two further forms of the same section are compile-time switches:
//  - LOGD: the decay input holds d with w = exp(-exp(d)) (paragraph
//    "Data-dependent decay"), w = 2^{-e^d log2(e)} (no precision is lost to
//    w rounding to 1 in bf16);
//  - C2: the Finch-C2 mixer -- keys enter as k (1 - w) (paragraph "Key
//    computation with normalization property"), no static bonus (the
//    diagonal of A is zero), and the second value u'_t (a fifth input stream,
//    staged like the others) is added to o (output equation).
//
// A chunk in which some channel decays by more than 2^96 over the chunk
// ("stiff": P_63 < 2^-96) would push 1/P out of range; such a chunk is
// evaluated token by token instead (exact, same registers), so the result is
// defined for every 0 < w <= 1.  The state pass, which needs only
// diag(P_63) S + sum_s (P_63 / P_s) k_s^T v_s, forms those factors (all <= 1)
// from log2 prefix sums and needs no such fallback.
//
// Workgroup = 4 waves, one (segment, head) work item.  Wave w owns value
// columns 16w..16w+15 of the state and of o; lane (i16 = lane%16, grp =
// lane/16) holds S[16*ib + 4*grp + e][16*w + i16] for ib, e in 0..3 (the
// accumulator layout of the 16x16 MFMA).  Every input is loaded as whole
// 128-byte token rows (16 bytes per lane, the next chunk prefetched into
// registers while the current one is processed); r, k, w (and u') pass
// through padded staging tiles in LDS into the pre-processing layout, v goes
// to its operand tile.  LDS holds every MFMA operand tile row-major
// [token][channel] with a row-dependent XOR swizzle of its column units
// (bank-conflict free); operands contracted over tokens are read with
// ds_read_b64_tr_b16.  Segments of a long sequence are independent work items
// whose starting states come from a state pass and a scan over segments.
#include <cstddef>

#include <hip/hip_ext.h>

#include "wkv_internal.h"

namespace finch {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr float kMinChunkDecay = 0x1p-96f;    // smaller chunk decay products take the token-serial path
constexpr float kLog2Floor = -127.f;          // floor of log2 w in the state pass (w = 0 stays finite)
constexpr unsigned kOnePair = 0x3F803F80u;    // two bf16 1.0 (padding value of w)
constexpr unsigned kNegInfPair = 0xFF80FF80u;  // two bf16 -inf (padding value of d: w = 1)
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kTileElems = kChunk * kHeadDim; // one 64 x 64 bf16 tile
constexpr int kStageRow = 72;                  // staging row pitch in bf16 (144 B)
constexpr int kStageElems = kChunk * kStageRow;

enum class Mode { Main, State };

// Registers holding one prefetched chunk: r, k, w, v (and the C2 second
// value) as 16-byte pieces of whole token rows (rows tid/8 and tid/8 + 32,
// piece tid%8), so that every load instruction covers complete 128-byte lines.
template <bool C2>
struct ChunkRegs {
    u32x4 r[2], k[2], w[2], v[2];
};
template <>
struct ChunkRegs<true> {
    u32x4 r[2], k[2], w[2], v[2], u2[2];
};

// ---- LDS tile layouts ---------------------------------------------------------
// Every tile is 64 rows x 64 bf16 (128 B per row, no padding).  Column units
// are XOR-swizzled with a function of the row.  The LDS has 64 banks of 4 B;
// 8-byte reads are served 32 lanes per pass and 8-byte writes 16 lanes per
// pass, and the swizzles keep every pass on distinct banks:
//   a     : 8-byte unit u -> u ^ (r & 15)
//   rt    : 8-byte unit u -> u ^ (r & 15) ^ (r >> 4)
//   kt    : 8-byte unit u -> u ^ L(r & 15) ^ phi(r >> 4), L(x) = (x0, x3, x2, x1)
//           (bits from low to high), phi(y) = y0 + 8 y1
//   v     : 16-byte unit u -> u ^ ((r & 3) << 1)
// The pre-processing writes rows 4x + a (x = lane % 16), so the rt and kt
// swizzles take row bits 4-5 as well; the operand reads name rows whose bits
// 4-5 are a compile-time constant, so each read address is a per-lane base
// XOR a constant (plus a constant).
__device__ __forceinline__ int l_kt(int x) { return (x & 5) | (((x >> 3) & 1) << 1) | (((x >> 1) & 1) << 3); }
__device__ __forceinline__ constexpr int phi_kt(int y) { return (y & 1) | (((y >> 1) & 1) << 3); }
__device__ __forceinline__ int swz_rt(int r) { return (r & 15) ^ (r >> 4); }
__device__ __forceinline__ int swz_kt(int r) { return l_kt(r & 15) ^ phi_kt(r >> 4); }
__device__ __forceinline__ int off_v(int r, int c) {
    return r * 64 + ((((c >> 3) ^ ((r & 3) << 1)) << 3) | (c & 7));
}
//   stage : 144-byte rows, 16-byte piece p -> p ^ f(r), f(r) = r bits (2, 4, 5);
//           conflict-free both for whole-row 16-byte writes and for the
//           pre-processing reads (8 bytes of rows 4x + a)
__device__ __forceinline__ int stage_f(int r) { return ((r >> 2) & 1) | (((r >> 4) & 1) << 1) | (((r >> 5) & 1) << 2); }
__device__ __forceinline__ int off_stage(int r, int piece) { return r * kStageRow + ((piece ^ stage_f(r)) << 3); }

// ---- global memory through buffer resources --------------------------------
// Each chunk gets resources whose base is (first token of the chunk, head h)
// and whose size ends after the chunk's last valid token row, so the per-lane
// byte offsets are loop invariant and rows past the end of a partial chunk
// read as zero and drop their stores (raw-buffer range checking).
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr int kRsrcWord3 = 0x00020000;         // raw dword access, no swizzle

__device__ __forceinline__ Rsrc chunk_rsrc(const void *base, int64_t row0, int rows, int H, int h,
                                           int row_bytes) {
    const char *p = static_cast<const char *>(base) + ((size_t)row0 * H + h) * row_bytes;
    const int bytes = ((rows - 1) * H + 1) * row_bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(p), (short)0, bytes, kRsrcWord3);
}

template <int NStage>
struct Smem {
    uint16_t v[kTileElems];          // values of the chunk
    uint16_t rt_hi[kTileElems];      // r~ = r P_{t-1}, bf16 hi/lo planes
    uint16_t rt_lo[kTileElems];
    uint16_t kt_hi[kTileElems];      // k~ = k / P_s (state pass: k 2^{Lam_63-Lam_s})
    uint16_t kt_lo[kTileElems];
    union {
        struct {
            uint16_t a_hi[kTileElems];   // in-chunk matrix A[t][s], hi/lo planes
            uint16_t a_lo[kTileElems];
        };
        uint16_t stage[NStage][kStageElems];  // raw r, k, w (, u') rows of the chunk (until the first barrier)
    };
    alignas(16) float bonus_part[4][kChunk];   // per-wave partial sums of r.u.k per token
    alignas(16) float row_dec[kHeadDim];       // decay of the whole chunk per key channel
    int stiff[4];
};
// the token-serial path stages 64 x 64 fp32 outputs across rt_hi and rt_lo
static_assert(offsetof(Smem<3>, rt_lo) == offsetof(Smem<3>, rt_hi) + sizeof(uint16_t) * kTileElems,
              "rt planes must be adjacent");
static_assert(offsetof(Smem<4>, rt_lo) == offsetof(Smem<4>, rt_hi) + sizeof(uint16_t) * kTileElems,
              "rt planes must be adjacent");
// two workgroups per compute unit (160 KB of LDS)
static_assert(sizeof(Smem<4>) <= 80 * 1024, "two workgroups per CU");

using lds_i16x4 = __attribute__((address_space(3))) i16x4;
using lds_u32x2 = __attribute__((address_space(3))) u32x2;
using lds_u32x4 = __attribute__((address_space(3))) u32x4;
using lds_u16 = __attribute__((address_space(3))) uint16_t;

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float bf16_lo(unsigned pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(unsigned pair) { return __uint_as_float(pair & 0xFFFF0000u); }

// x = hi + lo with hi the bf16 truncation of x (exact difference) and lo
// rounded to bf16; returns packed pairs for two values.
struct HiLo {
    unsigned hi, lo;
};
__device__ __forceinline__ HiLo split2(float x0, float x1) {
    const unsigned b0 = __float_as_uint(x0), b1 = __float_as_uint(x1);
    HiLo r;
    r.hi = __builtin_amdgcn_perm(b1, b0, 0x07060302u);      // {x1.hi16, x0.hi16}
    const float l0 = x0 - __uint_as_float(b0 & 0xFFFF0000u);
    const float l1 = x1 - __uint_as_float(b1 & 0xFFFF0000u);
    f32x2 l = {l0, l1};
    r.lo = __builtin_bit_cast(unsigned, __builtin_convertvector(l, bf16x2));
    return r;
}
// four values -> packed (hi, lo) planes of 4 bf16 each
__device__ __forceinline__ void split4(float x0, float x1, float x2, float x3, u32x2 &hi, u32x2 &lo) {
    const HiLo a = split2(x0, x1), b = split2(x2, x3);
    hi = u32x2{a.hi, b.hi};
    lo = u32x2{a.lo, b.lo};
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x2 a, u32x2 b) {
    u32x4 v = {a.x, a.y, b.x, b.y};
    return __builtin_bit_cast(bf16x8, v);
}
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Operand reads are volatile so that the compiler keeps each one a separate
// ds_read_b64 landing directly in its MFMA operand registers (merged reads of
// neighbouring tiles would need register copies to regroup).
__device__ __forceinline__ u32x2 lds_read_b64(const uint16_t *tile, int elem) {
    return *((const volatile lds_u32x2 *)((const lds_u16 *)tile + elem));
}
__device__ __forceinline__ void lds_write_b64(uint16_t *tile, int elem, u32x2 v) {
    *((lds_u32x2 *)((lds_u16 *)tile + elem)) = v;
}
__device__ __forceinline__ void lds_write_b128(uint16_t *tile, int elem, u32x4 v) {
    *((lds_u32x4 *)((lds_u16 *)tile + elem)) = v;
}

// Transposed read (ds_read_b64_tr_b16): the 16 lanes of a group each name one
// 8-byte piece of a 4 x 16 block (rows k0..k0+3, columns n0..n0+15); lane i16
// receives column n0 + i16 as four 16-bit values, rows k0..k0+3.  `elem` is
// this lane's piece: row k0 + i16/4, columns n0 + 4*(i16%4) .. +3.
__device__ __forceinline__ u32x2 lds_read_tr(const uint16_t *tile, int elem) {
    i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)((const lds_u16 *)tile + elem));
    return __builtin_bit_cast(u32x2, v);
}

// MFMA K order.  For the 16x16x32 instruction lane group grp holds 8 K slots;
// here slots 0..3 are indices 32*kk + 4*grp + 0..3 and slots 4..7 are
// 32*kk + 16 + 4*grp + 0..3, for contractions over channels and over tokens
// alike (the state's accumulator layout provides exactly this order).

// Per-lane LDS element offsets (lane i16 = x, group grp, wave w), computed once.
struct LdsBases {
    int ro_x[4];   // channel-contracted rows 16*b + x of a: [2*kk + hh] (+ 1024*b);
                   // of rt: (ro_x ^ 4*b) + 1024*b
    int ro_k[4];   // same for kt: (ro_k ^ 4*phi(b)) + 1024*b
    int pw_rt[4];  // pre-processing writes, rows 4*x + a: [a]
    int pw_kt[4];
    int aw[4];     // A tile writes, row 16*TB + x, columns 16*SB + 4*grp: [SB] (+ 1024*TB)
    int tr_kt[4];  // token-contracted kt columns 16*ib + x: [ib], used as
                   // (tr_kt ^ 4*phi(2*kk + hh)) + 64*(32*kk + 16*hh)
    int tr_v;      // token-contracted v columns 16*w + x (+ 64*(32*kk + 16*hh))
    int vw;        // v writes, rows tid/8 (+ 64*32*m), 16-byte piece tid%8
};

__device__ __forceinline__ LdsBases make_bases(int tid) {
    const int lane = tid & 63, x = lane & 15, grp = lane >> 4, w = tid >> 6;
    LdsBases b;
    #pragma unroll
    for (int q = 0; q < 4; ++q) {                 // q = 2*kk + hh -> column unit 4*q + grp
        b.ro_x[q] = x * 64 + (((4 * q + grp) ^ x) << 2);
        b.ro_k[q] = x * 64 + (((4 * q + grp) ^ l_kt(x)) << 2);
    }
    #pragma unroll
    for (int a = 0; a < 4; ++a) {
        b.pw_rt[a] = (4 * x + a) * 64 + (((4 * w + grp) ^ swz_rt(4 * x + a)) << 2);
        b.pw_kt[a] = (4 * x + a) * 64 + (((4 * w + grp) ^ swz_kt(4 * x + a)) << 2);
        b.aw[a] = x * 64 + ((((4 * a) ^ (x & 12)) | (grp ^ (x & 3))) << 2);
        const int row0 = 4 * grp + (x >> 2);
        b.tr_kt[a] = row0 * 64 + (((4 * a + (x & 3)) ^ l_kt(row0)) << 2);
    }
    b.tr_v = (4 * grp + (x >> 2)) * 64 + (((2 * w + ((x & 3) >> 1)) ^ (((x >> 2) & 3) << 1)) << 3) + 4 * (x & 1);
    const int ld_row = tid >> 3;
    b.vw = ld_row * 64 + (((tid & 7) ^ ((ld_row & 3) << 1)) << 3);
    return b;
}

// channel-contracted operand of a (row 16*b + x); of rt (rt_op) and kt (kt_op)
__device__ __forceinline__ bf16x8 row_op(const uint16_t *tile, const int (&ro)[4], int b, int kk) {
    return as_bf16x8(lds_read_b64(tile, ro[2 * kk] + 1024 * b), lds_read_b64(tile, ro[2 * kk + 1] + 1024 * b));
}
__device__ __forceinline__ bf16x8 rt_op(const uint16_t *tile, const int (&ro)[4], int b, int kk) {
    return as_bf16x8(lds_read_b64(tile, (ro[2 * kk] ^ (4 * b)) + 1024 * b),
                     lds_read_b64(tile, (ro[2 * kk + 1] ^ (4 * b)) + 1024 * b));
}
__device__ __forceinline__ bf16x8 kt_op(const uint16_t *tile, const int (&ro)[4], int b, int kk) {
    return as_bf16x8(lds_read_b64(tile, (ro[2 * kk] ^ (4 * phi_kt(b))) + 1024 * b),
                     lds_read_b64(tile, (ro[2 * kk + 1] ^ (4 * phi_kt(b))) + 1024 * b));
}
// token-contracted operand: lane i16 gets column n0 + i16 (base chosen by the caller)
__device__ __forceinline__ bf16x8 col_op(const uint16_t *tile, int base, int kk) {
    return as_bf16x8(lds_read_tr(tile, base + 64 * (32 * kk)), lds_read_tr(tile, base + 64 * (32 * kk + 16)));
}
// the same for kt, whose swizzle also takes row bits 4-5 (= 2*kk + hh)
__device__ __forceinline__ bf16x8 kt_col_op(const uint16_t *tile, int base, int kk) {
    return as_bf16x8(lds_read_tr(tile, (base ^ (4 * phi_kt(2 * kk))) + 64 * (32 * kk)),
                     lds_read_tr(tile, (base ^ (4 * phi_kt(2 * kk + 1))) + 64 * (32 * kk + 16)));
}

// Inclusive prefix sum over the 16 lanes of each DPP row.
__device__ __forceinline__ float row_scan16(float x) {
    int v = __float_as_int(x);
    v = __float_as_int(__int_as_float(v) + __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true)));
    v = __float_as_int(__int_as_float(v) + __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true)));
    v = __float_as_int(__int_as_float(v) + __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true)));
    v = __float_as_int(__int_as_float(v) + __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true)));
    return __int_as_float(v);
}

// Inclusive product over the 16 lanes of each DPP row (lanes without a
// source keep the old value, 1).
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

// Value of lane N of this lane's 16-lane row (DPP row_newbcast).
template <int N>
__device__ __forceinline__ float row_bcast(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x150 + N, 0xF, 0xF, false));
}

// Sum over the four 16-lane rows (lane, lane ^ 16, lane ^ 32, lane ^ 48),
// with the row-swapping permutes (VALU, no LDS round trip).
__device__ __forceinline__ float sum_rows4(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Tiles of the in-chunk matrix, A[t][s] for t in block TB, s in block SB
// (SB <= TB), computed as A^T = k~ r~^T and masked on diagonal blocks (bonus
// on the diagonal, zeros above), split and stored.  NT tiles are processed
// together so that their MFMA chains interleave.
template <bool Bonus, int NT, typename SM>
__device__ __forceinline__ void a_tiles(SM &sm, const LdsBases &lb, const int (&TB)[NT],
                                        const int (&SB)[NT], int i16, int grp) {
    f32x4 a[NT];
    #pragma unroll
    for (int n = 0; n < NT; ++n) a[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    #pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        bf16x8 k_hi[NT], k_lo[NT], r_hi[NT], r_lo[NT];
        #pragma unroll
        for (int n = 0; n < NT; ++n) {
            k_hi[n] = kt_op(sm.kt_hi, lb.ro_k, SB[n], kk);
            k_lo[n] = kt_op(sm.kt_lo, lb.ro_k, SB[n], kk);
            r_hi[n] = rt_op(sm.rt_hi, lb.ro_x, TB[n], kk);
            r_lo[n] = rt_op(sm.rt_lo, lb.ro_x, TB[n], kk);
        }
        #pragma unroll
        for (int n = 0; n < NT; ++n) a[n] = mfma(k_hi[n], r_hi[n], a[n]);
        #pragma unroll
        for (int n = 0; n < NT; ++n) a[n] = mfma(k_hi[n], r_lo[n], a[n]);
        #pragma unroll
        for (int n = 0; n < NT; ++n) a[n] = mfma(k_lo[n], r_hi[n], a[n]);
    }
    #pragma unroll
    for (int n = 0; n < NT; ++n) {
        // a[n][e] = A[t][s], t = 16*TB + i16, s = 16*SB + 4*grp + e
        const int t = 16 * TB[n] + i16;
        if (SB[n] == TB[n]) {
            const float b = Bonus ? sm.bonus_part[0][t] + sm.bonus_part[1][t] + sm.bonus_part[2][t] + sm.bonus_part[3][t]
                                  : 0.f;
            #pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int s_loc = 4 * grp + e;
                a[n][e] = s_loc < i16 ? a[n][e] : (s_loc == i16 ? b : 0.f);
            }
        }
        u32x2 hi, lo;
        split4(a[n][0], a[n][1], a[n][2], a[n][3], hi, lo);
        const int elem = lb.aw[SB[n]] + 1024 * TB[n];
        lds_write_b64(sm.a_hi, elem, hi);
        lds_write_b64(sm.a_lo, elem, lo);
    }
}

// 1 - w for the key factor of Finch-C2, from the decay input x (w itself, or
// d with e = exp(d) already formed).  Exact for a bf16 w.  For d it is
// 1 - exp(-e): below e = 1/32 from its Taylor series (four terms, truncation
// below 1e-8 relative), above from 1 - 2^{-e log2 e} (relative error a few
// 1e-6, since 1 - w > 0.03 there).
template <bool LOGD>
__device__ __forceinline__ float one_minus_w(float x, float e) {
    if (!LOGD) return 1.f - x;
    const float series = e * (1.f - 0.5f * e * (1.f - e * (1.f / 3.f) * (1.f - 0.25f * e)));
    const float direct = 1.f - __builtin_amdgcn_exp2f(-e * kLog2e);
    return e < 0.03125f ? series : direct;
}

template <Mode M, bool LOGD, bool C2>
__global__ __launch_bounds__(256, 2) void wkv_chunk_kernel(Geometry g, Tensors t, Workspace ws) {
    constexpr bool kU2 = M == Mode::Main && C2;            // second value staged and added
    using SM = Smem<kU2 ? 4 : 3>;
    __shared__ SM sm;

    const int item = blockIdx.x;
    const int h = item % g.H;
    const ItemRange it = decode_segment(g, item / g.H);
    if (!it.valid) return;
    if (M == Mode::State && it.p == it.P - 1) return;      // last segment's aggregate is unused
    // a split the host did not plan (device offsets differing from the host
    // copy) has no workspace behind it: leave the item alone
    if (it.P > 1 && (ws.seg_start == nullptr || ws.seg_state == nullptr)) return;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int i16 = lane & 15;
    const int grp = lane >> 4;
    const int H = g.H;
    const LdsBases lb = make_bases(tid);

    // ---- carried state ------------------------------------------------------
    // lane (i16, grp) of wave w holds S[16*ib + 4*grp + e][16*w + i16]
    float S[4][4];
    const float *s_src = nullptr;
    if (M == Mode::Main) {
        if (it.P > 1)
            s_src = ws.seg_start + (size_t)item * kSegStartFloats;
        else if (t.state_in)
            s_src = t.state_in + ((size_t)it.n * H + h) * (kHeadDim * kHeadDim);
    }
    #pragma unroll
    for (int ib = 0; ib < 4; ++ib)
        #pragma unroll
        for (int e = 0; e < 4; ++e)
            S[ib][e] = s_src ? s_src[(16 * ib + 4 * grp + e) * kHeadDim + 16 * wave + i16] : 0.f;

    // pre-processing layout: channels c0..c0+3, tokens 4*i16 .. 4*i16+3
    const int c0 = 16 * wave + 4 * grp;
    f32x4 u4 = {0.f, 0.f, 0.f, 0.f};
    if (M == Mode::Main && !C2) u4 = *reinterpret_cast<const f32x4 *>(t.u + (size_t)h * kHeadDim + c0);
    float lam_seg[4] = {0.f, 0.f, 0.f, 0.f};                // State: segment log2-decay per channel


    const uint16_t *gr = static_cast<const uint16_t *>(t.r);
    const uint16_t *gk = static_cast<const uint16_t *>(t.k);
    const uint16_t *gw = static_cast<const uint16_t *>(t.w);

    // ---- global -> register prefetch of one chunk ------------------------------
    // r, k, w, v as whole-row 16-byte pieces (rows tid/8 and tid/8 + 32); r, k,
    // w go through the staging tiles into the pre-processing layout, v into
    // its operand tile.  Rows past the segment end read as zero (buffer range
    // check); w's padding value 1 is substituted after the staging read.
    const int ld_row = tid >> 3;
    const int ld_col = (tid & 7) * 8;
    constexpr int kRowIn = kHeadDim * 2;                 // bytes of one bf16 token row of a head
    constexpr int kRowOut = kHeadDim * 4;                // bytes of one fp32 token row of a head
    int off_vin[2], st_wr[2], st_rd[4];
    #pragma unroll
    for (int m = 0; m < 2; ++m) {
        off_vin[m] = (ld_row + 32 * m) * H * kRowIn + 2 * ld_col;
        st_wr[m] = off_stage(ld_row + 32 * m, tid & 7);
    }
    // pre-processing read of rows 4*i16 + a, channels c0..c0+3: half (grp & 1)
    // of 16-byte piece 2*wave + grp/2
    #pragma unroll
    for (int a = 0; a < 4; ++a) st_rd[a] = off_stage(4 * i16 + a, 2 * wave + (grp >> 1)) + 4 * (grp & 1);
    // second value in the accumulator layout: rows 16*tb + i16, channels
    // 16*wave + 4*grp .. +3
    int st_u2[4];
    #pragma unroll
    for (int tb = 0; tb < 4; ++tb) st_u2[tb] = off_stage(16 * tb + i16, 2 * wave + (grp >> 1)) + 4 * (grp & 1);
    int off_out[4];                                      // o rows 16*tb + i16, columns 16*wave + 4*grp
    #pragma unroll
    for (int tb = 0; tb < 4; ++tb) off_out[tb] = (16 * tb + i16) * H * kRowOut + 4 * (16 * wave + 4 * grp);
    auto issue_loads = [&](ChunkRegs<kU2> &P, int64_t tc) {
        const int rows = (int)min<int64_t>(kChunk, it.t1 - tc);
        const Rsrc rk = chunk_rsrc(t.k, tc, rows, H, h, kRowIn);
        const Rsrc rw = chunk_rsrc(t.w, tc, rows, H, h, kRowIn);
        const Rsrc rv = chunk_rsrc(t.v, tc, rows, H, h, kRowIn);
        if (M == Mode::Main) {
            const Rsrc rr = chunk_rsrc(t.r, tc, rows, H, h, kRowIn);
            #pragma unroll
            for (int m = 0; m < 2; ++m) P.r[m] = __builtin_amdgcn_raw_buffer_load_b128(rr, off_vin[m], 0, 0);
        }
        if constexpr (kU2) {
            // no second value: a resource with no records (every load reads 0)
            const Rsrc ru = t.u2 ? chunk_rsrc(t.u2, tc, rows, H, h, kRowIn)
                                 : __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(t.v), (short)0, 0, kRsrcWord3);
            #pragma unroll
            for (int m = 0; m < 2; ++m) P.u2[m] = __builtin_amdgcn_raw_buffer_load_b128(ru, off_vin[m], 0, 0);
        }
        #pragma unroll
        for (int m = 0; m < 2; ++m) {
            P.k[m] = __builtin_amdgcn_raw_buffer_load_b128(rk, off_vin[m], 0, 0);
            P.w[m] = __builtin_amdgcn_raw_buffer_load_b128(rw, off_vin[m], 0, 0);
            P.v[m] = __builtin_amdgcn_raw_buffer_load_b128(rv, off_vin[m], 0, 0);
        }
    };

    const int64_t n_tok = it.t1 - it.t0;
    const int n_chunks = (int)((n_tok + kChunk - 1) / kChunk);
    // o of chunk c (acc[tb][e] = o[16*tb + i16][16*wave + 4*grp + e]) is held
    // until chunk c + 1 has its inputs, and stored just before the loads of
    // chunk c + 2 are issued: a store queued behind the prefetch would make
    // the next wait for inputs wait for the store's completion as well.
    f32x4 o_pend[4];
    int64_t tc_pend = 0;
    int nt_pend = 0;
    auto store_o = [&]() {
        const Rsrc ro = chunk_rsrc(t.o, tc_pend, nt_pend, H, h, kRowOut);
        #pragma unroll
        for (int tb = 0; tb < 4; ++tb)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o_pend[tb]), ro, off_out[tb], 0, 0);
    };

    ChunkRegs<kU2> P;
    if (n_chunks > 0) issue_loads(P, it.t0);

    for (int c = 0; c < n_chunks; ++c) {
        const int64_t tc = it.t0 + (int64_t)c * kChunk;
        const int nt = (int)min<int64_t>(kChunk, it.t1 - tc);

        // Wave priority falls with progress through the segment: the two
        // workgroups sharing a CU then advance together (instead of the older
        // one finishing first and leaving the CU half idle at the end).
        switch ((4 * c) / n_chunks) {
        case 0: __builtin_amdgcn_s_setprio(3); break;
        case 1: __builtin_amdgcn_s_setprio(2); break;
        case 2: __builtin_amdgcn_s_setprio(1); break;
        default: __builtin_amdgcn_s_setprio(0); break;
        }

        // ---- stage this chunk's rows; prefetch the next chunk --------------------
        #pragma unroll
        for (int m = 0; m < 2; ++m) {
            lds_write_b128(sm.v, lb.vw + 64 * 32 * m, P.v[m]);
            lds_write_b128(sm.stage[1], st_wr[m], P.k[m]);
            lds_write_b128(sm.stage[2], st_wr[m], P.w[m]);
            if (M == Mode::Main) lds_write_b128(sm.stage[0], st_wr[m], P.r[m]);
            if constexpr (kU2) lds_write_b128(sm.stage[3], st_wr[m], P.u2[m]);
        }
        if (M == Mode::Main && c > 0) store_o();
        if (c + 1 < n_chunks) issue_loads(P, tc + kChunk);
        __syncthreads();

        // ---- r, k, w of this lane's 4 tokens x 4 channels from the staging tiles ----
        u32x2 pr[4], pk[4], pw[4];
        #pragma unroll
        for (int a = 0; a < 4; ++a) {
            pk[a] = lds_read_b64(sm.stage[1], st_rd[a]);
            pw[a] = lds_read_b64(sm.stage[2], st_rd[a]);
            if (M == Mode::Main) pr[a] = lds_read_b64(sm.stage[0], st_rd[a]);
        }
        u32x2 pu2[4];
        if constexpr (kU2) {
            #pragma unroll
            for (int tb = 0; tb < 4; ++tb) pu2[tb] = lds_read_b64(sm.stage[3], st_u2[tb]);
        }
        if (nt < kChunk) {                      // partial last chunk: w = 1 on padding rows
            constexpr unsigned kPad = LOGD ? kNegInfPair : kOnePair;
            #pragma unroll
            for (int a = 0; a < 4; ++a)
                if (4 * i16 + a >= nt) pw[a] = u32x2{kPad, kPad};
        }
        float lam[4][4], kk_[4][4], rr[4][4];
        #pragma unroll
        for (int a = 0; a < 4; ++a) {
            lam[a][0] = bf16_lo(pw[a].x); lam[a][1] = bf16_hi(pw[a].x);
            lam[a][2] = bf16_lo(pw[a].y); lam[a][3] = bf16_hi(pw[a].y);
            kk_[a][0] = bf16_lo(pk[a].x); kk_[a][1] = bf16_hi(pk[a].x);
            kk_[a][2] = bf16_lo(pk[a].y); kk_[a][3] = bf16_hi(pk[a].y);
            if (M == Mode::Main) {
                rr[a][0] = bf16_lo(pr[a].x); rr[a][1] = bf16_hi(pr[a].x);
                rr[a][2] = bf16_lo(pr[a].y); rr[a][3] = bf16_hi(pr[a].y);
            }
        }

        // ---- pre-processing: decay prefix, rescaled operands, bonus ----------
        if (M == Mode::Main) {
            // Products of the decays from the chunk start, P_t = w_0 ... w_t per key
            // channel: r~_t = r_t P_{t-1} and k~_s = k_s / P_s multiply to the decay
            // w_{s+1} ... w_{t-1} of the state equation.  lam holds the decay
            // inputs (w, or d); pw becomes the in-lane inclusive products.
            float pw[4][4];
            #pragma unroll
            for (int a = 0; a < 4; ++a)
                #pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float x = lam[a][q];
                    const float e = LOGD ? __builtin_amdgcn_exp2f(x * kLog2e) : 0.f;   // exp(d)
                    if (C2) kk_[a][q] *= one_minus_w<LOGD>(x, e);
                    pw[a][q] = LOGD ? __builtin_amdgcn_exp2f(-e * kLog2e) : x;
                }
            // in-lane products over 4 tokens, then across the 16 lanes: excl =
            // P before the lane's first token, total = P_63
            float excl[4], total[4];
            bool stiff = false;
            #pragma unroll
            for (int q = 0; q < 4; ++q) {
                pw[1][q] *= pw[0][q];
                pw[2][q] *= pw[1][q];
                pw[3][q] *= pw[2][q];
                const float incl = row_prod16(pw[3][q]);
                excl[q] = row_prev(incl);
                total[q] = row_bcast<15>(incl);
                stiff |= !(total[q] >= kMinChunkDecay);
            }
            stiff = __any(stiff);
            if (lane == 0) sm.stiff[wave] = stiff ? 1 : 0;
            if (i16 == 15) {
                #pragma unroll
                for (int q = 0; q < 4; ++q) sm.row_dec[c0 + q] = total[q];
            }
            float bp[4];
            #pragma unroll
            for (int a = 0; a < 4; ++a) {
                float rs[4], ks[4];
                bp[a] = 0.f;
                #pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float p_prev = a == 0 ? excl[q] : excl[q] * pw[a - 1][q];   // P_{t-1}
                    const float p_cur = excl[q] * pw[a][q];                            // P_t
                    rs[q] = rr[a][q] * p_prev;
                    ks[q] = kk_[a][q] * __builtin_amdgcn_rcpf(p_cur);
                    if (!C2) bp[a] += rr[a][q] * u4[q] * kk_[a][q];
                }
                u32x2 rh, rl, kh, kl;
                split4(rs[0], rs[1], rs[2], rs[3], rh, rl);
                split4(ks[0], ks[1], ks[2], ks[3], kh, kl);
                lds_write_b64(sm.rt_hi, lb.pw_rt[a], rh);
                lds_write_b64(sm.rt_lo, lb.pw_rt[a], rl);
                lds_write_b64(sm.kt_hi, lb.pw_kt[a], kh);
                lds_write_b64(sm.kt_lo, lb.pw_kt[a], kl);
                if (!C2) bp[a] = sum_rows4(bp[a]);
            }
            if (!C2 && grp == 0) {
                f32x4 b4 = {bp[0], bp[1], bp[2], bp[3]};
                *reinterpret_cast<f32x4 *>(&sm.bonus_part[wave][4 * i16]) = b4;
            }
        } else {
            // State pass: log2 decays relative to the chunk end, k~_s = k_s
            // 2^{Lam_63 - Lam_s} <= k_s (no factor exceeds 1, so it needs no
            // token-serial fallback).  lam holds the decay inputs (w, or d).
            #pragma unroll
            for (int a = 0; a < 4; ++a)
                #pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float x = lam[a][q];
                    const float e = LOGD ? __builtin_amdgcn_exp2f(x * kLog2e) : 0.f;   // exp(d)
                    if (C2) kk_[a][q] *= one_minus_w<LOGD>(x, e);
                    lam[a][q] = fmaxf(LOGD ? -e * kLog2e : __builtin_amdgcn_logf(x), kLog2Floor);
                }
            // inclusive prefix over the chunk: in-lane over 4 tokens, then across
            // the 16 lanes; lam becomes Lam_t - Lam_63
            float total[4];
            #pragma unroll
            for (int q = 0; q < 4; ++q) {
                lam[1][q] += lam[0][q];
                lam[2][q] += lam[1][q];
                lam[3][q] += lam[2][q];
                const float incl = row_scan16(lam[3][q]);
                total[q] = row_bcast<15>(incl);                         // Lam_63
                const float off = (incl - lam[3][q]) - total[q];
                #pragma unroll
                for (int a = 0; a < 4; ++a) lam[a][q] += off;
            }
            if (i16 == 15) {
                #pragma unroll
                for (int q = 0; q < 4; ++q) {
                    sm.row_dec[c0 + q] = __builtin_amdgcn_exp2f(total[q]);
                    lam_seg[q] += total[q];
                }
            }
            #pragma unroll
            for (int a = 0; a < 4; ++a) {
                float ks[4];
                #pragma unroll
                for (int q = 0; q < 4; ++q)
                    ks[q] = kk_[a][q] * __builtin_amdgcn_exp2f(-lam[a][q]);   // Lam_63 - Lam_t
                u32x2 kh, kl;
                split4(ks[0], ks[1], ks[2], ks[3], kh, kl);
                lds_write_b64(sm.kt_hi, lb.pw_kt[a], kh);
                lds_write_b64(sm.kt_lo, lb.pw_kt[a], kl);
            }
        }
        __syncthreads();

        // value operand, shared by the in-chunk product and the state update:
        // lane (i16, grp) holds v[K slots of step kk][16*wave + i16]
        bf16x8 vop[2];
        vop[0] = col_op(sm.v, lb.tr_v, 0);
        vop[1] = col_op(sm.v, lb.tr_v, 1);

        if (M == Mode::State) {
            f32x4 p[4];
            #pragma unroll
            for (int ib = 0; ib < 4; ++ib) p[ib] = f32x4{0.f, 0.f, 0.f, 0.f};
            #pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                bf16x8 k_hi[4], k_lo[4];
                #pragma unroll
                for (int ib = 0; ib < 4; ++ib) {
                    k_hi[ib] = kt_col_op(sm.kt_hi, lb.tr_kt[ib], kk);
                    k_lo[ib] = kt_col_op(sm.kt_lo, lb.tr_kt[ib], kk);
                }
                #pragma unroll
                for (int ib = 0; ib < 4; ++ib) p[ib] = mfma(k_hi[ib], vop[kk], p[ib]);
                #pragma unroll
                for (int ib = 0; ib < 4; ++ib) p[ib] = mfma(k_lo[ib], vop[kk], p[ib]);
            }
            #pragma unroll
            for (int ib = 0; ib < 4; ++ib) {
                const f32x4 dec = *reinterpret_cast<const f32x4 *>(&sm.row_dec[16 * ib + 4 * grp]);
                #pragma unroll
                for (int e = 0; e < 4; ++e) S[ib][e] = dec[e] * S[ib][e] + p[ib][e];
            }
            __syncthreads();
            continue;
        }

        const bool stiff = (sm.stiff[0] | sm.stiff[1] | sm.stiff[2] | sm.stiff[3]) != 0;
        f32x4 acc[4];
        if (stiff) {
            // exact token-by-token evaluation of this chunk (rare path); raw
            // r, k, w of this lane's 16 state rows come straight from memory;
            // outputs are staged as fp32 [t][j] in the r~ planes, which this
            // path does not read and the next chunk rewrites (the A planes
            // must keep their zero tiles)
            float *o_stage = reinterpret_cast<float *>(sm.rt_hi);
            for (int tt = 0; tt < nt; ++tt) {
                const size_t base = ((size_t)(tc + tt) * H + h) * kHeadDim;
                float part = 0.f;
                float kv[4][4], wv[4][4];
                #pragma unroll
                for (int ib = 0; ib < 4; ++ib) {
                    const size_t off = base + 16 * ib + 4 * grp;
                    const u32x2 a = *reinterpret_cast<const u32x2 *>(gr + off);
                    const u32x2 b = *reinterpret_cast<const u32x2 *>(gk + off);
                    const u32x2 d = *reinterpret_cast<const u32x2 *>(gw + off);
                    const float rv[4] = {bf16_lo(a.x), bf16_hi(a.x), bf16_lo(a.y), bf16_hi(a.y)};
                    kv[ib][0] = bf16_lo(b.x); kv[ib][1] = bf16_hi(b.x); kv[ib][2] = bf16_lo(b.y); kv[ib][3] = bf16_hi(b.y);
                    wv[ib][0] = bf16_lo(d.x); wv[ib][1] = bf16_hi(d.x); wv[ib][2] = bf16_lo(d.y); wv[ib][3] = bf16_hi(d.y);
                    #pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        part += rv[e] * S[ib][e];
                        const float x = wv[ib][e];
                        const float ex = LOGD ? __builtin_amdgcn_exp2f(x * kLog2e) : 0.f;
                        if (C2) kv[ib][e] *= one_minus_w<LOGD>(x, ex);
                        if (LOGD) wv[ib][e] = __builtin_amdgcn_exp2f(-ex * kLog2e);
                    }
                }
                part = sum_rows4(part);
                const unsigned vbits = sm.v[off_v(tt, 16 * wave + i16)];
                const float vj = __uint_as_float(vbits << 16);
                const float b = C2 ? 0.f : sm.bonus_part[0][tt] + sm.bonus_part[1][tt] +
                                           sm.bonus_part[2][tt] + sm.bonus_part[3][tt];
                if (grp == (tt & 3)) o_stage[tt * kHeadDim + 16 * wave + i16] = part + b * vj;
                #pragma unroll
                for (int ib = 0; ib < 4; ++ib)
                    #pragma unroll
                    for (int e = 0; e < 4; ++e) S[ib][e] = wv[ib][e] * S[ib][e] + kv[ib][e] * vj;
            }
            __syncthreads();
            #pragma unroll
            for (int tb = 0; tb < 4; ++tb)
                acc[tb] = *reinterpret_cast<const f32x4 *>(&o_stage[(16 * tb + i16) * kHeadDim + 16 * wave + 4 * grp]);
        } else {
        // ---- in-chunk matrix A: 10 lower 16x16 tiles spread over the waves -------
        // (the staging tiles share the A planes: the zero tiles above the
        // diagonal ones that the A.v product reads are rewritten every chunk)
        if (wave == 2 || wave == 3) {
            const int TB = wave == 2 ? 0 : 2, SB = TB + 1;
            const u32x2 z = {0u, 0u};
            lds_write_b64(sm.a_hi, lb.aw[SB] + 1024 * TB, z);
            lds_write_b64(sm.a_lo, lb.aw[SB] + 1024 * TB, z);
        }
        if (wave == 0) {
            const int TB[3] = {0, 1, 2}, SB[3] = {0, 0, 0};
            a_tiles<!C2, 3>(sm, lb, TB, SB, i16, grp);
        } else if (wave == 1) {
            const int TB[3] = {1, 2, 3}, SB[3] = {1, 1, 0};
            a_tiles<!C2, 3>(sm, lb, TB, SB, i16, grp);
        } else if (wave == 2) {
            const int TB[2] = {2, 3}, SB[2] = {2, 1};
            a_tiles<!C2, 2>(sm, lb, TB, SB, i16, grp);
        } else {
            const int TB[2] = {3, 3}, SB[2] = {3, 2};
            a_tiles<!C2, 2>(sm, lb, TB, SB, i16, grp);
        }

        // ---- read-out of the carried state: o^T = S^T r~^T ---------------------------
        {
            bf16x8 s_hi[2], s_lo[2];
            #pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                unsigned hi[4], lo[4];
                #pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const int ib = 2 * kk + half;
                    const HiLo x = split2(S[ib][0], S[ib][1]);
                    const HiLo y = split2(S[ib][2], S[ib][3]);
                    hi[2 * half] = x.hi; lo[2 * half] = x.lo;
                    hi[2 * half + 1] = y.hi; lo[2 * half + 1] = y.lo;
                }
                const u32x4 h4 = {hi[0], hi[1], hi[2], hi[3]}, l4 = {lo[0], lo[1], lo[2], lo[3]};
                s_hi[kk] = as_bf16x8(h4);
                s_lo[kk] = as_bf16x8(l4);
            }
            #pragma unroll
            for (int tb = 0; tb < 4; ++tb) acc[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
            #pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                bf16x8 r_hi[4], r_lo[4];
                #pragma unroll
                for (int tb = 0; tb < 4; ++tb) {
                    r_hi[tb] = rt_op(sm.rt_hi, lb.ro_x, tb, kk);
                    r_lo[tb] = rt_op(sm.rt_lo, lb.ro_x, tb, kk);
                }
                #pragma unroll
                for (int tb = 0; tb < 4; ++tb) acc[tb] = mfma(s_hi[kk], r_hi[tb], acc[tb]);
                #pragma unroll
                for (int tb = 0; tb < 4; ++tb) acc[tb] = mfma(s_hi[kk], r_lo[tb], acc[tb]);
                #pragma unroll
                for (int tb = 0; tb < 4; ++tb) acc[tb] = mfma(s_lo[kk], r_hi[tb], acc[tb]);
            }
        }
        // ---- state update: S = diag(2^Lam63) S + diag(2^{Lam63-R}) k~^T v --------
        // (the read-out above has taken the old S; k~ and v are ready since B1)
        {
            f32x4 p[4];
            #pragma unroll
            for (int ib = 0; ib < 4; ++ib) p[ib] = f32x4{0.f, 0.f, 0.f, 0.f};
            #pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                bf16x8 k_hi[4], k_lo[4];
                #pragma unroll
                for (int ib = 0; ib < 4; ++ib) {
                    k_hi[ib] = kt_col_op(sm.kt_hi, lb.tr_kt[ib], kk);
                    k_lo[ib] = kt_col_op(sm.kt_lo, lb.tr_kt[ib], kk);
                }
                #pragma unroll
                for (int ib = 0; ib < 4; ++ib) p[ib] = mfma(k_hi[ib], vop[kk], p[ib]);
                #pragma unroll
                for (int ib = 0; ib < 4; ++ib) p[ib] = mfma(k_lo[ib], vop[kk], p[ib]);
            }
            #pragma unroll
            for (int ib = 0; ib < 4; ++ib) {
                const f32x4 dec = *reinterpret_cast<const f32x4 *>(&sm.row_dec[16 * ib + 4 * grp]);
                #pragma unroll
                for (int e = 0; e < 4; ++e) S[ib][e] = dec[e] * (S[ib][e] + p[ib][e]);
            }
        }

        __syncthreads();

        // ---- in-chunk pairs: o^T += v^T A^T ----------------------------------------
        // A is zero for s >= 32 when t < 32: K step 1 only for row blocks 2, 3
        #pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            bf16x8 a_hi[4], a_lo[4];
            #pragma unroll
            for (int tb = 2 * kk; tb < 4; ++tb) {
                a_hi[tb] = row_op(sm.a_hi, lb.ro_x, tb, kk);
                a_lo[tb] = row_op(sm.a_lo, lb.ro_x, tb, kk);
            }
            #pragma unroll
            for (int tb = 2 * kk; tb < 4; ++tb) acc[tb] = mfma(vop[kk], a_hi[tb], acc[tb]);
            #pragma unroll
            for (int tb = 2 * kk; tb < 4; ++tb) acc[tb] = mfma(vop[kk], a_lo[tb], acc[tb]);
        }

        }

        // o of this chunk is stored early in the next iteration (see store_o)
        if constexpr (kU2) {                               // + u'_t (Finch-C2 output)
            #pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                acc[tb][0] += bf16_lo(pu2[tb].x);
                acc[tb][1] += bf16_hi(pu2[tb].x);
                acc[tb][2] += bf16_lo(pu2[tb].y);
                acc[tb][3] += bf16_hi(pu2[tb].y);
            }
        }
        #pragma unroll
        for (int tb = 0; tb < 4; ++tb) o_pend[tb] = acc[tb];
        tc_pend = tc;
        nt_pend = nt;
        __syncthreads();
    }
    if (M == Mode::Main && n_chunks > 0) store_o();

    // ---- outputs of the work item ------------------------------------------------
    if (M == Mode::State) {
        float *dst = ws.seg_state + (size_t)item * kSegStateFloats;
        #pragma unroll
        for (int ib = 0; ib < 4; ++ib)
            #pragma unroll
            for (int e = 0; e < 4; ++e)
                dst[(16 * ib + 4 * grp + e) * kHeadDim + 16 * wave + i16] = S[ib][e];
        if (i16 == 15) {
            #pragma unroll
            for (int q = 0; q < 4; ++q) dst[kHeadDim * kHeadDim + c0 + q] = lam_seg[q];
        }
    } else if (t.state_out && it.p == it.P - 1) {
        float *dst = t.state_out + ((size_t)it.n * H + h) * (kHeadDim * kHeadDim);
        #pragma unroll
        for (int ib = 0; ib < 4; ++ib)
            #pragma unroll
            for (int e = 0; e < 4; ++e)
                dst[(16 * ib + 4 * grp + e) * kHeadDim + 16 * wave + i16] = S[ib][e];
    }
}

// Combine of segment aggregates: the state entering segment p of a sequence is
//   S_{p+1} = diag(2^{Lam_p}) S_p + B_p,   S_0 = state_in (or zeros),
// a first-order recurrence per state entry.  Entries are independent: each
// thread chains four neighbouring entries of one row (16-byte accesses), the
// 4096 entries of a (sequence, head) spread over 16 one-wave workgroups,
// and the loads of a batch of segments are issued before the chain.
constexpr int kScanSlices = 16;
constexpr int kScanThreads = 64;      // 16 workgroups x 64 threads x 4 entries = 4096
constexpr int kScanBatch = 16;

__global__ __launch_bounds__(kScanThreads) void wkv_segment_scan_kernel(Geometry g, Tensors t, Workspace ws) {
    const int nh = blockIdx.x / kScanSlices;
    const int n = nh / g.H;
    const int h = nh % g.H;
    int first, P;
    if (g.uniform_T >= 0) {
        first = n * g.segs_per_seq;
        P = g.segs_per_seq;
    } else {
        first = g.seg_off[n];
        P = g.seg_off[n + 1] - first;
        if (first < 0 || first + P > g.n_seg) return;
    }
    if (P <= 1) return;
    const int idx = ((blockIdx.x % kScanSlices) * kScanThreads + threadIdx.x) * 4;   // entries [i][j..j+3]
    const int row = idx >> 6;
    f32x4 S = {0.f, 0.f, 0.f, 0.f};
    if (t.state_in)
        S = *reinterpret_cast<const f32x4 *>(t.state_in + ((size_t)n * g.H + h) * (kHeadDim * kHeadDim) + idx);
    for (int p0 = 0; p0 < P; p0 += kScanBatch) {
        f32x4 b[kScanBatch];
        float lam[kScanBatch];
        #pragma unroll
        for (int q = 0; q < kScanBatch; ++q) {
            b[q] = f32x4{0.f, 0.f, 0.f, 0.f};
            lam[q] = 0.f;
            if (p0 + q < P - 1) {
                const float *agg = ws.seg_state + ((size_t)(first + p0 + q) * g.H + h) * kSegStateFloats;
                b[q] = *reinterpret_cast<const f32x4 *>(agg + idx);
                lam[q] = agg[kHeadDim * kHeadDim + row];
            }
        }
        #pragma unroll
        for (int q = 0; q < kScanBatch; ++q) {
            if (p0 + q < P) {
                *reinterpret_cast<f32x4 *>(ws.seg_start + ((size_t)(first + p0 + q) * g.H + h) * kSegStartFloats + idx) = S;
                if (p0 + q < P - 1) {
                    const float d = __builtin_amdgcn_exp2f(lam[q]);
                    #pragma unroll
                    for (int e = 0; e < 4; ++e) S[e] = d * S[e] + b[q][e];
                }
            }
        }
    }
}

template <Mode M>
using ChunkKernel = void (*)(Geometry, Tensors, Workspace);

template <Mode M>
ChunkKernel<M> chunk_kernel_for(Variant v) {
    if (v.log_decay)
        return v.c2 ? wkv_chunk_kernel<M, true, true> : wkv_chunk_kernel<M, true, false>;
    return v.c2 ? wkv_chunk_kernel<M, false, true> : wkv_chunk_kernel<M, false, false>;
}

}  // namespace

hipError_t launch_segment_states(const Geometry &g, const Tensors &t, const Workspace &ws,
                                 Variant v, hipStream_t st) {
    const int64_t items = (int64_t)g.n_seg * g.H;
    if (items <= 0) return hipSuccess;
    hipLaunchKernelGGL(chunk_kernel_for<Mode::State>(v), dim3((unsigned)items), dim3(256), 0, st, g, t, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(wkv_segment_scan_kernel, dim3((unsigned)(g.n_seq * g.H * kScanSlices)), dim3(kScanThreads), 0, st,
                       g, t, ws);
    return hipGetLastError();
}

hipError_t launch_chunked_main(const Geometry &g, const Tensors &t, const Workspace &ws,
                               Variant v, hipStream_t st, KernelTiming tm) {
    const int64_t items = (int64_t)g.n_seg * g.H;
    if (items <= 0) return hipSuccess;
    const ChunkKernel<Mode::Main> kern = chunk_kernel_for<Mode::Main>(v);
    if (tm.start || tm.stop)
        hipExtLaunchKernelGGL(kern, dim3((unsigned)items), dim3(256), 0, st, tm.start, tm.stop, 0, g, t, ws);
    else
        hipLaunchKernelGGL(kern, dim3((unsigned)items), dim3(256), 0, st, g, t, ws);
    return hipGetLastError();
}

}  // namespace finch
