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

#include <atomic>

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
    const int bytes = rows > 0 ? ((rows - 1) * H + 1) * row_bytes : 0;   // no rows: every load reads 0
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

// x = hi + lo with hi = x rounded to the nearest bf16 (ties to even) and lo
// the remainder x - hi (exact in fp32) rounded the same way; returns packed
// pairs for two values.  Rounding hi to nearest rather than truncating it
// leaves a remainder of at most half a bf16 ulp, one bit more for lo: on the
// layer workload the chunked scan's errors against the fp64 recurrence fall
// from 1.8e-5 to 7.5e-6 (o) and 8.0e-6 to 4.8e-6 (state) in a CPU
// emulation of this arithmetic, for the same instruction count (one packing
// convert in place of one byte permute).
struct HiLo {
    unsigned hi, lo;
};
__device__ __forceinline__ HiLo split2(float x0, float x1) {
    const f32x2 x = {x0, x1};
    HiLo r;
    r.hi = __builtin_bit_cast(unsigned, __builtin_convertvector(x, bf16x2));   // {x1.hi, x0.hi}
    const float l0 = x0 - __uint_as_float(r.hi << 16);
    const float l1 = x1 - __uint_as_float(r.hi & 0xFFFF0000u);
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

// Inclusive product over the 16 lanes of each DPP row, in four steps.  A
// step multiplies x by the value SHIFT lanes earlier in the row, as one
// v_mul_f32_dpp whose lanes without such a predecessor are masked off (bound
// control clear) and so keep x.  (Written out because the compiler does not
// fold a DPP move with fill value 1 into a float multiply, which costs two
// more instructions per step.)  s_nop 1 gives the two wait states a DPP read
// needs after a VALU write of its source.
#define FINCH_ROW_MUL_SHR(x, SHIFT) \
    asm("s_nop 1\n\tv_mul_f32_dpp %0, %0, %0 row_shr:" #SHIFT " row_mask:0xf bank_mask:0xf" : "+v"(x))
__device__ __forceinline__ float row_prod16(float x) {
    FINCH_ROW_MUL_SHR(x, 1);
    FINCH_ROW_MUL_SHR(x, 2);
    FINCH_ROW_MUL_SHR(x, 4);
    FINCH_ROW_MUL_SHR(x, 8);
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

// The 64 x 64 fp32 state in the accumulator layout (lane (i16, grp) of wave
// w holds S[16*ib + 4*grp + e][16*w + i16]), from [key][value] memory (zeros
// for a null source).
__device__ __forceinline__ void load_public_state(const float *src, float (&S)[4][4], int tid = threadIdx.x) {
    const int wave = tid >> 6, i16 = tid & 15, grp = (tid & 63) >> 4;
    #pragma unroll
    for (int ib = 0; ib < 4; ++ib)
        #pragma unroll
        for (int e = 0; e < 4; ++e)
            S[ib][e] = src ? src[(16 * ib + 4 * grp + e) * kHeadDim + 16 * wave + i16] : 0.f;
}

// Wave priority falls with progress through a run of n chunks: workgroups
// sharing a CU then advance together, instead of the older one (which wins
// arbitration at equal priority) finishing first and leaving the CU half idle
// at the end.
__device__ __forceinline__ void set_progress_priority(int c, int n) {
    switch ((4 * c) / n) {
    case 0: __builtin_amdgcn_s_setprio(3); break;
    case 1: __builtin_amdgcn_s_setprio(2); break;
    case 2: __builtin_amdgcn_s_setprio(1); break;
    default: __builtin_amdgcn_s_setprio(0); break;
    }
}

// Where a segment's starting state comes from: begin() runs before the first
// chunk's loads are issued, load(S) after them.
struct PublicState {                      // state_in, a start state of the scan, or zeros (null)
    const float *src;
    __device__ void begin() {}
    __device__ void load(float (&S)[4][4]) { load_public_state(src, S); }
};

// One segment of one head, chunk by chunk, from the state that src.load(S)
// puts in registers: o of every token is stored and, with keep_state, S ends
// as the state after the segment (without it the last chunk skips the state
// update: a segment that does not end its sequence hands no state on, its
// successor starts from the combined start state).  The state is loaded after
// the first chunk's loads are issued, so that the first wait for inputs does
// not also wait for the state (load counters drain in issue order); it is
// first read after the pre-processing of that chunk.
template <bool LOGD, bool C2, typename SM, typename Src>
__device__ __forceinline__ void scan_chunks(SM &sm, const Tensors &t, int64_t seg_t0, int64_t seg_t1,
                                            int h, int H, Src &src, bool keep_state,
                                            float (&S)[4][4]) {
    constexpr bool kU2 = C2;                               // second value staged and added
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int i16 = lane & 15;
    const int grp = lane >> 4;
    const LdsBases lb = make_bases(tid);

    // pre-processing layout: channels c0..c0+3, tokens 4*i16 .. 4*i16+3
    const int c0 = 16 * wave + 4 * grp;
    f32x4 u4 = {0.f, 0.f, 0.f, 0.f};
    if (!C2) u4 = *reinterpret_cast<const f32x4 *>(t.u + (size_t)h * kHeadDim + c0);


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
        const int rows = (int)min<int64_t>(kChunk, seg_t1 - tc);
        const Rsrc rk = chunk_rsrc(t.k, tc, rows, H, h, kRowIn);
        const Rsrc rw = chunk_rsrc(t.w, tc, rows, H, h, kRowIn);
        const Rsrc rv = chunk_rsrc(t.v, tc, rows, H, h, kRowIn);
        {
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

    const int64_t n_tok = seg_t1 - seg_t0;
    const int n_chunks = (int)((n_tok + kChunk - 1) / kChunk);
    // o of chunk c (acc[tb][e] = o[16*tb + i16][16*wave + 4*grp + e]) is held
    // until chunk c + 1 has its inputs, and stored just before the loads of
    // chunk c + 2 are issued: a store queued behind the prefetch would make
    // the next wait for inputs wait for the store's completion as well.
    f32x4 o_pend[4];
    int64_t tc_pend = 0;
    int nt_pend = 0;
    auto store_o = [&]() {
        if (t.o_bf16) {                                  // 4 bf16 (RNE) per lane and row
            const Rsrc ro = chunk_rsrc(t.o, tc_pend, nt_pend, H, h, kRowIn);
            #pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                const f32x2 a = {o_pend[tb][0], o_pend[tb][1]}, b = {o_pend[tb][2], o_pend[tb][3]};
                const u32x2 pk = {__builtin_bit_cast(unsigned, __builtin_convertvector(a, bf16x2)),
                                  __builtin_bit_cast(unsigned, __builtin_convertvector(b, bf16x2))};
                __builtin_amdgcn_raw_buffer_store_b64(pk, ro, off_out[tb] / 2, 0, 0);
            }
        } else {
            const Rsrc ro = chunk_rsrc(t.o, tc_pend, nt_pend, H, h, kRowOut);
            #pragma unroll
            for (int tb = 0; tb < 4; ++tb)
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o_pend[tb]), ro, off_out[tb], 0, 0);
        }
    };

    ChunkRegs<kU2> P;
    src.begin();
    if (n_chunks > 0) issue_loads(P, seg_t0);
    src.load(S);

    for (int c = 0; c < n_chunks; ++c) {
        const int64_t tc = seg_t0 + (int64_t)c * kChunk;
        const int nt = (int)min<int64_t>(kChunk, seg_t1 - tc);

        set_progress_priority(c, n_chunks);

        // ---- stage this chunk's rows; prefetch the next chunk --------------------
        #pragma unroll
        for (int m = 0; m < 2; ++m) {
            lds_write_b128(sm.v, lb.vw + 64 * 32 * m, P.v[m]);
            lds_write_b128(sm.stage[1], st_wr[m], P.k[m]);
            lds_write_b128(sm.stage[2], st_wr[m], P.w[m]);
            lds_write_b128(sm.stage[0], st_wr[m], P.r[m]);
            if constexpr (kU2) lds_write_b128(sm.stage[3], st_wr[m], P.u2[m]);
        }
        if (c > 0) store_o();
        if (c + 1 < n_chunks) issue_loads(P, tc + kChunk);
        __syncthreads();

        // ---- r, k, w of this lane's 4 tokens x 4 channels from the staging tiles ----
        u32x2 pr[4], pk[4], pw[4];
        #pragma unroll
        for (int a = 0; a < 4; ++a) {
            pk[a] = lds_read_b64(sm.stage[1], st_rd[a]);
            pw[a] = lds_read_b64(sm.stage[2], st_rd[a]);
            pr[a] = lds_read_b64(sm.stage[0], st_rd[a]);
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
            rr[a][0] = bf16_lo(pr[a].x); rr[a][1] = bf16_hi(pr[a].x);
            rr[a][2] = bf16_lo(pr[a].y); rr[a][3] = bf16_hi(pr[a].y);
        }

        // ---- pre-processing: decay prefix, rescaled operands, bonus ----------
        {
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
        }
        __syncthreads();

        // value operand, shared by the in-chunk product and the state update:
        // lane (i16, grp) holds v[K slots of step kk][16*wave + i16]
        bf16x8 vop[2];
        vop[0] = col_op(sm.v, lb.tr_v, 0);
        vop[1] = col_op(sm.v, lb.tr_v, 1);


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
        if (keep_state || c + 1 < n_chunks) {
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
    if (n_chunks > 0) store_o();

}

// LDS of the state pass, 42.7 KB (three workgroups per compute unit).  The
// k~ planes have space of their own rather than sharing the staging tile's:
// sharing saves 16 KB but needs one more barrier per chunk (every staged row
// read before a plane is written), which measured slower on long segments.
struct SmemState {
    uint16_t v[kTileElems];                      // values of the chunk
    uint16_t kt_hi[kTileElems];                  // k~ = k 2^{Lam_63 - Lam_s}, bf16 hi/lo planes
    uint16_t kt_lo[kTileElems];
    uint16_t stage[2][kStageElems];              // raw k, w rows of the chunk
};
static_assert(sizeof(SmemState) <= 53 * 1024, "three state workgroups per CU");

// The state pass over one run of tokens (zero start): S ends as the run's
// aggregate B = sum_s diag(P_end / P_s) k_s^T v_s and lam_seg (lanes with
// i16 == 15, channels c0 .. c0+3) as its total log2-decay.  The sum does not
// depend on the order of its terms, so the chunks are taken from the last to
// the first: each chunk's k~ carries its whole decay to the run end (the
// log2-decay of the later chunks, lam_after, plus its own to the chunk end),
// the products accumulate into S with no rescaling, and the run's first
// chunk is read last, so a chunked scan of the same tokens that follows on
// the same XCD finds its first inputs in L2.  One chunk is prefetched ahead
// (keeping two or three chunks of each item in flight was measured slower).
template <bool LOGD, bool C2>
__device__ __forceinline__ void state_run(SmemState &sm, const Tensors &t, int64_t t0, int64_t t1, int h, int H,
                                          float (&S)[4][4], float (&lam_seg)[4]) {
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int i16 = lane & 15;
    const int grp = lane >> 4;
    const LdsBases lb = make_bases(tid);
    const int ld_row = tid >> 3;
    const int ld_col = (tid & 7) * 8;
    constexpr int kRowIn = kHeadDim * 2;
    int off_vin[2], st_wr[2], st_rd[4];
    #pragma unroll
    for (int m = 0; m < 2; ++m) {
        off_vin[m] = (ld_row + 32 * m) * H * kRowIn + 2 * ld_col;
        st_wr[m] = off_stage(ld_row + 32 * m, tid & 7);
    }
    #pragma unroll
    for (int a = 0; a < 4; ++a) st_rd[a] = off_stage(4 * i16 + a, 2 * wave + (grp >> 1)) + 4 * (grp & 1);

    u32x4 Qk[2], Qw[2], Qv[2];
    auto issue = [&](int64_t tc) {
        // integer clamps: the device max() overload for 64-bit integers goes
        // through double arithmetic on the vector unit, which would leave the
        // record count (and so the buffer resource) in vector registers and
        // turn every load into a loop over distinct resources
        const int64_t left = t1 - tc;
        const int rows = left <= 0 ? 0 : (left >= kChunk ? kChunk : (int)left);
        const Rsrc rk = chunk_rsrc(t.k, tc, rows, H, h, kRowIn);
        const Rsrc rw = chunk_rsrc(t.w, tc, rows, H, h, kRowIn);
        const Rsrc rv = chunk_rsrc(t.v, tc, rows, H, h, kRowIn);
        #pragma unroll
        for (int m = 0; m < 2; ++m) {
            Qk[m] = __builtin_amdgcn_raw_buffer_load_b128(rk, off_vin[m], 0, 0);
            Qw[m] = __builtin_amdgcn_raw_buffer_load_b128(rw, off_vin[m], 0, 0);
            Qv[m] = __builtin_amdgcn_raw_buffer_load_b128(rv, off_vin[m], 0, 0);
        }
    };

    const int n_chunks = (int)((t1 - t0 + kChunk - 1) / kChunk);
    float lam_after[4] = {0.f, 0.f, 0.f, 0.f};  // log2-decay from the current chunk's end to the run end
    if (n_chunks > 0) issue(t0 + (int64_t)(n_chunks - 1) * kChunk);
    for (int i = 0; i < n_chunks; ++i) {
        const int c = n_chunks - 1 - i;
        const int64_t tc = t0 + (int64_t)c * kChunk;
        const int nt = (int)min<int64_t>(kChunk, t1 - tc);
        set_progress_priority(i, n_chunks);
        #pragma unroll
        for (int m = 0; m < 2; ++m) {
            lds_write_b128(sm.v, lb.vw + 64 * 32 * m, Qv[m]);
            lds_write_b128(sm.stage[0], st_wr[m], Qk[m]);
            lds_write_b128(sm.stage[1], st_wr[m], Qw[m]);
        }
        if (c > 0) issue(tc - kChunk);
        __syncthreads();
        u32x2 pk[4], pw[4];
        #pragma unroll
        for (int a = 0; a < 4; ++a) {
            pk[a] = lds_read_b64(sm.stage[0], st_rd[a]);
            pw[a] = lds_read_b64(sm.stage[1], st_rd[a]);
        }
        if (nt < kChunk) {                      // partial chunk: w = 1 on padding rows
            constexpr unsigned kPad = LOGD ? kNegInfPair : kOnePair;
            #pragma unroll
            for (int a = 0; a < 4; ++a)
                if (4 * i16 + a >= nt) pw[a] = u32x2{kPad, kPad};
        }
        float lam[4][4], kk_[4][4];
        #pragma unroll
        for (int a = 0; a < 4; ++a) {
            lam[a][0] = bf16_lo(pw[a].x); lam[a][1] = bf16_hi(pw[a].x);
            lam[a][2] = bf16_lo(pw[a].y); lam[a][3] = bf16_hi(pw[a].y);
            kk_[a][0] = bf16_lo(pk[a].x); kk_[a][1] = bf16_hi(pk[a].x);
            kk_[a][2] = bf16_lo(pk[a].y); kk_[a][3] = bf16_hi(pk[a].y);
        }
        // log2 decays relative to the chunk end, k~_s = k_s 2^{Lam_63 - Lam_s}
        // <= k_s (no factor exceeds 1, so no token-serial fallback is needed)
        #pragma unroll
        for (int a = 0; a < 4; ++a)
            #pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float x = lam[a][q];
                const float e = LOGD ? __builtin_amdgcn_exp2f(x * kLog2e) : 0.f;   // exp(d)
                if (C2) kk_[a][q] *= one_minus_w<LOGD>(x, e);
                lam[a][q] = fmaxf(LOGD ? -e * kLog2e : __builtin_amdgcn_logf(x), kLog2Floor);
            }
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
        #pragma unroll
        for (int a = 0; a < 4; ++a) {
            float ks[4];
            #pragma unroll
            for (int q = 0; q < 4; ++q) ks[q] = kk_[a][q] * __builtin_amdgcn_exp2f(lam_after[q] - lam[a][q]);
            u32x2 kh, kl;
            split4(ks[0], ks[1], ks[2], ks[3], kh, kl);
            lds_write_b64(sm.kt_hi, lb.pw_kt[a], kh);
            lds_write_b64(sm.kt_lo, lb.pw_kt[a], kl);
        }
        #pragma unroll
        for (int q = 0; q < 4; ++q) lam_after[q] += total[q];
        __syncthreads();
        bf16x8 vop[2];
        vop[0] = col_op(sm.v, lb.tr_v, 0);
        vop[1] = col_op(sm.v, lb.tr_v, 1);
        f32x4 pp[4];
        #pragma unroll
        for (int ib = 0; ib < 4; ++ib) pp[ib] = f32x4{S[ib][0], S[ib][1], S[ib][2], S[ib][3]};
        #pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            bf16x8 k_hi[4], k_lo[4];
            #pragma unroll
            for (int ib = 0; ib < 4; ++ib) {
                k_hi[ib] = kt_col_op(sm.kt_hi, lb.tr_kt[ib], kk);
                k_lo[ib] = kt_col_op(sm.kt_lo, lb.tr_kt[ib], kk);
            }
            #pragma unroll
            for (int ib = 0; ib < 4; ++ib) pp[ib] = mfma(k_hi[ib], vop[kk], pp[ib]);
            #pragma unroll
            for (int ib = 0; ib < 4; ++ib) pp[ib] = mfma(k_lo[ib], vop[kk], pp[ib]);
        }
        #pragma unroll
        for (int ib = 0; ib < 4; ++ib)
            #pragma unroll
            for (int e = 0; e < 4; ++e) S[ib][e] = pp[ib][e];
        __syncthreads();                       // planes and values read before the next staging
    }
    if (i16 == 15) {
        #pragma unroll
        for (int q = 0; q < 4; ++q) lam_seg[q] = lam_after[q];
    }
}

__device__ __forceinline__ void store_public_state(float *dst, const float (&S)[4][4], int tid = threadIdx.x) {
    const int wave = tid >> 6, i16 = tid & 15, grp = (tid & 63) >> 4;
    #pragma unroll
    for (int ib = 0; ib < 4; ++ib)
        #pragma unroll
        for (int e = 0; e < 4; ++e)
            dst[(16 * ib + 4 * grp + e) * kHeadDim + 16 * wave + i16] = S[ib][e];
}

// State pass: the zero-start aggregate of every run of every segment but the
// last of its sequence: B (D*D, [key][value]) followed by the run's total
// log2-decay per key channel (D), stored at index ((s - n) * runs + r) * H + h
// for run r of global segment s of sequence n.  A segment is cut into several
// runs only when its items alone would leave most of the device idle (the
// planner's choice); where the items already fill it (four per compute unit
// at the 1.5B-class layer) shorter runs were measured slower.
template <bool LOGD, bool C2>
__global__ __launch_bounds__(256, 3) void wkv_state_kernel(Geometry g, Tensors t, Workspace ws) {
    __shared__ SmemState sm;
    const int item = blockIdx.x;
    const int h = item % g.H;
    const int q = item / g.H;
    const int seg = q / g.runs, r = q - seg * g.runs;
    const ItemRange it = decode_segment(g, seg);
    if (!it.valid || it.p == it.P - 1) return;           // the last segment's aggregate is unused
    if (ws.seg_state == nullptr) return;                 // a split the host did not plan
    // run r of the segment, clamped into it (integer clamps, see state_run)
    const int64_t a = it.t0 + (int64_t)r * g.run_len;
    const int64_t r0 = a < it.t1 ? a : it.t1;
    const int64_t r1 = it.t1 - r0 > g.run_len ? r0 + g.run_len : it.t1;
    float S[4][4], lam[4] = {0.f, 0.f, 0.f, 0.f};
    #pragma unroll
    for (int ib = 0; ib < 4; ++ib)
        #pragma unroll
        for (int e = 0; e < 4; ++e) S[ib][e] = 0.f;
    state_run<LOGD, C2>(sm, t, r0, r1, h, g.H, S, lam);
    float *dst = ws.seg_state + (((size_t)(seg - it.n) * g.runs + r) * g.H + h) * kSegStateFloats;
    store_public_state(dst, S);
    const int tid = threadIdx.x;
    if ((tid & 15) == 15) {
        const int c0 = 16 * (tid >> 6) + 4 * ((tid & 63) >> 4);
        #pragma unroll
        for (int q = 0; q < 4; ++q) dst[kHeadDim * kHeadDim + c0 + q] = lam[q];
    }
}

// Combine of run aggregates: over the runs j of a sequence in order,
//   S <- diag(2^{Lam_j}) S + B_j,   from S = state_in (or zeros),
// and S before the first run of segment p is the state entering segment p;
// a first-order recurrence per state entry.  Entries are independent: each
// thread chains four neighbouring entries of one row (16-byte accesses), the
// 4096 entries of a (sequence, head) spread over 16 one-wave workgroups,
// and the loads of a batch of runs are issued before the chain.
constexpr int kScanSlices = 16;
constexpr int kScanThreads = 64;      // 16 workgroups x 64 threads x 4 entries = 4096
constexpr int kScanBatch = 16;
static_assert(kScanSlices * kScanThreads == kScanGroupThreads, "scan launch size known to the planner");

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
    const int R = g.runs;
    const int steps = (P - 1) * R;                        // runs before the last segment
    const size_t agg0 = (size_t)(first - n) * R;          // first run of the sequence
    f32x4 S = {0.f, 0.f, 0.f, 0.f};
    if (t.state_in)
        S = *reinterpret_cast<const f32x4 *>(t.state_in + ((size_t)n * g.H + h) * (kHeadDim * kHeadDim) + idx);
    for (int j0 = 0; j0 < steps; j0 += kScanBatch) {
        f32x4 b[kScanBatch];
        float lam[kScanBatch];
        #pragma unroll
        for (int q = 0; q < kScanBatch; ++q) {
            b[q] = f32x4{0.f, 0.f, 0.f, 0.f};
            lam[q] = 0.f;
            if (j0 + q < steps) {
                const float *agg = ws.seg_state + ((agg0 + j0 + q) * g.H + h) * kSegStateFloats;
                b[q] = *reinterpret_cast<const f32x4 *>(agg + idx);
                lam[q] = agg[kHeadDim * kHeadDim + row];
            }
        }
        #pragma unroll
        for (int q = 0; q < kScanBatch; ++q) {
            const int j = j0 + q;
            if (j < steps) {
                if (j % R == 0)                          // the state entering segment j / R
                    *reinterpret_cast<f32x4 *>(ws.seg_start + ((size_t)(first + j / R) * g.H + h) * kSegStartFloats +
                                               idx) = S;
                const float d = __builtin_amdgcn_exp2f(lam[q]);
                #pragma unroll
                for (int e = 0; e < 4; ++e) S[e] = d * S[e] + b[q][e];
            }
        }
    }
    *reinterpret_cast<f32x4 *>(ws.seg_start + ((size_t)(first + P - 1) * g.H + h) * kSegStartFloats + idx) = S;
}

// The chunked scan: one workgroup per (segment, head), from the state that
// enters the segment (state_in for a sequence's first segment, else the
// combined start state of the segment scan).
template <bool LOGD, bool C2>
__global__ __launch_bounds__(256, 2) void wkv_chunk_kernel(Geometry g, Tensors t, Workspace ws) {
    using SM = Smem<C2 ? 4 : 3>;
    __shared__ SM sm;
    const int h = blockIdx.x % g.H;
    const int rank = blockIdx.x / g.H;
    const int seg = g.seg_rank ? g.seg_rank[rank] : rank;      // packed calls: longest first
    const ItemRange it = decode_segment(g, seg);
    if (!it.valid) return;
    // a split the host did not plan (device offsets differing from the host
    // copy) has no workspace behind it: leave the item alone
    if (it.P > 1 && ws.seg_start == nullptr) return;
    float S[4][4];
    const float *s_src = nullptr;
    if (it.P > 1)
        s_src = ws.seg_start + ((size_t)seg * g.H + h) * kSegStartFloats;
    else if (t.state_in)
        s_src = t.state_in + ((size_t)it.n * g.H + h) * (kHeadDim * kHeadDim);
    const bool keep = t.state_out && it.p == it.P - 1;
    PublicState src{s_src};
    scan_chunks<LOGD, C2>(sm, t, it.t0, it.t1, h, g.H, src, keep, S);
    if (keep)
        store_public_state(t.state_out + ((size_t)it.n * g.H + h) * (kHeadDim * kHeadDim), S);
}


// ---- one launch for split sequences ---------------------------------------------
//
// The state pass, the segment scan and the chunked scan of a split call as one
// grid of 2 * items workgroups, so that no kernel boundary separates them and
// the chunked scan of a segment starts as soon as a compute unit frees up.
// Workgroups [0, items) take the state role for item = blockIdx: for every
// segment but the last of its sequence, the zero-start aggregate B_p and its
// log2-decay, published to the workspace; then, once every aggregate of the
// (sequence, head) is there, each of its P - 1 state workgroups chains a
// share of the 4096 state entries through all segments,
//   S_{q+1} = diag(2^{Lam_q}) S_q + B_q,   S_0 = state_in (or zeros),
// and writes its share of every start state.  Workgroups [items, 2 * items)
// take the main role for item = blockIdx - items: the chunked scan of the
// segment, from state_in (first segment) or from the start state, which it
// waits for after issuing its first chunk's loads.
//
// Relay form (Relay = true): one workgroup per item takes the state role (if
// its segment has one) and then the main role of the same item.  Its chunked
// scan so needs no second dispatch, has its first chunk's loads in flight
// while the chain finishes, and reads that chunk's k, v, w soon after the
// state pass read them (it takes the run's chunks last to first), so they can
// still be in L2.  The first segments' chunked scans wait for their own
// state pass: starting them at once (with the last segment's workgroup taking
// segment 0's state pass) was measured slower, since they then take bandwidth
// from the state passes.  The host launches this form only when every item of
// the grid fits on the device at once.
//
// Waits.  A state workgroup waits only for the other state workgroups of its
// (sequence, head), and a main workgroup only for those.  Workgroups are
// dispatched in index order, every state workgroup precedes every main
// workgroup, and the host launches the two-role form only when all state
// workgroups fit on the device at once (the relay form only when all
// workgroups do), so every workgroup waited for is resident or finished.
// Each wait is bounded (g.wait_ticks) and marks the record's error word if the
// bound expires, so no launch can hang.
//
// Memory.  Everything handed between workgroups (aggregates, start states,
// counters) is written and read with agent-scope atomic accesses, which go
// through to the level that every XCD shares; a publisher waits for its
// stores to complete before it counts itself.  No cache-wide release or
// acquire is needed.  Waiters poll the counters of the per-(sequence, head)
// control record (SplitCtl) themselves, so the last arrival needs no second
// store to release them.  The counters of a call are reset by the last main
// workgroup of a later segment to finish, when every workgroup of the record
// has passed its waits, so no record is cleared between calls.
constexpr int kChainBatch = 16;                 // aggregates whose loads are issued together

__device__ __forceinline__ int ctl_load(int *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void ctl_store(int *p, int x) {
    __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float x_load(const float *p) {
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void x_store(float *p, float x) {
    __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Every thread: wait until its stores have completed, then meet the others,
// so that thread 0 may announce them.
__device__ __forceinline__ void complete_stores() {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
}
// Thread 0: count the workgroup in *ctr; returns the count before it.
__device__ __forceinline__ int ctl_add(int *ctr) {
    return __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Thread 0: wait until *ctr == n (bounded; on expiry the record is marked).
__device__ __forceinline__ void ctl_wait(int *ctr, int n, int *err, unsigned bound) {
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    while (ctl_load(ctr) != n) {
        __builtin_amdgcn_s_sleep(2);
        if (__builtin_amdgcn_s_memrealtime() - t0 > bound) {
            ctl_store(err, 1);
            return;
        }
    }
}

// Start state of a main-role workgroup: state_in (or zeros) for the first
// segment of a sequence, else the published start state.  Then the counter
// of written start-state slices is read before the first chunk's loads are
// issued, so that checking it waits for that one load only, and the state is
// read with agent-scope loads.
struct SplitStartState {
    SplitCtl *rec;                          // null: a first segment
    const float *first;                     // state_in of the sequence, or null
    const float *src;                       // published start state
    int n_state;                            // state workgroups of the (sequence, head)
    unsigned bound;                         // of the wait, in ticks of the 100 MHz clock
    int seen = 0;
    __device__ void begin() {
        if (rec && threadIdx.x == 0) seen = ctl_load(&rec->scanned);
    }
    __device__ void load(float (&S)[4][4]) {
        if (!rec) {
            load_public_state(first, S);
            return;
        }
        const int tid = threadIdx.x;
        if (tid == 0 && seen != n_state) ctl_wait(&rec->scanned, n_state, &rec->error, bound);
        __syncthreads();
        const int wave = tid >> 6, i16 = tid & 15, grp = (tid & 63) >> 4;
        #pragma unroll
        for (int ib = 0; ib < 4; ++ib)
            #pragma unroll
            for (int e = 0; e < 4; ++e) S[ib][e] = x_load(src + (16 * ib + 4 * grp + e) * kHeadDim + 16 * wave + i16);
    }
};

template <bool C2>
union SmemSplit {
    Smem<C2 ? 4 : 3> main;
    SmemState state;
};

template <bool LOGD, bool C2, bool Relay>
__global__ __launch_bounds__(256, 2) void wkv_split_kernel(Geometry g, Tensors t, Workspace ws) {
    __shared__ SmemSplit<C2> sm;
    const int items = g.n_seg * g.H;
    const bool state_role = Relay || (int)blockIdx.x < items;
    const int item = state_role ? (int)blockIdx.x : (int)blockIdx.x - items;
    const int h = item % g.H;
    const int seg = item / g.H;
    const ItemRange it = decode_segment(g, seg);
    if (!it.valid) return;
    const bool split = it.P > 1;
    // a split the host did not plan (device offsets differing from the host
    // copy) has no workspace behind it: leave the item alone
    if (split && (ws.ctl == nullptr || ws.seg_state == nullptr || ws.seg_start == nullptr)) return;
    const bool has_state = split && it.p < it.P - 1;       // the last segment's aggregate is unused
    if (!Relay && state_role && !has_state) return;
    const int tid = threadIdx.x;
    const int n_state = it.P - 1;
    const size_t slot = ((size_t)it.n * g.H + h) * (kHeadDim * kHeadDim);
    SplitCtl *rec = split ? ws.ctl + ((size_t)it.n * g.H + h) : nullptr;

    if (state_role && has_state) {
        float S[4][4], lam[4] = {0.f, 0.f, 0.f, 0.f};
        #pragma unroll
        for (int ib = 0; ib < 4; ++ib)
            #pragma unroll
            for (int e = 0; e < 4; ++e) S[ib][e] = 0.f;
        state_run<LOGD, C2>(sm.state, t, it.t0, it.t1, h, g.H, S, lam);
        // publish B_p ([key][value]) and its log2-decays
        const size_t agg0 = (size_t)(seg - it.p - it.n) * g.H + h;   // aggregate of segment 0
        float *dst = ws.seg_state + (agg0 + (size_t)it.p * g.H) * kSegStateFloats;
        {
            const int wave = tid >> 6, i16 = tid & 15, grp = (tid & 63) >> 4;
            #pragma unroll
            for (int ib = 0; ib < 4; ++ib)
                #pragma unroll
                for (int e = 0; e < 4; ++e)
                    x_store(dst + (16 * ib + 4 * grp + e) * kHeadDim + 16 * wave + i16, S[ib][e]);
            if (i16 == 15) {
                #pragma unroll
                for (int q = 0; q < 4; ++q) x_store(dst + kHeadDim * kHeadDim + 16 * wave + 4 * grp + q, lam[q]);
            }
        }
        complete_stores();
        if (tid == 0 && ctl_add(&rec->arrived) != n_state - 1)
            ctl_wait(&rec->arrived, n_state, &rec->error, g.wait_ticks);
        __syncthreads();
        // this workgroup's share of the chain: rows of 256 entries (one per
        // thread) numbered p, p + P - 1, ...; two rows at a time, their loads
        // issued together (with 15 state workgroups the first has two rows,
        // and the head's start states wait for the slowest share)
        const float *s_in = t.state_in ? t.state_in + slot : nullptr;
        const size_t start0 = (size_t)(seg - it.p) * g.H + h;         // start state of segment 0
        constexpr int kRows = (kHeadDim * kHeadDim) / 256;
        for (int sl = it.p; sl < kRows; sl += 2 * n_state) {
            const bool two = sl + n_state < kRows;
            const int e0 = 256 * sl + tid, e1 = e0 + 256 * n_state;
            float x0 = s_in ? s_in[e0] : 0.f;
            float x1 = s_in && two ? s_in[e1] : 0.f;
            for (int q0 = 0; q0 < n_state; q0 += kChainBatch) {
                float b0[kChainBatch], l0[kChainBatch], b1[kChainBatch], l1[kChainBatch];
                #pragma unroll
                for (int q = 0; q < kChainBatch; ++q) {
                    b0[q] = l0[q] = b1[q] = l1[q] = 0.f;
                    if (q0 + q < n_state) {
                        const float *agg = ws.seg_state + (agg0 + (size_t)(q0 + q) * g.H) * kSegStateFloats;
                        b0[q] = x_load(agg + e0);
                        l0[q] = x_load(agg + kHeadDim * kHeadDim + e0 / kHeadDim);
                        if (two) {
                            b1[q] = x_load(agg + e1);
                            l1[q] = x_load(agg + kHeadDim * kHeadDim + e1 / kHeadDim);
                        }
                    }
                }
                #pragma unroll
                for (int q = 0; q < kChainBatch; ++q) {
                    if (q0 + q < n_state) {
                        float *dst = ws.seg_start + (start0 + (size_t)(q0 + q + 1) * g.H) * kSegStartFloats;
                        const float d0 = __builtin_amdgcn_exp2f(l0[q]);
                        x0 = d0 * x0 + b0[q];
                        x_store(dst + e0, x0);
                        if (two) {
                            const float d1 = __builtin_amdgcn_exp2f(l1[q]);
                            x1 = d1 * x1 + b1[q];
                            x_store(dst + e1, x1);
                        }
                    }
                }
            }
        }
        complete_stores();
        if (tid == 0) ctl_add(&rec->scanned);
        if constexpr (!Relay) return;
        // relay: the main role follows; every thread has passed the barrier
        // above, so the state role's LDS is free
    }

    // main role
    const bool keep = t.state_out && it.p == it.P - 1;
    float S[4][4];
    const bool later = split && it.p > 0;
    SplitStartState src{later ? rec : nullptr, t.state_in ? t.state_in + slot : nullptr,
                        later ? ws.seg_start + (size_t)item * kSegStartFloats : nullptr, n_state,
                        g.wait_ticks};
    scan_chunks<LOGD, C2>(sm.main, t, it.t0, it.t1, h, g.H, src, keep, S);
    // the main workgroups of later segments count the call done: each has seen
    // every start state published, so every other use of the record in this
    // call is over (every wait passed) once all of them have arrived, and the
    // last resets its counters for the next call
    if (later && tid == 0 && ctl_add(&rec->done) == n_state - 1) {
        ctl_store(&rec->arrived, 0);
        ctl_store(&rec->scanned, 0);
        ctl_store(&rec->done, 0);
        ctl_add(&rec->epoch);
    }
    if (keep) store_public_state(t.state_out + slot, S);
}

// ---- producer/consumer form of the chunked scan (fixed-length batches) -------
//
// One workgroup of eight waves per compute unit and work item.  Waves 0-3
// (producers) load chunk j, stage it and write its pre-processed planes
// (r~, k~ hi/lo, v, bonus partial sums, chunk decay, stiff votes) into plane
// set j % 2, while waves 4-7 (consumers) run the matrix phases of chunk j - 1
// from the other set and store its o.  One workgroup barrier per step hands
// the sets over; each group orders its own LDS traffic with a counter barrier
// in LDS that the other group never waits on.  The consumers issue no loads
// (only o stores), so their stores never delay the producers' waits for
// inputs, and the producers' loads never delay the consumers.  The
// arithmetic of every chunk is that of scan_chunks.

struct PlaneSet {
    uint16_t v[kTileElems];
    uint16_t rt_hi[kTileElems];
    uint16_t rt_lo[kTileElems];
    uint16_t kt_hi[kTileElems];
    uint16_t kt_lo[kTileElems];
    alignas(16) float bonus_part[4][kChunk];
    alignas(16) float row_dec[kHeadDim];
    int stiff[4];
};
// the token-serial path stages 64 x 64 fp32 outputs across rt_hi and rt_lo
static_assert(offsetof(PlaneSet, rt_lo) == offsetof(PlaneSet, rt_hi) + sizeof(uint16_t) * kTileElems,
              "rt planes must be adjacent");

template <bool C2>
struct SmemPC {
    PlaneSet set[2];
    uint16_t a_hi[kTileElems];                     // in-chunk matrix A (consumers only)
    uint16_t a_lo[kTileElems];
    uint16_t stage[C2 ? 4 : 3][kStageElems];       // raw r, k, w (, u') rows (producers only)
    u32x2 u2[C2 ? 2 : 1][4][C2 ? 256 : 1];         // u' in the accumulator layout, per set
    int bar[2];                                    // counter barriers: producers, consumers
};
static_assert(sizeof(SmemPC<true>) <= 160 * 1024, "one producer/consumer workgroup per CU");

// What the consumer phases read: one plane set plus the A planes (the names
// a_tiles and the operand helpers expect).
struct PCView {
    uint16_t *v, *rt_hi, *rt_lo, *kt_hi, *kt_lo, *a_hi, *a_lo;
    float (*bonus_part)[kChunk];
    float *row_dec;
    int *stiff;
};

// Barrier of the four waves of one group: each wave's LDS traffic is complete
// (lgkmcnt 0) before it counts itself in, and a wave leaves once all four have
// counted in this many times.  Memory operations of other kinds are not
// waited for (the producers' prefetch loads stay in flight).
__device__ __forceinline__ void group_barrier(int *ctr, int &gen) {
    gen += 4;
    __builtin_amdgcn_s_waitcnt(0xC07F);            // lgkmcnt(0), vmcnt and expcnt unconstrained
    if ((threadIdx.x & 63) == 0) __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    while (__builtin_amdgcn_readfirstlane(__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) < gen)
        __builtin_amdgcn_s_sleep(1);
    __asm__ __volatile__("" ::: "memory");
}

// One work item: tokens [t0, t1) of head h, from the state at s_src (zeros if
// null); with keep_state S ends as the state after the item and is stored to
// state_dst.
template <bool LOGD, bool C2>
__device__ __forceinline__ void pc_item(SmemPC<C2> &sm, const Tensors &t, int64_t t0, int64_t t1, int h, int H,
                                        const float *s_src, float *state_dst) {
    constexpr bool kU2 = C2;
    const int tid = threadIdx.x;
    const bool producer = tid < 256;                 // waves 0-3 (wave-uniform)
    const int ltid = tid & 255;                      // index within the group
    const int wave = __builtin_amdgcn_readfirstlane(ltid >> 6);
    const int lane = tid & 63;
    const int i16 = lane & 15;
    const int grp = lane >> 4;
    const LdsBases lb = make_bases(ltid);
    const int c0 = 16 * wave + 4 * grp;              // pre-processing channels (producers)
    constexpr int kRowIn = kHeadDim * 2;
    constexpr int kRowOut = kHeadDim * 4;
    const int n_chunks = (int)((t1 - t0 + kChunk - 1) / kChunk);

    if (tid == 0) { sm.bar[0] = 0; sm.bar[1] = 0; }
    __syncthreads();
    int gen = 0;

    // ---- producer state ----------------------------------------------------------
    f32x4 u4 = {0.f, 0.f, 0.f, 0.f};
    const int ld_row = ltid >> 3;
    const int ld_col = (ltid & 7) * 8;
    int off_vin[2], st_wr[2], st_rd[4], st_u2[4];
    #pragma unroll
    for (int m = 0; m < 2; ++m) {
        off_vin[m] = (ld_row + 32 * m) * H * kRowIn + 2 * ld_col;
        st_wr[m] = off_stage(ld_row + 32 * m, ltid & 7);
    }
    #pragma unroll
    for (int a = 0; a < 4; ++a) st_rd[a] = off_stage(4 * i16 + a, 2 * wave + (grp >> 1)) + 4 * (grp & 1);
    #pragma unroll
    for (int tb = 0; tb < 4; ++tb) st_u2[tb] = off_stage(16 * tb + i16, 2 * wave + (grp >> 1)) + 4 * (grp & 1);
    ChunkRegs<kU2> P;
    auto issue_loads = [&](int64_t tc) {
        const int64_t left = t1 - tc;
        const int rows = left >= kChunk ? kChunk : (int)left;
        const Rsrc rk = chunk_rsrc(t.k, tc, rows, H, h, kRowIn);
        const Rsrc rw = chunk_rsrc(t.w, tc, rows, H, h, kRowIn);
        const Rsrc rv = chunk_rsrc(t.v, tc, rows, H, h, kRowIn);
        const Rsrc rr = chunk_rsrc(t.r, tc, rows, H, h, kRowIn);
        #pragma unroll
        for (int m = 0; m < 2; ++m) P.r[m] = __builtin_amdgcn_raw_buffer_load_b128(rr, off_vin[m], 0, 0);
        if constexpr (kU2) {
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

    // ---- consumer state ----------------------------------------------------------
    float S[4][4];
    int off_out[4];
    #pragma unroll
    for (int tb = 0; tb < 4; ++tb) off_out[tb] = (16 * tb + i16) * H * kRowOut + 4 * (16 * wave + 4 * grp);
    const uint16_t *gr = static_cast<const uint16_t *>(t.r);
    const uint16_t *gk = static_cast<const uint16_t *>(t.k);
    const uint16_t *gw = static_cast<const uint16_t *>(t.w);

    // Step j (one workgroup barrier each, n_chunks + 1 steps): the producers
    // make chunk j in set j % 2, the consumers finish chunk j - 1 from set
    // (j - 1) % 2.  Each role runs its own loop, so that the registers of one
    // are free for the other.
    // Each SIMD holds one producer and one consumer wave, and the consumers'
    // matrix phases bound each step: the consumers win issue arbitration
    // (8 % faster on 8 x 4096 x 32 than equal priority; the reverse is slower).
    if (producer) {
        __builtin_amdgcn_s_setprio(0);
        if (!C2) u4 = *reinterpret_cast<const f32x4 *>(t.u + (size_t)h * kHeadDim + c0);
        if (n_chunks > 0) issue_loads(t0);
        for (int j = 0; j < n_chunks; ++j) {
            {
                PlaneSet &ps = sm.set[j & 1];
                const int64_t tc = t0 + (int64_t)j * kChunk;
                const int64_t left = t1 - tc;
                const int nt = left >= kChunk ? kChunk : (int)left;
                #pragma unroll
                for (int m = 0; m < 2; ++m) {
                    lds_write_b128(sm.stage[0], st_wr[m], P.r[m]);
                    lds_write_b128(sm.stage[1], st_wr[m], P.k[m]);
                    lds_write_b128(sm.stage[2], st_wr[m], P.w[m]);
                    if constexpr (kU2) lds_write_b128(sm.stage[3], st_wr[m], P.u2[m]);
                    lds_write_b128(ps.v, lb.vw + 64 * 32 * m, P.v[m]);
                }
                if (j + 1 < n_chunks) issue_loads(tc + kChunk);
                group_barrier(&sm.bar[0], gen);

                u32x2 pr[4], pk[4], pw[4];
                #pragma unroll
                for (int a = 0; a < 4; ++a) {
                    pk[a] = lds_read_b64(sm.stage[1], st_rd[a]);
                    pw[a] = lds_read_b64(sm.stage[2], st_rd[a]);
                    pr[a] = lds_read_b64(sm.stage[0], st_rd[a]);
                }
                if constexpr (kU2) {
                    #pragma unroll
                    for (int tb = 0; tb < 4; ++tb) sm.u2[j & 1][tb][ltid] = lds_read_b64(sm.stage[3], st_u2[tb]);
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
                    rr[a][0] = bf16_lo(pr[a].x); rr[a][1] = bf16_hi(pr[a].x);
                    rr[a][2] = bf16_lo(pr[a].y); rr[a][3] = bf16_hi(pr[a].y);
                }
                float pwv[4][4];
                #pragma unroll
                for (int a = 0; a < 4; ++a)
                    #pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float x = lam[a][q];
                        const float e = LOGD ? __builtin_amdgcn_exp2f(x * kLog2e) : 0.f;
                        if (C2) kk_[a][q] *= one_minus_w<LOGD>(x, e);
                        pwv[a][q] = LOGD ? __builtin_amdgcn_exp2f(-e * kLog2e) : x;
                    }
                float excl[4], total[4];
                bool stiff = false;
                #pragma unroll
                for (int q = 0; q < 4; ++q) {
                    pwv[1][q] *= pwv[0][q];
                    pwv[2][q] *= pwv[1][q];
                    pwv[3][q] *= pwv[2][q];
                    const float incl = row_prod16(pwv[3][q]);
                    excl[q] = row_prev(incl);
                    total[q] = row_bcast<15>(incl);
                    stiff |= !(total[q] >= kMinChunkDecay);
                }
                stiff = __any(stiff);
                if (lane == 0) ps.stiff[wave] = stiff ? 1 : 0;
                if (i16 == 15) {
                    #pragma unroll
                    for (int q = 0; q < 4; ++q) ps.row_dec[c0 + q] = total[q];
                }
                float bp[4];
                #pragma unroll
                for (int a = 0; a < 4; ++a) {
                    float rs[4], ks[4];
                    bp[a] = 0.f;
                    #pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float p_prev = a == 0 ? excl[q] : excl[q] * pwv[a - 1][q];
                        const float p_cur = excl[q] * pwv[a][q];
                        rs[q] = rr[a][q] * p_prev;
                        ks[q] = kk_[a][q] * __builtin_amdgcn_rcpf(p_cur);
                        if (!C2) bp[a] += rr[a][q] * u4[q] * kk_[a][q];
                    }
                    u32x2 rh, rl, kh, kl;
                    split4(rs[0], rs[1], rs[2], rs[3], rh, rl);
                    split4(ks[0], ks[1], ks[2], ks[3], kh, kl);
                    lds_write_b64(ps.rt_hi, lb.pw_rt[a], rh);
                    lds_write_b64(ps.rt_lo, lb.pw_rt[a], rl);
                    lds_write_b64(ps.kt_hi, lb.pw_kt[a], kh);
                    lds_write_b64(ps.kt_lo, lb.pw_kt[a], kl);
                    if (!C2) bp[a] = sum_rows4(bp[a]);
                }
                if (!C2 && grp == 0) {
                    f32x4 b4 = {bp[0], bp[1], bp[2], bp[3]};
                    *reinterpret_cast<f32x4 *>(&ps.bonus_part[wave][4 * i16]) = b4;
                }
            }
            __syncthreads();
        }
        __syncthreads();                                 // the consumers' last step
    } else {
        __builtin_amdgcn_s_setprio(3);
        load_public_state(s_src, S, ltid);
        __syncthreads();                                 // step 0: nothing to consume yet
        for (int c = 0; c < n_chunks; ++c) {
            PlaneSet &ps = sm.set[c & 1];
            PCView sv{ps.v, ps.rt_hi, ps.rt_lo, ps.kt_hi, ps.kt_lo, sm.a_hi, sm.a_lo, ps.bonus_part, ps.row_dec,
                      ps.stiff};
            const int64_t tc = t0 + (int64_t)c * kChunk;
            const int64_t left = t1 - tc;
            const int nt = left >= kChunk ? kChunk : (int)left;
            bf16x8 vop[2];
            vop[0] = col_op(ps.v, lb.tr_v, 0);
            vop[1] = col_op(ps.v, lb.tr_v, 1);
            const bool stiff = (ps.stiff[0] | ps.stiff[1] | ps.stiff[2] | ps.stiff[3]) != 0;
            f32x4 acc[4];
            if (stiff) {
                // exact token-by-token evaluation of this chunk (rare path),
                // outputs staged as fp32 [t][j] in this set's r~ planes
                float *o_stage = reinterpret_cast<float *>(ps.rt_hi);
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
                    const unsigned vbits = ps.v[off_v(tt, 16 * wave + i16)];
                    const float vj = __uint_as_float(vbits << 16);
                    const float b = C2 ? 0.f : ps.bonus_part[0][tt] + ps.bonus_part[1][tt] +
                                               ps.bonus_part[2][tt] + ps.bonus_part[3][tt];
                    if (grp == (tt & 3)) o_stage[tt * kHeadDim + 16 * wave + i16] = part + b * vj;
                    #pragma unroll
                    for (int ib = 0; ib < 4; ++ib)
                        #pragma unroll
                        for (int e = 0; e < 4; ++e) S[ib][e] = wv[ib][e] * S[ib][e] + kv[ib][e] * vj;
                }
                group_barrier(&sm.bar[1], gen);
                #pragma unroll
                for (int tb = 0; tb < 4; ++tb)
                    acc[tb] = *reinterpret_cast<const f32x4 *>(&o_stage[(16 * tb + i16) * kHeadDim + 16 * wave + 4 * grp]);
            } else {
                if (wave == 2 || wave == 3) {
                    const int TB = wave == 2 ? 0 : 2, SB = TB + 1;
                    const u32x2 z = {0u, 0u};
                    lds_write_b64(sm.a_hi, lb.aw[SB] + 1024 * TB, z);
                    lds_write_b64(sm.a_lo, lb.aw[SB] + 1024 * TB, z);
                }
                if (wave == 0) {
                    const int TB[3] = {0, 1, 2}, SB[3] = {0, 0, 0};
                    a_tiles<!C2, 3>(sv, lb, TB, SB, i16, grp);
                } else if (wave == 1) {
                    const int TB[3] = {1, 2, 3}, SB[3] = {1, 1, 0};
                    a_tiles<!C2, 3>(sv, lb, TB, SB, i16, grp);
                } else if (wave == 2) {
                    const int TB[2] = {2, 3}, SB[2] = {2, 1};
                    a_tiles<!C2, 2>(sv, lb, TB, SB, i16, grp);
                } else {
                    const int TB[2] = {3, 3}, SB[2] = {3, 2};
                    a_tiles<!C2, 2>(sv, lb, TB, SB, i16, grp);
                }
                {   // read-out of the carried state: o^T = S^T r~^T
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
                            r_hi[tb] = rt_op(ps.rt_hi, lb.ro_x, tb, kk);
                            r_lo[tb] = rt_op(ps.rt_lo, lb.ro_x, tb, kk);
                        }
                        #pragma unroll
                        for (int tb = 0; tb < 4; ++tb) acc[tb] = mfma(s_hi[kk], r_hi[tb], acc[tb]);
                        #pragma unroll
                        for (int tb = 0; tb < 4; ++tb) acc[tb] = mfma(s_hi[kk], r_lo[tb], acc[tb]);
                        #pragma unroll
                        for (int tb = 0; tb < 4; ++tb) acc[tb] = mfma(s_lo[kk], r_hi[tb], acc[tb]);
                    }
                }
                // state update, skipped in the last chunk when the end state is not wanted
                if (state_dst || c + 1 < n_chunks) {
                    f32x4 p[4];
                    #pragma unroll
                    for (int ib = 0; ib < 4; ++ib) p[ib] = f32x4{0.f, 0.f, 0.f, 0.f};
                    #pragma unroll
                    for (int kk = 0; kk < 2; ++kk) {
                        bf16x8 k_hi[4], k_lo[4];
                        #pragma unroll
                        for (int ib = 0; ib < 4; ++ib) {
                            k_hi[ib] = kt_col_op(ps.kt_hi, lb.tr_kt[ib], kk);
                            k_lo[ib] = kt_col_op(ps.kt_lo, lb.tr_kt[ib], kk);
                        }
                        #pragma unroll
                        for (int ib = 0; ib < 4; ++ib) p[ib] = mfma(k_hi[ib], vop[kk], p[ib]);
                        #pragma unroll
                        for (int ib = 0; ib < 4; ++ib) p[ib] = mfma(k_lo[ib], vop[kk], p[ib]);
                    }
                    #pragma unroll
                    for (int ib = 0; ib < 4; ++ib) {
                        const f32x4 dec = *reinterpret_cast<const f32x4 *>(&ps.row_dec[16 * ib + 4 * grp]);
                        #pragma unroll
                        for (int e = 0; e < 4; ++e) S[ib][e] = dec[e] * (S[ib][e] + p[ib][e]);
                    }
                }
                group_barrier(&sm.bar[1], gen);          // every A tile is written
                // in-chunk pairs: o^T += v^T A^T (A is zero for s >= 32 when t < 32)
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
            if constexpr (kU2) {                         // + u'_t (Finch-C2 output)
                #pragma unroll
                for (int tb = 0; tb < 4; ++tb) {
                    const u32x2 u = sm.u2[c & 1][tb][ltid];
                    acc[tb][0] += bf16_lo(u.x);
                    acc[tb][1] += bf16_hi(u.x);
                    acc[tb][2] += bf16_lo(u.y);
                    acc[tb][3] += bf16_hi(u.y);
                }
            }
            if (t.o_bf16) {
                const Rsrc ro = chunk_rsrc(t.o, tc, nt, H, h, kRowIn);
                #pragma unroll
                for (int tb = 0; tb < 4; ++tb) {
                    const f32x2 a = {acc[tb][0], acc[tb][1]}, b = {acc[tb][2], acc[tb][3]};
                    const u32x2 pk = {__builtin_bit_cast(unsigned, __builtin_convertvector(a, bf16x2)),
                                      __builtin_bit_cast(unsigned, __builtin_convertvector(b, bf16x2))};
                    __builtin_amdgcn_raw_buffer_store_b64(pk, ro, off_out[tb] / 2, 0, 0);
                }
            } else {
                const Rsrc ro = chunk_rsrc(t.o, tc, nt, H, h, kRowOut);
                #pragma unroll
                for (int tb = 0; tb < 4; ++tb)
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[tb]), ro, off_out[tb], 0, 0);
            }
            __syncthreads();
        }
        if (state_dst) store_public_state(state_dst, S, ltid);
    }
}

// Batches whose (sequence, head) pairs fill the GPU: one workgroup per
// (sequence, head), the whole sequence from state_in (no segments, no state
// pass).  The plan has one segment per sequence; a packed call's sequences
// are taken longest first when the rank table is there.  Any length works,
// zero included (both roles then pass one barrier and the state is copied
// through).  With a split plan (long segments, about one per CU) a segment
// starts from the combined start state of the segment scan, and only the
// last segment of a sequence writes state_out.
template <bool LOGD, bool C2>
__global__ __launch_bounds__(512, 1) void wkv_chunk_pc_kernel(Geometry g, Tensors t, Workspace ws) {
    __shared__ SmemPC<C2> sm;
    const int h = blockIdx.x % g.H;
    const int rank = blockIdx.x / g.H;
    const int seg = g.seg_rank ? g.seg_rank[rank] : rank;
    const ItemRange it = decode_segment(g, seg);
    if (!it.valid) return;
    if (it.P > 1 && ws.seg_start == nullptr) return;     // a split the host did not plan
    const size_t slot = ((size_t)it.n * g.H + h) * (kHeadDim * kHeadDim);
    const float *s_src = it.P > 1 ? ws.seg_start + ((size_t)seg * g.H + h) * kSegStartFloats
                                  : (t.state_in ? t.state_in + slot : nullptr);
    float *s_dst = t.state_out && it.p == it.P - 1 ? t.state_out + slot : nullptr;
    pc_item<LOGD, C2>(sm, t, it.t0, it.t1, h, g.H, s_src, s_dst);
}

}  // namespace

namespace {
using KernelFn = void (*)(Geometry, Tensors, Workspace);
template <bool Relay>
KernelFn split_kernel_form(const Variant &v) {
    return v.log_decay ? (v.c2 ? wkv_split_kernel<true, true, Relay> : wkv_split_kernel<true, false, Relay>)
                       : (v.c2 ? wkv_split_kernel<false, true, Relay> : wkv_split_kernel<false, false, Relay>);
}
KernelFn split_kernel_for(const Variant &v, bool relay) {
    return relay ? split_kernel_form<true>(v) : split_kernel_form<false>(v);
}
}  // namespace

hipError_t split_launch_capacity(const Variant &v, bool relay, int64_t *capacity) {
    constexpr int kMaxDevices = 64;
    static std::atomic<int64_t> cache[kMaxDevices][8];       // 0: not yet measured
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const int form = (v.log_decay ? 1 : 0) + (v.c2 ? 2 : 0) + (relay ? 4 : 0);
    if (dev >= 0 && dev < kMaxDevices) {
        const int64_t c = cache[dev][form].load(std::memory_order_relaxed);
        if (c > 0) {
            *capacity = c;
            return hipSuccess;
        }
    }
    int cus = 0, per_cu = 0;
    if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, split_kernel_for(v, relay), 256, 0)) != hipSuccess)
        return e;
    *capacity = (int64_t)cus * per_cu;
    if (dev >= 0 && dev < kMaxDevices && *capacity > 0) cache[dev][form].store(*capacity, std::memory_order_relaxed);
    return hipSuccess;
}

hipError_t launch_chunked(const Geometry &g, const Tensors &t, const Workspace &ws, bool split,
                          Variant v, hipStream_t st, KernelTiming tm) {
    const int64_t items = (int64_t)g.n_seg * g.H;
    if (items <= 0) return hipSuccess;
    const dim3 grid((unsigned)items), block(256);
    if (split && ws.ctl) {                             // one launch: state, scan and chunked roles
        const dim3 grid2((unsigned)(g.relay ? items : 2 * items));
        const KernelFn k = split_kernel_for(v, g.relay != 0);
        if (tm.start || tm.stop)
            hipExtLaunchKernelGGL(k, grid2, block, 0, st, tm.start, tm.stop, 0, g, t, ws);
        else
            hipLaunchKernelGGL(k, grid2, block, 0, st, g, t, ws);
        return hipGetLastError();
    }
    if (split) {
        void (*ks)(Geometry, Tensors, Workspace) =
            v.log_decay ? (v.c2 ? wkv_state_kernel<true, true> : wkv_state_kernel<true, false>)
                        : (v.c2 ? wkv_state_kernel<false, true> : wkv_state_kernel<false, false>);
        hipLaunchKernelGGL(ks, dim3((unsigned)(items * g.runs)), block, 0, st, g, t, ws);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(wkv_segment_scan_kernel, dim3((unsigned)(g.n_seq * g.H * kScanSlices)), dim3(kScanThreads),
                           0, st, g, t, ws);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (g.whole_seqs || g.pc_split) {                  // producer/consumer kernel
        const dim3 pc_grid((unsigned)items), pc_block(512);
        void (*k)(Geometry, Tensors, Workspace) =
            v.log_decay ? (v.c2 ? wkv_chunk_pc_kernel<true, true> : wkv_chunk_pc_kernel<true, false>)
                        : (v.c2 ? wkv_chunk_pc_kernel<false, true> : wkv_chunk_pc_kernel<false, false>);
        if (tm.start || tm.stop)
            hipExtLaunchKernelGGL(k, pc_grid, pc_block, 0, st, tm.start, tm.stop, 0, g, t, ws);
        else
            hipLaunchKernelGGL(k, pc_grid, pc_block, 0, st, g, t, ws);
        return hipGetLastError();
    }
    void (*k)(Geometry, Tensors, Workspace) =
        v.log_decay ? (v.c2 ? wkv_chunk_kernel<true, true> : wkv_chunk_kernel<true, false>)
                    : (v.c2 ? wkv_chunk_kernel<false, true> : wkv_chunk_kernel<false, false>);
    if (tm.start || tm.stop)
        hipExtLaunchKernelGGL(k, grid, block, 0, st, tm.start, tm.stop, 0, g, t, ws);
    else
        hipLaunchKernelGGL(k, grid, block, 0, st, g, t, ws);
    return hipGetLastError();
}

}  // namespace finch
