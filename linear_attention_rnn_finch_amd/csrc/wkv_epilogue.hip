// The two steps after the scan in Finch-C2 pre-fill (gfx950):
//
// - LayerNorm over the concatenated heads of each token (GoldFinch
//   architecture summary, section 3.4, "Finch-C2 Time Mixing", output
//   equation: the norm spans all heads, replacing base Finch's per-head
//   GroupNorm).  It cannot ride along with the scan's store: a scan workgroup
//   owns one head of a segment, and a token's statistics need every head.  So
//   it is its own bandwidth-bound pass: persistent workgroups, one token row at
//   a time (the next one already loading), the row held in registers between
//   the two reductions (mean, then variance about the mean), the scale and
//   shift loaded once per workgroup.
//
// - GOLD key compression c_t = x_t W_KD, D -> D/16 (same page, "GOLD Key
//   Compression and TokenCat Decompression", compression step).  A small
//   contraction over D on v_mfma_f32_16x16x32_bf16, computed as
//   c^T = W x^T so that both operands are read as 16-byte row pieces (the
//   weight is stored [D/16, D]) and every lane's four results are adjacent
//   outputs of one token.  Operands are staged through LDS in slices of
//   d_model, loaded as whole 128-byte lines two slices ahead (see
//   gold_compress_kernel).
#include <hip/hip_ext.h>

#include "wkv_internal.h"

namespace finch {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kLnThreads = 256;
static_assert(kMaxNormWidth == 8 * 4 * kLnThreads, "the LayerNorm kernels are built for up to 8 float4 per thread");

__device__ inline float wave_sum(float x) {
    #pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
    return x;
}

// sum over the workgroup (four waves), result in every thread
__device__ inline float block_sum(float x, float *red) {
    x = wave_sum(x);
    const int wave = threadIdx.x >> 6;
    __syncthreads();                                   // red[] free from the previous use
    if ((threadIdx.x & 63) == 0) red[wave] = x;
    __syncthreads();
    return red[0] + red[1] + red[2] + red[3];
}

// NV = float4 per thread in a row (width = 1024 * NV).  The next row's loads
// are issued before the current row's reductions, so one row's memory latency
// hides behind the previous row's arithmetic.
template <int NV, bool OutBf16>
__global__ __launch_bounds__(kLnThreads) void layernorm_rows_kernel(const float *x, const float *gamma,
                                                                   const float *beta, float eps, void *y,
                                                                   int64_t rows, int width) {
    __shared__ float red[4];
    const int tid = threadIdx.x;
    f32x4 g[NV], b[NV], v[NV], vn[NV];
    #pragma unroll
    for (int i = 0; i < NV; ++i) {
        g[i] = *reinterpret_cast<const f32x4 *>(gamma + 4 * (tid + kLnThreads * i));
        b[i] = *reinterpret_cast<const f32x4 *>(beta + 4 * (tid + kLnThreads * i));
    }
    const float inv_w = 1.f / (float)width;
    int64_t row = blockIdx.x;
    if (row < rows) {
        #pragma unroll
        for (int i = 0; i < NV; ++i) v[i] = *reinterpret_cast<const f32x4 *>(x + row * width + 4 * (tid + kLnThreads * i));
    }
    for (; row < rows; row += gridDim.x) {
        const int64_t next = row + gridDim.x;
        if (next < rows) {
            #pragma unroll
            for (int i = 0; i < NV; ++i)
                vn[i] = *reinterpret_cast<const f32x4 *>(x + next * width + 4 * (tid + kLnThreads * i));
        }
        float s = 0.f;
        #pragma unroll
        for (int i = 0; i < NV; ++i) s += (v[i][0] + v[i][1]) + (v[i][2] + v[i][3]);
        const float mean = block_sum(s, red) * inv_w;
        float q = 0.f;
        #pragma unroll
        for (int i = 0; i < NV; ++i)
            #pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[i][e] -= mean;
                q += v[i][e] * v[i][e];
            }
        const float rstd = 1.f / sqrtf(block_sum(q, red) * inv_w + eps);
        #pragma unroll
        for (int i = 0; i < NV; ++i) {
            f32x4 o;
            #pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = v[i][e] * rstd * g[i][e] + b[i][e];
            const int64_t at = row * width + 4 * (tid + kLnThreads * i);
            if (OutBf16)
                *reinterpret_cast<bf16x4 *>(static_cast<uint16_t *>(y) + at) = __builtin_convertvector(o, bf16x4);
            else
                *reinterpret_cast<f32x4 *>(static_cast<float *>(y) + at) = o;
        }
        #pragma unroll
        for (int i = 0; i < NV; ++i) v[i] = vn[i];
    }
}

template <bool OutBf16>
void (*layernorm_kernel_for(int nv))(const float *, const float *, const float *, float, void *, int64_t, int) {
    switch (nv) {
    case 1: return layernorm_rows_kernel<1, OutBf16>;
    case 2: return layernorm_rows_kernel<2, OutBf16>;
    case 3: return layernorm_rows_kernel<3, OutBf16>;
    case 4: return layernorm_rows_kernel<4, OutBf16>;
    case 5: return layernorm_rows_kernel<5, OutBf16>;
    case 6: return layernorm_rows_kernel<6, OutBf16>;
    case 7: return layernorm_rows_kernel<7, OutBf16>;
    default: return layernorm_rows_kernel<8, OutBf16>;
    }
}

constexpr int kCmpRows = 32;      // tokens per workgroup (two 16-token tiles)
constexpr int kCmpCols = 64;      // outputs per workgroup (four 16-output tiles)
constexpr int kCmpK = 256;        // d_model slice per step (512-byte row pieces)
constexpr int kCmpThreads = 512;  // eight waves: 32 tokens x 32 outputs each, a quarter of every slice
constexpr int kCmpBufs = 3;       // slices in LDS: one being read, two loading
constexpr int kCmpPieces = kCmpK / 8;                              // 16-byte pieces per row slice
constexpr int kCmpSliceRows = kCmpRows + kCmpCols;                 // x rows, then weight rows
constexpr int kCmpRowsPerLoad = 64 / kCmpPieces;                   // rows one wave instruction covers
constexpr int kCmpLoadsPerWave = kCmpSliceRows / kCmpRowsPerLoad / (kCmpThreads / 64);
static_assert(kCmpLoadsPerWave * kCmpRowsPerLoad * (kCmpThreads / 64) == kCmpSliceRows, "whole slice per step");

struct alignas(16) CmpSmem {
    uint16_t buf[kCmpBufs][kCmpSliceRows][kCmpK];   // 3 x 48 KB, rows unpadded, 16-byte pieces swizzled
};

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

using lds_void = __attribute__((address_space(3))) void;

// s_waitcnt immediates (gfx9 encoding: vmcnt bits 3:0, expcnt 6:4, lgkmcnt
// 11:8): wait until at most N vector-memory operations of this wave are
// outstanding, leaving the other counters unconstrained
constexpr int kWaitVm0 = 0xF70;
constexpr int kWaitVmAhead = 0xF70 | (kCmpLoadsPerWave * (kCmpBufs - 2));   // later slices may be in flight
static_assert(kCmpLoadsPerWave * (kCmpBufs - 2) < 16, "vmcnt field");

// Workgroup: 32 tokens x 64 outputs over the whole of d_model, in slices of
// 256.  Each slice goes from global memory straight into LDS
// (global_load_lds_dwordx4: a wave instruction writes 1 KB, two whole
// 512-byte rows, contiguously): no registers and no LDS store instructions on
// the way.  The 16-byte piece that lane L of a load writes (slot L % 32 of row
// r) is the global piece (L % 32) ^ (r % 16) of that row, so each row is
// stored XOR-swizzled and the operand reads -- 16 rows at one piece -- fall
// on 16 different bank groups.  Three slices are in LDS at once (one read,
// two loading), with one barrier per slice; five 128-wide slices in flight
// instead were measured slower.  Wave v computes all 32 tokens against
// outputs n0 + 32 (v % 2) .. + 31 (2 x 2 tiles of 16 x 16, each operand read
// once for two products) over the quarter v / 2 of every slice; the four
// quarters' partial tiles are added through LDS at the end.
template <bool OutBf16>
__global__ __launch_bounds__(kCmpThreads) void gold_compress_kernel(const uint16_t *x, const uint16_t *w, void *c,
                                                                    int64_t M, int K, int N) {
    __shared__ CmpSmem sm;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int i16 = lane & 15, grp = lane >> 4;
    const int64_t m0 = (int64_t)blockIdx.x * kCmpRows;
    const int n0 = blockIdx.y * kCmpCols;
    const int steps = K / kCmpK;

    // load j of this wave covers slice rows 2q, 2q + 1 (q = wave + 8 j); lane
    // L takes row 2q + L / 32, global piece (L % 32) ^ (row % 16)
    const uint16_t *src[kCmpLoadsPerWave];
    int dst[kCmpLoadsPerWave];
    #pragma unroll
    for (int j = 0; j < kCmpLoadsPerWave; ++j) {
        const int q = wave + (kCmpThreads / 64) * j, row = kCmpRowsPerLoad * q + lane / kCmpPieces;
        const int piece = (lane % kCmpPieces) ^ (row & 15);
        const uint16_t *base;
        if (row < kCmpRows) {
            int64_t m = m0 + row;
            if (m >= M) m = M - 1;                          // rows past M: loaded, never stored
            base = x + (size_t)m * K;
        } else {
            base = w + (size_t)(n0 + row - kCmpRows) * K;
        }
        src[j] = base + 8 * piece;
        dst[j] = kCmpRowsPerLoad * q * kCmpK;               // element offset of the 1 KB block
    }
    auto load = [&](int s) {                                // slice s into buffer s % 3 (no-op past the end)
        if (s >= steps) return;
        uint16_t *b = &sm.buf[s % kCmpBufs][0][0];
        const int k0 = s * kCmpK;
        #pragma unroll
        for (int j = 0; j < kCmpLoadsPerWave; ++j)
            __builtin_amdgcn_global_load_lds(src[j] + k0, (lds_void *)(b + dst[j]), 16, 0, 0);
    };
    // operand read: piece p of slice row r sits in slot p ^ (r % 16)
    auto read = [&](const uint16_t *b, int row, int piece) {
        return *reinterpret_cast<const bf16x8 *>(b + row * kCmpK + 8 * (piece ^ (row & 15)));
    };
    const int nh = wave & 1, kq = wave >> 1;
    f32x4 acc[2][2] = {{f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}},
                       {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}}};
    auto compute = [&](int s) {
        const uint16_t *b = &sm.buf[s % kCmpBufs][0][0];
        #pragma unroll
        for (int u = 2 * kq; u < 2 * kq + 2; ++u) {
            const int piece = 4 * u + grp;                  // d_model slots 32u + 8grp .. +7
            bf16x8 a[2], bb[2];
            #pragma unroll
            for (int t = 0; t < 2; ++t) {
                a[t] = read(b, kCmpRows + 32 * nh + 16 * t + i16, piece);
                bb[t] = read(b, 16 * t + i16, piece);
            }
            #pragma unroll
            for (int ta = 0; ta < 2; ++ta)
                #pragma unroll
                for (int tb = 0; tb < 2; ++tb) acc[ta][tb] = mfma(a[ta], bb[tb], acc[ta][tb]);
        }
    };

    #pragma unroll
    for (int s = 0; s < kCmpBufs - 1; ++s) load(s);
    for (int s = 0; s < steps; ++s) {
        // this wave's loads of slice s are complete (later ones may not be),
        // then everyone's are, and every wave has finished reading slice s - 1
        // (a plain barrier: __syncthreads' fence would wait for the later
        // slices too; every LDS read of slice s - 1 has returned, its products
        // used them)
        if (s + kCmpBufs - 2 < steps)
            __builtin_amdgcn_s_waitcnt(kWaitVmAhead);
        else
            __builtin_amdgcn_s_waitcnt(kWaitVm0);
        __builtin_amdgcn_s_barrier();
        load(s + kCmpBufs - 1);                             // into the buffer slice s - 1 used
        compute(s);
    }
    __syncthreads();

    // the four quarters' partial tiles, through LDS: part[kq][nh][tile][lane],
    // then wave v adds the quarters of tile v / 2 of output half v % 2 and stores it
    f32x4 *part = reinterpret_cast<f32x4 *>(&sm.buf[0][0][0]);   // 32 KB (buffers 0 and 1)
    #pragma unroll
    for (int ta = 0; ta < 2; ++ta)
        #pragma unroll
        for (int tb = 0; tb < 2; ++tb) part[((kq * 2 + nh) * 4 + 2 * ta + tb) * 64 + lane] = acc[ta][tb];
    __syncthreads();
    const int tile = wave >> 1, ta = tile >> 1, tb = tile & 1;
    f32x4 sum = part[((0 * 2 + nh) * 4 + tile) * 64 + lane];
    #pragma unroll
    for (int q = 1; q < 4; ++q) sum += part[((q * 2 + nh) * 4 + tile) * 64 + lane];
    // acc layout: value e of lane (i16, grp) is c[m0 + 16tb + i16][n0 + 32nh + 16ta + 4grp + e]
    const int64_t m = m0 + 16 * tb + i16;
    if (m < M) {
        const size_t at = (size_t)m * N + n0 + 32 * nh + 16 * ta + 4 * grp;
        if (OutBf16)
            *reinterpret_cast<bf16x4 *>(static_cast<uint16_t *>(c) + at) = __builtin_convertvector(sum, bf16x4);
        else
            *reinterpret_cast<f32x4 *>(static_cast<float *>(c) + at) = sum;
    }
}

}  // namespace

hipError_t launch_layernorm_rows(const float *x, const float *gamma, const float *beta, float eps, void *y,
                                 bool out_bf16, int64_t rows, int width, hipStream_t st, KernelTiming tm) {
    if (rows <= 0) return hipSuccess;
    const unsigned grid = (unsigned)std::min<int64_t>(rows, 4096);
    const int nv = width / (4 * kLnThreads);
    if (out_bf16)
        hipExtLaunchKernelGGL(layernorm_kernel_for<true>(nv), dim3(grid), dim3(kLnThreads), 0, st, tm.start, tm.stop, 0,
                              x, gamma, beta, eps, y, rows, width);
    else
        hipExtLaunchKernelGGL(layernorm_kernel_for<false>(nv), dim3(grid), dim3(kLnThreads), 0, st, tm.start, tm.stop, 0,
                              x, gamma, beta, eps, y, rows, width);
    return hipGetLastError();
}

hipError_t launch_gold_compress(const uint16_t *x, const uint16_t *w, void *c, bool out_bf16, int64_t M, int K,
                                int N, hipStream_t st, KernelTiming tm) {
    if (M <= 0) return hipSuccess;
    if (K % kCmpK != 0 || N % kCmpCols != 0) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((M + kCmpRows - 1) / kCmpRows), (unsigned)(N / kCmpCols));
    if (out_bf16)
        hipExtLaunchKernelGGL(gold_compress_kernel<true>, grid, dim3(kCmpThreads), 0, st, tm.start, tm.stop, 0,
                              x, w, c, M, K, N);
    else
        hipExtLaunchKernelGGL(gold_compress_kernel<false>, grid, dim3(kCmpThreads), 0, st, tm.start, tm.stop, 0,
                              x, w, c, M, K, N);
    return hipGetLastError();
}

}  // namespace finch
