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
//   outputs of one token.  The contraction is split over the eight waves of
//   a workgroup (see gold_compress_kernel): with only one workgroup per CU
//   at this size, latency is hidden by having each wave's loads in flight at
//   once rather than by occupancy.
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
constexpr int kCmpWaves = 8;      // the contraction over d_model is split over the waves
constexpr int kCmpBatch = 8;      // K steps of 32 whose loads a wave issues together

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Workgroup: 32 tokens x 64 outputs; wave w contracts over its own eighth of
// d_model for all eight 16 x 16 tiles (every operand byte is read once per
// workgroup), with all of its loads for up to 8 K steps in flight at once;
// the eight partial tiles are summed through LDS.
template <bool OutBf16>
__global__ __launch_bounds__(64 * kCmpWaves) void gold_compress_kernel(const uint16_t *x, const uint16_t *w,
                                                                       void *c, int64_t M, int K, int N) {
    __shared__ f32x4 part[kCmpWaves][2 * 4][64];          // [wave][tile][lane]: 64 KB
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int i16 = lane & 15, grp = lane >> 4;
    const int64_t m0 = (int64_t)blockIdx.x * kCmpRows;
    const int n0 = blockIdx.y * kCmpCols;
    const int kw = K / kCmpWaves;                           // this wave's share, a multiple of 128
    const int kb = wave * kw;
    // A = weight rows n0 + 16*nt + i16, B = token rows m0 + 16*mt + i16 (rows past
    // M read row M - 1 and are not stored); lane takes K slots 8*grp .. +7
    const uint16_t *wa[4], *xb[2];
    #pragma unroll
    for (int nt = 0; nt < 4; ++nt) wa[nt] = w + (size_t)(n0 + 16 * nt + i16) * K + kb + 8 * grp;
    #pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
        int64_t m = m0 + 16 * mt + i16;
        if (m >= M) m = M - 1;
        xb[mt] = x + (size_t)m * K + kb + 8 * grp;
    }
    f32x4 acc[2][4];
    #pragma unroll
    for (int mt = 0; mt < 2; ++mt)
        #pragma unroll
        for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < kw; k0 += 32 * kCmpBatch) {
        u32x4 a[kCmpBatch][4], b[kCmpBatch][2];
        #pragma unroll
        for (int u = 0; u < kCmpBatch; ++u) {
            if (k0 + 32 * u < kw) {
                #pragma unroll
                for (int nt = 0; nt < 4; ++nt) a[u][nt] = *reinterpret_cast<const u32x4 *>(wa[nt] + k0 + 32 * u);
                #pragma unroll
                for (int mt = 0; mt < 2; ++mt) b[u][mt] = *reinterpret_cast<const u32x4 *>(xb[mt] + k0 + 32 * u);
            }
        }
        #pragma unroll
        for (int u = 0; u < kCmpBatch; ++u) {
            if (k0 + 32 * u < kw) {
                #pragma unroll
                for (int mt = 0; mt < 2; ++mt)
                    #pragma unroll
                    for (int nt = 0; nt < 4; ++nt)
                        acc[mt][nt] = mfma(__builtin_bit_cast(bf16x8, a[u][nt]), __builtin_bit_cast(bf16x8, b[u][mt]),
                                           acc[mt][nt]);
            }
        }
    }
    #pragma unroll
    for (int mt = 0; mt < 2; ++mt)
        #pragma unroll
        for (int nt = 0; nt < 4; ++nt) part[wave][4 * mt + nt][lane] = acc[mt][nt];
    __syncthreads();
    // thread = (tile, lane): acc layout value e is c[m0 + 16*mt + i16][n0 + 16*nt + 4*grp + e]
    const int tile = threadIdx.x >> 6;                      // 8 tiles, one per wave's worth of threads
    f32x4 sum = part[0][tile][lane];
    #pragma unroll
    for (int v = 1; v < kCmpWaves; ++v) sum += part[v][tile][lane];
    const int mt = tile >> 2, nt = tile & 3;
    const int64_t m = m0 + 16 * mt + i16;
    if (m < M) {
        const size_t at = (size_t)m * N + n0 + 16 * nt + 4 * grp;
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
    const dim3 grid((unsigned)((M + kCmpRows - 1) / kCmpRows), (unsigned)(N / kCmpCols));
    if (out_bf16)
        hipExtLaunchKernelGGL(gold_compress_kernel<true>, grid, dim3(64 * kCmpWaves), 0, st, tm.start, tm.stop, 0,
                              x, w, c, M, K, N);
    else
        hipExtLaunchKernelGGL(gold_compress_kernel<false>, grid, dim3(64 * kCmpWaves), 0, st, tm.start, tm.stop, 0,
                              x, w, c, M, K, N);
    return hipGetLastError();
}

}  // namespace finch
