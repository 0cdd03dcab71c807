// Prefill-shaped dequantized product on the bf16 matrix cores:
//   y[m, n] = s[n] * sum_k x[m, k] * q[n, k]
// DynaQuant page, "自定义内核架构" (packed codes expanded to the matrix unit's
// input format; its 9-15 bit template feeds BF16 matrix units) and the BPDQ
// article, section 3.2 (dequantize fused with the product; fp32 scales and
// output).  The scale is factored out of the sum and applied in the epilogue.
//
// Exactness: bf16 carries 8 significant bits, so every integer |q| <= 256 is
// exact and b <= 9 codes go to the matrix cores as they are.  For b >= 10 each
// code is split as q = 64*hi + lo with hi = q >> 6 in [-256, 255] and
// lo = q & 63 in [0, 63]; bf16(64*hi) and bf16(lo) are both exact and are
// multiplied against the same x slice into the same fp32 accumulator.
//
// Tiling: a 256-thread workgroup computes a 128 x 128 tile of y; the K loop
// stages a 128 x 64 slice of x and the matching 128 x 64 slice of expanded
// codes in LDS (k contiguous for both), and each wave issues
// v_mfma_f32_16x16x32_bf16 over its 64 x 64 sub-tile.
#include "common.hpp"
#include "launch.hpp"

namespace dq {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kBM = 128;
constexpr int kBN = 128;
constexpr int kBK = 64;
constexpr int kLd = kBK + 8;  // LDS row pitch in bf16 elements (16 B pad)
constexpr int kGemmThreads = 256;

// bf16 bits of a small integer value v (|v| has at most 8 significant bits, so
// dropping the low half of its fp32 pattern is exact).
__device__ __forceinline__ uint16_t exact_bf16_bits(int32_t v)
{
    return (uint16_t)(__float_as_uint((float)v) >> 16);
}

template <int B>
__global__ __launch_bounds__(kGemmThreads) void gemm_kernel(
    const uint16_t* __restrict__ x, int64_t M, const uint32_t* __restrict__ packed,
    const float* __restrict__ scales, int64_t N, int64_t K, int64_t row_words,
    float* __restrict__ y)
{
    constexpr bool kSplit = B >= 10;
    constexpr int kPlanes = kSplit ? 2 : 1;
    __shared__ __attribute__((aligned(16))) uint16_t As[kBM * kLd];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[kPlanes][kBN * kLd];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int wm = wave >> 1;
    const int wn = wave & 1;
    const int64_t ntn = ceil_div(N, kBN);
    const int64_t tile = blockIdx.x;
    const int64_t m0 = (tile / ntn) * kBM;
    const int64_t n0 = (tile % ntn) * kBN;
    const int64_t nchunks = ceil_div(K, kChunk);
    const bool xvec = (K & 7) == 0;

    f32x4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

    const int sr = tid >> 1;  // staging row within the tile
    const int sh = tid & 1;   // which 32-wide half of the k slice

    for (int64_t k0 = 0; k0 < K; k0 += kBK) {
        // ---- x slice -> LDS
        {
            const int64_t m = m0 + sr;
            const int64_t kb = k0 + kChunk * sh;
            uint16_t* dst = &As[sr * kLd + kChunk * sh];
            if (m < M && xvec && kb + kChunk <= K) {
                const uint4* src = reinterpret_cast<const uint4*>(x + m * K + kb);
#pragma unroll
                for (int i = 0; i < 4; ++i) reinterpret_cast<uint4*>(dst)[i] = src[i];
            } else {
#pragma unroll
                for (int j = 0; j < kChunk; ++j)
                    dst[j] = (m < M && kb + j < K) ? x[m * K + kb + j] : (uint16_t)0;
            }
        }
        // ---- packed codes -> exact bf16 -> LDS
        {
            const int64_t n = n0 + sr;
            const int64_t c = k0 / kChunk + sh;
            uint32_t wd[B];
            const bool live = n < N && c < nchunks;
            if (live) {
                load_chunk_words<B>(packed + n * row_words, c, row_words, wd);
            } else {
#pragma unroll
                for (int i = 0; i < B; ++i) wd[i] = 0;
            }
#pragma unroll
            for (int i = 0; i < B; ++i) wd[i] ^= code_msb_mask<B>(i);
            uint16_t* d0 = &Bs[0][sr * kLd + kChunk * sh];
            uint16_t* d1 = &Bs[kPlanes - 1][sr * kLd + kChunk * sh];
#pragma unroll
            for (int j = 0; j < kChunk; ++j) {
                int32_t q = chunk_code_signed<B>(wd, j);
                if (!live || c * kChunk + j >= K) q = 0;
                if (kSplit) {
                    d0[j] = exact_bf16_bits((q >> 6) * 64);
                    d1[j] = exact_bf16_bits(q & 63);
                } else {
                    d0[j] = exact_bf16_bits(q);
                }
            }
        }
        __syncthreads();

#pragma unroll
        for (int kk = 0; kk < kBK / 32; ++kk) {
            const int kcol = kk * 32 + 8 * (lane >> 4);
            bf16x8_t a[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                a[i] = *reinterpret_cast<const bf16x8_t*>(
                    &As[(wm * 64 + i * 16 + (lane & 15)) * kLd + kcol]);
#pragma unroll
            for (int p = 0; p < kPlanes; ++p) {
                bf16x8_t b[4];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    b[j] = *reinterpret_cast<const bf16x8_t*>(
                        &Bs[p][(wn * 64 + j * 16 + (lane & 15)) * kLd + kcol]);
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j],
                                                                            0, 0, 0);
            }
        }
        __syncthreads();
    }

    // ---- epilogue: y = s[n] * acc; lane holds column lane&15, rows 4*(lane>>4)+r
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t n = n0 + wn * 64 + j * 16 + (lane & 15);
        if (n >= N) continue;
        const float s = scales[n];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t m = m0 + wm * 64 + i * 16 + 4 * (lane >> 4) + r;
                if (m < M) y[m * N + n] = s * acc[i][j][r];
            }
        }
    }
}

template <int B>
hipError_t launch_gemm_b(const uint16_t* x, int64_t M, const uint32_t* packed, const float* scales,
                         int64_t N, int64_t K, float* y, hipStream_t stream)
{
    const int64_t rw = packed_row_words(K, B);
    const int64_t tiles = ceil_div(N, kBN) * ceil_div(M, kBM);
    if (tiles > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)tiles);
    gemm_kernel<B><<<grid, dim3(kGemmThreads), 0, stream>>>(x, M, packed, scales, N, K, rw, y);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const uint16_t* x, int64_t M, const uint32_t* packed, const float* scales,
                       int64_t N, int64_t K, int bits, float* y, hipStream_t stream)
{
#define CALL(B) launch_gemm_b<B>(x, M, packed, scales, N, K, y, stream)
    DQ_BITS_SWITCH(bits, CALL)
#undef CALL
}

}  // namespace dq
