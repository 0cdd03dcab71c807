// Decode-shaped dequantized product, 1 <= M <= 16:
//   y[m, n] = s[n] * sum_k x[m, k] * q[n, k]
// BPDQ article, section 3.2 (dequantize fused with the matrix product; fp32
// scales and output) and the DynaQuant page, "自定义内核架构" (packed codes are
// streamed from memory and expanded in registers).  At M = 1 the product is
// bound by the bytes of the packed weights (decode is memory-bound, as the
// Quantization tutorial's closing remark on prefill vs decode puts it).
//
// Work split: a wave owns kRows rows; lane l walks the chunks l, l+64, ... of
// those rows (a chunk = 32 codes = B whole words, so a wave's loads of one row
// cover 64*B contiguous words).  Codes are turned into signed integers with one
// XOR per word plus a signed bit-field extract, converted to fp32 and
// accumulated with fp32 FMAs against x (widened exactly from bf16).  The row
// scale multiplies the reduced sum once.
#include "common.hpp"
#include "launch.hpp"

namespace dq {

namespace {

constexpr int kGemvThreads = 256;

// x[m, 32c .. 32c+32) widened to fp32; zero at k >= K (the padding codes of a
// row's last chunk are then multiplied by an exact zero).
__device__ __forceinline__ void load_x_chunk(const uint16_t* __restrict__ xrow, int64_t K, int64_t c,
                                             bool vec_ok, float* xv)
{
    const int64_t k0 = c * kChunk;
    if (vec_ok && k0 + kChunk <= K) {
        const uint4* p4 = reinterpret_cast<const uint4*>(xrow + k0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint4 d = p4[i];
            const uint32_t u[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                xv[i * 8 + e * 2 + 0] = __uint_as_float(u[e] << 16);
                xv[i * 8 + e * 2 + 1] = __uint_as_float(u[e] & 0xffff0000u);
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < kChunk; ++j)
            xv[j] = (k0 + j < K) ? bf16_bits_to_float(xrow[k0 + j]) : 0.0f;
    }
}

template <int B, int MT, int kRows>
__global__ __launch_bounds__(kGemvThreads) void gemv_kernel(
    const uint16_t* __restrict__ x, int M, const uint32_t* __restrict__ packed,
    const float* __restrict__ scales, int64_t N, int64_t K, int64_t row_words,
    float* __restrict__ y)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int64_t n0 = ((int64_t)blockIdx.x * (kGemvThreads / kWave) + wave) * kRows;
    if (n0 >= N) return;
    const int64_t nchunks = ceil_div(K, kChunk);
    const bool vec_ok = (K & 7) == 0;

    float acc[kRows][MT];
#pragma unroll
    for (int r = 0; r < kRows; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[r][m] = 0.0f;

    for (int64_t c = lane; c < nchunks; c += kWave) {
        float qf[kRows][kChunk];
#pragma unroll
        for (int r = 0; r < kRows; ++r) {
            uint32_t wd[B];
            const int64_t n = n0 + r < N ? n0 + r : N - 1;
            load_chunk_words<B>(packed + n * row_words, c, row_words, wd);
#pragma unroll
            for (int i = 0; i < B; ++i) wd[i] ^= code_msb_mask<B>(i);
#pragma unroll
            for (int j = 0; j < kChunk; ++j) qf[r][j] = (float)chunk_code_signed<B>(wd, j);
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            if (m < M) {
                float xv[kChunk];
                load_x_chunk(x + (int64_t)m * K, K, c, vec_ok, xv);
#pragma unroll
                for (int r = 0; r < kRows; ++r)
#pragma unroll
                    for (int j = 0; j < kChunk; ++j) acc[r][m] = fmaf(xv[j], qf[r][j], acc[r][m]);
            }
        }
    }

#pragma unroll
    for (int r = 0; r < kRows; ++r) {
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[r][m] = wave_sum(acc[r][m]);
    }
    if (lane == 0) {
#pragma unroll
        for (int r = 0; r < kRows; ++r) {
            const int64_t n = n0 + r;
            if (n < N) {
                const float s = scales[n];
#pragma unroll
                for (int m = 0; m < MT; ++m)
                    if (m < M) y[(int64_t)m * N + n] = s * acc[r][m];
            }
        }
    }
}

template <int B, int MT>
hipError_t launch_gemv_bm(const uint16_t* x, int64_t M, const uint32_t* packed, const float* scales,
                          int64_t N, int64_t K, float* y, hipStream_t stream)
{
    constexpr int kRows = 2;
    const int64_t rw = packed_row_words(K, B);
    const int64_t rows_per_block = (kGemvThreads / kWave) * kRows;
    const int64_t blocks = ceil_div(N, rows_per_block);
    gemv_kernel<B, MT, kRows><<<dim3((unsigned)blocks), dim3(kGemvThreads), 0, stream>>>(
        x, (int)M, packed, scales, N, K, rw, y);
    return hipGetLastError();
}

template <int B>
hipError_t launch_gemv_b(const uint16_t* x, int64_t M, const uint32_t* packed, const float* scales,
                         int64_t N, int64_t K, float* y, hipStream_t stream)
{
    if (M <= 1) return launch_gemv_bm<B, 1>(x, M, packed, scales, N, K, y, stream);
    if (M <= 2) return launch_gemv_bm<B, 2>(x, M, packed, scales, N, K, y, stream);
    if (M <= 4) return launch_gemv_bm<B, 4>(x, M, packed, scales, N, K, y, stream);
    if (M <= 8) return launch_gemv_bm<B, 8>(x, M, packed, scales, N, K, y, stream);
    return launch_gemv_bm<B, 16>(x, M, packed, scales, N, K, y, stream);
}

}  // namespace

hipError_t launch_gemv(const uint16_t* x, int64_t M, const uint32_t* packed, const float* scales,
                       int64_t N, int64_t K, int bits, float* y, hipStream_t stream)
{
#define CALL(B) launch_gemv_b<B>(x, M, packed, scales, N, K, y, stream)
    DQ_BITS_SWITCH(bits, CALL)
#undef CALL
}

}  // namespace dq
