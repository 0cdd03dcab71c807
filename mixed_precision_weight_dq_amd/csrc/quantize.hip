// Quantize + pack and unpack kernels.
//
// Quantizer: "量化" (Quantization) tutorial, aiknowledge.cn, "how quantization
// works" and the per-channel code of "Step 1" -- per row n of W[N, K]:
//   s = fl32(max|w| / qmax) (1.0 replaces a zero max), q = clip(rint(fl32(w/s)))
// in IEEE fp32 with a correctly rounded divide and round-half-to-even
// (v_rndne_f32).  Packing: DynaQuant page, "自定义内核架构" and "项目现状与路线图"
// (dense b-bit codes; pack / unpack utilities).
//
// One workgroup owns one row.  Pass 1 reduces max|w| over the row (as fp32
// bit patterns with the sign cleared: an order-independent integer max, so the
// result is exact and NaN/Inf are seen as larger than every finite value).
// Pass 2 re-reads the row (L2-resident), and each lane turns 32 consecutive
// elements into exactly B whole output words, so no two lanes share a word.
#include "common.hpp"
#include "launch.hpp"

namespace dq {

namespace {

constexpr int kQuantThreads = 256;

template <bool BF16>
__device__ __forceinline__ void load_row_chunk(const void* __restrict__ w, int64_t row_off, int64_t K,
                                               int64_t c, bool vec_ok, float* v)
{
    const int64_t k0 = c * kChunk;
    if (BF16) {
        const uint16_t* p = reinterpret_cast<const uint16_t*>(w) + row_off + k0;
        if (vec_ok && k0 + kChunk <= K) {
            const uint4* p4 = reinterpret_cast<const uint4*>(p);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint4 d = p4[i];
                const uint32_t u[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[i * 8 + e * 2 + 0] = __uint_as_float(u[e] << 16);
                    v[i * 8 + e * 2 + 1] = __uint_as_float(u[e] & 0xffff0000u);
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < kChunk; ++j)
                v[j] = (k0 + j < K) ? bf16_bits_to_float(p[j]) : 0.0f;
        }
    } else {
        const float* p = reinterpret_cast<const float*>(w) + row_off + k0;
        if (vec_ok && k0 + kChunk <= K) {
            const float4* p4 = reinterpret_cast<const float4*>(p);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float4 d = p4[i];
                v[i * 4 + 0] = d.x;
                v[i * 4 + 1] = d.y;
                v[i * 4 + 2] = d.z;
                v[i * 4 + 3] = d.w;
            }
        } else {
#pragma unroll
            for (int j = 0; j < kChunk; ++j) v[j] = (k0 + j < K) ? p[j] : 0.0f;
        }
    }
}

template <int B, bool BF16>
__global__ __launch_bounds__(kQuantThreads) void quantize_pack_kernel(
    const void* __restrict__ w, int64_t K, int64_t row_words, uint32_t* __restrict__ packed,
    float* __restrict__ scales)
{
    constexpr int32_t kQmax = (1 << (B - 1)) - 1;
    constexpr uint32_t kBias = 1u << (B - 1);
    __shared__ uint32_t red[kQuantThreads / kWave];

    const int64_t n = blockIdx.x;
    const int tid = threadIdx.x;
    const int64_t nchunks = ceil_div(K, kChunk);
    const int64_t row_off = n * K;
    const int esize = BF16 ? 2 : 4;
    // 16-byte vector loads need every row start 16-byte aligned
    const bool vec_ok = ((K * esize) & 15) == 0;

    // ---- pass 1: max |w| as an integer max over sign-cleared bit patterns
    uint32_t amax = 0;
    for (int64_t c = tid; c < nchunks; c += kQuantThreads) {
        float v[kChunk];
        load_row_chunk<BF16>(w, row_off, K, c, vec_ok, v);
#pragma unroll
        for (int j = 0; j < kChunk; ++j) {
            const uint32_t m = __float_as_uint(v[j]) & 0x7fffffffu;
            amax = m > amax ? m : amax;
        }
    }
    amax = wave_max_u32(amax);
    if ((tid & (kWave - 1)) == 0) red[tid / kWave] = amax;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kQuantThreads / kWave; ++i) amax = red[i] > amax ? red[i] : amax;

    // ---- scale
    const float qmaxf = (float)kQmax;
    float s;
    bool zero_codes;
    if (amax >= 0x7f800000u) {  // a NaN or an infinity in the row
        s = __uint_as_float(0x7fc00000u);
        zero_codes = true;
    } else {
        const float a = __uint_as_float(amax);
        s = (a == 0.0f ? 1.0f : a) / qmaxf;
        zero_codes = (a == 0.0f);
        if (s == 0.0f) {  // max / qmax underflowed: treated as an all-zero row
            s = 1.0f / qmaxf;
            zero_codes = true;
        }
    }
    if (tid == 0) scales[n] = s;

    // ---- pass 2: quantize, offset, pack 32 codes into B whole words
    uint32_t* __restrict__ prow = packed + n * row_words;
    for (int64_t c = tid; c < nchunks; c += kQuantThreads) {
        float v[kChunk];
        load_row_chunk<BF16>(w, row_off, K, c, vec_ok, v);
        uint32_t out[B];
#pragma unroll
        for (int i = 0; i < B; ++i) out[i] = 0;
#pragma unroll
        for (int j = 0; j < kChunk; ++j) {
            float r = rintf(v[j] / s);
            r = fminf(fmaxf(r, -qmaxf - 1.0f), qmaxf);
            const int32_t q = zero_codes ? 0 : (int32_t)r;
            const uint32_t u = (c * kChunk + j < K) ? (uint32_t)(q + (int32_t)kBias) : 0u;
            const int pos = j * B;
            const int wi = pos >> 5;
            const int off = pos & 31;
            out[wi] |= u << off;
            if (off + B > 32) out[wi + 1] |= u >> (32 - off);
        }
        const int64_t base = c * B;
        if (base + B <= row_words) {
#pragma unroll
            for (int i = 0; i < B; ++i) prow[base + i] = out[i];
        } else {
#pragma unroll
            for (int i = 0; i < B; ++i)
                if (base + i < row_words) prow[base + i] = out[i];
        }
    }
    // words past the last chunk are row padding
    for (int64_t i = nchunks * B + tid; i < row_words; i += kQuantThreads) prow[i] = 0u;
}

// One thread per chunk: B words -> 32 int32 codes (and fl32(q * s)).
template <int B>
__global__ __launch_bounds__(256) void unpack_kernel(const uint32_t* __restrict__ packed,
                                                     const float* __restrict__ scales, int64_t N,
                                                     int64_t K, int64_t row_words,
                                                     int32_t* __restrict__ q_out,
                                                     float* __restrict__ w_out)
{
    constexpr int32_t kBias = 1 << (B - 1);
    const int64_t nchunks = ceil_div(K, kChunk);
    const int64_t total = N * nchunks;
    for (int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; gid < total;
         gid += (int64_t)gridDim.x * blockDim.x) {
    const int64_t n = gid / nchunks;
    const int64_t c = gid - n * nchunks;
    uint32_t wd[B];
    load_chunk_words<B>(packed + n * row_words, c, row_words, wd);
    const float s = w_out ? scales[n] : 0.0f;
    const int64_t k0 = c * kChunk;
    const int64_t o = n * K + k0;
    const bool full = k0 + kChunk <= K;
#pragma unroll
    for (int j = 0; j < kChunk; ++j) {
        if (full || k0 + j < K) {
            const int32_t q = (int32_t)chunk_code_unsigned<B>(wd, j) - kBias;
            if (q_out) q_out[o + j] = q;
            if (w_out) w_out[o + j] = (float)q * s;
        }
    }
    }
}

template <int B>
hipError_t launch_quantize_pack_b(const void* w, bool bf16, int64_t N, int64_t K, uint32_t* packed,
                                  float* scales, hipStream_t stream)
{
    const int64_t rw = packed_row_words(K, B);
    if (bf16)
        quantize_pack_kernel<B, true><<<dim3((unsigned)N), dim3(kQuantThreads), 0, stream>>>(
            w, K, rw, packed, scales);
    else
        quantize_pack_kernel<B, false><<<dim3((unsigned)N), dim3(kQuantThreads), 0, stream>>>(
            w, K, rw, packed, scales);
    return hipGetLastError();
}

template <int B>
hipError_t launch_unpack_b(const uint32_t* packed, const float* scales, int64_t N, int64_t K,
                           int32_t* q_out, float* w_out, hipStream_t stream)
{
    const int64_t rw = packed_row_words(K, B);
    const int64_t threads = N * ceil_div(K, kChunk);
    const int64_t blocks = ceil_div(threads, 256) < 65536 ? ceil_div(threads, 256) : 65536;
    unpack_kernel<B><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(packed, scales, N, K, rw,
                                                                       q_out, w_out);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_pack(const void* w, bool bf16, int64_t N, int64_t K, int bits,
                                uint32_t* packed, float* scales, hipStream_t stream)
{
#define CALL(B) launch_quantize_pack_b<B>(w, bf16, N, K, packed, scales, stream)
    DQ_BITS_SWITCH(bits, CALL)
#undef CALL
}

hipError_t launch_unpack(const uint32_t* packed, const float* scales, int64_t N, int64_t K,
                         int bits, int32_t* q_out, float* w_out, hipStream_t stream)
{
#define CALL(B) launch_unpack_b<B>(packed, scales, N, K, q_out, w_out, stream)
    DQ_BITS_SWITCH(bits, CALL)
#undef CALL
}

}  // namespace dq
