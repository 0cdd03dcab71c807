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
//
// The statistic behind a matrix's sensitivity (DynaQuant page, "第一步：敏感度
// 测量": mean(w^2)) rides along in pass 1 when asked for: an fp64 sum of
// squares per row, and optionally one more launch that adds the rows up.
#include "common.hpp"
#include "launch.hpp"
#include "quant_rule.hpp"

namespace dq {

namespace {

constexpr int kQuantThreads = 256;

template <bool BF16, bool kAligned>
__device__ __forceinline__ void load_row_chunk(const void* __restrict__ w, int64_t row_off, int64_t K,
                                               int64_t c, bool vec_ok, float* v)
{
    const int64_t k0 = c * kChunk;
    if (BF16) {
        const uint16_t* p = reinterpret_cast<const uint16_t*>(w) + row_off + k0;
        if (kAligned || (vec_ok && k0 + kChunk <= K)) {
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
        if (kAligned || (vec_ok && k0 + kChunk <= K)) {
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

// q = clip(rint(fl32(w / s))) for the 32 elements of a chunk, as offset-binary
// codes packed into B words (elements at or past K give code 0 = zero bits).
// The divide: rounded_quotient (quant_rule.hpp) multiplies by r = fl32(1/s)
// and takes the IEEE divide only near a rounding tie.
template <int B>
__device__ __forceinline__ void quantize_chunk(const float (&v)[kChunk], float s, float r,
                                               float margin, bool zero_codes, int64_t k0,
                                               int64_t K, uint32_t (&out)[B])
{
    constexpr int32_t kQmax = (1 << (B - 1)) - 1;
    constexpr float kLo = (float)(-kQmax - 1);
    constexpr float kHi = (float)kQmax;
    constexpr float kBias = (float)(1 << (B - 1));
#pragma unroll
    for (int i = 0; i < B; ++i) out[i] = 0;
#pragma unroll
    for (int j = 0; j < kChunk; ++j) {
        float q = rounded_quotient(v[j], s, r, margin);
        q = fminf(fmaxf(q, kLo), kHi);
        // code u = q + 2^(B-1) in [0, 2^B): exact in fp32, converted once
        const uint32_t u = (zero_codes || k0 + j >= K) ? (k0 + j >= K ? 0u : (uint32_t)kBias)
                                                         : (uint32_t)(q + kBias);
        const int pos = j * B;
        const int wi = pos >> 5;
        const int off = pos & 31;
        out[wi] |= u << off;
        if (off + B > 32) out[wi + 1] |= u >> (32 - off);
    }
}

template <int B>
__device__ __forceinline__ void store_chunk(uint32_t* __restrict__ prow, int64_t c, int64_t row_words,
                                            const uint32_t (&out)[B])
{
    const int64_t base = c * B;
    if (base + B <= row_words) {
        store_words<B>(prow + base, out);
    } else {
#pragma unroll
        for (int i = 0; i < B; ++i)
            if (base + i < row_words) prow[base + i] = out[i];
    }
}

// Sum of squares of a chunk, added to acc in fp64: each square of an fp32
// value is exact in fp64, so the only roundings are those of the additions.
__device__ __forceinline__ double chunk_sumsq(const float (&v)[kChunk], double acc)
{
#pragma unroll
    for (int j = 0; j < kChunk; ++j) {
        const double d = (double)v[j];
        acc += d * d;
    }
    return acc;
}

// One workgroup of 64..256 threads per row (enough for one chunk per thread
// when K <= 8192).  kAligned (K a multiple of 32): every chunk is whole, so
// loads take the 16-byte vector path without per-lane bounds checks.  Each thread keeps its first chunk in registers between the
// max pass and the quantize pass; further chunks (long rows) are read again.
// kSumsq: pass 1 also sums w^2 over the row in fp64 (per lane in chunk order,
// then across the wave by a fixed butterfly, then over the waves in order) and
// writes it to row_sumsq[n]; the codes and scales are unchanged.
// nonfinite (may be null): a counter, zeroed before the launch, that gains one
// for every row holding a NaN or an infinity.
template <int B, bool BF16, bool kAligned, bool kSumsq>
__global__ __launch_bounds__(kQuantThreads) void quantize_pack_kernel(
    const void* __restrict__ w, int64_t K, int64_t row_words, uint32_t* __restrict__ packed,
    float* __restrict__ scales, double* __restrict__ row_sumsq, uint32_t* __restrict__ nonfinite)
{
    constexpr int32_t kQmax = (1 << (B - 1)) - 1;
    __shared__ uint32_t red[kQuantThreads / kWave];
    __shared__ double red_sq[kQuantThreads / kWave];

    const int64_t n = blockIdx.x;
    const int tid = threadIdx.x;
    const int threads = blockDim.x;
    const int waves = threads / kWave;
    const int64_t nchunks = ceil_div(K, kChunk);
    const int64_t row_off = n * K;
    const int esize = BF16 ? 2 : 4;
    // 16-byte vector loads need every row start 16-byte aligned
    const bool vec_ok = ((K * esize) & 15) == 0;

    // ---- pass 1: max |w| as an integer max over sign-cleared bit patterns
    float v0[kChunk];
    uint32_t amax = 0;
    double sq = 0.0;
    if (tid < nchunks) {
        load_row_chunk<BF16, kAligned>(w, row_off, K, tid, vec_ok, v0);
#pragma unroll
        for (int j = 0; j < kChunk; ++j) {
            const uint32_t m = __float_as_uint(v0[j]) & 0x7fffffffu;
            amax = m > amax ? m : amax;
        }
        if (kSumsq) sq = chunk_sumsq(v0, sq);
    }
    for (int64_t c = tid + threads; c < nchunks; c += threads) {
        float v[kChunk];
        load_row_chunk<BF16, kAligned>(w, row_off, K, c, vec_ok, v);
#pragma unroll
        for (int j = 0; j < kChunk; ++j) {
            const uint32_t m = __float_as_uint(v[j]) & 0x7fffffffu;
            amax = m > amax ? m : amax;
        }
        if (kSumsq) sq = chunk_sumsq(v, sq);
    }
    amax = wave_max_u32(amax);
    if ((tid & (kWave - 1)) == 0) red[tid / kWave] = amax;
    if (kSumsq) {
#pragma unroll
        for (int d = kWave / 2; d >= 1; d >>= 1) sq += __shfl_xor(sq, d, kWave);
        if ((tid & (kWave - 1)) == 0) red_sq[tid / kWave] = sq;
    }
    __syncthreads();
    for (int i = 0; i < waves; ++i) amax = red[i] > amax ? red[i] : amax;
    if (kSumsq && tid == 0) {
        double row = red_sq[0];
        for (int i = 1; i < waves; ++i) row += red_sq[i];
        row_sumsq[n] = row;
    }

    // ---- scale
    const float qmaxf = (float)kQmax;
    float s;
    bool zero_codes;
    if (amax >= 0x7f800000u) {  // a NaN or an infinity in the row
        s = __uint_as_float(0x7fc00000u);
        zero_codes = true;
        if (tid == 0 && nonfinite) atomicAdd(nonfinite, 1u);
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
    const float r = 1.0f / s;
    const float margin = quotient_margin(qmaxf + 1.0f);

    // ---- pass 2: quantize, offset, pack 32 codes into B whole words
    uint32_t* __restrict__ prow = packed + n * row_words;
    if (tid < nchunks) {
        uint32_t out[B];
        quantize_chunk<B>(v0, s, r, margin, zero_codes, (int64_t)tid * kChunk, K, out);
        store_chunk<B>(prow, tid, row_words, out);
    }
    for (int64_t c = tid + threads; c < nchunks; c += threads) {
        float v[kChunk];
        load_row_chunk<BF16, kAligned>(w, row_off, K, c, vec_ok, v);
        uint32_t out[B];
        quantize_chunk<B>(v, s, r, margin, zero_codes, c * kChunk, K, out);
        store_chunk<B>(prow, c, row_words, out);
    }
    // words past the last chunk are row padding
    for (int64_t i = nchunks * B + tid; i < row_words; i += threads) prow[i] = 0u;
}

// Group-wise scales ("量化" tutorial, exercise 1 of its exercises: one scale
// per group of g consecutive weights of a row, g = 32 gpc with gpc a power of
// two up to 64).  Each group is quantized exactly as a row of the per-row
// kernel above, with its own scale at scales[n * G + j], G = ceil(K / g).
// A group is gpc whole chunks held by gpc neighbouring lanes (aligned, inside
// one wave), so its max|w| is a butterfly over those lanes and the kernel
// needs one pass: every lane loads its chunk once, quantizes and stores it.
template <int B, bool BF16, bool kAligned>
__global__ __launch_bounds__(kQuantThreads) void quantize_pack_group_kernel(
    const void* __restrict__ w, int64_t K, int64_t row_words, int gpc, int64_t G,
    uint32_t* __restrict__ packed, float* __restrict__ scales)
{
    constexpr int32_t kQmax = (1 << (B - 1)) - 1;
    const int64_t n = blockIdx.x;
    const int tid = threadIdx.x;
    const int threads = blockDim.x;
    const int64_t nchunks = ceil_div(K, kChunk);
    const int64_t row_off = n * K;
    const int esize = BF16 ? 2 : 4;
    const bool vec_ok = ((K * esize) & 15) == 0;
    const float qmaxf = (float)kQmax;
    const float margin = quotient_margin(qmaxf + 1.0f);
    uint32_t* __restrict__ prow = packed + n * row_words;

    // every lane of a wave takes part in each round (the butterfly needs them)
    for (int64_t c0 = 0; c0 < nchunks; c0 += threads) {
        const int64_t c = c0 + tid;
        float v[kChunk];
        uint32_t amax = 0;
        if (c < nchunks) {
            load_row_chunk<BF16, kAligned>(w, row_off, K, c, vec_ok, v);
#pragma unroll
            for (int j = 0; j < kChunk; ++j) {
                const uint32_t m = __float_as_uint(v[j]) & 0x7fffffffu;
                amax = m > amax ? m : amax;
            }
        }
        for (int d = 1; d < gpc; d <<= 1) {
            const uint32_t o = (uint32_t)__shfl_xor((int)amax, d, kWave);
            amax = o > amax ? o : amax;
        }
        float s;
        bool zero_codes;
        if (amax >= 0x7f800000u) {  // a NaN or an infinity in the group
            s = __uint_as_float(0x7fc00000u);
            zero_codes = true;
        } else {
            const float a = __uint_as_float(amax);
            s = (a == 0.0f ? 1.0f : a) / qmaxf;
            zero_codes = (a == 0.0f);
            if (s == 0.0f) {  // max / qmax underflowed: an all-zero group
                s = 1.0f / qmaxf;
                zero_codes = true;
            }
        }
        if (c < nchunks) {
            if (c % gpc == 0) scales[n * G + c / gpc] = s;
            uint32_t out[B];
            quantize_chunk<B>(v, s, 1.0f / s, margin, zero_codes, c * kChunk, K, out);
            store_chunk<B>(prow, c, row_words, out);
        }
    }
    for (int64_t i = nchunks * B + tid; i < row_words; i += threads) prow[i] = 0u;
}

// Asymmetric scheme ("量化" tutorial, "量化怎么工作": a zero point added to the
// rounded quotient, for rows not centred on zero).  Per row, with L = 2^b - 1:
// lo = min(0, min w), hi = max(0, max w), s = fl32(fl32(hi - lo) / L) (1.0
// replaces a zero range), z = clip(rint(fl32(-lo / s)), 0, L), codes
// u = clip(rint(fl32(w / s)) + z, 0, L), stored unsigned.  A row with a NaN
// or an infinity, or whose range overflows, gets s = NaN and z = every code =
// 2^(b-1); a row whose s underflows gets s = fl32(1/L), z = 0, codes 0.  Same
// structure as the symmetric kernel: pass 1 reduces the row's min and max
// (order-independent, exact), pass 2 turns each lane's chunk into B words.
template <int B>
__device__ __forceinline__ void quantize_chunk_asym(const float (&v)[kChunk], float s, float r,
                                                    float margin, float zf, int mode, int64_t k0,
                                                    int64_t K, uint32_t (&out)[B])
{
    constexpr float kL = (float)((1 << B) - 1);
#pragma unroll
    for (int i = 0; i < B; ++i) out[i] = 0;
#pragma unroll
    for (int j = 0; j < kChunk; ++j) {
        float q = rounded_quotient(v[j], s, r, margin);
        const float c = fminf(fmaxf(q + zf, 0.0f), kL);
        uint32_t u = mode == 0 ? (uint32_t)c : (mode == 1 ? (1u << (B - 1)) : 0u);
        if (k0 + j >= K) u = 0;
        const int pos = j * B;
        const int wi = pos >> 5;
        const int off = pos & 31;
        out[wi] |= u << off;
        if (off + B > 32) out[wi + 1] |= u >> (32 - off);
    }
}

template <int B, bool BF16, bool kAligned>
__global__ __launch_bounds__(kQuantThreads) void quantize_pack_asym_kernel(
    const void* __restrict__ w, int64_t K, int64_t row_words, uint32_t* __restrict__ packed,
    float* __restrict__ scales, int32_t* __restrict__ zeros)
{
    constexpr int32_t kL = (1 << B) - 1;
    __shared__ float red_lo[kQuantThreads / kWave], red_hi[kQuantThreads / kWave];
    __shared__ int red_bad[kQuantThreads / kWave];

    const int64_t n = blockIdx.x;
    const int tid = threadIdx.x;
    const int threads = blockDim.x;
    const int waves = threads / kWave;
    const int64_t nchunks = ceil_div(K, kChunk);
    const int64_t row_off = n * K;
    const int esize = BF16 ? 2 : 4;
    const bool vec_ok = ((K * esize) & 15) == 0;

    // ---- pass 1: min and max (with 0) and whether anything is not finite
    float v0[kChunk];
    float lo = 0.0f, hi = 0.0f;
    bool bad = false;
    auto scan = [&](const float (&v)[kChunk]) {
#pragma unroll
        for (int j = 0; j < kChunk; ++j) {
            bad |= !__builtin_isfinite(v[j]);
            lo = fminf(lo, v[j]);
            hi = fmaxf(hi, v[j]);
        }
    };
    if (tid < nchunks) {
        load_row_chunk<BF16, kAligned>(w, row_off, K, tid, vec_ok, v0);
        scan(v0);
    }
    for (int64_t c = tid + threads; c < nchunks; c += threads) {
        float v[kChunk];
        load_row_chunk<BF16, kAligned>(w, row_off, K, c, vec_ok, v);
        scan(v);
    }
#pragma unroll
    for (int d = kWave / 2; d >= 1; d >>= 1) {
        lo = fminf(lo, __shfl_xor(lo, d, kWave));
        hi = fmaxf(hi, __shfl_xor(hi, d, kWave));
    }
    const bool wave_bad = __any(bad);
    if ((tid & (kWave - 1)) == 0) {
        red_lo[tid / kWave] = lo;
        red_hi[tid / kWave] = hi;
        red_bad[tid / kWave] = wave_bad ? 1 : 0;
    }
    __syncthreads();
    int any_bad = 0;
    for (int i = 0; i < waves; ++i) {
        lo = fminf(lo, red_lo[i]);
        hi = fmaxf(hi, red_hi[i]);
        any_bad |= red_bad[i];
    }

    // ---- scale and zero point
    const float Lf = (float)kL;
    const float range = hi - lo;
    float s, zf = 0.0f;
    int mode = 0;  // 0 quantize, 1 every code 2^(b-1), 2 every code 0
    if (any_bad || !__builtin_isfinite(range)) {
        s = __uint_as_float(0x7fc00000u);
        zf = (float)(1 << (B - 1));
        mode = 1;
    } else {
        s = (range == 0.0f ? 1.0f : range) / Lf;
        if (s == 0.0f) {  // range / L underflowed: treated as an all-zero row
            s = 1.0f / Lf;
            mode = 2;
        } else {
            zf = fminf(fmaxf(rintf(-lo / s), 0.0f), Lf);
        }
    }
    if (tid == 0) {
        scales[n] = s;
        zeros[n] = (int32_t)zf;
    }
    const float r = 1.0f / s;
    // |w / s| <= L (1 + 2^-22): the reciprocal product stays within
    // 2^-22 (L + 1) of fl32(w / s), so rint agrees outside that margin
    const float margin = quotient_margin(Lf + 1.0f);

    // ---- pass 2: codes, packed 32 to B whole words
    uint32_t* __restrict__ prow = packed + n * row_words;
    if (tid < nchunks) {
        uint32_t out[B];
        quantize_chunk_asym<B>(v0, s, r, margin, zf, mode, (int64_t)tid * kChunk, K, out);
        store_chunk<B>(prow, tid, row_words, out);
    }
    for (int64_t c = tid + threads; c < nchunks; c += threads) {
        float v[kChunk];
        load_row_chunk<BF16, kAligned>(w, row_off, K, c, vec_ok, v);
        uint32_t out[B];
        quantize_chunk_asym<B>(v, s, r, margin, zf, mode, c * kChunk, K, out);
        store_chunk<B>(prow, c, row_words, out);
    }
    for (int64_t i = nchunks * B + tid; i < row_words; i += threads) prow[i] = 0u;
}

// One workgroup per row; thread t turns codes 4t .. 4t+3 (then + 1024, ...)
// into int32 q (and fl32(q * s)), so every store instruction of a wave writes
// one contiguous 1 KB run (or 256 B of dword stores when rows are not 16-byte
// aligned).  The 4 codes occupy 4B bits from bit 4tB of the row stream: at most
// three words, read through the L1 (neighbouring lanes share them), with
// run-time funnel shifts.
constexpr int kUnpackThreads = 256;

template <int B>
__global__ __launch_bounds__(kUnpackThreads) void unpack_kernel(
    const uint32_t* __restrict__ packed, const float* __restrict__ scales,
    const int32_t* __restrict__ zeros, int64_t group, int64_t K, int64_t row_words,
    int32_t* __restrict__ q_out, float* __restrict__ w_out)
{
    constexpr uint32_t kMask = (1u << B) - 1u;
    const int64_t n = blockIdx.x;
    // the code's offset: 2^(b-1) (symmetric scheme) or the row's zero point
    const int32_t kBias = zeros ? zeros[n] : (1 << (B - 1));
    const uint32_t* __restrict__ row = packed + n * row_words;
    // group > 0: a scale per group of `group` codes (a multiple of 4, so the
    // 4 codes of a thread share it); else one per row
    const int64_t G = group > 0 ? ceil_div(K, group) : 0;
    const float s_row = w_out && group == 0 ? scales[n] : 0.0f;
    // 16-byte stores need every output row start 16-byte aligned
    const bool vec = (K & 3) == 0 && ((reinterpret_cast<uintptr_t>(q_out) | reinterpret_cast<uintptr_t>(w_out)) & 15) == 0;
    for (int64_t k0 = 4 * (int64_t)threadIdx.x; k0 < K; k0 += 4 * kUnpackThreads) {
        const int64_t bit = k0 * B;
        const int64_t wi = bit >> 5;
        const uint32_t off = (uint32_t)(bit & 31);
        const uint32_t w0 = row[wi];
        const uint32_t w1 = wi + 1 < row_words ? row[wi + 1] : 0u;
        const uint32_t w2 = wi + 2 < row_words ? row[wi + 2] : 0u;
        const uint32_t lo = __builtin_amdgcn_alignbit(w1, w0, off);  // stream bits [bit, bit+32)
        const uint32_t hi = __builtin_amdgcn_alignbit(w2, w1, off);  // [bit+32, bit+64)
        const uint64_t v = (uint64_t)hi << 32 | lo;
        int32_t q[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) q[j] = (int32_t)((uint32_t)(v >> (j * B)) & kMask) - kBias;
        const int64_t o = n * K + k0;
        const float s = w_out && group > 0 ? scales[n * G + k0 / group] : s_row;
        if (vec) {
            if (q_out) *reinterpret_cast<int4*>(q_out + o) = make_int4(q[0], q[1], q[2], q[3]);
            if (w_out)
                *reinterpret_cast<float4*>(w_out + o) =
                    make_float4((float)q[0] * s, (float)q[1] * s, (float)q[2] * s, (float)q[3] * s);
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (k0 + j < K) {
                    if (q_out) q_out[o + j] = q[j];
                    if (w_out) w_out[o + j] = (float)q[j] * s;
                }
            }
        }
    }
}

// The statistic alone (the measurement step comes before any width is
// chosen): one wave per row, so a row needs no workgroup barrier, and each
// lane keeps 256 bytes of loads in flight (4 chunks of bf16, 2 of fp32), held
// as raw words until they are added.  Lane l adds the chunks l, l + 64,
// l + 128, ... of its row in that order, element by element, then the wave
// meets by a fixed butterfly: the same bits on every call.
constexpr int kSumsqWaves = 4;

__device__ __forceinline__ double add_sq(double acc, float v)
{
    const double d = (double)v;
    return acc + d * d;
}

template <bool BF16, bool kAligned>
__global__ __launch_bounds__(kSumsqWaves * kWave) void row_sumsq_kernel(
    const void* __restrict__ w, int64_t N, int64_t K, double* __restrict__ row_sumsq)
{
    constexpr int kU = BF16 ? 4 : 2;            // chunks per lane per round
    constexpr int kVec = BF16 ? 4 : 8;          // 16-byte loads per chunk
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t n = (int64_t)blockIdx.x * kSumsqWaves + (threadIdx.x >> 6);
    if (n >= N) return;  // the whole wave leaves; nothing below waits on it
    const int64_t nchunks = ceil_div(K, kChunk);
    const int esize = BF16 ? 2 : 4;
    const bool vec_ok = ((K * esize) & 15) == 0;
    double sq = 0.0;
    if (kAligned && vec_ok) {
        const uint4* row = reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(w) +
                                                          n * K * esize);
        for (int64_t c0 = lane; c0 < nchunks; c0 += (int64_t)kWave * kU) {
            uint4 raw[kU][kVec];
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                const int64_t c = c0 + (int64_t)u * kWave;
#pragma unroll
                for (int i = 0; i < kVec; ++i)
                    raw[u][i] = c < nchunks ? row[c * kVec + i] : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int u = 0; u < kU; ++u) {
#pragma unroll
                for (int i = 0; i < kVec; ++i) {
                    const uint32_t e[4] = {raw[u][i].x, raw[u][i].y, raw[u][i].z, raw[u][i].w};
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        if (BF16) {
                            sq = add_sq(sq, __uint_as_float(e[j] << 16));
                            sq = add_sq(sq, __uint_as_float(e[j] & 0xffff0000u));
                        } else {
                            sq = add_sq(sq, __uint_as_float(e[j]));
                        }
                    }
                }
            }
        }
    } else {
        for (int64_t c = lane; c < nchunks; c += kWave) {
            float v[kChunk];
            load_row_chunk<BF16, false>(w, n * K, K, c, vec_ok, v);
            sq = chunk_sumsq(v, sq);
        }
    }
#pragma unroll
    for (int d = kWave / 2; d >= 1; d >>= 1) sq += __shfl_xor(sq, d, kWave);
    if (lane == 0) row_sumsq[n] = sq;
}

// One workgroup adds the N row sums in a fixed order: thread t takes the
// runs of 8 rows starting at 8t, 8t + 8192, ... (all 8 loads issued before the
// adds), then the 1024 partial sums meet by a fixed tree in LDS.
constexpr int kSumThreads = 1024;
constexpr int kSumRun = 8;

__global__ __launch_bounds__(kSumThreads) void sum_rows_kernel(const double* __restrict__ rows,
                                                               int64_t N, double* __restrict__ out)
{
    __shared__ double part[kSumThreads];
    double acc = 0.0;
    for (int64_t base = (int64_t)threadIdx.x * kSumRun; base < N;
         base += (int64_t)kSumThreads * kSumRun) {
        double v[kSumRun];
#pragma unroll
        for (int u = 0; u < kSumRun; ++u) v[u] = base + u < N ? rows[base + u] : 0.0;
#pragma unroll
        for (int u = 0; u < kSumRun; ++u) acc += v[u];
    }
    part[threadIdx.x] = acc;
    __syncthreads();
    for (int d = kSumThreads / 2; d >= 1; d >>= 1) {
        if ((int)threadIdx.x < d) part[threadIdx.x] += part[threadIdx.x + d];
        __syncthreads();
    }
    if (threadIdx.x == 0) out[0] = part[0];
}

__global__ void zero_u32_kernel(uint32_t* __restrict__ p)
{
    if (threadIdx.x == 0) *p = 0u;
}

template <int B, bool kSumsq>
hipError_t launch_quantize_pack_b(const void* w, bool bf16, int64_t N, int64_t K, uint32_t* packed,
                                  float* scales, double* row_sumsq, uint32_t* nonfinite,
                                  hipStream_t stream)
{
    const int64_t rw = packed_row_words(K, B);
    if (nonfinite) {  // a fill kernel rather than a memset node (graph-capture safe)
        zero_u32_kernel<<<dim3(1), dim3(kWave), 0, stream>>>(nonfinite);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // one chunk per thread where the row allows, in whole waves, 64..256 threads
    const int64_t nchunks = ceil_div(K, kChunk);
    const int threads = (int)(nchunks >= kQuantThreads ? kQuantThreads
                                                       : ceil_div(nchunks, kWave) * kWave);
    const dim3 grid((unsigned)N), block(threads);
    const bool aligned = K % kChunk == 0;
    if (bf16 && aligned)
        quantize_pack_kernel<B, true, true, kSumsq>
            <<<grid, block, 0, stream>>>(w, K, rw, packed, scales, row_sumsq, nonfinite);
    else if (bf16)
        quantize_pack_kernel<B, true, false, kSumsq>
            <<<grid, block, 0, stream>>>(w, K, rw, packed, scales, row_sumsq, nonfinite);
    else if (aligned)
        quantize_pack_kernel<B, false, true, kSumsq>
            <<<grid, block, 0, stream>>>(w, K, rw, packed, scales, row_sumsq, nonfinite);
    else
        quantize_pack_kernel<B, false, false, kSumsq>
            <<<grid, block, 0, stream>>>(w, K, rw, packed, scales, row_sumsq, nonfinite);
    return hipGetLastError();
}

template <int B>
hipError_t launch_unpack_b(const uint32_t* packed, const float* scales, const int32_t* zeros,
                           int64_t group, int64_t N, int64_t K, int32_t* q_out, float* w_out,
                           hipStream_t stream)
{
    const int64_t rw = packed_row_words(K, B);
    unpack_kernel<B><<<dim3((unsigned)N), dim3(kUnpackThreads), 0, stream>>>(
        packed, scales, zeros, group, K, rw, q_out, w_out);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_pack(const void* w, bool bf16, int64_t N, int64_t K, int bits,
                                uint32_t* packed, float* scales, uint32_t* nonfinite,
                                hipStream_t stream)
{
#define CALL(B) launch_quantize_pack_b<B, false>(w, bf16, N, K, packed, scales, nullptr, nonfinite, stream)
    DQ_BITS_SWITCH(bits, CALL)
#undef CALL
}

hipError_t launch_quantize_pack_sumsq(const void* w, bool bf16, int64_t N, int64_t K, int bits,
                                      uint32_t* packed, float* scales, double* row_sumsq,
                                      double* matrix_sumsq, hipStream_t stream)
{
    hipError_t e;
#define CALL(B) launch_quantize_pack_b<B, true>(w, bf16, N, K, packed, scales, row_sumsq, nullptr, stream)
    e = [&]() -> hipError_t { DQ_BITS_SWITCH(bits, CALL) }();
#undef CALL
    if (e != hipSuccess || !matrix_sumsq) return e;
    sum_rows_kernel<<<dim3(1), dim3(kSumThreads), 0, stream>>>(row_sumsq, N, matrix_sumsq);
    return hipGetLastError();
}

template <int B>
hipError_t launch_quantize_pack_asym_b(const void* w, bool bf16, int64_t N, int64_t K,
                                       uint32_t* packed, float* scales, int32_t* zeros,
                                       hipStream_t stream)
{
    const int64_t rw = packed_row_words(K, B);
    const int64_t nchunks = ceil_div(K, kChunk);
    const int threads = (int)(nchunks >= kQuantThreads ? kQuantThreads
                                                       : ceil_div(nchunks, kWave) * kWave);
    const dim3 grid((unsigned)N), block(threads);
    const bool aligned = K % kChunk == 0;
    if (bf16 && aligned)
        quantize_pack_asym_kernel<B, true, true><<<grid, block, 0, stream>>>(w, K, rw, packed, scales,
                                                                             zeros);
    else if (bf16)
        quantize_pack_asym_kernel<B, true, false><<<grid, block, 0, stream>>>(w, K, rw, packed,
                                                                              scales, zeros);
    else if (aligned)
        quantize_pack_asym_kernel<B, false, true><<<grid, block, 0, stream>>>(w, K, rw, packed,
                                                                              scales, zeros);
    else
        quantize_pack_asym_kernel<B, false, false><<<grid, block, 0, stream>>>(w, K, rw, packed,
                                                                               scales, zeros);
    return hipGetLastError();
}

template <int B>
hipError_t launch_quantize_pack_group_b(const void* w, bool bf16, int64_t N, int64_t K,
                                        int64_t group, uint32_t* packed, float* scales,
                                        hipStream_t stream)
{
    const int64_t rw = packed_row_words(K, B);
    const int64_t nchunks = ceil_div(K, kChunk);
    const int threads = (int)(nchunks >= kQuantThreads ? kQuantThreads
                                                       : ceil_div(nchunks, kWave) * kWave);
    const dim3 grid((unsigned)N), block(threads);
    const int gpc = (int)(group / kChunk);
    const int64_t G = ceil_div(K, group);
    const bool aligned = K % kChunk == 0;
    if (bf16 && aligned)
        quantize_pack_group_kernel<B, true, true>
            <<<grid, block, 0, stream>>>(w, K, rw, gpc, G, packed, scales);
    else if (bf16)
        quantize_pack_group_kernel<B, true, false>
            <<<grid, block, 0, stream>>>(w, K, rw, gpc, G, packed, scales);
    else if (aligned)
        quantize_pack_group_kernel<B, false, true>
            <<<grid, block, 0, stream>>>(w, K, rw, gpc, G, packed, scales);
    else
        quantize_pack_group_kernel<B, false, false>
            <<<grid, block, 0, stream>>>(w, K, rw, gpc, G, packed, scales);
    return hipGetLastError();
}

hipError_t launch_row_sumsq(const void* w, bool bf16, int64_t N, int64_t K, double* row_sumsq,
                            double* matrix_sumsq, hipStream_t stream)
{
    const dim3 grid((unsigned)ceil_div(N, kSumsqWaves)), block(kSumsqWaves * kWave);
    const bool aligned = K % kChunk == 0;
    if (bf16 && aligned)
        row_sumsq_kernel<true, true><<<grid, block, 0, stream>>>(w, N, K, row_sumsq);
    else if (bf16)
        row_sumsq_kernel<true, false><<<grid, block, 0, stream>>>(w, N, K, row_sumsq);
    else if (aligned)
        row_sumsq_kernel<false, true><<<grid, block, 0, stream>>>(w, N, K, row_sumsq);
    else
        row_sumsq_kernel<false, false><<<grid, block, 0, stream>>>(w, N, K, row_sumsq);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !matrix_sumsq) return e;
    sum_rows_kernel<<<dim3(1), dim3(kSumThreads), 0, stream>>>(row_sumsq, N, matrix_sumsq);
    return hipGetLastError();
}

hipError_t launch_quantize_pack_asym(const void* w, bool bf16, int64_t N, int64_t K, int bits,
                                     uint32_t* packed, float* scales, int32_t* zeros,
                                     hipStream_t stream)
{
#define CALL(B) launch_quantize_pack_asym_b<B>(w, bf16, N, K, packed, scales, zeros, stream)
    DQ_BITS_SWITCH(bits, CALL)
#undef CALL
}

hipError_t launch_quantize_pack_group(const void* w, bool bf16, int64_t N, int64_t K, int bits,
                                      int64_t group, uint32_t* packed, float* scales,
                                      hipStream_t stream)
{
#define CALL(B) launch_quantize_pack_group_b<B>(w, bf16, N, K, group, packed, scales, stream)
    DQ_BITS_SWITCH(bits, CALL)
#undef CALL
}

hipError_t launch_unpack(const uint32_t* packed, const float* scales, const int32_t* zeros,
                         int64_t group, int64_t N, int64_t K, int bits, int32_t* q_out,
                         float* w_out, hipStream_t stream)
{
#define CALL(B) launch_unpack_b<B>(packed, scales, zeros, group, N, K, q_out, w_out, stream)
    DQ_BITS_SWITCH(bits, CALL)
#undef CALL
}

}  // namespace dq
