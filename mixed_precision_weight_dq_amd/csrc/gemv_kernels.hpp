// Device code shared by the decode-shaped product kernels (gemv.hip, one
// matrix per launch; gemv_batch.hip, several matrices per launch): the x
// staging helpers, the per-chunk dot products of both schemes, and the body of
// the resident-x kernel (1 <= M <= 2).
//
// Packed layout, scheme and exactness as in gemv.hip's header: a lane owns a
// chunk (32 codes = B whole words); codes become signed integers and meet x
// in exact bf16 pair dot products (fp32 FMAs for wide codes), accumulated in
// fp32; the row scale multiplies the reduced sum once.
#pragma once

#include <type_traits>

#include "common.hpp"
#include "gemm_tiles.hpp"

namespace dq {

namespace {

// byte offset past the end of any buffer: a buffer load there returns zeros
// and moves no data
constexpr uint32_t kOutsideOffset = 0xfffff000u;

// A slice is 64 chunks (2048 codes), one per lane of a wave; x sits in LDS
// one 80-byte slot per chunk (64 bytes of bf16 plus 16 bytes of padding).
constexpr int kSlice = 64;            // chunks per slice (one per lane)
constexpr int kGemvMfmaWaves = 4;     // waves of a matrix-core GEMV workgroup
constexpr int kXPitch = 40;           // LDS slot per chunk in bf16 units (64 B + 16 B pad)

// E (8 or 4) consecutive x elements of each of the MT rows starting at element
// k, packed as bf16 pairs; zero past K or for rows m >= M.
template <int MT, int E>
__device__ __forceinline__ void stage_x_load(const uint16_t* __restrict__ x, int M, int64_t K,
                                             int64_t k, bool xvec, uint4 (&v)[MT])
{
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const uint16_t* src = x + (int64_t)m * K + k;
        if (m < M && xvec && k + E <= K) {
            if constexpr (E == 8) {
                v[m] = *reinterpret_cast<const uint4*>(src);
            } else {
                const uint2 d = *reinterpret_cast<const uint2*>(src);
                v[m] = make_uint4(d.x, d.y, 0u, 0u);
            }
        } else {
            uint32_t d[4] = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int i = 0; i < E / 2; ++i) {
                const uint32_t lo = (m < M && k + 2 * i < K) ? src[2 * i] : 0u;
                const uint32_t hi = (m < M && k + 2 * i + 1 < K) ? src[2 * i + 1] : 0u;
                d[i] = lo | hi << 16;
            }
            v[m] = make_uint4(d[0], d[1], d[2], d[3]);
        }
    }
}

// LDS slot of x row m is dst + m * kSlice * kXPitch elements.
template <int MT, int E>
__device__ __forceinline__ void stage_x_store(uint16_t* dst, const uint4 (&v)[MT])
{
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        if constexpr (E == 8)
            *reinterpret_cast<uint4*>(dst + m * kSlice * kXPitch) = v[m];
        else
            *reinterpret_cast<uint2*>(dst + m * kSlice * kXPitch) = make_uint2(v[m].x, v[m].y);
    }
}

template <int B, int kRows>
__device__ __forceinline__ void stage_w_load(const uint32_t* const (&rowp)[kRows], int64_t c,
                                             int64_t nchunks, int64_t row_words,
                                             uint32_t (&w)[kRows][B])
{
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
        if (c < nchunks) {
            load_chunk_words<B>(rowp[r], c, row_words, w[r]);
        } else {
#pragma unroll
            for (int i = 0; i < B; ++i) w[r][i] = 0;
        }
    }
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x2_t bf16_pair(float lo, float hi)
{
    return __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t);  // v_cvt_pk_bf16_f32
}

// acc + q.lo * x.lo + q.hi * x.hi (v_dot2c_f32_bf16; both products are exact in fp32)
__device__ __forceinline__ float dot2(bf16x2_t q, uint32_t xpair, float acc)
{
    return __builtin_amdgcn_fdot2_f32_bf16(q, __builtin_bit_cast(bf16x2_t, xpair), acc, false);
}

__device__ __forceinline__ float sbyte(uint32_t w, int j) { return (float)(int8_t)(w >> (8 * j)); }

// log2 of the factor by which chunk_dot<B> scales its sums (codes are
// converted from the top bits of a byte, i.e. multiplied by 2^(8-B)).
template <int B>
__host__ __device__ constexpr int chunk_dot_shift() { return B == 2 ? 6 : (B == 4 ? 4 : 0); }

// acc[m] += 2^shift * sum_j x[m][j] q[j] over one chunk of 32 codes.  xw[m][p]
// is the bf16 pair (x[2p], x[2p+1]); w the chunk's B raw words.  Codes are made
// exact bf16 pairs (|q| <= 256, or 2^(8-B) q for B = 2, 4) and multiplied with
// v_dot2c_f32_bf16.  Widths 2, 4 and 8 convert whole bytes (signed byte select)
// after one XOR flips every code's top bit (offset binary -> two's complement).
template <int B, int MT>
__device__ __forceinline__ void chunk_dot(const uint32_t (&w)[B], const uint32_t (&xw)[MT][16],
                                          float (&acc)[MT])
{
    static_assert(B <= 9, "bf16 holds the codes exactly only up to 9 bits");
    if constexpr (B == 8) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t v = w[i] ^ 0x80808080u;
            const bf16x2_t p0 = bf16_pair(sbyte(v, 0), sbyte(v, 1));
            const bf16x2_t p1 = bf16_pair(sbyte(v, 2), sbyte(v, 3));
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                acc[m] = dot2(p0, xw[m][2 * i], acc[m]);
                acc[m] = dot2(p1, xw[m][2 * i + 1], acc[m]);
            }
        }
    } else if constexpr (B == 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t v = w[i] ^ 0x88888888u;
            const uint32_t lo = (v << 4) & 0xf0f0f0f0u;  // codes 8i+2j, times 16
            const uint32_t hi = v & 0xf0f0f0f0u;         // codes 8i+2j+1, times 16
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bf16x2_t p = bf16_pair(sbyte(lo, j), sbyte(hi, j));
#pragma unroll
                for (int m = 0; m < MT; ++m) acc[m] = dot2(p, xw[m][4 * i + j], acc[m]);
            }
        }
    } else if constexpr (B == 2) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint32_t v = w[i] ^ 0xaaaaaaaau;
            const uint32_t t0 = (v << 6) & 0xc0c0c0c0u;  // code 16i+4j+0 at the top of byte j
            const uint32_t t1 = (v << 4) & 0xc0c0c0c0u;
            const uint32_t t2 = (v << 2) & 0xc0c0c0c0u;
            const uint32_t t3 = v & 0xc0c0c0c0u;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bf16x2_t p0 = bf16_pair(sbyte(t0, j), sbyte(t1, j));
                const bf16x2_t p1 = bf16_pair(sbyte(t2, j), sbyte(t3, j));
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    acc[m] = dot2(p0, xw[m][8 * i + 2 * j], acc[m]);
                    acc[m] = dot2(p1, xw[m][8 * i + 2 * j + 1], acc[m]);
                }
            }
        }
    } else {
        uint32_t v[B];
#pragma unroll
        for (int i = 0; i < B; ++i) v[i] = w[i] ^ code_msb_mask<B>(i);
#pragma unroll
        for (int p = 0; p < 16; ++p) {
            const bf16x2_t q = bf16_pair((float)chunk_code_signed<B>(v, 2 * p),
                                         (float)chunk_code_signed<B>(v, 2 * p + 1));
#pragma unroll
            for (int m = 0; m < MT; ++m) acc[m] = dot2(q, xw[m][p], acc[m]);
        }
    }
}

// Same contract for 10 <= B <= 15 (codes too wide for bf16): fp32 FMAs on x
// widened exactly from its bf16 pairs.
template <int B, int MT>
__device__ __forceinline__ void chunk_fma(const uint32_t (&w)[B], const uint32_t (&xw)[MT][16],
                                          float (&acc)[MT])
{
    uint32_t v[B];
#pragma unroll
    for (int i = 0; i < B; ++i) v[i] = w[i] ^ code_msb_mask<B>(i);
#pragma unroll
    for (int p = 0; p < 16; ++p) {
        const float q0 = (float)chunk_code_signed<B>(v, 2 * p);
        const float q1 = (float)chunk_code_signed<B>(v, 2 * p + 1);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            acc[m] = fmaf(__uint_as_float(xw[m][p] << 16), q0, acc[m]);
            acc[m] = fmaf(__uint_as_float(xw[m][p] & 0xffff0000u), q1, acc[m]);
        }
    }
}

// Asymmetric codes (q = u - z, |q| <= 2^B - 1), same contract as chunk_dot
// (no pre-shift): B <= 8 as exact bf16 pairs through v_dot2c_f32_bf16; B >= 9
// as fp32 FMAs on x widened exactly (x has 8 significant bits and q at most
// 15, so every product is exact in fp32).  Codes are extracted unsigned and
// the zero point subtracted in fp32 (both are integers below 2^15: exact).
template <int B, int MT>
__device__ __forceinline__ void chunk_dot_asym(const uint32_t (&w)[B], int32_t z,
                                               const uint32_t (&xw)[MT][16], float (&acc)[MT])
{
    const float zf = (float)z;
#pragma unroll
    for (int p = 0; p < 16; ++p) {
        const float q0 = (float)chunk_code_unsigned<B>(w, 2 * p) - zf;
        const float q1 = (float)chunk_code_unsigned<B>(w, 2 * p + 1) - zf;
        if constexpr (B <= 8) {
            const bf16x2_t q = bf16_pair(q0, q1);
#pragma unroll
            for (int m = 0; m < MT; ++m) acc[m] = dot2(q, xw[m][p], acc[m]);
        } else {
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                acc[m] = fmaf(__uint_as_float(xw[m][p] << 16), q0, acc[m]);
                acc[m] = fmaf(__uint_as_float(xw[m][p] & 0xffff0000u), q1, acc[m]);
            }
        }
    }
}

// acc[m] += (scaled) sum over one chunk of x[m][j] * q[j] for either scheme; z
// is the row's zero point (ignored when symmetric).  product_unscale undoes
// the pre-shift of the symmetric byte paths.
template <int B, int MT, bool kAsym>
__device__ __forceinline__ void chunk_product(const uint32_t (&w)[B], int32_t z,
                                              const uint32_t (&xw)[MT][16], float (&acc)[MT])
{
    if constexpr (kAsym)
        chunk_dot_asym<B, MT>(w, z, xw, acc);
    else if constexpr (B <= 9)
        chunk_dot<B, MT>(w, xw, acc);
    else
        chunk_fma<B, MT>(w, xw, acc);
}

template <int B, bool kAsym>
__host__ __device__ constexpr float product_unscale()
{
    return (kAsym || B > 9) ? 1.0f : 1.0f / (float)(1 << chunk_dot_shift<B>());
}


// M <= 2, K a multiple of 32 and x small enough to sit in LDS whole
// (MT * K / 32 chunk slots of 80 B): x is staged once per workgroup (kR
// 16-byte pieces per thread, a fixed count; threads past the last piece
// repeat it, or load nothing with kXExact), so the slice loop has no barriers, and each wave keeps the codes
// of up to three slices in flight (register stages by slice % 3, unrolled by
// three).  Loads: x first, then the codes of slices 0 and 1, then x to LDS
// (waiting only for x), then the slice loop.
constexpr int kXResMax = 48 * 1024;

//
// The body below serves the one-matrix kernel (gemv_xres_kernel) and the
// batched one (gemv_batch.hip): bid is the workgroup's index within this
// matrix's grid and xs_dyn the workgroup's LDS for x.  kXExact: threads past
// the last x piece load nothing (an offset outside the buffer) and store
// nothing, instead of repeating the last piece -- for launches whose kR is
// sized for the largest x of several matrices.
template <int B, int MT, int kWaves, int kR, class ZP, int kRW, bool kXExact = false>
__device__ __forceinline__ void gemv_xres_body(
    const uint16_t* __restrict__ x, int M, const uint32_t* __restrict__ packed,
    const float* __restrict__ scales, int64_t N, int64_t K, int64_t row_words,
    float* __restrict__ y, ZP zp, int64_t bid, uint16_t* __restrict__ xs_dyn)
{
    constexpr int kThreads = kWaves * kWave;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    // kRW rows per wave (1 or 2): their chunks form one stream of kRW * nchunks
    // chunks, so a row whose chunk count fills its last 64-chunk slice poorly
    // shares that slice with the next row
    static_assert(kRW == 1 || (kRW == 2 && !is_group_scales<ZP>::value && !ZP::kAsym),
                  "two rows: symmetric per-row scales");
    const int64_t n = (bid * kWaves + wave) * kRW;
    const int64_t nchunks = K / kChunk;
    const int64_t tchunks = kRW * nchunks;
    const int64_t nslices = ceil_div(tchunks, kSlice);
    const int64_t wrows = n < N ? (N - n < kRW ? N - n : kRW) : 1;
    const BufRef wbuf = uniform_buf(packed + (n < N ? n : N - 1) * row_words,
                                    (uint32_t)(wrows * row_words * 4));
    const BufRef xall = uniform_buf(x, (uint32_t)((int64_t)M * K * 2));
    const int32_t z = zp.zero(n < N ? n : N - 1);  // the row's zero point (asymmetric codes)

    // x piece p (8 elements) = piece p % 4 of chunk slot p / 4 (slot = m * nchunks + chunk)
    const int pieces = (int)(MT * nchunks * 4);
    uint4 xv[kR];
    int xdst[kR];
#pragma unroll
    for (int r = 0; r < kR; ++r) {
        const int p = kXExact ? tid + r * kThreads : min(tid + r * kThreads, pieces - 1);
        const int slot = p >> 2;
        xdst[r] = slot * kXPitch + (p & 3) * 8;
        // slot m * nchunks + c holds x[m][32 c ..]: its elements start at element
        // 32 * slot of the M x K row-major x (rows m >= M lie past the buffer: zeros)
        const uint32_t off = (uint32_t)(slot * kChunk * 2 + (p & 3) * 16);
        const u32x4v_t d = buf_load_b128(xall, kXExact && p >= pieces ? kOutsideOffset : off, 0u);
        xv[r] = make_uint4(d.x, d.y, d.z, d.w);
    }
    uint32_t w[3][B];
    // group-wise scales: each chunk's scale, loaded (a fixed count) with its codes
    constexpr bool kGroup = is_group_scales<ZP>::value;
    uint32_t gsc[3];
    [[maybe_unused]] BufRef sbuf{};
    [[maybe_unused]] int gshift = 0;  // log2 of the chunks per group
    if constexpr (kGroup) {
        sbuf = uniform_buf(zp.scales + (n < N ? n : N - 1) * zp.G, (uint32_t)(zp.G * 4));
        gshift = __builtin_ctzll((unsigned long long)(zp.group / kChunk));
    }
    auto load_w = [&](auto S, int64_t sl) {  // past the last slice: zeros
        const int64_t gc = sl * kSlice + lane;
        const int64_t r = (kRW == 2 && gc >= nchunks) ? 1 : 0;
        buf_load_words<B>(wbuf, (uint32_t)((r * row_words + (gc - r * nchunks) * B) * 4), 0u,
                          w[decltype(S)::value]);
        if constexpr (kGroup) {
            uint32_t t[1];
            buf_load_words<1>(sbuf, (uint32_t)(((sl * kSlice + lane) >> gshift) * 4), 0u, t);
            gsc[decltype(S)::value] = t[0];
        }
    };
    load_w(std::integral_constant<int, 0>{}, 0);
    load_w(std::integral_constant<int, 1>{}, 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int r = 0; r < kR; ++r)
        if (!kXExact || tid + r * kThreads < pieces) *reinterpret_cast<uint4*>(xs_dyn + xdst[r]) = xv[r];
    __syncthreads();

    float acc[MT], acc2[kRW == 2 ? MT : 1];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = 0.0f;
    if constexpr (kRW == 2) {
#pragma unroll
        for (int m = 0; m < MT; ++m) acc2[m] = 0.0f;
    }
    auto step = [&](auto S, int64_t sl) {
        constexpr int st = decltype(S)::value;
        load_w(std::integral_constant<int, (st + 2) % 3>{}, sl + 2);
        const int64_t gc = sl * kSlice + lane;
        if (gc < tchunks) {
            const int64_t r = (kRW == 2 && gc >= nchunks) ? 1 : 0;
            const int64_t c = gc - r * nchunks;
            uint32_t xw[MT][16];
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const uint4* src = reinterpret_cast<const uint4*>(xs_dyn + (m * nchunks + c) * kXPitch);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint4 d = src[i];
                    xw[m][4 * i + 0] = d.x;
                    xw[m][4 * i + 1] = d.y;
                    xw[m][4 * i + 2] = d.z;
                    xw[m][4 * i + 3] = d.w;
                }
            }
            if constexpr (kGroup) {  // the chunk's sum, scaled by its group's scale
                float part[MT];
#pragma unroll
                for (int m = 0; m < MT; ++m) part[m] = 0.0f;
                chunk_product<B, MT, false>(w[st], 0, xw, part);
                const float sg = __uint_as_float(gsc[st]);
#pragma unroll
                for (int m = 0; m < MT; ++m) acc[m] = fmaf(part[m], sg, acc[m]);
            } else if constexpr (kRW == 2) {  // the chunk's sum goes to its row
                float part[MT];
#pragma unroll
                for (int m = 0; m < MT; ++m) part[m] = 0.0f;
                chunk_product<B, MT, false>(w[st], 0, xw, part);
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    acc[m] += r ? 0.0f : part[m];
                    acc2[kRW == 2 ? m : 0] += r ? part[m] : 0.0f;
                }
            } else {
                chunk_product<B, MT, ZP::kAsym>(w[st], z, xw, acc);
            }
        }
    };
    int64_t sl = 0;
    for (; sl + 3 <= nslices; sl += 3) {
        step(std::integral_constant<int, 0>{}, sl);
        step(std::integral_constant<int, 1>{}, sl + 1);
        step(std::integral_constant<int, 2>{}, sl + 2);
    }
    if (sl < nslices) step(std::integral_constant<int, 0>{}, sl);
    if (sl + 1 < nslices) step(std::integral_constant<int, 1>{}, sl + 1);

#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = wave_sum(acc[m]);
    if constexpr (kRW == 2) {
#pragma unroll
        for (int m = 0; m < MT; ++m) acc2[m] = wave_sum(acc2[m]);
    }
    if (lane == 0 && n < N) {
        constexpr float kUnscale = product_unscale<B, ZP::kAsym>();
        const float s = kGroup ? 1.0f : scales[n];
#pragma unroll
        for (int m = 0; m < MT; ++m)
            if (m < M) y[(int64_t)m * N + n] = s * (acc[m] * kUnscale);
        if constexpr (kRW == 2) {
            if (n + 1 < N) {
                const float s2 = scales[n + 1];
#pragma unroll
                for (int m = 0; m < MT; ++m)
                    if (m < M) y[(int64_t)m * N + n + 1] = s2 * (acc2[m] * kUnscale);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Streaming resident-x body (1 <= M <= 2, K a multiple of 32 with at least
// 64 chunks per row, x resident in LDS): the workgroup owns rows
// [row0, row0 + kWaves * rpw) of the matrix, dealt to its waves in turn (wave
// w takes rows row0 + w, row0 + w + kWaves, ...), so at any time the
// workgroup reads one contiguous block of rows.  A wave reads its rows' codes
// as one stream of chunks
// (lane l takes chunk l, l + 64, ... of the stream; the row changes inside a
// slice when a row's chunk count is not a multiple of 64) with the loads of
// two slices in flight ahead of the one being computed, across row
// boundaries, so the vector work of one row overlaps the transfer of the
// next.  Each chunk's dot product joins the accumulator of its row's parity
// (a slice holds at most two rows, as a row has at least 64 chunks); when a
// slice completes a row, the wave reduces that row's accumulator, stores it
// and clears it.  The arithmetic per chunk is that of the resident-x body.
// The workgroup's rows must span less than 2^31 bytes of packed words.
template <int B, int MT, int kWaves, int kR>
__device__ __forceinline__ void gemv_stream_body(
    const uint16_t* __restrict__ x, int M, const uint32_t* __restrict__ packed,
    const float* __restrict__ scales, int64_t N, int64_t K, int64_t row_words,
    float* __restrict__ y, int64_t row0, int64_t rpw, uint16_t* __restrict__ xs_dyn)
{
    constexpr int kThreads = kWaves * kWave;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int32_t nchunks = (int32_t)(K / kChunk);
    const int64_t wrow0 = row0 + wave;  // the wave's first row; then every kWaves-th
    const int64_t wend = row0 + kWaves * rpw < N ? row0 + kWaves * rpw : N;
    const int32_t wrows = (int32_t)(wrow0 < wend ? (wend - wrow0 + kWaves - 1) / kWaves : 0);
    // the wave's stream: wrows * nchunks chunks, within the workgroup's rows
    // (below 2^31 bytes, so 32-bit counters and byte offsets hold it)
    const int32_t nslices = (int32_t)ceil_div((int64_t)wrows * nchunks, kSlice);
    const uint32_t row_bytes = (uint32_t)(row_words * 4);
    const BufRef wbuf =
        uniform_buf(packed + (wrows > 0 ? wrow0 : 0) * row_words,
                    wrows > 0 ? (uint32_t)((wrows - 1) * kWaves + 1) * row_bytes : 0u);
    const BufRef xall = uniform_buf(x, (uint32_t)((int64_t)M * K * 2));

    // x staged once per workgroup, as in gemv_xres_body (exact piece count)
    const int pieces = (int)(MT * nchunks * 4);
    uint4 xv[kR];
#pragma unroll
    for (int r = 0; r < kR; ++r) {
        const int p = tid + r * kThreads;
        const uint32_t off = (uint32_t)((p >> 2) * kChunk * 2 + (p & 3) * 16);
        const u32x4v_t d = buf_load_b128(xall, p < pieces ? off : kOutsideOffset, 0u);
        xv[r] = make_uint4(d.x, d.y, d.z, d.w);
    }

    // load position: lane's (row, chunk) in the stream and its byte offset,
    // advanced one slice per load (a row has at least 64 chunks, so at most
    // one row boundary is crossed; the row's padding bytes and the other
    // waves' rows are skipped then)
    const uint32_t pad = row_bytes - (uint32_t)(nchunks * B * 4) + (kWaves - 1) * row_bytes;
    int32_t lr = 0, lc = lane;
    uint32_t loff = (uint32_t)(lane * B * 4);
    uint32_t w[3][B];
    int32_t rowof[3], colof[3];
    auto load_w = [&](auto S) {
        constexpr int st = decltype(S)::value;
        buf_load_words<B>(wbuf, lr < wrows ? loff : kOutsideOffset, 0u, w[st]);
        rowof[st] = lr;
        colof[st] = lc;
        lc += kSlice;
        loff += kSlice * B * 4;
        if (lc >= nchunks) {
            lc -= nchunks;
            ++lr;
            loff += pad;
        }
    };
    load_w(std::integral_constant<int, 0>{});
    load_w(std::integral_constant<int, 1>{});
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int r = 0; r < kR; ++r) {
        const int p = tid + r * kThreads;
        if (p < pieces)
            *reinterpret_cast<uint4*>(xs_dyn + (p >> 2) * kXPitch + (p & 3) * 8) = xv[r];
    }
    __syncthreads();

    constexpr float kUnscale = product_unscale<B, false>();
    float acc[2][MT];  // by row parity
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[q][m] = 0.0f;
    int32_t next_row = 0;        // the next row to complete (wave-uniform)
    int32_t next_end = nchunks;  // its end in the stream, in chunks
    auto step = [&](auto S, int32_t sl) {
        constexpr int st = decltype(S)::value;
        load_w(std::integral_constant<int, (st + 2) % 3>{});
        if (rowof[st] < wrows) {
            uint32_t xw[MT][16];
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const uint4* src =
                    reinterpret_cast<const uint4*>(xs_dyn + (m * nchunks + colof[st]) * kXPitch);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint4 d = src[i];
                    xw[m][4 * i + 0] = d.x;
                    xw[m][4 * i + 1] = d.y;
                    xw[m][4 * i + 2] = d.z;
                    xw[m][4 * i + 3] = d.w;
                }
            }
            float part[MT];
#pragma unroll
            for (int m = 0; m < MT; ++m) part[m] = 0.0f;
            chunk_product<B, MT, false>(w[st], 0, xw, part);
            const bool odd = rowof[st] & 1;
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                acc[0][m] += odd ? 0.0f : part[m];
                acc[1][m] += odd ? part[m] : 0.0f;
            }
        }
        // a row whose last chunk lies in this slice is complete
        if (next_row < wrows && next_end <= (sl + 1) * kSlice) {
            const bool par = next_row & 1;
            float v[MT];
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                v[m] = wave_sum(par ? acc[1][m] : acc[0][m]);
                acc[0][m] = par ? acc[0][m] : 0.0f;
                acc[1][m] = par ? 0.0f : acc[1][m];
            }
            // the scale at a wave-uniform address in uniform control flow: a
            // scalar load, which leaves the vector loads in flight alone (a
            // vector load here would be followed by a wait for all of them)
            const int64_t n = wrow0 + (int64_t)next_row * kWaves;
            const float s = scales[n];
            if (lane == 0) {
#pragma unroll
                for (int m = 0; m < MT; ++m)
                    if (m < M) y[(int64_t)m * N + n] = s * (v[m] * kUnscale);
            }
            ++next_row;
            next_end += nchunks;
        }
    };
    int32_t sl = 0;
    for (; sl + 3 <= nslices; sl += 3) {
        step(std::integral_constant<int, 0>{}, sl);
        step(std::integral_constant<int, 1>{}, sl + 1);
        step(std::integral_constant<int, 2>{}, sl + 2);
    }
    if (sl < nslices) step(std::integral_constant<int, 0>{}, sl);
    if (sl + 1 < nslices) step(std::integral_constant<int, 1>{}, sl + 1);
}

// Streaming GEMV, row-sliced: the workgroup's rows row0 .. row0 + kWaves * rpw
// are dealt to its waves in turn (wave w takes rows row0 + w, row0 + w +
// kWaves, ...), so at any time the workgroup reads one contiguous block of
// kWaves rows.  A wave works on kRPS of its rows at a time, each on 64 / kRPS
// of its lanes (kRPS = 1: the whole wave on one row; kRPS = 2: lanes 0 .. 31
// on one row and 32 .. 63 on the next), and cuts them into slices of 64 /
// kRPS chunks per row that never span two rows.  The row's chunk count must
// be a multiple of 64 / kRPS (K a multiple of 2048 for kRPS = 1, of 1024 for
// kRPS = 2), so every lane has a chunk in every slice.
// Everything that locates a slice -- its rows, its place in them, its byte
// offset -- is wave-uniform (each lane adds a constant), so the per-chunk work
// is the load, the x reads and the dot products; each lane's chunk adds into
// one running total, reduced across the row's lanes when the row's last slice
// is done.  Loads run two slices ahead of the arithmetic, across row
// boundaries.  The policy ZP: NoZeroPoints (the row scale times the reduced
// sum), ZeroPoints (each code's row zero point, loaded with the slice's codes,
// is taken off before it meets x) or GroupScales (each chunk's sum times its
// group's scale, loaded with the codes; no row scale).
template <int B, int MT, int kWaves, int kR, int kRPS = 1, class ZP = NoZeroPoints, int kStages = 3>
__device__ __forceinline__ void gemv_rowslice_body(
    const uint16_t* __restrict__ x, int M, const uint32_t* __restrict__ packed,
    const float* __restrict__ scales, int64_t N, int64_t K, int64_t row_words,
    float* __restrict__ y, int64_t row0, int64_t rpw, uint16_t* __restrict__ xs_dyn,
    ZP zp = ZP{})
{
    constexpr bool kAsym = ZP::kAsym;
    constexpr bool kGroup = is_group_scales<ZP>::value;
    constexpr int kThreads = kWaves * kWave;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    static_assert(kRPS == 1 || kRPS == 2, "one or two rows per slice");
    constexpr int kRowLanes = kWave / kRPS;  // lanes (and chunks per slice) of one row
    const int half = lane / kRowLanes;       // which of the slice's rows this lane serves
    const int rlane = lane % kRowLanes;
    const int32_t nchunks = (int32_t)(K / kChunk);
    const int32_t spr = (int32_t)ceil_div((int64_t)nchunks, kRowLanes);  // slices per row
    const int64_t wrow0 = row0 + wave;  // the wave's first row; then every kWaves-th
    const int64_t wend = row0 + kWaves * rpw < N ? row0 + kWaves * rpw : N;
    const int32_t wrows = (int32_t)(wrow0 < wend ? (wend - wrow0 + kWaves - 1) / kWaves : 0);
    const int32_t ngroups = (wrows + kRPS - 1) / kRPS;  // groups of kRPS rows
    // the workgroup's rows span below 2^31 bytes, so 32-bit offsets hold them
    const int32_t nslices = ngroups * spr;
    const uint32_t row_bytes = (uint32_t)(row_words * 4);
    const BufRef wbuf =
        uniform_buf(packed + (wrows > 0 ? wrow0 : 0) * row_words,
                    wrows > 0 ? (uint32_t)((wrows - 1) * kWaves + 1) * row_bytes : 0u);
    const BufRef xall = uniform_buf(x, (uint32_t)((int64_t)M * K * 2));

    // x staged once per workgroup, as in gemv_xres_body (exact piece count)
    const int pieces = (int)(MT * nchunks * 4);
    uint4 xv[kR];
#pragma unroll
    for (int r = 0; r < kR; ++r) {
        const int p = tid + r * kThreads;
        const uint32_t off = (uint32_t)((p >> 2) * kChunk * 2 + (p & 3) * 16);
        const u32x4v_t d = buf_load_b128(xall, p < pieces ? off : kOutsideOffset, 0u);
        xv[r] = make_uint4(d.x, d.y, d.z, d.w);
    }

    // load position, wave-uniform: slices issued, the next slice's row group
    // and place in its rows, and the byte offset of its first chunk (each lane
    // adds its row's and its chunk's constant offset)
    const uint32_t lane_off = (uint32_t)(half * kWaves) * row_bytes + (uint32_t)(rlane * B * 4);
    int32_t ld_n = 0, ld_sir = 0, ld_grp = 0;
    uint32_t ld_row = 0, ld_off = 0;
    uint32_t w[kStages][B];
    int32_t sir_of[kStages];
    // per lane, the zero point of its row (ZeroPoints) or the scale of its
    // chunk's group (GroupScales), loaded with the slice's codes
    [[maybe_unused]] uint32_t pol[kStages];
    [[maybe_unused]] int gshift = 0;  // log2 of the chunks per group
    if constexpr (kGroup) gshift = __builtin_ctzll((unsigned long long)(zp.group / kChunk));
    auto load_w = [&](auto S) {
        constexpr int st = decltype(S)::value;
        const bool live = ld_n < nslices && ld_grp * kRPS + half < wrows;
        buf_load_words<B>(wbuf, live ? ld_off + lane_off : kOutsideOffset, 0u, w[st]);
        if constexpr (kAsym || kGroup) {
            // the lane's row (one of the wave's; a row of the matrix when not live)
            const int32_t r = live ? ld_grp * kRPS + half : 0;
            const int64_t nr = wrow0 + (int64_t)r * kWaves;
            const int64_t n = nr < N ? nr : N - 1;
            if constexpr (kAsym) {
                pol[st] = (uint32_t)zp.zero(n);
            } else {
                const int32_t c = ld_sir * kRowLanes + rlane;  // the lane's chunk in the row
                pol[st] = __float_as_uint(zp.scales[n * zp.G + (c >> gshift)]);
            }
        }
        sir_of[st] = ld_sir;
        ++ld_n;
        if (++ld_sir == spr) {
            ld_sir = 0;
            ++ld_grp;
            ld_row += kRPS * kWaves * row_bytes;
            ld_off = ld_row;
        } else {
            ld_off += kRowLanes * B * 4;
        }
    };
    static_for<kStages - 1>([&](auto S) { load_w(S); });
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int r = 0; r < kR; ++r) {
        const int p = tid + r * kThreads;
        if (p < pieces)
            *reinterpret_cast<uint4*>(xs_dyn + (p >> 2) * kXPitch + (p & 3) * 8) = xv[r];
    }
    __syncthreads();

    constexpr float kUnscale = product_unscale<B, kAsym>();
    float acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = 0.0f;
    int32_t grp = 0;  // the row group of the slice being multiplied
    const uint16_t* xlane = xs_dyn + rlane * kXPitch;
    auto step = [&](auto S) {
        constexpr int st = decltype(S)::value;
        load_w(std::integral_constant<int, (st + kStages - 1) % kStages>{});
        const int32_t sir = sir_of[st];
        {
            uint32_t xw[MT][16];
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const uint4* src =
                    reinterpret_cast<const uint4*>(xlane + (m * nchunks + sir * kRowLanes) * kXPitch);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint4 d = src[i];
                    xw[m][4 * i + 0] = d.x;
                    xw[m][4 * i + 1] = d.y;
                    xw[m][4 * i + 2] = d.z;
                    xw[m][4 * i + 3] = d.w;
                }
            }
            if constexpr (kGroup) {  // the chunk's sum, scaled by its group's scale
                float part[MT];
#pragma unroll
                for (int m = 0; m < MT; ++m) part[m] = 0.0f;
                chunk_product<B, MT, false>(w[st], 0, xw, part);
                const float sg = __uint_as_float(pol[st]);
#pragma unroll
                for (int m = 0; m < MT; ++m) acc[m] = fmaf(part[m], sg, acc[m]);
            } else if constexpr (kAsym) {
                chunk_product<B, MT, true>(w[st], (int32_t)pol[st], xw, acc);
            } else {
                chunk_product<B, MT, false>(w[st], 0, xw, acc);
            }
        }
        if (sir == spr - 1) {  // the rows' last slice: reduce, scale, store
            float v[kRPS][MT];
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                if constexpr (kRPS == 1)
                    v[0][m] = wave_sum(acc[m]);
                else
                    half_sums(acc[m], v[0][m], v[kRPS - 1][m]);
                acc[m] = 0.0f;
            }
            // the scales at wave-uniform addresses in uniform control flow:
            // scalar loads, which leave the vector loads in flight alone
#pragma unroll
            for (int h = 0; h < kRPS; ++h) {
                const int32_t r = grp * kRPS + h;
                if (r < wrows) {
                    const int64_t n = wrow0 + (int64_t)r * kWaves;
                    const float s = kGroup ? 1.0f : scales[n];
                    if (lane == 0) {
#pragma unroll
                        for (int m = 0; m < MT; ++m)
                            if (m < M) y[(int64_t)m * N + n] = s * (v[h][m] * kUnscale);
                    }
                }
            }
            ++grp;
        }
    };
    int32_t sl = 0;
    for (; sl + kStages <= nslices; sl += kStages) static_for<kStages>([&](auto S) { step(S); });
    static_for<kStages - 1>([&](auto S) {
        if (sl + decltype(S)::value < nslices) step(S);
    });
}

// ---------------------------------------------------------------------------
// Matrix-core body, 3 <= M <= 16 and K a multiple of 32 (one workgroup of
// kGemvMfmaWaves waves per tile of 16 kNT rows, the waves taking the K steps
// in turn and adding their sums in LDS at the end).  The codes are expanded
// to exact bf16 operands of v_mfma_f32_16x16x32_bf16, so the vector work per
// code does not grow with M.  Loaded straight into registers in the MFMA lane
// layout, each load instruction would spread its lanes over 16 rows (lane
// 16 g + c: row c, chunk g) and x would cost as much as the code stream (each
// lane needs 64 bytes of one row, so a 16-byte load touches 64 cache lines,
// and lanes of rows past M load too).  Instead each wave copies the codes and x of its own steps
// straight into a ring of LDS stages of its own (buffer_load ... lds): the
// codes row by row (a step is 4 chunks = 16 B bytes of each of the 16 kNT
// rows, so row r fills slots r B .. r B + B - 1), x for rows below kMR only
// (4 rows of 256 bytes per instruction).  Lanes then read their chunk's B
// words and the A operands (ds_read_b128) back.  x piece p of row i sits at
// slot 16 i + (p ^ i), so the 16 lanes of a read that take the same piece of
// 16 rows hit distinct banks.  The ring is private to the wave, so the loop
// has no barriers; an explicit vmcnt wait before each step covers the LDS
// copies, which the compiler does not track.  x pieces past K (the last step
// of a K not a multiple of 128) and rows past M read an offset outside the x
// buffer, which loads zeros; codes past a row's end meet those zeros, and
// rows past N read zeros.
template <int B, int kNT, int kDepth, int kMR, bool kAsym>
struct MfmaXldsLayout {
    static constexpr int kStages = kDepth + 1;
    static constexpr int kSlots = kMR * 16;  // 16-byte x pieces of one step
    static constexpr int kCodeSlots = (16 * kNT * B + 63) / 64 * 64;  // 16-byte code pieces of one step
    // byte offsets: x ring (stage, wave, slot), code ring (stage, wave, slot),
    // the waves' sums (wave - 1, row tile, register, lane)
    static constexpr size_t kXBytes = (size_t)kStages * kGemvMfmaWaves * kSlots * 16;
    static constexpr size_t kCodeBytes = (size_t)kStages * kGemvMfmaWaves * kCodeSlots * 16;
    static constexpr size_t kRedBytes = (size_t)(kGemvMfmaWaves - 1) * kNT * 4 * kWave * 4;
    static constexpr size_t kBytes = kXBytes + kCodeBytes + kRedBytes;
};

// LDS bytes of one workgroup of gemv_mfma_xlds_body
template <int B, int kNT, int kDepth, int kMR, bool kAsym>
__host__ __device__ constexpr size_t mfma_xlds_lds_bytes()
{
    return MfmaXldsLayout<B, kNT, kDepth, kMR, kAsym>::kBytes;
}

// Tile `tile` (rows 16 kNT tile ..) of y = s * (x q^T); lds holds
// mfma_xlds_lds_bytes() bytes, 16-byte aligned.
template <int B, int kNT, int kDepth, int kMR, class ZP>
__device__ __forceinline__ void gemv_mfma_xlds_body(
    const uint16_t* __restrict__ x, int M, const uint32_t* __restrict__ packed,
    const float* __restrict__ scales, int64_t N, int64_t K, int64_t row_words,
    float* __restrict__ y, ZP zp, int64_t tile, unsigned char* __restrict__ lds)
{
    using L = MfmaXldsLayout<B, kNT, kDepth, kMR, ZP::kAsym>;
    typedef __bf16 bf16x8m_t __attribute__((ext_vector_type(8)));
    typedef float f32x4m_t __attribute__((ext_vector_type(4)));
    constexpr bool kSplit = split_codes<B, ZP::kAsym>();
    constexpr int kStages = L::kStages;
    constexpr int kXCopies = kMR / 4;
    constexpr int kCodeSlots = L::kCodeSlots;
    constexpr int kCodeCopies = kCodeSlots / 64;
    // group-wise scales (groups of whole 128-code steps): each step's scales of
    // this lane's rows come into registers with the step's codes (kNT more
    // loads).  Not through the LDS ring: the fold that reads them is plain
    // arithmetic the compiler may sink past the next step's copies, and a copy
    // into a slot whose read is still in flight would race with it.
    constexpr bool kGroup = is_group_scales<ZP>::value;
    constexpr int kPerStage = kCodeCopies + kXCopies + (kGroup ? kNT : 0);
    constexpr int kSlots = L::kSlots;
    static_assert(kDepth >= 1 && kDepth <= 2, "one or two steps ahead");
    static_assert(kMR == 8 || kMR == 16, "x rows staged: 8 or 16");
    static_assert(kDepth * kPerStage < 64, "vmcnt holds at most 63");
    uint4* const xs = reinterpret_cast<uint4*>(lds);
    uint4* const cs = reinterpret_cast<uint4*>(lds + L::kXBytes);
    float* const red = reinterpret_cast<float*>(lds + L::kXBytes + L::kCodeBytes);

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int c = lane & 15;
    const int g = lane >> 4;
    auto cring = [&](auto S) -> uint4* {
        return cs + (decltype(S)::value * kGemvMfmaWaves + wave) * kCodeSlots;
    };
    auto ring = [&](auto S) -> uint4* { return xs + (decltype(S)::value * kGemvMfmaWaves + wave) * kSlots; };
    auto red_at = [&](int w, int j, int r) -> float* { return red + ((w * kNT + j) * 4 + r) * kWave; };

    const int64_t n0 = tile * 16 * kNT;
    const int64_t nchunks = K / kChunk;
    const int64_t nsteps = ceil_div(nchunks, 4);
    const int64_t nrows = N - n0 < 16 * kNT ? N - n0 : 16 * kNT;
    const BufRef wb = uniform_buf(packed + n0 * row_words, (uint32_t)(nrows * row_words * 4));
    const BufRef xb = uniform_buf(x, (uint32_t)((int64_t)M * K * 2));
    constexpr uint32_t kOutside = 0xfffff000u;

    // copy instruction q: lane l fills slot 64 q + l = row r, position l % 16,
    // which holds piece p = (l % 16) ^ r of that row (chunk 4 ks + p / 4)
    uint32_t xbase[kXCopies];
    int xchunk[kXCopies];
#pragma unroll
    for (int q = 0; q < kXCopies; ++q) {
        const int r = 4 * q + (lane >> 4);
        const int pc = (lane & 15) ^ r;
        xbase[q] = r < M ? (uint32_t)(r * K * 2 + 16 * pc) : kOutside;
        xchunk[q] = pc >> 2;
    }
    // A operand of substep t: row c (rows past kMR repeat rows below it; their
    // sums land in output rows that are never stored), piece 4 g + t
    const int ar = c & (kMR - 1);
    int aslot[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) aslot[t] = 16 * ar + ((4 * g + t) ^ ar);

    // codes: copy q fills slot s = 64 q + l with piece s % B of row s / B of
    // the step (16-byte pieces; slots past the tile's rows get zeros)
    uint32_t cbase[kCodeCopies];
#pragma unroll
    for (int q = 0; q < kCodeCopies; ++q) {
        const int sl = 64 * q + lane;
        const int r = sl / B, pc = sl % B;
        cbase[q] = r < 16 * kNT ? (uint32_t)(r * row_words * 4 + pc * 16) : kOutside;
    }
    int32_t zr[kNT];  // zero point of this lane's row in each row tile
#pragma unroll
    for (int j = 0; j < kNT; ++j) zr[j] = zp.zero(n0 + 16 * j + c < N ? n0 + 16 * j + c : N - 1);
    [[maybe_unused]] BufRef sb{};
    [[maybe_unused]] int gshift = 0;  // log2 of the 128-code steps per group
    if constexpr (kGroup) {
        sb = uniform_buf(zp.scales + n0 * zp.G, (uint32_t)(nrows * zp.G * 4));
        gshift = __builtin_ctzll((unsigned long long)(zp.group / 128));
    }
    float gsc[kGroup ? kStages : 1][kGroup ? kNT : 1];  // group scales by stage
    auto load = [&](auto P, int64_t ks) {
        if constexpr (kGroup) {  // the scale of row 16 j + c for step ks's group
            const int64_t gi = ks >> gshift;
#pragma unroll
            for (int j = 0; j < kNT; ++j) {
                const bool in = 16 * j + c < nrows && gi < zp.G;
                uint32_t t[1];
                buf_load_words<1>(sb, in ? (uint32_t)(((16 * j + c) * zp.G + gi) * 4) : kOutside, 0u, t);
                gsc[kGroup ? decltype(P)::value : 0][kGroup ? j : 0] = __uint_as_float(t[0]);
            }
        }
        uint4* cdst = cring(P);
#pragma unroll
        for (int q = 0; q < kCodeCopies; ++q)
            buf_load_lds16(wb, cdst + 64 * q, cbase[q] != kOutside ? cbase[q] + (uint32_t)(ks * 16 * B) : kOutside, 0u);
        uint4* dst = ring(P);
#pragma unroll
        for (int q = 0; q < kXCopies; ++q) {
            const bool in = xbase[q] != kOutside && 4 * ks + xchunk[q] < nchunks;
            buf_load_lds16(xb, dst + 64 * q, in ? xbase[q] + (uint32_t)(ks * 256) : kOutside, 0u);
        }
    };
    f32x4m_t acc[kNT];
#pragma unroll
    for (int j = 0; j < kNT; ++j) acc[j] = (f32x4m_t){0.0f, 0.0f, 0.0f, 0.0f};
    // vmcnt(n) with expcnt and lgkmcnt left at their maxima
    auto compute = [&](auto P, auto Wait) {
        constexpr int n = decltype(Wait)::value;
        __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
        const uint4* src = ring(P);
        // this lane's chunk (chunk g of the step) of row c of each row tile
        uint32_t wl[kNT][B];
        const uint32_t* cw = reinterpret_cast<const uint32_t*>(cring(P));
#pragma unroll
        for (int j = 0; j < kNT; ++j)
#pragma unroll
            for (int i = 0; i < B; ++i) wl[j][i] = cw[(16 * j + c) * 4 * B + g * B + i];
        f32x4m_t part[kNT];  // group-wise scales: this step's sums, scaled below
#pragma unroll
        for (int j = 0; j < kNT; ++j) part[j] = (f32x4m_t){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const bf16x8m_t a = __builtin_bit_cast(bf16x8m_t, src[aslot[t]]);
#pragma unroll
            for (int j = 0; j < kNT; ++j) {
                bf16x8_t bh, bl;
                expand8z<B, ZP::kAsym>(wl[j], zr[j], t, bh, bl);
                f32x4m_t& d = kGroup ? part[j] : acc[j];
                d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bh, d, 0, 0, 0);
                if constexpr (kSplit) d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bl, d, 0, 0, 0);
            }
        }
        if constexpr (kGroup) {
#pragma unroll
            for (int j = 0; j < kNT; ++j) {
                const float sg = gsc[kGroup ? decltype(P)::value : 0][kGroup ? j : 0];
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[j][r] = fmaf(sg, part[j][r], acc[j][r]);
            }
        }
    };

    // Stage i of the ring holds step ks + i kW; each step's loads are issued
    // before the computation of the step kDepth before it.
    constexpr int64_t kW = kGemvMfmaWaves;
    int64_t ks = wave;
    load(std::integral_constant<int, 0>{}, ks);
    if constexpr (kDepth > 1) load(std::integral_constant<int, 1>{}, ks + kW);
    if constexpr (kDepth > 2) load(std::integral_constant<int, 2>{}, ks + 2 * kW);
    __builtin_amdgcn_sched_barrier(0);
    auto stage = [&](auto I) {
        constexpr int i = decltype(I)::value;
        load(std::integral_constant<int, (i + kDepth) % kStages>{}, ks + (i + kDepth) * kW);
        __builtin_amdgcn_sched_barrier(0);
        compute(I, std::integral_constant<int, kDepth * kPerStage>{});
        __builtin_amdgcn_sched_barrier(0);
    };
    for (; ks + kDepth * kW < nsteps; ks += kStages * kW) {
        stage(std::integral_constant<int, 0>{});
        stage(std::integral_constant<int, 1>{});
        if constexpr (kStages > 2) stage(std::integral_constant<int, 2>{});
        if constexpr (kStages > 3) stage(std::integral_constant<int, 3>{});
    }
    // the last loads in flight are those of stages 0 .. kDepth-1, in order
    if (ks < nsteps) compute(std::integral_constant<int, 0>{}, std::integral_constant<int, (kDepth - 1) * kPerStage>{});
    if constexpr (kDepth > 1)
        if (ks + kW < nsteps) compute(std::integral_constant<int, 1>{}, std::integral_constant<int, (kDepth - 2) * kPerStage>{});
    if constexpr (kDepth > 2)
        if (ks + 2 * kW < nsteps) compute(std::integral_constant<int, 2>{}, std::integral_constant<int, 0>{});
    // copies past the last step may still be in flight: drain them before
    // the workgroup's LDS can be handed to another workgroup
    __builtin_amdgcn_s_waitcnt(0);

    if (wave > 0) {
#pragma unroll
        for (int j = 0; j < kNT; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) red_at(wave - 1, j, r)[lane] = acc[j][r];
    }
    __syncthreads();
    if (wave == 0) {
        constexpr float kUnscale = 1.0f / expand8_scale<B, ZP::kAsym>();
#pragma unroll
        for (int j = 0; j < kNT; ++j) {
            const int64_t n = n0 + 16 * j + c;
            if (n >= N) continue;
            const float s = kGroup ? 1.0f : scales[n];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float v = acc[j][r];
#pragma unroll
                for (int q = 0; q < kGemvMfmaWaves - 1; ++q) v += red_at(q, j, r)[lane];
                const int m = 4 * g + r;
                if (m < M) y[(int64_t)m * N + n] = s * (v * kUnscale);
            }
        }
    }
}

}  // namespace

}  // namespace dq
