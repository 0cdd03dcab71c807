// Decode-shaped dequantized product, 1 <= M <= 16:
//   y[m, n] = s[n] * sum_k x[m, k] * q[n, k]
// BPDQ article, section 3.2 (dequantize fused with the matrix product; fp32
// scales and output) and the DynaQuant page, "自定义内核架构" (packed codes are
// streamed from memory and expanded in registers).  At M = 1 the product is
// bound by the bytes of the packed weights (decode is memory-bound, as the
// Quantization tutorial's closing remark on prefill vs decode puts it).
//
// Kernels by M (the row scale always multiplies the reduced sum once):
//   * M <= 2 (gemv_xres_kernel when K is a multiple of 32 and x fits in LDS
//     whole, else gemv_lds_kernel): a wave owns a row (or two, when a row's
//     chunks fill their last slice poorly); lane l walks the chunks
//     l, l+64, ... of it (a chunk = 32 codes = B whole words, so a wave's
//     loads of one row cover 64*B contiguous words); x sits in LDS; codes
//     become signed integers with one XOR per word plus a signed bit-field
//     extract and meet x in bf16 pair dot products (fp32 FMAs for B >= 10);
//   * 3 <= M <= 16 (gemv_mfma_xlds_kernel when K is a multiple of 32, codes
//     and x copied through LDS; else gemv_mfma_kernel): codes expanded to
//     exact bf16 operands of v_mfma_f32_16x16x32_bf16, so the VALU cost per
//     code no longer grows with M.
// The product kernels take a policy type for the variants: NoZeroPoints (the
// scheme above), ZeroPoints (asymmetric codes: a zero-point term in the
// epilogue) and GroupScales (a scale per group of codes): the resident-x
// kernel applies it per chunk; gemv_mfma_xlds_kernel, for groups of whole
// 128-code steps, scales each step's MFMA sums before adding them in.
// gemv_group_kernel serves group-wise scales for the other shapes.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "gemm_tiles.hpp"

namespace dq {

namespace {

// ---------------------------------------------------------------------------
// M <= 2: x is staged per K-slice of 64 chunks (2048 codes) in LDS by the whole
// workgroup (coalesced 16-byte loads); each wave owns kRows rows and each lane
// one chunk of each of them per slice.  The next slice's packed words and x are
// loaded into registers before the current slice is computed, so every wave
// keeps two slices of loads in flight.
constexpr int kSlice = 64;            // chunks per slice (one per lane)
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

template <int B, int MT, int kRows, int kWaves, bool kAligned, class ZP>
__global__ __launch_bounds__(kWaves * kWave) void gemv_lds_kernel(
    const uint16_t* __restrict__ x, int M, const uint32_t* __restrict__ packed,
    const float* __restrict__ scales, int64_t N, int64_t K, int64_t row_words,
    float* __restrict__ y, ZP zp)
{
    constexpr int kThreads = kWaves * kWave;
    constexpr int kXPerThread = kSlice * kChunk / kThreads;  // x elements staged per thread
    static_assert(kXPerThread == 8 || kXPerThread == 4, "staging is 16 or 8 bytes per thread");
    __shared__ __attribute__((aligned(16))) uint16_t xs[2][MT][kSlice * kXPitch];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int64_t n0 = ((int64_t)blockIdx.x * kWaves + wave) * kRows;
    const int64_t nchunks = ceil_div(K, kChunk);
    const int64_t nslices = ceil_div(nchunks, kSlice);
    const bool xvec = (K & 7) == 0;

    // rows of this wave (clamped for loads; stores are guarded)
    const uint32_t* rowp_[kRows];
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
        const int64_t n = n0 + r < N ? n0 + r : N - 1;
        rowp_[r] = packed + n * row_words;
    }
    const uint32_t* const(&rowp)[kRows] = rowp_;

    // x staging: thread t moves kXPerThread elements of each x row per slice
    const int xc = tid * kXPerThread / kChunk;                 // chunk within the slice
    const int xp = (tid * kXPerThread) % kChunk;               // element offset within the chunk

    // K a multiple of 32: every chunk lies inside its row, so codes and x come
    // in with buffer loads of a fixed count (no per-lane branches, so the
    // compiler can wait for exactly the loads it needs); past the end of a
    // row (or for rows m >= M of x) the buffer bounds return zeros
    BufRef xbuf[MT], wbuf[kRows];
    if constexpr (kAligned) {
#pragma unroll
        for (int m = 0; m < MT; ++m)
            xbuf[m] = uniform_buf(x + (int64_t)(m < M ? m : 0) * K, m < M ? (uint32_t)(K * 2) : 0u);
#pragma unroll
        for (int r = 0; r < kRows; ++r) wbuf[r] = uniform_buf(rowp[r], (uint32_t)(row_words * 4));
    }
    auto load_x = [&](int64_t s, uint4 (&v)[MT]) {
        const int64_t k = (s * kSlice + xc) * kChunk + xp;
        if constexpr (kAligned) {
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                if constexpr (kXPerThread == 8) {
                    const u32x4v_t d = buf_load_b128(xbuf[m], (uint32_t)(k * 2), 0u);
                    v[m] = make_uint4(d.x, d.y, d.z, d.w);
                } else {
                    const u32x2v_t d = __builtin_amdgcn_raw_buffer_load_b64(
                        make_rsrc(xbuf[m].base, xbuf[m].bytes), (uint32_t)(k * 2), 0u, 0);
                    v[m] = make_uint4(d.x, d.y, 0u, 0u);
                }
            }
        } else {
            stage_x_load<MT, kXPerThread>(x, M, K, k, xvec, v);
        }
    };
    auto load_w = [&](int64_t s, uint32_t (&w)[kRows][B]) {
        const int64_t c = s * kSlice + lane;
        if constexpr (kAligned) {
#pragma unroll
            for (int r = 0; r < kRows; ++r) buf_load_words<B>(wbuf[r], (uint32_t)(c * B * 4), 0u, w[r]);
        } else {
            stage_w_load<B, kRows>(rowp, c, nchunks, row_words, w);
        }
    };

    float acc[kRows][MT];
#pragma unroll
    for (int r = 0; r < kRows; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[r][m] = 0.0f;

    // slice s: x from LDS buffer s & 1, codes from registers, accumulated into acc
    auto compute = [&](int buf, int64_t s, const uint32_t (&w)[kRows][B]) {
        if (s * kSlice + lane < nchunks) {
            uint32_t xw[MT][16];
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const uint4* src = reinterpret_cast<const uint4*>(&xs[buf][m][lane * kXPitch]);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint4 d = src[i];
                    xw[m][4 * i + 0] = d.x;
                    xw[m][4 * i + 1] = d.y;
                    xw[m][4 * i + 2] = d.z;
                    xw[m][4 * i + 3] = d.w;
                }
            }
#pragma unroll
            for (int r = 0; r < kRows; ++r) {
                if constexpr (B <= 9)
                    chunk_dot<B, MT>(w[r], xw, acc[r]);
                else
                    chunk_fma<B, MT>(w[r], xw, acc[r]);
            }
        }
    };
    uint4 xnxt[MT];
    if constexpr (kAligned) {
        // codes in two register sets by slice parity (unrolled by two, so each
        // set keeps its registers and the waits count exactly); the loads of
        // slice s+1 are issued unconditionally (past the last slice they read
        // zeros) so their number is fixed
        uint32_t w[2][kRows][B];
        load_x(0, xnxt);
        load_w(0, w[0]);
        __builtin_amdgcn_sched_barrier(0);  // both in flight before x goes to LDS
        stage_x_store<MT, kXPerThread>(&xs[0][0][xc * kXPitch + xp], xnxt);
        auto step = [&](auto P, int64_t s) {
            constexpr int p = decltype(P)::value;
            load_x(s + 1, xnxt);
            load_w(s + 1, w[p ^ 1]);
            __syncthreads();
            compute(p, s, w[p]);
            stage_x_store<MT, kXPerThread>(&xs[p ^ 1][0][xc * kXPitch + xp], xnxt);
        };
        int64_t s = 0;
        for (; s + 2 <= nslices; s += 2) {
            step(std::integral_constant<int, 0>{}, s);
            step(std::integral_constant<int, 1>{}, s + 1);
        }
        if (s < nslices) step(std::integral_constant<int, 0>{}, s);
    } else {
        uint32_t wcur[kRows][B], wnxt[kRows][B];
        load_x(0, xnxt);
        load_w(0, wcur);
        stage_x_store<MT, kXPerThread>(&xs[0][0][xc * kXPitch + xp], xnxt);
        for (int64_t s = 0; s < nslices; ++s) {
            const bool more = s + 1 < nslices;
            if (more) {
                load_x(s + 1, xnxt);
                load_w(s + 1, wnxt);
            }
            __syncthreads();
            compute((int)(s & 1), s, wcur);
            if (more) {
                stage_x_store<MT, kXPerThread>(&xs[(s & 1) ^ 1][0][xc * kXPitch + xp], xnxt);
#pragma unroll
                for (int r = 0; r < kRows; ++r)
#pragma unroll
                    for (int i = 0; i < B; ++i) wcur[r][i] = wnxt[r][i];
            }
        }
    }

#pragma unroll
    for (int r = 0; r < kRows; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[r][m] = wave_sum(acc[r][m]);
    if (lane == 0) {
        constexpr float kUnscale = 1.0f / (float)(1 << (B <= 9 ? chunk_dot_shift<B>() : 0));
#pragma unroll
        for (int r = 0; r < kRows; ++r) {
            const int64_t n = n0 + r;
            if (n < N) {
                const float s = scales[n];
                const float zc = zp.template coef<B>(n);
#pragma unroll
                for (int m = 0; m < MT; ++m)
                    if (m < M) y[(int64_t)m * N + n] = s * zp.apply(acc[r][m] * kUnscale, zc, m);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// 3 <= M <= 16 on the matrix cores (v_mfma_f32_16x16x32_bf16): with up to 16
// rows of x the VALU dot products would cost up to 8 instructions per code,
// so the codes are expanded once into exact bf16 operands (2-3 instructions
// per code) and the products run on the MFMA units, leaving the kernel bound
// by the bytes of the packed weights again.
//
// A workgroup owns 16 kNT weight rows; its 4 waves take the 128-code K steps
// w, w+4, w+8, ... (together they stream each row's consecutive 512-code
// blocks) and add their partial 16 x 16 sums in LDS at the end.  In a step,
// lane l = 16 g + c takes chunk 4 ks + g of row c (B whole words) and, for
// MFMA substep t, its codes 8t .. 8t+7 as the B operand (column c, k rows
// 8g .. 8g+7 of the 16x16x32 shape); the A operand of lane l is x[c][32 (4 ks
// + g) + 8 t .. + 8], so both sides use the same order of k.  Rows m >= M of x
// are zero.  The codes and x of the next kDepth steps are loaded before this
// step is computed.  This kernel serves K not a multiple of 32 (per-lane
// guarded loads); gemv_mfma_xlds_kernel below serves the rest.
#ifndef DQ_GEMV_MFMA_WAVES
#define DQ_GEMV_MFMA_WAVES 4
#endif
constexpr int kGemvMfmaWaves = DQ_GEMV_MFMA_WAVES;

template <int B, int kNT, int kDepth, class ZP>
__global__ __launch_bounds__(kGemvMfmaWaves * kWave) void gemv_mfma_kernel(
    const uint16_t* __restrict__ x, int M, const uint32_t* __restrict__ packed,
    const float* __restrict__ scales, int64_t N, int64_t K, int64_t row_words,
    float* __restrict__ y, ZP zp)
{
    typedef __bf16 bf16x8m_t __attribute__((ext_vector_type(8)));
    typedef float f32x4m_t __attribute__((ext_vector_type(4)));
    constexpr bool kSplit = B >= 10;
    constexpr int kStages = kDepth + 1;
    static_assert(kDepth >= 1 && kDepth <= 3, "one to three steps ahead");
    __shared__ float red[kGemvMfmaWaves - 1][kNT][4][kWave];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int c = lane & 15;
    const int g = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * 16 * kNT;
    const uint32_t* rowp[kNT];
#pragma unroll
    for (int j = 0; j < kNT; ++j) {
        const int64_t n = n0 + 16 * j + c;
        rowp[j] = packed + (n < N ? n : N - 1) * row_words;
    }
    const int64_t nchunks = ceil_div(K, kChunk);
    const int64_t nsteps = ceil_div(nchunks, 4);
    const bool xrow = c < M;
    const uint16_t* xr = x + (int64_t)(xrow ? c : 0) * K;
    const bool xvec = (K & 7) == 0;

    uint32_t w[kStages][kNT][B];
    uint4 xa[kStages][4];
    auto load = [&](auto P, int64_t ks) {
        constexpr int p = decltype(P)::value;
        const int64_t ch = 4 * ks + g;
#pragma unroll
        for (int j = 0; j < kNT; ++j) {
            if (ks < nsteps && ch < nchunks) {
                load_chunk_words<B>(rowp[j], ch, row_words, w[p][j]);
            } else {
#pragma unroll
                for (int i = 0; i < B; ++i) w[p][j][i] = 0;
            }
        }
        const int64_t k0 = ch * kChunk;
        if (xrow && ks < nsteps && xvec && k0 + kChunk <= K) {
            const uint4* src = reinterpret_cast<const uint4*>(xr + k0);
#pragma unroll
            for (int i = 0; i < 4; ++i) xa[p][i] = src[i];
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint32_t d[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int64_t k = k0 + 8 * i + 2 * e;
                    const uint32_t lo = (xrow && ks < nsteps && k < K) ? xr[k] : 0u;
                    const uint32_t hi = (xrow && ks < nsteps && k + 1 < K) ? xr[k + 1] : 0u;
                    d[e] = lo | hi << 16;
                }
                xa[p][i] = make_uint4(d[0], d[1], d[2], d[3]);
            }
        }
    };
    f32x4m_t acc[kNT];
#pragma unroll
    for (int j = 0; j < kNT; ++j) acc[j] = (f32x4m_t){0.0f, 0.0f, 0.0f, 0.0f};
    auto compute = [&](auto P) {
        constexpr int p = decltype(P)::value;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const bf16x8m_t a = __builtin_bit_cast(bf16x8m_t, xa[p][t]);
#pragma unroll
            for (int j = 0; j < kNT; ++j) {
                bf16x8_t bh, bl;
                expand8<B>(w[p][j], t, bh, bl);
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bh, acc[j], 0, 0, 0);
                if constexpr (kSplit) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bl, acc[j], 0, 0, 0);
            }
        }
    };
    // Stage i of the register ring holds step ks + i kW.  Each step's loads
    // are pinned ahead of the computation of the step kDepth before it, so
    // the wait for a stage leaves the later stages' loads in flight.
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
        compute(I);
    };
    for (; ks + kDepth * kW < nsteps; ks += kStages * kW) {
        stage(std::integral_constant<int, 0>{});
        stage(std::integral_constant<int, 1>{});
        if constexpr (kStages > 2) stage(std::integral_constant<int, 2>{});
        if constexpr (kStages > 3) stage(std::integral_constant<int, 3>{});
    }
    if (ks < nsteps) compute(std::integral_constant<int, 0>{});
    if constexpr (kDepth > 1) if (ks + kW < nsteps) compute(std::integral_constant<int, 1>{});
    if constexpr (kDepth > 2) if (ks + 2 * kW < nsteps) compute(std::integral_constant<int, 2>{});

    // lane (g, c) holds rows 4 g + r of column c; waves 1..3 hand theirs to wave 0
    if (wave > 0) {
#pragma unroll
        for (int j = 0; j < kNT; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[wave - 1][j][r][lane] = acc[j][r];
    }
    __syncthreads();
    if (wave == 0) {
        constexpr float kUnscale = 1.0f / expand8_scale<B>();
#pragma unroll
        for (int j = 0; j < kNT; ++j) {
            const int64_t n = n0 + 16 * j + c;
            if (n >= N) continue;
            const float s = scales[n];
            const float zc = zp.template coef<B>(n);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float v = acc[j][r];
#pragma unroll
                for (int q = 0; q < kGemvMfmaWaves - 1; ++q) v += red[q][j][r][lane];
                const int m = 4 * g + r;
                if (m < M) y[(int64_t)m * N + n] = s * zp.apply(v * kUnscale, zc, m);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// 3 <= M <= 16 and K a multiple of 32: gemv_mfma_kernel with the codes and x
// taken through LDS.  Loaded into registers in the MFMA lane layout, each
// load instruction spreads its lanes over 16 rows (lane 16 g + c: row c,
// chunk g) and x costs as much as the code stream (each lane needs 64 bytes
// of one row, so a 16-byte load touches 64 cache lines, and lanes of rows
// past M load too).  Here each wave copies the codes and x of its own steps
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
template <int B>
constexpr int words_loads() { return B / 4 + (B % 4 != 0 ? 1 : 0); }

template <int B, int kNT, int kDepth, int kMR, class ZP>
__global__ __launch_bounds__(kGemvMfmaWaves * kWave) void gemv_mfma_xlds_kernel(
    const uint16_t* __restrict__ x, int M, const uint32_t* __restrict__ packed,
    const float* __restrict__ scales, int64_t N, int64_t K, int64_t row_words,
    float* __restrict__ y, ZP zp)
{
    typedef __bf16 bf16x8m_t __attribute__((ext_vector_type(8)));
    typedef float f32x4m_t __attribute__((ext_vector_type(4)));
    constexpr bool kSplit = B >= 10;
    constexpr int kStages = kDepth + 1;
    constexpr int kXCopies = kMR / 4;
    constexpr int kCodeSlots = (16 * kNT * B + 63) / 64 * 64;  // 16-byte code pieces of one step
    constexpr int kCodeCopies = kCodeSlots / 64;
    // group-wise scales (groups of whole 128-code steps): each step's scales of
    // the tile's rows come into LDS with the step's codes, one more copy
    constexpr bool kGroup = is_group_scales<ZP>::value;
    constexpr int kPerStage = kCodeCopies + kXCopies + (kGroup ? 1 : 0);
    constexpr int kSlots = kMR * 16;  // 16-byte x pieces of one step
    static_assert(kDepth >= 1 && kDepth <= 2, "one or two steps ahead");
    static_assert(kMR == 8 || kMR == 16, "x rows staged: 8 or 16");
    static_assert(kDepth * kPerStage < 64, "vmcnt holds at most 63");
    // one LDS object per stage, so each copy and read names its stage
    __shared__ __attribute__((aligned(16))) uint4 xs0[kGemvMfmaWaves][kSlots];
    __shared__ __attribute__((aligned(16))) uint4 xs1[kGemvMfmaWaves][kSlots];
    __shared__ __attribute__((aligned(16))) uint4 xs2[kStages > 2 ? kGemvMfmaWaves : 1][kStages > 2 ? kSlots : 1];
    __shared__ __attribute__((aligned(16))) uint4 xs3[kStages > 3 ? kGemvMfmaWaves : 1][kStages > 3 ? kSlots : 1];
    __shared__ float red[kGemvMfmaWaves - 1][kNT][4][kWave];
    __shared__ __attribute__((aligned(16))) uint4 cs0[kGemvMfmaWaves][kCodeSlots];
    __shared__ __attribute__((aligned(16))) uint4 cs1[kGemvMfmaWaves][kCodeSlots];
    __shared__ __attribute__((aligned(16))) uint4 cs2[kStages > 2 ? kGemvMfmaWaves : 1][kStages > 2 ? kCodeSlots : 1];
    __shared__ float ss[kGroup ? kStages : 1][kGroup ? kGemvMfmaWaves : 1][kGroup ? kWave : 1];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int c = lane & 15;
    const int g = lane >> 4;
    auto cring = [&](auto S) -> uint4* {
        constexpr int st = decltype(S)::value;
        if constexpr (st == 0) return cs0[wave];
        else if constexpr (st == 1) return cs1[wave];
        else return cs2[kStages > 2 ? wave : 0];
    };
    auto ring = [&](auto S) -> uint4* {
        constexpr int st = decltype(S)::value;
        if constexpr (st == 0) return xs0[wave];
        else if constexpr (st == 1) return xs1[wave];
        else if constexpr (st == 2) return xs2[kStages > 2 ? wave : 0];
        else return xs3[kStages > 3 ? wave : 0];
    };

    const int64_t n0 = (int64_t)blockIdx.x * 16 * kNT;
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
    [[maybe_unused]] BufRef sb{};
    [[maybe_unused]] int64_t steps_per_group = 1;
    if constexpr (kGroup) {
        sb = uniform_buf(zp.scales + n0 * zp.G, (uint32_t)(nrows * zp.G * 4));
        steps_per_group = zp.group / 128;
    }
    auto load = [&](auto P, int64_t ks) {
        if constexpr (kGroup) {  // lane r < 16 kNT: the scale of row r for step ks's group
            const int64_t gi = ks / steps_per_group;
            const bool in = lane < 16 * kNT && lane < nrows && gi < zp.G;
            buf_load_lds4(sb, &ss[kGroup ? decltype(P)::value : 0][kGroup ? wave : 0][0],
                          in ? (uint32_t)((lane * zp.G + gi) * 4) : kOutside, 0u);
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
                expand8<B>(wl[j], t, bh, bl);
                f32x4m_t& d = kGroup ? part[j] : acc[j];
                d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bh, d, 0, 0, 0);
                if constexpr (kSplit) d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bl, d, 0, 0, 0);
            }
        }
        if constexpr (kGroup) {
#pragma unroll
            for (int j = 0; j < kNT; ++j) {
                const float sg = ss[kGroup ? decltype(P)::value : 0][kGroup ? wave : 0][16 * j + c];
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
            for (int r = 0; r < 4; ++r) red[wave - 1][j][r][lane] = acc[j][r];
    }
    __syncthreads();
    if (wave == 0) {
        constexpr float kUnscale = 1.0f / expand8_scale<B>();
#pragma unroll
        for (int j = 0; j < kNT; ++j) {
            const int64_t n = n0 + 16 * j + c;
            if (n >= N) continue;
            const float s = kGroup ? 1.0f : scales[n];
            const float zc = zp.template coef<B>(n);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float v = acc[j][r];
#pragma unroll
                for (int q = 0; q < kGemvMfmaWaves - 1; ++q) v += red[q][j][r][lane];
                const int m = 4 * g + r;
                if (m < M) y[(int64_t)m * N + n] = s * zp.apply(v * kUnscale, zc, m);
            }
        }
    }
}

#ifndef DQ_GEMV_MFMA_DEPTH
#define DQ_GEMV_MFMA_DEPTH 2
#endif

template <int B, int kNT, class ZP>
hipError_t launch_gemv_mfma_nt(const uint16_t* x, int64_t M, const uint32_t* packed,
                               const float* scales, int64_t N, int64_t K, float* y, ZP zp,
                            hipStream_t stream)
{
    const int64_t rw = packed_row_words(K, B);
    const dim3 grid((unsigned)ceil_div(N, 16 * kNT)), block(kGemvMfmaWaves * kWave);
    if (K % kChunk == 0 && M <= 8)
        gemv_mfma_xlds_kernel<B, kNT, 2, 8><<<grid, block, 0, stream>>>(
            x, (int)M, packed, scales, N, K, rw, y, zp);
    else if (K % kChunk == 0)  // twice the x per stage: one step ahead, so two workgroups fit per CU
        gemv_mfma_xlds_kernel<B, kNT, 1, 16><<<grid, block, 0, stream>>>(
            x, (int)M, packed, scales, N, K, rw, y, zp);
    else if constexpr (!is_group_scales<ZP>::value)  // group scales come here with K % 32 == 0 only
        gemv_mfma_kernel<B, kNT, DQ_GEMV_MFMA_DEPTH><<<grid, block, 0, stream>>>(
            x, (int)M, packed, scales, N, K, rw, y, zp);
    return hipGetLastError();
}

// 32 rows per workgroup (x fragments shared by two row tiles) above 2^24
// weights, where there are workgroups enough for every CU; 16 rows below
template <int B, class ZP>
hipError_t launch_gemv_mfma(const uint16_t* x, int64_t M, const uint32_t* packed,
                            const float* scales, int64_t N, int64_t K, float* y, ZP zp,
                            hipStream_t stream)
{
#ifndef DQ_GEMV_MFMA_NT2_MIN
#define DQ_GEMV_MFMA_NT2_MIN (1LL << 24)
#endif
    if (N * K > DQ_GEMV_MFMA_NT2_MIN) return launch_gemv_mfma_nt<B, 2>(x, M, packed, scales, N, K, y, zp, stream);
    return launch_gemv_mfma_nt<B, 1>(x, M, packed, scales, N, K, y, zp, stream);
}

#ifndef DQ_GEMV_ROWS_NARROW
#define DQ_GEMV_ROWS_NARROW 1
#endif
#ifndef DQ_GEMV_ROWS_WIDE
#define DQ_GEMV_ROWS_WIDE 1
#endif
#ifndef DQ_GEMV_WAVES
#define DQ_GEMV_WAVES 8
#endif

// M <= 2, K a multiple of 32 and x small enough to sit in LDS whole
// (MT * K / 32 chunk slots of 80 B): x is staged once per workgroup (kR
// 16-byte pieces per thread, a fixed count; threads past the last piece
// repeat it), so the slice loop has no barriers, and each wave keeps the codes
// of up to three slices in flight (register stages by slice % 3, unrolled by
// three).  Loads: x first, then the codes of slices 0 and 1, then x to LDS
// (waiting only for x), then the slice loop.
constexpr int kXResMax = 48 * 1024;

template <int B, int MT, int kWaves, int kR, class ZP, int kRW>
__global__ __launch_bounds__(kWaves * kWave) void gemv_xres_kernel(
    const uint16_t* __restrict__ x, int M, const uint32_t* __restrict__ packed,
    const float* __restrict__ scales, int64_t N, int64_t K, int64_t row_words,
    float* __restrict__ y, ZP zp)
{
    extern __shared__ __attribute__((aligned(16))) uint16_t xs_dyn[];
    constexpr int kThreads = kWaves * kWave;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    // kRW rows per wave (1 or 2): their chunks form one stream of kRW * nchunks
    // chunks, so a row whose chunk count fills its last 64-chunk slice poorly
    // shares that slice with the next row
    static_assert(kRW == 1 || (kRW == 2 && !is_group_scales<ZP>::value), "two rows: per-row scales");
    const int64_t n = ((int64_t)blockIdx.x * kWaves + wave) * kRW;
    const int64_t nchunks = K / kChunk;
    const int64_t tchunks = kRW * nchunks;
    const int64_t nslices = ceil_div(tchunks, kSlice);
    const int64_t wrows = n < N ? (N - n < kRW ? N - n : kRW) : 1;
    const BufRef wbuf = uniform_buf(packed + (n < N ? n : N - 1) * row_words,
                                    (uint32_t)(wrows * row_words * 4));
    const BufRef xall = uniform_buf(x, (uint32_t)((int64_t)M * K * 2));

    // x piece p (8 elements) = piece p % 4 of chunk slot p / 4 (slot = m * nchunks + chunk)
    const int pieces = (int)(MT * nchunks * 4);
    uint4 xv[kR];
    int xdst[kR];
#pragma unroll
    for (int r = 0; r < kR; ++r) {
        const int p = min(tid + r * kThreads, pieces - 1);
        const int slot = p >> 2;
        xdst[r] = slot * kXPitch + (p & 3) * 8;
        // slot m * nchunks + c holds x[m][32 c ..]: its elements start at element
        // 32 * slot of the M x K row-major x (rows m >= M lie past the buffer: zeros)
        const u32x4v_t d = buf_load_b128(xall, (uint32_t)(slot * kChunk * 2 + (p & 3) * 16), 0u);
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
    for (int r = 0; r < kR; ++r) *reinterpret_cast<uint4*>(xs_dyn + xdst[r]) = xv[r];
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
                if constexpr (B <= 9)
                    chunk_dot<B, MT>(w[st], xw, part);
                else
                    chunk_fma<B, MT>(w[st], xw, part);
                const float sg = __uint_as_float(gsc[st]);
#pragma unroll
                for (int m = 0; m < MT; ++m) acc[m] = fmaf(part[m], sg, acc[m]);
            } else if constexpr (kRW == 2) {  // the chunk's sum goes to its row
                float part[MT];
#pragma unroll
                for (int m = 0; m < MT; ++m) part[m] = 0.0f;
                if constexpr (B <= 9)
                    chunk_dot<B, MT>(w[st], xw, part);
                else
                    chunk_fma<B, MT>(w[st], xw, part);
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    acc[m] += r ? 0.0f : part[m];
                    acc2[kRW == 2 ? m : 0] += r ? part[m] : 0.0f;
                }
            } else if constexpr (B <= 9) {
                chunk_dot<B, MT>(w[st], xw, acc);
            } else {
                chunk_fma<B, MT>(w[st], xw, acc);
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
        constexpr float kUnscale = 1.0f / (float)(1 << (B <= 9 ? chunk_dot_shift<B>() : 0));
        const float s = kGroup ? 1.0f : scales[n];
        const float zc = zp.template coef<B>(n);
#pragma unroll
        for (int m = 0; m < MT; ++m)
            if (m < M) y[(int64_t)m * N + n] = s * zp.apply(acc[m] * kUnscale, zc, m);
        if constexpr (kRW == 2) {
            if (n + 1 < N) {
                const float s2 = scales[n + 1];
                const float zc2 = zp.template coef<B>(n + 1);
#pragma unroll
                for (int m = 0; m < MT; ++m)
                    if (m < M)
                        y[(int64_t)m * N + n + 1] = s2 * zp.apply(acc2[m] * kUnscale, zc2, m);
            }
        }
    }
}

#ifndef DQ_GEMV_XRES_WAVES
#define DQ_GEMV_XRES_WAVES 4
#endif

template <int B, int MT, class ZP>
hipError_t launch_gemv_xres(const uint16_t* x, int64_t M, const uint32_t* packed,
                            const float* scales, int64_t N, int64_t K, float* y, ZP zp,
                            hipStream_t stream)
{
    constexpr int kWaves = DQ_GEMV_XRES_WAVES;
    constexpr int kThreads = kWaves * kWave;
    const int64_t rw = packed_row_words(K, B);
    const int64_t nchunks = K / kChunk;
    const size_t lds = (size_t)MT * nchunks * kXPitch * 2;
    const int64_t pieces = MT * nchunks * 4;
    const dim3 block(kThreads);
    // two rows per wave when a row's chunks fill their last 64-chunk slice
    // poorly and two rows' chunks fill theirs clearly better (per-row scales
    // only).  Measured: 160 chunks per row (83 % -> 100 % full) gains 5-14 %,
    // 544 chunks (94 % -> 100 %) loses 3 %, hence the 10-point margin.
    auto fill = [](int64_t c) { return (double)c / (double)(ceil_div(c, kSlice) * kSlice); };
    const bool two = std::is_same<ZP, NoZeroPoints>::value && fill(2 * nchunks) > fill(nchunks) + 0.1;
    // pieces per thread: every piece of x must be covered
    static_assert(10 * kThreads >= kXResMax / (kXPitch * 2) * 4, "x staging covers the largest x");
#define DQ_XRES_RW(R, RW)                                                                         \
    gemv_xres_kernel<B, MT, kWaves, R, ZP, RW>                                                    \
        <<<dim3((unsigned)ceil_div(N, kWaves * RW)), block, lds, stream>>>(x, (int)M, packed,     \
                                                                          scales, N, K, rw, y, zp)
#define DQ_XRES(R)                                                                                \
    do {                                                                                          \
        if constexpr (std::is_same<ZP, NoZeroPoints>::value) {                                   \
            if (two) {                                                                            \
                DQ_XRES_RW(R, 2);                                                                 \
                break;                                                                            \
            }                                                                                     \
        }                                                                                         \
        DQ_XRES_RW(R, 1);                                                                         \
    } while (0)
    if (pieces <= kThreads) DQ_XRES(1);
    else if (pieces <= 2 * kThreads) DQ_XRES(2);
    else if (pieces <= 3 * kThreads) DQ_XRES(3);
    else if (pieces <= 5 * kThreads) DQ_XRES(5);
    else DQ_XRES(10);
#undef DQ_XRES
#undef DQ_XRES_RW
    return hipGetLastError();
}

template <int B, int MT, class ZP>
hipError_t launch_gemv_lds(const uint16_t* x, int64_t M, const uint32_t* packed,
                           const float* scales, int64_t N, int64_t K, float* y, ZP zp,
                            hipStream_t stream)
{
    constexpr int kRows = B <= 8 ? DQ_GEMV_ROWS_NARROW : DQ_GEMV_ROWS_WIDE;
    constexpr int kWaves = DQ_GEMV_WAVES;
    const int64_t rw = packed_row_words(K, B);
    const int64_t rows_per_block = kWaves * kRows;
    const int64_t blocks = ceil_div(N, rows_per_block);
    if (K % kChunk == 0)
        gemv_lds_kernel<B, MT, kRows, kWaves, true><<<dim3((unsigned)blocks), dim3(kWaves * kWave), 0, stream>>>(
            x, (int)M, packed, scales, N, K, rw, y, zp);
    else
        gemv_lds_kernel<B, MT, kRows, kWaves, false><<<dim3((unsigned)blocks), dim3(kWaves * kWave), 0, stream>>>(
            x, (int)M, packed, scales, N, K, rw, y, zp);
    return hipGetLastError();
}

template <int B, class ZP>
hipError_t launch_gemv_b(const uint16_t* x, int64_t M, const uint32_t* packed, const float* scales,
                         int64_t N, int64_t K, float* y, ZP zp, hipStream_t stream)
{
#ifndef DQ_GEMV_NO_XRES
    // x resident in LDS when it fits, up to 2^27 weights (beyond, the sliced
    // kernel's eight waves per workgroup stream slightly faster)
    if (M <= 2 && K % kChunk == 0 && M * (K / kChunk) * kXPitch * 2 <= kXResMax &&
        N * K <= (1LL << 27)) {
        if (M <= 1) return launch_gemv_xres<B, 1>(x, M, packed, scales, N, K, y, zp, stream);
        return launch_gemv_xres<B, 2>(x, M, packed, scales, N, K, y, zp, stream);
    }
#endif
    if (M <= 1) return launch_gemv_lds<B, 1>(x, M, packed, scales, N, K, y, zp, stream);
    if (M <= 2) return launch_gemv_lds<B, 2>(x, M, packed, scales, N, K, y, zp, stream);
    return launch_gemv_mfma<B>(x, M, packed, scales, N, K, y, zp, stream);
}

// Group-wise scales ("量化" tutorial, exercise 1 of its exercises: one scale
// per group of g = 32 gpc consecutive codes of a row, scales [N, G]): each
// chunk's partial dot product is multiplied by its group's scale before it
// joins the row's sum, so no scale is left for the epilogue.  M <= 2 with x
// small enough for LDS takes the resident-x kernel above with a GroupScales
// policy; otherwise this kernel: four waves, one row per wave; lanes take
// chunks lane, lane + 64, ...; x read straight from global memory (at most 16
// rows, cached).
template <int B, int MT>
__global__ __launch_bounds__(4 * kWave) void gemv_group_kernel(
    const uint16_t* __restrict__ x, int M, const uint32_t* __restrict__ packed,
    const float* __restrict__ scales, int64_t N, int64_t K, int64_t row_words, int gpc, int64_t G,
    float* __restrict__ y)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t n = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (n >= N) return;  // the whole wave leaves; nothing waits on it
    const int64_t nchunks = ceil_div(K, kChunk);
    const uint32_t* __restrict__ row = packed + n * row_words;
    const bool xvec = (K & 7) == 0;
    float acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = 0.0f;
    for (int64_t c = lane; c < nchunks; c += kWave) {
        const int64_t k0 = c * kChunk;
        uint32_t wd[B];
        load_chunk_words<B>(row, c, row_words, wd);
#pragma unroll
        for (int i = 0; i < B; ++i) wd[i] ^= code_msb_mask<B>(i);
        float q[kChunk];
#pragma unroll
        for (int j = 0; j < kChunk; ++j)
            q[j] = k0 + j < K ? (float)chunk_code_signed<B>(wd, j) : 0.0f;
        const float sg = scales[n * G + c / gpc];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            if (m >= M) break;
            const uint16_t* xr = x + (int64_t)m * K + k0;
            float dot = 0.0f;
            if (xvec && k0 + kChunk <= K) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint4 d = reinterpret_cast<const uint4*>(xr)[i];
                    const uint32_t e[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        dot = fmaf(__uint_as_float(e[t] << 16), q[8 * i + 2 * t], dot);
                        dot = fmaf(__uint_as_float(e[t] & 0xffff0000u), q[8 * i + 2 * t + 1], dot);
                    }
                }
            } else {
#pragma unroll
                for (int j = 0; j < kChunk; ++j)
                    if (k0 + j < K) dot = fmaf(bf16_bits_to_float(xr[j]), q[j], dot);
            }
            acc[m] = fmaf(dot, sg, acc[m]);
        }
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = wave_sum(acc[m]);
    if (lane == 0) {
#pragma unroll
        for (int m = 0; m < MT; ++m)
            if (m < M) y[(int64_t)m * N + n] = acc[m];
    }
}

template <int B>
hipError_t launch_gemv_group_b(const uint16_t* x, int64_t M, const uint32_t* packed,
                               const float* scales, int64_t N, int64_t K, int64_t group, float* y,
                               hipStream_t stream)
{
    // M <= 2 with x resident in LDS: the per-row kernel with a scale per chunk
    if (M <= 2 && K % kChunk == 0 && M * (K / kChunk) * kXPitch * 2 <= kXResMax &&
        N * K <= (1LL << 27)) {
        const GroupScales gs{scales, ceil_div(K, group), group};
        if (M <= 1) return launch_gemv_xres<B, 1>(x, M, packed, scales, N, K, y, gs, stream);
        return launch_gemv_xres<B, 2>(x, M, packed, scales, N, K, y, gs, stream);
    }
    // 3 <= M <= 16, groups of whole 128-code steps: the matrix-core kernel,
    // each step's sums scaled by the step's group scales
    if (M >= 3 && K % kChunk == 0 && group % 128 == 0)
        return launch_gemv_mfma<B>(x, M, packed, scales, N, K, y,
                                   GroupScales{scales, ceil_div(K, group), group}, stream);
    const int64_t rw = packed_row_words(K, B);
    const dim3 grid((unsigned)ceil_div(N, 4)), block(4 * kWave);
    const int gpc = (int)(group / kChunk);
    const int64_t G = ceil_div(K, group);
#define DQ_GROUP(MT) \
    gemv_group_kernel<B, MT><<<grid, block, 0, stream>>>(x, (int)M, packed, scales, N, K, rw, gpc, G, y)
    if (M <= 1) DQ_GROUP(1);
    else if (M <= 2) DQ_GROUP(2);
    else if (M <= 4) DQ_GROUP(4);
    else if (M <= 8) DQ_GROUP(8);
    else DQ_GROUP(16);
#undef DQ_GROUP
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_group(const uint16_t* x, int64_t M, const uint32_t* packed,
                             const float* scales, int64_t N, int64_t K, int bits, int64_t group,
                             float* y, hipStream_t stream)
{
#define CALL(B) launch_gemv_group_b<B>(x, M, packed, scales, N, K, group, y, stream)
    DQ_BITS_SWITCH(bits, CALL)
#undef CALL
}

hipError_t launch_gemv(const uint16_t* x, int64_t M, const uint32_t* packed, const float* scales,
                       int64_t N, int64_t K, int bits, float* y, const int32_t* zeros,
                       const float* xsum, hipStream_t stream)
{
    if (zeros) {
        const ZeroPoints zp{zeros, xsum};
#define CALL(B) launch_gemv_b<B>(x, M, packed, scales, N, K, y, zp, stream)
        DQ_BITS_SWITCH(bits, CALL)
#undef CALL
    }
    const NoZeroPoints zp{};
#define CALL(B) launch_gemv_b<B>(x, M, packed, scales, N, K, y, zp, stream)
    DQ_BITS_SWITCH(bits, CALL)
#undef CALL
}

}  // namespace dq
