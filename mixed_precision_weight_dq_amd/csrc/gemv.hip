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
// scheme above), ZeroPoints (asymmetric codes: each code has the row's zero
// point taken off before it meets x, so every product is exact) and
// GroupScales (a scale per group of codes): the resident-x
// kernel applies it per chunk; gemv_mfma_xlds_kernel, for groups of whole
// 128-code steps, scales each step's MFMA sums before adding them in.
// gemv_group_kernel serves group-wise scales for the other shapes.
#include <type_traits>

#include "common.hpp"
#include "gemm_tiles.hpp"
#include "gemv_kernels.hpp"
#include "launch.hpp"

namespace dq {

namespace {

// ---------------------------------------------------------------------------
// M <= 2: x is staged per K-slice of 64 chunks (2048 codes) in LDS by the whole
// workgroup (coalesced 16-byte loads); each wave owns kRows rows and each lane
// one chunk of each of them per slice.  The next slice's packed words and x are
// loaded into registers before the current slice is computed, so every wave
// keeps two slices of loads in flight.
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
    int32_t zr[kRows];  // zero points of the wave's rows (asymmetric codes)
#pragma unroll
    for (int r = 0; r < kRows; ++r) zr[r] = zp.zero(n0 + r < N ? n0 + r : N - 1);

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
            for (int r = 0; r < kRows; ++r) chunk_product<B, MT, ZP::kAsym>(w[r], zr[r], xw, acc[r]);
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
        constexpr float kUnscale = product_unscale<B, ZP::kAsym>();
#pragma unroll
        for (int r = 0; r < kRows; ++r) {
            const int64_t n = n0 + r;
            if (n < N) {
                const float s = scales[n];
#pragma unroll
                for (int m = 0; m < MT; ++m)
                    if (m < M) y[(int64_t)m * N + n] = s * (acc[r][m] * kUnscale);
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

template <int B, int kNT, int kDepth, class ZP>
__global__ __launch_bounds__(kGemvMfmaWaves * kWave) void gemv_mfma_kernel(
    const uint16_t* __restrict__ x, int M, const uint32_t* __restrict__ packed,
    const float* __restrict__ scales, int64_t N, int64_t K, int64_t row_words,
    float* __restrict__ y, ZP zp)
{
    typedef __bf16 bf16x8m_t __attribute__((ext_vector_type(8)));
    typedef float f32x4m_t __attribute__((ext_vector_type(4)));
    constexpr bool kSplit = split_codes<B, ZP::kAsym>();
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
    int32_t zr[kNT];  // zero point of this lane's row in each row tile
#pragma unroll
    for (int j = 0; j < kNT; ++j) {
        const int64_t n = n0 + 16 * j + c;
        rowp[j] = packed + (n < N ? n : N - 1) * row_words;
        zr[j] = zp.zero(n < N ? n : N - 1);
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
                expand8z<B, ZP::kAsym>(w[p][j], zr[j], t, bh, bl);
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
        constexpr float kUnscale = 1.0f / expand8_scale<B, ZP::kAsym>();
#pragma unroll
        for (int j = 0; j < kNT; ++j) {
            const int64_t n = n0 + 16 * j + c;
            if (n >= N) continue;
            const float s = scales[n];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float v = acc[j][r];
#pragma unroll
                for (int q = 0; q < kGemvMfmaWaves - 1; ++q) v += red[q][j][r][lane];
                const int m = 4 * g + r;
                if (m < M) y[(int64_t)m * N + n] = s * (v * kUnscale);
            }
        }
    }
}

// 3 <= M <= 16 and K a multiple of 32: the matrix-core body with codes and x
// taken through LDS (gemv_kernels.hpp), one workgroup per 16 kNT rows.
template <int B, int kNT, int kDepth, int kMR, class ZP>
__global__ __launch_bounds__(kGemvMfmaWaves * kWave) void gemv_mfma_xlds_kernel(
    const uint16_t* __restrict__ x, int M, const uint32_t* __restrict__ packed,
    const float* __restrict__ scales, int64_t N, int64_t K, int64_t row_words,
    float* __restrict__ y, ZP zp)
{
    __shared__ __attribute__((aligned(16)))
    unsigned char lds[mfma_xlds_lds_bytes<B, kNT, kDepth, kMR, ZP::kAsym>()];
    gemv_mfma_xlds_body<B, kNT, kDepth, kMR, ZP>(x, M, packed, scales, N, K, row_words, y, zp,
                                                 (int64_t)blockIdx.x, lds);
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

template <int B, class ZP>
hipError_t launch_gemv_mfma(const uint16_t* x, int64_t M, const uint32_t* packed,
                            const float* scales, int64_t N, int64_t K, float* y, ZP zp,
                            hipStream_t stream)
{
    if (gemv_mfma_rows(N, K) == 32) return launch_gemv_mfma_nt<B, 2>(x, M, packed, scales, N, K, y, zp, stream);
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

#ifndef DQ_GEMV_XRES_WAVES
#define DQ_GEMV_XRES_WAVES 4
#endif

// one matrix per launch: workgroup blockIdx.x of its grid
template <int B, int MT, int kWaves, int kR, class ZP, int kRW>
__global__ __launch_bounds__(kWaves * kWave) void gemv_xres_kernel(
    const uint16_t* __restrict__ x, int M, const uint32_t* __restrict__ packed,
    const float* __restrict__ scales, int64_t N, int64_t K, int64_t row_words,
    float* __restrict__ y, ZP zp)
{
    extern __shared__ __attribute__((aligned(16))) uint16_t xs_dyn[];
    gemv_xres_body<B, MT, kWaves, kR, ZP, kRW>(x, M, packed, scales, N, K, row_words, y, zp,
                                               (int64_t)blockIdx.x, xs_dyn);
}

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

// 32 rows per workgroup (x fragments shared by two row tiles) above 2^24
// weights, where there are workgroups enough for every CU; 16 rows below
int gemv_mfma_rows(int64_t N, int64_t K) { return N * K > (1LL << 24) ? 32 : 16; }

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
                       hipStream_t stream)
{
    if (zeros) {
        const ZeroPoints zp{zeros};
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
