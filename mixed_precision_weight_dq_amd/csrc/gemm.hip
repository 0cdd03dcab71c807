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
#include "gemm_tiles.hpp"
#include "launch.hpp"

namespace dq {

namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

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

// ---------------------------------------------------------------------------
// Main kernel (K a multiple of 64).  256 threads = 4 waves in a 2 x 2 grid; a
// wave owns a (32*kMT) x (32*kNT) block of y as kMT x kNT tiles of
// v_mfma_f32_32x32x16_bf16, so the workgroup tile is (64*kMT) x (64*kNT).
//
// K order inside a 64-wide step: MFMA substep t (0..3) multiplies, for lane
// half h (lanes 32h .. 32h+31), the 8 elements k = 32h + 8t + e.  Any fixed
// permutation of k is fine as long as x and the codes use the same one; this
// one lets lane (c, h) take all of its B operands from chunk h (32 codes = B
// whole words) of its own weight row, so codes go from HBM to registers to the
// matrix cores with no LDS round trip.
//
// x goes through LDS: each step's tile (rows x 64 bf16, 128 B per row) is
// copied with global_load_lds_dwordx4 into a double buffer; 16-byte piece p of
// row r is stored at slot p ^ (r & 7) so the fragment reads are bank-conflict
// free.  Rows past M are clamped to M-1 and weight rows past N to N-1 (their
// outputs are never stored).
template <int kMT, int kNT>
struct BigTile {
    static constexpr int BM = 64 * kMT;
    static constexpr int BN = 64 * kNT;
    static constexpr int BK = 64;
    static constexpr int kPiecesPerBuf = BM * 8;  // 16-byte pieces of one x tile
};

template <int B, int kMT, int kNT>
__global__ __launch_bounds__(256, 1) void gemm_big_kernel(
    const uint16_t* __restrict__ x, int64_t M, const uint32_t* __restrict__ packed,
    const float* __restrict__ scales, int64_t N, int64_t K, int64_t row_words,
    float* __restrict__ y)
{
    using T = BigTile<kMT, kNT>;
    constexpr bool kSplit = B >= 10;
    __shared__ __attribute__((aligned(16))) uint4 As[2][T::kPiecesPerBuf];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int wm = wave >> 1;
    const int wn = wave & 1;
    const int c = lane & 31;
    const int h = lane >> 5;

    // tile order: consecutive workgroups go to different XCDs (round robin over 8);
    // give each XCD a contiguous range of column tiles so the weight rows it
    // streams stay in its own L2.
    const int64_t ntm = ceil_div(M, T::BM);
    const int64_t ntn = ceil_div(N, T::BN);
    const int64_t tiles = ntm * ntn;
    int64_t L = blockIdx.x;
    if ((tiles & 7) == 0) L = (L & 7) * (tiles >> 3) + (L >> 3);
    const int64_t tm = L % ntm;
    const int64_t tn = L / ntm;
    const int64_t m0 = tm * T::BM;
    const int64_t n0 = tn * T::BN;
    const int64_t nk = K / T::BK;

    // x tile copy: wave w moves rows [w*BM/4, (w+1)*BM/4); one instruction moves
    // 8 rows x 8 pieces; lane -> (row r = 8i + lane/8, slot lane&7) <- piece slot^(r&7).
    // Buffer loads straight into LDS; the per-lane byte offsets are loop invariant
    // and the step advances the scalar offset.
    constexpr int kRowsPerWave = T::BM / 4;
    constexpr int kCopyInstr = kRowsPerWave / 8;
    const int64_t mrows = M - m0 < T::BM ? M - m0 : T::BM;
    const BufRef xbuf{x + m0 * K, (uint32_t)(mrows * K * 2)};
    uint32_t xoff[kCopyInstr];
#pragma unroll
    for (int i = 0; i < kCopyInstr; ++i) {
        const int r = wave * kRowsPerWave + i * 8 + (lane >> 3);
        const int64_t rl = r < mrows ? r : mrows - 1;
        xoff[i] = (uint32_t)(rl * K * 2 + 16 * ((lane & 7) ^ (r & 7)));
    }
    auto copy_x = [&](int64_t ks, int buf) {
#pragma unroll
        for (int i = 0; i < kCopyInstr; ++i) {
            buf_load_lds16(xbuf, &As[buf][(wave * kRowsPerWave + i * 8) * 8], xoff[i],
                           (uint32_t)(ks * T::BK * 2));
        }
    };

    // weight rows of this lane (one per n tile): chunk h of step ks starts at
    // byte (ks * 2 + h) * 4B of the row
    const int64_t nrows = N - n0 < T::BN ? N - n0 : T::BN;
    const BufRef wbuf{packed + n0 * row_words, (uint32_t)(nrows * row_words * 4)};
    uint32_t woff[kNT];
#pragma unroll
    for (int j = 0; j < kNT; ++j) {
        const int64_t nl = wn * 32 * kNT + j * 32 + c;
        woff[j] = (uint32_t)((nl < nrows ? nl : nrows - 1) * row_words * 4 + h * B * 4);
    }
    auto load_w = [&](int64_t ks, uint32_t (&w)[kNT][B]) {
#pragma unroll
        for (int j = 0; j < kNT; ++j) buf_load_words<B>(wbuf, woff[j], (uint32_t)(ks * 8 * B), w[j]);
    };

    f32x16_t acc[kMT][kNT];
#pragma unroll
    for (int i = 0; i < kMT; ++i)
#pragma unroll
        for (int j = 0; j < kNT; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // LDS slot of x fragment (row r of this wave's tile i, piece p)
    int arow_lds[kMT];
#pragma unroll
    for (int i = 0; i < kMT; ++i) arow_lds[i] = wm * 32 * kMT + i * 32 + c;

    uint32_t wcur[kNT][B];
    copy_x(0, 0);
    load_w(0, wcur);
    __builtin_amdgcn_s_waitcnt(0);  // all of step 0 in LDS / registers
    __syncthreads();

    for (int64_t ks = 0; ks < nk; ++ks) {
        const int cur = (int)(ks & 1);
        // x fragments of this step, all four substeps
        bf16x8_t a[4][kMT];
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int i = 0; i < kMT; ++i) {
                const int r = arow_lds[i];
                a[t][i] = __builtin_bit_cast(bf16x8_t, As[cur][r * 8 + ((4 * h + t) ^ (r & 7))]);
            }
        const bool more = ks + 1 < nk;
        uint32_t wnxt[kNT][B];
        if (more) {
            copy_x(ks + 1, cur ^ 1);
            load_w(ks + 1, wnxt);
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
#pragma unroll
            for (int j = 0; j < kNT; ++j) {
                bf16x8_t bh, bl;
                expand8<B>(wcur[j], t, bh, bl);
#pragma unroll
                for (int i = 0; i < kMT; ++i) {
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[t][i], bh, acc[i][j], 0, 0, 0);
                    if constexpr (kSplit)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[t][i], bl, acc[i][j], 0, 0, 0);
                }
            }
        }
        if (more) {
#pragma unroll
            for (int j = 0; j < kNT; ++j)
#pragma unroll
                for (int e = 0; e < B; ++e) wcur[j][e] = wnxt[j][e];
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }

    // epilogue: lane (c, h) holds column c of each tile, rows 8*(r/4) + 4*h + r%4
    constexpr float kUnscale = 1.0f / expand8_scale<B>();
#pragma unroll
    for (int j = 0; j < kNT; ++j) {
        const int64_t n = n0 + wn * 32 * kNT + j * 32 + c;
        if (n >= N) continue;
        const float s = scales[n];
#pragma unroll
        for (int i = 0; i < kMT; ++i) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t m = m0 + wm * 32 * kMT + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                if (m < M) y[m * N + n] = s * (acc[i][j][r] * kUnscale);
            }
        }
    }
}

template <int B, int kMT, int kNT>
hipError_t launch_gemm_big(const uint16_t* x, int64_t M, const uint32_t* packed,
                           const float* scales, int64_t N, int64_t K, float* y, hipStream_t stream)
{
    using T = BigTile<kMT, kNT>;
    const int64_t rw = packed_row_words(K, B);
    const int64_t tiles = ceil_div(N, T::BN) * ceil_div(M, T::BM);
    if (tiles > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    gemm_big_kernel<B, kMT, kNT><<<dim3((unsigned)tiles), dim3(256), 0, stream>>>(
        x, M, packed, scales, N, K, rw, y);
    return hipGetLastError();
}

template <int B>
hipError_t launch_gemm_b(const uint16_t* x, int64_t M, const uint32_t* packed, const float* scales,
                         int64_t N, int64_t K, float* y, hipStream_t stream)
{
    if (K % 64 == 0) {
        // 256 x 256 tiles when they fill the 256 CUs, else 128 x 128
        if (ceil_div(M, 256) * ceil_div(N, 256) >= 240)
            return launch_gemm_big<B, 4, 4>(x, M, packed, scales, N, K, y, stream);
        return launch_gemm_big<B, 2, 2>(x, M, packed, scales, N, K, y, stream);
    }
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
