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
// v_mfma_f32_16x16x32_bf16 over its 64 x 64 sub-tile.  That is the simple
// fallback (K not a multiple of 64); the main kernels below pipeline the
// codes through registers and x through LDS.  Variants: asymmetric codes
// have the row's zero point taken off each code before expansion, so every
// product stays exact (ZeroPoints policy); group-wise scales fold each
// group's sum in as it ends (GroupScales in the 128-row kernel, whose two
// waves per SIMD hide the fold's vector work behind each other's matrix
// work; gemm_group_kernel for groups of 32 codes).  The wide kernel holds no
// group-wise variant: its accumulators fill the accumulation registers, so a
// second set for the group's sum would not fit beside them.
#include <type_traits>

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

template <int B, class ZP>
__global__ __launch_bounds__(kGemmThreads) void gemm_kernel(
    const uint16_t* __restrict__ x, int64_t M, const uint32_t* __restrict__ packed,
    const float* __restrict__ scales, int64_t N, int64_t K, int64_t row_words,
    float* __restrict__ y, ZP zp)
{
    constexpr bool kAsym = ZP::kAsym;
    constexpr bool kSplit = split_codes<B, kAsym>();
    // two exact bf16 halves: q = 2^kShift * (q >> kShift) + (q & (2^kShift - 1))
    constexpr int kShift = kAsym ? B - 8 : 6;
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
    const int32_t zs = zp.zero(n0 + sr < N ? n0 + sr : N - 1);  // the staging row's zero point

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
            if constexpr (!kAsym) {
#pragma unroll
                for (int i = 0; i < B; ++i) wd[i] ^= code_msb_mask<B>(i);
            }
            uint16_t* d0 = &Bs[0][sr * kLd + kChunk * sh];
            uint16_t* d1 = &Bs[kPlanes - 1][sr * kLd + kChunk * sh];
#pragma unroll
            for (int j = 0; j < kChunk; ++j) {
                int32_t q = kAsym ? (int32_t)chunk_code_unsigned<B>(wd, j) - zs
                                  : chunk_code_signed<B>(wd, j);
                if (!live || c * kChunk + j >= K) q = 0;
                if (kSplit) {
                    d0[j] = exact_bf16_bits((q >> kShift) * (1 << kShift));
                    d1[j] = exact_bf16_bits(q & ((1 << kShift) - 1));
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
// Main kernel (K a multiple of 64).  256 threads = 4 waves side by side along
// N: wave w owns columns [w*32*kNT, (w+1)*32*kNT) of the workgroup tile and all
// 32*kMT of its rows, as kMT x kNT tiles of v_mfma_f32_32x32x16_bf16.  No two
// waves expand the same codes.
//
// K order inside a 64-wide step: MFMA substep t (0..3) multiplies, for lane
// half h (lanes 32h .. 32h+31), the 8 elements k = 32h + 8t + e.  Any fixed
// permutation of k is fine as long as x and the codes use the same one; this
// one lets lane (c, h) take all of its operands for one weight row from chunk
// h (32 codes = B whole words) of that row, so codes go from HBM to registers
// to the matrix cores with no LDS round trip.
//
// x goes through LDS: each step's tile (rows x 64 bf16 = 128 B per row) is
// loaded with coalesced 16-byte buffer loads into registers and written to a
// double buffer after the step's MFMAs are issued; 16-byte piece p of row r
// sits at slot p ^ ((r >> 1) & 7), which spreads the 16 rows that one
// ds_read_b128 pass touches over all 64 banks.  Loads for step ks+1 (x and
// codes) are issued right after the barrier that opens step ks; kOcc
// workgroups share a CU so one's MFMAs cover another's waits.
// Rows past M are clamped to M-1 and weight rows past N to N-1; their outputs
// are never stored.
#ifndef DQ_GEMM_MT
#define DQ_GEMM_MT 4
#endif
#ifndef DQ_GEMM_NT
#define DQ_GEMM_NT 2
#endif
#ifndef DQ_GEMM_OCC
#define DQ_GEMM_OCC 2
#endif

template <int kMT, int kNT>
struct MfmaTile {
    static constexpr int BM = 32 * kMT;
    static constexpr int BN = 4 * 32 * kNT;
    static constexpr int BK = 64;
    static constexpr int kStages = 2;
    static constexpr int kPieces = BM * 8;  // 16-byte pieces of one x tile
};

__device__ __forceinline__ int xswz(int r) { return (r >> 1) & 7; }

template <int B, int kMT, int kNT, int kOcc, class ZP>
__global__ __launch_bounds__(256, kOcc) void gemm_mfma_kernel(
    const uint16_t* __restrict__ x, int64_t M, const uint32_t* __restrict__ packed,
    const float* __restrict__ scales, int64_t N, int64_t K, int64_t row_words,
    float* __restrict__ y, ZP zp)
{
    using T = MfmaTile<kMT, kNT>;
    constexpr bool kAsym = ZP::kAsym;
    constexpr bool kSplit = split_codes<B, kAsym>();
    constexpr bool kGroup = is_group_scales<ZP>::value;
    constexpr int kCopyInstr = T::BM / 32;  // 16-byte x pieces per thread per step
    __shared__ __attribute__((aligned(16))) uint4 As[T::kStages][T::kPieces];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int c = lane & 31;
    const int h = lane >> 5;

    // tile order: consecutive workgroups go to different XCDs (round robin over
    // 8); give each XCD a contiguous range of tiles, column tiles outermost, so
    // the weight rows an XCD streams stay in its own L2.
    const int64_t ntm = ceil_div(M, T::BM);
    const int64_t ntn = ceil_div(N, T::BN);
    const int64_t tiles = ntm * ntn;
    int64_t L = blockIdx.x;
    if ((tiles & 7) == 0) L = (L & 7) * (tiles >> 3) + (L >> 3);
    const int64_t m0 = (L % ntm) * T::BM;
    const int64_t n0 = (L / ntm) * T::BN;
    const int64_t nk = K / T::BK;

    // x copy: thread t moves 16-byte piece p = t & 7 of rows r = 32 i + t / 8
    // (i < BM / 32), global -> registers during step ks -> LDS slot
    // 8 r + (p ^ xswz(r)) of the other stage once the step's MFMAs are issued.
    const int64_t mrows = M - m0 < T::BM ? M - m0 : T::BM;
    const BufRef xbuf = uniform_buf(x + m0 * K, (uint32_t)(mrows * K * 2));
    uint32_t xoff[kCopyInstr];
    int xslot[kCopyInstr];
#pragma unroll
    for (int i = 0; i < kCopyInstr; ++i) {
        const int r = i * 32 + (tid >> 3);
        const int p = tid & 7;
        const int64_t rl = r < mrows ? r : mrows - 1;
        xoff[i] = (uint32_t)(rl * K * 2 + 16 * p);
        xslot[i] = r * 8 + (p ^ xswz(r));
    }
    // weight rows of this lane: chunk h of step ks starts at byte (2 ks + h) * 4B
    const int64_t nrows = N - n0 < T::BN ? N - n0 : T::BN;
    const BufRef wbuf = uniform_buf(packed + n0 * row_words, (uint32_t)(nrows * row_words * 4));
    uint32_t woff[kNT];
    int32_t zr[kNT];  // zero point of this lane's weight row in each column tile
#pragma unroll
    for (int j = 0; j < kNT; ++j) {
        const int64_t nl = wave * 32 * kNT + j * 32 + c;
        woff[j] = (uint32_t)((nl < nrows ? nl : nrows - 1) * row_words * 4 + h * B * 4);
        zr[j] = zp.zero(n0 + (nl < nrows ? nl : nrows - 1));
    }
    // LDS slot of this lane's x fragment for tile i, substep t: row r = 32i + c,
    // and xswz(32i + c) = xswz(c), so the slot is 256 i + a constant per t
    int abase[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) abase[t] = c * 8 + ((4 * h + t) ^ xswz(c));

    f32x16_t acc[kMT][kNT];
    // group-wise scales: the current group's MFMAs accumulate here (the
    // group's first step starts them from zero)
    f32x16_t part[kGroup ? kMT : 1][kGroup ? kNT : 1];
#pragma unroll
    for (int i = 0; i < kMT; ++i)
#pragma unroll
        for (int j = 0; j < kNT; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // codes, ping-pong by step parity: stage st holds step ks (loaded during
    // step ks-1) and is expanded to MFMA operands at the top of step ks while
    // step ks+1 loads into stage st^1
    uint32_t w[2][kNT][B];
    uint4 xr[kCopyInstr];
    auto load_x = [&](int64_t ks) {
#pragma unroll
        for (int i = 0; i < kCopyInstr; ++i) {
            const u32x4v_t v = buf_load_b128(xbuf, xoff[i], (uint32_t)(ks * T::BK * 2));
            xr[i] = make_uint4(v.x, v.y, v.z, v.w);
        }
    };
    auto store_x = [&](auto S) {
        constexpr int st = decltype(S)::value;
#pragma unroll
        for (int i = 0; i < kCopyInstr; ++i) As[st][xslot[i]] = xr[i];
    };
    auto load_w = [&](auto S, int64_t ks) {
        constexpr int st = decltype(S)::value;
#pragma unroll
        for (int j = 0; j < kNT; ++j) buf_load_words<B>(wbuf, woff[j], (uint32_t)(ks * 8 * B), w[st][j]);
    };
    // group-wise scales: a group is 2^gsh whole steps (the group size is a
    // power of two of at least 64 codes here)
    [[maybe_unused]] int gsh = 0;
    if constexpr (kGroup) gsh = __builtin_ctzll((unsigned long long)(zp.group / 64));
    [[maybe_unused]] const int64_t gmask = ((int64_t)1 << gsh) - 1;
    // kFirst: step ks opens a group, so its first MFMAs start from zero
    // instead of the group sum (which therefore never needs clearing)
    auto step = [&](auto S, int64_t ks, auto kFirst) __attribute__((always_inline)) {
        // MFMAs of step ks from stage S
        constexpr int st = decltype(S)::value;
        constexpr bool first = decltype(kFirst)::value;
        __syncthreads();  // step ks in LDS for every wave; stage st^1 free again
        // this step's group scales, loaded every step (unconditional loads
        // keep the compiler's waits counted) before the next step's prefetch
        float sg[kNT];
        if constexpr (kGroup) {
#pragma unroll
            for (int j = 0; j < kNT; ++j) {
                const int64_t n = n0 + wave * 32 * kNT + j * 32 + c;
                sg[j] = zp.scales[(n < N ? n : N - 1) * zp.G + (ks >> gsh)];
            }
        }
        bf16x8_t bh[4][kNT], bl[4][kNT];
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int j = 0; j < kNT; ++j) expand8z<B, kAsym>(w[st][j], zr[j], t, bh[t][j], bl[t][j]);
        // step ks+1 (after the last step, the last step again: loads stay
        // inside the buffers and the data is never used)
        const int64_t kn = ks + 1 < nk ? ks + 1 : nk - 1;
        load_w(std::integral_constant<int, st ^ 1>{}, kn);
        load_x(kn);
        // keep the loads here, a whole step ahead of their use (the scheduler
        // would otherwise sink them next to the LDS stores to save registers)
        __builtin_amdgcn_sched_barrier(0);
        bf16x8_t a[2][kMT];  // x fragments of substep t (and t+1, read ahead)
#pragma unroll
        for (int i = 0; i < kMT; ++i) a[0][i] = __builtin_bit_cast(bf16x8_t, As[st][abase[0] + 256 * i]);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            if (t < 3) {
#pragma unroll
                for (int i = 0; i < kMT; ++i)
                    a[(t + 1) & 1][i] = __builtin_bit_cast(bf16x8_t, As[st][abase[t + 1] + 256 * i]);
            }
#pragma unroll
            for (int i = 0; i < kMT; ++i)
#pragma unroll
                for (int j = 0; j < kNT; ++j) {
                    f32x16_t& d = kGroup ? part[kGroup ? i : 0][kGroup ? j : 0] : acc[i][j];
                    const f32x16_t d0 = first && t == 0 ? f32x16_t{} : d;
                    d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[t & 1][i], bh[t][j], d0, 0, 0, 0);
                    if constexpr (kSplit)
                        d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[t & 1][i], bl[t][j], d, 0, 0, 0);
                }
        }
        store_x(std::integral_constant<int, st ^ 1>{});
        if constexpr (kGroup) {  // the group ends with this step: fold it in
            if (((ks + 1) & gmask) == 0 || ks + 1 == nk) {
#pragma unroll
                for (int i = 0; i < kMT; ++i)
#pragma unroll
                    for (int j = 0; j < kNT; ++j)
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            acc[i][j][r] = fmaf(sg[j], part[i][j][r], acc[i][j][r]);
            }
        }
    };
    // step ks from stage S, as a group's first step when it opens one
    auto run = [&](auto S, int64_t ks) __attribute__((always_inline)) {
        if constexpr (kGroup) {
            if ((ks & gmask) == 0)
                step(S, ks, std::true_type{});
            else
                step(S, ks, std::false_type{});
        } else {
            step(S, ks, std::false_type{});
        }
    };

    load_x(0);
    load_w(std::integral_constant<int, 0>{}, 0);
    store_x(std::integral_constant<int, 0>{});
    int64_t ks = 0;
    for (; ks + 2 <= nk; ks += 2) {
        run(std::integral_constant<int, 0>{}, ks);
        run(std::integral_constant<int, 1>{}, ks + 1);
    }
    if (ks < nk) run(std::integral_constant<int, 0>{}, ks);

    // epilogue: lane (c, h) holds column c of each tile, rows 8*(r/4) + 4*h + r%4;
    // whole tiles store without bounds checks, as streaming stores
    constexpr float kUnscale = 1.0f / expand8_scale<B, kAsym>();
    if (m0 + T::BM <= M && n0 + T::BN <= N) {
#pragma unroll
        for (int j = 0; j < kNT; ++j) {
            const int64_t n = n0 + wave * 32 * kNT + j * 32 + c;
            const float s = kGroup ? 1.0f : scales[n];
#pragma unroll
            for (int i = 0; i < kMT; ++i) {
                float* yp = y + (m0 + i * 32 + 4 * h) * N + n;
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    __builtin_nontemporal_store(s * (acc[i][j][r] * kUnscale),
                                                yp + (8 * (r >> 2) + (r & 3)) * N);
            }
        }
        return;
    }
#pragma unroll
    for (int j = 0; j < kNT; ++j) {
        const int64_t n = n0 + wave * 32 * kNT + j * 32 + c;
        if (n >= N) continue;
        const float s = kGroup ? 1.0f : scales[n];
#pragma unroll
        for (int i = 0; i < kMT; ++i) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t m = m0 + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                if (m < M) y[m * N + n] = s * (acc[i][j][r] * kUnscale);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Wide kernel for large M and N (K a multiple of 64): one 256-thread workgroup
// per CU computes a 256 x (128 kNT) tile.  Each wave owns all 256 rows and
// 32 kNT columns, so every expanded code operand feeds eight MFMAs (one per
// 32-row sub-tile of x): half the expansion work per MFMA of the 128-row
// kernel above.  The accumulators fill the 256 AGPRs (kNT = 2), which leaves
// one wave per SIMD, so the step is software-pipelined inside the wave:
//   * x goes from global memory straight into LDS (buffer_load ... lds; three
//     stages, same swizzle as above), a step ahead of its use;
//   * codes of step ks+2 are loaded at the top of step ks (three register
//     stages), so they have two steps to arrive;
//   * the operands of substep t+1 (and of the next step's substep 0) are
//     expanded while the MFMAs of substep t run.
// Tile order: consecutive workgroups go round robin to the 8 XCDs; each XCD
// gets a contiguous range of tiles laid out as groups of 4 row tiles by all
// column tiles, so an XCD streams half of x and a quarter of W (at 8 x 32
// tiles) instead of all of x.
#ifndef DQ_WIDE_DEPTH
#define DQ_WIDE_DEPTH 2
#endif

template <int kNT>
struct WideTile {
    static constexpr int BM = 256;
    static constexpr int BN = 4 * 32 * kNT;
    static constexpr int BK = 64;
    static constexpr int kPieces = BM * 8;  // 16-byte pieces of one x tile
};

template <int B, int kNT, int kDepth, class ZP>
__global__ __launch_bounds__(256, 1) void gemm_wide_kernel(
    const uint16_t* __restrict__ x, int64_t M, const uint32_t* __restrict__ packed,
    const float* __restrict__ scales, int64_t N, int64_t K, int64_t row_words,
    float* __restrict__ y, ZP zp)
{
    using T = WideTile<kNT>;
    constexpr int kStages = kDepth + 1;  // x (LDS) and code (register) stages
    constexpr int kMT = T::BM / 32;
    constexpr bool kAsym = ZP::kAsym;
    constexpr bool kSplit = split_codes<B, kAsym>();
    constexpr int kCopyInstr = T::BM / 32;  // 16-byte x pieces per thread per step
    __shared__ __attribute__((aligned(16))) uint4 As[kStages][T::kPieces];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int c = lane & 31;
    const int h = lane >> 5;

    const int64_t ntm = ceil_div(M, T::BM);
    const int64_t ntn = ceil_div(N, T::BN);
    const int64_t tiles = ntm * ntn;
    int64_t L = blockIdx.x;
    if ((tiles & 7) == 0) L = (L & 7) * (tiles >> 3) + (L >> 3);
    const int64_t gm = (ntm & 3) == 0 ? 4 : 1;
    const int64_t grp = L / (gm * ntn), rem = L % (gm * ntn);
    const int64_t m0 = (grp * gm + rem % gm) * T::BM;
    const int64_t n0 = (rem / gm) * T::BN;
    const int64_t nk = K / T::BK;

    // x copy, global -> LDS directly (buffer_load ... lds): instruction i of
    // wave w fills the 64 consecutive 16-byte LDS slots (8 w + i) * 64 + lane,
    // so lane l fetches the piece that belongs in its slot: row r = slot / 8,
    // piece p = (slot % 8) ^ xswz(r)
    const int64_t mrows = M - m0 < T::BM ? M - m0 : T::BM;
    const BufRef xbuf = uniform_buf(x + m0 * K, (uint32_t)(mrows * K * 2));
    uint32_t xoff[kCopyInstr];
#pragma unroll
    for (int i = 0; i < kCopyInstr; ++i) {
        const int slot = (wave * kCopyInstr + i) * 64 + lane;
        const int r = slot >> 3;
        const int p = (slot & 7) ^ xswz(r);
        const int64_t rl = r < mrows ? r : mrows - 1;
        xoff[i] = (uint32_t)(rl * K * 2 + 16 * p);
    }
    const int64_t nrows = N - n0 < T::BN ? N - n0 : T::BN;
    const BufRef wbuf = uniform_buf(packed + n0 * row_words, (uint32_t)(nrows * row_words * 4));
    uint32_t woff[kNT];
    int32_t zr[kNT];  // zero point of this lane's weight row in each column tile
#pragma unroll
    for (int j = 0; j < kNT; ++j) {
        const int64_t nl = wave * 32 * kNT + j * 32 + c;
        woff[j] = (uint32_t)((nl < nrows ? nl : nrows - 1) * row_words * 4 + h * B * 4);
        zr[j] = zp.zero(n0 + (nl < nrows ? nl : nrows - 1));
    }
    int abase[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) abase[t] = c * 8 + ((4 * h + t) ^ xswz(c));

    f32x16_t acc[kMT][kNT];
#pragma unroll
    for (int i = 0; i < kMT; ++i)
#pragma unroll
        for (int j = 0; j < kNT; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    uint32_t w[kStages][kNT][B];  // codes of steps ks .. ks+kDepth (stage = step % kStages)
    bf16x8_t bh[kNT], bl[kNT];  // operands of the current substep
    auto load_x = [&](auto S, int64_t ks) {  // x of step ks -> LDS stage S
        constexpr int st = decltype(S)::value;
#pragma unroll
        for (int i = 0; i < kCopyInstr; ++i)
            buf_load_lds16(xbuf, &As[st][(wave * kCopyInstr + i) * 64], xoff[i],
                           (uint32_t)(ks * T::BK * 2));
    };
    auto load_w = [&](auto S, int64_t ks) {
        constexpr int st = decltype(S)::value;
#pragma unroll
        for (int j = 0; j < kNT; ++j) buf_load_words<B>(wbuf, woff[j], (uint32_t)(ks * 8 * B), w[st][j]);
    };
    // MFMAs of one substep and the instructions that prepare the next one,
    // interleaved: every MFMA (32 cycles) covers a share of the next
    // substep's LDS reads and code expansion.
    constexpr int kMfmaPerSub = kMT * kNT * (kSplit ? 2 : 1);
    auto interleave = [&]() {
#pragma unroll
        for (int g = 0; g < kMT; ++g) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                // 1 LDS read
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                // 1 MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);                // 6 VALU
#pragma unroll
            for (int e = 1; e < kMfmaPerSub / kMT; ++e) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
            }
        }
    };
    bf16x8_t a[2][kMT];  // x operands of the current and the next substep
    auto read_a = [&](auto S, int t, bf16x8_t (&dst)[kMT]) {
        constexpr int st = decltype(S)::value;
#pragma unroll
        for (int i = 0; i < kMT; ++i) dst[i] = __builtin_bit_cast(bf16x8_t, As[st][abase[t] + 256 * i]);
    };
    // Vector-memory operations a wave may leave in flight when it waits for
    // its copy of x(ks+1) before the barrier of step ks: the code loads issued
    // at the tops of steps ks+2-kDepth .. ks and the x copies issued in the
    // middle of steps ks+2-kDepth .. ks-1 (all issued after that copy).
    constexpr int kWLoads = kNT * (B / 4 + (B % 4 != 0 ? 1 : 0));
    constexpr int kAfter = (kDepth - 1) * kWLoads + (kDepth - 2) * kCopyInstr;
    // s_waitcnt with only the vector-memory count limited (gfx9 encoding:
    // vmcnt bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at maximum)
    constexpr int kWaitX = (kAfter & 15) | ((kAfter >> 4) << 14) | (7 << 4) | (15 << 8);
    // prologue: x(0) .. x(kDepth-1), then the codes of steps 0 .. kDepth-1
    constexpr int kPro = (kDepth - 1) * kCopyInstr + kDepth * kWLoads;
    constexpr int kWaitPro = (kPro & 15) | ((kPro >> 4) << 14) | (7 << 4) | (15 << 8);
    static_assert(kPro < 64 && kAfter < 64, "vmcnt holds at most 63");

    // step ks with its x in LDS stage S and its codes in register stage S
    // (both ks % kStages).  Top: the codes of step ks+kDepth are loaded.
    // After substep 2 each wave waits for its copy of x(ks+1) into LDS (only
    // operations issued after it may remain), and a barrier makes stage ks+1
    // visible; substep 3 reads its first operands, and x of step ks+kDepth is
    // copied into its stage, which no wave reads any more (its last reads came
    // before the barrier of step ks-1).  After the last step the loads fetch
    // the last step again (in bounds, never used).
    auto step = [&](auto S, int64_t ks) {
        constexpr int st = decltype(S)::value;
        constexpr int s1 = (st + 1) % kStages, sd = (st + kDepth) % kStages;
        const int64_t kd = ks + kDepth < nk ? ks + kDepth : nk - 1;
        load_w(std::integral_constant<int, sd>{}, kd);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            if (t < 3)
                read_a(S, t + 1, a[(t + 1) & 1]);
            else
                read_a(std::integral_constant<int, s1>{}, 0, a[0]);
            bf16x8_t nh[kNT], nl[kNT];
#pragma unroll
            for (int j = 0; j < kNT; ++j) {
                if (t < 3)
                    expand8z<B, kAsym>(w[st][j], zr[j], t + 1, nh[j], nl[j]);
                else
                    expand8z<B, kAsym>(w[s1][j], zr[j], 0, nh[j], nl[j]);
            }
#pragma unroll
            for (int i = 0; i < kMT; ++i)
#pragma unroll
                for (int j = 0; j < kNT; ++j) {
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[t & 1][i], bh[j], acc[i][j], 0, 0, 0);
                    if constexpr (kSplit)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[t & 1][i], bl[j], acc[i][j], 0, 0, 0);
                }
#pragma unroll
            for (int j = 0; j < kNT; ++j) {
                bh[j] = nh[j];
                bl[j] = nl[j];
            }
            interleave();
            __builtin_amdgcn_sched_barrier(0);
            if (t == 2) {
                __builtin_amdgcn_s_waitcnt(kWaitX);
                __syncthreads();  // stage ks+1 written by every wave
                load_x(std::integral_constant<int, sd>{}, kd);
            }
        }
    };

    static_assert(kDepth == 2 || kDepth == 3, "pipeline depth 2 or 3");
    load_x(std::integral_constant<int, 0>{}, 0);
    load_x(std::integral_constant<int, 1>{}, nk > 1 ? 1 : nk - 1);
    if constexpr (kDepth > 2) load_x(std::integral_constant<int, 2 % kStages>{}, nk > 2 ? 2 : nk - 1);
    load_w(std::integral_constant<int, 0>{}, 0);
    load_w(std::integral_constant<int, 1>{}, nk > 1 ? 1 : nk - 1);
    if constexpr (kDepth > 2) load_w(std::integral_constant<int, 2 % kStages>{}, nk > 2 ? 2 : nk - 1);
    __builtin_amdgcn_s_waitcnt(kWaitPro);  // x(0) in LDS
    __syncthreads();
    read_a(std::integral_constant<int, 0>{}, 0, a[0]);
#pragma unroll
    for (int j = 0; j < kNT; ++j) expand8z<B, kAsym>(w[0][j], zr[j], 0, bh[j], bl[j]);
    int64_t ks = 0;
    for (; ks + kStages <= nk; ks += kStages) {
        step(std::integral_constant<int, 0>{}, ks);
        step(std::integral_constant<int, 1>{}, ks + 1);
        step(std::integral_constant<int, 2>{}, ks + 2);
        if constexpr (kStages > 3) step(std::integral_constant<int, 3 % kStages>{}, ks + 3);
    }
    if (ks < nk) step(std::integral_constant<int, 0>{}, ks);
    if (ks + 1 < nk) step(std::integral_constant<int, 1>{}, ks + 1);
    if constexpr (kStages > 3)
        if (ks + 2 < nk) step(std::integral_constant<int, 2>{}, ks + 2);
    // the copies into LDS issued by the last step are never waited for by a
    // barrier; let them land before the workgroup ends, so they cannot write
    // into the LDS of the next workgroup placed on this CU
    __builtin_amdgcn_s_waitcnt(0);

    // epilogue: lane (c, h) holds column c of each 32 x 32 tile, rows
    // 8 (r / 4) + 4 h + r % 4 of accumulator register r.  Whole tiles store
    // without bounds checks, as streaming (nontemporal) stores: y is written
    // once and not read back by this kernel.  They are buffer stores whose row
    // offset is a scalar (the same for every lane), so no per-store address
    // arithmetic runs on the vector units; the tile's 256 rows of y must span
    // less than 4 GiB (N < 2^22), else the checked stores below serve.
    constexpr float kUnscale = 1.0f / expand8_scale<B, kAsym>();
    if (m0 + T::BM <= M && n0 + T::BN <= N && (int64_t)T::BM * N * 4 <= 0xffffffffLL) {
        const BufRef yb = uniform_buf(y + m0 * N, (uint32_t)(T::BM * N * 4));
        const uint32_t row4 = (uint32_t)(N * 4);
#pragma unroll
        for (int j = 0; j < kNT; ++j) {
            const int64_t n = n0 + wave * 32 * kNT + j * 32 + c;
            const float s = scales[n];
            const uint32_t voff = (uint32_t)(4 * h) * row4 + (uint32_t)n * 4;
#pragma unroll
            for (int i = 0; i < kMT; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    buf_store_f32_nt(yb, s * (acc[i][j][r] * kUnscale), voff,
                                     (uint32_t)(i * 32 + 8 * (r >> 2) + (r & 3)) * row4);
        }
        return;
    }
#pragma unroll
    for (int j = 0; j < kNT; ++j) {
        const int64_t n = n0 + wave * 32 * kNT + j * 32 + c;
        if (n >= N) continue;
        const float s = scales[n];
#pragma unroll
        for (int i = 0; i < kMT; ++i) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t m = m0 + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                if (m < M) y[m * N + n] = s * (acc[i][j][r] * kUnscale);
            }
        }
    }
}

template <int B, int kNT, int kDepth, class ZP>
hipError_t launch_gemm_wide(const uint16_t* x, int64_t M, const uint32_t* packed,
                            const float* scales, int64_t N, int64_t K, float* y, ZP zp,
                            hipStream_t stream)
{
    using T = WideTile<kNT>;
    const int64_t rw = packed_row_words(K, B);
    const int64_t tiles = ceil_div(N, T::BN) * ceil_div(M, T::BM);
    if (tiles > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    gemm_wide_kernel<B, kNT, kDepth><<<dim3((unsigned)tiles), dim3(256), 0, stream>>>(
        x, M, packed, scales, N, K, rw, y, zp);
    return hipGetLastError();
}

template <int B, int kMT, int kNT, int kOcc, class ZP>
hipError_t launch_gemm_mfma(const uint16_t* x, int64_t M, const uint32_t* packed,
                            const float* scales, int64_t N, int64_t K, float* y, ZP zp,
                            hipStream_t stream)
{
    using T = MfmaTile<kMT, kNT>;
    const int64_t rw = packed_row_words(K, B);
    const int64_t tiles = ceil_div(N, T::BN) * ceil_div(M, T::BM);
    if (tiles > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    gemm_mfma_kernel<B, kMT, kNT, kOcc><<<dim3((unsigned)tiles), dim3(256), 0, stream>>>(
        x, M, packed, scales, N, K, rw, y, zp);
    return hipGetLastError();
}

template <int B, class ZP>
hipError_t launch_gemm_b(const uint16_t* x, int64_t M, const uint32_t* packed, const float* scales,
                         int64_t N, int64_t K, float* y, ZP zp, hipStream_t stream)
{
    if (K % 64 == 0) {
        // 256-row tiles with one workgroup per CU when they fill the 256 CUs
        // in whole rounds (at least 80 % of the last round busy)
        constexpr int kWideNT = 2;
        const int64_t wide = ceil_div(M, 256) * ceil_div(N, WideTile<kWideNT>::BN);
        if (M >= 256 && wide >= 256 && wide * 5 >= ceil_div(wide, 256) * 256 * 4)
            return launch_gemm_wide<B, kWideNT, DQ_WIDE_DEPTH>(x, M, packed, scales, N, K, y, zp, stream);
        // 256 x 128 tiles when the wider ones are too few (e.g. M = 256 with N
        // in the tens of thousands): taken when they fill the CUs in at most
        // two rounds, at least 85 % busy; one row tile then reads each code
        // once where the 128-row tiles read it twice
        const int64_t wide1 = ceil_div(M, 256) * ceil_div(N, WideTile<1>::BN);
        const int64_t rounds1 = ceil_div(wide1, 256);
        if (M >= 256 && rounds1 <= 2 && wide1 * 20 >= rounds1 * 256 * 17)
            return launch_gemm_wide<B, 1, DQ_WIDE_DEPTH>(x, M, packed, scales, N, K, y, zp, stream);
        // 128 x 256 tiles (codes up to 8 bits: wider ones need more registers
        // than two workgroups per CU leave), when they fill the 256 CUs twice
        // over; else 128 x 128
        if constexpr (B <= 8) {
            if (ceil_div(M, 128) * ceil_div(N, 256) >= 400)
                return launch_gemm_mfma<B, DQ_GEMM_MT, DQ_GEMM_NT, DQ_GEMM_OCC>(x, M, packed, scales,
                                                                               N, K, y, zp, stream);
        }
        return launch_gemm_mfma<B, 4, 1, 2>(x, M, packed, scales, N, K, y, zp, stream);
    }
    const int64_t rw = packed_row_words(K, B);
    const int64_t tiles = ceil_div(N, kBN) * ceil_div(M, kBM);
    if (tiles > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)tiles);
    gemm_kernel<B><<<grid, dim3(kGemmThreads), 0, stream>>>(x, M, packed, scales, N, K, rw, y, zp);
    return hipGetLastError();
}

// Group-wise scales ("量化" tutorial, exercise 1 of its exercises; scales
// [N, G], one per group of g codes, g a multiple of 32).  The 128 x 128 tile of
// gemm_kernel with one change: each 32-wide K slice lies inside one group, so
// the MFMAs of a group accumulate into a second set of registers that is
// scaled per output column by that group's scale and added to the result
// when the group ends.  No scale is left for the epilogue.
template <int B>
__global__ __launch_bounds__(kGemmThreads) void gemm_group_kernel(
    const uint16_t* __restrict__ x, int64_t M, const uint32_t* __restrict__ packed,
    const float* __restrict__ scales, int64_t N, int64_t K, int64_t row_words, int64_t group,
    int64_t G, float* __restrict__ y)
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

    f32x4_t acc[4][4], part[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            acc[i][j] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
            part[i][j] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
        }

    const int sr = tid >> 1;  // staging row within the tile
    const int sh = tid & 1;   // which 32-wide half of the k slice

    for (int64_t k0 = 0; k0 < K; k0 += kBK) {
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
                        part[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j],
                                                                             part[i][j], 0, 0, 0);
            }
            // the slice [kend - 32, kend) closes its group: fold it in
            const int64_t kend = k0 + 32 * (kk + 1);
            if (kend % group == 0 || kend >= K) {
                const int64_t gi = (kend - 1) / group;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int64_t n = n0 + wn * 64 + j * 16 + (lane & 15);
                    const float sg = n < N ? scales[n * G + gi] : 0.0f;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
#pragma unroll
                        for (int r = 0; r < 4; ++r) acc[i][j][r] = fmaf(sg, part[i][j][r], acc[i][j][r]);
                        part[i][j] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
                    }
                }
            }
            if (kend >= K) break;
        }
        __syncthreads();
    }

    // ---- epilogue: lane holds column lane&15, rows 4*(lane>>4)+r
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t n = n0 + wn * 64 + j * 16 + (lane & 15);
        if (n >= N) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t m = m0 + wm * 64 + i * 16 + 4 * (lane >> 4) + r;
                if (m < M) y[m * N + n] = acc[i][j][r];
            }
        }
    }
}

template <int B>
hipError_t launch_gemm_group_b(const uint16_t* x, int64_t M, const uint32_t* packed,
                               const float* scales, int64_t N, int64_t K, int64_t group, float* y,
                               hipStream_t stream)
{
    // groups of whole 64-wide K steps: the pipelined 128-row kernel, whose
    // MFMAs take codes from two neighbouring 32-code chunks at once
    if (K % 64 == 0 && group % 64 == 0)
        return launch_gemm_mfma<B, 4, 1, 2>(x, M, packed, scales, N, K, y,
                                            GroupScales{scales, ceil_div(K, group), group},
                                            stream);
    const int64_t rw = packed_row_words(K, B);
    const int64_t tiles = ceil_div(N, kBN) * ceil_div(M, kBM);
    if (tiles > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    gemm_group_kernel<B><<<dim3((unsigned)tiles), dim3(kGemmThreads), 0, stream>>>(
        x, M, packed, scales, N, K, rw, group, ceil_div(K, group), y);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_group(const uint16_t* x, int64_t M, const uint32_t* packed,
                             const float* scales, int64_t N, int64_t K, int bits, int64_t group,
                             float* y, hipStream_t stream)
{
#define CALL(B) launch_gemm_group_b<B>(x, M, packed, scales, N, K, group, y, stream)
    DQ_BITS_SWITCH(bits, CALL)
#undef CALL
}

hipError_t launch_gemm(const uint16_t* x, int64_t M, const uint32_t* packed, const float* scales,
                       int64_t N, int64_t K, int bits, float* y, const int32_t* zeros,
                       hipStream_t stream)
{
    if (zeros) {
        const ZeroPoints zp{zeros};
#define CALL(B) launch_gemm_b<B>(x, M, packed, scales, N, K, y, zp, stream)
        DQ_BITS_SWITCH(bits, CALL)
#undef CALL
    }
    const NoZeroPoints zp{};
#define CALL(B) launch_gemm_b<B>(x, M, packed, scales, N, K, y, zp, stream)
    DQ_BITS_SWITCH(bits, CALL)
#undef CALL
}

}  // namespace dq
