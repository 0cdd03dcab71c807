// Decode-shaped products of several matrices in one launch:
//   y_i[m, n] = s_i[n] * sum_k x_i[m, k] * q_i[n, k]   for items i = 0 .. count-1
// DynaQuant page, "自定义内核架构" (the bit saving turns into decode speed on
// bandwidth-bound hardware).  At M = 1 a 4096 x 4096 matrix is 8-17 MB of
// codes, a transfer of 1-2 us at HBM speed, comparable to the fixed cost of
// one kernel launch; a decode step multiplies the same activation by several
// such matrices (the projections of a layer), so giving all of them to one
// launch pays that cost once.
//
// The item descriptors travel by value in the kernel arguments (no device
// memory is allocated or written besides the outputs).  Each workgroup finds
// its item from a table of first-workgroup indices (a scalar scan over at most
// 32 entries) and runs one of the bodies of gemv_kernels.hpp for the item's
// width.  At M <= 2 there is one launch per scheme present among the items
// (per-row scales, zero points, group scales), the scheme a template policy of
// the bodies:
//   * rows of at least 64 chunks (K >= 2048): a streaming body.  The host
//     gives each item a share of two rounds of workgroups (twice as many as
//     the GPU holds at once) in proportion to its bytes, so each wave streams several
//     rows with its loads running ahead across row boundaries: the row-sliced
//     body when K is a multiple of 2048 (one row per slice) or of 1024 (two
//     rows per slice), else the stream body (per-row scales only; items of
//     the other schemes with such K take a launch of their own);
//   * shorter rows: the resident-x body, one (or, per-row scales, two) rows
//     per wave.
// At 3 <= M <= 16: the matrix-core body, one workgroup per row tile, as in
// dq_gemv (so a layer's 5120-row matrices, 160 tiles each, fill the GPU
// together where one alone leaves CUs idle); items with zero points or group
// scales take a launch of their own.
// Per chunk the arithmetic is that of the one-matrix resident-x kernel, so
// every output is within the same bound; the summation order differs only in
// that the streaming body adds each chunk's dot product to the row total
// instead of chaining it.  Items of different widths and shapes mix freely;
// the LDS per workgroup is sized for the largest x of the launch, and x is
// staged with a fixed count of loads sized for the largest x the kernel
// accepts (threads past an item's last piece load nothing).
#include <algorithm>

#include "common.hpp"
#include "gemv_kernels.hpp"
#include "launch.hpp"

namespace dq {

namespace {

// waves per workgroup: x is copied into LDS once per workgroup, so eight
// waves share each copy (the copies of a launch halve against four waves:
// decode 3.7 -> 4.2 TB/s; twelve or sixteen waves leave fewer workgroups per
// CU than the registers allow and ran slower)
constexpr int kBatchWaves = 8;
constexpr int kBatchXPieces = 5;  // x pieces per thread: covers kXResMax
static_assert(kBatchXPieces * kBatchWaves * kWave >= kXResMax / (kXPitch * 2) * 4,
              "x staging covers the largest x");

// item modes
constexpr int kModeRow = 0;     // one row per wave (resident-x body)
constexpr int kModeTwoRows = 1; // two rows per wave (resident-x body)
constexpr int kModeStream = 2;    // rpw rows per wave, streamed (K >= 2048)
constexpr int kModeRowSlice = 3;  // rpw rows per wave in whole-row slices (K % 2048 == 0)
constexpr int kModeRowSlice2 = 4; // the same, two rows per slice (K % 1024 == 0)

struct BatchItemArgs {
    const uint16_t* x;
    const uint32_t* packed;
    const float* scales;   // [N], or [N, G] group scales
    float* y;
    const int32_t* zeros;  // [N] zero points (asymmetric items)
    int32_t N;
    int32_t K;
    int32_t row_words;
    int32_t code;   // M <= 2: 8 * bits + mode; M >= 3: 2 * bits + row tiles - 1
    int32_t rpw;    // rows per wave (streaming modes)
    int32_t G;      // group scales per row (group-scale items)
    int32_t group;  // codes per group (group-scale items)
};

struct BatchArgs {
    BatchItemArgs item[kGemvBatchMax];
    int32_t first[kGemvBatchMax + 1];  // first workgroup of each item; first[count] = grid
    int32_t count;
    int32_t M;
};
static_assert(sizeof(BatchArgs) <= 4096, "kernel arguments stay within 4 KB");

// The arguments are read through the kernel-argument segment pointer (the
// struct is the only argument, at offset 0), so indexing them by the
// run-time item number is a scalar load; indexing the by-value parameter
// instead makes the compiler copy the whole struct into per-lane scratch.
__device__ __forceinline__ const BatchArgs& batch_args()
{
    // an address-space cast of the constant kernel-argument pointer; the
    // compiler infers the address space back and loads with scalar loads
    return *(const BatchArgs*)__builtin_amdgcn_kernarg_segment_ptr();
}

// The item's policy for the bodies: symmetric codes with a row scale,
// asymmetric codes (a zero point per row) or group-wise scales.
template <class ZP>
__device__ __forceinline__ ZP item_policy(const BatchItemArgs& it);
template <>
__device__ __forceinline__ NoZeroPoints item_policy<NoZeroPoints>(const BatchItemArgs&)
{
    return NoZeroPoints{};
}
template <>
__device__ __forceinline__ ZeroPoints item_policy<ZeroPoints>(const BatchItemArgs& it)
{
    return ZeroPoints{it.zeros};
}
template <>
__device__ __forceinline__ GroupScales item_policy<GroupScales>(const BatchItemArgs& it)
{
    return GroupScales{it.scales, it.G, it.group};
}

// kMaxB: the widest code the instance serves.  Launches whose items are all
// at most 8 bits take the narrow instance, whose register count (and so its
// occupancy) is not set by the wide codes' bodies.  ZP: the items' scheme (one
// launch per scheme); the two-rows and stream modes serve symmetric items only.
template <int MT, int kMaxB, class ZP>
__global__ __launch_bounds__(kBatchWaves * kWave) void gemv_xres_batch_kernel(const BatchArgs args)
{
    extern __shared__ __attribute__((aligned(16))) uint16_t xs_dyn[];
    (void)args;
    auto& a = batch_args();
    const int32_t bid = (int32_t)blockIdx.x;
    int i = 0;
    while (i + 1 < a.count && bid >= a.first[i + 1]) ++i;
    auto& it = a.item[i];
    const int64_t local = bid - a.first[i];
    const ZP zp = item_policy<ZP>(it);
    constexpr bool kSym = std::is_same<ZP, NoZeroPoints>::value;
    switch (it.code) {
#define DQ_BATCH_CASE(B)                                                                          \
    case 8 * B + kModeRow:                                                                        \
        if constexpr (B <= kMaxB)                                                                 \
            gemv_xres_body<B, MT, kBatchWaves, kBatchXPieces, ZP, 1, true>(                       \
                it.x, a.M, it.packed, it.scales, it.N, it.K, it.row_words, it.y, zp, local,       \
                xs_dyn);                                                                          \
        break;                                                                                    \
    case 8 * B + kModeTwoRows:                                                                    \
        if constexpr (B <= kMaxB && kSym)                                                         \
            gemv_xres_body<B, MT, kBatchWaves, kBatchXPieces, NoZeroPoints, 2, true>(             \
                it.x, a.M, it.packed, it.scales, it.N, it.K, it.row_words, it.y, NoZeroPoints{},  \
                local, xs_dyn);                                                                   \
        break;                                                                                    \
    case 8 * B + kModeStream:                                                                     \
        if constexpr (B <= kMaxB && kSym)                                                         \
            gemv_stream_body<B, MT, kBatchWaves, kBatchXPieces>(                                  \
                it.x, a.M, it.packed, it.scales, it.N, it.K, it.row_words, it.y,                  \
                local * kBatchWaves * it.rpw, it.rpw, xs_dyn);                                    \
        break;                                                                                    \
    case 8 * B + kModeRowSlice:                                                                   \
        if constexpr (B <= kMaxB)                                                                 \
            gemv_rowslice_body<B, MT, kBatchWaves, kBatchXPieces, 1, ZP>(                         \
                it.x, a.M, it.packed, it.scales, it.N, it.K, it.row_words, it.y,                  \
                local * kBatchWaves * it.rpw, it.rpw, xs_dyn, zp);                                \
        break;                                                                                    \
    case 8 * B + kModeRowSlice2:                                                                  \
        if constexpr (B <= kMaxB)                                                                 \
            gemv_rowslice_body<B, MT, kBatchWaves, kBatchXPieces, 2, ZP>(                         \
                it.x, a.M, it.packed, it.scales, it.N, it.K, it.row_words, it.y,                  \
                local * kBatchWaves * it.rpw, it.rpw, xs_dyn, zp);                                \
        break;
        DQ_BATCH_CASE(2)
        DQ_BATCH_CASE(3)
        DQ_BATCH_CASE(4)
        DQ_BATCH_CASE(5)
        DQ_BATCH_CASE(6)
        DQ_BATCH_CASE(7)
        DQ_BATCH_CASE(8)
        DQ_BATCH_CASE(9)
        DQ_BATCH_CASE(10)
        DQ_BATCH_CASE(11)
        DQ_BATCH_CASE(12)
        DQ_BATCH_CASE(13)
        DQ_BATCH_CASE(14)
        DQ_BATCH_CASE(15)
#undef DQ_BATCH_CASE
    default:
        break;
    }
}

// 3 <= M <= 16: the matrix-core body of dq_gemv, one workgroup per tile of
// 16 or 32 rows of an item (item code 2 * bits + kNT - 1, the tile height
// dq_gemv picks for that item), so every output equals dq_gemv's bit for bit.
// kMR: x rows staged, 8 (two steps of loads ahead) or 16 (one step ahead),
// as dq_gemv picks by M.  The LDS is sized for the widest code the instance
// serves; launches whose items are all at most 8 bits take the narrow one.
template <int kMR>
constexpr int mfma_batch_depth() { return kMR == 8 ? 2 : 1; }

template <int kMR, int... Bm2>
constexpr size_t mfma_batch_lds_of(std::integer_sequence<int, Bm2...>)
{
    size_t m = 0;
    ((m = std::max(m, mfma_xlds_lds_bytes<Bm2 + 2, 2, mfma_batch_depth<kMR>(), kMR, false>())), ...);
    return m;
}
template <int kMR, int kMaxB>
constexpr size_t mfma_batch_lds()
{
    return mfma_batch_lds_of<kMR>(std::make_integer_sequence<int, kMaxB - 1>{});
}

template <int kMR, int kMaxB>
__global__ __launch_bounds__(kGemvMfmaWaves * kWave) void gemv_mfma_batch_kernel(const BatchArgs args)
{
    constexpr int kDepth = mfma_batch_depth<kMR>();
    __shared__ __attribute__((aligned(16))) unsigned char lds[mfma_batch_lds<kMR, kMaxB>()];
    (void)args;
    auto& a = batch_args();
    const int32_t bid = (int32_t)blockIdx.x;
    int i = 0;
    while (i + 1 < a.count && bid >= a.first[i + 1]) ++i;
    auto& it = a.item[i];
    const int64_t tile = bid - a.first[i];
    const NoZeroPoints zp{};
    switch (it.code) {
#define DQ_MFMA_BATCH_CASE(B)                                                                     \
    case 2 * B:                                                                                   \
        if constexpr (B <= kMaxB)                                                                 \
            gemv_mfma_xlds_body<B, 1, kDepth, kMR, NoZeroPoints>(                                 \
                it.x, a.M, it.packed, it.scales, it.N, it.K, it.row_words, it.y, zp, tile, lds);  \
        break;                                                                                    \
    case 2 * B + 1:                                                                               \
        if constexpr (B <= kMaxB)                                                                 \
            gemv_mfma_xlds_body<B, 2, kDepth, kMR, NoZeroPoints>(                                 \
                it.x, a.M, it.packed, it.scales, it.N, it.K, it.row_words, it.y, zp, tile, lds);  \
        break;
        DQ_MFMA_BATCH_CASE(2)
        DQ_MFMA_BATCH_CASE(3)
        DQ_MFMA_BATCH_CASE(4)
        DQ_MFMA_BATCH_CASE(5)
        DQ_MFMA_BATCH_CASE(6)
        DQ_MFMA_BATCH_CASE(7)
        DQ_MFMA_BATCH_CASE(8)
        DQ_MFMA_BATCH_CASE(9)
        DQ_MFMA_BATCH_CASE(10)
        DQ_MFMA_BATCH_CASE(11)
        DQ_MFMA_BATCH_CASE(12)
        DQ_MFMA_BATCH_CASE(13)
        DQ_MFMA_BATCH_CASE(14)
        DQ_MFMA_BATCH_CASE(15)
#undef DQ_MFMA_BATCH_CASE
    default:
        break;
    }
}

// the resident-x kernel's two-rows-per-wave rule (see launch_gemv_xres)
bool two_rows(int64_t nchunks)
{
    auto fill = [](int64_t c) { return (double)c / (double)(ceil_div(c, kSlice) * kSlice); };
    return fill(2 * nchunks) > fill(nchunks) + 0.1;
}

// The body a streamed item takes: row-sliced when its rows are a whole number
// of slices of one row (K a multiple of 2048) or of two rows (K a multiple of
// 1024), so no lane idles; else the stream body, whose per-lane bookkeeping
// costs less than lanes idling in each row's last slice.
int stream_mode(int64_t nchunks)
{
    if (nchunks % kSlice == 0) return kModeRowSlice;
    if (nchunks % (kSlice / 2) == 0) return kModeRowSlice2;
    return kModeStream;
}

}  // namespace

bool gemv_batch_eligible(int64_t M, int64_t K)
{
    if (M > 2) return M <= 16 && K % kChunk == 0;
    return K % kChunk == 0 && M * (K / kChunk) * kXPitch * 2 <= kXResMax;
}

namespace {

// an item's scheme
enum Scheme { kSymmetric = 0, kAsymmetric = 1, kGrouped = 2 };
Scheme scheme_of(const GemvItem& g) { return g.zeros ? kAsymmetric : (g.group ? kGrouped : kSymmetric); }

// an item on its own: the one-matrix entry point of its scheme
hipError_t launch_alone(const GemvItem& g, int64_t M, hipStream_t stream)
{
    if (g.group) return launch_gemv_group(g.x, M, g.packed, g.scales, g.N, g.K, g.bits, g.group, g.y, stream);
    return launch_gemv(g.x, M, g.packed, g.scales, g.N, g.K, g.bits, g.y, g.zeros, stream);
}

BatchItemArgs item_args(const GemvItem& g, int32_t code, int32_t rpw)
{
    return BatchItemArgs{g.x, g.packed, g.scales, g.y, g.zeros, (int32_t)g.N, (int32_t)g.K,
                         (int32_t)packed_row_words(g.K, g.bits), code, rpw,
                         (int32_t)(g.group ? ceil_div(g.K, g.group) : 0), (int32_t)g.group};
}

// 3 <= M <= 16: symmetric items with K a multiple of 32 in one grid (each
// item's tile height as dq_gemv picks it), the rest one launch each
hipError_t launch_gemv_batched_mfma(const GemvItem* items, int count, int64_t M, hipStream_t stream)
{
    auto joins = [&](const GemvItem& g) { return scheme_of(g) == kSymmetric && gemv_batch_eligible(M, g.K); };
    bool narrow = true;
    for (int i = 0; i < count; ++i)
        if (joins(items[i]) && items[i].bits > 8) narrow = false;
    BatchArgs a;
    a.M = (int32_t)M;
    int n = 0;
    int64_t blocks = 0;
    auto flush = [&]() -> hipError_t {
        if (n == 0) return hipSuccess;
        a.count = n;
        a.first[n] = (int32_t)blocks;
        const dim3 grid((unsigned)blocks), block(kGemvMfmaWaves * kWave);
        if (M <= 8 && narrow)
            gemv_mfma_batch_kernel<8, 8><<<grid, block, 0, stream>>>(a);
        else if (M <= 8)
            gemv_mfma_batch_kernel<8, 15><<<grid, block, 0, stream>>>(a);
        else if (narrow)
            gemv_mfma_batch_kernel<16, 8><<<grid, block, 0, stream>>>(a);
        else
            gemv_mfma_batch_kernel<16, 15><<<grid, block, 0, stream>>>(a);
        n = 0;
        blocks = 0;
        return hipGetLastError();
    };
    for (int i = 0; i < count; ++i) {
        const GemvItem& g = items[i];
        if (!joins(g)) {  // this item takes its own launch
            const hipError_t e = launch_alone(g, M, stream);
            if (e != hipSuccess) return e;
            continue;
        }
        const int nt = gemv_mfma_rows(g.N, g.K) / 16;
        const int64_t nb = ceil_div(g.N, (int64_t)16 * nt);
        if (blocks + nb > 0x7fffffffLL) {  // the grid's index space is full: launch what we have
            const hipError_t e = flush();
            if (e != hipSuccess) return e;
        }
        a.item[n] = item_args(g, 2 * g.bits + nt - 1, 0);
        a.first[n] = (int32_t)blocks;
        blocks += nb;
        ++n;
    }
    return flush();
}

template <int MT, class ZP>
const void* xres_batch_kernel(bool narrow)
{
    return narrow ? reinterpret_cast<const void*>(&gemv_xres_batch_kernel<MT, 8, ZP>)
                  : reinterpret_cast<const void*>(&gemv_xres_batch_kernel<MT, 15, ZP>);
}

// M <= 2: the items of one scheme (indices idx[0 .. count)) that fit the
// launch, in one grid; the others one launch each
template <class ZP>
hipError_t launch_batched_xres(const GemvItem* items, const int* idx, int count, int64_t M,
                               hipStream_t stream)
{
    constexpr bool kSym = std::is_same<ZP, NoZeroPoints>::value;
    // the mode an item takes in the launch, or -1 for a launch of its own
    auto mode_of = [&](const GemvItem& g) -> int {
        if (!gemv_batch_eligible(M, g.K)) return -1;
        const int64_t nchunks = g.K / kChunk;
        if (nchunks < kSlice) return kSym && two_rows(nchunks) ? kModeTwoRows : kModeRow;
        const int mode = stream_mode(nchunks);
        return kSym || mode != kModeStream ? mode : -1;  // the stream body is symmetric only
    };
    // workgroups the GPU holds at once for this kernel (registers and LDS)
    size_t lds = 0;
    bool narrow = true;  // every item of the single launch at most 8 bits
    for (int k = 0; k < count; ++k) {
        const GemvItem& g = items[idx[k]];
        if (mode_of(g) < 0) continue;
        lds = std::max(lds, (size_t)(M * (g.K / kChunk) * kXPitch * 2));
        if (g.bits > 8) narrow = false;
    }
    const void* kernel = M <= 1 ? xres_batch_kernel<1, ZP>(narrow) : xres_batch_kernel<2, ZP>(narrow);
    int dev = 0, cus = 0, per_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kBatchWaves * kWave, lds);
    if (e != hipSuccess) return e;
    // two rounds of the workgroups the GPU holds at once: the second round
    // starts as the first one's workgroups end, which evens out their finish
    const int64_t slots = (int64_t)std::max(1, cus) * std::max(1, per_cu) * 2;
    double stream_bytes = 0;  // bytes of the streamed items, shared out over the slots
    for (int k = 0; k < count; ++k) {
        const GemvItem& g = items[idx[k]];
        const int mode = mode_of(g);
        if (mode == kModeStream || mode == kModeRowSlice || mode == kModeRowSlice2)
            stream_bytes += (double)g.N * packed_row_words(g.K, g.bits) * 4;
    }

    BatchArgs a;
    a.M = (int32_t)M;
    int n = 0;
    int64_t blocks = 0;
    auto flush = [&]() -> hipError_t {
        if (n == 0) return hipSuccess;
        a.count = n;
        a.first[n] = (int32_t)blocks;
        const dim3 grid((unsigned)blocks), block(kBatchWaves * kWave);
        if (M <= 1 && narrow)
            gemv_xres_batch_kernel<1, 8, ZP><<<grid, block, lds, stream>>>(a);
        else if (M <= 1)
            gemv_xres_batch_kernel<1, 15, ZP><<<grid, block, lds, stream>>>(a);
        else if (narrow)
            gemv_xres_batch_kernel<2, 8, ZP><<<grid, block, lds, stream>>>(a);
        else
            gemv_xres_batch_kernel<2, 15, ZP><<<grid, block, lds, stream>>>(a);
        n = 0;
        blocks = 0;
        return hipGetLastError();
    };
    for (int k = 0; k < count; ++k) {
        const GemvItem& g = items[idx[k]];
        const int mode = mode_of(g);
        if (mode < 0) {  // this item takes its own launch
            e = launch_alone(g, M, stream);
            if (e != hipSuccess) return e;
            continue;
        }
        const int64_t rw = packed_row_words(g.K, g.bits);
        int rpw = 1;
        int64_t nb;
        if (mode == kModeStream || mode == kModeRowSlice || mode == kModeRowSlice2) {
            // this item's share of the workgroups, in proportion to its
            // bytes; a workgroup's rows stay below 2^31 bytes
            const double share = (double)g.N * rw * 4 / stream_bytes;
            const int64_t wgs = std::max<int64_t>(1, (int64_t)(share * (double)slots));
            const int64_t rmax = std::max<int64_t>(1, 0x7fffffffLL / (rw * 4 * kBatchWaves));
            int64_t r = std::min<int64_t>(ceil_div(g.N, wgs * kBatchWaves), rmax);
            if (mode == kModeRowSlice2 && (r & 1))  // whole pairs of rows per wave (else half idles)
                r = std::min<int64_t>(r + 1, rmax);
            rpw = (int)r;
            nb = ceil_div(g.N, (int64_t)kBatchWaves * rpw);
        } else {
            nb = ceil_div(g.N, kBatchWaves * (mode == kModeTwoRows ? 2 : 1));
        }
        if (blocks + nb > 0x7fffffffLL) {  // the grid's index space is full: launch what we have
            e = flush();
            if (e != hipSuccess) return e;
        }
        a.item[n] = item_args(g, 8 * g.bits + mode, rpw);
        a.first[n] = (int32_t)blocks;
        blocks += nb;
        ++n;
    }
    return flush();
}

}  // namespace

hipError_t launch_gemv_batched(const GemvItem* items, int count, int64_t M, hipStream_t stream)
{
    if (M > 2) return launch_gemv_batched_mfma(items, count, M, stream);
    // one launch per scheme present, items in their given order within it
    int idx[3][kGemvBatchMax];
    int cnt[3] = {0, 0, 0};
    for (int i = 0; i < count; ++i) {
        const int sc = scheme_of(items[i]);
        idx[sc][cnt[sc]++] = i;
    }
    hipError_t e = hipSuccess;
    if (cnt[kSymmetric]) e = launch_batched_xres<NoZeroPoints>(items, idx[kSymmetric], cnt[kSymmetric], M, stream);
    if (e == hipSuccess && cnt[kAsymmetric])
        e = launch_batched_xres<ZeroPoints>(items, idx[kAsymmetric], cnt[kAsymmetric], M, stream);
    if (e == hipSuccess && cnt[kGrouped])
        e = launch_batched_xres<GroupScales>(items, idx[kGrouped], cnt[kGrouped], M, stream);
    return e;
}

}  // namespace dq
