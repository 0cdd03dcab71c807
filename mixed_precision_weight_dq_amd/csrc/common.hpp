// Shared device helpers for the packed b-bit kernels (gfx950, wave64).
//
// Packed layout (DynaQuant page, "自定义内核架构": b-bit codes stored densely and
// expanded in registers): code u = q + 2^(b-1) of element k of a row sits at
// stream bits [k*b, k*b+b); stream bit i is bit (i & 31) of word i >> 5.
// A run of 32 consecutive codes therefore fills exactly b whole words, which
// is the unit ("chunk") every kernel here works on: one lane owns one chunk and
// never shares a word with another lane.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dq {

constexpr int kWave = 64;
constexpr int kChunk = 32;  // codes per chunk; a chunk is exactly B words

__host__ __device__ constexpr int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

__device__ __forceinline__ float bf16_bits_to_float(uint32_t h) { return __uint_as_float(h << 16); }

// Word i of a chunk holds the top bit of every code whose last bit lands in it.
// XOR-ing a word with this mask turns each offset-binary code (q + 2^(b-1))
// into the b-bit two's complement of q, so a signed bit-field extract yields q.
template <int B>
__host__ __device__ constexpr uint32_t code_msb_mask(int word)
{
    uint32_t m = 0;
    for (int j = 0; j < kChunk; ++j) {
        const int pos = j * B + B - 1;
        if ((pos >> 5) == word) m |= 1u << (pos & 31);
    }
    return m;
}

// Signed code j (0..31) of a chunk whose words were XOR-ed with code_msb_mask.
// j is a compile-time constant after unrolling, so this is a bfe_i32 or an
// alignbit + bfe_i32.
template <int B>
__device__ __forceinline__ int32_t chunk_code_signed(const uint32_t* w, int j)
{
    const int pos = j * B;
    const int wi = pos >> 5;
    const int off = pos & 31;
    uint32_t v;
    if (off + B <= 32) {
        v = w[wi] >> off;
    } else {
        v = __builtin_amdgcn_alignbit(w[wi + 1], w[wi], off);  // bits [off, off+32) of {w1:w0}
    }
    return ((int32_t)(v << (32 - B))) >> (32 - B);
}

// Unsigned (offset-binary) code j of an unmodified chunk.
template <int B>
__device__ __forceinline__ uint32_t chunk_code_unsigned(const uint32_t* w, int j)
{
    const int pos = j * B;
    const int wi = pos >> 5;
    const int off = pos & 31;
    uint32_t v;
    if (off + B <= 32) {
        v = w[wi] >> off;
    } else {
        v = __builtin_amdgcn_alignbit(w[wi + 1], w[wi], off);  // bits [off, off+32) of {w1:w0}
    }
    return v & ((1u << B) - 1u);
}

typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x3_a4 __attribute__((ext_vector_type(3), aligned(4)));
typedef uint32_t u32x2_a4 __attribute__((ext_vector_type(2), aligned(4)));

// Loads B consecutive words with as few instructions as possible (dwordx4
// pieces, then x3/x2/x1); global memory only needs dword alignment for these.
template <int B>
__device__ __forceinline__ void load_words(const uint32_t* __restrict__ p, uint32_t* w)
{
#pragma unroll
    for (int i = 0; i + 4 <= B; i += 4) {
        const u32x4_a4 v = *reinterpret_cast<const u32x4_a4*>(p + i);
        w[i] = v.x;
        w[i + 1] = v.y;
        w[i + 2] = v.z;
        w[i + 3] = v.w;
    }
    constexpr int r = B & 3;
    constexpr int o = B - r;
    if (r == 3) {
        const u32x3_a4 v = *reinterpret_cast<const u32x3_a4*>(p + o);
        w[o] = v.x;
        w[o + 1] = v.y;
        w[o + 2] = v.z;
    } else if (r == 2) {
        const u32x2_a4 v = *reinterpret_cast<const u32x2_a4*>(p + o);
        w[o] = v.x;
        w[o + 1] = v.y;
    } else if (r == 1) {
        w[o] = p[o];
    }
}

// Stores B consecutive words with as few instructions as possible (the
// counterpart of load_words).
template <int B>
__device__ __forceinline__ void store_words(uint32_t* __restrict__ p, const uint32_t* w)
{
#pragma unroll
    for (int i = 0; i + 4 <= B; i += 4)
        *reinterpret_cast<u32x4_a4*>(p + i) = (u32x4_a4){w[i], w[i + 1], w[i + 2], w[i + 3]};
    constexpr int r = B & 3;
    constexpr int o = B - r;
    if (r == 3) {
        *reinterpret_cast<u32x3_a4*>(p + o) = (u32x3_a4){w[o], w[o + 1], w[o + 2]};
    } else if (r == 2) {
        *reinterpret_cast<u32x2_a4*>(p + o) = (u32x2_a4){w[o], w[o + 1]};
    } else if (r == 1) {
        p[o] = w[o];
    }
}

// Loads the B words of chunk c of a packed row.  Words at or beyond row_words
// (possible only in a row's last chunk) read as zero.
template <int B>
__device__ __forceinline__ void load_chunk_words(const uint32_t* __restrict__ row, int64_t c,
                                                 int64_t row_words, uint32_t* w)
{
    const int64_t base = c * B;
    if (base + B <= row_words) {
        load_words<B>(row + base, w);
    } else {
#pragma unroll
        for (int i = 0; i < B; ++i) w[i] = (base + i < row_words) ? row[base + i] : 0u;
    }
}

// Wave-wide reductions through cross-lane shuffles.
__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const uint32_t t = (uint32_t)__shfl_xor((int)v, o, kWave);
        v = t > v ? t : v;
    }
    return v;
}

// Zero points of the asymmetric scheme, for the products' epilogues.  Codes
// are stored unsigned, u = rint(w / s) + z[n]; every product kernel sums
// x * (u - 2^(b-1)) (the two's-complement view of the code), so adding
// (2^(b-1) - z[n]) * sum_k x[m, k] gives sum_k x * (u - z[n]).  The product
// kernels take the type as a template parameter: NoZeroPoints (the symmetric
// scheme) adds nothing and compiles to the plain epilogue.
// Each type gives coef<B>(n), read once per output column before any store
// (a load issued after the stores would wait for all of them), and
// apply(v, coef, m) = v + coef * sum_k x[m, k].
struct NoZeroPoints {
    template <int B>
    __device__ __forceinline__ float coef(int64_t) const
    {
        return 0.0f;
    }
    __device__ __forceinline__ float apply(float v, float, int64_t) const { return v; }
};

struct ZeroPoints {
    const int32_t* zeros;  // [N]
    const float* xsum;     // [M]: sum_k x[m, k]

    template <int B>
    __device__ __forceinline__ float coef(int64_t n) const
    {
        return (float)((1 << (B - 1)) - zeros[n]);
    }
    __device__ __forceinline__ float apply(float v, float c, int64_t m) const
    {
        return fmaf(c, xsum[m], v);
    }
};

// ZeroPoints with one tile's activation sums staged in LDS (row m at
// xs[m - m0]), for epilogues that read each row's sum many times.
struct TileZeroPoints {
    const int32_t* zeros;
    const float* xs;
    int64_t m0;

    template <int B>
    __device__ __forceinline__ float coef(int64_t n) const
    {
        return (float)((1 << (B - 1)) - zeros[n]);
    }
    __device__ __forceinline__ float apply(float v, float c, int64_t m) const
    {
        return fmaf(c, xs[m - m0], v);
    }
};

// Group-wise scales for the pipelined 128-row GEMM and the resident-x GEMV:
// one scale per row and group of `group` codes (scales [N, G]).  The kernels
// accumulate a group's (or a chunk's) products apart and add them in scaled,
// so the epilogue applies no row scale.
struct GroupScales {
    const float* scales;
    int64_t G;
    int64_t group;  // codes per group, a power of two >= 32

    // no zero points: the epilogue adds nothing
    template <int B>
    __device__ __forceinline__ float coef(int64_t) const
    {
        return 0.0f;
    }
    __device__ __forceinline__ float apply(float v, float, int64_t) const { return v; }
};

template <class P>
struct is_group_scales {
    static constexpr bool value = false;
};
template <>
struct is_group_scales<GroupScales> {
    static constexpr bool value = true;
};

// Stage rows [m0, m0 + rows) of the activation sums into `lds` (a buffer the
// workgroup no longer uses) between two barriers; every thread of the
// workgroup must call it.  The symmetric scheme stages nothing.
__device__ __forceinline__ NoZeroPoints stage_tile_zero_points(NoZeroPoints, float*, int64_t,
                                                               int64_t, int)
{
    return {};
}

__device__ __forceinline__ NoZeroPoints stage_tile_zero_points(GroupScales, float*, int64_t, int64_t,
                                                               int)
{
    return {};
}

__device__ __forceinline__ TileZeroPoints stage_tile_zero_points(ZeroPoints zp, float* lds,
                                                                 int64_t m0, int64_t M, int rows)
{
    __syncthreads();
    for (int i = threadIdx.x; i < rows; i += blockDim.x)
        lds[i] = m0 + i < M ? zp.xsum[m0 + i] : 0.0f;
    __syncthreads();
    return {zp.zeros, lds, m0};
}

}  // namespace dq
