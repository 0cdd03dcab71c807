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

#include <utility>

namespace dq {

// f(std::integral_constant<int, 0>{}), ..., f(std::integral_constant<int, N - 1>{})
// in order: a loop over pipeline stages whose index stays a compile-time
// constant, so each stage's registers are named statically.
template <typename F, int... I>
__device__ __forceinline__ void static_for_seq(F&& f, std::integer_sequence<int, I...>)
{
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f)
{
    static_for_seq(f, std::make_integer_sequence<int, N>{});
}

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

// Sum over the 64 lanes of a wave, returned to every lane, in a fixed order
// (so the same inputs give the same bits on every call).  DPP steps: within
// each row of 16 lanes an inclusive prefix sum by row_shr 1, 2, 4, 8 (lanes
// shifted in from outside the row read 0), which leaves each row's total in
// its lane 15; row_bcast:15 adds row 0's total into row 1 and row 2's into
// row 3, row_bcast:31 adds rows 0 + 1 into rows 2 and 3; lane 63 then holds
// the wave's total, which a readlane hands to every lane.  Seven VALU
// instructions instead of the shuffle form's bounds-checked permutes.
// v + (v moved by DPP control kCtrl in the rows of kRowMask; 0 elsewhere)
template <int kCtrl, int kRowMask>
__device__ __forceinline__ float dpp_add(float v)
{
    const int s = __builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, kRowMask, 0xf, true);
    return v + __int_as_float(s);
}

__device__ __forceinline__ float wave_sum(float v)
{
    v = dpp_add<0x111, 0xf>(v);  // row_shr:1
    v = dpp_add<0x112, 0xf>(v);  // row_shr:2
    v = dpp_add<0x114, 0xf>(v);  // row_shr:4
    v = dpp_add<0x118, 0xf>(v);  // row_shr:8
    v = dpp_add<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
    v = dpp_add<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Sums over the two halves of a wave (lanes 0 .. 31 and 32 .. 63), in a fixed
// order: the first five steps of wave_sum leave the first half's total in
// lane 31 and the second half's in lane 63.
__device__ __forceinline__ void half_sums(float v, float& lo, float& hi)
{
    v = dpp_add<0x111, 0xf>(v);  // row_shr:1
    v = dpp_add<0x112, 0xf>(v);  // row_shr:2
    v = dpp_add<0x114, 0xf>(v);  // row_shr:4
    v = dpp_add<0x118, 0xf>(v);  // row_shr:8
    v = dpp_add<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
    lo = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 31));
    hi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
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

// Zero points of the asymmetric scheme.  Codes are stored unsigned,
// u = rint(w / s) + z[n], and dequantize as q = u - z[n].  The product kernels
// take the scheme as a template type and, for ZeroPoints, subtract the row's
// zero point from every code before it meets x, so each product x * (u - z)
// is formed exactly, as in the symmetric scheme (where q = u - 2^(b-1)).
// Nothing is folded into an activation-sum term afterwards: such a fold adds
// two large terms that cancel when most codes equal z.
//
// |u - z| < 2^b, one bit more than a symmetric code, so the asymmetric
// kernels treat b = 9 like the wide codes (fp32 FMAs, or two exact bf16
// halves on the matrix cores).
struct NoZeroPoints {
    static constexpr bool kAsym = false;
    __device__ __forceinline__ int32_t zero(int64_t) const { return 0; }
};

struct ZeroPoints {
    static constexpr bool kAsym = true;
    const int32_t* zeros;  // [N]
    __device__ __forceinline__ int32_t zero(int64_t n) const { return zeros[n]; }
};

// Group-wise scales for the pipelined 128-row GEMM and the resident-x GEMV:
// one scale per row and group of `group` codes (scales [N, G]).  The kernels
// accumulate a group's (or a chunk's) products apart and add them in scaled,
// so the epilogue applies no row scale.
struct GroupScales {
    const float* scales;
    int64_t G;
    int64_t group;  // codes per group, a power of two >= 32

    static constexpr bool kAsym = false;
    __device__ __forceinline__ int32_t zero(int64_t) const { return 0; }
};

template <class P>
struct is_group_scales {
    static constexpr bool value = false;
};
template <>
struct is_group_scales<GroupScales> {
    static constexpr bool value = true;
};

}  // namespace dq
