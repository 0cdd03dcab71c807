// Code expansion for the matrix-core GEMM: 8 consecutive codes of a chunk
// (32 codes in B whole words) become one exact bf16x8 MFMA operand.
#pragma once

#include "common.hpp"

namespace dq {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
typedef float f32x2v_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t bf16x2_bits(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2v_t){lo, hi}, bf16x2v_t));
}

__device__ __forceinline__ bf16x8_t bf16x8_from_words(uint32_t a, uint32_t b, uint32_t c, uint32_t d)
{
    typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
    return __builtin_bit_cast(bf16x8_t, (u32x4_t){a, b, c, d});
}

__device__ __forceinline__ float sbyte_f(uint32_t w, int j) { return (float)(int8_t)(w >> (8 * j)); }

// Factor by which expand8<B> scales the codes (converted from the top bits of a
// byte): 16 for symmetric B = 4, else 1.  The kernels divide their sums by it.
template <int B, bool kAsym = false>
__host__ __device__ constexpr float expand8_scale() { return (!kAsym && B == 4) ? 16.0f : 1.0f; }

// Whether a code needs two bf16 operands: symmetric |q| <= 2^(B-1) - 1 is exact
// in bf16 up to B = 9, asymmetric |u - z| <= 2^B - 1 up to B = 8.
template <int B, bool kAsym>
__host__ __device__ constexpr bool split_codes() { return kAsym ? B >= 9 : B >= 10; }

// Codes 8t .. 8t+7 of a chunk (raw words w) as exact bf16: for B <= 9 one
// operand (q, or 16q for B = 4); for B >= 10 two operands, bf16(q & ~63) =
// bf16(64 * (q >> 6)) and bf16(q & 63), whose sum is q.
template <int B>
__device__ __forceinline__ void expand8(const uint32_t (&w)[B], int t, bf16x8_t& hi, bf16x8_t& lo)
{
    if constexpr (B == 8) {
        const uint32_t v0 = w[2 * t] ^ 0x80808080u, v1 = w[2 * t + 1] ^ 0x80808080u;
        hi = bf16x8_from_words(bf16x2_bits(sbyte_f(v0, 0), sbyte_f(v0, 1)),
                               bf16x2_bits(sbyte_f(v0, 2), sbyte_f(v0, 3)),
                               bf16x2_bits(sbyte_f(v1, 0), sbyte_f(v1, 1)),
                               bf16x2_bits(sbyte_f(v1, 2), sbyte_f(v1, 3)));
    } else if constexpr (B == 4) {
        const uint32_t v = w[t] ^ 0x88888888u;
        const uint32_t ev = (v << 4) & 0xf0f0f0f0u;  // codes 8t+2j, times 16
        const uint32_t od = v & 0xf0f0f0f0u;         // codes 8t+2j+1, times 16
        hi = bf16x8_from_words(bf16x2_bits(sbyte_f(ev, 0), sbyte_f(od, 0)),
                               bf16x2_bits(sbyte_f(ev, 1), sbyte_f(od, 1)),
                               bf16x2_bits(sbyte_f(ev, 2), sbyte_f(od, 2)),
                               bf16x2_bits(sbyte_f(ev, 3), sbyte_f(od, 3)));
    } else {
        uint32_t v[B];
#pragma unroll
        for (int i = 0; i < B; ++i) v[i] = w[i] ^ code_msb_mask<B>(i);
        int32_t q[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) q[e] = chunk_code_signed<B>(v, 8 * t + e);
        if constexpr (B <= 9) {
            hi = bf16x8_from_words(bf16x2_bits((float)q[0], (float)q[1]),
                                   bf16x2_bits((float)q[2], (float)q[3]),
                                   bf16x2_bits((float)q[4], (float)q[5]),
                                   bf16x2_bits((float)q[6], (float)q[7]));
        } else {
            hi = bf16x8_from_words(bf16x2_bits((float)(q[0] & ~63), (float)(q[1] & ~63)),
                                   bf16x2_bits((float)(q[2] & ~63), (float)(q[3] & ~63)),
                                   bf16x2_bits((float)(q[4] & ~63), (float)(q[5] & ~63)),
                                   bf16x2_bits((float)(q[6] & ~63), (float)(q[7] & ~63)));
            lo = bf16x8_from_words(bf16x2_bits((float)(q[0] & 63), (float)(q[1] & 63)),
                                   bf16x2_bits((float)(q[2] & 63), (float)(q[3] & 63)),
                                   bf16x2_bits((float)(q[4] & 63), (float)(q[5] & 63)),
                                   bf16x2_bits((float)(q[6] & 63), (float)(q[7] & 63)));
        }
    }
}

// Asymmetric codes: q = u - z for codes 8t .. 8t+7 of a chunk (raw unsigned
// words w), |q| <= 2^B - 1.  B <= 8: one exact operand.  B >= 9: with
// S = B - 8, bf16(q & ~(2^S - 1)) = bf16(2^S * (q >> S)), q >> S in
// [-256, 255], and bf16(q & (2^S - 1)) in [0, 127]; both exact, summing to q.
template <int B>
__device__ __forceinline__ void expand8_asym(const uint32_t (&w)[B], int32_t z, int t, bf16x8_t& hi,
                                             bf16x8_t& lo)
{
    int32_t q[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) q[e] = (int32_t)chunk_code_unsigned<B>(w, 8 * t + e) - z;
    if constexpr (B <= 8) {
        hi = bf16x8_from_words(bf16x2_bits((float)q[0], (float)q[1]),
                               bf16x2_bits((float)q[2], (float)q[3]),
                               bf16x2_bits((float)q[4], (float)q[5]),
                               bf16x2_bits((float)q[6], (float)q[7]));
    } else {
        constexpr int32_t kLo = (1 << (B - 8)) - 1;
        hi = bf16x8_from_words(bf16x2_bits((float)(q[0] & ~kLo), (float)(q[1] & ~kLo)),
                               bf16x2_bits((float)(q[2] & ~kLo), (float)(q[3] & ~kLo)),
                               bf16x2_bits((float)(q[4] & ~kLo), (float)(q[5] & ~kLo)),
                               bf16x2_bits((float)(q[6] & ~kLo), (float)(q[7] & ~kLo)));
        lo = bf16x8_from_words(bf16x2_bits((float)(q[0] & kLo), (float)(q[1] & kLo)),
                               bf16x2_bits((float)(q[2] & kLo), (float)(q[3] & kLo)),
                               bf16x2_bits((float)(q[4] & kLo), (float)(q[5] & kLo)),
                               bf16x2_bits((float)(q[6] & kLo), (float)(q[7] & kLo)));
    }
}

// expand8 for either scheme: z is the row's zero point (ignored when symmetric).
template <int B, bool kAsym>
__device__ __forceinline__ void expand8z(const uint32_t (&w)[B], int32_t z, int t, bf16x8_t& hi,
                                         bf16x8_t& lo)
{
    if constexpr (kAsym)
        expand8_asym<B>(w, z, t, hi, lo);
    else
        expand8<B>(w, t, hi, lo);
}

typedef uint32_t u32x4v_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x3v_t __attribute__((ext_vector_type(3)));
typedef uint32_t u32x2v_t __attribute__((ext_vector_type(2)));

// Buffer resource over `bytes` bytes at `base` (raw buffer: byte offsets,
// dword accesses, out-of-range reads return 0).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// A buffer is passed around as (base, bytes); the resource descriptor is built
// inside the device-only helpers below (the compiler hoists it out of loops),
// so kernel bodies never name the target-specific descriptor type.
struct BufRef {
    const void* base;
    uint32_t bytes;
};

// A BufRef whose fields are provably wave-uniform (scalar registers), so the
// descriptor is built once with scalar ops and hoisted out of loops.
__device__ __forceinline__ BufRef uniform_buf(const void* base, uint32_t bytes)
{
    const uint64_t v = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return BufRef{reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo),
                  (uint32_t)__builtin_amdgcn_readfirstlane(bytes)};
}

// B consecutive words at byte offset voff + soff of a buffer, in as few
// buffer loads as possible (dwordx4 pieces, then x3/x2/x1).
template <int B>
__device__ __forceinline__ void buf_load_words(BufRef buf, uint32_t voff, uint32_t soff,
                                               uint32_t (&w)[B])
{
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(buf.base, buf.bytes);
#pragma unroll
    for (int i = 0; i + 4 <= B; i += 4) {
        const u32x4v_t v = __builtin_amdgcn_raw_buffer_load_b128(rs, voff + 4 * i, soff, 0);
        w[i] = v.x;
        w[i + 1] = v.y;
        w[i + 2] = v.z;
        w[i + 3] = v.w;
    }
    constexpr int r = B & 3;
    constexpr int o = B - r;
    if constexpr (r == 3) {
        const u32x3v_t v = __builtin_amdgcn_raw_buffer_load_b96(rs, voff + 4 * o, soff, 0);
        w[o] = v.x;
        w[o + 1] = v.y;
        w[o + 2] = v.z;
    } else if constexpr (r == 2) {
        const u32x2v_t v = __builtin_amdgcn_raw_buffer_load_b64(rs, voff + 4 * o, soff, 0);
        w[o] = v.x;
        w[o + 1] = v.y;
    } else if constexpr (r == 1) {
        w[o] = __builtin_amdgcn_raw_buffer_load_b32(rs, voff + 4 * o, soff, 0);
    }
}

__device__ __forceinline__ u32x4v_t buf_load_b128(BufRef buf, uint32_t voff, uint32_t soff)
{
    return __builtin_amdgcn_raw_buffer_load_b128(make_rsrc(buf.base, buf.bytes), voff, soff, 0);
}

// One fp32 per lane to byte offset voff + soff of a buffer, as a streaming
// (nontemporal) store.
__device__ __forceinline__ void buf_store_f32_nt(BufRef buf, float v, uint32_t voff, uint32_t soff)
{
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), make_rsrc(buf.base, buf.bytes),
                                          voff, soff, 2 /* nt */);
}

// 16 bytes per lane from byte offset voff + soff of a buffer straight into LDS
// at lds + 16 * lane (buffer_load_dwordx4 ... lds).
__device__ __forceinline__ void buf_load_lds16(BufRef buf, void* lds, uint32_t voff, uint32_t soff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(buf.base, buf.bytes),
                                             (__attribute__((address_space(3))) void*)lds, 16, voff,
                                             soff, 0, 0);
}

// 4 bytes per lane from byte offset voff + soff of a buffer straight into LDS
// at lds + 4 * lane (buffer_load_dword ... lds).
__device__ __forceinline__ void buf_load_lds4(BufRef buf, void* lds, uint32_t voff, uint32_t soff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(buf.base, buf.bytes),
                                             (__attribute__((address_space(3))) void*)lds, 4, voff,
                                             soff, 0, 0);
}

}  // namespace dq
