// Host-side launchers of the kernels (internal to the library; the public
// surface is the C ABI in include/dq.h).  Arguments are validated by the
// caller; each launcher only picks a configuration and enqueues on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.hpp"

namespace dq {

// nonfinite: optional count of rows holding a NaN or an infinity (zeroed first)
hipError_t launch_quantize_pack(const void* w, bool bf16, int64_t N, int64_t K, int bits,
                                uint32_t* packed, float* scales, uint32_t* nonfinite,
                                hipStream_t stream);
hipError_t launch_quantize_pack_sumsq(const void* w, bool bf16, int64_t N, int64_t K, int bits,
                                      uint32_t* packed, float* scales, double* row_sumsq,
                                      double* matrix_sumsq, hipStream_t stream);
hipError_t launch_row_sumsq(const void* w, bool bf16, int64_t N, int64_t K, double* row_sumsq,
                            double* matrix_sumsq, hipStream_t stream);
// zeros: null for the symmetric scheme (q = u - 2^(b-1)), else q = u - zeros[n];
// group: 0 for one scale per row, else scales [N, ceil(K / group)]
hipError_t launch_unpack(const uint32_t* packed, const float* scales, const int32_t* zeros,
                         int64_t group, int64_t N, int64_t K, int bits, int32_t* q_out,
                         float* w_out, hipStream_t stream);
hipError_t launch_quantize_pack_group(const void* w, bool bf16, int64_t N, int64_t K, int bits,
                                      int64_t group, uint32_t* packed, float* scales,
                                      hipStream_t stream);
hipError_t launch_gemv_group(const uint16_t* x, int64_t M, const uint32_t* packed,
                             const float* scales, int64_t N, int64_t K, int bits, int64_t group,
                             float* y, hipStream_t stream);
hipError_t launch_gemm_group(const uint16_t* x, int64_t M, const uint32_t* packed,
                             const float* scales, int64_t N, int64_t K, int bits, int64_t group,
                             float* y, hipStream_t stream);
// zeros: the asymmetric scheme's zero points [N] (q = u - zeros[n]); null for
// the symmetric scheme (q = u - 2^(b-1)).
hipError_t launch_gemv(const uint16_t* x, int64_t M, const uint32_t* packed, const float* scales,
                       int64_t N, int64_t K, int bits, float* y, const int32_t* zeros,
                       hipStream_t stream);
hipError_t launch_gemm(const uint16_t* x, int64_t M, const uint32_t* packed, const float* scales,
                       int64_t N, int64_t K, int bits, float* y, const int32_t* zeros,
                       hipStream_t stream);
// One matrix of a batched decode product (arguments as for launch_gemv).
struct GemvItem {
    const uint16_t* x;
    const uint32_t* packed;
    const float* scales;
    float* y;
    int64_t N;
    int64_t K;
    int bits;
    int64_t group;          // 0: a scale per row; else codes per group (scales [N, ceil(K / group)])
    const int32_t* zeros;  // nullptr, or [N] zero points (asymmetric codes; group 0)
};
constexpr int kGemvBatchMax = 32;  // items per call (DQ_GEMV_BATCH_MAX)
// Whether an item of this shape joins the single launch (else it gets its own).
bool gemv_batch_eligible(int64_t M, int64_t K);
// rows per workgroup of the matrix-core GEMV (3 <= M <= 16) for an N x K matrix
int gemv_mfma_rows(int64_t N, int64_t K);
// Symmetric per-row products of `count` matrices sharing M (<= 2 for the
// single launch; items outside it run one launch each).
hipError_t launch_gemv_batched(const GemvItem* items, int count, int64_t M, hipStream_t stream);
hipError_t launch_quantize_pack_asym(const void* w, bool bf16, int64_t N, int64_t K, int bits,
                                     uint32_t* packed, float* scales, int32_t* zeros,
                                     hipStream_t stream);
hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* partial, int64_t nparts,
                              hipStream_t stream);

// DQ_OK for hipSuccess; otherwise keeps the HIP message for dq_last_error on
// this thread and returns DQ_ERR_HIP (defined with the C ABI in api.cpp).
int32_t record_hip_error(hipError_t e);

// Expands CALL(B) for the run-time bit width, one template instance per width.
#define DQ_BITS_SWITCH(bits, CALL)                                                                \
    switch (bits) {                                                                               \
    case 2: return CALL(2);                                                                       \
    case 3: return CALL(3);                                                                       \
    case 4: return CALL(4);                                                                       \
    case 5: return CALL(5);                                                                       \
    case 6: return CALL(6);                                                                       \
    case 7: return CALL(7);                                                                       \
    case 8: return CALL(8);                                                                       \
    case 9: return CALL(9);                                                                       \
    case 10: return CALL(10);                                                                     \
    case 11: return CALL(11);                                                                     \
    case 12: return CALL(12);                                                                     \
    case 13: return CALL(13);                                                                     \
    case 14: return CALL(14);                                                                     \
    case 15: return CALL(15);                                                                     \
    default: return hipErrorInvalidValue;                                                         \
    }

}  // namespace dq
