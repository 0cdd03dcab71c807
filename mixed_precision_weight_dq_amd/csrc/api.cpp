// C ABI of the library (declared in include/dq.h): argument validation on the
// host, then the kernel launches on the caller's stream.  No allocation, no
// synchronisation, no state beyond the per-thread text of the last HIP error.
// (The host-only allocation entry points live in recipe.cpp, the file format's
// writer and parser in packfile.cpp.)
#include "../../include/dq.h"

#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstring>

#include "launch.hpp"

namespace {

thread_local char g_last_error[256] = "";

dq_status hip_status(hipError_t e)
{
    if (e == hipSuccess) return DQ_OK;
    std::snprintf(g_last_error, sizeof g_last_error, "%s: %s", hipGetErrorName(e),
                  hipGetErrorString(e));
    return DQ_ERR_HIP;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

dq_status check_common(int64_t N, int64_t K, int32_t bits)
{
    if (bits < DQ_MIN_BITS || bits > DQ_MAX_BITS) return DQ_ERR_BITS;
    if (N < 1 || N > 0x7fffffffLL || K < 1 || K > DQ_MAX_K) return DQ_ERR_SHAPE;
    return DQ_OK;
}

// group sizes: powers of two from one chunk (32 codes) to 2048
bool valid_group(int64_t g) { return g >= 32 && g <= DQ_MAX_GROUP && (g & (g - 1)) == 0; }

}  // namespace

int32_t dq::record_hip_error(hipError_t e) { return hip_status(e); }

extern "C" {

size_t dq_packed_row_bytes(int64_t K, int32_t bits)
{
    if (bits < DQ_MIN_BITS || bits > DQ_MAX_BITS || K < 1 || K > DQ_MAX_K) return 0;
    return (size_t)dq::packed_row_words(K, bits) * 4;
}

dq_status dq_quantize_pack(const void* w, int32_t w_dtype, int64_t N, int64_t K, int32_t bits,
                           uint32_t* packed, float* scales, uint32_t* nonfinite_rows,
                           void* stream)
{
    if (!w || !packed || !scales) return DQ_ERR_NULL;
    dq_status st = check_common(N, K, bits);
    if (st != DQ_OK) return st;
    if (w_dtype != DQ_F32 && w_dtype != DQ_BF16) return DQ_ERR_DTYPE;
    if (!aligned(w, 16) || !aligned(packed, 16) || !aligned(scales, 4) ||
        !aligned(nonfinite_rows, 4))
        return DQ_ERR_ALIGN;
    return hip_status(dq::launch_quantize_pack(w, w_dtype == DQ_BF16, N, K, bits, packed, scales,
                                               nonfinite_rows, static_cast<hipStream_t>(stream)));
}

dq_status dq_quantize_pack_sumsq(const void* w, int32_t w_dtype, int64_t N, int64_t K,
                                 int32_t bits, uint32_t* packed, float* scales,
                                 double* row_sumsq, double* matrix_sumsq, void* stream)
{
    if (!w || !packed || !scales || !row_sumsq) return DQ_ERR_NULL;
    dq_status st = check_common(N, K, bits);
    if (st != DQ_OK) return st;
    if (w_dtype != DQ_F32 && w_dtype != DQ_BF16) return DQ_ERR_DTYPE;
    if (!aligned(w, 16) || !aligned(packed, 16) || !aligned(scales, 4) || !aligned(row_sumsq, 8) ||
        !aligned(matrix_sumsq, 8))
        return DQ_ERR_ALIGN;
    return hip_status(dq::launch_quantize_pack_sumsq(w, w_dtype == DQ_BF16, N, K, bits, packed,
                                                     scales, row_sumsq, matrix_sumsq,
                                                     static_cast<hipStream_t>(stream)));
}

dq_status dq_row_sumsq(const void* w, int32_t w_dtype, int64_t N, int64_t K, double* row_sumsq,
                       double* matrix_sumsq, void* stream)
{
    if (!w || !row_sumsq) return DQ_ERR_NULL;
    if (N < 1 || N > 0x7fffffffLL || K < 1 || K > DQ_MAX_K) return DQ_ERR_SHAPE;
    if (w_dtype != DQ_F32 && w_dtype != DQ_BF16) return DQ_ERR_DTYPE;
    if (!aligned(w, 16) || !aligned(row_sumsq, 8) || !aligned(matrix_sumsq, 8))
        return DQ_ERR_ALIGN;
    return hip_status(dq::launch_row_sumsq(w, w_dtype == DQ_BF16, N, K, row_sumsq, matrix_sumsq,
                                           static_cast<hipStream_t>(stream)));
}

dq_status dq_unpack(const uint32_t* packed, const float* scales, int64_t N, int64_t K,
                    int32_t bits, int32_t* q_out, float* w_out, void* stream)
{
    if (!packed || (!q_out && !w_out) || (w_out && !scales)) return DQ_ERR_NULL;
    dq_status st = check_common(N, K, bits);
    if (st != DQ_OK) return st;
    if (!aligned(packed, 16) || !aligned(scales, 4) || !aligned(q_out, 4) || !aligned(w_out, 4))
        return DQ_ERR_ALIGN;
    return hip_status(dq::launch_unpack(packed, scales, nullptr, 0, N, K, bits, q_out, w_out,
                                        static_cast<hipStream_t>(stream)));
}

dq_status dq_quantize_pack_asym(const void* w, int32_t w_dtype, int64_t N, int64_t K, int32_t bits,
                                uint32_t* packed, float* scales, int32_t* zeros, void* stream)
{
    if (!w || !packed || !scales || !zeros) return DQ_ERR_NULL;
    dq_status st = check_common(N, K, bits);
    if (st != DQ_OK) return st;
    if (w_dtype != DQ_F32 && w_dtype != DQ_BF16) return DQ_ERR_DTYPE;
    if (!aligned(w, 16) || !aligned(packed, 16) || !aligned(scales, 4) || !aligned(zeros, 4))
        return DQ_ERR_ALIGN;
    return hip_status(dq::launch_quantize_pack_asym(w, w_dtype == DQ_BF16, N, K, bits, packed,
                                                    scales, zeros,
                                                    static_cast<hipStream_t>(stream)));
}

dq_status dq_unpack_asym(const uint32_t* packed, const float* scales, const int32_t* zeros,
                         int64_t N, int64_t K, int32_t bits, int32_t* q_out, float* w_out,
                         void* stream)
{
    if (!packed || !zeros || (!q_out && !w_out) || (w_out && !scales)) return DQ_ERR_NULL;
    dq_status st = check_common(N, K, bits);
    if (st != DQ_OK) return st;
    if (!aligned(packed, 16) || !aligned(scales, 4) || !aligned(zeros, 4) || !aligned(q_out, 4) ||
        !aligned(w_out, 4))
        return DQ_ERR_ALIGN;
    return hip_status(dq::launch_unpack(packed, scales, zeros, 0, N, K, bits, q_out, w_out,
                                        static_cast<hipStream_t>(stream)));
}

dq_status dq_quantize_pack_group(const void* w, int32_t w_dtype, int64_t N, int64_t K,
                                 int32_t bits, int64_t group, uint32_t* packed, float* scales,
                                 void* stream)
{
    if (!w || !packed || !scales) return DQ_ERR_NULL;
    dq_status st = check_common(N, K, bits);
    if (st != DQ_OK) return st;
    if (!valid_group(group)) return DQ_ERR_SHAPE;
    if (w_dtype != DQ_F32 && w_dtype != DQ_BF16) return DQ_ERR_DTYPE;
    if (!aligned(w, 16) || !aligned(packed, 16) || !aligned(scales, 4)) return DQ_ERR_ALIGN;
    return hip_status(dq::launch_quantize_pack_group(w, w_dtype == DQ_BF16, N, K, bits, group,
                                                     packed, scales,
                                                     static_cast<hipStream_t>(stream)));
}

dq_status dq_unpack_group(const uint32_t* packed, const float* scales, int64_t N, int64_t K,
                          int32_t bits, int64_t group, int32_t* q_out, float* w_out, void* stream)
{
    if (!packed || (!q_out && !w_out) || (w_out && !scales)) return DQ_ERR_NULL;
    dq_status st = check_common(N, K, bits);
    if (st != DQ_OK) return st;
    if (!valid_group(group)) return DQ_ERR_SHAPE;
    if (!aligned(packed, 16) || !aligned(scales, 4) || !aligned(q_out, 4) || !aligned(w_out, 4))
        return DQ_ERR_ALIGN;
    return hip_status(dq::launch_unpack(packed, scales, nullptr, group, N, K, bits, q_out, w_out,
                                        static_cast<hipStream_t>(stream)));
}

dq_status dq_gemv_group(const uint16_t* x, int64_t M, const uint32_t* packed, const float* scales,
                        int64_t N, int64_t K, int32_t bits, int64_t group, float* y, void* stream)
{
    if (!x || !packed || !scales || !y) return DQ_ERR_NULL;
    dq_status st = check_common(N, K, bits);
    if (st != DQ_OK) return st;
    if (M < 1 || M > DQ_GEMV_MAX_M || !valid_group(group)) return DQ_ERR_SHAPE;
    if (!aligned(x, 16) || !aligned(packed, 16) || !aligned(scales, 4) || !aligned(y, 4))
        return DQ_ERR_ALIGN;
    return hip_status(dq::launch_gemv_group(x, M, packed, scales, N, K, bits, group, y,
                                            static_cast<hipStream_t>(stream)));
}

dq_status dq_gemm_group(const uint16_t* x, int64_t M, const uint32_t* packed, const float* scales,
                        int64_t N, int64_t K, int32_t bits, int64_t group, float* y, void* stream)
{
    if (!x || !packed || !scales || !y) return DQ_ERR_NULL;
    dq_status st = check_common(N, K, bits);
    if (st != DQ_OK) return st;
    if (M < 1 || M > 0x7fffffffLL || !valid_group(group)) return DQ_ERR_SHAPE;
    if (!aligned(x, 16) || !aligned(packed, 16) || !aligned(scales, 4) || !aligned(y, 4))
        return DQ_ERR_ALIGN;
    return hip_status(dq::launch_gemm_group(x, M, packed, scales, N, K, bits, group, y,
                                            static_cast<hipStream_t>(stream)));
}

dq_status dq_gemv(const uint16_t* x, int64_t M, const uint32_t* packed, const float* scales,
                  int64_t N, int64_t K, int32_t bits, float* y, void* stream)
{
    if (!x || !packed || !scales || !y) return DQ_ERR_NULL;
    dq_status st = check_common(N, K, bits);
    if (st != DQ_OK) return st;
    if (M < 1 || M > DQ_GEMV_MAX_M) return DQ_ERR_SHAPE;
    if (!aligned(x, 16) || !aligned(packed, 16) || !aligned(scales, 4) || !aligned(y, 4))
        return DQ_ERR_ALIGN;
    return hip_status(dq::launch_gemv(x, M, packed, scales, N, K, bits, y, nullptr,
                                      static_cast<hipStream_t>(stream)));
}

dq_status dq_gemv_batched(const dq_gemv_item* items, int32_t count, int64_t M, void* stream)
{
    if (!items) return DQ_ERR_NULL;
    if (count < 1 || count > DQ_GEMV_BATCH_MAX || M < 1 || M > DQ_GEMV_MAX_M) return DQ_ERR_SHAPE;
    static_assert(DQ_GEMV_BATCH_MAX == dq::kGemvBatchMax, "batch size");
    dq::GemvItem g[DQ_GEMV_BATCH_MAX];
    for (int32_t i = 0; i < count; ++i) {  // every item is checked before anything is enqueued
        const dq_gemv_item& it = items[i];
        if (!it.x || !it.packed || !it.scales || !it.y) return DQ_ERR_NULL;
        const dq_status st = check_common(it.N, it.K, it.bits);
        if (st != DQ_OK) return st;
        if (it.group != 0 && (!valid_group(it.group) || it.zeros)) return DQ_ERR_SHAPE;
        if (!aligned(it.x, 16) || !aligned(it.packed, 16) || !aligned(it.scales, 4) ||
            !aligned(it.y, 4) || !aligned(it.zeros, 4))
            return DQ_ERR_ALIGN;
        g[i] = dq::GemvItem{it.x, it.packed, it.scales, it.y, it.N, it.K, it.bits, it.group, it.zeros};
    }
    return hip_status(dq::launch_gemv_batched(g, count, M, static_cast<hipStream_t>(stream)));
}

dq_status dq_gemv_asym(const uint16_t* x, int64_t M, const uint32_t* packed, const float* scales,
                       const int32_t* zeros, int64_t N, int64_t K, int32_t bits, float* y,
                       void* stream)
{
    if (!x || !packed || !scales || !zeros || !y) return DQ_ERR_NULL;
    dq_status st = check_common(N, K, bits);
    if (st != DQ_OK) return st;
    if (M < 1 || M > DQ_GEMV_MAX_M) return DQ_ERR_SHAPE;
    if (!aligned(x, 16) || !aligned(packed, 16) || !aligned(scales, 4) || !aligned(y, 4) ||
        !aligned(zeros, 4))
        return DQ_ERR_ALIGN;
    return hip_status(dq::launch_gemv(x, M, packed, scales, N, K, bits, y, zeros,
                                      static_cast<hipStream_t>(stream)));
}

dq_status dq_gemm(const uint16_t* x, int64_t M, const uint32_t* packed, const float* scales,
                  int64_t N, int64_t K, int32_t bits, float* y, void* stream)
{
    if (!x || !packed || !scales || !y) return DQ_ERR_NULL;
    dq_status st = check_common(N, K, bits);
    if (st != DQ_OK) return st;
    if (M < 1 || M > 0x7fffffffLL) return DQ_ERR_SHAPE;
    if (!aligned(x, 16) || !aligned(packed, 16) || !aligned(scales, 4) || !aligned(y, 4))
        return DQ_ERR_ALIGN;
    return hip_status(dq::launch_gemm(x, M, packed, scales, N, K, bits, y, nullptr,
                                      static_cast<hipStream_t>(stream)));
}

dq_status dq_gemm_asym(const uint16_t* x, int64_t M, const uint32_t* packed, const float* scales,
                       const int32_t* zeros, int64_t N, int64_t K, int32_t bits, float* y,
                       void* stream)
{
    if (!x || !packed || !scales || !zeros || !y) return DQ_ERR_NULL;
    dq_status st = check_common(N, K, bits);
    if (st != DQ_OK) return st;
    if (M < 1 || M > 0x7fffffffLL) return DQ_ERR_SHAPE;
    if (!aligned(x, 16) || !aligned(packed, 16) || !aligned(scales, 4) || !aligned(y, 4) ||
        !aligned(zeros, 4))
        return DQ_ERR_ALIGN;
    return hip_status(dq::launch_gemm(x, M, packed, scales, N, K, bits, y, zeros,
                                      static_cast<hipStream_t>(stream)));
}

dq_status dq_file_load(const dq_file* f, int64_t i, void* data, float* scales, void* stream)
{
    if (!f || !data) return DQ_ERR_NULL;
    dq_file_matrix m;
    const dq_status st = dq_file_matrix_info(f, i, &m);
    if (st != DQ_OK) return st;
    if (m.scales && !scales) return DQ_ERR_NULL;
    if (!aligned(data, 16) || !aligned(scales, 4)) return DQ_ERR_ALIGN;
    // region sizes follow from the entry's shape, which dq_file_open checked
    // against the file's extent
    const uint64_t db = m.bits == DQ_TOP_BITS
                            ? (uint64_t)m.N * (uint64_t)m.K * 2
                            : (uint64_t)m.N * (uint64_t)dq::packed_row_words(m.K, m.bits) * 4;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t err = hipMemcpyAsync(data, m.data, db, hipMemcpyHostToDevice, s);
    if (err == hipSuccess && m.scales)
        err = hipMemcpyAsync(scales, m.scales, (uint64_t)m.N * 4, hipMemcpyHostToDevice, s);
    return hip_status(err);
}

dq_status dq_stream_read(const void* buf, int64_t bytes, uint32_t* partial, int64_t nparts,
                         void* stream)
{
    if (!buf || !partial) return DQ_ERR_NULL;
    if (bytes < 16 || bytes % 16 != 0 || nparts < 1 || nparts > DQ_STREAM_MAX_PARTS)
        return DQ_ERR_SHAPE;
    if (!aligned(buf, 16) || !aligned(partial, 4)) return DQ_ERR_ALIGN;
    return hip_status(
        dq::launch_stream_read(buf, bytes, partial, nparts, static_cast<hipStream_t>(stream)));
}

const char* dq_status_string(dq_status status)
{
    switch (status) {
    case DQ_OK: return "ok";
    case DQ_ERR_NULL: return "a required pointer is NULL";
    case DQ_ERR_BITS: return "bits must be in [2, 15] (allocation levels: increasing, in [2, 16])";
    case DQ_ERR_SHAPE: return "N, K or M out of range";
    case DQ_ERR_ALIGN:
        return "pointer not aligned (W, packed, x: 16 bytes; fp64 sums: 8; others: 4)";
    case DQ_ERR_DTYPE: return "w_dtype must be DQ_F32 or DQ_BF16";
    case DQ_ERR_HIP: return "HIP launch or runtime error";
    case DQ_ERR_BUDGET: return "bit budget below every matrix at its lowest level";
    case DQ_ERR_VALUE:
        return "sensitivity, trace or sum not finite and >= 0, parameter count out of range, or "
               "a name without its terminating NUL";
    case DQ_ERR_IO: return "file could not be opened, written, sized or mapped";
    case DQ_ERR_FORMAT: return "file is not a packed-weight file of this version, or is corrupt";
    default: return "unknown status";
    }
}

const char* dq_last_error(void) { return g_last_error; }

}  // extern "C"
