/*
 * dq.h -- C ABI of the packed b-bit weight library for MI355X (gfx950).
 *
 * What it computes (pages as titled on the web):
 *  - Quantizer: the symmetric per-channel scheme of the "量化" (Quantization)
 *    tutorial, aiknowledge.cn, sections "量化怎么工作" (how quantization works)
 *    and "Step 1" (per-channel code), with one channel = one row of W[N, K]:
 *      qmax = 2^(b-1) - 1;  s[n] = fl32(max_k |W[n,k]| / qmax)  (1.0 replaces a
 *      zero max before the divide);  q = clip(rint(fl32(W / s)), -qmax-1, qmax)
 *    with IEEE fp32 arithmetic, a correctly rounded divide and
 *    round-half-to-even.  One bit width b in [2, 15] per call (per matrix), the
 *    recipe application step of the DynaQuant page (zingnex.cn), section
 *    "第三步：应用配方".
 *  - Packed storage: DynaQuant page, "自定义内核架构" (packed N-bit codes in
 *    memory, expanded in registers before the matrix unit) and "项目现状与路线图"
 *    (pack / unpack utilities).  Code u = q + 2^(b-1) (offset binary); the K
 *    codes of a row form one bit stream, code k at stream bits [k*b, k*b+b),
 *    stream bit i = bit (i mod 32) of 32-bit word i/32 (little-endian words);
 *    each row is zero-padded to dq_packed_row_bytes(K, b), a multiple of 128.
 *  - Dequantized matmul: BPDQ article (devpress.csdn.net), section 3.2
 *    (dequantize fused into the matrix product; int weights, fp32 scales, fp32
 *    output):  y[m,n] = s[n] * sum_k x[m,k] * q[n,k],  i.e. y = x . W_hat^T.
 *
 *  - Bit allocation (the step before quantization): DynaQuant page,
 *    "第一步：敏感度测量" (sensitivity = Hessian trace x mean(w^2)) and
 *    "第二步：比特分配" (water-filling on a max-heap; hardware-native levels
 *    {4, 8, 16} or every width 4 .. 16, where 16 keeps the BF16 weights).
 *    mean(w^2) is measured on the GPU (dq_row_sumsq, or fused into the
 *    quantize pass: dq_quantize_pack_sumsq); dq_sensitivity and
 *    dq_allocate_bits run on the host.
 *
 * Conventions for every entry point:
 *  - All array pointers are DEVICE pointers (memory of the current HIP
 *    device), except for dq_sensitivity and dq_allocate_bits, which take HOST
 *    pointers, enqueue nothing and return when done.  The caller allocates
 *    and owns every buffer; the library allocates no device memory (the
 *    allocator keeps O(n) host memory during the call), keeps no state
 *    between calls and is re-entrant.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Work
 *    is enqueued asynchronously; nothing is synchronised.
 *  - Argument errors are detected on the host and returned BEFORE any HIP call;
 *    then nothing is enqueued and no output is touched.  A launch failure
 *    returns DQ_ERR_HIP; dq_last_error() then gives the HIP message (per
 *    calling thread).
 *  - Layouts are row-major and contiguous:
 *      W       [N, K]          fp32 or bf16 bit patterns (uint16)
 *      packed  [N, row_words]  uint32, row_words = dq_packed_row_bytes(K,b)/4
 *      scales  [N]             fp32
 *      x       [M, K]          bf16 bit patterns (uint16)
 *      y       [M, N]          fp32 (overwritten, never accumulated into)
 *  - Sizes: 1 <= N <= 2^31-1, 1 <= K <= DQ_MAX_K; dq_gemv: 1 <= M <= 16;
 *    dq_gemm: 1 <= M <= 2^31-1.
 *  - Alignment: W, packed and x must be 16-byte aligned (DQ_ERR_ALIGN);
 *    scales, q_out, w_out and y 4-byte aligned; row_sumsq and matrix_sumsq
 *    8-byte aligned.
 */
#ifndef DQ_H
#define DQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t dq_status;

#define DQ_OK 0
#define DQ_ERR_NULL 1  /* a required pointer is NULL                         */
#define DQ_ERR_BITS 2  /* bits outside [2, 15]                               */
#define DQ_ERR_SHAPE 3 /* N, K or M outside the ranges above                 */
#define DQ_ERR_ALIGN 4 /* a pointer is not aligned as required               */
#define DQ_ERR_DTYPE 5 /* w_dtype is neither DQ_F32 nor DQ_BF16              */
#define DQ_ERR_HIP 6   /* a HIP launch or runtime call failed                */
#define DQ_ERR_BUDGET 7 /* bit budget below every matrix at its lowest level */
#define DQ_ERR_VALUE 8 /* a sensitivity, trace, sum or parameter count out of range */
#define DQ_ERR_IO 9     /* a file could not be opened, written, sized or mapped   */
#define DQ_ERR_FORMAT 10 /* a file is not a packed-weight file, or is corrupt     */

#define DQ_F32 0  /* W holds IEEE fp32 values                               */
#define DQ_BF16 1 /* W holds bf16 bit patterns (uint16)                     */

#define DQ_MIN_BITS 2
#define DQ_MAX_BITS 15
#define DQ_GEMV_MAX_M 16
#define DQ_MAX_K (1LL << 22)
#define DQ_TOP_BITS 16                 /* allocation level meaning "BF16 kept" */
#define DQ_MAX_MATRICES (1LL << 24)    /* matrices per allocation              */
#define DQ_MAX_PARAMS (1LL << 40)      /* parameters per matrix                */
#define DQ_MAX_GROUP 2048              /* largest group of the group-wise scales */

/* Bytes of one packed row: ceil(K*bits/8) rounded up to a multiple of 128.
 * Returns 0 when K or bits is out of range.  Host-only, no HIP call. */
size_t dq_packed_row_bytes(int64_t K, int32_t bits);

/* Quantize W[N, K] row by row to `bits` bits and pack it.
 *   w              in   device, [N, K], dtype w_dtype (DQ_F32 or DQ_BF16)
 *   packed         out  device, [N, row_words] uint32, fully written (padding = 0)
 *   scales         out  device, [N] fp32
 *   nonfinite_rows out  device, [1] uint32, 4-byte aligned, may be NULL: the
 *                       number of rows holding a NaN or +-Inf (the pages take
 *                       finite weights; this reports where that fails)
 * A row holding a NaN or +-Inf gets scale = quiet NaN (bits 0x7FC00000) and
 * every code = 2^(b-1) (q = 0).  A row whose max|W| / qmax underflows to 0 is
 * treated like an all-zero row: scale = fl32(1/qmax), q = 0. */
dq_status dq_quantize_pack(const void* w, int32_t w_dtype, int64_t N, int64_t K, int32_t bits,
                           uint32_t* packed, float* scales, uint32_t* nonfinite_rows,
                           void* stream);

/* Group-wise scales ("量化" tutorial, exercise 1 of its exercises: one scale
 * per group of weights instead of per channel, groups of 32 to 256 as
 * GPTQ/AWQ use).  Group j of row n holds columns [j*g, min(K, (j+1)*g)) and
 * is quantized exactly as a row of dq_quantize_pack (its own absmax, scale,
 * zero, non-finite and underflow rules); codes are packed per row as before.
 *   group   g, a power of two in [32, DQ_MAX_GROUP] (else DQ_ERR_SHAPE)
 *   scales  device, fp32 [N, G], G = ceil(K / g), scale of group j of row n at
 *           scales[n * G + j]
 * dq_unpack_group: q_out as dq_unpack, w_out = fl32(q * s[n, k / g]).
 * dq_gemv_group / dq_gemm_group: y[m,n] = sum_k x[m,k] q[n,k] s[n, k/g]; each
 * group's partial sum (fp32, exact products) is scaled as the group ends.
 * Other arguments as for the per-row entry points. */
dq_status dq_quantize_pack_group(const void* w, int32_t w_dtype, int64_t N, int64_t K,
                                 int32_t bits, int64_t group, uint32_t* packed, float* scales,
                                 void* stream);
dq_status dq_unpack_group(const uint32_t* packed, const float* scales, int64_t N, int64_t K,
                          int32_t bits, int64_t group, int32_t* q_out, float* w_out, void* stream);
dq_status dq_gemv_group(const uint16_t* x, int64_t M, const uint32_t* packed, const float* scales,
                        int64_t N, int64_t K, int32_t bits, int64_t group, float* y, void* stream);
dq_status dq_gemm_group(const uint16_t* x, int64_t M, const uint32_t* packed, const float* scales,
                        int64_t N, int64_t K, int32_t bits, int64_t group, float* y, void* stream);

/* Asymmetric variant ("量化" tutorial, "量化怎么工作": a zero point added to
 * the rounded quotient, for distributions not centred on zero).  Per row n,
 * with L = 2^b - 1:  lo = min(0, min_k W), hi = max(0, max_k W);
 * s[n] = fl32(fl32(hi - lo) / L) (1.0 replaces a zero range);
 * z[n] = clip(rint(fl32(-lo / s)), 0, L);
 * code u = clip(rint(fl32(W / s)) + z, 0, L), stored unsigned in the same
 * packed layout (no offset added); w_hat = (u - z) * s.
 *   zeros   out  device, [N] int32 zero points
 * A row with a NaN or +-Inf, or whose range overflows fp32, gets s = NaN and
 * z = every code = 2^(b-1); a row whose s underflows to 0 gets s = fl32(1/L),
 * z = 0 and codes 0. */
dq_status dq_quantize_pack_asym(const void* w, int32_t w_dtype, int64_t N, int64_t K,
                                int32_t bits, uint32_t* packed, float* scales, int32_t* zeros,
                                void* stream);

/* Inverse of dq_quantize_pack_asym: q_out = u - zeros[n] (int32), w_out =
 * fl32(q * s[n]); arguments as for dq_unpack plus zeros (device, [N]). */
dq_status dq_unpack_asym(const uint32_t* packed, const float* scales, const int32_t* zeros,
                         int64_t N, int64_t K, int32_t bits, int32_t* q_out, float* w_out,
                         void* stream);

/* Asymmetric products: y[m,n] = s[n] * sum_k x[m,k] (u[n,k] - z[n]), with the
 * kernels of dq_gemv / dq_gemm (same M ranges and layouts; zeros [N] int32,
 * device, 4-byte aligned).  Each code has the row's zero point subtracted
 * before it meets x, so every product x * (u - z) is exact (|u - z| < 2^b:
 * for b >= 9 the codes go through fp32 FMAs on the vector units, or as two
 * exact bf16 halves on the matrix cores); accumulation is fp32 and the scale
 * is applied once per output, as in the symmetric products. */
dq_status dq_gemv_asym(const uint16_t* x, int64_t M, const uint32_t* packed, const float* scales,
                       const int32_t* zeros, int64_t N, int64_t K, int32_t bits, float* y,
                       void* stream);
dq_status dq_gemm_asym(const uint16_t* x, int64_t M, const uint32_t* packed, const float* scales,
                       const int32_t* zeros, int64_t N, int64_t K, int32_t bits, float* y,
                       void* stream);

/* The statistic a matrix's sensitivity needs (DynaQuant page, "第一步：敏感度
 * 测量": mean(w^2) of the matrix), measured before any width is chosen: one
 * read of W.
 *   w             in   device, [N, K], dtype w_dtype (DQ_F32 or DQ_BF16)
 *   row_sumsq     out  device, [N] fp64, sum_k W[n,k]^2 (8-byte aligned)
 *   matrix_sumsq  out  device, [1] fp64, sum of row_sumsq; may be NULL
 * Every square of an fp32 or bf16 value is exact in fp64; the sums are fp64
 * in a fixed order (the same bits on every call), within (count - 1) * 2^-53
 * of the exact sum relative to it.  A row with a NaN gives NaN, one with an
 * infinity +inf.  mean(w^2) = matrix_sumsq / (N * K). */
dq_status dq_row_sumsq(const void* w, int32_t w_dtype, int64_t N, int64_t K, double* row_sumsq,
                       double* matrix_sumsq, void* stream);

/* dq_quantize_pack and dq_row_sumsq in one pass over W, for callers that
 * quantize a matrix anyway and want the statistic of exactly what they store
 * (say, to re-run the allocation after a change).  packed and scales are
 * bit-identical to dq_quantize_pack's; the sums obey the same bound as
 * dq_row_sumsq's (and are the same on every call) but add in another fixed
 * order, so they may differ from dq_row_sumsq's in the last bits. */
dq_status dq_quantize_pack_sumsq(const void* w, int32_t w_dtype, int64_t N, int64_t K,
                                 int32_t bits, uint32_t* packed, float* scales,
                                 double* row_sumsq, double* matrix_sumsq, void* stream);

/* Inverse of the packing.
 *   packed  in   device, [N, row_words] uint32
 *   scales  in   device, [N] fp32; may be NULL when w_out is NULL
 *   q_out   out  device, [N, K] int32, q = u - 2^(b-1); may be NULL
 *   w_out   out  device, [N, K] fp32, fl32(q * s[n]); may be NULL
 * At least one of q_out and w_out must be non-NULL. */
dq_status dq_unpack(const uint32_t* packed, const float* scales, int64_t N, int64_t K,
                    int32_t bits, int32_t* q_out, float* w_out, void* stream);

/* Decode-shaped product, 1 <= M <= 16:  y[m,n] = s[n] * sum_k x[m,k] q[n,k].
 *   x       in   device, [M, K] bf16 bits
 *   packed  in   device, [N, row_words] uint32 (from dq_quantize_pack)
 *   scales  in   device, [N] fp32
 *   y       out  device, [M, N] fp32
 * Accumulates in fp32; the scale is applied once per output after the sum. */
dq_status dq_gemv(const uint16_t* x, int64_t M, const uint32_t* packed, const float* scales,
                  int64_t N, int64_t K, int32_t bits, float* y, void* stream);

/* Decode-shaped products of several matrices in one call (DynaQuant page,
 * "自定义内核架构": the bit saving becomes decode speed on bandwidth-bound
 * hardware; at decode sizes one launch per matrix costs about as much as the
 * matrix's transfer, so the matrices a token multiplies share a launch).
 * For each item i: y_i[m,n] = s_i[n] * sum_k x_i[m,k] q_i[n,k], exactly as
 * dq_gemv on that item (same validation, layouts and tolerance); an item with
 * zero points (`zeros` non-NULL) is served as dq_gemv_asym, one with group
 * scales (`group` non-zero) as dq_gemv_group.
 *   items  in   HOST array of `count` descriptors, 1 <= count <=
 *               DQ_GEMV_BATCH_MAX; read during the call only (the library
 *               copies them into the kernel arguments)
 *   M           rows of every item's x, 1 <= M <= DQ_GEMV_MAX_M
 * Items may share x, packed and scales; no y may overlap another item's y or
 * any input.  With M <= 2, the items of one scheme (symmetric, zero points,
 * group scales) whose K is a multiple of 32 and whose x fits the LDS
 * (M * K / 32 * 80 bytes <= 48 KB) run in ONE kernel launch per scheme
 * (workgroups of all such items in one grid, widths mixed), except items with
 * zero points or group scales whose rows hold 64 chunks or more but not a
 * multiple of 32 chunks; with 3 <= M <= 16, every symmetric item whose K is a
 * multiple of 32 does (its outputs then equal dq_gemv's bit for bit).  Each
 * other item runs as its own launch of the matching one-matrix entry point.
 * Argument errors in any item (including a `group` that is not 0 or a power of
 * two in [32, 2048], or `zeros` and `group` both set) are returned before
 * anything is enqueued. */
#define DQ_GEMV_BATCH_MAX 32
typedef struct {
    const uint16_t* x;       /* device, [M, K] bf16 bits, 16-byte aligned        */
    const uint32_t* packed;  /* device, [N, row_words] (a dq_quantize_pack* call), 16 B */
    const float* scales;     /* device, [N] fp32 ([N, ceil(K / group)] with group), 4 B */
    float* y;                /* device, [M, N] fp32 out, 4-byte aligned           */
    int64_t N;
    int64_t K;
    int32_t bits;            /* 2 .. 15 */
    int32_t group;           /* 0: a scale per row; else codes per group scale    */
    const int32_t* zeros;    /* NULL, or device [N] zero points (dq_quantize_pack_asym) */
} dq_gemv_item;

dq_status dq_gemv_batched(const dq_gemv_item* items, int32_t count, int64_t M, void* stream);

/* Prefill-shaped product, any M >= 1 (tuned for M >= 256).  Same arguments
 * and result as dq_gemv.  Codes are expanded exactly to bf16 (for b >= 10 as
 * two exact bf16 halves, 64*hi + lo) and multiplied on the bf16 matrix cores
 * with fp32 accumulation. */
dq_status dq_gemm(const uint16_t* x, int64_t M, const uint32_t* packed, const float* scales,
                  int64_t N, int64_t K, int32_t bits, float* y, void* stream);

/* Not a step of the method: a plain streaming read of `bytes` bytes, the
 * yardstick for the bandwidth-bound entry points above (the rate a kernel
 * that only reads the same bytes reaches at the same size).  `nparts`
 * workgroups each read a contiguous share with 16-byte loads and write the
 * XOR of its 32-bit words to partial[i], so the XOR of partial[0 .. nparts)
 * is the XOR of every word of the buffer (a share may be empty: then 0).
 *   buf      in   device, bytes >= 16 and a multiple of 16, 16-byte aligned
 *   partial  out  device, [nparts] uint32, 4-byte aligned
 *   1 <= nparts <= DQ_STREAM_MAX_PARTS (else DQ_ERR_SHAPE, as is a bad size) */
#define DQ_STREAM_MAX_PARTS 65536
dq_status dq_stream_read(const void* buf, int64_t bytes, uint32_t* partial, int64_t nparts,
                         void* stream);

/* Sensitivity of each of n matrices (HOST pointers; DynaQuant page,
 * "第一步：敏感度测量"):  out[i] = h_trace[i] * (sumsq[i] / params[i]), an fp64
 * divide then an fp64 multiply.  h_trace and sumsq must be finite and >= 0,
 * 1 <= params[i] <= DQ_MAX_PARAMS (else DQ_ERR_VALUE); 1 <= n <= DQ_MAX_MATRICES. */
dq_status dq_sensitivity(const double* h_trace, const double* sumsq, const int64_t* params,
                         int64_t n, double* out);

/* Water-filling bit allocation over n matrices (HOST pointers; DynaQuant page,
 * "第二步：比特分配").  Every matrix starts at levels[0]; a step raises one
 * matrix to its next level; the step removing the most predicted loss per
 * byte goes first (ties: the lower matrix index).  Predicted loss of matrix i
 * at b bits: sensitivity[i] * 4^-b, and 0 at DQ_TOP_BITS (BF16 kept).  A step
 * that does not fit in the budget is dropped for good and the others go on;
 * a step that removes no loss is never taken.
 *   sensitivity    in   [n] fp64, finite, >= 0
 *   params         in   [n] parameters per matrix, 1 .. DQ_MAX_PARAMS
 *   levels         in   [n_levels] strictly increasing widths in [2, 16]
 *                       ({4, 8, 16} hardware-native, {4, ..., 16} full)
 *   budget_bits        total bits sum_i params[i] * bits[i] allowed; < 0 = no
 *                       limit (the whole frontier); below the floor
 *                       sum_i params[i] * levels[0]: DQ_ERR_BUDGET
 *   bits_out       out  [n] chosen width per matrix (the recipe)
 *   step_matrix,
 *   step_bits      out  [step_capacity] the steps taken, in order (matrix,
 *                       new width); may be NULL when step_capacity == 0;
 *                       only the first step_capacity are written
 *   n_steps        out  number of steps taken (may exceed step_capacity); may be NULL
 *   loss           out  predicted total loss sum_i L_i(bits_out[i]); may be NULL
 * Priorities are fp64 in a fixed order of operations, so the result is the
 * same bit for bit on every platform with IEEE doubles. */
dq_status dq_allocate_bits(const double* sensitivity, const int64_t* params, int64_t n,
                           const int32_t* levels, int32_t n_levels, int64_t budget_bits,
                           int32_t* bits_out, int64_t* step_matrix, int32_t* step_bits,
                           int64_t step_capacity, int64_t* n_steps, double* loss);

/* On-disk packed-weight format (DynaQuant page, "项目现状与路线图": a packed
 * storage format on disk is listed as in progress; this layout is the
 * library's own).  One file holds a recipe: every matrix's name, shape and
 * width, its packed words exactly as in device memory and its scales, each
 * region at a 4096-byte boundary so that the file maps straight into memory.
 * Layout (little-endian): 64-byte header {"DQWPACK1", u32 version = 1, u32
 * count, u64 table offset = 64, u64 file bytes, 32 zero bytes}; then count
 * 128-byte entries {char name[64] NUL-padded, i64 N, i64 K, i32 bits, u32 0,
 * u64 data offset, u64 data bytes, u64 scales offset (0 if none), u64
 * checksum, u64 0}; then the regions in entry order.  bits 2..15: data =
 * packed [N, row_words] uint32 and fp32 scales [N]; bits 16: the BF16 weights
 * kept, data = bf16 [N, K], no scales.  checksum = 64-bit FNV-1a over the
 * data bytes then the scale bytes: h = 0xcbf29ce484222325, then for each byte
 * h = (h ^ byte) * 0x100000001b3 mod 2^64. */
#define DQ_FILE_MAX_MATRICES (1LL << 20)

typedef struct {
    char name[64];        /* UTF-8, NUL-terminated within the 64 bytes        */
    int64_t N;
    int64_t K;
    int32_t bits;         /* 2..15 packed, 16 = BF16 weights kept             */
    const void* data;     /* HOST: packed words [N, row_words] or bf16 [N, K]  */
    const float* scales;  /* HOST: fp32 [N]; NULL when bits == 16             */
} dq_file_matrix;

typedef struct dq_file dq_file; /* an open, memory-mapped file (read only) */

/* Write `count` matrices (host buffers) to `path` (created or truncated).
 * Descriptions are checked before the file is touched: DQ_ERR_BITS,
 * DQ_ERR_SHAPE (N, K as for dq_quantize_pack; 1 <= count <=
 * DQ_FILE_MAX_MATRICES), DQ_ERR_NULL, DQ_ERR_VALUE (a name without its NUL);
 * DQ_ERR_IO if writing fails (the file may then be partial). */
dq_status dq_file_write(const char* path, const dq_file_matrix* mats, int64_t count);

/* Map `path` read-only and check its header and every entry (magic, version,
 * sizes consistent with N, K and bits, regions aligned, in order and inside
 * the file): DQ_ERR_FORMAT otherwise.  The handle is the caller's until
 * dq_file_close. */
dq_status dq_file_open(const char* path, dq_file** out);

/* Number of matrices in an open file (0 for NULL). */
int64_t dq_file_count(const dq_file* f);

/* Entry i: name, shape, width, and host pointers into the mapping (valid
 * until dq_file_close). */
dq_status dq_file_matrix_info(const dq_file* f, int64_t i, dq_file_matrix* out);

/* Recompute entry i's checksum: DQ_OK if it matches, DQ_ERR_FORMAT if not. */
dq_status dq_file_verify(const dq_file* f, int64_t i);

/* Copy entry i into device buffers on `stream` (hipMemcpyAsync from the
 * mapping; the mapping must stay open until the copy is done):
 *   data    out  device, the entry's data bytes (16-byte aligned)
 *   scales  out  device, fp32 [N] (4-byte aligned); ignored and may be NULL
 *                when the entry has no scales */
dq_status dq_file_load(const dq_file* f, int64_t i, void* data, float* scales, void* stream);

/* Unmap and free the handle (NULL is ignored). */
void dq_file_close(dq_file* f);

/* Static text for a status code. */
const char* dq_status_string(dq_status status);

/* Text of the last DQ_ERR_HIP on the calling thread ("" if none). */
const char* dq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DQ_H */
