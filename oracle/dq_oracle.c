/*
 * dq_oracle.c -- plain CPU reference for per-row symmetric b-bit weight
 * quantization, LSB-first bit packing, unpacking and the dequantized matmul.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no header, helper, table or constant
 * with the GPU kernels.
 *
 * Sources followed (pages as titled on the web):
 *  [TUT]  "量化" (Quantization) tutorial, aiknowledge.cn -- section
 *         "量化怎么工作" (how quantization works: scale = absmax / max_int,
 *         q = round(t / scale), dequant q * scale, error at most scale / 2,
 *         per-channel = one scale per output channel) and the code of
 *         "Step 1: 对称量化 (逐张量与逐通道)" (symmetric per-tensor and
 *         per-channel quantizer: qmax = 2^(b-1) - 1, zero channel replaced
 *         before the divide, numpy round = half-to-even, clip to
 *         [-qmax-1, qmax], int32 codes).
 *  [DYN]  "DynaQuant: 通过比特级水填充算法实现大语言模型的动态精度量化",
 *         zingnex.cn -- "第三步：应用配方" (apply one b-bit quantizer per
 *         matrix), "自定义内核架构" (packed N-bit storage in memory, expanded
 *         in registers before the matrix unit), "项目现状与路线图" (bit pack /
 *         unpack utilities, widths up to 15).
 *  [BPDQ] devpress.csdn.net BPDQ article, section 3.2 "推理加速优化" (fused
 *         dequantize + matmul taking int weights, fp32 scales, fp32 output).
 *
 * Readings where the pages are silent are stated beside the code that takes
 * them.  Arithmetic: the quantizer works in IEEE fp32 with correctly rounded
 * divide and round-half-to-even (numpy semantics on fp32 arrays); the matmul
 * reference works in fp64.  Build with -O2 -fno-fast-math -ffp-contract=off
 * so that no FMA contraction or flush-to-zero changes any rounding.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- element access ---------------------------------------------------- */

/* bf16 is the top half of an fp32 pattern; widening is exact. */
static float bf16_bits_to_float(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* dtype 0 = fp32, 1 = bf16 (bit patterns) */
static float load_weight(const void *w, int dtype, int64_t i)
{
    if (dtype == 0)
        return ((const float *)w)[i];
    return bf16_bits_to_float(((const uint16_t *)w)[i]);
}

/* ---- sizes -------------------------------------------------------------- */

/* Packed storage per row: K codes of b bits each, as one bit stream, rounded
 * up to whole bytes and then to a 128-byte multiple (row padding).  [DYN]
 * "自定义内核架构" stores b-bit codes densely; the 128-byte padding is the
 * layout this library fixes for its rows. */
int64_t oracle_row_bytes(int64_t K, int32_t bits)
{
    int64_t payload_bytes = (K * bits + 7) / 8;
    return (payload_bytes + 127) / 128 * 128;
}

/* ---- quantizer ([TUT] symmetric per-channel, one channel = one row) ------ */

/*
 * Quantize one row of K weights to b-bit signed integers.
 *   qmax  = 2^(b-1) - 1
 *   a     = max |w|                       (fp32, exact)
 *   s     = fl32(a / qmax); if a == 0 the divide uses 1.0 instead of a
 *   q[k]  = clip(rint(fl32(w[k] / s)), -qmax-1, qmax)
 * Readings:
 *   - rint under the default rounding mode is round-half-to-even, the rule
 *     numpy's round follows;
 *   - a row holding any NaN or +-Inf is not quantizable: its scale is the
 *     canonical quiet NaN (0x7FC00000) and every q is 0;
 *   - if a > 0 but a / qmax underflows to 0, the row is treated like an
 *     all-zero row (s = fl32(1/qmax), every q = 0).
 */
static void quantize_row(const void *w, int dtype, int64_t row, int64_t K,
                         int32_t bits, int32_t *q, float *scale)
{
    const int32_t qmax = (1 << (bits - 1)) - 1;
    const float lo = (float)(-qmax - 1);
    const float hi = (float)qmax;
    float a = 0.0f;
    int nonfinite = 0;

    for (int64_t k = 0; k < K; k++) {
        float v = load_weight(w, dtype, row * K + k);
        if (!isfinite(v)) {
            nonfinite = 1;
        } else if (fabsf(v) > a) {
            a = fabsf(v);
        }
    }

    if (nonfinite) {
        uint32_t nan_bits = 0x7FC00000u;
        memcpy(scale, &nan_bits, sizeof *scale);
        for (int64_t k = 0; k < K; k++)
            q[k] = 0;
        return;
    }

    float s = (a == 0.0f ? 1.0f : a) / (float)qmax;
    if (s == 0.0f) {
        /* a > 0 and a / qmax underflowed: same as an all-zero row. */
        s = 1.0f / (float)qmax;
        *scale = s;
        for (int64_t k = 0; k < K; k++)
            q[k] = 0;
        return;
    }
    *scale = s;

    for (int64_t k = 0; k < K; k++) {
        float v = load_weight(w, dtype, row * K + k);
        float t = v / s;        /* one IEEE fp32 divide */
        float r = rintf(t);     /* half-to-even */
        if (r < lo)
            r = lo;
        if (r > hi)
            r = hi;
        q[k] = (int32_t)r;
    }
}

/* ---- bit packing ([DYN] pack/unpack utilities) ------------------------- */

/*
 * Code k of a row is u = q + 2^(b-1) (offset binary, in [0, 2^b)).
 * Its bit j is stream bit k*b + j; stream bit i lives in bit (i mod 32) of
 * 32-bit word i / 32 of the row.  Every bit not written here is zero.
 * Deliberately bit by bit.
 */
static void pack_row(const int32_t *q, int64_t K, int32_t bits,
                     uint32_t *words, int64_t row_words)
{
    const uint32_t bias = 1u << (bits - 1);
    for (int64_t i = 0; i < row_words; i++)
        words[i] = 0;
    for (int64_t k = 0; k < K; k++) {
        uint32_t u = (uint32_t)(q[k] + (int32_t)bias);
        for (int32_t j = 0; j < bits; j++) {
            int64_t pos = k * bits + j;
            uint32_t bit = (u >> j) & 1u;
            words[pos / 32] |= bit << (pos % 32);
        }
    }
}

static void unpack_row(const uint32_t *words, int64_t K, int32_t bits,
                       int32_t *q)
{
    const int32_t bias = 1 << (bits - 1);
    for (int64_t k = 0; k < K; k++) {
        uint32_t u = 0;
        for (int32_t j = 0; j < bits; j++) {
            int64_t pos = k * bits + j;
            uint32_t bit = (words[pos / 32] >> (pos % 32)) & 1u;
            u |= bit << j;
        }
        q[k] = (int32_t)u - bias;
    }
}

/* ---- exported entry points --------------------------------------------- */

/* Quantize an [N, K] row-major matrix and pack it.  q_out (nullable) receives
 * the int32 codes before the offset; packed is [N, row_bytes/4] words. */
void oracle_quantize_pack(const void *w, int32_t dtype, int64_t N, int64_t K,
                          int32_t bits, uint32_t *packed, float *scales,
                          int32_t *q_out)
{
    const int64_t row_words = oracle_row_bytes(K, bits) / 4;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t n = 0; n < N; n++) {
        int32_t qbuf_small[256];
        int32_t *q = q_out ? q_out + n * K : NULL;
        int32_t *heap = NULL;
        if (!q) {
            if (K <= 256) {
                q = qbuf_small;
            } else {
                heap = (int32_t *)malloc((size_t)K * sizeof *heap);
                q = heap;
            }
        }
        quantize_row(w, dtype, n, K, bits, q, &scales[n]);
        pack_row(q, K, bits, packed + n * row_words, row_words);
        if (heap)
            free(heap);
    }
}

/* Pack given int32 codes q[N, K] (each in [-2^(b-1), 2^(b-1))) without
 * quantizing; lets the packing be checked over the whole code range. */
void oracle_pack(const int32_t *q, int64_t N, int64_t K, int32_t bits,
                 uint32_t *packed)
{
    const int64_t row_words = oracle_row_bytes(K, bits) / 4;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t n = 0; n < N; n++)
        pack_row(q + n * K, K, bits, packed + n * row_words, row_words);
}

/* Inverse of the packing; w_out[n,k] = fl32(q * s[n]), the dequantized weight
 * of [TUT] "how quantization works" (reconstructed = quantized * scale). */
void oracle_unpack(const uint32_t *packed, const float *scales, int64_t N,
                   int64_t K, int32_t bits, int32_t *q_out, float *w_out)
{
    const int64_t row_words = oracle_row_bytes(K, bits) / 4;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t n = 0; n < N; n++) {
        int32_t *q = q_out + n * K;
        unpack_row(packed + n * row_words, K, bits, q);
        if (w_out) {
            for (int64_t k = 0; k < K; k++)
                w_out[n * K + k] = (float)q[k] * scales[n];
        }
    }
}

/*
 * Dequantized matmul reference in fp64 ([BPDQ] 3.2: dequantize fused with the
 * product; fp32 scales, fp32 output):
 *     y[m,n]     = s[n] * sum_k x[m,k] * q[n,k]
 *     bound[m,n] = |s[n]| * sum_k |x[m,k] * q[n,k]|   (= sum_k |x * w_hat|)
 * x is bf16 bit patterns [M, K].  Each x*q product is exact in fp64.  The
 * outputs are computed for the (m, n) pairs listed in ms/ns (count pairs), so
 * that full-size problems can be checked on samples.
 */
void oracle_matmul_pairs(const uint16_t *x, int64_t M, const uint32_t *packed,
                         const float *scales, int64_t N, int64_t K,
                         int32_t bits, const int64_t *ms, const int64_t *ns,
                         int64_t count, double *y, double *bound)
{
    const int64_t row_words = oracle_row_bytes(K, bits) / 4;
    (void)M;
    (void)N;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < count; i++) {
        int64_t m = ms[i], n = ns[i];
        int32_t *q = (int32_t *)malloc((size_t)(K > 0 ? K : 1) * sizeof *q);
        unpack_row(packed + n * row_words, K, bits, q);
        double acc = 0.0, mag = 0.0;
        for (int64_t k = 0; k < K; k++) {
            double p = (double)bf16_bits_to_float(x[m * K + k]) * (double)q[k];
            acc += p;
            mag += fabs(p);
        }
        y[i] = (double)scales[n] * acc;
        bound[i] = fabs((double)scales[n]) * mag;
        free(q);
    }
}

/* Full [M, N] product: every pair, row n unpacked once. */
void oracle_matmul(const uint16_t *x, int64_t M, const uint32_t *packed,
                   const float *scales, int64_t N, int64_t K, int32_t bits,
                   double *y, double *bound)
{
    const int64_t row_words = oracle_row_bytes(K, bits) / 4;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t n = 0; n < N; n++) {
        int32_t *q = (int32_t *)malloc((size_t)(K > 0 ? K : 1) * sizeof *q);
        unpack_row(packed + n * row_words, K, bits, q);
        for (int64_t m = 0; m < M; m++) {
            double acc = 0.0, mag = 0.0;
            for (int64_t k = 0; k < K; k++) {
                double p = (double)bf16_bits_to_float(x[m * K + k]) * (double)q[k];
                acc += p;
                mag += fabs(p);
            }
            y[m * N + n] = (double)scales[n] * acc;
            bound[m * N + n] = fabs((double)scales[n]) * mag;
        }
        free(q);
    }
}

/* ---- asymmetric variant ([TUT] "量化怎么工作": a zero point added to the
 * rounded quotient, for distributions not centred on zero) ---------------- */

/*
 * Quantize one row to unsigned b-bit codes with a zero point.
 *   L     = 2^b - 1                       (largest code)
 *   lo    = min(0, min w), hi = max(0, max w)   (the range holds zero)
 *   s     = fl32(fl32(hi - lo) / L); if hi == lo the divide uses 1.0
 *   z     = clip(rint(fl32(-lo / s)), 0, L)
 *   u[k]  = clip(rint(fl32(w[k] / s)) + z, 0, L)
 *   w_hat = (u - z) * s
 * Readings (the pages give only "rounded quotient plus zero point"):
 *   - the range is widened to hold 0, so w = 0 is exactly representable;
 *   - a row with a NaN or +-Inf, or whose range overflows fp32, has scale NaN
 *     and z = every code = 2^(b-1);
 *   - if the range is > 0 but s underflows to 0, the row is treated like an
 *     all-zero row (s = fl32(1/L), z = 0, every code 0).
 */
static void quantize_row_asym(const void *w, int dtype, int64_t row, int64_t K,
                              int32_t bits, uint32_t *u, float *scale,
                              int32_t *zero)
{
    const int32_t L = (1 << bits) - 1;
    const uint32_t half = 1u << (bits - 1);
    float lo = 0.0f, hi = 0.0f;
    int nonfinite = 0;
    for (int64_t k = 0; k < K; k++) {
        float v = load_weight(w, dtype, row * K + k);
        if (!isfinite(v))
            nonfinite = 1;
        else {
            if (v < lo)
                lo = v;
            if (v > hi)
                hi = v;
        }
    }
    float range = hi - lo;
    if (nonfinite || !isfinite(range)) {
        uint32_t nan_bits = 0x7FC00000u;
        memcpy(scale, &nan_bits, sizeof *scale);
        *zero = (int32_t)half;
        for (int64_t k = 0; k < K; k++)
            u[k] = half;
        return;
    }
    float s = (range == 0.0f ? 1.0f : range) / (float)L;
    if (s == 0.0f) {
        *scale = 1.0f / (float)L;
        *zero = 0;
        for (int64_t k = 0; k < K; k++)
            u[k] = 0;
        return;
    }
    *scale = s;
    float zf = rintf(-lo / s);
    if (zf < 0.0f)
        zf = 0.0f;
    if (zf > (float)L)
        zf = (float)L;
    *zero = (int32_t)zf;
    for (int64_t k = 0; k < K; k++) {
        float v = load_weight(w, dtype, row * K + k);
        float quot = v / s;     /* one IEEE fp32 divide */
        float c = rintf(quot) + zf; /* both integers of at most 16 bits: exact */
        if (c < 0.0f)
            c = 0.0f;
        if (c > (float)L)
            c = (float)L;
        u[k] = (uint32_t)c;
    }
}

/* Pack unsigned codes u (each in [0, 2^b)) bit by bit, as pack_row does for
 * the offset codes of the symmetric scheme. */
static void pack_row_unsigned(const uint32_t *u, int64_t K, int32_t bits,
                              uint32_t *words, int64_t row_words)
{
    for (int64_t i = 0; i < row_words; i++)
        words[i] = 0;
    for (int64_t k = 0; k < K; k++) {
        for (int32_t j = 0; j < bits; j++) {
            int64_t pos = k * bits + j;
            words[pos / 32] |= ((u[k] >> j) & 1u) << (pos % 32);
        }
    }
}

static void unpack_row_unsigned(const uint32_t *words, int64_t K, int32_t bits,
                                uint32_t *u)
{
    for (int64_t k = 0; k < K; k++) {
        uint32_t v = 0;
        for (int32_t j = 0; j < bits; j++) {
            int64_t pos = k * bits + j;
            v |= ((words[pos / 32] >> (pos % 32)) & 1u) << j;
        }
        u[k] = v;
    }
}

/* Quantize [N, K] with per-row scale and zero point; u_out (nullable) gets
 * the unsigned codes. */
void oracle_quantize_pack_asym(const void *w, int32_t dtype, int64_t N,
                               int64_t K, int32_t bits, uint32_t *packed,
                               float *scales, int32_t *zeros, uint32_t *u_out)
{
    const int64_t row_words = oracle_row_bytes(K, bits) / 4;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t n = 0; n < N; n++) {
        uint32_t *u = u_out ? u_out + n * K
                            : (uint32_t *)malloc((size_t)K * sizeof *u);
        quantize_row_asym(w, dtype, n, K, bits, u, &scales[n], &zeros[n]);
        pack_row_unsigned(u, K, bits, packed + n * row_words, row_words);
        if (!u_out)
            free(u);
    }
}

/* Inverse: q_out[n,k] = u - z[n]; w_out (nullable) = fl32((u - z) * s[n]). */
void oracle_unpack_asym(const uint32_t *packed, const float *scales,
                        const int32_t *zeros, int64_t N, int64_t K,
                        int32_t bits, int32_t *q_out, float *w_out)
{
    const int64_t row_words = oracle_row_bytes(K, bits) / 4;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t n = 0; n < N; n++) {
        uint32_t *u = (uint32_t *)malloc((size_t)K * sizeof *u);
        unpack_row_unsigned(packed + n * row_words, K, bits, u);
        for (int64_t k = 0; k < K; k++) {
            int32_t q = (int32_t)u[k] - zeros[n];
            q_out[n * K + k] = q;
            if (w_out)
                w_out[n * K + k] = (float)q * scales[n];
        }
        free(u);
    }
}

/* fp64 reference of the asymmetric product:
 *     y[m,n]     = s[n] * sum_k x[m,k] * (u[n,k] - z[n])
 *     bound[m,n] = |s[n]| * sum_k |x[m,k] * (u[n,k] - z[n])| */
void oracle_matmul_asym(const uint16_t *x, int64_t M, const uint32_t *packed,
                        const float *scales, const int32_t *zeros, int64_t N,
                        int64_t K, int32_t bits, double *y, double *bound)
{
    const int64_t row_words = oracle_row_bytes(K, bits) / 4;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t n = 0; n < N; n++) {
        uint32_t *u = (uint32_t *)malloc((size_t)(K > 0 ? K : 1) * sizeof *u);
        unpack_row_unsigned(packed + n * row_words, K, bits, u);
        for (int64_t m = 0; m < M; m++) {
            double sum = 0.0, absum = 0.0;
            for (int64_t k = 0; k < K; k++) {
                double term = (double)bf16_bits_to_float(x[m * K + k]) *
                              (double)((int32_t)u[k] - zeros[n]);
                sum += term;
                absum += fabs(term);
            }
            y[m * N + n] = (double)scales[n] * sum;
            bound[m * N + n] = fabs((double)scales[n]) * absum;
        }
        free(u);
    }
}

/* ---- group-wise scales ([TUT] exercise 1 of "五、练习": one scale per group
 * of g consecutive weights of a row instead of one per channel) ---------- */

/*
 * Row n, group j holds columns [j*g, min(K, (j+1)*g)).  Each group is
 * quantized exactly like a row of the symmetric per-channel quantizer above
 * (same absmax, scale, zero-group, non-finite and underflow rules), with its
 * own scale scales[n*G + j], G = ceil(K/g).  Codes are packed per row as
 * before, one bit stream over all K codes.
 */
void oracle_quantize_pack_group(const void *w, int32_t dtype, int64_t N,
                                int64_t K, int32_t bits, int64_t g,
                                uint32_t *packed, float *scales, int32_t *q_out)
{
    const int64_t row_words = oracle_row_bytes(K, bits) / 4;
    const int64_t G = (K + g - 1) / g;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t n = 0; n < N; n++) {
        int32_t *q = (int32_t *)malloc((size_t)K * sizeof *q);
        float *piece = (float *)malloc((size_t)g * sizeof *piece);
        for (int64_t j = 0; j < G; j++) {
            int64_t k0 = j * g, len = (K - k0 < g) ? K - k0 : g;
            for (int64_t k = 0; k < len; k++)
                piece[k] = load_weight(w, dtype, n * K + k0 + k);
            /* the group as a one-row fp32 matrix */
            quantize_row(piece, 0, 0, len, bits, q + k0, &scales[n * G + j]);
        }
        pack_row(q, K, bits, packed + n * row_words, row_words);
        if (q_out)
            memcpy(q_out + n * K, q, (size_t)K * sizeof *q);
        free(piece);
        free(q);
    }
}

/* Inverse with group scales: q_out = u - 2^(b-1), w_out = fl32(q * s[n, k/g]). */
void oracle_unpack_group(const uint32_t *packed, const float *scales, int64_t N,
                         int64_t K, int32_t bits, int64_t g, int32_t *q_out,
                         float *w_out)
{
    const int64_t row_words = oracle_row_bytes(K, bits) / 4;
    const int64_t G = (K + g - 1) / g;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t n = 0; n < N; n++) {
        int32_t *q = q_out + n * K;
        unpack_row(packed + n * row_words, K, bits, q);
        if (w_out)
            for (int64_t k = 0; k < K; k++)
                w_out[n * K + k] = (float)q[k] * scales[n * G + k / g];
    }
}

/* fp64 reference with group scales:
 *     y[m,n]     = sum_k x[m,k] * q[n,k] * s[n, k/g]
 *     bound[m,n] = sum_k |x[m,k] * q[n,k] * s[n, k/g]| */
void oracle_matmul_group(const uint16_t *x, int64_t M, const uint32_t *packed,
                         const float *scales, int64_t N, int64_t K, int32_t bits,
                         int64_t g, double *y, double *bound)
{
    const int64_t row_words = oracle_row_bytes(K, bits) / 4;
    const int64_t G = (K + g - 1) / g;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t n = 0; n < N; n++) {
        int32_t *q = (int32_t *)malloc((size_t)(K > 0 ? K : 1) * sizeof *q);
        unpack_row(packed + n * row_words, K, bits, q);
        for (int64_t m = 0; m < M; m++) {
            double total = 0.0, total_abs = 0.0;
            for (int64_t k = 0; k < K; k++) {
                double term = (double)bf16_bits_to_float(x[m * K + k]) * (double)q[k] *
                              (double)scales[n * G + k / g];
                total += term;
                total_abs += fabs(term);
            }
            y[m * N + n] = total;
            bound[m * N + n] = total_abs;
        }
        free(q);
    }
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Thread count of the OpenMP loops that follow (n < 1 means 1); timing only. */
void oracle_set_threads(int n)
{
#ifdef _OPENMP
    omp_set_num_threads(n > 0 ? n : 1);
#else
    (void)n;
#endif
}
