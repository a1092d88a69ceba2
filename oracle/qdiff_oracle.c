/*
 * Oracle for the rotated, dynamically quantized INT8 (and INT4) linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  This plain, slow, single-purpose C file defines
 * the exact results that the GPU library must reproduce.  It shares no code,
 * header, table or helper with the GPU path and must never be linked into,
 * or called from, the product.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load it.
 *
 * Sources (cited by page title and section):
 *  - comfy-kitchen 0.2.40 PyPI page, "Huawei Ascend backend": the operation
 *    split (quantize_int8_rowwise = per-row dynamic quantization;
 *    quantize_and_rotate_rowwise = rotation followed by per-row quantization;
 *    int8_linear = dynamic quantization + INT8 matmul; dequantize_int8_simple;
 *    convrot_w4a4_linear = signed INT4 codes kept in INT8 storage, packed INT4
 *    weights unpacked to INT8, INT32 accumulation, then cast and scale).
 *  - SGLang PR "Tune Kitchen INT8 row splitting for SM120", "Accuracy Test":
 *    BF16 activations and bias, INT8 weights, FP32 row scales, ConvRot256.
 *  - ComfyUI-AppleSilicon-FP8 README, "What it fixes", row 17: the W8A8 path
 *    rotates the activation online, quantizes it per row, multiplies
 *    INT8 x INT8 -> INT32 and applies the per-row rescale and the bias in the
 *    store epilogue; quantizing before the rotation is the wrong order.
 *
 * Readings where the pages are silent (all arithmetic is IEEE binary32 with
 * round-to-nearest-even, no fused multiply-add, no reassociation, subnormals
 * kept; build with -ffp-contract=off and without fast-math):
 *  - The 256-wide rotation is the Sylvester-ordered Walsh-Hadamard matrix
 *    H[i][j] = (-1)^popcount(i & j) scaled by 1/16, applied to each aligned
 *    256-element block of a row.  It is evaluated by the in-place butterfly
 *    with the pair distance h taking the values 1, 2, 4, ..., 128 in that
 *    order, each pair (j, j+h) becoming (a+c, a-c); the 1/16 multiply comes
 *    after the last stage.
 *  - Row scale s = amax / qmax (one correctly rounded division), qmax = 127
 *    for INT8 and 7 for INT4; amax is the exact maximum of |v| over the row.
 *  - Code q = clamp(rne(fl(v / s)), -qmax, qmax); a row with s == 0 gets
 *    all-zero codes.
 *  - Accumulator acc = sum_k a[k] * w[k] exactly (int64 here, must fit int32).
 *  - Output y = bf16_rne(((float)acc * sx[m]) * sw[n] + (float)bias[n]),
 *    evaluated left to right in FP32.
 *  - Dequantization out = fl(q * s), optionally rounded to BF16.
 *  - INT4 packing: byte i of a row holds code 2i in its low nibble and code
 *    2i+1 in its high nibble, both two's complement.
 *  - Input activation (int8_linear's input_act, comfy-kitchen 0.2.40, "HIP
 *    backend"): act(x) is applied to each input element and rounded to
 *    nearest in the input's 16-bit type, as an unfused act() would store
 *    it (an exact activation value is never halfway between two neighbours);
 *    the layer then proceeds on those values.  GELU (tanh form
 *    with 0.044715), GELU (erf form), SiLU and ReLU, evaluated in long
 *    double.
 *  - INT8 attention (int8_attention: comfy-kitchen's INT8-quantized
 *    attention kernel behind ComfyUI's --use-ck-attention, per the
 *    ai-jitan-hub article on ComfyUI v0.32.0; the article gives no formula,
 *    only that q, k and v are quantized to INT8).  Reading: q, k and v are
 *    each quantized per token (one row of D values per head) by the row rule
 *    above; scores S[i][j] = acc(i, j) * sq[i] * sk[j] * scale with the exact
 *    integer dot product acc of the codes and scale = 1/sqrt(D) unless given;
 *    softmax over j; out[i] = sum_j p[i][j] * (sv[j] * v[j]) / sum_j p[i][j].
 *    Evaluated in double precision (the GPU result is compared within a
 *    bound derived from its own rounding steps).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_F32 0
#define ORACLE_BF16 1
#define ORACLE_F16 2

/* ---- scalar conversions ------------------------------------------------ */

static float bf16_bits_to_float(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* IEEE binary16 -> binary32, exact (every half value is a float value). */
static float f16_bits_to_float(uint16_t h) {
    int sign = (h >> 15) & 1;
    int exp = (h >> 10) & 0x1f;
    int man = h & 0x3ff;
    float v;
    if (exp == 0) {
        v = ldexpf((float)man, -24);               /* subnormal half */
    } else if (exp == 31) {
        v = man ? NAN : INFINITY;
    } else {
        v = ldexpf((float)(man | 0x400), exp - 25); /* 1.man * 2^(exp-15) */
    }
    return sign ? -v : v;
}

/* FP32 -> BF16 bits, round to nearest, ties to even; NaN stays NaN. */
uint16_t oracle_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7fffu + lsb) >> 16);
}

static float load_elem(const void* x, int dtype, int64_t idx) {
    switch (dtype) {
        case ORACLE_F32: return ((const float*)x)[idx];
        case ORACLE_BF16: return bf16_bits_to_float(((const uint16_t*)x)[idx]);
        default: return f16_bits_to_float(((const uint16_t*)x)[idx]);
    }
}

/* ---- input activations --------------------------------------------------- */

#define ORACLE_ACT_GELU_TANH 1
#define ORACLE_ACT_GELU_ERF 2
#define ORACLE_ACT_SILU 3
#define ORACLE_ACT_RELU 4

/* The activation in long double, written without cancellation:
 * x/2 (1 + tanh u) = x / (1 + e^(-2u)); x/2 (1 + erf(x/sqrt2)) = x/2 erfc(-x/sqrt2). */
static long double act_value(int act, long double x) {
    const long double pi = acosl(-1.0L);
    switch (act) {
        case ORACLE_ACT_GELU_TANH: {
            long double u = sqrtl(2.0L / pi) * (x + 0.044715L * x * x * x);
            return x / (1.0L + expl(-2.0L * u));
        }
        case ORACLE_ACT_GELU_ERF: return 0.5L * x * erfcl(-x / sqrtl(2.0L));
        case ORACLE_ACT_SILU: return x / (1.0L + expl(-x));
        case ORACLE_ACT_RELU: return x > 0.0L ? x : 0.0L;
        default: return x;
    }
}

/* Round the computed activation d to nearest on the grid of a binary type with
 * `mant` fraction bits and smallest normal exponent `emin` (subnormals
 * included).  The exact activation is never halfway between grid points; a
 * computed d that is exactly halfway is x/2 with the positive remainder
 * x/2 * g(x) (g = tanh(u), tanh(x/2) or erf(x/sqrt2)) lost to rounding, which
 * happens for the smallest |x|, so such a d is rounded up. */
static float round_to_grid(long double d, int mant, int emin) {
    if (d == 0.0L) return (float)d;
    int e = ilogbl(d);
    if (e < emin) e = emin;
    long double t = ldexpl(d, mant - e);      /* |t| < 2^(mant+1), exact */
    long double r = floorl(t + 0.5L);         /* nearest, halfway upwards */
    if (r == 0.0L && d < 0.0L) r = -0.0L;
    return (float)(r * ldexpl(1.0L, e - mant));
}

/* act(v) rounded to the 16-bit input type (BF16: 7 fraction bits, FP16: 10). */
static float act_elem(int act, int dtype, float v) {
    if (act == 0) return v;
    long double a = act_value(act, (long double)v);
    return dtype == ORACLE_BF16 ? round_to_grid(a, 7, -126) : round_to_grid(a, 10, -14);
}

/* Exact FP16 bits of a float that lies on the FP16 grid. */
static uint16_t f16_bits_exact(float f) {
    uint16_t sign = signbit(f) ? 0x8000u : 0u;
    float a = fabsf(f);
    if (a == 0.0f) return sign;
    int e = ilogbf(a);
    if (e > 15) return (uint16_t)(sign | 0x7C00u);
    if (e < -14) return (uint16_t)(sign | (uint16_t)ldexpf(a, 24));
    return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)((int)ldexpf(a, 10 - e) - 1024));
}

/* out[i] = act(x[i]) in the 16-bit input type (BF16 or FP16 bits). */
void oracle_input_act(const uint16_t* x, int dtype, int64_t n, int act, uint16_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) {
        float v = load_elem(x, dtype, i);
        float a = act_elem(act, dtype, v);
        uint32_t u;
        memcpy(&u, &a, 4);
        out[i] = dtype == ORACLE_BF16 ? (uint16_t)(u >> 16) : f16_bits_exact(a);
    }
}

/* ---- rotation ---------------------------------------------------------- */

/* In-place normalised Walsh-Hadamard transform of one 256-element block. */
void oracle_hadamard256(float* u) {
    for (int h = 1; h < 256; h *= 2) {
        for (int j = 0; j < 256; j++) {
            if (j & h) continue;
            float a = u[j];
            float c = u[j + h];
            u[j] = a + c;
            u[j + h] = a - c;
        }
    }
    for (int j = 0; j < 256; j++) u[j] = u[j] * 0.0625f;
}

/* Widen rows of x ([M, K], row stride ldx elements) to FP32, apply the input
 * activation `act` (0: none; 16-bit inputs only) and, when block == 256,
 * rotate every 256-block.  out is [M, K] dense.
 * Returns 0, or -1 for an unsupported block / K / activation. */
int oracle_rotate_rows_act(const void* x, int dtype, int64_t M, int64_t K, int64_t ldx,
                           int block, int act, float* out) {
    if (block != 0 && block != 256) return -1;
    if (block == 256 && K % 256 != 0) return -1;
    if (act != 0 && dtype == ORACLE_F32) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; m++) {
        float* row = out + m * K;
        for (int64_t k = 0; k < K; k++) row[k] = act_elem(act, dtype, load_elem(x, dtype, m * ldx + k));
        if (block == 256)
            for (int64_t b = 0; b < K; b += 256) oracle_hadamard256(row + b);
    }
    return 0;
}

int oracle_rotate_rows(const void* x, int dtype, int64_t M, int64_t K, int64_t ldx,
                       int block, float* out) {
    return oracle_rotate_rows_act(x, dtype, M, K, ldx, block, 0, out);
}

/* ---- per-row symmetric quantization ------------------------------------ */

/* Quantize each row of v ([M, K] dense FP32) to codes in [-qmax, qmax]. */
void oracle_quantize_rows(const float* v, int64_t M, int64_t K, int qmax,
                          int8_t* q, int64_t ldq, float* scale) {
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; m++) {
        const float* row = v + m * K;
        float amax = 0.0f;
        for (int64_t k = 0; k < K; k++) {
            float a = fabsf(row[k]);
            if (a > amax) amax = a;
        }
        float s = amax / (float)qmax;
        scale[m] = s;
        for (int64_t k = 0; k < K; k++) {
            int c = 0;
            if (s != 0.0f) {
                float t = rintf(row[k] / s);
                if (t > (float)qmax) t = (float)qmax;
                if (t < (float)-qmax) t = (float)-qmax;
                c = (int)t;
            }
            q[m * ldq + k] = (int8_t)c;
        }
    }
}

/* Activation (act, 0 for none), rotation (block 256) or not (block 0), then
 * per-row quantization. */
int oracle_quantize_rowwise_act(const void* x, int dtype, int64_t M, int64_t K, int64_t ldx,
                                int block, int act, int qmax, int8_t* q, int64_t ldq, float* scale) {
    float* v = (float*)malloc((size_t)(M * K) * sizeof(float));
    if (!v) return -2;
    int rc = oracle_rotate_rows_act(x, dtype, M, K, ldx, block, act, v);
    if (rc == 0) oracle_quantize_rows(v, M, K, qmax, q, ldq, scale);
    free(v);
    return rc;
}

int oracle_quantize_rowwise(const void* x, int dtype, int64_t M, int64_t K, int64_t ldx,
                            int block, int qmax, int8_t* q, int64_t ldq, float* scale) {
    return oracle_quantize_rowwise_act(x, dtype, M, K, ldx, block, 0, qmax, q, ldq, scale);
}

/* ---- tensor-wise symmetric quantization --------------------------------- */

/* quantize_int8_tensorwise (comfy-kitchen 0.2.40, "Huawei Ascend backend"):
 * one scale for the whole [M, K] tensor, s = amax / qmax with amax the
 * largest |x| over every element; codes clamp(rne(fl(x / s))); s == 0 gives
 * all-zero codes.  No rotation.  *scale receives s. */
int oracle_quantize_tensorwise(const void* x, int dtype, int64_t M, int64_t K, int64_t ldx,
                               int qmax, int8_t* q, int64_t ldq, float* scale) {
    float tmax = 0.0f;
    for (int64_t r = 0; r < M; r++)
        for (int64_t k = 0; k < K; k++) {
            float a = fabsf(load_elem(x, dtype, r * ldx + k));
            if (a > tmax) tmax = a;
        }
    const float ts = tmax / (float)qmax;
    *scale = ts;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; m++)
        for (int64_t k = 0; k < K; k++) {
            int c = 0;
            if (ts != 0.0f) {
                float t = rintf(load_elem(x, dtype, m * ldx + k) / ts);
                if (t > (float)qmax) t = (float)qmax;
                if (t < (float)-qmax) t = (float)-qmax;
                c = (int)t;
            }
            q[m * ldq + k] = (int8_t)c;
        }
    return 0;
}

/* ---- exact integer GEMM ------------------------------------------------ */

/* acc[m, n] = sum_k a[m, k] * w[n, k]; a is [M, K], w is [N, K] (both K
 * contiguous).  Returns the number of sums that do not fit in int32 (those
 * entries are left saturated), so 0 means every entry is exact. */
int64_t oracle_gemm_i32(const int8_t* a, int64_t M, int64_t K, int64_t lda,
                        const int8_t* w, int64_t N, int64_t ldw, int32_t* acc) {
    int64_t bad = 0;
#pragma omp parallel for schedule(static) reduction(+ : bad)
    for (int64_t m = 0; m < M; m++) {
        for (int64_t n = 0; n < N; n++) {
            int64_t s = 0;
            for (int64_t k = 0; k < K; k++) s += (int64_t)a[m * lda + k] * (int64_t)w[n * ldw + k];
            if (s > INT32_MAX) { s = INT32_MAX; bad++; }
            if (s < INT32_MIN) { s = INT32_MIN; bad++; }
            acc[m * N + n] = (int32_t)s;
        }
    }
    return bad;
}

/* ---- dequantizing epilogue --------------------------------------------- */

static float epilogue_value(int32_t acc, float sx, float sw, const uint16_t* bias, int64_t n) {
    float t = (float)acc;
    t = t * sx;
    t = t * sw;
    if (bias) t = t + bf16_bits_to_float(bias[n]);
    return t;
}

/* y[m, n] (BF16 bits) from INT32 accumulators, row scales, column scales and
 * an optional BF16 bias. */
void oracle_epilogue(const int32_t* acc, int64_t M, int64_t N, const float* sx,
                     const float* sw, const uint16_t* bias, uint16_t* y) {
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; m++)
        for (int64_t n = 0; n < N; n++)
            y[m * N + n] = oracle_bf16_rne(epilogue_value(acc[m * N + n], sx[m], sw[n], bias, n));
}

/* The FP32 value before the final BF16 rounding (used by the pins). */
void oracle_epilogue_f32(const int32_t* acc, int64_t M, int64_t N, const float* sx,
                         const float* sw, const uint16_t* bias, float* t) {
    for (int64_t m = 0; m < M; m++)
        for (int64_t n = 0; n < N; n++)
            t[m * N + n] = epilogue_value(acc[m * N + n], sx[m], sw[n], bias, n);
}

/* ---- the whole layer --------------------------------------------------- */

/* y = epilogue(quantize(rotate(x)) . wq^T).  x is [M, K] in dtype, wq [N, K]
 * INT8 codes (already rotated offline), sw [N], bias [N] BF16 or NULL,
 * y [M, N] BF16 bits.  qmax 127 (INT8) or 7 (INT4 codes in INT8 storage).
 * Returns 0, -1 (bad arguments), -2 (no memory) or -3 (INT32 overflow). */
int oracle_linear_act(const void* x, int dtype, int64_t M, int64_t K, int64_t ldx, int act,
                      const int8_t* wq, const float* sw, const uint16_t* bias, int64_t N,
                      int block, int qmax, uint16_t* y) {
    int8_t* q = (int8_t*)malloc((size_t)(M * K));
    float* sx = (float*)malloc((size_t)M * sizeof(float));
    int32_t* acc = (int32_t*)malloc((size_t)(M * N) * sizeof(int32_t));
    int rc = (q && sx && acc) ? 0 : -2;
    if (rc == 0) rc = oracle_quantize_rowwise_act(x, dtype, M, K, ldx, block, act, qmax, q, K, sx);
    if (rc == 0 && oracle_gemm_i32(q, M, K, K, wq, N, K, acc) != 0) rc = -3;
    if (rc == 0) oracle_epilogue(acc, M, N, sx, sw, bias, y);
    free(q);
    free(sx);
    free(acc);
    return rc;
}

int oracle_linear(const void* x, int dtype, int64_t M, int64_t K, int64_t ldx,
                  const int8_t* wq, const float* sw, const uint16_t* bias, int64_t N,
                  int block, int qmax, uint16_t* y) {
    return oracle_linear_act(x, dtype, M, K, ldx, 0, wq, sw, bias, N, block, qmax, y);
}

/* Selected outputs only: y_out[i] = y[rows[i], cols[i]] for a layer whose
 * activation codes and row scales (aq [.., K], sx) were produced by
 * oracle_quantize_rowwise on the rows in question (aq row i <-> rows[i] is
 * the caller's bookkeeping: aq_row[i] indexes aq). */
void oracle_linear_points(const int8_t* aq, int64_t K, const float* sx, const int64_t* aq_row,
                          const int8_t* wq, const float* sw, const uint16_t* bias,
                          const int64_t* cols, int64_t npts, uint16_t* y_out, int32_t* acc_out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < npts; i++) {
        const int8_t* a = aq + aq_row[i] * K;
        const int8_t* w = wq + cols[i] * K;
        int64_t s = 0;
        for (int64_t k = 0; k < K; k++) s += (int64_t)a[k] * (int64_t)w[k];
        int32_t acc = (int32_t)s;
        if (acc_out) acc_out[i] = acc;
        y_out[i] = oracle_bf16_rne(epilogue_value(acc, sx[aq_row[i]], sw[cols[i]], bias, cols[i]));
    }
}

/* ---- dequantization ---------------------------------------------------- */

/* out = fl(q * s) with s per row (per_row != 0, scale[M]) or per tensor
 * (scale[0]); out_bf16 != 0 rounds the FP32 product to BF16 bits. */
void oracle_dequantize(const int8_t* q, int64_t M, int64_t K, int64_t ldq, const float* scale,
                       int per_row, int out_bf16, void* out) {
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; m++) {
        float s = per_row ? scale[m] : scale[0];
        for (int64_t k = 0; k < K; k++) {
            float v = (float)q[m * ldq + k] * s;
            if (out_bf16) ((uint16_t*)out)[m * K + k] = oracle_bf16_rne(v);
            else ((float*)out)[m * K + k] = v;
        }
    }
}

/* ---- INT4 storage ------------------------------------------------------ */

/* Pack codes in [-8, 7] two per byte along K (low nibble = even index). */
void oracle_pack_int4(const int8_t* q, int64_t R, int64_t K, uint8_t* packed) {
    for (int64_t r = 0; r < R; r++)
        for (int64_t i = 0; i < K / 2; i++) {
            uint8_t lo = (uint8_t)q[r * K + 2 * i] & 0x0f;
            uint8_t hi = (uint8_t)q[r * K + 2 * i + 1] & 0x0f;
            packed[r * (K / 2) + i] = (uint8_t)(lo | (hi << 4));
        }
}

/* Inverse of oracle_pack_int4 (sign-extends each nibble). */
void oracle_unpack_int4(const uint8_t* packed, int64_t R, int64_t K, int8_t* q) {
    for (int64_t r = 0; r < R; r++)
        for (int64_t i = 0; i < K / 2; i++) {
            int lo = packed[r * (K / 2) + i] & 0x0f;
            int hi = packed[r * (K / 2) + i] >> 4;
            q[r * K + 2 * i] = (int8_t)(lo >= 8 ? lo - 16 : lo);
            q[r * K + 2 * i + 1] = (int8_t)(hi >= 8 ? hi - 16 : hi);
        }
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Array form of oracle_bf16_rne. */
void oracle_bf16_rne_array(const float* f, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; i++) out[i] = oracle_bf16_rne(f[i]);
}

/* One query row of INT8 attention on codes (reading in the header): e[j] =
 * exp(S[i][j] - max_j S[i][j]) for the Lk keys of query qi's head; returns
 * sum_j e[j]. */
static double attention_row(const int8_t* qc, const float* sq, const int8_t* kc, const float* sk, int64_t qi,
                            int64_t Lq, int64_t Lk, int64_t D, double scale, double* e) {
    const int64_t bh = qi / Lq;
    double mx = -INFINITY;
    for (int64_t j = 0; j < Lk; j++) {
        const int64_t kr = bh * Lk + j;
        int64_t acc = 0;
        for (int64_t d = 0; d < D; d++) acc += (int64_t)qc[qi * D + d] * (int64_t)kc[kr * D + d];
        e[j] = (double)acc * (double)sq[qi] * (double)sk[kr] * scale;
        if (e[j] > mx) mx = e[j];
    }
    double den = 0.0;
    for (int64_t j = 0; j < Lk; j++) {
        e[j] = exp(e[j] - mx);
        den += e[j];
    }
    return den;
}

/* INT8 attention on codes (reading in the header).  qc [BH*Lq, D], kc and vc
 * [BH*Lk, D] INT8 codes with one FP32 scale per row; out [BH*Lq, D] double. */
void oracle_attention_i8(const int8_t* qc, const float* sq, const int8_t* kc, const float* sk,
                         const int8_t* vc, const float* sv, int64_t BH, int64_t Lq, int64_t Lk,
                         int64_t D, double scale, double* out) {
#pragma omp parallel for schedule(static)
    for (int64_t qi = 0; qi < BH * Lq; qi++) {
        const int64_t bh = qi / Lq;
        double* sc = (double*)malloc((size_t)Lk * sizeof(double));
        const double den = attention_row(qc, sq, kc, sk, qi, Lq, Lk, D, scale, sc);
        for (int64_t d = 0; d < D; d++) {
            double num = 0.0;
            for (int64_t j = 0; j < Lk; j++) {
                const int64_t vr = bh * Lk + j;
                num += sc[j] * ((double)sv[vr] * (double)vc[vr * D + d]);
            }
            out[qi * D + d] = num / den;
        }
        free(sc);
    }
}

/* The softmax probabilities of INT8 attention on codes: P [BH*Lq, Lk]
 * double, P[i][j] = exp(S[i][j] - max_j S[i][j]) / sum_j of the same, so
 * that out = P (sv * v) row by row. */
void oracle_attention_probs(const int8_t* qc, const float* sq, const int8_t* kc, const float* sk,
                            int64_t BH, int64_t Lq, int64_t Lk, int64_t D, double scale, double* P) {
#pragma omp parallel for schedule(static)
    for (int64_t qi = 0; qi < BH * Lq; qi++) {
        double* pr = P + qi * Lk;
        const double den = attention_row(qc, sq, kc, sk, qi, Lq, Lk, D, scale, pr);
        for (int64_t j = 0; j < Lk; j++) pr[j] = pr[j] / den;
    }
}
