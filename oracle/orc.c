/*
 * orc.c -- CPU oracle for per-row symmetric weight quantization.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's CPU
 * baseline may load this library.  It shares no code, header, table or helper with
 * the GPU library; the two meet only through the seeded synthetic inputs.
 *
 * Plain, slow and single-threaded on purpose: every value is computed with IEEE-754
 * binary32 basic operations (+ - * / sqrt, compare) in the order written, followed by
 * explicit round-to-nearest-even conversions that this file implements from the
 * format definitions.  Build with -O2 -ffp-contract=off -fno-fast-math (x86-64 SSE
 * scalar arithmetic, default rounding, no flush-to-zero), so that a*b+c is never
 * fused and divisions and square roots are correctly rounded.
 *
 * What it follows (Parameter Golf submission pages):
 *   - "Swiglu gating ... 10min/16MB Track" (PR #2159), list "Key Explored
 *     Modifications": per-row / per-tensor quantization, percentile clipping for
 *     export, small-tensor FP16 passthrough, STE-based fake quantization.
 *   - "SubSixteen v2: Int6 QAT + MLP 3x + SWA" card (PR #69), section Quantization
 *     (STE QAT, 6 bits) and section Other (STE fake quantization in the forward pass,
 *     quant range [-31, 31]).
 *   - "12L 24min Vocab1792 ... Int6AWQ MixedBits" (PR #1495), Submission summary
 *     (mixed-bit int6 AWQ export) and Mixed-bit quantization details (int8 for the
 *     named sensitive tensors).
 *   - "Discriminative TTT + SLOT-24" card (PR #1414), Novel Contributions: averaging
 *     quantize-dequantize snapshots (SQWA); Weight Averaging: EMA with decay 0.997.
 *   - "SubSixteen v2" card (PR #69), Novel Contributions and Weight Averaging: SWA over 16
 *     checkpoints.
 * Where the pages leave the arithmetic open (rounding of the scale, tie rule, zero
 * scale, percentile rank, mask boundary, AWQ exponent) the readings are: scale =
 * fp16_rne(fp32(clip / Q)), 1.0 when that is zero; codes = clamp(rne(fp32(x / s)));
 * k = ceil(num * n / den) computed in integers; mask = |x / s| <= Q + 1/2 on the fp32
 * quotient; AWQ multiplier a_j = fp16_rne(sqrt(s_j)).
 *
 * Parity pins for every function here live in tests/test_oracle_*.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_NONFINITE 1u
#define ORC_SCALE_OVF 2u
#define ORC_F16_OVF   4u
#define ORC_BAD_AWQ   8u

static uint32_t bits_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float float_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* Round the non-negative integer m / 2^sh to the nearest integer, ties to even. */
static uint64_t shift_rne(uint64_t m, int sh)
{
    if (sh <= 0) return m << (-sh);
    if (sh >= 64) return 0;
    uint64_t q = m >> sh;
    uint64_t rem = m - (q << sh);
    uint64_t half = (uint64_t)1 << (sh - 1);
    if (rem > half || (rem == half && (q & 1))) q += 1;
    return q;
}

/* binary32 -> binary16, round to nearest even, with gradual underflow and
 * overflow to infinity (IEEE 754-2008 convertFormat). */
uint16_t orc_f32_to_f16(float f)
{
    uint32_t u = bits_of(f);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    uint32_t biased = (u >> 23) & 0xFFu;
    uint32_t frac = u & 0x7FFFFFu;
    if (biased == 0xFFu) {
        if (frac == 0) return sign | 0x7C00u;                 /* infinity */
        return sign | 0x7E00u | (uint16_t)(frac >> 13);        /* quiet NaN, payload kept */
    }
    if (biased == 0) return sign;   /* binary32 subnormals are below half the smallest binary16 subnormal */
    /* value = m * 2^(e - 23), m in [2^23, 2^24) */
    int e = (int)biased - 127;
    uint64_t m = (uint64_t)frac | 0x800000u;
    if (e >= -14) {
        /* normal binary16 range: 10 fraction bits, so count units of 2^(e - 10) */
        uint64_t n = shift_rne(m, 13);          /* in [2^10, 2^11] */
        int ee = e;
        if (n == 2048) { n = 1024; ee += 1; }
        if (ee > 15) return sign | 0x7C00u;
        return sign | (uint16_t)(((uint32_t)(ee + 15) << 10) | (uint32_t)(n - 1024));
    }
    /* subnormal binary16: count units of 2^-24; value / 2^-24 = m * 2^(e + 1) */
    uint64_t n = shift_rne(m, -(e + 1));        /* 0 .. 1024; 1024 is the smallest normal */
    return sign | (uint16_t)n;
}

/* binary16 -> binary32 (exact). */
float orc_f16_to_f32(uint16_t h)
{
    uint32_t sign = ((uint32_t)h & 0x8000u) << 16;
    uint32_t ex = ((uint32_t)h >> 10) & 0x1Fu;
    uint32_t fr = (uint32_t)h & 0x3FFu;
    if (ex == 0x1Fu) return float_of(sign | 0x7F800000u | (fr << 13));
    if (ex == 0) {
        /* fr * 2^-24, exact in binary32 */
        float v = (float)fr * 0x1p-24f;
        return float_of(sign | bits_of(v));
    }
    return float_of(sign | ((ex - 15 + 127) << 23) | (fr << 13));
}

/* binary32 -> bfloat16 (8 exponent bits, 7 fraction bits), round to nearest even. */
uint16_t orc_f32_to_bf16(float f)
{
    uint32_t u = bits_of(f);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x7FFFFFu))
        return (uint16_t)((u >> 16) | 0x40u);                  /* quiet NaN */
    uint32_t hi = u >> 16, lo = u & 0xFFFFu;
    if (lo > 0x8000u || (lo == 0x8000u && (hi & 1u))) hi += 1; /* may carry into the exponent: correct */
    return (uint16_t)hi;
}

float orc_bf16_to_f32(uint16_t b) { return float_of((uint32_t)b << 16); }

void orc_f32_to_f16_n(const float* x, uint16_t* y, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) y[i] = orc_f32_to_f16(x[i]);
}

void orc_f32_to_bf16_n(const float* x, uint16_t* y, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) y[i] = orc_f32_to_bf16(x[i]);
}

/* Rank of the percentile clip: the k-th smallest |x| with k = ceil(num * n / den),
 * computed exactly in integers and clamped to [1, n]. */
int64_t orc_percentile_rank(int64_t n, uint32_t num, uint32_t den)
{
    if (n <= 0 || den == 0) return 0;
    unsigned __int128 p = (unsigned __int128)num * (unsigned __int128)n;
    int64_t k = (int64_t)((p + den - 1) / den);
    if (k < 1) k = 1;
    if (k > n) k = n;
    return k;
}

static int cmp_abs(const void* pa, const void* pb)
{
    float a = *(const float*)pa, b = *(const float*)pb;
    int na = isnan(a), nb = isnan(b);
    if (na || nb) return na - nb;              /* NaN sorts last */
    return (a > b) - (a < b);
}

/* One row.  x: n input values (already binary32); awq: n binary16 multipliers or NULL.
 * Outputs (each nullable except scale): codes[n], dq[n], t[n] (the quotient x/s),
 * clip.  Returns status bits. */
uint32_t orc_quantize_row(const float* w, int64_t n, int32_t Q, uint32_t num, uint32_t den,
                          const uint16_t* awq, int8_t* codes, uint16_t* scale, float* dq,
                          float* tq, float* clip_out)
{
    uint32_t st = 0;
    float* x = (float*)malloc((size_t)n * sizeof(float));
    float* mag = (float*)malloc((size_t)n * sizeof(float));
    /* step 1: the row in binary32, with the AWQ column multiplier applied first */
    for (int64_t j = 0; j < n; ++j) {
        float v = w[j];
        if (awq) v = v * orc_f16_to_f32(awq[j]);
        x[j] = v;
        if (!isfinite(v)) st |= ORC_NONFINITE;
        mag[j] = fabsf(v);
    }
    /* step 2: the clip is the k-th smallest magnitude (k = n gives the absolute maximum) */
    int64_t k = orc_percentile_rank(n, num, den);
    qsort(mag, (size_t)n, sizeof(float), cmp_abs);
    float clip = mag[k - 1];
    if (clip_out) *clip_out = clip;
    /* step 3: scale = fp16(clip / Q), replaced by 1 when it rounds to zero */
    float s32 = clip / (float)Q;
    uint16_t s16 = orc_f32_to_f16(s32);
    if ((s16 & 0x7FFFu) == 0) s16 = 0x3C00u;
    if ((s16 & 0x7FFFu) == 0x7C00u) st |= ORC_SCALE_OVF;
    *scale = s16;
    float s = orc_f16_to_f32(s16);
    /* steps 4 and 5: code = clamp(rne(x / s), -Q, Q); dequant = code * s (AWQ: / a_j) */
    for (int64_t j = 0; j < n; ++j) {
        float t = x[j] / s;
        float r = rintf(t);                       /* default rounding mode: ties to even */
        int32_t q;
        if (isnan(r)) q = 0;
        else if (r < (float)(-Q)) q = -Q;
        else if (r > (float)Q) q = Q;
        else q = (int32_t)r;
        if (codes) codes[j] = (int8_t)q;
        if (tq) tq[j] = t;
        if (dq) {
            float d = (float)q * s;
            if (awq) d = d / orc_f16_to_f32(awq[j]);
            dq[j] = d;
        }
    }
    free(mag);
    free(x);
    return st;
}

/* rows x cols matrix with row stride ld (elements); codes/dq are dense rows x cols. */
uint32_t orc_quantize_rows(const float* w, int64_t rows, int64_t cols, int64_t ld, int32_t Q,
                           uint32_t num, uint32_t den, const uint16_t* awq, int8_t* codes,
                           uint16_t* scales, float* dq, float* tq, float* clips)
{
    uint32_t st = 0;
    for (int64_t r = 0; r < rows; ++r)
        st |= orc_quantize_row(w + r * ld, cols, Q, num, den, awq,
                               codes ? codes + r * cols : NULL, scales + r,
                               dq ? dq + r * cols : NULL, tq ? tq + r * cols : NULL,
                               clips ? clips + r : NULL);
    return st;
}

/* Per-tensor quantization ("Per-row / per-tensor quantization strategy" with "Percentile
 * clipping for stable int8 export", PR #2159 Key Explored Modifications): one scale for the
 * whole tensor, the clip being the k-th smallest |w| over all rows * cols elements.  That is
 * the row quantizer applied to the tensor read as one row; codes / dq are dense rows x cols. */
uint32_t orc_quantize_tensor(const float* w, int64_t rows, int64_t cols, int64_t ld, int32_t Q,
                             uint32_t num, uint32_t den, int8_t* codes, uint16_t* scale, float* dq,
                             float* clip)
{
    int64_t n = rows * cols;
    float* flat = (float*)malloc((size_t)(n > 0 ? n : 1) * sizeof(float));
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t j = 0; j < cols; ++j) flat[r * cols + j] = w[r * ld + j];
    uint32_t st = orc_quantize_row(flat, n, Q, num, den, NULL, codes, scale, dq, NULL, clip);
    free(flat);
    return st;
}

/* 6-bit code storage (the "int6 artifact savings" of the PR #69 card's Novel Contributions; the
 * pages give no byte layout).  Reading: each row's int6 codes, as 6-bit two's complement, four
 * to three bytes, least significant bits first: group g holds codes 4g .. 4g+3 in the 24-bit
 * little-endian word bytes[3g] | bytes[3g+1] << 8 | bytes[3g+2] << 16, code 4g + t in bits
 * 6t .. 6t+5.  A row takes 3 * ceil(cols / 4) bytes; a short last group is padded with code 0. */
int64_t orc_pack6_row_bytes(int64_t cols) { return 3 * ((cols + 3) / 4); }

void orc_pack6_rows(const int8_t* codes, int64_t rows, int64_t cols, uint8_t* out)
{
    int64_t rb = orc_pack6_row_bytes(cols);
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t g = 0; g < (cols + 3) / 4; ++g) {
            uint32_t word = 0;
            for (int t = 0; t < 4; ++t) {
                int64_t j = 4 * g + t;
                int32_t c = j < cols ? codes[r * cols + j] : 0;
                word |= ((uint32_t)c & 0x3Fu) << (6 * t);
            }
            out[r * rb + 3 * g] = (uint8_t)(word & 0xFFu);
            out[r * rb + 3 * g + 1] = (uint8_t)((word >> 8) & 0xFFu);
            out[r * rb + 3 * g + 2] = (uint8_t)((word >> 16) & 0xFFu);
        }
    }
}

void orc_unpack6_rows(const uint8_t* in, int64_t rows, int64_t cols, int8_t* codes)
{
    int64_t rb = orc_pack6_row_bytes(cols);
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t j = 0; j < cols; ++j) {
            int64_t g = j / 4;
            uint32_t word = (uint32_t)in[r * rb + 3 * g] | ((uint32_t)in[r * rb + 3 * g + 1] << 8) |
                            ((uint32_t)in[r * rb + 3 * g + 2] << 16);
            int32_t f = (int32_t)((word >> (6 * (j % 4))) & 0x3Fu);
            codes[r * cols + j] = (int8_t)(f >= 32 ? f - 64 : f);
        }
}

/* Decode of stored codes (the dequant the export defines): x = code * s, divided by a_j when the
 * tensor has AWQ multipliers; s = scales[r], or scales[0] for a per-tensor scale. */
void orc_dequant_rows(const int8_t* codes, int64_t rows, int64_t cols, const uint16_t* scales, int32_t per_tensor,
                      const uint16_t* awq, float* out)
{
    for (int64_t r = 0; r < rows; ++r) {
        float s = orc_f16_to_f32(scales[per_tensor ? 0 : r]);
        for (int64_t j = 0; j < cols; ++j) {
            float d = (float)codes[r * cols + j] * s;
            if (awq) d = d / orc_f16_to_f32(awq[j]);
            out[r * cols + j] = d;
        }
    }
}

/* The QAT forward's consumer GEMM with the fake-quantized weights (STE fake quantization in the
 * forward pass, PR #69 card section Other): Y = X * What^T, X bf16 [M x K] (row stride ldx),
 * What[n][k] = bf16_rne(fp32(code[n][k] * s_n)) -- the STE forward's dequantized weight -- from
 * int8 codes [N x K] (row stride ldc) and fp16 row scales.  Accumulated in double: every product
 * of two bf16 values is exact in double, so y is the exact sum up to double rounding.  bound[m][n]
 * receives sum_k |x * What| (for the tolerance of a binary32 accumulation). */
void orc_qgemm_bf16(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const int8_t* codes, int64_t ldc,
                    const uint16_t* scales, int64_t N, double* y, double* bound)
{
    float* wq = (float*)malloc((size_t)(N * K > 0 ? N * K : 1) * sizeof(float));
    for (int64_t n = 0; n < N; ++n) {
        float s = orc_f16_to_f32(scales[n]);
        for (int64_t k = 0; k < K; ++k) {
            float d = (float)codes[n * ldc + k] * s;
            wq[n * K + k] = orc_bf16_to_f32(orc_f32_to_bf16(d));
        }
    }
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0, mag = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double p = (double)orc_bf16_to_f32(x[m * ldx + k]) * (double)wq[n * K + k];
                acc += p;
                mag += fabs(p);
            }
            y[m * N + n] = acc;
            if (bound) bound[m * N + n] = mag;
        }
    free(wq);
}

/* AWQ column multipliers a_j = fp16_rne(sqrt(s_j)) (exponent 1/2), s_j > 0 and finite. */
uint32_t orc_awq_multipliers(const float* s, int64_t cols, uint16_t* a)
{
    uint32_t st = 0;
    for (int64_t j = 0; j < cols; ++j) {
        float v = s[j];
        if (!(v > 0.0f) || !isfinite(v)) st |= ORC_BAD_AWQ;
        a[j] = orc_f32_to_f16(sqrtf(v));
    }
    return st;
}

/* STE fake quantization of a bfloat16 matrix (forward and backward).
 * Forward: dq = bf16_rne(code * s); mask bit j = (|x_j / s| <= Q + 1/2), row-major,
 * least significant bit first, ceil(cols / 8) bytes per row.
 * Backward: g_out = mask ? g : +0.  g / g_out may be NULL (forward only). */
uint32_t orc_fakequant_rows(const uint16_t* w, int64_t rows, int64_t cols, int64_t ld, int32_t Q,
                            uint32_t num, uint32_t den, uint16_t* dq, uint16_t* scales,
                            uint8_t* mask, const uint16_t* g, uint16_t* g_out, int8_t* codes)
{
    uint32_t st = 0;
    int64_t mb = (cols + 7) / 8;
    float* x = (float*)malloc((size_t)cols * sizeof(float));
    float* t = (float*)malloc((size_t)cols * sizeof(float));
    float* d = (float*)malloc((size_t)cols * sizeof(float));
    int8_t* c = (int8_t*)malloc((size_t)cols);
    float lim = (float)Q + 0.5f;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t j = 0; j < cols; ++j) x[j] = orc_bf16_to_f32(w[r * ld + j]);
        st |= orc_quantize_row(x, cols, Q, num, den, NULL, c, scales + r, d, t, NULL);
        if (mask) memset(mask + r * mb, 0, (size_t)mb);
        for (int64_t j = 0; j < cols; ++j) {
            int keep = fabsf(t[j]) <= lim;
            if (dq) dq[r * cols + j] = orc_f32_to_bf16(d[j]);
            if (codes) codes[r * cols + j] = c[j];
            if (mask && keep) mask[r * mb + j / 8] |= (uint8_t)(1u << (j % 8));
            if (g && g_out) g_out[r * cols + j] = keep ? g[r * cols + j] : (uint16_t)0;
        }
    }
    free(c); free(d); free(t); free(x);
    return st;
}

/* fp16 passthrough: y_j = fp16_rne(x_j). */
uint32_t orc_f16_passthrough(const float* x, int64_t n, uint16_t* y)
{
    uint32_t st = 0;
    for (int64_t j = 0; j < n; ++j) {
        y[j] = orc_f32_to_f16(x[j]);
        if (!isfinite(x[j])) st |= ORC_NONFINITE;
        else if ((y[j] & 0x7FFFu) == 0x7C00u) st |= ORC_F16_OVF;
    }
    return st;
}

/* Exponential moving average of the weights (the "EMA" weight averaging of the PR #1414 and
 * PR #1202 cards, section Weight Averaging, decay 0.997): after a step, e = decay * e +
 * (1 - decay) * w; the first update (init != 0) starts the average at the weights, e = w.
 * Reading of the arithmetic (the pages give only the decay): binary32 throughout; the weight
 * factor c = fp32(1 - decay) is formed once; then fp32(fp32(decay * e) + fp32(c * w)), two
 * products and a sum, no fused multiply-add.  Returns NONFINITE when a weight or a new
 * average is NaN or infinite. */
uint32_t orc_ema_update(float* e, const float* w, int64_t n, float decay, int32_t init)
{
    uint32_t st = 0;
    const float c = 1.0f - decay;
    for (int64_t j = 0; j < n; ++j) {
        if (init) {
            e[j] = w[j];
        } else {
            float kept = decay * e[j];
            float added = c * w[j];
            e[j] = kept + added;
        }
        if (!isfinite(w[j]) || !isfinite(e[j])) st |= ORC_NONFINITE;
    }
    return st;
}

/* SWA (PR #69 card: "Stochastic Weight Averaging over 16 checkpoints", Weight Averaging
 * parameters checkpoints 16, interval 200 steps): the arithmetic mean of the checkpoints
 * handed over in order, k = 1, 2, ..., kept as a running mean with the same binary32 update
 * as orc_sqwa_update below (there on quantize-dequantized snapshots, here on the weights). */
void orc_sqwa_update(float* mean, const float* xhat, int64_t n, int32_t k);

uint32_t orc_swa_update(float* mean, const float* w, int64_t n, int32_t k)
{
    uint32_t st = 0;
    orc_sqwa_update(mean, w, n, k);
    for (int64_t j = 0; j < n; ++j)
        if (!isfinite(w[j]) || !isfinite(mean[j])) st |= ORC_NONFINITE;
    return st;
}

/* SQWA running mean over snapshots k = 1, 2, ...:  mean = xhat when k = 1, else
 * mean = mean + (xhat - mean) / k, three correctly rounded binary32 operations. */
void orc_sqwa_update(float* mean, const float* xhat, int64_t n, int32_t k)
{
    if (k == 1) {
        for (int64_t j = 0; j < n; ++j) mean[j] = xhat[j];
        return;
    }
    float kf = (float)k;
    for (int64_t j = 0; j < n; ++j) {
        float diff = xhat[j] - mean[j];
        float step = diff / kf;
        mean[j] = mean[j] + step;
    }
}
