/*
 * q4_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * The plain, slow, single-threaded fp64 CPU definition of what the INT4
 * weight-streaming decode path computes.  Only the tests, the smoke check
 * and the CPU-baseline leg of the benchmark may load this library; the
 * product path never calls it and shares no code, header or table with it.
 *
 * What is computed, and where it comes from:
 *
 *   PIPO: Pipelined Offloading for Efficient Inference on Consumer Devices,
 *   "Method", bullet "Computation optimization": the kernel multiplies a
 *   vector directly by 4-bit quantized weights without first dequantizing
 *   them.  The result it reaches is, up to summation order, the ordinary
 *   matrix-vector product with the dequantized matrix, so this file writes
 *   that definition out: dequantize one weight, multiply, add, in k order.
 *
 *   The pages give no bit layout.  The reading used throughout (and stated
 *   in the design notes):
 *     - codes are unsigned 4-bit values 0..15 with zero point 8;
 *     - weight w[n][k] = s[n][k/32] * (c[n][k] - 8);
 *     - one IEEE binary16 scale per group of 32 consecutive k, scales stored
 *       row-major [N][K/32];
 *     - two codes per byte, row-major [N][K/2]: byte j of a row holds
 *       code 2j in bits 0..3 and code 2j+1 in bits 4..7;
 *     - codes given to pack are masked to their low nibble.
 *
 *   The decode-layer glue (RMSNorm, one-token attention stand-in, SiLU gate)
 *   is not described on the pages at all; what is written here is the plain
 *   Llama-shaped reading of a per-layer decode step whose matrices are fused
 *   QKV, O, fused gate+up and down (see q4o_decode_layer).
 *
 * Everything is fp64 except where the method itself stores fp16: the
 * activation vectors fed to each matrix product are binary16, rounded
 * to nearest-even by q4o_f64_to_f16 below.
 *
 * Parity pins for every function live in tests/test_oracle_pins.py.
 *
 * Built single-threaded (oracle.build).  Only the CPU-baseline leg of the
 * benchmark also times an all-core build of this file (oracle.build_omp,
 * -fopenmp: the product rows split over threads), labelled as a baseline,
 * never used as the oracle.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* binary16 <-> double, written from the IEEE 754 definition            */
/* ------------------------------------------------------------------ */

/* IEEE 754-2008 binary16: 1 sign bit, 5 exponent bits (bias 15), 10
 * fraction bits.  exponent 0 = zero/subnormal (value = f * 2^-24),
 * exponent 31 = inf/nan, otherwise (1024 + f) * 2^(e - 25). */
double q4o_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int f = h & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = (f == 0) ? INFINITY : NAN;
    else
        v = ldexp((double)(1024 + f), e - 25);
    return sign ? -v : v;
}

/* Round a non-negative double that holds an exact value q (< 2^12) to the
 * nearest integer, ties to even. */
static double round_half_even(double q)
{
    double fl = floor(q);
    double fr = q - fl; /* exact: q has few integer bits */
    if (fr > 0.5)
        return fl + 1.0;
    if (fr < 0.5)
        return fl;
    return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
}

/* double -> binary16, round to nearest, ties to even; overflow -> inf. */
uint16_t q4o_f64_to_f16(double v)
{
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    double a = fabs(v);
    if (isnan(v))
        return (uint16_t)(sign | 0x7E00u);
    /* 65504 is the largest finite value; 65520 is the midpoint to the next
     * (virtual) step, and ties go to the even neighbour, which is inf. */
    if (a >= 65520.0)
        return (uint16_t)(sign | 0x7C00u);
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: fixed quantum 2^-24.  r may reach 1024, which is
         * exactly the encoding of the smallest normal number. */
        double r = round_half_even(ldexp(a, 24));
        return (uint16_t)(sign | (uint16_t)r);
    }
    int e2;
    frexp(a, &e2); /* a in [2^(e2-1), 2^e2) */
    int unb = e2 - 1; /* unbiased exponent, -14..15 */
    double r = round_half_even(ldexp(a, 10 - unb)); /* in [1024, 2048] */
    /* r == 2048 carries into the exponent field, which is what the plain
     * sum below does. */
    uint32_t bits = ((uint32_t)(unb + 15) << 10) + ((uint32_t)r - 1024u);
    return (uint16_t)(sign | bits);
}

void q4o_f16_to_f64_array(const uint16_t *h, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = q4o_f16_to_f64(h[i]);
}

void q4o_f64_to_f16_array(const double *v, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = q4o_f64_to_f16(v[i]);
}

/* ------------------------------------------------------------------ */
/* packing                                                              */
/* ------------------------------------------------------------------ */

/* codes u8[N][K] (only the low nibble is used) -> packed u8[N][K/2]. */
void q4o_pack(const uint8_t *codes, uint8_t *packed, int64_t N, int64_t K)
{
    for (int64_t n = 0; n < N; ++n)
        for (int64_t j = 0; j < K / 2; ++j) {
            uint8_t lo = codes[n * K + 2 * j] & 0x0F;
            uint8_t hi = codes[n * K + 2 * j + 1] & 0x0F;
            packed[n * (K / 2) + j] = (uint8_t)(lo | (hi << 4));
        }
}

/* packed u8[N][K/2] -> codes u8[N][K], each 0..15. */
void q4o_unpack(const uint8_t *packed, uint8_t *codes, int64_t N, int64_t K)
{
    for (int64_t n = 0; n < N; ++n)
        for (int64_t j = 0; j < K / 2; ++j) {
            uint8_t b = packed[n * (K / 2) + j];
            codes[n * K + 2 * j] = b & 0x0F;
            codes[n * K + 2 * j + 1] = b >> 4;
        }
}

/* One dequantized weight, straight from the definition. */
static double weight_at(const uint8_t *packed, const uint16_t *scales,
                        int64_t K, int64_t n, int64_t k)
{
    uint8_t b = packed[n * (K / 2) + k / 2];
    int code = (k % 2 == 0) ? (b & 0x0F) : (b >> 4);
    double s = q4o_f16_to_f64(scales[n * (K / 32) + k / 32]);
    return s * (double)(code - 8);
}

/* Dense fp64 dequantized matrix W[N][K] (small cases only). */
void q4o_dequant(const uint8_t *packed, const uint16_t *scales, double *W,
                 int64_t N, int64_t K)
{
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            W[n * K + k] = weight_at(packed, scales, K, n, k);
}

/* ------------------------------------------------------------------ */
/* matrix-vector and small-batch products                               */
/* ------------------------------------------------------------------ */

/* binary16 -> double for every bit pattern, filled once from
 * q4o_f16_to_f64 above (a lookup, not a second decoder). */
static double g_f16_table[65536];
static int g_f16_table_ready = 0;

static void f16_table_init(void)
{
    if (!g_f16_table_ready) {
        for (uint32_t h = 0; h < 65536; ++h)
            g_f16_table[h] = q4o_f16_to_f64((uint16_t)h);
        g_f16_table_ready = 1;
    }
}

/* One output row: y = sum_k w[n][k] * x[k] in k order, and the magnitude
 * m = sum_k |w[n][k] * x[k]| that scales the acceptance bound.  The scale
 * of a group is decoded once for its 32 columns. */
static void row_dot(const uint8_t *packed, const uint16_t *scales,
                    const double *x, int64_t K, int64_t n,
                    double *y, double *m)
{
    double acc = 0.0, mag = 0.0;
    const uint8_t *prow = packed + n * (K / 2);
    const uint16_t *srow = scales + n * (K / 32);
    for (int64_t g = 0; g < K / 32; ++g) {
        double s = g_f16_table[srow[g]];
        for (int64_t k = 32 * g; k < 32 * g + 32; ++k) {
            uint8_t b = prow[k / 2];
            int code = (k % 2 == 0) ? (b & 0x0F) : (b >> 4);
            double w = s * (double)(code - 8);
            double t = w * x[k];
            acc += t;
            mag += fabs(t);
        }
    }
    *y = acc;
    if (m)
        *m = mag;
}

/* y[n] = sum_k w[n][k] * x[k] for binary16 x.  mag may be NULL.
 * The oracle is built without OpenMP, so the pragma below does nothing; the
 * separately labelled all-core CPU baseline compiles this same file with
 * -fopenmp, which splits the rows (each row's sum is unchanged). */
void q4o_gemv(const uint8_t *packed, const uint16_t *scales,
              const uint16_t *x_f16, int64_t N, int64_t K,
              double *y, double *mag)
{
    double *x = (double *)malloc(sizeof(double) * (size_t)K);
    f16_table_init();
    q4o_f16_to_f64_array(x_f16, x, K);
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        row_dot(packed, scales, x, K, n, &y[n], mag ? &mag[n] : NULL);
    free(x);
}

/* Same product for a chosen subset of rows (used to check very large
 * matrices one output at a time).  y and mag are indexed like rows. */
void q4o_gemv_rows(const uint8_t *packed, const uint16_t *scales,
                   const uint16_t *x_f16, int64_t K,
                   const int64_t *rows, int64_t nrows,
                   double *y, double *mag)
{
    double *x = (double *)malloc(sizeof(double) * (size_t)K);
    f16_table_init();
    q4o_f16_to_f64_array(x_f16, x, K);
    for (int64_t i = 0; i < nrows; ++i)
        row_dot(packed, scales, x, K, rows[i], &y[i], mag ? &mag[i] : NULL);
    free(x);
}

/* Y[b][n] = sum_k w[n][k] * X[b][k]; X is binary16 [B][K]. */
void q4o_gemm(const uint8_t *packed, const uint16_t *scales,
              const uint16_t *X_f16, int64_t N, int64_t K, int64_t B,
              double *Y, double *M)
{
    for (int64_t b = 0; b < B; ++b)
        q4o_gemv(packed, scales, X_f16 + b * K, N, K, Y + b * N,
                 M ? M + b * N : NULL);
}

/* ------------------------------------------------------------------ */
/* decode-layer glue (a reading: the pages describe none of it)          */
/* ------------------------------------------------------------------ */

/* a = f16(h / sqrt(mean(h^2) + eps)), unit gain. */
void q4o_rmsnorm_f16(const double *h, int64_t d, double eps, uint16_t *a)
{
    double ss = 0.0;
    for (int64_t i = 0; i < d; ++i)
        ss += h[i] * h[i];
    double r = 1.0 / sqrt(ss / (double)d + eps);
    for (int64_t i = 0; i < d; ++i)
        a[i] = q4o_f64_to_f16(h[i] * r);
}

/* One-token attention: with a single key, softmax is 1 and RoPE at
 * position 0 is the identity, so query head hq outputs the V vector of its
 * key/value group hq / (H / Hkv).  qkv holds Q | K | V (H*hd, Hkv*hd,
 * Hkv*hd values); out is f16[H*hd]. */
void q4o_gqa_gather_f16(const double *qkv, int64_t H, int64_t Hkv,
                        int64_t hd, uint16_t *out)
{
    const double *V = qkv + (H + Hkv) * hd;
    int64_t per_group = H / Hkv;
    for (int64_t hq = 0; hq < H; ++hq) {
        int64_t g = hq / per_group;
        for (int64_t i = 0; i < hd; ++i)
            out[hq * hd + i] = q4o_f64_to_f16(V[g * hd + i]);
    }
}

/* Rotary position embedding, rotate-half form: for i < hd/2, dims i and
 * i + hd/2 of a head vector turn by the angle pos * base^(-2i/hd). */
void q4o_rope(double *x, int64_t hd, int64_t pos, double base)
{
    int64_t half = hd / 2;
    for (int64_t i = 0; i < half; ++i) {
        double ang = (double)pos * pow(base, -2.0 * (double)i / (double)hd);
        double c = cos(ang), s = sin(ang);
        double a = x[i], b = x[i + half];
        x[i] = a * c - b * s;
        x[i + half] = a * s + b * c;
    }
}

/*
 * Decode attention of one token at position pos with grouped-query heads
 * (query head hq reads key/value head hq / (H / Hkv)).  qkv holds Q | K | V
 * for this token.  The rotated key and the value are first stored, rounded
 * to binary16, into row pos of the caches (layout [Hkv][max_ctx][hd]); then
 * every query head, rotated at pos, attends over rows 0..pos of its
 * group's caches:
 *     s_j = (q . k_j) / sqrt(hd),   p = softmax(s),   o = sum_j p_j v_j.
 * out: o (fp64, [H*hd]); mag (may be NULL): sum_j p_j |v_j| per element,
 * the scale of the rounding error of an fp32 evaluation.
 */
void q4o_attention(const double *qkv, int64_t H, int64_t Hkv, int64_t hd,
                   int64_t pos, int64_t max_ctx, double base,
                   uint16_t *kcache, uint16_t *vcache, double *out, double *mag)
{
    int64_t per_group = H / Hkv;
    double *q = (double *)malloc(sizeof(double) * (size_t)hd);
    double *k = (double *)malloc(sizeof(double) * (size_t)hd);
    double *s = (double *)malloc(sizeof(double) * (size_t)(pos + 1));
    for (int64_t g = 0; g < Hkv; ++g) {
        const double *kn = qkv + (H + g) * hd;
        const double *vn = qkv + (H + Hkv + g) * hd;
        for (int64_t i = 0; i < hd; ++i)
            k[i] = kn[i];
        q4o_rope(k, hd, pos, base);
        uint16_t *krow = kcache + (g * max_ctx + pos) * hd;
        uint16_t *vrow = vcache + (g * max_ctx + pos) * hd;
        for (int64_t i = 0; i < hd; ++i) {
            krow[i] = q4o_f64_to_f16(k[i]);
            vrow[i] = q4o_f64_to_f16(vn[i]);
        }
    }
    double scale = 1.0 / sqrt((double)hd);
    for (int64_t hq = 0; hq < H; ++hq) {
        int64_t g = hq / per_group;
        for (int64_t i = 0; i < hd; ++i)
            q[i] = qkv[hq * hd + i];
        q4o_rope(q, hd, pos, base);
        double smax = -INFINITY;
        for (int64_t j = 0; j <= pos; ++j) {
            const uint16_t *kr = kcache + (g * max_ctx + j) * hd;
            double dot = 0.0;
            for (int64_t i = 0; i < hd; ++i)
                dot += q[i] * q4o_f16_to_f64(kr[i]);
            s[j] = dot * scale;
            if (s[j] > smax)
                smax = s[j];
        }
        double sum = 0.0;
        for (int64_t j = 0; j <= pos; ++j) {
            s[j] = exp(s[j] - smax);
            sum += s[j];
        }
        for (int64_t i = 0; i < hd; ++i) {
            double acc = 0.0, m = 0.0;
            for (int64_t j = 0; j <= pos; ++j) {
                double v = q4o_f16_to_f64(vcache[(g * max_ctx + j) * hd + i]);
                acc += (s[j] / sum) * v;
                m += (s[j] / sum) * fabs(v);
            }
            out[hq * hd + i] = acc;
            if (mag)
                mag[hq * hd + i] = m;
        }
    }
    free(q);
    free(k);
    free(s);
}

/* ------------------------------------------------------------------ */
/* quantization of real weights                                         */
/* ------------------------------------------------------------------ */

/*
 * The pages name 4-bit weights (PIPO, "Method", bullet "Computation
 * optimization") but no rule for producing them.  Reading: symmetric
 * round-to-nearest per group of 32 consecutive k, in the format above:
 *     amax = max |w| over the group
 *     s    = binary16(amax / 8), round to nearest even (the stored scale)
 *     c    = clamp(rint(w / s) + 8, 0, 15)   (rint: ties to even)
 * where w / s is the exact real quotient.  An fp64 division decides it
 * exactly: w has at most 24 significant bits and s at most 11, so a
 * quotient that is not a half-integer n + 1/2 (|n| <= 8) differs from one
 * by at least 2^-26, while the fp64 division errs by less than 2^-49; and a
 * half-integer quotient is computed exactly.  A group whose stored scale is
 * 0 (all zero, or amax / 8 below half the smallest binary16 subnormal) gets
 * code 8 everywhere.  The largest weight of a group, when positive, maps to
 * w / s = 8 and is clipped to code 15 (7 s).  Inputs are finite with
 * amax / 8 below 65520 (else the scale is infinite).
 * codes: u8[N][K], one code per byte; scales: u16[N][K/32].
 */
static void quantize_group(const float *w, uint8_t *codes, uint16_t *scale)
{
    double amax = 0.0;
    for (int i = 0; i < 32; ++i) {
        double a = fabs((double)w[i]);
        if (a > amax)
            amax = a;
    }
    uint16_t s16 = q4o_f64_to_f16(amax / 8.0); /* amax / 8 is exact in fp64 */
    *scale = s16;
    double s = q4o_f16_to_f64(s16);
    for (int i = 0; i < 32; ++i) {
        if (s == 0.0) {
            codes[i] = 8;
            continue;
        }
        double r = rint((double)w[i] / s); /* default rounding: ties to even */
        double c = r + 8.0;
        if (c < 0.0)
            c = 0.0;
        if (c > 15.0)
            c = 15.0;
        codes[i] = (uint8_t)c;
    }
}

void q4o_quantize_f32(const float *w, int64_t N, int64_t K, uint8_t *codes, uint16_t *scales)
{
    for (int64_t n = 0; n < N; ++n)
        for (int64_t g = 0; g < K / 32; ++g)
            quantize_group(w + n * K + g * 32, codes + n * K + g * 32, scales + n * (K / 32) + g);
}

/* binary16 weights (bit patterns): each value is exactly a binary32. */
void q4o_quantize_f16(const uint16_t *w, int64_t N, int64_t K, uint8_t *codes, uint16_t *scales)
{
    float buf[32];
    for (int64_t n = 0; n < N; ++n)
        for (int64_t g = 0; g < K / 32; ++g) {
            for (int i = 0; i < 32; ++i)
                buf[i] = (float)q4o_f16_to_f64(w[n * K + g * 32 + i]);
            quantize_group(buf, codes + n * K + g * 32, scales + n * (K / 32) + g);
        }
}

/* mlp[j] = f16(silu(gate[j]) * up[j]), gate | up stacked in gu. */
void q4o_silu_mul_f16(const double *gu, int64_t dff, uint16_t *out)
{
    for (int64_t j = 0; j < dff; ++j) {
        double g = gu[j];
        double silu = g / (1.0 + exp(-g));
        out[j] = q4o_f64_to_f16(silu * gu[dff + j]);
    }
}

/* One quantized matrix as the caller lays it out. */
typedef struct {
    const uint8_t *packed;
    const uint16_t *scales;
} q4o_mat;

/*
 * One decoder layer on the residual h (fp64, in place):
 *   a   = f16(rmsnorm(h))
 *   qkv = Wqkv a                 rows: Q [0,H*hd) | K | V
 *   o   = f16(gather V by GQA group)
 *   h  += Wo o
 *   a2  = f16(rmsnorm(h))
 *   gu  = Wgu a2                 rows: gate [0,dff) | up [dff,2dff)
 *   m   = f16(silu(gate) * up)
 *   h  += Wdown m
 * mag_h (may be NULL) accumulates, per element of h, the magnitudes
 * sum_k |w*x| of the two products added into h, which bounds how far a
 * correctly rounded fp32 evaluation may drift from this fp64 one.
 */
/*
 * The same layer with attention over the caches in place of the one-token
 * stand-in: o = f16(attention at position pos) (q4o_attention; the caches
 * of this layer gain row pos).  Everything else as q4o_decode_layer.
 */
void q4o_decode_layer_attn(const q4o_mat *qkv_m, const q4o_mat *o_m,
                           const q4o_mat *gu_m, const q4o_mat *down_m,
                           int64_t d, int64_t H, int64_t Hkv, int64_t hd,
                           int64_t dff, double eps, int64_t pos, int64_t max_ctx,
                           double base, uint16_t *kcache, uint16_t *vcache,
                           double *h, double *mag_h)
{
    int64_t nqkv = (H + 2 * Hkv) * hd;
    uint16_t *a = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(d > dff ? d : dff));
    uint16_t *o = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(H * hd));
    double *att = (double *)malloc(sizeof(double) * (size_t)(H * hd));
    double *qkv = (double *)malloc(sizeof(double) * (size_t)nqkv);
    double *gu = (double *)malloc(sizeof(double) * (size_t)(2 * dff));
    double *y = (double *)malloc(sizeof(double) * (size_t)d);
    double *m = (double *)malloc(sizeof(double) * (size_t)d);

    q4o_rmsnorm_f16(h, d, eps, a);
    q4o_gemv(qkv_m->packed, qkv_m->scales, a, nqkv, d, qkv, NULL);
    q4o_attention(qkv, H, Hkv, hd, pos, max_ctx, base, kcache, vcache, att, NULL);
    for (int64_t i = 0; i < H * hd; ++i)
        o[i] = q4o_f64_to_f16(att[i]);
    q4o_gemv(o_m->packed, o_m->scales, o, d, H * hd, y, m);
    for (int64_t i = 0; i < d; ++i) {
        h[i] += y[i];
        if (mag_h)
            mag_h[i] += m[i];
    }
    q4o_rmsnorm_f16(h, d, eps, a);
    q4o_gemv(gu_m->packed, gu_m->scales, a, 2 * dff, d, gu, NULL);
    q4o_silu_mul_f16(gu, dff, a);
    q4o_gemv(down_m->packed, down_m->scales, a, d, dff, y, m);
    for (int64_t i = 0; i < d; ++i) {
        h[i] += y[i];
        if (mag_h)
            mag_h[i] += m[i];
    }
    free(a);
    free(o);
    free(att);
    free(qkv);
    free(gu);
    free(y);
    free(m);
}

void q4o_decode_layer(const q4o_mat *qkv_m, const q4o_mat *o_m,
                      const q4o_mat *gu_m, const q4o_mat *down_m,
                      int64_t d, int64_t H, int64_t Hkv, int64_t hd,
                      int64_t dff, double eps, double *h, double *mag_h)
{
    int64_t nqkv = (H + 2 * Hkv) * hd;
    uint16_t *a = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(d > dff ? d : dff));
    uint16_t *o = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(H * hd));
    double *qkv = (double *)malloc(sizeof(double) * (size_t)nqkv);
    double *gu = (double *)malloc(sizeof(double) * (size_t)(2 * dff));
    double *y = (double *)malloc(sizeof(double) * (size_t)d);
    double *m = (double *)malloc(sizeof(double) * (size_t)d);

    q4o_rmsnorm_f16(h, d, eps, a);
    q4o_gemv(qkv_m->packed, qkv_m->scales, a, nqkv, d, qkv, NULL);
    q4o_gqa_gather_f16(qkv, H, Hkv, hd, o);
    q4o_gemv(o_m->packed, o_m->scales, o, d, H * hd, y, m);
    for (int64_t i = 0; i < d; ++i) {
        h[i] += y[i];
        if (mag_h)
            mag_h[i] += m[i];
    }
    q4o_rmsnorm_f16(h, d, eps, a);
    q4o_gemv(gu_m->packed, gu_m->scales, a, 2 * dff, d, gu, NULL);
    q4o_silu_mul_f16(gu, dff, a);
    q4o_gemv(down_m->packed, down_m->scales, a, d, dff, y, m);
    for (int64_t i = 0; i < d; ++i) {
        h[i] += y[i];
        if (mag_h)
            mag_h[i] += m[i];
    }
    free(a);
    free(o);
    free(qkv);
    free(gu);
    free(y);
    free(m);
}
