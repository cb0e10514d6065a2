/*
 * oracle.c -- CPU oracle for the batched single-token decode step.
 *
 * TEST INFRASTRUCTURE.  Only the test-suite, the smoke check and the bench's
 * CPU-baseline leg may load this library.  The HIP product path never links,
 * loads or calls it, and it shares no code, header or table with that path.
 *
 * Everything here is the plain definition of a result, accumulated in fp64,
 * one output row per loop iteration (rows may be spread over OpenMP threads;
 * each row's sum is a fixed sequential loop, so results do not depend on the
 * thread count).  No blocking, fusion or reordering beyond the definitions.
 *
 * Sources (docs.rs source pages):
 *   [batched_forward] realizar 0.8.5, src/cuda/executor/layers/batched_forward.rs
 *   [head_dim]        realizar 0.8.5, src/cuda/executor/head_dim.rs
 * and the block formats of the quantised workloads (Q8: 32 int8 values and one
 * fp16 scale per block, value = scale*q; Q4: 32 unsigned 4-bit values and one
 * fp16 scale, value = scale*(q-8)).  FP8 (the pages' other weight precision,
 * [batched_forward] LM-head notes) is 32 OCP FP8 E4M3 values and one fp16
 * scale per block, value = scale*e4m3(q).  Q6K (the 6-bit K-quant those notes
 * also name; its block layout is not on the pages) is read as the K-quant
 * family's 6-bit format, see orc_dequant_row.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_Q8 1
#define ORC_Q4 2
#define ORC_FP8 3
#define ORC_Q6K 4
#define ORC_QBLOCK 32
#define ORC_Q6K_SUPER 256
#define ORC_Q6K_CODE_BYTES 192
#define ORC_Q6K_SCALE_BYTES 18

/* IEEE 754 binary16 -> binary64, from the bit fields: sign, 5-bit exponent
 * (bias 15), 10-bit fraction; exponent 0 encodes subnormals 2^-14 * f/1024,
 * exponent 31 encodes inf (f == 0) and NaN. */
double orc_f16_to_f64(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int f = h & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24); /* 2^-14 * f / 2^10 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp(1.0 + (double)f / 1024.0, e - 15);
    return sign ? -v : v;
}

/* OCP 8-bit floating point E4M3 -> binary64, from the bit fields: sign,
 * 4-bit exponent (bias 7), 3-bit fraction; exponent 0 encodes subnormals
 * 2^-6 * f/8; there is no infinity, and exponent 15 with fraction 7 is NaN
 * (so the largest finite magnitude is 1.75 * 2^8 = 448). */
double orc_e4m3_to_f64(uint8_t c) {
    int sign = (c >> 7) & 1;
    int e = (c >> 3) & 0xF;
    int f = c & 0x7;
    double v;
    if (e == 0)
        v = ldexp((double)f, -9); /* 2^-6 * f / 2^3 */
    else if (e == 15 && f == 7)
        v = NAN;
    else
        v = ldexp(1.0 + (double)f / 8.0, e - 7);
    return sign ? -v : v;
}

/* Dequantised row `row` of an [n][k] weight in the planar layout:
 *   F32: data is float[n][k];
 *   Q8 : data is int8[n][k], scale is fp16[n][k/32]; w = scale * q;
 *   Q4 : data is uint8[n][k/2] (byte j: element 2j low nibble, 2j+1 high
 *        nibble), scale fp16[n][k/32]; w = scale * (q - 8);
 *   FP8: data is E4M3 codes uint8[n][k], scale fp16[n][k/32]; w = scale * e4m3(q);
 *   Q6K: the 6-bit K-quant the pages name for LM heads: super-blocks of 256
 *        values, each of 16 sub-blocks of 16 values with a signed int8 scale
 *        sc, and one fp16 scale d per super-block; 6-bit codes q in 0..63;
 *        w = d * sc[sub-block] * (q - 32).  data is uint8[n][k/256][192]: 128
 *        bytes of the codes' low 4 bits (byte j: element 2j low nibble, 2j+1
 *        high nibble), then 64 bytes of their high 2 bits (byte j: element
 *        4j + e at bits 2e, 2e+1); scale is uint8[n][k/256][18]: the 16
 *        sub-scales, then d (fp16, low byte first). */
void orc_dequant_row(int fmt, const void *data, const uint16_t *scale, int64_t k,
                     int64_t row, double *out) {
    int64_t nb = k / ORC_QBLOCK;
    if (fmt == ORC_Q6K) {
        const int64_t nsb = k / ORC_Q6K_SUPER;
        const uint8_t *codes = (const uint8_t *)data + row * nsb * ORC_Q6K_CODE_BYTES;
        const uint8_t *recs = (const uint8_t *)scale + row * nsb * ORC_Q6K_SCALE_BYTES;
        for (int64_t sb = 0; sb < nsb; ++sb) {
            const uint8_t *lo = codes + sb * ORC_Q6K_CODE_BYTES, *hi = lo + 128;
            const uint8_t *rec = recs + sb * ORC_Q6K_SCALE_BYTES;
            double d = orc_f16_to_f64((uint16_t)(rec[16] | (rec[17] << 8)));
            for (int i = 0; i < ORC_Q6K_SUPER; ++i) {
                int low = (i % 2 == 0) ? (lo[i / 2] & 0xF) : (lo[i / 2] >> 4);
                int high = (hi[i / 4] >> (2 * (i % 4))) & 3;
                int q = low | (high << 4);
                double sc = (double)(int8_t)rec[i / 16];
                out[sb * ORC_Q6K_SUPER + i] = d * sc * (double)(q - 32);
            }
        }
        return;
    }
    if (fmt == ORC_F32) {
        const float *w = (const float *)data + row * k;
        for (int64_t i = 0; i < k; ++i) out[i] = (double)w[i];
    } else if (fmt == ORC_Q8) {
        const int8_t *q = (const int8_t *)data + row * k;
        for (int64_t b = 0; b < nb; ++b) {
            double s = orc_f16_to_f64(scale[row * nb + b]);
            for (int64_t i = b * ORC_QBLOCK; i < (b + 1) * ORC_QBLOCK; ++i)
                out[i] = s * (double)q[i];
        }
    } else if (fmt == ORC_FP8) {
        const uint8_t *q = (const uint8_t *)data + row * k;
        for (int64_t b = 0; b < nb; ++b) {
            double s = orc_f16_to_f64(scale[row * nb + b]);
            for (int64_t i = b * ORC_QBLOCK; i < (b + 1) * ORC_QBLOCK; ++i)
                out[i] = s * orc_e4m3_to_f64(q[i]);
        }
    } else {
        const uint8_t *q = (const uint8_t *)data + row * (k / 2);
        for (int64_t b = 0; b < nb; ++b) {
            double s = orc_f16_to_f64(scale[row * nb + b]);
            for (int64_t i = b * ORC_QBLOCK; i < (b + 1) * ORC_QBLOCK; ++i) {
                uint8_t byte = q[i / 2];
                int nib = (i % 2 == 0) ? (byte & 0xF) : (byte >> 4);
                out[i] = s * (double)(nib - 8);
            }
        }
    }
}

/* Batched GEMV [batched_forward: forward_batched_to_token_ids doc -- the M
 * inputs share one read of the weights; per sequence the result is the plain
 * matrix-vector product]:
 *   y[mi][r] = sum_i W[rows[r]][i] * x[mi][i],   mi < m, r < nrows.
 * rows == NULL means every row (nrows must then equal n). */
void orc_gemv(int fmt, const void *data, const uint16_t *scale, int64_t n, int64_t k,
              const double *x, int64_t m, const int64_t *rows, int64_t nrows, double *y) {
    (void)n;
#pragma omp parallel
    {
        double *w = (double *)malloc(sizeof(double) * (size_t)(k > 0 ? k : 1));
#pragma omp for schedule(static)
        for (int64_t r = 0; r < nrows; ++r) {
            int64_t row = rows ? rows[r] : r;
            orc_dequant_row(fmt, data, scale, k, row, w);
            for (int64_t mi = 0; mi < m; ++mi) {
                const double *xm = x + mi * k;
                double acc = 0.0;
                for (int64_t i = 0; i < k; ++i) acc += w[i] * xm[i];
                y[mi * nrows + r] = acc;
            }
        }
        free(w);
    }
}

/* Decode attention for one sequence [head_dim: flash_decoding_attention_into
 * -- Q [num_heads][head_dim] against the cached K/V of num_kv_heads groups]:
 *   for head h, g = h / (nq / nkv), over cache rows t in [0, len):
 *     s_t = <q_h, K[g][t]> / sqrt(hd),  o_h = sum_t softmax(s)_t V[g][t].
 * kc, vc are [nkv][ld][hd]; out is [nq][hd].  len == 0 leaves out untouched.
 * (Subtracting the row maximum before exp leaves softmax unchanged.) */
void orc_attention(const double *q, const double *kc, const double *vc, int64_t nq,
                   int64_t nkv, int64_t hd, int64_t ld, int64_t len, double *out) {
    if (len <= 0) return;
    int64_t group = nq / nkv;
    double inv = 1.0 / sqrt((double)hd);
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)len);
#pragma omp for schedule(static)
        for (int64_t h = 0; h < nq; ++h) {
            int64_t g = h / group;
            const double *qh = q + h * hd;
            const double *K = kc + g * ld * hd;
            const double *V = vc + g * ld * hd;
            double mx = -INFINITY;
            for (int64_t t = 0; t < len; ++t) {
                double d = 0.0;
                for (int64_t i = 0; i < hd; ++i) d += qh[i] * K[t * hd + i];
                s[t] = d * inv;
                if (s[t] > mx) mx = s[t];
            }
            double l = 0.0;
            for (int64_t t = 0; t < len; ++t) {
                s[t] = exp(s[t] - mx);
                l += s[t];
            }
            for (int64_t i = 0; i < hd; ++i) {
                double o = 0.0;
                for (int64_t t = 0; t < len; ++t) o += s[t] * V[t * hd + i];
                out[h * hd + i] = o / l;
            }
        }
        free(s);
    }
}

/* The same attention in split-K form [head_dim: flash_decoding_attention_into
 * doc -- the cache is split into chunks processed independently, then the
 * partial results are combined with softmax rescaling].  Chunk c covers rows
 * [c*chunk, min((c+1)*chunk, len)); for it
 *     m_c = max s,  l_c = sum e^(s - m_c),  o~_c = sum e^(s - m_c) v / l_c,
 *     lse_c = m_c + ln l_c;
 * the combine is  LSE = max_c lse_c,  w_c = e^(lse_c - LSE),
 *     o = sum_c w_c o~_c / sum_c w_c.
 * Empty chunks contribute nothing.  Used only to check that the split form
 * equals the unsplit definition. */
void orc_attention_splitk(const double *q, const double *kc, const double *vc, int64_t nq,
                          int64_t nkv, int64_t hd, int64_t ld, int64_t len, int64_t chunk,
                          double *out) {
    if (len <= 0 || chunk <= 0) return;
    int64_t group = nq / nkv;
    int64_t nc = (len + chunk - 1) / chunk;
    double inv = 1.0 / sqrt((double)hd);
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)chunk);
        double *ot = (double *)malloc(sizeof(double) * (size_t)(nc * hd));
        double *lse = (double *)malloc(sizeof(double) * (size_t)nc);
#pragma omp for schedule(static)
        for (int64_t h = 0; h < nq; ++h) {
            int64_t g = h / group;
            const double *qh = q + h * hd;
            const double *K = kc + g * ld * hd;
            const double *V = vc + g * ld * hd;
            for (int64_t c = 0; c < nc; ++c) {
                int64_t t0 = c * chunk, t1 = t0 + chunk < len ? t0 + chunk : len;
                double mc = -INFINITY;
                for (int64_t t = t0; t < t1; ++t) {
                    double d = 0.0;
                    for (int64_t i = 0; i < hd; ++i) d += qh[i] * K[t * hd + i];
                    s[t - t0] = d * inv;
                    if (s[t - t0] > mc) mc = s[t - t0];
                }
                double lc = 0.0;
                for (int64_t t = t0; t < t1; ++t) {
                    s[t - t0] = exp(s[t - t0] - mc);
                    lc += s[t - t0];
                }
                for (int64_t i = 0; i < hd; ++i) {
                    double o = 0.0;
                    for (int64_t t = t0; t < t1; ++t) o += s[t - t0] * V[t * hd + i];
                    ot[c * hd + i] = o / lc;
                }
                lse[c] = mc + log(lc);
            }
            double LSE = -INFINITY;
            for (int64_t c = 0; c < nc; ++c)
                if (lse[c] > LSE) LSE = lse[c];
            double wsum = 0.0;
            for (int64_t c = 0; c < nc; ++c) wsum += exp(lse[c] - LSE);
            for (int64_t i = 0; i < hd; ++i) {
                double o = 0.0;
                for (int64_t c = 0; c < nc; ++c) o += exp(lse[c] - LSE) * ot[c * hd + i];
                out[h * hd + i] = o / wsum;
            }
        }
        free(s);
        free(ot);
        free(lse);
    }
}
