/*
 * CPU oracle for the K-quant decode GEMV -- TEST INFRASTRUCTURE ONLY.
 *
 * Only tests/, the smoke check and the benchmark's CPU-baseline leg use this
 * file.  It shares no code, header or table with the GPU library: it reads
 * the GGUF super-block bytes itself, decodes fp16 and bf16 itself, and
 * computes in double precision.
 *
 * What it computes (the decode-step product y[b,:] = dequant(W) . x[b,:] that
 * the Core AI card's decode table prices in weight bytes per token, "Muse-
 * Glimmer-30B (text decoder) - Apple Core AI", decode table and the paragraph
 * after it; batch 1..8 as in the SGLang Day-0 post's batch sweep):
 *
 *   Q4_K / Q5_K :  w = d * sc_g * q - dmin * m_g      (g = element / 32)
 *   Q6_K        :  w = d * sc_g * (q - 32)            (g = element / 16)
 *
 * The quant formats are the ones the daily.dev summary names (Q&A "How does
 * ExecuTorch export Muse Glimmer GGUF checkpoints ...": Q4_K/Q5_K/Q6_K).  The
 * byte layout is the public GGUF one, which the pages do not print; compatibility
 * with real GGUF files is therefore a reading, not pinned by any page.
 *
 * Exactness: an fp16 value is D * 2^E with |D| < 2^11.  d*sc*q < 2^22 * 2^E and
 * dmin*m < 2^17 * 2^E', so every w above is an exact binary64 value; rounding
 * it once to binary32 gives the single correctly rounded dequantised weight.
 * The dot product is summed in double in index order.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define KQO_Q4_K 1
#define KQO_Q5_K 2
#define KQO_Q6_K 3
#define KQO_X_F32 0
#define KQO_X_BF16 1

#define KQO_OK 0
#define KQO_ERR_ARG 1
#define KQO_ERR_NONFINITE 2

/* IEEE-754 binary16 bit pattern -> double.  Returns NAN for inf/nan inputs. */
double kqo_f16_to_double(uint16_t h) {
    int sign = (h >> 15) & 1;
    int exp = (h >> 10) & 0x1F;
    int man = h & 0x3FF;
    double v;
    if (exp == 0x1F) return NAN;
    if (exp == 0)
        v = ldexp((double)man, -24);                 /* subnormal: man * 2^-24 */
    else
        v = ldexp((double)(man | 0x400), exp - 25);  /* (1024+man) * 2^(exp-15-10) */
    return sign ? -v : v;
}

/* bfloat16 bit pattern -> double (it is the top half of a binary32). */
double kqo_bf16_to_double(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

static int64_t sb_bytes(int type) {
    switch (type) {
    case KQO_Q4_K: return 144;
    case KQO_Q5_K: return 176;
    case KQO_Q6_K: return 210;
    default: return 0;
    }
}

static uint16_t rd16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* 6-bit scale and min of sub-block j (0..7) from the 12 packed bytes. */
static void q4k_scale_min(const uint8_t *s, int j, int *sc, int *m) {
    if (j < 4) {
        *sc = s[j] & 63;
        *m = s[j + 4] & 63;
    } else {
        *sc = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4);
        *m = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
    }
}

/* Decode one super-block into 256 exact doubles.  Returns KQO_OK or an error. */
static int decode_sb(int type, const uint8_t *b, double *w) {
    if (type == KQO_Q4_K || type == KQO_Q5_K) {
        double d = kqo_f16_to_double(rd16(b));
        double dmin = kqo_f16_to_double(rd16(b + 2));
        const uint8_t *scales = b + 4;
        const uint8_t *qh = b + 16;                                /* Q5_K only */
        const uint8_t *qs = (type == KQO_Q4_K) ? b + 16 : b + 48;
        if (isnan(d) || isnan(dmin)) return KQO_ERR_NONFINITE;
        for (int e = 0; e < 256; ++e) {
            int g = e / 32;
            int c = e / 64, r = e % 64;
            int byte = qs[32 * c + (r % 32)];
            int q = (r < 32) ? (byte & 15) : (byte >> 4);
            if (type == KQO_Q5_K) q += ((qh[e % 32] >> g) & 1) << 4;
            int sc, m;
            q4k_scale_min(scales, g, &sc, &m);
            w[e] = d * sc * q - dmin * m;
        }
        return KQO_OK;
    }
    if (type == KQO_Q6_K) {
        const uint8_t *ql = b, *qh = b + 128;
        const int8_t *scales = (const int8_t *)(b + 192);
        double d = kqo_f16_to_double(rd16(b + 208));
        if (isnan(d)) return KQO_ERR_NONFINITE;
        for (int e = 0; e < 256; ++e) {
            int h = e / 128, r = (e % 128) / 32, i = e % 32;
            int lbyte = ql[64 * h + 32 * (r & 1) + i];
            int lo = (r < 2) ? (lbyte & 15) : (lbyte >> 4);
            int hi = (qh[32 * h + i] >> (2 * r)) & 3;
            int q = lo | (hi << 4);
            w[e] = d * scales[e / 16] * (q - 32);
        }
        return KQO_OK;
    }
    return KQO_ERR_ARG;
}

/* Dequantise rows x cols weights (GGUF row-major super-blocks) into w[rows*cols]. */
int kqo_dequant(int type, int64_t rows, int64_t cols, const uint8_t *gguf, double *w) {
    int64_t sbb = sb_bytes(type);
    if (!sbb || rows < 0 || cols < 0 || cols % 256 || !gguf || !w) return KQO_ERR_ARG;
    int64_t nsb = cols / 256;
    int err = KQO_OK;
#pragma omp parallel for schedule(static) reduction(| : err)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t s = 0; s < nsb; ++s)
            err |= decode_sb(type, gguf + (r * nsb + s) * sbb, w + r * cols + s * 256);
    return err;
}

/*
 * y[b*rows + r] = sum_k w[r,k] * x[b*ldx + k] and a[b*rows + r] = sum_k |w[r,k] * x[b*ldx + k]|,
 * for b < batch; x is fp32 (xtype 0) or bf16 bit patterns (xtype 1).
 */
int kqo_gemv(int type, int64_t rows, int64_t cols, const uint8_t *gguf, int xtype, const void *x,
             int64_t ldx, int batch, double *y, double *a) {
    int64_t sbb = sb_bytes(type);
    if (!sbb || rows < 0 || cols < 0 || cols % 256 || !gguf || !x || !y || !a) return KQO_ERR_ARG;
    if (batch < 1 || ldx < cols || (xtype != KQO_X_F32 && xtype != KQO_X_BF16)) return KQO_ERR_ARG;
    int64_t nsb = cols / 256;
    double *xd = (double *)malloc(sizeof(double) * (size_t)(batch * cols));
    if (!xd) return KQO_ERR_ARG;
    for (int b = 0; b < batch; ++b)
        for (int64_t k = 0; k < cols; ++k)
            xd[b * cols + k] = (xtype == KQO_X_F32) ? (double)((const float *)x)[b * ldx + k]
                                                     : kqo_bf16_to_double(((const uint16_t *)x)[b * ldx + k]);
    int err = KQO_OK;
#pragma omp parallel for schedule(dynamic, 16) reduction(| : err)
    for (int64_t r = 0; r < rows; ++r) {
        double w[256];
        double acc[8] = {0}, mag[8] = {0};
        double *accp = acc, *magp = mag;
        double *heap = NULL;
        if (batch > 8) {
            heap = (double *)calloc((size_t)(2 * batch), sizeof(double));
            accp = heap;
            magp = heap + batch;
        }
        for (int64_t s = 0; s < nsb; ++s) {
            err |= decode_sb(type, gguf + (r * nsb + s) * sbb, w);
            for (int b = 0; b < batch; ++b) {
                const double *xb = xd + b * cols + s * 256;
                for (int e = 0; e < 256; ++e) {
                    double p = w[e] * xb[e];
                    accp[b] += p;
                    magp[b] += fabs(p);
                }
            }
        }
        for (int b = 0; b < batch; ++b) {
            y[b * rows + r] = accp[b];
            a[b * rows + r] = magp[b];
        }
        free(heap);
    }
    free(xd);
    return err;
}
