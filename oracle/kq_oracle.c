/*
 * kq_oracle.c -- plain, slow, scalar CPU oracle of the K-quant x Q8_K
 * matmul ("kq v2").
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load or call this code.  It shares no
 * code, header, table or constant with the HIP library, and the HIP
 * library never calls it.
 *
 * What it computes follows the K-quant kernel arc page (daScript PR
 * "dasLLAMA: K-quant kernel arc -- kq v2 integer folds, kq v3 panel-scratch
 * tiles, chain regrain, parity gates"):
 *
 *  - activations in Q8_K form: one float scale per 256 values plus int16
 *    sums per 16 ("The pieces", kq v2 item; the k4 v2 commit message names
 *    quantize_q8_k_into and the per-16 bsums);
 *  - per superblock, the sub-scale x int32-dot and min x bsums terms are
 *    accumulated in integers, with ONE float fold per superblock (k4 v2
 *    commit message: one d*d8 fma and one dmin*d8 fms per superblock);
 *  - Q5_K reuses the Q4_K scale block; only the high bit of each quant
 *    differs (k5/k6 v2 commit message);
 *  - Q6_K folds its signed per-16 sub-scales exactly in int32 as
 *    iacc - 32*bacc, closed by one float multiply by d*d8 (same message).
 *
 * The byte layouts of the three weight records are the ggml K-quant
 * records (Q4_K 144 B, Q5_K 176 B, Q6_K 210 B); the pages give only their
 * sizes, the field positions are the ggml format's.
 *
 * Floating point: the Q8_K quantizer decides integers, so it runs in IEEE
 * binary32 exactly as written (amax/127 and x/d8 are single divisions,
 * rintf rounds half to even).  Everything else is double.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define QK 256

enum { ORC_Q4_K = 4, ORC_Q5_K = 5, ORC_Q6_K = 6 };

/* binary16 bit pattern -> double, exactly (subnormals kept). */
double orc_f16_to_double(uint16_t h)
{
    int sign = h >> 15;
    int e = (h >> 10) & 31;
    int f = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);              /* 0.f * 2^-14 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);  /* 1.f * 2^(e-15) */
    return sign ? -v : v;
}

static uint16_t rd16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }

int orc_block_bytes(int fmt)
{
    switch (fmt) {
    case ORC_Q4_K: return 144;
    case ORC_Q5_K: return 176;
    case ORC_Q6_K: return 210;
    default: return 0;
    }
}

/* Decoded integer fields of one superblock.
 * Q4_K/Q5_K: sub-block j (32 weights) has unsigned 6-bit scale sc[j] and
 * min m[j]; w = d*sc*q - dmin*m.  Q6_K: sub-block j (16 weights) has signed
 * 8-bit scale sc[j]; w = d*sc*(q - 32). */
typedef struct {
    double d, dmin;
    int sc[16];
    int m[16];
    int q[QK];
} orc_block;

/* The 12-byte packing of eight 6-bit scales and eight 6-bit mins shared
 * by Q4_K and Q5_K. */
static void decode_scale_min_12(const uint8_t *s, int *sc, int *m)
{
    for (int j = 0; j < 4; ++j) {
        sc[j] = s[j] & 63;
        m[j] = s[j + 4] & 63;
    }
    for (int j = 4; j < 8; ++j) {
        sc[j] = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4);
        m[j] = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
    }
}

/* Decode one record.  Returns 0, or -1 for an unknown format. */
int orc_decode(int fmt, const uint8_t *rec, orc_block *b)
{
    memset(b, 0, sizeof *b);
    if (fmt == ORC_Q4_K || fmt == ORC_Q5_K) {
        b->d = orc_f16_to_double(rd16(rec));
        b->dmin = orc_f16_to_double(rd16(rec + 2));
        decode_scale_min_12(rec + 4, b->sc, b->m);
        const uint8_t *qh = rec + 16;                      /* Q5_K only */
        const uint8_t *qs = rec + (fmt == ORC_Q4_K ? 16 : 48);
        for (int j = 0; j < 8; ++j) {
            for (int l = 0; l < 32; ++l) {
                uint8_t byte = qs[32 * (j / 2) + l];
                int q = (j % 2 == 0) ? (byte & 15) : (byte >> 4);
                if (fmt == ORC_Q5_K)
                    q += ((qh[l] >> j) & 1) << 4;
                b->q[32 * j + l] = q;
            }
        }
        return 0;
    }
    if (fmt == ORC_Q6_K) {
        const uint8_t *ql = rec, *qh = rec + 128, *sc = rec + 192;
        b->d = orc_f16_to_double(rd16(rec + 208));
        b->dmin = 0.0;
        for (int j = 0; j < 16; ++j)
            b->sc[j] = (int8_t)sc[j];
        for (int h = 0; h < 2; ++h)
            for (int t = 0; t < 4; ++t)
                for (int l = 0; l < 32; ++l) {
                    uint8_t lo = ql[64 * h + l + 32 * (t % 2)];
                    int low = (t < 2) ? (lo & 15) : (lo >> 4);
                    int high = (qh[32 * h + l] >> (2 * t)) & 3;
                    b->q[128 * h + 32 * t + l] = low | (high << 4);
                }
        return 0;
    }
    return -1;
}

/* Dequantise rows: w[n][k] (double).  Dequantisation is the format's
 * definition: Q4_K/Q5_K w = d*sc_j*q - dmin*m_j, Q6_K w = d*sc_j*(q-32);
 * in double every such value is exact. */
int orc_dequantize(int fmt, const uint8_t *recs, int64_t n, int64_t k, double *w)
{
    int bb = orc_block_bytes(fmt);
    if (!bb || k % QK) return -1;
    int64_t nsb = k / QK;
    orc_block b;
    for (int64_t r = 0; r < n; ++r)
        for (int64_t s = 0; s < nsb; ++s) {
            orc_decode(fmt, recs + (r * nsb + s) * bb, &b);
            double *o = w + r * k + s * QK;
            for (int i = 0; i < QK; ++i) {
                if (fmt == ORC_Q6_K)
                    o[i] = b.d * b.sc[i / 16] * (b.q[i] - 32);
                else
                    o[i] = b.d * b.sc[i / 32] * b.q[i] - b.dmin * b.m[i / 32];
            }
        }
    return 0;
}

/* Q8_K quantisation of x[t][k]: per 256 values, amax = max |x|,
 * d8 = amax / 127 (binary32 division), a = rint(x / d8) (binary32
 * division, round half to even) clamped to [-127, 127], bsum of each 16.
 * An all-zero chunk gives d8 = 0, a = 0, bsums = 0.
 * xq[t][k] int8, xs[t][k/256] float, xbs[t][k/16] int16. */
int orc_quantize_q8k(const float *x, int64_t t, int64_t k, int8_t *xq, float *xs, int16_t *xbs)
{
    if (k % QK) return -1;
    int64_t nsb = k / QK;
    for (int64_t r = 0; r < t; ++r)
        for (int64_t s = 0; s < nsb; ++s) {
            const float *c = x + r * k + s * QK;
            float amax = 0.0f;
            for (int i = 0; i < QK; ++i) {
                float a = fabsf(c[i]);
                if (a > amax) amax = a;
            }
            int8_t *q = xq + r * k + s * QK;
            int16_t *bs = xbs + r * (k / 16) + s * 16;
            if (amax == 0.0f) {
                xs[r * nsb + s] = 0.0f;
                memset(q, 0, QK);
                memset(bs, 0, 16 * sizeof(int16_t));
                continue;
            }
            float d8 = amax / 127.0f;
            xs[r * nsb + s] = d8;
            for (int i = 0; i < QK; ++i) {
                float v = c[i] / d8;
                long a = lrintf(v);
                if (a > 127) a = 127;
                if (a < -127) a = -127;
                q[i] = (int8_t)a;
            }
            for (int g = 0; g < 16; ++g) {
                int sum = 0;
                for (int i = 0; i < 16; ++i) sum += q[16 * g + i];
                bs[g] = (int16_t)sum;
            }
        }
    return 0;
}

/* Per-superblock integer partials of row n against token t, by the kq v2
 * folds:
 *   Q4_K/Q5_K  P = sum_j sc_j * dot_j,  dot_j = sum over sub-block j (32)
 *              M = sum_j m_j * (bsum_{2j} + bsum_{2j+1})
 *   Q6_K       iacc = sum_j sc_j * dot_j (16-wide sub-blocks, raw q),
 *              bacc = sum_j sc_j * bsum_j,   P = iacc - 32*bacc,  M = 0.
 * Each sum is formed in int64 and must fit int32 (else returns -2).
 * P[t][n][sb], M[t][n][sb].  Returns 0. */
int orc_partials(int fmt, const uint8_t *recs, int64_t n, int64_t k,
                 const int8_t *xq, const int16_t *xbs, int64_t t,
                 int32_t *P, int32_t *M)
{
    int bb = orc_block_bytes(fmt);
    if (!bb || k % QK) return -1;
    int64_t nsb = k / QK;
    orc_block b;
    int rc = 0;
    for (int64_t r = 0; r < n; ++r)
        for (int64_t s = 0; s < nsb; ++s) {
            orc_decode(fmt, recs + (r * nsb + s) * bb, &b);
            for (int64_t tt = 0; tt < t; ++tt) {
                const int8_t *a = xq + tt * k + s * QK;
                const int16_t *bs = xbs + tt * (k / 16) + s * 16;
                int64_t p, m;
                if (fmt == ORC_Q6_K) {
                    int64_t iacc = 0, bacc = 0;
                    for (int j = 0; j < 16; ++j) {
                        int64_t dot = 0;
                        for (int i = 0; i < 16; ++i) dot += (int64_t)b.q[16 * j + i] * a[16 * j + i];
                        iacc += b.sc[j] * dot;
                        bacc += b.sc[j] * (int64_t)bs[j];
                    }
                    if (iacc != (int32_t)iacc || 32 * bacc != (int32_t)(32 * bacc)) rc = -2;
                    p = iacc - 32 * bacc;
                    m = 0;
                } else {
                    p = 0;
                    m = 0;
                    for (int j = 0; j < 8; ++j) {
                        int64_t dot = 0;
                        for (int i = 0; i < 32; ++i) dot += (int64_t)b.q[32 * j + i] * a[32 * j + i];
                        p += b.sc[j] * dot;
                        m += b.m[j] * ((int64_t)bs[2 * j] + bs[2 * j + 1]);
                    }
                }
                if (p != (int32_t)p || m != (int32_t)m) rc = -2;
                int64_t o = (tt * n + r) * nsb + s;
                P[o] = (int32_t)p;
                M[o] = (int32_t)m;
            }
        }
    return rc;
}

/* Output y[t][n] = sum over superblocks of the one float fold
 *   Q4_K/Q5_K  d*d8*P - dmin*d8*M,     Q6_K  d*d8*P,
 * formed in double from the integer partials. */
int orc_matmul(int fmt, const uint8_t *recs, int64_t n, int64_t k,
               const int8_t *xq, const float *xs, const int16_t *xbs, int64_t t,
               double *y)
{
    int bb = orc_block_bytes(fmt);
    if (!bb || k % QK) return -1;
    int64_t nsb = k / QK;
    orc_block b;
    int32_t P, M;
    int rc = 0;
    for (int64_t r = 0; r < n; ++r) {
        for (int64_t tt = 0; tt < t; ++tt) y[tt * n + r] = 0.0;
        for (int64_t s = 0; s < nsb; ++s) {
            const uint8_t *rec = recs + (r * nsb + s) * bb;
            orc_decode(fmt, rec, &b);
            for (int64_t tt = 0; tt < t; ++tt) {
                /* the partials of this one (row, superblock, token) */
                int e = orc_partials(fmt, rec, 1, QK, xq + tt * k + s * QK, xbs + tt * (k / 16) + s * 16,
                                     1, &P, &M);
                if (e) rc = e;
                double d8 = xs[tt * nsb + s];
                y[tt * n + r] += b.d * d8 * P - b.dmin * d8 * M;
            }
        }
    }
    return rc;
}

/* Row-magnitude tolerance denominator R[t][n] = sum_i |w_i * xhat_i| with
 * xhat_i = d8 * a_i (the Q8_K-dequantised activation). */
int orc_rowmag(int fmt, const uint8_t *recs, int64_t n, int64_t k,
               const int8_t *xq, const float *xs, int64_t t, double *R)
{
    int bb = orc_block_bytes(fmt);
    if (!bb || k % QK) return -1;
    int64_t nsb = k / QK;
    double w[QK];
    for (int64_t r = 0; r < n; ++r) {
        for (int64_t tt = 0; tt < t; ++tt) R[tt * n + r] = 0.0;
        for (int64_t s = 0; s < nsb; ++s) {
            orc_dequantize(fmt, recs + (r * nsb + s) * bb, 1, QK, w);
            for (int64_t tt = 0; tt < t; ++tt) {
                double d8 = xs[tt * nsb + s], acc = 0.0;
                const int8_t *a = xq + tt * k + s * QK;
                for (int i = 0; i < QK; ++i) acc += fabs(w[i] * (d8 * a[i]));
                R[tt * n + r] += acc;
            }
        }
    }
    return 0;
}
