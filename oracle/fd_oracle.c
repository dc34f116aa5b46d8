/*
 * fd_oracle.c -- reference for single-query decode attention, fp64, CPU.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path
 * (the HIP library under split_kv_fd_amd/) never links, loads or calls it,
 * and the two share no code: this file has its own dtype decoders, its own
 * addressing and its own arithmetic.
 *
 * What it computes (the plain definition, written out):
 *
 *   For every batch row b and query head h, with kv head j = h / (Hq/Hkv)
 *   and valid length T_b (seq_lens[b], or T when no lengths are given):
 *
 *     s_t   = scale * sum_d q[b,h,d] * K[b,j,t,d]          t = 0 .. T_b-1
 *     m     = max_t s_t
 *     l     = sum_t exp(s_t - m)
 *     out_d = sum_t exp(s_t - m) * V[b,j,t,d] / l
 *     lse   = m + log(l)            (natural-log log-sum-exp of the logits)
 *
 * Sources:
 *   - "Kernel visualization: Flash Decoding" (tinyvolt), opening section:
 *     decode has one query row per (batch, head); flash decoding keeps the
 *     attention math and only changes how the KV axis is divided.  Its
 *     fd_split listing applies `scale` to the dot product before the max.
 *   - Zenaique Flash-Decoding explainer, "What decode looks like": Q is
 *     (batch, n_heads, 1, d_head), K and V are (batch, n_kv_heads, T,
 *     d_head); and its interview answer: the split/combine result equals
 *     the whole softmax exactly (shift invariance).
 *   - dupenodi guide "FlashDecoding and split-KV", "Walking through it":
 *     the split reduction keeps the math exact; engines also need paged /
 *     ragged KV layouts and GQA head grouping.
 *
 * Because the split method reaches this exact value (up to fp rounding
 * order), the oracle does NOT split, tile or rescale online: subtracting m
 * is only the textbook stable form of one softmax over all T_b logits.
 *
 * Readings taken where the pages are silent:
 *   - GQA: query head h reads kv head h / (Hq/Hkv) (consecutive groups).
 *   - Paged layout: pool [num_pages, Hkv, P, D]; token t of sequence b lives
 *     in page page_table[b*max_pages + t/P] at in-page row t % P.
 *   - LSE is the natural-log log-sum-exp of the scaled logits.
 *   - T_b == 0 gives out = 0 and lse = -inf (the pages' formula is 0/0
 *     there); parity of this convention is unpinned.
 *   - No causal mask: the decode query sees every cached token.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { FDO_F32 = 0, FDO_F16 = 1, FDO_BF16 = 2, FDO_F64 = 3 };

/* IEEE binary16 -> double, from the format's definition (exact). */
static double fdo_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int mant = h & 0x3ff;
    double mag;
    if (expo == 0)
        mag = ldexp((double)mant, -24);              /* zero / subnormal */
    else if (expo == 31)
        mag = mant ? NAN : INFINITY;
    else
        mag = ldexp((double)(1024 + mant), expo - 25);
    return sign ? -mag : mag;
}

/* bfloat16 is the top half of an IEEE binary32 (exact). */
static double fdo_bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double fdo_load(const void *base, size_t idx, int dtype)
{
    switch (dtype) {
    case FDO_F32: return (double)((const float *)base)[idx];
    case FDO_F16: return fdo_half_to_double(((const uint16_t *)base)[idx]);
    case FDO_BF16: return fdo_bf16_to_double(((const uint16_t *)base)[idx]);
    default: return ((const double *)base)[idx];
    }
}

/* Element offset of K[b, j, t, 0] (same for V). */
static size_t fdo_kv_row(int b, int j, int t, int Hkv, int T, int D,
                         const int32_t *page_table, int page_size,
                         int max_pages)
{
    if (!page_table)
        return (((size_t)b * Hkv + j) * (size_t)T + t) * (size_t)D;
    {
        int32_t page = page_table[(size_t)b * max_pages + t / page_size];
        int row = t % page_size;
        return (((size_t)page * Hkv + j) * (size_t)page_size + row) * (size_t)D;
    }
}

/*
 * out/lse rows: with rows == NULL every (b, h) pair is computed and out is
 * [B, Hq, D], lse [B, Hq].  Otherwise rows holds n_rows flat indices
 * b*Hq + h and out is [n_rows, D], lse [n_rows].  lse may be NULL.
 * Returns 0 on success, a negative code on invalid arguments.
 */
int fdo_decode(const void *q, const void *k, const void *v, int dtype,
               const int32_t *page_table, const int32_t *seq_lens,
               int page_size, int max_pages,
               int B, int Hq, int Hkv, int T, int D, double scale,
               const int32_t *rows, int n_rows,
               double *out, double *lse, int nthreads)
{
    int group, total, i;
    if (!q || !k || !v || !out) return -1;
    if (dtype < FDO_F32 || dtype > FDO_F64) return -2;
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || T <= 0 || D <= 0) return -3;
    if (Hq % Hkv != 0) return -4;
    if (page_table && (page_size <= 0 || max_pages <= 0)) return -5;
    if (page_table && (long)max_pages * page_size < T) return -5;
    if (rows && n_rows < 0) return -6;
    if (seq_lens)
        for (i = 0; i < B; ++i)
            if (seq_lens[i] < 0 || seq_lens[i] > T) return -7;
    if (rows)
        for (i = 0; i < n_rows; ++i)
            if (rows[i] < 0 || rows[i] >= B * Hq) return -8;
    group = Hq / Hkv;
    total = rows ? n_rows : B * Hq;

#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif

#pragma omp parallel for schedule(dynamic, 1)
    for (i = 0; i < total; ++i) {
        int bh = rows ? rows[i] : i;
        int b = bh / Hq, h = bh % Hq, j = h / group;
        int Tb = seq_lens ? seq_lens[b] : T;
        double *o = out + (size_t)i * D;
        const size_t qoff = ((size_t)b * Hq + h) * (size_t)D;
        double *s, m, l;
        int t, d;

        if (Tb == 0) {
            for (d = 0; d < D; ++d) o[d] = 0.0;
            if (lse) lse[i] = -INFINITY;
            continue;
        }
        s = (double *)malloc(sizeof(double) * (size_t)Tb);

        /* logits */
        for (t = 0; t < Tb; ++t) {
            size_t kr = fdo_kv_row(b, j, t, Hkv, T, D, page_table, page_size,
                                   max_pages);
            double dot = 0.0;
            for (d = 0; d < D; ++d)
                dot += fdo_load(q, qoff + d, dtype) * fdo_load(k, kr + d, dtype);
            s[t] = scale * dot;
        }

        /* one softmax over all T_b logits */
        m = s[0];
        for (t = 1; t < Tb; ++t)
            if (s[t] > m) m = s[t];
        l = 0.0;
        for (t = 0; t < Tb; ++t) {
            s[t] = exp(s[t] - m);
            l += s[t];
        }

        /* weighted sum of value rows, divided once by the normaliser */
        for (d = 0; d < D; ++d) o[d] = 0.0;
        for (t = 0; t < Tb; ++t) {
            size_t vr = fdo_kv_row(b, j, t, Hkv, T, D, page_table, page_size,
                                   max_pages);
            for (d = 0; d < D; ++d)
                o[d] += s[t] * fdo_load(v, vr + d, dtype);
        }
        for (d = 0; d < D; ++d) o[d] /= l;
        if (lse) lse[i] = m + log(l);
        free(s);
    }
    return 0;
}

/* Decoder entry points, exported so the tests can pin them against library
 * conversions (numpy float16, torch bfloat16). */
double fdo_decode_f16(uint16_t h) { return fdo_half_to_double(h); }
double fdo_decode_bf16(uint16_t b) { return fdo_bf16_to_double(b); }

int fdo_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
