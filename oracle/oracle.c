/*
 * CPU oracle for single-query decode attention over a growing KV cache.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or
 * call this file: only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it. It shares no code, header, table or constant with the
 * HIP library; it is written from the method's definition alone.
 *
 * What it computes (page "MoA-Structured Decode Attention", §2 Decode DNF):
 *   Step I   (eq. 1)  s[l] = scale * sum_j q[j] * K[l][j]     K read row by row
 *   Step II  (eq. 2)  m = max_l s[l];  e[l] = exp(s[l] - m);  Z = sum_l e[l];
 *                     a[l] = e[l] / Z
 *   Step III (eq. 3)  out[d] = sum_l a[l] * V[l][d]
 * lifted to a batch of sequences and heads (same page, rank lifting of the
 * Omega inner product) with grouped-query selection: query head h of a
 * sequence reads KV head h / g, g = h_q / h_kv (same page, §6 GQA/MQA, the
 * psi-selection of the KV group). Every sum runs in ascending index order in
 * IEEE double precision, one head at a time, so the result does not depend on
 * how many threads run the loop over heads.
 *
 * Cache layout (same page, §4, the gamma offset of row-major storage lifted
 * to rank 4): element (b, kvh, l, j) of a cache of capacity cap rows lies at
 * flat offset ((b*h_kv + kvh)*cap + l)*d + j.
 *
 * The KV-cache accumulation (same page, §5: concatenation # of one row per
 * step at the precomputed gamma offset) is oracle_kv_append below.
 *
 * Inputs are widened exactly to double: fp32 directly, bf16 by placing its
 * 16 bits in the top half of an fp32, fp8 e4m3fn with the decoder below
 * (OCP definition: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits,
 * subnormals at exponent 0, the two all-ones codes 0x7F / 0xFF are NaN, no
 * infinities). An fp8 element's value is decode(code) * scale, computed in
 * double, which is exact. An int8 element is its two's-complement code, also
 * times its slot's scale (symmetric 8-bit quantisation, the same per-(sequence,
 * KV head, K or V) scale as fp8). The decode-attention roofline page names
 * int8 and fp8 KV together as the lever that halves the bytes read per step
 * (its flop/byte derivation: AI = 2g with one byte per element); it fixes no
 * scale granularity, so both 8-bit types share the fp8 slots.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_F32 0
#define ORACLE_BF16 1
#define ORACLE_FP8_E4M3FN 2
#define ORACLE_INT8 3

double oracle_bf16_to_f64(uint16_t bits) {
    uint32_t w = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

double oracle_e4m3fn_to_f64(uint8_t code) {
    int sign = (code >> 7) & 1;
    int expo = (code >> 3) & 0xF;
    int mant = code & 0x7;
    double v;
    if (expo == 0xF && mant == 0x7) return NAN; /* 0x7F and 0xFF */
    if (expo == 0)
        v = ldexp((double)mant, -9);            /* 2^(1-7) * mant/8 */
    else
        v = ldexp(1.0 + mant / 8.0, expo - 7);
    return sign ? -v : v;
}

double oracle_int8_to_f64(int8_t code) { return (double)code; }

static int elem_bytes(int dtype) {
    switch (dtype) {
    case ORACLE_F32: return 4;
    case ORACLE_BF16: return 2;
    case ORACLE_FP8_E4M3FN: return 1;
    case ORACLE_INT8: return 1;
    default: return 0;
    }
}

/* Element types whose values carry a per-slot scale. */
static int scaled(int dtype) { return dtype == ORACLE_FP8_E4M3FN || dtype == ORACLE_INT8; }

/* Element idx of a flat array of the given dtype, widened to double. */
static double load_elem(const void *base, int dtype, size_t idx) {
    switch (dtype) {
    case ORACLE_F32: return (double)((const float *)base)[idx];
    case ORACLE_BF16: return oracle_bf16_to_f64(((const uint16_t *)base)[idx]);
    case ORACLE_INT8: return oracle_int8_to_f64(((const int8_t *)base)[idx]);
    default: return oracle_e4m3fn_to_f64(((const uint8_t *)base)[idx]);
    }
}

/*
 * One head, Steps I-III on fp64 arrays: q[d_k], K[n][d_k], V[n][d_v].
 * Optional intermediates s, e, a (length n) and m, Z may be NULL.
 * Returns 0, or -1 when n < 1 (softmax of an empty score vector is undefined).
 */
int oracle_head_f64(int n, int d_k, int d_v, double scale, const double *q,
                    const double *K, const double *V, double *s_out,
                    double *e_out, double *a_out, double *m_out, double *Z_out,
                    double *out) {
    if (n < 1) return -1;
    double *s = (double *)malloc(sizeof(double) * (size_t)n * 3);
    if (!s) return -2;
    double *e = s + n, *a = s + 2 * (size_t)n;
    /* Step I: one score per cached row, the row contracted with q. */
    for (int l = 0; l < n; ++l) {
        double acc = 0.0;
        for (int j = 0; j < d_k; ++j) acc += q[j] * K[(size_t)l * d_k + j];
        s[l] = scale * acc;
    }
    /* Step II: stable softmax. */
    double m = s[0];
    for (int l = 1; l < n; ++l)
        if (s[l] > m) m = s[l];
    double Z = 0.0;
    for (int l = 0; l < n; ++l) {
        e[l] = exp(s[l] - m);
        Z += e[l];
    }
    for (int l = 0; l < n; ++l) a[l] = e[l] / Z;
    /* Step III: weighted sum of the value rows. */
    for (int d = 0; d < d_v; ++d) {
        double acc = 0.0;
        for (int l = 0; l < n; ++l) acc += a[l] * V[(size_t)l * d_v + d];
        out[d] = acc;
    }
    if (s_out) memcpy(s_out, s, sizeof(double) * n);
    if (e_out) memcpy(e_out, e, sizeof(double) * n);
    if (a_out) memcpy(a_out, a, sizeof(double) * n);
    if (m_out) *m_out = m;
    if (Z_out) *Z_out = Z;
    free(s);
    return 0;
}

/*
 * Batched, multi-head, grouped-query decode attention over typed caches.
 *   q        [B, h_q, d_k]            dtype q_dtype
 *   k_cache  [B, h_kv, cap, d_k]      dtype kv_dtype
 *   v_cache  [B, h_kv, cap, d_v]      dtype kv_dtype
 *   lens     [B]                      rows attended per sequence (1..cap)
 *   kv_scales[B, h_kv, 2] fp32        (K scale, V scale); only for fp8 / int8, else NULL
 *   out      [B, h_q, d_v]  double
 * The optional byte maps q_mark / k_mark / v_mark (one byte per element of
 * q, k_cache, v_cache) are set to 1 for every element the loops read; with
 * any of them given the loop runs on one thread. Returns 0 or a negative
 * code for invalid arguments.
 */
int oracle_decode_f64_traced(int B, int h_q, int h_kv, int d_k, int d_v,
                             int cap, int q_dtype, int kv_dtype, float scale,
                             const void *q, const void *k_cache,
                             const void *v_cache, const int32_t *lens,
                             const float *kv_scales, double *out, int nthreads,
                             uint8_t *q_mark, uint8_t *k_mark, uint8_t *v_mark) {
    if (B < 0 || h_q < 1 || h_kv < 1 || h_q % h_kv || d_k < 1 || d_v < 1 || cap < 1)
        return -1;
    if (!elem_bytes(q_dtype) || !elem_bytes(kv_dtype)) return -1;
    if (scaled(kv_dtype) && !kv_scales) return -1;
    for (int b = 0; b < B; ++b)
        if (lens[b] < 1 || lens[b] > cap) return -3;
    const int g = h_q / h_kv;
    const int traced = q_mark || k_mark || v_mark;
    const int nthr = traced ? 1 : (nthreads > 0 ? nthreads : omp_get_max_threads());
    int status = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthr) reduction(min : status)
    for (long bh = 0; bh < (long)B * h_q; ++bh) {
        const int b = (int)(bh / h_q), h = (int)(bh % h_q);
        const int kvh = h / g; /* the KV group this query head selects */
        const int n = lens[b];
        const size_t slot = (size_t)b * h_kv + kvh;
        double ks = 1.0, vs = 1.0;
        if (scaled(kv_dtype)) {
            ks = (double)kv_scales[slot * 2 + 0];
            vs = (double)kv_scales[slot * 2 + 1];
        }
        double *qd = (double *)malloc(sizeof(double) * (size_t)d_k);
        double *Kd = (double *)malloc(sizeof(double) * (size_t)n * d_k);
        double *Vd = (double *)malloc(sizeof(double) * (size_t)n * d_v);
        if (!qd || !Kd || !Vd) {
            free(qd); free(Kd); free(Vd);
            status = -2;
            continue;
        }
        for (int j = 0; j < d_k; ++j) {
            size_t idx = (size_t)bh * d_k + j;
            qd[j] = load_elem(q, q_dtype, idx);
            if (q_mark) q_mark[idx] = 1;
        }
        for (int l = 0; l < n; ++l) {
            for (int j = 0; j < d_k; ++j) {
                size_t idx = (slot * cap + l) * d_k + j;
                Kd[(size_t)l * d_k + j] = load_elem(k_cache, kv_dtype, idx) * ks;
                if (k_mark) k_mark[idx] = 1;
            }
            for (int d = 0; d < d_v; ++d) {
                size_t idx = (slot * cap + l) * d_v + d;
                Vd[(size_t)l * d_v + d] = load_elem(v_cache, kv_dtype, idx) * vs;
                if (v_mark) v_mark[idx] = 1;
            }
        }
        int rc = oracle_head_f64(n, d_k, d_v, (double)scale, qd, Kd, Vd, NULL,
                                 NULL, NULL, NULL, NULL, out + (size_t)bh * d_v);
        if (rc < status) status = rc;
        free(qd); free(Kd); free(Vd);
    }
    return status;
}

int oracle_decode_f64(int B, int h_q, int h_kv, int d_k, int d_v, int cap,
                      int q_dtype, int kv_dtype, float scale, const void *q,
                      const void *k_cache, const void *v_cache,
                      const int32_t *lens, const float *kv_scales, double *out,
                      int nthreads) {
    return oracle_decode_f64_traced(B, h_q, h_kv, d_k, d_v, cap, q_dtype,
                                    kv_dtype, scale, q, k_cache, v_cache, lens,
                                    kv_scales, out, nthreads, NULL, NULL, NULL);
}

/*
 * Multi-query causal decode (several query rows per sequence, as in speculative decoding
 * or a chunked prefill). Page "MoA-Structured Decode Attention", introduction: the decode
 * DNF is the forward DNF with the query-row index fixed to the current step; here it takes
 * the last T positions of each sequence instead of one. Page "Phase 3, Section 6:
 * StoryLM-0 head-parallel attention", §3: T query rows, softmax over the key axis of the
 * scaled scores plus a mask. The mask is causal: query t of sequence b sits at position
 * lens[b] - T + t, and its own row and every earlier row are visible, so it attends over
 * the first n = lens[b] - T + 1 + t rows with Steps I-III unchanged (T = 1 is
 * oracle_decode_f64).
 *   q   [B, T, h_q, d_k]   out [B, T, h_q, d_v] double   lens[b] >= T
 * Everything else as oracle_decode_f64.
 */
int oracle_decode_multi_f64(int B, int T, int h_q, int h_kv, int d_k, int d_v, int cap,
                            int q_dtype, int kv_dtype, float scale, const void *q,
                            const void *k_cache, const void *v_cache,
                            const int32_t *lens, const float *kv_scales, double *out,
                            int nthreads) {
    if (B < 0 || T < 1 || h_q < 1 || h_kv < 1 || h_q % h_kv || d_k < 1 || d_v < 1 || cap < 1)
        return -1;
    if (!elem_bytes(q_dtype) || !elem_bytes(kv_dtype)) return -1;
    if (scaled(kv_dtype) && !kv_scales) return -1;
    for (int b = 0; b < B; ++b)
        if (lens[b] < T || lens[b] > cap) return -3;
    const int g = h_q / h_kv;
    const int nthr = nthreads > 0 ? nthreads : omp_get_max_threads();
    int status = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthr) reduction(min : status)
    for (long bth = 0; bth < (long)B * T * h_q; ++bth) {
        const int b = (int)(bth / ((long)T * h_q));
        const int t = (int)(bth / h_q % T), h = (int)(bth % h_q);
        const int kvh = h / g; /* its KV group */
        const int n = lens[b] - T + 1 + t; /* causal: rows 0 .. lens[b] - T + t */
        const size_t slot = (size_t)b * h_kv + kvh;
        double ks = 1.0, vs = 1.0;
        if (scaled(kv_dtype)) {
            ks = (double)kv_scales[slot * 2 + 0];
            vs = (double)kv_scales[slot * 2 + 1];
        }
        double *qd = (double *)malloc(sizeof(double) * (size_t)d_k);
        double *Kd = (double *)malloc(sizeof(double) * (size_t)n * d_k);
        double *Vd = (double *)malloc(sizeof(double) * (size_t)n * d_v);
        if (!qd || !Kd || !Vd) {
            free(qd); free(Kd); free(Vd);
            status = -2;
            continue;
        }
        for (int j = 0; j < d_k; ++j) qd[j] = load_elem(q, q_dtype, (size_t)bth * d_k + j);
        for (int l = 0; l < n; ++l) {
            for (int j = 0; j < d_k; ++j)
                Kd[(size_t)l * d_k + j] = load_elem(k_cache, kv_dtype, (slot * cap + l) * d_k + j) * ks;
            for (int d = 0; d < d_v; ++d)
                Vd[(size_t)l * d_v + d] = load_elem(v_cache, kv_dtype, (slot * cap + l) * d_v + d) * vs;
        }
        int rc = oracle_head_f64(n, d_k, d_v, (double)scale, qd, Kd, Vd, NULL,
                                 NULL, NULL, NULL, NULL, out + (size_t)bth * d_v);
        if (rc < status) status = rc;
        free(qd); free(Kd); free(Vd);
    }
    return status;
}

/*
 * Decode attention over one shard of the rows, with each query row's log-sum-exp, for a
 * context split over several devices: each holds a contiguous part of every sequence's rows as
 * a cache of its own. Page "MoA-Structured Decode Attention", §2 eq. (2): Step II normalises by
 * Z = sum_l exp(s[l] - m); over a union of disjoint row sets the normalisation is the
 * log-sum-exp-weighted combination of the sets' own (oracle_merge_lse_f64), which needs each
 * set's lse = ln sum_l exp(s[l]) = m + ln Z.
 * Query t of sequence b attends over the first n = lens[b] - T + 1 + t rows of this cache
 * (T = 1: all lens[b] rows), Steps I-III as oracle_head_f64; lse takes that head's m and Z.
 * lens[b] = 0 (the shard holds no rows of sequence b): out 0 and lse -inf.
 *   q [B, T, h_q, d_k]   out [B, T, h_q, d_v] double   lse [B, T, h_q] double
 * Everything else as oracle_decode_multi_f64. Returns -3 if a lens[b] is in [1, T) or above cap.
 */
int oracle_decode_lse_f64(int B, int T, int h_q, int h_kv, int d_k, int d_v, int cap,
                          int q_dtype, int kv_dtype, float scale, const void *q,
                          const void *k_cache, const void *v_cache,
                          const int32_t *lens, const float *kv_scales, double *out,
                          double *lse, int nthreads) {
    if (B < 0 || T < 1 || h_q < 1 || h_kv < 1 || h_q % h_kv || d_k < 1 || d_v < 1 || cap < 1)
        return -1;
    if (!elem_bytes(q_dtype) || !elem_bytes(kv_dtype)) return -1;
    if (scaled(kv_dtype) && !kv_scales) return -1;
    for (int b = 0; b < B; ++b)
        if (lens[b] < 0 || (lens[b] > 0 && lens[b] < T) || lens[b] > cap) return -3;
    const int g = h_q / h_kv;
    const int nthr = nthreads > 0 ? nthreads : omp_get_max_threads();
    int status = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthr) reduction(min : status)
    for (long bth = 0; bth < (long)B * T * h_q; ++bth) {
        const int b = (int)(bth / ((long)T * h_q));
        const int t = (int)((bth / h_q) % T);
        const int h = (int)(bth % h_q), kvh = h / g;
        if (lens[b] == 0) { /* no rows of this sequence in the shard */
            for (int d = 0; d < d_v; ++d) out[(size_t)bth * d_v + d] = 0.0;
            lse[bth] = -INFINITY;
            continue;
        }
        const int n = t + 1 + lens[b] - T; /* causal: its own row and every earlier one */
        const size_t slot = (size_t)b * h_kv + kvh;
        double ks = 1.0, vs = 1.0;
        if (scaled(kv_dtype)) {
            ks = (double)kv_scales[slot * 2 + 0];
            vs = (double)kv_scales[slot * 2 + 1];
        }
        double *qd = (double *)malloc(sizeof(double) * (size_t)d_k);
        double *Kd = (double *)malloc(sizeof(double) * (size_t)n * d_k);
        double *Vd = (double *)malloc(sizeof(double) * (size_t)n * d_v);
        if (!qd || !Kd || !Vd) {
            free(qd); free(Kd); free(Vd);
            status = -2;
            continue;
        }
        for (int j = 0; j < d_k; ++j) qd[j] = load_elem(q, q_dtype, (size_t)bth * d_k + j);
        for (int l = 0; l < n; ++l) {
            for (int j = 0; j < d_k; ++j)
                Kd[(size_t)l * d_k + j] = load_elem(k_cache, kv_dtype, (slot * cap + l) * d_k + j) * ks;
            for (int d = 0; d < d_v; ++d)
                Vd[(size_t)l * d_v + d] = load_elem(v_cache, kv_dtype, (slot * cap + l) * d_v + d) * vs;
        }
        double m = 0.0, Z = 0.0;
        int rc = oracle_head_f64(n, d_k, d_v, (double)scale, qd, Kd, Vd, NULL, NULL, NULL, &m, &Z,
                                 out + (size_t)bth * d_v);
        lse[bth] = m + log(Z);
        if (rc < status) status = rc;
        free(qd); free(Kd); free(Vd);
    }
    return status;
}

/*
 * Merge of P results over disjoint row sets (same passage): for every row r, with
 * M = max_p lses[p][r] and w_p = exp(lses[p][r] - M),
 *   out[r] = sum_p w_p * outs[p][r] / sum_p w_p,   lse_out[r] = M + ln sum_p w_p.
 * A row that no part holds (every lse -inf) gets out 0 and lse -inf.
 *   outs [P, rows, d], lses [P, rows]; out [rows, d], lse_out [rows]; all double.
 */
void oracle_merge_lse_f64(int P, long rows, int d, const double *outs, const double *lses,
                          double *out, double *lse_out) {
    for (long r = 0; r < rows; ++r) {
        double M = -INFINITY;
        for (int p = 0; p < P; ++p)
            if (lses[(size_t)p * rows + r] > M) M = lses[(size_t)p * rows + r];
        if (M == -INFINITY) {
            for (int c = 0; c < d; ++c) out[(size_t)r * d + c] = 0.0;
            lse_out[r] = -INFINITY;
            continue;
        }
        double W = 0.0;
        for (int p = 0; p < P; ++p) W += exp(lses[(size_t)p * rows + r] - M);
        for (int c = 0; c < d; ++c) {
            double acc = 0.0;
            for (int p = 0; p < P; ++p)
                acc += exp(lses[(size_t)p * rows + r] - M) * outs[((size_t)p * rows + r) * d + c];
            out[(size_t)r * d + c] = acc / W;
        }
        lse_out[r] = M + log(W);
    }
}

/*
 * KV-cache accumulation: for every sequence b and KV head kvh, copy row
 * k_new[b][kvh] into k_cache at row lens[b] (and v_new into v_cache), then
 * lens[b] += 1. Byte copies; every other byte of the caches is unchanged.
 * Returns -1 (and changes nothing) if some lens[b] is outside [0, cap).
 */
int oracle_kv_append(int B, int h_kv, int d_k, int d_v, int cap, int kv_dtype,
                     void *k_cache, void *v_cache, int32_t *lens,
                     const void *k_new, const void *v_new) {
    const int eb = elem_bytes(kv_dtype);
    if (!eb) return -1;
    for (int b = 0; b < B; ++b)
        if (lens[b] < 0 || lens[b] >= cap) return -1;
    for (int b = 0; b < B; ++b) {
        for (int kvh = 0; kvh < h_kv; ++kvh) {
            size_t slot = (size_t)b * h_kv + kvh;
            size_t krow = (slot * cap + (size_t)lens[b]) * d_k * eb;
            size_t vrow = (slot * cap + (size_t)lens[b]) * d_v * eb;
            memcpy((char *)k_cache + krow, (const char *)k_new + slot * d_k * eb, (size_t)d_k * eb);
            memcpy((char *)v_cache + vrow, (const char *)v_new + slot * d_v * eb, (size_t)d_v * eb);
        }
        lens[b] += 1;
    }
    return 0;
}
