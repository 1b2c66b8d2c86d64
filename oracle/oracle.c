/*
 * oracle.c -- plain, slow CPU reference for one decode step of attention over
 * a per-head, budget-limited KV cache and the eviction that keeps it at budget.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark load this file's library.  It shares no code,
 * header, table or constant with the HIP library; the two are checked against
 * each other, never built from each other.
 *
 * Everything is double precision, single threaded, one loop per definition.
 *
 * Sources (cited by page title and section):
 *  [P1] "Rethinking KV Cache Compression: from memory savings back to real
 *       serving end-to-end gains" (guide page), sections "2. cost structure of
 *       the 4 baselines", "16. background -- KV cache capacity formula" and
 *       "16. -- the 4 methods step by step".
 *  [P2] "KV Cache eviction in practice: when to drop the scorer and evict at
 *       random", sections "scorers are overrated", "six steps to land it" and
 *       "reference implementation".
 *  [R123] J. Salmon, M. Moraes, R. Dror, D. Shaw, "Parallel random numbers: as
 *       easy as 1, 2, 3", SC'11 -- the Philox4x32-10 counter-based generator.
 *  [OCP8] "OCP 8-bit Floating Point Specification (OFP8)", Open Compute
 *       Project -- the E5M2 format.
 *  [P1 KIVI] the guide page's KIVI passages: "2. cost structure of the 4
 *       baselines" (group 32, residual 128), "16. -- KV cache capacity
 *       formula" (keep every token, fewer bits, a full-precision recent
 *       residual), "16. -- the 4 methods step by step" (K quantized along
 *       channels, V along tokens) and "16. -- limits and conclusion" (scale
 *       granularity, periodic conversion when the residual fills).
 *
 * Readings where the pages are silent (each listed in the design notes):
 *  - scale 1/sqrt(D); no position encoding applied here (keys already carry it,
 *    [P2] "reference implementation", note on sort()).
 *  - q head i reads kv head floor(i / G).
 *  - a step attends first (the new token included), then evicts.
 *  - H2O score of a key = sum over the decode steps it was attended and over
 *    the G query heads of its group of the normalised softmax probability.
 *  - ties in any ranking go to the lower original position.
 *  - random keys: word 0 of Philox4x32-10 with counter (pos, step, kv head,
 *    sequence) and key (seed low word, seed high word); keep the n_keep
 *    smallest keys.
 *
 * Parity status: every function below is pinned by the not-gpu tests (closed
 * forms, brute force, published known-answer vectors, statistics).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_API __attribute__((visibility("default")))

/* ------------------------------------------------------------------------ */
/* KV bytes per token: 2 (K and V) x layers x kv heads x head_dim x dtype
 * bytes.  [P1] "16. KV cache capacity formula"; [P2] "six steps", last step.
 * Any non-positive argument gives 0. */
ORC_API uint64_t orc_bytes_per_token(int64_t layers, int64_t kv_heads,
                                     int64_t head_dim, int64_t dtype_bytes)
{
    if (layers <= 0 || kv_heads <= 0 || head_dim <= 0 || dtype_bytes <= 0)
        return 0;
    return (uint64_t)2 * (uint64_t)layers * (uint64_t)kv_heads *
           (uint64_t)head_dim * (uint64_t)dtype_bytes;
}

/* ------------------------------------------------------------------------ */
/* bf16 bit pattern -> double, exact: a bf16 value is the upper half of an
 * IEEE binary32 word. */
ORC_API void orc_bf16_to_f64(int64_t n, const uint16_t *bits, double *out)
{
    for (int64_t i = 0; i < n; ++i) {
        uint32_t w = (uint32_t)bits[i] << 16;
        float f;
        memcpy(&f, &w, sizeof f);
        out[i] = (double)f;
    }
}

/* ------------------------------------------------------------------------ */
/* 8-bit floating point E5M2 [OCP8]: the fp8 KV-cache dtype of the serving
 * command on [P2] ("fp8_e5m2").  1 sign bit, 5 exponent bits (bias 15), 2
 * mantissa bits; exponent field 0 holds zero and the subnormals m * 2^-16,
 * field 31 holds infinity (m = 0) and NaN (m != 0).  Exact in double. */
static double e5m2_value(unsigned c)
{
    const unsigned s = c >> 7, e = (c >> 2) & 31u, m = c & 3u;
    double v;
    if (e == 31u) v = (m == 0u) ? INFINITY : NAN;
    else if (e == 0u) v = ldexp((double)m, -16);
    else v = ldexp((double)(4u + m), (int)e - 17);   /* (1 + m/4) * 2^(e-15) */
    return s ? -v : v;
}

ORC_API void orc_e5m2_to_f64(int64_t n, const uint8_t *codes, double *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = e5m2_value(codes[i]);
}

/* The E5M2 code nearest to x, by plain search over the 124 non-negative
 * finite codes: ties go to the even code (round to nearest even);
 * magnitudes at or beyond the largest finite value, 57344, become +-57344
 * (saturation, as a fp8 cache write does); NaN becomes the NaN code 0x7F
 * with x's sign. */
ORC_API void orc_f64_to_e5m2(int64_t n, const double *x, uint8_t *out)
{
    for (int64_t i = 0; i < n; ++i) {
        const double v = x[i];
        const unsigned sign = signbit(v) ? 0x80u : 0u;
        if (isnan(v)) {
            out[i] = (uint8_t)(sign | 0x7Fu);
            continue;
        }
        const double a = fabs(v);
        unsigned best = 0x7Bu;
        if (a < 57344.0) {
            double bestd = INFINITY;
            for (unsigned c = 0; c <= 0x7Bu; ++c) {
                const double d = fabs(e5m2_value(c) - a);
                if (d < bestd || (d == bestd && (c & 1u) == 0u)) {
                    bestd = d;
                    best = c;
                }
            }
        }
        out[i] = (uint8_t)(sign | best);
    }
}

/* ------------------------------------------------------------------------ */
/* Philox4x32-10 [R123]: ten rounds of an S-box built from two 32x32->64
 * multiplications; round r uses key + r * (Weyl constants). */
static void philox_round(uint32_t c[4], uint32_t k0, uint32_t k1)
{
    const uint64_t m0 = 0xD2511F53u, m1 = 0xCD9E8D57u;
    uint64_t p0 = m0 * (uint64_t)c[0];
    uint64_t p1 = m1 * (uint64_t)c[2];
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t n0 = hi1 ^ c[1] ^ k0;
    uint32_t n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
}

ORC_API void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2],
                               uint32_t out[4])
{
    uint32_t c[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
    uint32_t k0 = key[0], k1 = key[1];
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        philox_round(c, k0, k1);
    }
    memcpy(out, c, sizeof c);
}

/* Random-eviction key of one cached token. */
ORC_API uint32_t orc_random_key(int32_t pos, uint64_t seed, uint32_t seq,
                                uint32_t head, uint32_t step)
{
    uint32_t ctr[4] = {(uint32_t)pos, step, head, seq};
    uint32_t key[2] = {(uint32_t)(seed & 0xFFFFFFFFu), (uint32_t)(seed >> 32)};
    uint32_t out[4];
    orc_philox4x32_10(ctr, key, out);
    return out[0];
}

/* ------------------------------------------------------------------------ */
/* Softmax attention of the G query heads of one kv head over n cached
 * entries (the new token is one of them):
 *   z_j = scale * <q, k_j>,  p_j = exp(z_j - max z) / sum_i exp(z_i - max z),
 *   o = sum_j p_j v_j.
 * q [G][D], K [n][D], V [n][D] row major; out [G][D]; p [G][n] or NULL.
 * A decode query sees every kept token and itself; nothing is masked.
 * [P1] "16. -- prefill, decode, TP" (decode reads all kept history). */
ORC_API void orc_attend(int32_t n, int32_t G, int32_t D, double scale,
                        const double *q, const double *K, const double *V,
                        double *out, double *p)
{
    double *z = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    for (int32_t g = 0; g < G; ++g) {
        const double *qg = q + (size_t)g * D;
        double *og = out + (size_t)g * D;
        for (int32_t d = 0; d < D; ++d)
            og[d] = 0.0;
        if (n <= 0)
            continue;
        double m = -INFINITY;
        for (int32_t j = 0; j < n; ++j) {
            double dot = 0.0;
            for (int32_t d = 0; d < D; ++d)
                dot += qg[d] * K[(size_t)j * D + d];
            z[j] = scale * dot;
            if (z[j] > m)
                m = z[j];
        }
        double l = 0.0;
        for (int32_t j = 0; j < n; ++j) {
            z[j] = exp(z[j] - m);
            l += z[j];
        }
        for (int32_t j = 0; j < n; ++j) {
            double pj = z[j] / l;
            if (p)
                p[(size_t)g * n + j] = pj;
            for (int32_t d = 0; d < D; ++d)
                og[d] += pj * V[(size_t)j * D + d];
        }
    }
    free(z);
}

/* ------------------------------------------------------------------------ */
/* StreamingLLM: keep the first n_sink positions (attention sinks) and the
 * n_recent most recent ones; drop the middle.  L = tokens seen so far, so the
 * recent window is positions L - n_recent .. L - 1.
 * [P1] "2. cost structure of the 4 baselines" and "16. -- the 4 methods step
 * by step" (64 sink + 448 recent = cache 512). */
ORC_API void orc_select_streaming(int32_t n, const int32_t *pos, int64_t L,
                                  int32_t n_sink, int32_t n_recent,
                                  uint8_t *keep)
{
    for (int32_t j = 0; j < n; ++j)
        keep[j] = (pos[j] < n_sink || (int64_t)pos[j] >= L - n_recent) ? 1 : 0;
}

/* ------------------------------------------------------------------------ */
/* ranking helpers for qsort: a total order, so the kept set is unique */
typedef struct {
    double score;   /* H2O: accumulated attention; random: key as a number */
    int32_t pos;
    int32_t idx;
} orc_rank;

static int by_score_desc_pos_asc(const void *a, const void *b)
{
    const orc_rank *x = (const orc_rank *)a, *y = (const orc_rank *)b;
    if (x->score > y->score) return -1;
    if (x->score < y->score) return 1;
    return (x->pos < y->pos) ? -1 : (x->pos > y->pos);
}

static int by_score_asc_pos_asc(const void *a, const void *b)
{
    const orc_rank *x = (const orc_rank *)a, *y = (const orc_rank *)b;
    if (x->score < y->score) return -1;
    if (x->score > y->score) return 1;
    return (x->pos < y->pos) ? -1 : (x->pos > y->pos);
}

/* H2O: the n_recent most recent tokens are always kept; among the others,
 * keep the n_heavy with the largest accumulated attention score (ties to the
 * lower position).  [P1] "2. cost structure" and "16. -- the 4 methods step
 * by step" (64 heavy + 448 recent; accumulate attention and update the kept
 * set). */
ORC_API void orc_select_h2o(int32_t n, const int32_t *pos, const double *score,
                            int64_t L, int32_t n_heavy, int32_t n_recent,
                            uint8_t *keep)
{
    orc_rank *c = (orc_rank *)malloc(sizeof(orc_rank) * (size_t)(n > 0 ? n : 1));
    int32_t nc = 0;
    for (int32_t j = 0; j < n; ++j) {
        if ((int64_t)pos[j] >= L - n_recent) {
            keep[j] = 1;
        } else {
            keep[j] = 0;
            c[nc].score = score[j];
            c[nc].pos = pos[j];
            c[nc].idx = j;
            ++nc;
        }
    }
    qsort(c, (size_t)nc, sizeof(orc_rank), by_score_desc_pos_asc);
    for (int32_t i = 0; i < nc && i < n_heavy; ++i)
        keep[c[i].idx] = 1;
    free(c);
}

/* Per-head uniform random eviction with the prompt pinned: positions below
 * prompt_len are never evicted; among the rest every head keeps the same
 * number n_keep, drawn independently per head (no union across heads).
 * Drawing a uniform n_keep-subset is done by giving every candidate an
 * independent random key and keeping the n_keep smallest keys (ties to the
 * lower position).  If there are at most n_keep candidates all are kept.
 * [P2] "scorers are overrated" (keep the prompt, evict uniformly inside each
 * head), "six steps" (pin the prompt), "reference implementation" (per-head
 * independent gather, equal counts, identity when nothing follows the
 * prompt). */
ORC_API void orc_select_random(int32_t n, const int32_t *pos, int32_t prompt_len,
                               int32_t n_keep, uint64_t seed, uint32_t seq,
                               uint32_t head, uint32_t step, uint8_t *keep)
{
    orc_rank *c = (orc_rank *)malloc(sizeof(orc_rank) * (size_t)(n > 0 ? n : 1));
    int32_t nc = 0;
    for (int32_t j = 0; j < n; ++j) {
        if (pos[j] < prompt_len) {
            keep[j] = 1;
        } else {
            keep[j] = 0;
            c[nc].score = (double)orc_random_key(pos[j], seed, seq, head, step);
            c[nc].pos = pos[j];
            c[nc].idx = j;
            ++nc;
        }
    }
    qsort(c, (size_t)nc, sizeof(orc_rank), by_score_asc_pos_asc);
    for (int32_t i = 0; i < nc && i < n_keep; ++i)
        keep[c[i].idx] = 1;
    free(c);
}

/* Random-eviction keys of n cached tokens of one unit: key[i] is
 * orc_random_key(pos[i], seed, seq, head, step), one token at a time. */
ORC_API void orc_random_keys(int64_t n, const int32_t *pos, uint64_t seed, uint32_t seq,
                             uint32_t head, uint32_t step, uint32_t *key)
{
    for (int64_t i = 0; i < n; ++i)
        key[i] = orc_random_key(pos[i], seed, seq, head, step);
}

/* Positions-only replay of per-head random eviction over a run of decode
 * steps of one unit (sequence seq, kv head head): the kept set depends on
 * positions and keys only, never on K, V or the queries, so a whole trace
 * can be followed without attention.  The unit starts with the n0 positions
 * pos0 (any order).  Step t = 0 .. steps-1 appends the token at position
 * first_pos + t (a step attends first, then evicts), then keeps what
 * orc_select_random keeps with step number first_step + t.  The positions
 * it drops are appended to evicted[] (at most ev_cap in all) and their count
 * goes to n_evicted[t].  The final kept positions, ascending, go to pos_out
 * (room for cap) and their count to *n_out.  Returns 0, or -1 when the kept
 * set would exceed cap or the drops ev_cap (nothing after that is valid).
 * [P2] "scorers are overrated" (evict uniformly inside each head every
 * time the cache is over budget), "six steps" (pin the prompt). */
ORC_API int32_t orc_random_replay(int32_t n0, const int32_t *pos0, int32_t cap, int32_t steps,
                                  int32_t first_pos, uint32_t first_step, int32_t prompt_len,
                                  int32_t n_keep, uint64_t seed, uint32_t seq, uint32_t head,
                                  int32_t *n_evicted, int32_t *evicted, int64_t ev_cap,
                                  int32_t *pos_out, int32_t *n_out)
{
    int32_t *cur = (int32_t *)malloc(sizeof(int32_t) * (size_t)(cap + 1));
    uint8_t *keep = (uint8_t *)malloc((size_t)(cap + 1));
    int32_t n = 0;
    int64_t ne = 0;
    int32_t rc = 0;
    if (n0 > cap) {
        rc = -1;
        goto done;
    }
    for (int32_t i = 0; i < n0; ++i)
        cur[n++] = pos0[i];
    for (int32_t t = 0; t < steps; ++t) {
        cur[n++] = first_pos + t;                       /* the new token */
        orc_select_random(n, cur, prompt_len, n_keep, seed, seq, head,
                          first_step + (uint32_t)t, keep);
        int32_t m = 0, dropped = 0;
        for (int32_t j = 0; j < n; ++j) {
            if (keep[j]) {
                cur[m++] = cur[j];
            } else {
                if (ne >= ev_cap) {
                    rc = -1;
                    goto done;
                }
                evicted[ne++] = cur[j];
                ++dropped;
            }
        }
        n_evicted[t] = dropped;
        n = m;
        if (n > cap) {
            rc = -1;
            goto done;
        }
    }
    /* ascending positions: insertion sort, plain and obviously correct */
    for (int32_t i = 1; i < n; ++i) {
        const int32_t x = cur[i];
        int32_t j = i - 1;
        while (j >= 0 && cur[j] > x) {
            cur[j + 1] = cur[j];
            --j;
        }
        cur[j + 1] = x;
    }
    for (int32_t i = 0; i < n; ++i)
        pos_out[i] = cur[i];
    *n_out = n;
done:
    free(cur);
    free(keep);
    return rc;
}

/* n_keep of the one-shot hook: max(1, int(N * keep_ratio)) with the product
 * taken in double and truncated, clamped to N (taking the first n_keep of a
 * permutation of N cannot give more than N); N <= 0 gives 0 (nothing to
 * evict, the cache is returned unchanged).  [P2] "reference implementation". */
ORC_API int64_t orc_n_keep(int64_t N, double keep_ratio)
{
    if (N <= 0)
        return 0;
    double prod = (double)N * keep_ratio;
    int64_t k = (int64_t)prod;       /* C truncation toward zero, like int() */
    if (k < 1)
        k = 1;
    if (k > N)
        k = N;
    return k;
}

/* ------------------------------------------------------------------------ */
/* KIVI-style quantization of groups of values [P1 KIVI].  Each group gets
 * its own asymmetric uniform grid of 2^bits levels between its minimum and
 * maximum:
 *     lo = min, scale = (max - lo) / (2^bits - 1),
 *     code = round-half-to-even((x - lo) / scale) clamped to [0, 2^bits - 1]
 *     (every code 0 when scale is 0),     value = code * scale + lo.
 * The pages fix neither the grid nor the precision of its parameters; the
 * reading taken is the plain min/max grid with lo and scale kept in binary32.
 * The code decisions are taken in binary32 arithmetic -- every operation
 * rounded to float, as the device kernel that must reproduce the codes bit
 * for bit takes them -- while the values are formed exactly in double.
 * x: n_groups consecutive groups of len values. */
ORC_API void orc_quantize_groups(int64_t n_groups, int32_t len, int32_t bits, const float *x,
                                 uint8_t *codes, float *scale, float *lo)
{
    const float top = (float)((1 << bits) - 1);
    for (int64_t g = 0; g < n_groups; ++g) {
        const float *xg = x + g * len;
        float mn = xg[0], mx = xg[0];
        for (int32_t i = 1; i < len; ++i) {
            if (xg[i] < mn)
                mn = xg[i];
            if (xg[i] > mx)
                mx = xg[i];
        }
        const float s = (mx - mn) / top;
        scale[g] = s;
        lo[g] = mn;
        for (int32_t i = 0; i < len; ++i) {
            float c = 0.0f;
            if (s > 0.0f) {
                const float t = (xg[i] - mn) / s;
                c = rintf(t);
                if (c < 0.0f)
                    c = 0.0f;
                if (c > top)
                    c = top;
            }
            codes[g * len + i] = (uint8_t)c;
        }
    }
}

/* value of each code: code * scale + lo in double, element i using
 * scale[i / len] and lo[i / len] */
ORC_API void orc_dequantize_groups(int64_t n_groups, int32_t len, const uint8_t *codes,
                                   const float *scale, const float *lo, double *out)
{
    for (int64_t g = 0; g < n_groups; ++g)
        for (int32_t i = 0; i < len; ++i)
            out[g * len + i] = (double)codes[g * len + i] * (double)scale[g] + (double)lo[g];
}
