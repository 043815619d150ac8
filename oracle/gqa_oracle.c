/*
 * gqa_oracle.c -- plain, slow fp64 CPU oracle for grouped-query attention.
 *
 * TEST INFRASTRUCTURE. Only the tests, the package smoke check and the
 * benchmark's CPU-baseline leg may load this library. The GPU library never
 * links it, includes it or calls it, and this file includes nothing from the
 * GPU library.
 *
 * Every floating-point input is read as its exact stored bits (bf16, fp32 or
 * fp64), widened to double, and every step below is computed in double with
 * plain loops in the order the definition states: no blocking, no online or
 * split softmax, no reordering. OpenMP only spreads independent output rows
 * over threads; it changes no arithmetic.
 *
 * Sources (the web pages this library follows):
 *  [KB]  "Grouped-Query Attention", llm-arch-kb (lizeman.github.io):
 *        section 1 Premise; section 2 Derivation (Setup, The grouping,
 *        KV-cache footprint, Uptraining recipe); section 3 Reference
 *        implementation (Sketch: grouping and broadcast).
 *  [CARD] "GQA: Training Generalized Multi-Query Transformer Models from
 *        Multi-Head Checkpoints", crackai.dev paper card: How It Works.
 *  [MQA] "Multi-Query and Grouped-Query Attention", praveentn.live:
 *        Grouped-query attention: the compromise that shipped.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_BF16 = 0, ORACLE_F32 = 1, ORACLE_F64 = 2, ORACLE_F16 = 3 };

static size_t elem_bytes(int dtype)
{
    return dtype == ORACLE_F64 ? 8 : (dtype == ORACLE_F32 ? 4 : 2);
}

/* Exact widening of one stored element to double. A bf16 value is the upper
 * half of an IEEE binary32, so shifting its 16 bits up gives the same number
 * as a float, which converts to double exactly. */
static double widen(const void *base, int64_t i, int dtype)
{
    if (dtype == ORACLE_BF16) {
        uint32_t u = ((uint32_t)((const uint16_t *)base)[i]) << 16;
        float f;
        memcpy(&f, &u, sizeof f);
        return (double)f;
    }
    if (dtype == ORACLE_F16) {
        /* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction
         * bits. Normal: (1024 + frac) * 2^(exp - 25); subnormal: frac * 2^-24. */
        uint16_t hbits = ((const uint16_t *)base)[i];
        int sign = hbits >> 15, ex = (hbits >> 10) & 31, frac = hbits & 1023;
        double mag;
        if (ex == 0)
            mag = ldexp((double)frac, -24);
        else if (ex == 31)
            mag = frac ? NAN : INFINITY;
        else
            mag = ldexp((double)(frac + 1024), ex - 25);
        return sign ? -mag : mag;
    }
    if (dtype == ORACLE_F32)
        return (double)((const float *)base)[i];
    return ((const double *)base)[i];
}

/* [KB] section 2, The grouping: G divides H, the query heads form G contiguous
 * groups, and query head i (1-indexed) reads key/value group
 * g(i) = ceil(i*G/H) (1-indexed). Written here in the page's 1-indexed form
 * and converted to 0-indexed head and group numbers at the edges. */
int oracle_group_of_head(int h0, int H, int G)
{
    int64_t i = (int64_t)h0 + 1;                 /* 1-indexed head */
    int64_t num = i * (int64_t)G;
    int64_t g1 = (num + H - 1) / H;              /* ceil(i*G/H) */
    return (int)(g1 - 1);                        /* 0-indexed group */
}

/* [KB] section 1 (MHA stores one key and one value vector per head, per
 * token, per layer) and section 2, KV-cache footprint (GQA stores G keys and
 * G values per token per layer); [CARD] How It Works: cache = 2 x kv_heads x
 * d_head per token. Multiplied by the number of layers and the bytes of one
 * stored scalar. kv_heads = H gives MHA, 1 gives MQA. */
double oracle_kv_cache_bytes_per_token(int kv_heads, int d_h, int layers, int bytes_per_scalar)
{
    return 2.0 * (double)kv_heads * (double)d_h * (double)layers * (double)bytes_per_scalar;
}

static int clamp_len(int32_t L, int Tmax)
{
    if (L < 0)
        return 0;
    if (L > Tmax)
        return Tmax;
    return (int)L;
}

/* One attention row: scores s_t = scale * <q, k_t> for t in [0, L), then the
 * max-subtracted softmax over t, then the probability-weighted sum of the
 * value rows. k_t and v_t are found at key_base + t*key_stride (elements).
 * Writes D outputs to out; writes normalised probabilities to probs (L of
 * them) when probs is not NULL. L = 0 gives a zero row. */
static void attend_row(const void *q, int64_t q_off, const void *k, const void *v, int64_t key_base,
                       int64_t key_stride, int L, int D, int dtype, double scale, double *out,
                       double *probs)
{
    int d, t;
    if (L <= 0) {
        for (d = 0; d < D; ++d)
            out[d] = 0.0;
        return;
    }
    double *s = (double *)malloc(sizeof(double) * (size_t)L);
    double m = -INFINITY;
    for (t = 0; t < L; ++t) {
        double dot = 0.0;
        for (d = 0; d < D; ++d)
            dot += widen(q, q_off + d, dtype) * widen(k, key_base + (int64_t)t * key_stride + d, dtype);
        s[t] = scale * dot;
        if (s[t] > m)
            m = s[t];
    }
    double denom = 0.0;
    for (t = 0; t < L; ++t) {
        s[t] = exp(s[t] - m);
        denom += s[t];
    }
    for (d = 0; d < D; ++d) {
        double acc = 0.0;
        for (t = 0; t < L; ++t)
            acc += s[t] * widen(v, key_base + (int64_t)t * key_stride + d, dtype);
        out[d] = acc / denom;
    }
    if (probs)
        for (t = 0; t < L; ++t)
            probs[t] = s[t] / denom;
    free(s);
}

/* Decode: one new query per sequence against its cached keys and values.
 * [KB] section 1: at a decode step every cached entry is read to produce one
 * token; section 2, Setup: head i attends over its cached K and V; The
 * grouping: head i reads group g(i); section 3 sketch: scores are q.k^T
 * scaled, softmax over the key axis, then times v.
 *
 *   q        [B, H, D]
 *   k, v     [B, Tmax, G, D]   only positions t < L_b are read
 *   seqlens  [B]               L_b = clamp(seqlens[b], 0, Tmax)
 *   out      [B, H, D]         fp64
 *   probs    [B, H, Tmax] or NULL; softmax weights, zero beyond L_b
 */
void oracle_decode(const void *q, const void *k, const void *v, int dtype, const int32_t *seqlens,
                   int B, int H, int G, int D, int Tmax, double scale, double *out, double *probs)
{
    int64_t rows = (int64_t)B * H;
    int64_t row;
#pragma omp parallel for schedule(dynamic, 1)
    for (row = 0; row < rows; ++row) {
        int b = (int)(row / H), h = (int)(row % H);
        int g = oracle_group_of_head(h, H, G);
        int L = clamp_len(seqlens[b], Tmax);
        int64_t key_base = ((int64_t)b * Tmax * G + g) * D;  /* k[b, 0, g, 0] */
        int64_t key_stride = (int64_t)G * D;                  /* one token    */
        double *p = NULL;
        if (probs) {
            p = probs + row * Tmax;
            for (int t = 0; t < Tmax; ++t)
                p[t] = 0.0;
        }
        attend_row(q, row * D, k, v, key_base, key_stride, L, D, dtype, scale, out + row * D, p);
    }
}

/* Prefill: every position of a sequence is a query.
 * [KB] section 3 sketch: q [B,T,H,d_h]; k, v [B,T,G,d_h] broadcast to the H
 * query heads group by group; scores divided by sqrt(d_h); causal mask; softmax
 * over keys; times v. The causal mask keeps key positions s <= t for query
 * position t (the diagonal included); causal = 0 keeps every key.
 *
 *   rows_b/t/h  NULL: compute every row into out [B, T, H, D]
 *               else: compute the n_rows listed rows into out [n_rows, D]
 */
void oracle_prefill(const void *q, const void *k, const void *v, int dtype, int B, int T, int H,
                    int G, int D, int causal, const int32_t *rows_b, const int32_t *rows_t,
                    const int32_t *rows_h, int64_t n_rows, double *out)
{
    int64_t rows = rows_b ? n_rows : (int64_t)B * T * H;
    double scale = 1.0 / sqrt((double)D);
    int64_t row;
#pragma omp parallel for schedule(dynamic, 1)
    for (row = 0; row < rows; ++row) {
        int b, t, h;
        if (rows_b) {
            b = rows_b[row];
            t = rows_t[row];
            h = rows_h[row];
        } else {
            b = (int)(row / ((int64_t)T * H));
            t = (int)((row / H) % T);
            h = (int)(row % H);
        }
        int g = oracle_group_of_head(h, H, G);
        int L = causal ? t + 1 : T;
        int64_t q_off = (((int64_t)b * T + t) * H + h) * D;
        int64_t key_base = ((int64_t)b * T * G + g) * D;
        attend_row(q, q_off, k, v, key_base, (int64_t)G * D, L, D, dtype, scale, out + row * D, NULL);
    }
}

/* Decode with the two common variants of a serving step, each optional:
 *
 *  Cache append (k_new, v_new not NULL). The new token's key and value join
 *  the cache before it is read: [KB] section 1, a decode step reads every
 *  cached entry, the new one included; section 2, Setup, head i attends over
 *  the keys and values cached so far. With L_b = clamp(seqlens[b], 0, Tmax):
 *  if L_b < Tmax, k_new[b] and v_new[b] ([G, D], every group) are written to
 *  cache position L_b and the sequence then holds L_b + 1 positions; a full
 *  cache (L_b = Tmax) is left unchanged and holds Tmax positions. k and v are
 *  updated in place.
 *
 *  Sliding window (window > 0): each query attends only to the `window` most
 *  recent positions of its sequence, [max(0, L - window), L) ([KB] section 4,
 *  Empirical evidence, Mistral 7B ablation: GQA-8 combined with
 *  sliding-window attention; the page gives no formula, and "the window most
 *  recent positions, the newest included" is the reading taken here).
 *  window = 0 keeps every position.
 *
 *   q            [B, H, D];  k_new, v_new [B, G, D] or NULL
 *   k, v         [B, Tmax, G, D]
 *   out          [B, H, D] fp64
 */
void oracle_decode_step(const void *q, const void *k_new, const void *v_new, void *k, void *v, int dtype,
                        const int32_t *seqlens, int B, int H, int G, int D, int Tmax, double scale, int window,
                        double *out)
{
    size_t es = elem_bytes(dtype);
    int *len = (int *)malloc(sizeof(int) * (size_t)(B > 0 ? B : 1));
    for (int b = 0; b < B; ++b) {
        int L = clamp_len(seqlens[b], Tmax);
        if (k_new && L < Tmax) {
            size_t row = (size_t)G * D * es;                     /* one token, every group */
            size_t dst = ((size_t)b * Tmax + L) * row;           /* k[b, L, 0, 0] */
            memcpy((char *)k + dst, (const char *)k_new + (size_t)b * row, row);
            memcpy((char *)v + dst, (const char *)v_new + (size_t)b * row, row);
            L = L + 1;
        }
        len[b] = L;
    }
    int64_t rows = (int64_t)B * H;
    int64_t row;
#pragma omp parallel for schedule(dynamic, 1)
    for (row = 0; row < rows; ++row) {
        int b = (int)(row / H), h = (int)(row % H);
        int g = oracle_group_of_head(h, H, G);
        int L = len[b];
        int lo = (window > 0 && L > window) ? L - window : 0;    /* first admissible position */
        int64_t key_stride = (int64_t)G * D;
        int64_t key_base = ((int64_t)b * Tmax * G + g) * D + (int64_t)lo * key_stride;
        attend_row(q, row * D, k, v, key_base, key_stride, L - lo, D, dtype, scale, out + row * D, NULL);
    }
    free(len);
}

/* Causal prefill with a sliding window: query position t attends to key
 * positions [max(0, t + 1 - window), t], the `window` most recent ones with
 * itself included (window = 0: every s <= t, the plain causal mask of [KB]
 * section 3). Rows as in oracle_prefill. */
void oracle_prefill_window(const void *q, const void *k, const void *v, int dtype, int B, int T, int H,
                           int G, int D, int window, const int32_t *rows_b, const int32_t *rows_t,
                           const int32_t *rows_h, int64_t n_rows, double *out)
{
    int64_t rows = rows_b ? n_rows : (int64_t)B * T * H;
    double inv_sqrt_d = 1.0 / sqrt((double)D);
    int64_t row;
#pragma omp parallel for schedule(dynamic, 1)
    for (row = 0; row < rows; ++row) {
        int b, t, h;
        if (rows_b) {
            b = rows_b[row];
            t = rows_t[row];
            h = rows_h[row];
        } else {
            b = (int)(row / ((int64_t)T * H));
            t = (int)((row / H) % T);
            h = (int)(row % H);
        }
        int g = oracle_group_of_head(h, H, G);
        int lo = (window > 0 && t + 1 > window) ? t + 1 - window : 0;
        int64_t q_off = (((int64_t)b * T + t) * H + h) * D;
        int64_t key_base = (((int64_t)b * T + lo) * G + g) * D;
        attend_row(q, q_off, k, v, key_base, (int64_t)G * D, t + 1 - lo, D, dtype, inv_sqrt_d, out + row * D,
                   NULL);
    }
}

/* Weighted conversion of key/value heads into G groups ([KB] section 4,
 * Empirical evidence, the Chinchilla-scale reproduction, which proposes
 * combining the heads of a group with per-head learned weights instead of the
 * plain mean): group g is sum_i w[i] * in[n, i, :] over the heads i assigned
 * to g by g(i). w = 1/r for every head is the mean-pool below.
 *
 *   in [N, H, D];  w [H] fp64;  out [N, G, D] fp64
 */
void oracle_weighted_pool(const void *in, int dtype, int64_t N, int H, int G, int D, const double *w,
                          double *out)
{
    int64_t n;
#pragma omp parallel for schedule(static)
    for (n = 0; n < N; ++n) {
        for (int g = 0; g < G; ++g) {
            double *o = out + (n * G + g) * D;
            for (int d = 0; d < D; ++d)
                o[d] = 0.0;
            for (int i = 0; i < H; ++i) {
                if (oracle_group_of_head(i, H, G) != g)
                    continue;
                for (int d = 0; d < D; ++d)
                    o[d] += w[i] * widen(in, (n * H + i) * D + d, dtype);
            }
        }
    }
}

/* Averaging conversion of multi-head key/value heads into G groups.
 * [KB] section 2, Uptraining recipe: each new group's weights start as the
 * mean of the original heads assigned to that group; [CARD] How It Works and
 * [MQA] the compromise that shipped: mean-pool the key/value heads within each
 * group. Heads are assigned with the same g(i) as attention.
 *
 *   in   [N, H, D]   (a weight matrix viewed as N rows of H heads, or
 *                     projected keys/values with N = tokens)
 *   out  [N, G, D]   fp64
 */
void oracle_mean_pool(const void *in, int dtype, int64_t N, int H, int G, int D, double *out)
{
    int64_t n;
#pragma omp parallel for schedule(static)
    for (n = 0; n < N; ++n) {
        for (int g = 0; g < G; ++g) {
            double *o = out + (n * G + g) * D;
            int members = 0;
            for (int d = 0; d < D; ++d)
                o[d] = 0.0;
            for (int i = 0; i < H; ++i) {
                if (oracle_group_of_head(i, H, G) != g)
                    continue;
                ++members;
                for (int d = 0; d < D; ++d)
                    o[d] += widen(in, (n * H + i) * D + d, dtype);
            }
            for (int d = 0; d < D; ++d)
                o[d] = o[d] / (double)members;
        }
    }
}

void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
