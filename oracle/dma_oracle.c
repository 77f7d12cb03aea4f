/*
 * CPU oracle for the forward hot path of Doge's Dynamic Mask Attention (DMA).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  The product path
 * (the HIP library and its Python binding) never links, loads or calls it, and
 * this file shares no code, header or table with the HIP kernels.
 *
 * Source of every step: the gitcode blog page "Transformers 中的 Doge 小语言模型
 * 完全指南：动态掩码注意力（DMA）与跨域 MoE（CDMoE）架构解析与实战" (called "the
 * Doge guide" below), section "动态掩码注意力（DMA）：从缓存 value states 生成稀疏掩码"
 * (forward chain, steps 3 and 4), and the DogeConfig parameter table in section
 * "DogeConfig 全参数详解" (keep_window_size, num_key_value_heads).
 *
 * Everything is plain and slow on purpose: fp64 arithmetic on the exact stored
 * input values, one qsort per query row for the top-w selection, no blocking,
 * no fusion, no reuse between rows.  OpenMP only splits independent rows over
 * host threads.
 *
 * Pins (checked by the CPU tests): the dt closed forms (W = 0 gives 2^A, A = 0
 * gives 1, the softplus identity softplus(x) - softplus(-x) = x, one-hot V
 * reads exactly one weight, inversion back to the projection), a literal NumPy
 * brute force of the masked-softmax procedure on tiny shapes, the library SDPA
 * routine when no row has more than w valid keys, and the selection
 * invariants.  Every function below has at least one such pin.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_F32 0
#define ORACLE_BF16 1

/* Read element i of a float32 or bfloat16 array as an exact double. */
static double elem(const void *p, int dtype, size_t i)
{
    if (dtype == ORACLE_F32)
        return (double)((const float *)p)[i];
    uint32_t u = (uint32_t)((const uint16_t *)p)[i] << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* softplus(x) = log(1 + e^x), written so that neither branch overflows. */
static double softplus(double x)
{
    if (x > 0.0)
        return x + log1p(exp(-x));
    return log1p(exp(x));
}

/*
 * dt for every (batch, kv head, position) -- Doge guide, DMA forward step 3:
 * dt_proj maps the value states to num_key_value_heads scores, then
 * dt = exp(A * softplus(dt_proj(V))).  dt_proj reads the value states of all
 * kv heads of one token, concatenated head-major (input width Hkv*d), and has
 * one output per kv head; bias is optional (attention_bias defaults to False).
 *
 *   V    [B][S][Hkv][d]   (dtype)
 *   W    [Hkv][Hkv*d]     (dtype)
 *   bias [Hkv] or NULL    (dtype)
 *   A    [Hkv]            float32
 *   out  [B][Hkv][S]      double
 */
void oracle_dt(const void *V, const void *W, const void *bias, const float *A,
               int dtype, int B, int S, int Hkv, int d, double *out)
{
    const size_t width = (size_t)Hkv * d;
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < B; ++b)
        for (int s = 0; s < S; ++s) {
            const size_t vrow = ((size_t)b * S + s) * width;
            for (int h = 0; h < Hkv; ++h) {
                double x = bias ? elem(bias, dtype, h) : 0.0;
                for (size_t c = 0; c < width; ++c)
                    x += elem(W, dtype, (size_t)h * width + c) * elem(V, dtype, vrow + c);
                out[((size_t)b * Hkv + h) * S + s] = exp((double)A[h] * softplus(x));
            }
        }
}

/* One key of a query row: its dt (compared as a real number) and its index. */
typedef struct {
    float dt;
    int32_t idx;
} key_t_;

/*
 * Order of the top-w selection: larger dt first; among equal dt the lower key
 * index first.  The Doge guide selects with torch.topk, whose order among
 * equal scores is unspecified; the lower-index rule makes the kept set unique.
 */
static int better_first(const void *pa, const void *pb)
{
    const key_t_ *a = (const key_t_ *)pa, *b = (const key_t_ *)pb;
    if (a->dt > b->dt)
        return -1;
    if (a->dt < b->dt)
        return 1;
    return (a->idx > b->idx) - (a->idx < b->idx);
}

/*
 * First key visible to row i: 0 for the full causal mask, i - win + 1 (at
 * least 0) under a sliding window of win positions (DogeConfig's
 * sliding_window: with a value, the attention mask is the sliding-window
 * causal mask, under which row i sees the keys i - win < j <= i).
 */
static int first_visible(int i, int win)
{
    return (win > 0 && i - win + 1 > 0) ? i - win + 1 : 0;
}

/*
 * Keys of query row i, in selection order, into buf (capacity >= i + 1).
 * Valid keys are first_visible(i, win) <= j <= i (causal mask, and the
 * sliding window when win > 0) and j < L (right padding).  Returns how many
 * of them the row keeps: all valid keys if there are at most w of them, else
 * the first w in the order above (Doge guide, DMA forward step 3: the
 * masked positions hold min_dtype before the top-k, so a masked key never
 * outranks a valid one; the top-k branch keeps keep_window_size positions
 * and masks the rest).
 */
static int row_kept(const float *dt_row, int i, int L, int w, int win, key_t_ *buf)
{
    const int lo = first_visible(i, win);
    const int hi = (i + 1 < L) ? i + 1 : L;
    int n = 0;
    for (int j = lo; j < hi; ++j) {
        buf[n].dt = dt_row[j];
        buf[n].idx = j;
        ++n;
    }
    qsort(buf, (size_t)n, sizeof *buf, better_first);
    return n < w ? n : w;
}

/*
 * Threshold pair (tau_i, t_i) of each query row: the dt and index of the
 * last (w-th) kept key.  A key j of row i is kept exactly when it is valid and
 * (dt_j > tau_i, or dt_j == tau_i and j <= t_i).  Canonical forms: a row with
 * at most w valid keys keeps them all and gets (-inf, -1); a padded row
 * (i >= L) keeps nothing and gets (+inf, -1).  win > 0: sliding window of win
 * positions (win <= 0: full causal).
 *
 *   dt      [B][Hkv][S] float32
 *   seqlens [B] int32 or NULL (then every batch has length S)
 *   rows    list of nrows (b, g, i) triples, or NULL for every row
 *   tau/tie one entry per requested row ([B][Hkv][S] when rows == NULL)
 */
void oracle_select(const float *dt, const int32_t *seqlens, int B, int Hkv, int S, int w, int win,
                   const int32_t *rows, int64_t nrows, float *tau, int32_t *tie)
{
    const int64_t total = rows ? nrows : (int64_t)B * Hkv * S;
#pragma omp parallel
    {
        key_t_ *buf = (key_t_ *)malloc(sizeof(key_t_) * (size_t)(S > 0 ? S : 1));
#pragma omp for schedule(dynamic, 16)
        for (int64_t r = 0; r < total; ++r) {
            int b, g, i;
            if (rows) {
                b = rows[3 * r];
                g = rows[3 * r + 1];
                i = rows[3 * r + 2];
            } else {
                b = (int)(r / ((int64_t)Hkv * S));
                g = (int)((r / S) % Hkv);
                i = (int)(r % S);
            }
            const int L = seqlens ? seqlens[b] : S;
            if (i >= L) {
                tau[r] = INFINITY;
                tie[r] = -1;
                continue;
            }
            if (i + 1 - first_visible(i, win) <= w) {
                tau[r] = -INFINITY;
                tie[r] = -1;
                continue;
            }
            int nk = row_kept(dt + ((size_t)b * Hkv + g) * S, i, L, w, win, buf);
            tau[r] = buf[nk - 1].dt;
            tie[r] = buf[nk - 1].idx;
        }
        free(buf);
    }
}

/*
 * Kept key indices of one query row, ascending, into out (capacity >= w).
 * Returns their count.  Used by the tests to materialise kept sets.
 */
int oracle_kept_row(const float *dt, const int32_t *seqlens, int Hkv, int S, int w, int win,
                    int b, int g, int i, int32_t *out)
{
    const int L = seqlens ? seqlens[b] : S;
    if (i >= L)
        return 0;
    key_t_ *buf = (key_t_ *)malloc(sizeof(key_t_) * (size_t)(i + 1));
    int nk = row_kept(dt + ((size_t)b * Hkv + g) * S, i, L, w, win, buf);
    /* report in index order */
    int n = 0;
    char *mark = (char *)calloc((size_t)i + 1, 1);
    for (int k = 0; k < nk; ++k)
        mark[buf[k].idx] = 1;
    for (int j = 0; j <= i; ++j)
        if (mark[j])
            out[n++] = j;
    free(mark);
    free(buf);
    return n;
}

/*
 * Attention of one query vector over an explicit kept set -- Doge guide, DMA
 * forward step 4: scores are scaled by head_dim**-0.5, the dt of each key is
 * the additive mask value at kept positions (masked positions hold min_dtype
 * and so contribute exactly zero weight), and the softmax is taken in full
 * precision: o = sum_j p_j v_j / sum_j p_j with p_j = exp(s_j - max s).
 *
 *   q    d values at q (dtype), k/v base pointers with row stride kv_stride
 *   keys nk kept key indices (nk >= 1), dtv the dt of each position
 */
static void attend(const void *q, size_t qoff, const void *K, const void *Vv, int dtype,
                   size_t kv_base, size_t kv_stride, int d, const float *dtv,
                   const key_t_ *keys, int nk, double *s_buf, double *o)
{
    const double scale = 1.0 / sqrt((double)d);
    double m = -INFINITY;
    for (int k = 0; k < nk; ++k) {
        const size_t kr = kv_base + (size_t)keys[k].idx * kv_stride;
        double dot = 0.0;
        for (int e = 0; e < d; ++e)
            dot += elem(q, dtype, qoff + e) * elem(K, dtype, kr + e);
        s_buf[k] = scale * dot + (double)dtv[keys[k].idx];
        if (s_buf[k] > m)
            m = s_buf[k];
    }
    double l = 0.0;
    for (int e = 0; e < d; ++e)
        o[e] = 0.0;
    for (int k = 0; k < nk; ++k) {
        const double p = exp(s_buf[k] - m);
        l += p;
        const size_t vr = kv_base + (size_t)keys[k].idx * kv_stride;
        for (int e = 0; e < d; ++e)
            o[e] += p * elem(Vv, dtype, vr + e);
    }
    for (int e = 0; e < d; ++e)
        o[e] /= l;
}

/*
 * Prefill attention with the dynamic mask, for all rows or for a list of
 * (b, g, i) rows (each list entry produces the G query heads of kv head g).
 * Query head hq uses kv head hq / G (contiguous groups, G = Hq / Hkv).  Padded
 * rows (i >= L) produce zeros.  win > 0: sliding window of win positions.
 *
 *   Q [B][S][Hq][d], K/V [B][S][Hkv][d] (dtype); dt [B][Hkv][S] float32
 *   out: [B][S][Hq][d] double when rows == NULL, else [nrows][G][d]
 */
void oracle_attn(const void *Q, const void *K, const void *V, int dtype, const float *dt,
                 const int32_t *seqlens, int B, int S, int Hq, int Hkv, int d, int w, int win,
                 const int32_t *rows, int64_t nrows, double *out)
{
    const int G = Hq / Hkv;
    const int64_t total = rows ? nrows : (int64_t)B * Hkv * S;
#pragma omp parallel
    {
        key_t_ *buf = (key_t_ *)malloc(sizeof(key_t_) * (size_t)(S > 0 ? S : 1));
        double *s_buf = (double *)malloc(sizeof(double) * (size_t)(S > 0 ? S : 1));
#pragma omp for schedule(dynamic, 8)
        for (int64_t r = 0; r < total; ++r) {
            int b, g, i;
            if (rows) {
                b = rows[3 * r];
                g = rows[3 * r + 1];
                i = rows[3 * r + 2];
            } else {
                b = (int)(r / ((int64_t)Hkv * S));
                g = (int)((r / S) % Hkv);
                i = (int)(r % S);
            }
            const int L = seqlens ? seqlens[b] : S;
            for (int hh = 0; hh < G; ++hh) {
                const int hq = g * G + hh;
                double *o = rows ? out + ((size_t)r * G + hh) * d
                                 : out + (((size_t)b * S + i) * Hq + hq) * d;
                if (i >= L) {
                    for (int e = 0; e < d; ++e)
                        o[e] = 0.0;
                    continue;
                }
                int nk = row_kept(dt + ((size_t)b * Hkv + g) * S, i, L, w, win, buf);
                attend(Q, (((size_t)b * S + i) * Hq + hq) * d, K, V, dtype,
                       ((size_t)b * S * Hkv + g) * d, (size_t)Hkv * d, d,
                       dt + ((size_t)b * Hkv + g) * S, buf, nk, s_buf, o);
            }
        }
        free(s_buf);
        free(buf);
    }
}

/*
 * One decode step per batch over a KV cache: the query sits at position
 * L_b - 1 and sees every cached position j < L_b; it keeps the top w of them
 * by dt (all if L_b <= w), read from the dt cache -- dt is a function of each
 * position's cached value state, so caching it per position equals
 * re-projecting every cached value (Doge guide, DMA forward step 3, remark
 * that dt comes from the cached value states).
 *
 *   q [B][Hq][d]; Kc/Vc [B][Lmax][Hkv][d] (dtype); dt_cache [B][Hkv][Lmax]
 *   cache_lens [B] in [1, Lmax]
 *   out [B][Hq][d] double; kept_idx [B][Hkv][w] int32 ascending, -1 padded
 *   (kept_idx may be NULL)
 */
void oracle_decode(const void *q, const void *Kc, const void *Vc, int dtype,
                   const float *dt_cache, const int32_t *cache_lens, int B, int Lmax,
                   int Hq, int Hkv, int d, int w, double *out, int32_t *kept_idx)
{
    const int G = Hq / Hkv;
#pragma omp parallel
    {
        key_t_ *buf = (key_t_ *)malloc(sizeof(key_t_) * (size_t)(Lmax > 0 ? Lmax : 1));
        double *s_buf = (double *)malloc(sizeof(double) * (size_t)(Lmax > 0 ? Lmax : 1));
#pragma omp for collapse(2) schedule(dynamic, 1)
        for (int b = 0; b < B; ++b)
            for (int g = 0; g < Hkv; ++g) {
                const int L = cache_lens[b];
                const float *drow = dt_cache + ((size_t)b * Hkv + g) * Lmax;
                int nk = row_kept(drow, L - 1, L, w, 0, buf);
                if (kept_idx) {
                    int32_t *ki = kept_idx + ((size_t)b * Hkv + g) * w;
                    char *mark = (char *)calloc((size_t)(L > 0 ? L : 1), 1);
                    for (int k = 0; k < nk; ++k)
                        mark[buf[k].idx] = 1;
                    int n = 0;
                    for (int j = 0; j < L; ++j)
                        if (mark[j])
                            ki[n++] = j;
                    for (; n < w; ++n)
                        ki[n] = -1;
                    free(mark);
                }
                for (int hh = 0; hh < G; ++hh) {
                    const int hq = g * G + hh;
                    attend(q, ((size_t)b * Hq + hq) * d, Kc, Vc, dtype,
                           ((size_t)b * Lmax * Hkv + g) * d, (size_t)Hkv * d, d, drow, buf,
                           nk, s_buf, out + ((size_t)b * Hq + hq) * d);
                }
            }
        free(s_buf);
        free(buf);
    }
}

/*
 * Q/K normalisation and rotary position embedding -- Doge guide, DMA forward
 * step 1: after q_proj/k_proj, Q and K go through q_norm/k_norm, an RMSNorm
 * over head_dim with one learnable weight per element (the T5 layer norm of
 * the Llama code it reuses; eps = rms_norm_eps), and then the rotary position
 * embedding reused from Llama.  Reading of the rotary step (the guide names
 * it only): element e < d/2 pairs with e + d/2, the pair turns by the angle
 * pos * theta^(-2e/d):
 *   out_e       = y_e cos(a) - y_{e+d/2} sin(a)
 *   out_{e+d/2} = y_{e+d/2} cos(a) + y_e sin(a)
 * x: nrows rows of d elements (dtype), row r at position pos[r]; w: d
 * weights (dtype); out: fp64, nrows x d.
 */
void oracle_qk_norm_rope(const void *x, const void *w, int dtype, double eps, double theta,
                         const int32_t *pos, int64_t nrows, int d, double *out)
{
    const int h = d / 2;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < nrows; ++r) {
        double ss = 0.0;
        for (int e = 0; e < d; ++e) {
            const double v = elem(x, dtype, (size_t)r * d + e);
            ss += v * v;
        }
        const double inv = 1.0 / sqrt(ss / d + eps);
        for (int e = 0; e < h; ++e) {
            const double a = (double)pos[r] * pow(theta, -2.0 * e / d);
            const double y0 = elem(x, dtype, (size_t)r * d + e) * inv * elem(w, dtype, e);
            const double y1 = elem(x, dtype, (size_t)r * d + e + h) * inv * elem(w, dtype, e + h);
            out[(size_t)r * d + e] = y0 * cos(a) - y1 * sin(a);
            out[(size_t)r * d + e + h] = y1 * cos(a) + y0 * sin(a);
        }
    }
}

/*
 * Gradients of the prefill attention (oracle_attn) with respect to Q, K, V and
 * dt, for an upstream gradient dO of the output.  The kept sets are those of
 * the forward (the top-w selection itself is piecewise constant in dt and has
 * no gradient; every kept key's dt enters its score additively, Doge guide,
 * DMA forward steps 3 and 4).  With s_k = c q.k_k + dt_k (c = d^-0.5) over the
 * kept keys k of a query row, p = softmax(s), o = sum_k p_k v_k:
 *   dp_k = dO . v_k,  ds_k = p_k (dp_k - dO . o)
 *   dq  = c sum_k ds_k k_k
 *   dk_k += c ds_k q,  dv_k += p_k dO,  ddt_k += ds_k
 * summed over every query row and query head that keeps key k.  Padded rows
 * contribute nothing.
 *
 *   dO [B][S][Hq][d] (dtype, like Q)
 *   dQ [B][S][Hq][d], dK/dV [B][S][Hkv][d], ddt [B][Hkv][S]: double (out)
 * Units (b, kv head) are independent and split over threads; within a unit
 * the rows run in order.
 */
void oracle_attn_bwd(const void *Q, const void *K, const void *V, int dtype, const float *dt,
                     const int32_t *seqlens, const void *dO, int B, int S, int Hq, int Hkv, int d, int w,
                     double *dQ, double *dK, double *dV, double *ddt)
{
    const int G = Hq / Hkv;
    const double c = 1.0 / sqrt((double)d);
    const size_t kvs = (size_t)Hkv * d;
#pragma omp parallel
    {
        key_t_ *buf = (key_t_ *)malloc(sizeof(key_t_) * (size_t)(S > 0 ? S : 1));
        double *s = (double *)malloc(sizeof(double) * (size_t)(S > 0 ? S : 1));
        double *dp = (double *)malloc(sizeof(double) * (size_t)(S > 0 ? S : 1));
        double *o = (double *)malloc(sizeof(double) * (size_t)d);
#pragma omp for collapse(2) schedule(dynamic, 1)
        for (int b = 0; b < B; ++b)
            for (int g = 0; g < Hkv; ++g) {
                const int L = seqlens ? seqlens[b] : S;
                const float *drow = dt + ((size_t)b * Hkv + g) * S;
                double *ddt_row = ddt + ((size_t)b * Hkv + g) * S;
                for (int j = 0; j < S; ++j) {
                    ddt_row[j] = 0.0;
                    for (int e = 0; e < d; ++e) {
                        dK[((size_t)b * S + j) * kvs + (size_t)g * d + e] = 0.0;
                        dV[((size_t)b * S + j) * kvs + (size_t)g * d + e] = 0.0;
                    }
                }
                for (int i = 0; i < S; ++i)
                    for (int hh = 0; hh < G; ++hh) {
                        const int hq = g * G + hh;
                        const size_t qo = (((size_t)b * S + i) * Hq + hq) * d;
                        double *dq = dQ + qo;
                        for (int e = 0; e < d; ++e)
                            dq[e] = 0.0;
                        if (i >= L)
                            continue;
                        const int nk = row_kept(drow, i, L, w, 0, buf);
                        /* forward: scores, softmax, output */
                        double m = -INFINITY;
                        for (int k = 0; k < nk; ++k) {
                            const size_t kr = ((size_t)b * S + buf[k].idx) * kvs + (size_t)g * d;
                            double dot = 0.0;
                            for (int e = 0; e < d; ++e)
                                dot += elem(Q, dtype, qo + e) * elem(K, dtype, kr + e);
                            s[k] = c * dot + (double)drow[buf[k].idx];
                            if (s[k] > m)
                                m = s[k];
                        }
                        double l = 0.0;
                        for (int k = 0; k < nk; ++k) {
                            s[k] = exp(s[k] - m);
                            l += s[k];
                        }
                        for (int e = 0; e < d; ++e)
                            o[e] = 0.0;
                        for (int k = 0; k < nk; ++k) {
                            s[k] /= l; /* s now holds p */
                            const size_t vr = ((size_t)b * S + buf[k].idx) * kvs + (size_t)g * d;
                            for (int e = 0; e < d; ++e)
                                o[e] += s[k] * elem(V, dtype, vr + e);
                        }
                        /* backward */
                        double dod = 0.0;
                        for (int e = 0; e < d; ++e)
                            dod += elem(dO, dtype, qo + e) * o[e];
                        for (int k = 0; k < nk; ++k) {
                            const size_t vr = ((size_t)b * S + buf[k].idx) * kvs + (size_t)g * d;
                            double t = 0.0;
                            for (int e = 0; e < d; ++e)
                                t += elem(dO, dtype, qo + e) * elem(V, dtype, vr + e);
                            dp[k] = s[k] * (t - dod); /* ds_k */
                        }
                        for (int k = 0; k < nk; ++k) {
                            const int j = buf[k].idx;
                            const size_t kr = ((size_t)b * S + j) * kvs + (size_t)g * d;
                            for (int e = 0; e < d; ++e) {
                                dq[e] += c * dp[k] * elem(K, dtype, kr + e);
                                dK[kr + e] += c * dp[k] * elem(Q, dtype, qo + e);
                                dV[kr + e] += s[k] * elem(dO, dtype, qo + e);
                            }
                            ddt_row[j] += dp[k];
                        }
                    }
            }
        free(o);
        free(dp);
        free(s);
        free(buf);
    }
}

/*
 * Gradients of dt (oracle_dt) for an upstream gradient ddt: with
 * x = bias + W . concat_h V (per token and kv head), dt = exp(A softplus(x)),
 *   ddt/dA = dt softplus(x),  ddt/dx = dt A sigmoid(x)
 * so dx = ddt dt A sigmoid(x) and
 *   dA[h] = sum ddt dt softplus(x),  dbias[h] = sum dx,
 *   dW[h][c] = sum dx[h] V[c],       dV[c] += sum_h dx[h] W[h][c]
 * (sums over batches and positions).  Doge guide, DMA forward step 3.
 *
 *   ddt [B][Hkv][S] double
 *   dV [B][S][Hkv][d] double (out, the dt path's part only), dW [Hkv][Hkv*d],
 *   dbias [Hkv], dA [Hkv] double (out)
 */
void oracle_dt_bwd(const void *V, const void *W, const void *bias, const float *A, int dtype,
                   int B, int S, int Hkv, int d, const double *ddt,
                   double *dV, double *dW, double *dbias, double *dA)
{
    const int width = Hkv * d;
    double *dx = (double *)malloc(sizeof(double) * (size_t)B * S * Hkv);
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < B; ++b)
        for (int s = 0; s < S; ++s) {
            const size_t vrow = ((size_t)b * S + s) * width;
            for (int h = 0; h < Hkv; ++h) {
                double x = bias ? elem(bias, dtype, h) : 0.0;
                for (int c = 0; c < width; ++c)
                    x += elem(W, dtype, (size_t)h * width + c) * elem(V, dtype, vrow + c);
                const double a = (double)A[h];
                const double dtv = exp(a * softplus(x));
                const double sig = 1.0 / (1.0 + exp(-x));
                const double g = ddt[((size_t)b * Hkv + h) * S + s];
                dx[((size_t)b * S + s) * Hkv + h] = g * dtv * a * sig;
            }
            for (int c = 0; c < width; ++c) {
                double acc = 0.0;
                for (int h = 0; h < Hkv; ++h)
                    acc += dx[((size_t)b * S + s) * Hkv + h] * elem(W, dtype, (size_t)h * width + c);
                dV[vrow + c] = acc;
            }
        }
    for (int h = 0; h < Hkv; ++h) {
        double sa = 0.0, sb = 0.0;
        for (int b = 0; b < B; ++b)
            for (int s = 0; s < S; ++s) {
                const size_t vrow = ((size_t)b * S + s) * width;
                double x = bias ? elem(bias, dtype, h) : 0.0;
                for (int c = 0; c < width; ++c)
                    x += elem(W, dtype, (size_t)h * width + c) * elem(V, dtype, vrow + c);
                const double sp = softplus(x);
                sa += ddt[((size_t)b * Hkv + h) * S + s] * exp((double)A[h] * sp) * sp;
                sb += dx[((size_t)b * S + s) * Hkv + h];
            }
        dA[h] = sa;
        dbias[h] = sb;
    }
#pragma omp parallel for schedule(static)
    for (int hc = 0; hc < Hkv * width; ++hc) {
        const int h = hc / width, c = hc % width;
        double acc = 0.0;
        for (int b = 0; b < B; ++b)
            for (int s = 0; s < S; ++s)
                acc += dx[((size_t)b * S + s) * Hkv + h] * elem(V, dtype, ((size_t)b * S + s) * width + c);
        dW[hc] = acc;
    }
    free(dx);
}

/*
 * Cross Domain MoE (CDMoE) routed experts -- Doge guide, section on CDMoE and
 * the DogeConfig table (num_experts, num_experts_per_tok, hidden_act).  Per
 * token with hidden state h (length H):
 *   logits = router_gate h, 2*nk values: the first nk are the x domain, the
 *            last nk the y domain (nk = floor(sqrt(num_experts)));
 *   the top k of each domain (larger first, lower index first among equal),
 *            a and b being the ranks in the two lists;
 *   every pair (a, b) of the two lists scores sx_a + sy_b and names expert
 *            ix_a * nk + iy_b; the token keeps the top k pairs (larger score
 *            first; among equal scores the lower a, then the lower b: the
 *            order of the two domains' own rankings);
 *   weights = softmax over the k kept scores;
 *   out = sum over kept experts e of weight_e * silu(down_e . h) * up_e.
 * Plain loops and qsort, fp64 on the stored values.
 *
 *   h [T][H], router [2*nk][H], down/up [nk*nk][H] (dtype)
 *   idx [T][k] int32 (out, in selection order), wts [T][k] double (out),
 *   out [T][H] double (out)
 */
typedef struct {
    double v;
    int32_t tb;  /* tie order: lower first */
    int32_t idx;
} score_t_;

static int score_first(const void *pa, const void *pb)
{
    const score_t_ *a = (const score_t_ *)pa, *b = (const score_t_ *)pb;
    if (a->v > b->v)
        return -1;
    if (a->v < b->v)
        return 1;
    return (a->tb > b->tb) - (a->tb < b->tb);
}

void oracle_cdmoe(const void *h, const void *router, const void *down, const void *up, int dtype, int T, int H,
                  int nk, int k, int32_t *idx, double *wts, double *out)
{
#pragma omp parallel
    {
        score_t_ *sx = (score_t_ *)malloc(sizeof(score_t_) * (size_t)nk);
        score_t_ *sy = (score_t_ *)malloc(sizeof(score_t_) * (size_t)nk);
        score_t_ *pairs = (score_t_ *)malloc(sizeof(score_t_) * (size_t)k * k);
#pragma omp for schedule(dynamic, 4)
        for (int t = 0; t < T; ++t) {
            const size_t hr = (size_t)t * H;
            for (int n = 0; n < 2 * nk; ++n) {
                double acc = 0.0;
                for (int c = 0; c < H; ++c)
                    acc += elem(router, dtype, (size_t)n * H + c) * elem(h, dtype, hr + c);
                score_t_ *dst = n < nk ? &sx[n] : &sy[n - nk];
                dst->v = acc;
                dst->idx = dst->tb = n < nk ? n : n - nk;
            }
            qsort(sx, (size_t)nk, sizeof *sx, score_first);
            qsort(sy, (size_t)nk, sizeof *sy, score_first);
            for (int a = 0; a < k; ++a)
                for (int b = 0; b < k; ++b) {
                    pairs[a * k + b].v = sx[a].v + sy[b].v;
                    pairs[a * k + b].tb = a * k + b;
                    pairs[a * k + b].idx = sx[a].idx * nk + sy[b].idx;
                }
            qsort(pairs, (size_t)k * k, sizeof *pairs, score_first);
            double m = pairs[0].v, l = 0.0;
            for (int e = 0; e < k; ++e)
                l += exp(pairs[e].v - m);
            for (int c = 0; c < H; ++c)
                out[hr + c] = 0.0;
            for (int e = 0; e < k; ++e) {
                const int x = pairs[e].idx;
                const double wgt = exp(pairs[e].v - m) / l;
                idx[(size_t)t * k + e] = x;
                wts[(size_t)t * k + e] = wgt;
                double z = 0.0;
                for (int c = 0; c < H; ++c)
                    z += elem(down, dtype, (size_t)x * H + c) * elem(h, dtype, hr + c);
                const double act = z / (1.0 + exp(-z));
                for (int c = 0; c < H; ++c)
                    out[hr + c] += wgt * act * elem(up, dtype, (size_t)x * H + c);
            }
        }
        free(pairs);
        free(sy);
        free(sx);
    }
}

/*
 * The routing step alone, from given router logits (float32 [T][2*nk]): the
 * kept experts in selection order and their weights, as oracle_cdmoe, except
 * that a pair's score is the float32 sum of its two float32 logits (the pages
 * fix no precision; the HIP kernel ranks pairs on that float32 sum, and a
 * ranking decided by floating point is taken in the kernel's precision).
 */
void oracle_cdmoe_route(const float *logits, int T, int nk, int k, int32_t *idx, double *wts)
{
#pragma omp parallel
    {
        score_t_ *sx = (score_t_ *)malloc(sizeof(score_t_) * (size_t)nk);
        score_t_ *sy = (score_t_ *)malloc(sizeof(score_t_) * (size_t)nk);
        score_t_ *pairs = (score_t_ *)malloc(sizeof(score_t_) * (size_t)k * k);
#pragma omp for schedule(static)
        for (int t = 0; t < T; ++t) {
            for (int n = 0; n < nk; ++n) {
                sx[n].v = logits[(size_t)t * 2 * nk + n];
                sx[n].idx = sx[n].tb = n;
                sy[n].v = logits[(size_t)t * 2 * nk + nk + n];
                sy[n].idx = sy[n].tb = n;
            }
            qsort(sx, (size_t)nk, sizeof *sx, score_first);
            qsort(sy, (size_t)nk, sizeof *sy, score_first);
            for (int a = 0; a < k; ++a)
                for (int b = 0; b < k; ++b) {
                    pairs[a * k + b].v = (double)((float)sx[a].v + (float)sy[b].v);
                    pairs[a * k + b].tb = a * k + b;
                    pairs[a * k + b].idx = sx[a].idx * nk + sy[b].idx;
                }
            qsort(pairs, (size_t)k * k, sizeof *pairs, score_first);
            double m = pairs[0].v, l = 0.0;
            for (int e = 0; e < k; ++e)
                l += exp(pairs[e].v - m);
            for (int e = 0; e < k; ++e) {
                idx[(size_t)t * k + e] = pairs[e].idx;
                wts[(size_t)t * k + e] = exp(pairs[e].v - m) / l;
            }
        }
        free(pairs);
        free(sy);
        free(sx);
    }
}

/* The router logits alone (as in oracle_cdmoe): logits [T][2*nk] double. */
void oracle_cdmoe_logits(const void *h, const void *router, int dtype, int T, int H, int nk, double *logits)
{
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t)
        for (int n = 0; n < 2 * nk; ++n) {
            double acc = 0.0;
            for (int c = 0; c < H; ++c)
                acc += elem(router, dtype, (size_t)n * H + c) * elem(h, dtype, (size_t)t * H + c);
            logits[(size_t)t * 2 * nk + n] = acc;
        }
}

/*
 * The experts alone, for given kept experts and weights (as in oracle_cdmoe):
 * out[t] = sum_e wts[t][e] * silu(down[idx[t][e]] . h[t]) * up[idx[t][e]].
 */
void oracle_cdmoe_experts(const void *h, const void *down, const void *up, int dtype, const int32_t *idx,
                          const double *wts, int T, int H, int k, double *out)
{
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        const size_t hr = (size_t)t * H;
        for (int c = 0; c < H; ++c)
            out[hr + c] = 0.0;
        for (int e = 0; e < k; ++e) {
            const size_t er = (size_t)idx[(size_t)t * k + e] * H;
            double z = 0.0;
            for (int c = 0; c < H; ++c)
                z += elem(down, dtype, er + c) * elem(h, dtype, hr + c);
            const double a = wts[(size_t)t * k + e] * z / (1.0 + exp(-z));
            for (int c = 0; c < H; ++c)
                out[hr + c] += a * elem(up, dtype, er + c);
        }
    }
}
