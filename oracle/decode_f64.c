/*
 * oracle/decode_f64.c -- plain fp64 CPU oracle for exact single-query attention decoding.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the slow, obviously correct definition the GPU
 * library is checked against.  Only the tests, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load it.  It includes no header of the product
 * library and the product library never links, includes or calls it.
 *
 * What it computes, for every batch row b, query head h and query token t of nq
 * (nq = 1 is single-token decode):
 *
 *   L    = seq_lens[b] clamped to [0, Lmax]           (Lmax when seq_lens is NULL)
 *   the nq query tokens are the row's last nq positions; token t sits at position
 *   L - nq + t and sees the keys up to it (causal among the new tokens), i.e. it is
 *   single-token decode over the first Lt = clamp(L - nq + t + 1, 0, L) keys:
 *   kh   = floor(h / (Hq / Hkv))                      (contiguous query-head groups)
 *   s_j  = d^(-1/2) * sum_i q[b,h,t,i] * k[b,kh,j,i] + beta_j,        0 <= j < Lt
 *   beta_j = -slope_h * (Lt - 1 - j)  with ALiBi slopes, else 0 (query position minus j)
 *   out[b,h,t,e] = sum_j exp(s_j - max_j s_j) v[b,kh,j,e] / sum_j exp(s_j - max_j s_j)
 *   Lt == 0 ->  out[b,h,t,:] = 0  (softmax over no keys is undefined; our convention)
 *
 * Sources:
 *   - "Tree Attention Decoding" (tree_attn_decode.py gist), function regular_decode:
 *     queries scaled by the inverse square root of the head dimension, dot products
 *     with every key, softmax over the keys, weighted sum of the value rows.
 *   - "ALiBi with causal=True unexpected bias?" (llm-foundry issue 186), the causal
 *     bias vector example: for the last query the bias of key j is -(L-1-j) times a
 *     per-head constant, added to the scaled scores.
 *   - "Flash Aandacht: Revolutie in Transformer Efficientie", section on the
 *     mathematics, softmax decomposition: subtracting the maximum score leaves the
 *     softmax unchanged (it only keeps exp() in range).
 *   - Several query tokens: the gist's einsum allows more than one query row (index i);
 *     the causal reading (each new token sees the cache up to its own position) is ours,
 *     the usual one for verifying several drafted tokens at once.
 *
 * FP8 keys and values (OCP E4M3 "fn" and E5M2 formats) carry dequantisation scales: one
 * per (batch row, KV head), or one per (batch row, KV head, block of `block` consecutive
 * key positions) -- key j uses block j / block.  The stored value times its scale is
 * the real value; the scores and the weighted sum use those real values.  (The pages
 * name FP8 attention only; both scale granularities are our reading.)
 *
 * All arithmetic is double precision on exactly widened inputs (bf16 -> fp32 -> fp64
 * and fp8 -> fp64 are exact).  Rows are independent, so rows are spread over POSIX threads; each row
 * is computed by one thread, in key order, with no blocking or reordering.
 * Every function here is pinned by the CPU tests (closed forms, invariants, a library
 * attention routine, the page's printed bias vector); nothing is "parity unpinned".
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_F32 0
#define OR_BF16 1
#define OR_FP8_E4M3 2
#define OR_FP8_E5M2 3

/* OCP FP8 E4M3 ("fn": no infinities, S.1111.111 is NaN): bias 7, 3 mantissa bits. */
double oracle_fp8_e4m3(uint8_t x)
{
    const int sign = x >> 7, e = (x >> 3) & 15, m = x & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m, -9);                 /* (m / 8) * 2^(1 - 7) */
    else v = ldexp(1.0 + m / 8.0, e - 7);
    return sign ? -v : v;
}

/* OCP FP8 E5M2: bias 15, 2 mantissa bits, IEEE-style infinities and NaNs. */
double oracle_fp8_e5m2(uint8_t x)
{
    const int sign = x >> 7, e = (x >> 2) & 31, m = x & 3;
    double v;
    if (e == 31) v = m ? NAN : INFINITY;
    else if (e == 0) v = ldexp((double)m, -16);           /* (m / 4) * 2^(1 - 15) */
    else v = ldexp(1.0 + m / 4.0, e - 15);
    return sign ? -v : v;
}

/* Widen one stored element to double.  bf16 is the upper half of an IEEE fp32. */
static double widen(const void *base, int dtype, int64_t idx)
{
    if (dtype == OR_F32)
        return (double)((const float *)base)[idx];
    if (dtype == OR_FP8_E4M3)
        return oracle_fp8_e4m3(((const uint8_t *)base)[idx]);
    if (dtype == OR_FP8_E5M2)
        return oracle_fp8_e5m2(((const uint8_t *)base)[idx]);
    uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* ALiBi bias of key j for a query at position L-1 ("ALiBi with causal=True" issue:
 * causal bias row arange(1-L, 1) times the head's slope). */
double oracle_alibi_bias(int64_t L, int64_t j, double slope)
{
    return -slope * (double)(L - 1 - j);
}

typedef struct {
    const void *q;
    int q_dtype;
    int64_t sqb, sqh, sqt;       /* q element strides for b, h, token (innermost stride 1) */
    int nq;                      /* query tokens per (b, h) */
    const void *k, *v;
    int kv_dtype;
    int64_t skb, skh, skj;       /* k element strides for b, kv-head, key */
    int64_t svb, svh, svj;       /* v element strides */
    int B, Hq, Hkv, Lmax, d;
    const int32_t *seq_lens;     /* [B] or NULL */
    const float *slopes;         /* [Hq] or NULL */
    const float *k_scale, *v_scale; /* dequantisation scales, or NULL (= 1): [B * Hkv] when the
                                       block is 0, else [B * Hkv * nblk] */
    int k_block, v_block;        /* keys per scale block, or 0 (one scale per (b, KV head)) */
    int64_t k_nblk, v_nblk;      /* scale blocks per (b, KV head) */
    const int32_t *rows;         /* flat (b*Hq+h)*nq+t indices to compute, or NULL for all */
    int n_rows;
    double *out;                 /* [n_rows, d] */
    int n_threads;
} oracle_job;

/* One (b, h, t) row of the definition above; s is scratch of length >= Lmax. */
static void decode_row(const oracle_job *J, int b, int h, int t, double *s, double *out)
{
    const int d = J->d;
    int64_t L = J->Lmax;
    if (J->seq_lens) {
        L = J->seq_lens[b];
        if (L < 0) L = 0;
        if (L > J->Lmax) L = J->Lmax;
    }
    L = L - J->nq + t + 1;               /* keys up to this token's own position */
    if (L < 0) L = 0;
    for (int e = 0; e < d; ++e) out[e] = 0.0;
    if (L == 0) return;

    const int kh = h / (J->Hq / J->Hkv);
    const double scale = 1.0 / sqrt((double)d);
    const int64_t bk = (int64_t)b * J->Hkv + kh;
    const double ks = (J->k_scale && !J->k_block) ? (double)J->k_scale[bk] : 1.0;
    const double vs = (J->v_scale && !J->v_block) ? (double)J->v_scale[bk] : 1.0;
    const int64_t qoff = (int64_t)b * J->sqb + (int64_t)h * J->sqh + (int64_t)t * J->sqt;
    const int64_t koff = (int64_t)b * J->skb + (int64_t)kh * J->skh;
    const int64_t voff = (int64_t)b * J->svb + (int64_t)kh * J->svh;

    /* scores s_j = (q . k_j) / sqrt(d) + beta_j */
    for (int64_t j = 0; j < L; ++j) {
        const double ksj = J->k_block ? (double)J->k_scale[bk * J->k_nblk + j / J->k_block] : ks;
        double dot = 0.0;
        for (int i = 0; i < d; ++i)
            dot += widen(J->q, J->q_dtype, qoff + i) * (ksj * widen(J->k, J->kv_dtype, koff + j * J->skj + i));
        s[j] = dot * scale;
        if (J->slopes) s[j] += oracle_alibi_bias(L, j, (double)J->slopes[h]);
    }
    /* softmax over the keys, with the maximum subtracted */
    double m = s[0];
    for (int64_t j = 1; j < L; ++j)
        if (s[j] > m) m = s[j];
    double z = 0.0;
    for (int64_t j = 0; j < L; ++j) {
        double w = exp(s[j] - m);
        const double vsj = J->v_block ? (double)J->v_scale[bk * J->v_nblk + j / J->v_block] : vs;
        z += w;
        for (int e = 0; e < d; ++e)
            out[e] += w * (vsj * widen(J->v, J->kv_dtype, voff + j * J->svj + e));
    }
    for (int e = 0; e < d; ++e) out[e] /= z;
}

typedef struct {
    const oracle_job *J;
    int tid;
    int fail;
} worker_arg;

static void *worker(void *p)
{
    worker_arg *a = (worker_arg *)p;
    const oracle_job *J = a->J;
    double *s = (double *)malloc(sizeof(double) * (size_t)(J->Lmax > 0 ? J->Lmax : 1));
    if (!s) { a->fail = 1; return NULL; }
    for (int r = a->tid; r < J->n_rows; r += J->n_threads) {
        int flat = J->rows ? J->rows[r] : r;
        int t = flat % J->nq, bh = flat / J->nq;
        int b = bh / J->Hq, h = bh % J->Hq;
        decode_row(J, b, h, t, s, J->out + (int64_t)r * J->d);
    }
    free(s);
    return NULL;
}

/*
 * Compute the decode output for the requested rows.
 *   q      : [B, Hq, nq, d] with element strides (sqb, sqh, sqt, 1); dtype OR_F32 or OR_BF16
 *   k, v   : [B, Hkv, Lmax, d] with element strides (s?b, s?h, s?j, 1); same dtype
 *            (OR_F32, OR_BF16, OR_FP8_E4M3, OR_FP8_E5M2)
 *   k_scale, v_scale: scales (real = stored * scale), or NULL: [B * Hkv] with block 0,
 *            else [B * Hkv * nblk], key j of (b, kv head kh) using entry
 *            (b * Hkv + kh) * nblk + j / block
 *   k_block, v_block: keys per scale block (0: one scale per (b, kv head))
 *   k_nblk, v_nblk: scale blocks per (b, kv head), at least ceil(Lmax / block)
 *   rows   : flat indices (b*Hq + h)*nq + t to compute (n_rows of them), or NULL for all
 *   out    : [n_rows, d] doubles, row r for rows[r]
 *   n_threads: POSIX threads to use (>= 1)
 * Returns 0, or -1 on bad arguments / allocation failure.
 */
int oracle_decode_f64(const void *q, int q_dtype, int64_t sqb, int64_t sqh, int64_t sqt, int nq,
                      const void *k, const void *v, int kv_dtype,
                      int64_t skb, int64_t skh, int64_t skj,
                      int64_t svb, int64_t svh, int64_t svj,
                      int B, int Hq, int Hkv, int Lmax, int d,
                      const int32_t *seq_lens, const float *slopes,
                      const float *k_scale, const float *v_scale,
                      int k_block, int64_t k_nblk, int v_block, int64_t v_nblk,
                      const int32_t *rows, int n_rows, double *out, int n_threads)
{
    if (!q || !k || !v || !out || B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || Lmax < 0 || d <= 0 || nq < 1)
        return -1;
    if ((q_dtype != OR_F32 && q_dtype != OR_BF16) || kv_dtype < OR_F32 || kv_dtype > OR_FP8_E5M2)
        return -1;
    if (k_block < 0 || v_block < 0) return -1;
    if (k_block && (!k_scale || k_nblk * k_block < (int64_t)Lmax)) return -1;
    if (v_block && (!v_scale || v_nblk * v_block < (int64_t)Lmax)) return -1;
    oracle_job J = {q, q_dtype, sqb, sqh, sqt, nq, k, v, kv_dtype, skb, skh, skj, svb, svh, svj,
                    B, Hq, Hkv, Lmax, d, seq_lens, slopes, k_scale, v_scale,
                    k_block, v_block, k_nblk, v_nblk,
                    rows, rows ? n_rows : B * Hq * nq, out, n_threads < 1 ? 1 : n_threads};
    for (int r = 0; rows && r < n_rows; ++r)
        if (rows[r] < 0 || rows[r] >= B * Hq * nq) return -1;
    if (J.n_threads > J.n_rows) J.n_threads = J.n_rows > 0 ? J.n_rows : 1;

    pthread_t th[256];
    worker_arg args[256];
    if (J.n_threads > 256) J.n_threads = 256;
    int rc = 0;
    int started[256];
    for (int t = 0; t < J.n_threads; ++t) {
        args[t].J = &J; args[t].tid = t; args[t].fail = 0;
        started[t] = pthread_create(&th[t], NULL, worker, &args[t]) == 0;
        if (!started[t]) worker(&args[t]);   /* no thread: do this share here */
    }
    for (int t = 0; t < J.n_threads; ++t) {
        if (started[t]) pthread_join(th[t], NULL);
        if (args[t].fail) rc = -1;
    }
    return rc;
}
