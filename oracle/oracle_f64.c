/*
 * oracle_f64.c -- plain fp64 CPU reference for DFlash block attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  It shares no code,
 * header, table or helper with the HIP path.
 *
 * What it computes (exact softmax attention over a per-query visible key set):
 *
 *   Each request r has a context of L = ctx_lens[r] keys and a block of
 *   n = block_lens[r] queries ("1 + num_speculative_tokens": kenforever1,
 *   "DFlash + Gemma 4 31B-it" notes, section "why non-causal attention is
 *   needed").  The block's own K/V sit at key positions L..L+n-1, so the
 *   request has T = L + n keys; query i of the block sits at position p = L+i.
 *
 *   Visible keys of query i (same section; vLLM PR #43445 report, "key code"):
 *     non-causal (the default): every key 0..T-1 -- the block is handled as a
 *       whole, with no left-to-right restriction;
 *     causal: a query sees itself and what lies to its left, keys 0..p;
 *     sliding window W > 0: additionally only keys j >= p - W + 1, i.e. the W
 *       keys ending at the query's position (the window bounds only the low
 *       side; for a non-causal request the high end stays T-1).
 *
 *   Bidirectional spans (optional).  The same notes, section "what
 *   MooreThreads/vllm-musa PR #52 did", only name an mm-prefix capability of
 *   the backend; the rule below is this project's reading of it (the plainest
 *   mask in which a multimodal prefix is seen as a whole while text stays
 *   causal): request r lists spans [s, e) of key positions (span_offsets[r] ..
 *   span_offsets[r+1]-1 in `spans`, any order, may overlap).  A query of a
 *   causal request whose position p lies in a span [s, e) also sees the keys of
 *   that span after it: the high end becomes max(p, e-1) over those spans, and
 *   never passes the request's last key T-1 (a query sees only its own
 *   request's keys).  Non-causal requests see every key anyway.
 *
 *   For q-head h, the kv-head is g = h / (Hq/Hkv) (contiguous GQA groups).
 *   z_j = scale * sum_d q[i,h,d] k[j,g,d]       (d ascending)
 *   m   = max_j z_j ;  e_j = exp(z_j - m) ;  s = sum_j e_j   (j ascending)
 *   o[i,h,d] = (sum_j e_j v[j,g,d]) / s
 *
 * Inputs are bf16 bit patterns; bf16 -> double is exact.  Keys are logical
 * (unpaged): request r's T keys are rows kv_start[r] .. kv_start[r]+T-1 of
 * k/v [total_kv][Hkv][D], kv_start being the running sum of L+n.
 *
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared -pthread (no fast-math).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static double bf16_to_f64(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

typedef struct {
    const uint16_t *q, *k, *v;
    const int32_t *ctx_lens, *block_lens;
    const uint8_t *causal;
    const int32_t *span_offsets; /* [B+1] or NULL */
    const int32_t *spans;        /* [num_spans][2] (start, end) */
    int32_t B, Hq, Hkv, D, window;
    double scale;
    const int64_t *kv_start; /* [B] */
    const int64_t *q_start;  /* [B] */
    const int64_t *tok_req;  /* [total_q] request of each packed query row */
    const int64_t *rows;     /* optional list of token*Hq+head; NULL = all */
    int64_t n_work;          /* number of (token, head) rows to compute */
    double *out;
    int64_t next;            /* shared work counter */
    pthread_mutex_t mu;
} job_t;

/* One output row: query token `tok` (packed index), q-head h. */
static void attend_one(const job_t *J, int64_t tok, int32_t h, double *o, double *z, double *qd)
{
    const int32_t D = J->D;
    const int32_t G = J->Hq / J->Hkv;
    const int64_t r = J->tok_req[tok];
    const int64_t L = J->ctx_lens[r];
    const int64_t n = J->block_lens[r];
    const int64_t T = L + n;
    const int64_t i = tok - J->q_start[r];
    const int64_t p = L + i;
    const int32_t g = h / G;
    const int is_causal = J->causal ? (J->causal[r] != 0) : 0;

    int64_t hi = is_causal ? p : T - 1;
    if (is_causal && J->span_offsets) {
        for (int32_t w = J->span_offsets[r]; w < J->span_offsets[r + 1]; ++w) {
            const int64_t s = J->spans[2 * w], e = J->spans[2 * w + 1];
            if (s <= p && p < e && e - 1 > hi)
                hi = e - 1;
        }
        if (hi > T - 1)
            hi = T - 1;
    }
    int64_t lo = 0;
    if (J->window > 0) {
        lo = p - (int64_t)J->window + 1;
        if (lo < 0)
            lo = 0;
    }

    for (int32_t d = 0; d < D; ++d)
        qd[d] = bf16_to_f64(J->q[(tok * J->Hq + h) * (int64_t)D + d]);

    const int64_t base = J->kv_start[r];
    double m = -INFINITY;
    for (int64_t j = lo; j <= hi; ++j) {
        const uint16_t *kr = J->k + ((base + j) * J->Hkv + g) * (int64_t)D;
        double acc = 0.0;
        for (int32_t d = 0; d < D; ++d)
            acc += qd[d] * bf16_to_f64(kr[d]);
        z[j - lo] = J->scale * acc;
        if (z[j - lo] > m)
            m = z[j - lo];
    }
    double s = 0.0;
    for (int64_t j = lo; j <= hi; ++j) {
        z[j - lo] = exp(z[j - lo] - m);
        s += z[j - lo];
    }
    for (int32_t d = 0; d < D; ++d)
        o[d] = 0.0;
    for (int64_t j = lo; j <= hi; ++j) {
        const uint16_t *vr = J->v + ((base + j) * J->Hkv + g) * (int64_t)D;
        const double e = z[j - lo];
        for (int32_t d = 0; d < D; ++d)
            o[d] += e * bf16_to_f64(vr[d]);
    }
    for (int32_t d = 0; d < D; ++d)
        o[d] = o[d] / s;
}

static void *worker(void *arg)
{
    job_t *J = (job_t *)arg;
    int64_t max_T = 1;
    for (int32_t r = 0; r < J->B; ++r) {
        int64_t T = (int64_t)J->ctx_lens[r] + J->block_lens[r];
        if (T > max_T)
            max_T = T;
    }
    double *z = (double *)malloc(sizeof(double) * (size_t)max_T);
    double *qd = (double *)malloc(sizeof(double) * (size_t)J->D);
    if (!z || !qd) {
        free(z);
        free(qd);
        return (void *)1;
    }
    for (;;) {
        pthread_mutex_lock(&J->mu);
        int64_t w = J->next++;
        pthread_mutex_unlock(&J->mu);
        if (w >= J->n_work)
            break;
        int64_t row = J->rows ? J->rows[w] : w;
        int64_t tok = row / J->Hq;
        int32_t h = (int32_t)(row % J->Hq);
        attend_one(J, tok, h, J->out + w * (int64_t)J->D, z, qd);
    }
    free(z);
    free(qd);
    return NULL;
}

/*
 * Compute the oracle output.
 *   rows == NULL : out is [total_q][Hq][D] (every row).
 *   rows != NULL : out is [n_rows][D], row w = (token rows[w]/Hq, head rows[w]%Hq).
 * Returns 0 on success, -1 on invalid arguments, -2 on allocation failure.
 */
int oracle_block_attn_spans_f64(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                const int32_t *ctx_lens, const int32_t *block_lens, const uint8_t *causal,
                                const int32_t *span_offsets, const int32_t *spans,
                                int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t window, double scale,
                                const int64_t *rows, int64_t n_rows, double *out, int32_t n_threads);

int oracle_block_attn_f64(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                          const int32_t *ctx_lens, const int32_t *block_lens, const uint8_t *causal,
                          int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t window, double scale,
                          const int64_t *rows, int64_t n_rows, double *out, int32_t n_threads)
{
    return oracle_block_attn_spans_f64(q, k, v, ctx_lens, block_lens, causal, NULL, NULL, B, Hq, Hkv, D, window,
                                       scale, rows, n_rows, out, n_threads);
}

/* As oracle_block_attn_f64, with optional bidirectional spans (both NULL = none). */
int oracle_block_attn_spans_f64(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                const int32_t *ctx_lens, const int32_t *block_lens, const uint8_t *causal,
                                const int32_t *span_offsets, const int32_t *spans,
                                int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t window, double scale,
                                const int64_t *rows, int64_t n_rows, double *out, int32_t n_threads)
{
    if ((span_offsets == NULL) != (spans == NULL))
        return -1;
    if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || (Hq % Hkv) != 0 || !out)
        return -1;
    int64_t total_q = 0;
    for (int32_t r = 0; r < B; ++r) {
        if (ctx_lens[r] < 0 || block_lens[r] < 0)
            return -1;
        total_q += block_lens[r];
    }
    int64_t *kv_start = (int64_t *)malloc(sizeof(int64_t) * (size_t)(B + 1));
    int64_t *q_start = (int64_t *)malloc(sizeof(int64_t) * (size_t)(B + 1));
    int64_t *tok_req = (int64_t *)malloc(sizeof(int64_t) * (size_t)(total_q + 1));
    if (!kv_start || !q_start || !tok_req) {
        free(kv_start);
        free(q_start);
        free(tok_req);
        return -2;
    }
    kv_start[0] = 0;
    q_start[0] = 0;
    for (int32_t r = 0; r < B; ++r) {
        kv_start[r + 1] = kv_start[r] + ctx_lens[r] + block_lens[r];
        q_start[r + 1] = q_start[r] + block_lens[r];
        for (int64_t t = q_start[r]; t < q_start[r + 1]; ++t)
            tok_req[t] = r;
    }
    if (rows) {
        for (int64_t w = 0; w < n_rows; ++w)
            if (rows[w] < 0 || rows[w] >= total_q * Hq) {
                free(kv_start);
                free(q_start);
                free(tok_req);
                return -1;
            }
    }
    job_t J;
    memset(&J, 0, sizeof J);
    J.q = q;
    J.k = k;
    J.v = v;
    J.ctx_lens = ctx_lens;
    J.block_lens = block_lens;
    J.causal = causal;
    J.span_offsets = span_offsets;
    J.spans = spans;
    J.B = B;
    J.Hq = Hq;
    J.Hkv = Hkv;
    J.D = D;
    J.window = window;
    J.scale = scale;
    J.kv_start = kv_start;
    J.q_start = q_start;
    J.tok_req = tok_req;
    J.rows = rows;
    J.n_work = rows ? n_rows : total_q * Hq;
    J.out = out;
    J.next = 0;
    pthread_mutex_init(&J.mu, NULL);

    if (n_threads < 1)
        n_threads = 1;
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)n_threads);
    int rc = 0;
    if (!th) {
        rc = -2;
    } else {
        int started = 0;
        for (int32_t t = 0; t < n_threads; ++t) {
            if (pthread_create(&th[t], NULL, worker, &J) != 0)
                break;
            ++started;
        }
        if (started == 0)
            worker(&J);
        for (int t = 0; t < started; ++t) {
            void *ret = NULL;
            pthread_join(th[t], &ret);
            if (ret)
                rc = -2;
        }
        free(th);
    }
    pthread_mutex_destroy(&J.mu);
    free(kv_start);
    free(q_start);
    free(tok_req);
    return rc;
}
