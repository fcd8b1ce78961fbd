/*
 * oracle_driver.c -- runs the fp64 oracle (oracle/oracle_f64.c, linked in) on
 * seeded inputs held in buffers of exactly the documented sizes, so that a build
 * with -fsanitize=address,undefined reports any read or write outside them and
 * any undefined arithmetic.  Built and run by tests/test_sanitizers.py on the CPU.
 *
 * Cases: empty blocks, zero-length contexts, causal and non-causal requests,
 * windows (including 1 and wider than the context), GQA groups, head_dim 8..512,
 * bidirectional spans (including spans past the request's keys), and row lists.
 * Each case also checks a closed form: with every value row of a kv-head equal to
 * a constant c, every output row of that head's q-heads is exactly c.
 * Prints "OK <cases>" or "FAIL <reason>".
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_block_attn_f64(const uint16_t *q, const uint16_t *k, const uint16_t *v, const int32_t *ctx_lens,
                          const int32_t *block_lens, const uint8_t *causal, int32_t B, int32_t Hq, int32_t Hkv,
                          int32_t D, int32_t window, double scale, const int64_t *rows, int64_t n_rows, double *out,
                          int32_t n_threads);
int oracle_block_attn_spans_f64(const uint16_t *q, const uint16_t *k, const uint16_t *v, const int32_t *ctx_lens,
                                const int32_t *block_lens, const uint8_t *causal, const int32_t *span_offsets,
                                const int32_t *spans, int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t window,
                                double scale, const int64_t *rows, int64_t n_rows, double *out, int32_t n_threads);

static uint64_t g_state = 0x9e3779b97f4a7c15ull;

static uint32_t next_u32(void)
{
    g_state = g_state * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(g_state >> 33);
}

/* bf16 bits of a value in [-2, 2) with 7 mantissa bits (exactly representable) */
static uint16_t rand_bf16(void)
{
    const float f = ((int)(next_u32() % 512) - 256) / 128.0f;
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

static uint16_t bf16_of(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

static int run_case(int B, int Hq, int Hkv, int D, int window, const int32_t *L, const int32_t *n,
                    const uint8_t *causal, int with_spans, int with_rows)
{
    int64_t total_q = 0, total_kv = 0;
    for (int r = 0; r < B; ++r) {
        total_q += n[r];
        total_kv += L[r] + n[r];
    }
    uint16_t *q = malloc(sizeof(uint16_t) * (size_t)(total_q * Hq * D + 1));
    uint16_t *k = malloc(sizeof(uint16_t) * (size_t)(total_kv * Hkv * D + 1));
    uint16_t *v = malloc(sizeof(uint16_t) * (size_t)(total_kv * Hkv * D + 1));
    for (int64_t i = 0; i < total_q * Hq * D; ++i)
        q[i] = rand_bf16();
    for (int64_t i = 0; i < total_kv * Hkv * D; ++i)
        k[i] = rand_bf16();
    /* value rows of kv-head g are the constant 0.25 * (g + 1) */
    for (int64_t t = 0; t < total_kv; ++t)
        for (int g = 0; g < Hkv; ++g)
            for (int d = 0; d < D; ++d)
                v[(t * Hkv + g) * D + d] = bf16_of(0.25f * (float)(g + 1));

    int32_t *offs = NULL, *spans = NULL;
    int nsp = 0;
    if (with_spans) {
        offs = malloc(sizeof(int32_t) * (size_t)(B + 1));
        spans = malloc(sizeof(int32_t) * (size_t)(2 * B * 2 + 2));
        offs[0] = 0;
        for (int r = 0; r < B; ++r) {
            const int T = L[r] + n[r];
            if (T > 0) {
                const int s = (int)(next_u32() % (uint32_t)T);
                spans[2 * nsp] = s;
                spans[2 * nsp + 1] = s + 1 + (int)(next_u32() % 40u); /* may pass T */
                ++nsp;
            }
            offs[r + 1] = nsp;
        }
    }

    int64_t n_rows = total_q * Hq;
    int64_t *rows = NULL;
    if (with_rows && n_rows > 0) {
        const int64_t m = n_rows < 7 ? n_rows : 7;
        rows = malloc(sizeof(int64_t) * (size_t)m);
        for (int64_t w = 0; w < m; ++w)
            rows[w] = (int64_t)(next_u32() % (uint32_t)n_rows);
        n_rows = m;
    }
    double *out = malloc(sizeof(double) * (size_t)(n_rows * D + 1));
    const double scale = 1.0 / sqrt((double)D);
    int rc;
    if (with_spans)
        rc = oracle_block_attn_spans_f64(q, k, v, L, n, causal, offs, spans, B, Hq, Hkv, D, window, scale, rows,
                                         rows ? n_rows : 0, out, 3);
    else
        rc = oracle_block_attn_f64(q, k, v, L, n, causal, B, Hq, Hkv, D, window, scale, rows, rows ? n_rows : 0,
                                   out, 3);
    int bad = rc != 0;
    const int G = Hq / Hkv;
    for (int64_t w = 0; w < n_rows && !bad; ++w) {
        const int64_t row = rows ? rows[w] : w;
        const int h = (int)(row % Hq);
        const double c = 0.25 * (double)(h / G + 1);
        for (int d = 0; d < D; ++d)
            if (!(fabs(out[w * D + d] - c) <= 1e-12 * c)) {
                bad = 1;
                break;
            }
    }
    free(q);
    free(k);
    free(v);
    free(offs);
    free(spans);
    free(rows);
    free(out);
    return bad;
}

int main(void)
{
    int cases = 0;
    const int dims[] = {8, 64, 128, 136, 256, 512};
    const int windows[] = {0, -4, 1, 2, 16, 33, 5000};
    for (int iter = 0; iter < 60; ++iter) {
        const int B = 1 + (int)(next_u32() % 6u);
        const int Hkv = 1 + (int)(next_u32() % 3u);
        const int G = 1 + (int)(next_u32() % 4u);
        const int D = dims[next_u32() % 6u];
        const int window = windows[next_u32() % 7u];
        int32_t L[6], n[6];
        uint8_t c[6];
        for (int r = 0; r < B; ++r) {
            L[r] = (next_u32() % 5u == 0) ? 0 : (int32_t)(next_u32() % 90u);
            n[r] = (next_u32() % 6u == 0) ? 0 : 1 + (int32_t)(next_u32() % 16u);
            c[r] = (uint8_t)(next_u32() & 1u);
        }
        const int with_spans = iter % 3 == 1;
        const int with_rows = iter % 4 == 2;
        if (run_case(B, Hkv * G, Hkv, D, window, L, n, c, with_spans, with_rows)) {
            printf("FAIL case %d (B=%d Hq=%d Hkv=%d D=%d window=%d spans=%d rows=%d)\n", iter, B, Hkv * G, Hkv, D,
                   window, with_spans, with_rows);
            return 1;
        }
        ++cases;
    }
    printf("OK %d\n", cases);
    return 0;
}
