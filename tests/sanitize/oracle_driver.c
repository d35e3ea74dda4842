/*
 * Runs every function of the CPU oracle (oracle/bitlinear_oracle.c) on small,
 * ragged and degenerate shapes, for a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_sanitize.py builds and runs it).
 * The sanitizers catch out-of-bounds accesses and undefined arithmetic; the
 * few checks below only make sure each call did its work (round trips,
 * the contraction against a plain loop).  Exit status 0 = clean.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double oracle_abs_sum(const float *W, int64_t count);
float oracle_gamma(const float *W, int64_t N, int64_t K);
int oracle_binarise(const float *W, int64_t N, int64_t K, int8_t *codes, float *alpha, float *beta);
int oracle_ternarise(const float *W, int64_t N, int64_t K, float gamma, float eps, int8_t *codes);
int64_t oracle_packed_bytes(int64_t N, int64_t K);
int oracle_encode(const int8_t *codes, int64_t N, int64_t K, uint8_t *packed);
int oracle_decode(const uint8_t *packed, int64_t N, int64_t K, int8_t *codes);
int oracle_encode_t1(const int8_t *codes, int64_t N, int64_t K, uint8_t *packed_t);
int oracle_decode_t1(const uint8_t *packed_t, int64_t N, int64_t K, int8_t *codes);
int64_t oracle_packed_bytes_b1(int64_t N, int64_t K);
int64_t oracle_packed_bytes_t3(int64_t N, int64_t K);
int oracle_encode_t3(const int8_t *codes, int64_t N, int64_t K, uint8_t *packed);
int oracle_decode_t3(const uint8_t *packed, int64_t N, int64_t K, int8_t *codes);
int oracle_encode_b1(const int8_t *codes, int64_t N, int64_t K, uint8_t *packed);
int oracle_decode_b1(const uint8_t *packed, int64_t N, int64_t K, int8_t *codes);
int oracle_quant_act(const uint16_t *x, int64_t M, int64_t K, float eps, int8_t *q, float *s);
int oracle_rmsnorm_quant_act(const uint16_t *x, const float *gain, int64_t M, int64_t K, float eps_norm, float eps,
                             int8_t *q, float *s, double *v);
int oracle_contract(const int8_t *q, const int8_t *codes, int64_t M, int64_t N, int64_t K, int32_t *acc);
int oracle_contract_pairs(const int8_t *q, const int8_t *codes, int64_t K, const int64_t *m_idx, const int64_t *n_idx,
                          int64_t P, int32_t *acc);
void oracle_epilogue(const int32_t *acc, int64_t M, int64_t N, float gamma, const float *s, float *y);
int oracle_backward_input(const uint16_t *dy, const int8_t *codes, int64_t M, int64_t N, int64_t K, float gamma,
                          const uint16_t *dx_prev, double *ref, double *mag, uint16_t *dx);
int oracle_adamw_flip(float *W, const float *g, float *m, float *v, int64_t n, int32_t t, double lr, double b1,
                      double b2, double eps, double wd, int16_t *flip_count, int16_t *last_flip);
int oracle_flip_stats(const int16_t *flip_count, const int16_t *last_flip, int64_t n, int32_t T, float *sign_age,
                      float *flip_rate);
int oracle_flip_update(const float *prev, const float *curr, int64_t n, int32_t step, int16_t *flip_count,
                       int16_t *last_flip);

static int failures = 0;
#define CHECK(c)                                                         \
    do {                                                                 \
        if (!(c)) {                                                      \
            fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
            ++failures;                                                  \
        }                                                                \
    } while (0)

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64(void)
{
    /* splitmix64 */
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
static float uniform_pm1(void) { return (float)((double)(next_u64() >> 11) * 0x1.0p-53 * 2.0 - 1.0); }
static uint16_t to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

/* exact-size heap buffers, so ASan sees every overrun */
static void *xmalloc(size_t n) { return malloc(n ? n : 1); }

static void one_shape(int64_t N, int64_t K, int64_t M)
{
    const int64_t NK = N * K, MK = M * K, MN = M * N;
    float *W = xmalloc((size_t)NK * sizeof(float));
    for (int64_t i = 0; i < NK; ++i) W[i] = 0.02f * uniform_pm1();
    if (NK > 2) W[1] = 0.0f;

    float g = oracle_gamma(W, N, K);
    CHECK(g >= 0.0f && fabs(oracle_abs_sum(W, NK) / (double)NK - (double)g) <= 1e-6 * (double)g + 1e-30);

    int8_t *codes = xmalloc((size_t)NK), *back = xmalloc((size_t)NK);
    CHECK(oracle_ternarise(W, N, K, g, 1e-5f, codes) == 0);
    const int64_t pb = oracle_packed_bytes(N, K);
    uint8_t *packed = xmalloc((size_t)pb);
    CHECK(oracle_encode(codes, N, K, packed) == 0);
    CHECK(oracle_decode(packed, N, K, back) == 0);
    CHECK(memcmp(codes, back, (size_t)NK) == 0);

    const int64_t pbt = oracle_packed_bytes(K, N);
    uint8_t *packed_t = xmalloc((size_t)pbt);
    CHECK(oracle_encode_t1(codes, N, K, packed_t) == 0);
    memset(back, 7, (size_t)NK);
    CHECK(oracle_decode_t1(packed_t, N, K, back) == 0);
    CHECK(memcmp(codes, back, (size_t)NK) == 0);

    const int64_t pb3 = oracle_packed_bytes_t3(N, K);
    if (K % 320 == 0) {
        uint8_t *packed_t3 = xmalloc((size_t)pb3);
        CHECK(oracle_encode_t3(codes, N, K, packed_t3) == 0);
        memset(back, 7, (size_t)NK);
        CHECK(oracle_decode_t3(packed_t3, N, K, back) == 0);
        CHECK(memcmp(codes, back, (size_t)NK) == 0);
        free(packed_t3);
    } else {
        CHECK(pb3 == -1 && oracle_encode_t3(codes, N, K, packed) != 0);
    }

    float alpha = 0.0f, beta = 0.0f;
    CHECK(oracle_binarise(W, N, K, back, &alpha, &beta) == 0);
    const int64_t pb1 = oracle_packed_bytes_b1(N, K);
    if (K % 64 == 0) {
        CHECK(pb1 == ((N + 15) / 16) * ((K + 127) / 128) * 256);
        uint8_t *packed_b1 = xmalloc((size_t)pb1);
        int8_t *bin = xmalloc((size_t)NK);
        CHECK(oracle_encode_b1(back, N, K, packed_b1) == 0);
        CHECK(oracle_decode_b1(packed_b1, N, K, bin) == 0);
        CHECK(memcmp(back, bin, (size_t)NK) == 0);
        CHECK(oracle_encode_b1(codes, N, K, packed_b1) != 0 || memchr(codes, 0, (size_t)NK) == NULL);
        free(packed_b1);
        free(bin);
    } else {
        CHECK(pb1 == -1);
        CHECK(oracle_encode_b1(back, N, K, packed) != 0);
    }

    uint16_t *x = xmalloc((size_t)MK * sizeof(uint16_t));
    for (int64_t i = 0; i < MK; ++i) x[i] = to_bf16(uniform_pm1() * 3.0f);
    if (MK > 0) x[0] = to_bf16(60.0f); /* an outlier */
    int8_t *q = xmalloc((size_t)MK);
    float *s = xmalloc((size_t)M * sizeof(float));
    CHECK(oracle_quant_act(x, M, K, 1e-5f, q, s) == 0);

    float *gain = xmalloc((size_t)K * sizeof(float));
    for (int64_t k = 0; k < K; ++k) gain[k] = 1.0f + 0.25f * uniform_pm1();
    double *v = xmalloc((size_t)MK * sizeof(double));
    int8_t *q2 = xmalloc((size_t)MK);
    float *s2 = xmalloc((size_t)M * sizeof(float));
    CHECK(oracle_rmsnorm_quant_act(x, gain, M, K, 1e-6f, 1e-5f, q2, s2, v) == 0);
    CHECK(oracle_rmsnorm_quant_act(x, NULL, M, K, 0.0f, 1e-5f, q2, s2, NULL) == 0);

    int32_t *acc = xmalloc((size_t)MN * sizeof(int32_t));
    CHECK(oracle_contract(q, codes, M, N, K, acc) == 0);
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            int64_t a = 0;
            for (int64_t k = 0; k < K; ++k) a += (int64_t)q[m * K + k] * (int64_t)codes[n * K + k];
            CHECK(a == acc[m * N + n]);
        }
    const int64_t P = MN < 5 ? MN : 5;
    int64_t *mi = xmalloc((size_t)P * sizeof(int64_t)), *ni = xmalloc((size_t)P * sizeof(int64_t));
    int32_t *accp = xmalloc((size_t)P * sizeof(int32_t));
    for (int64_t p = 0; p < P; ++p) {
        mi[p] = (M - 1 - p % M);
        ni[p] = (p * 7) % N;
    }
    CHECK(oracle_contract_pairs(q, codes, K, mi, ni, P, accp) == 0);
    for (int64_t p = 0; p < P; ++p) CHECK(accp[p] == acc[mi[p] * N + ni[p]]);

    float *y = xmalloc((size_t)MN * sizeof(float));
    oracle_epilogue(acc, M, N, g, s, y);

    uint16_t *dy = xmalloc((size_t)MN * sizeof(uint16_t)), *dx = xmalloc((size_t)MK * sizeof(uint16_t));
    for (int64_t i = 0; i < MN; ++i) dy[i] = to_bf16(uniform_pm1());
    double *ref = xmalloc((size_t)MK * sizeof(double)), *mag = xmalloc((size_t)MK * sizeof(double));
    CHECK(oracle_backward_input(dy, codes, M, N, K, g, NULL, ref, mag, dx) == 0);
    CHECK(oracle_backward_input(dy, codes, M, N, K, g, x, ref, mag, dx) == 0);

    float *Wc = xmalloc((size_t)NK * sizeof(float)), *gr = xmalloc((size_t)NK * sizeof(float));
    float *m1 = xmalloc((size_t)NK * sizeof(float)), *v1 = xmalloc((size_t)NK * sizeof(float));
    int16_t *fc = xmalloc((size_t)NK * sizeof(int16_t)), *lf = xmalloc((size_t)NK * sizeof(int16_t));
    memcpy(Wc, W, (size_t)NK * sizeof(float));
    for (int64_t i = 0; i < NK; ++i) {
        gr[i] = 0.5f * uniform_pm1();
        m1[i] = v1[i] = 0.0f;
        fc[i] = (int16_t)(i % 3 == 0 ? 32767 : 0);
        lf[i] = 0;
    }
    CHECK(oracle_adamw_flip(Wc, gr, m1, v1, NK, 1, 0.05, 0.9, 0.999, 1e-8, 0.1, fc, lf) == 0);
    CHECK(oracle_adamw_flip(Wc, gr, m1, v1, NK, 2, 0.05, 0.9, 0.999, 1e-8, 0.1, NULL, NULL) == 0);
    CHECK(oracle_flip_update(W, Wc, NK, 32767, fc, lf) == 0);
    CHECK(oracle_flip_update(W, Wc, NK, 0, fc, lf) != 0);
    for (int64_t i = 0; i < NK; ++i) CHECK(fc[i] >= 0 && fc[i] <= 32767);
    float *age = xmalloc((size_t)NK * sizeof(float)), *rate = xmalloc((size_t)NK * sizeof(float));
    CHECK(oracle_flip_stats(fc, lf, NK, 32767, age, rate) == 0);

    free(W); free(codes); free(back); free(packed); free(packed_t); free(x); free(q); free(s);
    free(gain); free(v); free(q2); free(s2); free(acc); free(mi); free(ni); free(accp); free(y);
    free(dy); free(dx); free(ref); free(mag); free(Wc); free(gr); free(m1); free(v1); free(fc); free(lf);
    free(age); free(rate);
}

int main(void)
{
    /* ragged and degenerate shapes: single row / column, K below a fragment,
     * N below a row block, partial groups of 1..3 fragments, an exact group */
    static const int64_t shapes[][3] = {{1, 1, 1},   {1, 3, 2},    {3, 1, 1},   {16, 64, 1}, {17, 65, 3},
                                        {15, 63, 2}, {33, 129, 5}, {5, 200, 4}, {40, 256, 2}, {64, 320, 3},
                                        {8, 1000, 2}, {20, 640, 3}, {17, 64, 1}};
    for (size_t i = 0; i < sizeof(shapes) / sizeof(shapes[0]); ++i)
        one_shape(shapes[i][0], shapes[i][1], shapes[i][2]);

    /* special values: all-zero weights and tokens (eps floors), huge tokens */
    {
        float W0[12] = {0};
        int8_t c[12];
        CHECK(oracle_ternarise(W0, 3, 4, oracle_gamma(W0, 3, 4), 1e-5f, c) == 0);
        CHECK(oracle_ternarise(W0, 3, 4, 0.0f, 0.0f, c) == 0);
        uint16_t xz[8] = {0}, xh[4] = {0x7F7F, 0xFF7F, 0x0001, 0x8000};
        int8_t q[8];
        float s[2];
        CHECK(oracle_quant_act(xz, 2, 4, 1e-5f, q, s) == 0);
        CHECK(oracle_quant_act(xh, 1, 4, 1e-5f, q, s) == 0);
        double v[8];
        CHECK(oracle_rmsnorm_quant_act(xz, NULL, 2, 4, 0.0f, 1e-5f, q, s, v) == 0);
        CHECK(oracle_rmsnorm_quant_act(xh, NULL, 1, 4, 1e-6f, 1e-5f, q, s, v) == 0);
        uint16_t xinf[2] = {0x7F80, 0};
        CHECK(oracle_quant_act(xinf, 1, 2, 1e-5f, q, s) != 0);
        /* a packed buffer holding the never-written code 10 is rejected */
        uint8_t bad[256];
        memset(bad, 0, sizeof bad);
        bad[0] = 0x2;
        CHECK(oracle_decode(bad, 1, 1, c) != 0);
    }
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("oracle sanitizer driver: clean\n");
    return 0;
}
