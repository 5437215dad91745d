/*
 * oracle_driver.c -- exercises every function of the CPU oracle on seeded
 * inputs and on edge cases (empty-ish shapes, K not a multiple of the partial
 * count, zero rows, code-3 bytes, error returns), so that an AddressSanitizer +
 * UndefinedBehaviorSanitizer build of the oracle can look for out-of-bounds
 * accesses, uninitialised reads, overflow and other undefined behaviour.
 * It checks the results only loosely (the pins check values); it prints "ok".
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int ref_weight_quant(const float *w, int64_t n, int64_t k, int8_t *t, float *s_w);
int ref_pack(const int8_t *t, int64_t n, int64_t k, uint8_t *packed);
int ref_unpack(const uint8_t *packed, int64_t n, int64_t k, int8_t *t);
double ref_sumsq(const float *x, int64_t k);
int ref_rmsnorm(const float *x, const float *g, float eps, int64_t m, int64_t k, float *y);
int ref_activation_quant(const float *y, int64_t m, int64_t k, int8_t *q, float *s_a, int32_t *qsum);
int ref_matmul_i32(const int8_t *t, const int8_t *q, int64_t m, int64_t n, int64_t k, int32_t *acc);
int ref_dequant(const int32_t *acc, const float *s_a, float s_w, int64_t m, int64_t n, float *y);
int ref_bitlinear(const uint8_t *packed, float s_w, int64_t n, int64_t k, const int8_t *q, const float *s_a,
                  int64_t m, float *y, int32_t *acc);
void ref_relu2_mul(const float *gate, const float *up, int64_t count, float *h);
void ref_residual_add(float *x, const float *d, int64_t count);
int ref_argmax_rows(const int32_t *acc, int64_t m, int64_t n, int32_t *idx);

static uint64_t state = 0x9E3779B97F4A7C15ull;

static uint32_t next_u32(void)
{
    state ^= state << 13;
    state ^= state >> 7;
    state ^= state << 17;
    return (uint32_t)(state >> 11);
}

static float next_f(void) { return ((float)(next_u32() % 20001) - 10000.0f) / 2500.0f; }

#define CHECK(c)                                                            \
    do {                                                                    \
        if (!(c)) {                                                         \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            return 1;                                                       \
        }                                                                   \
    } while (0)

static int one_shape(int64_t m, int64_t n, int64_t k)
{
    /* every buffer is allocated at its exact size, so ASan sees any overrun */
    float *w = malloc(sizeof(float) * n * k), *x = malloc(sizeof(float) * m * k), *gain = malloc(sizeof(float) * k);
    float *y = malloc(sizeof(float) * m * k), *s_a = malloc(sizeof(float) * m), *out = malloc(sizeof(float) * m * n);
    float *out2 = malloc(sizeof(float) * m * n), *h = malloc(sizeof(float) * m * n);
    int8_t *t = malloc(n * k), *t2 = malloc(n * k), *q = malloc(m * k);
    uint8_t *p = malloc(n * k / 4);
    int32_t *qs = malloc(sizeof(int32_t) * m), *acc = malloc(sizeof(int32_t) * m * n);
    int32_t *acc2 = malloc(sizeof(int32_t) * m * n), *idx = malloc(sizeof(int32_t) * m);
    float s_w = 0.0f;
    for (int64_t i = 0; i < n * k; i++) w[i] = next_f() * 0.01f;
    for (int64_t i = 0; i < m * k; i++) x[i] = next_f();
    for (int64_t i = 0; i < k; i++) gain[i] = 0.5f + (float)(next_u32() % 1000) / 1000.0f;
    if (m > 1)
        for (int64_t i = 0; i < k; i++) x[(m - 1) * k + i] = 0.0f; /* a zero row */
    CHECK(ref_weight_quant(w, n, k, t, &s_w) == 0 && s_w > 0.0f);
    CHECK(ref_pack(t, n, k, p) == 0);
    CHECK(ref_unpack(p, n, k, t2) == 0 && memcmp(t, t2, n * k) == 0);
    CHECK(ref_rmsnorm(x, gain, 1e-5f, m, k, y) == 0);
    CHECK(ref_activation_quant(y, m, k, q, s_a, qs) == 0);
    CHECK(ref_activation_quant(y, m, k, q, s_a, NULL) == 0);
    CHECK(ref_sumsq(x, k) >= 0.0);
    CHECK(ref_matmul_i32(t, q, m, n, k, acc) == 0);
    CHECK(ref_dequant(acc, s_a, s_w, m, n, out) == 0);
    CHECK(ref_bitlinear(p, s_w, n, k, q, s_a, m, out2, acc2) == 0);
    CHECK(memcmp(acc, acc2, sizeof(int32_t) * m * n) == 0);
    CHECK(ref_bitlinear(p, s_w, n, k, q, s_a, m, out2, NULL) == 0);
    ref_relu2_mul(out, out2, m * n, h);
    ref_residual_add(out, h, m * n);
    CHECK(ref_argmax_rows(acc, m, n, idx) == 0);
    for (int64_t r = 0; r < m; r++) CHECK(idx[r] >= 0 && idx[r] < n);
    free(w), free(x), free(gain), free(y), free(s_a), free(out), free(out2), free(h);
    free(t), free(t2), free(q), free(p), free(qs), free(acc), free(acc2), free(idx);
    return 0;
}

int main(void)
{
    static const int64_t shapes[][3] = {{1, 1, 4},   {1, 3, 8},    {2, 5, 12},   {3, 16, 64},  {4, 7, 516},
                                        {2, 9, 1028}, {5, 33, 260}, {1, 2, 2560}, {3, 4, 4100}};
    for (size_t i = 0; i < sizeof shapes / sizeof shapes[0]; i++)
        if (one_shape(shapes[i][0], shapes[i][1], shapes[i][2])) return 1;

    /* error returns: bad shapes, values outside {-1,0,1}, code-3 bytes */
    int8_t tb[8] = {0, 1, -1, 2, 0, 0, 0, 0}, tt[8];
    uint8_t pb[2] = {0x55, 0xFF};
    float dummy = 1.0f;
    CHECK(ref_pack(tb, 1, 8, pb) == -4);
    CHECK(ref_pack(tb, 1, 6, pb) == -2);
    CHECK(ref_unpack(pb, 1, 8, tt) == -4);
    CHECK(ref_weight_quant(&dummy, 0, 1, tt, &dummy) == -2);
    CHECK(ref_matmul_i32(tt, tt, 0, 1, 1, NULL) == -2);
    CHECK(ref_argmax_rows(NULL, 1, 0, NULL) == -2);
    /* an all-zero tensor takes the 1e-5 floor */
    float wz[8] = {0};
    float s = 0.0f;
    CHECK(ref_weight_quant(wz, 2, 4, tt, &s) == 0 && s == (float)(1.0 / 1e-5));
    puts("ok");
    return 0;
}
