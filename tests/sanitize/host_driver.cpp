// host_driver.cpp -- exercises the host part of the C ABI (bitlinear_pack,
// bitlinear_weight_quant, bitlinear_strerror, bitlinear_abi_version) on seeded
// inputs and every error path, so that an AddressSanitizer +
// UndefinedBehaviorSanitizer build of host.cpp can look for out-of-bounds
// accesses and undefined behaviour. Buffers have their exact sizes. Prints "ok".
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <vector>

#include "../../include/bitlinear.h"

static uint64_t state = 0x2545F4914F6CDD1Dull;

static uint32_t next_u32()
{
    state ^= state << 13;
    state ^= state >> 7;
    state ^= state << 17;
    return (uint32_t)(state >> 11);
}

#define CHECK(c)                                                            \
    do {                                                                    \
        if (!(c)) {                                                         \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            return 1;                                                       \
        }                                                                   \
    } while (0)

int main()
{
    const int64_t shapes[][2] = {{1, 4}, {3, 8}, {17, 64}, {5, 10244}, {2, 2560}};
    for (auto& sh : shapes) {
        const int64_t n = sh[0], k = sh[1];
        std::vector<int8_t> t(n * k);
        for (auto& v : t) v = (int8_t)((int)(next_u32() % 3) - 1);
        std::vector<uint8_t> p(n * k / 4);
        CHECK(bitlinear_pack(t.data(), n, k, p.data()) == BL_OK);
        for (int64_t i = 0; i < n * k; ++i) CHECK((((p[i / 4] >> (2 * (i % 4))) & 3) - 1) == t[i]);
        std::vector<float> w(n * k);
        for (auto& v : w) v = ((float)(next_u32() % 2001) - 1000.0f) * 1e-4f;
        std::vector<int8_t> tq(n * k);
        float s = 0.0f;
        CHECK(bitlinear_weight_quant(w.data(), n, k, tq.data(), &s) == BL_OK && s > 0.0f);
        for (auto v : tq) CHECK(v >= -1 && v <= 1);
    }
    int8_t bad[8] = {0, 0, 0, 2, 0, 0, 0, 0};
    uint8_t out[2] = {0xAA, 0xAA};
    CHECK(bitlinear_pack(bad, 1, 8, out) == BL_ERR_VALUE && out[0] == 0xAA && out[1] == 0xAA);
    CHECK(bitlinear_pack(bad, 1, 6, out) == BL_ERR_SHAPE);
    CHECK(bitlinear_pack(nullptr, 1, 8, out) == BL_ERR_NULL);
    CHECK(bitlinear_pack(bad, 0, 8, out) == BL_ERR_SHAPE);
    float wn[4] = {1.0f, NAN, 0.0f, 0.0f}, s = 0.0f;
    int8_t tq[4];
    CHECK(bitlinear_weight_quant(wn, 1, 4, tq, &s) == BL_ERR_VALUE);
    CHECK(bitlinear_weight_quant(wn, 1, 4, nullptr, &s) == BL_ERR_NULL);
    CHECK(bitlinear_weight_quant(wn, -1, 4, tq, &s) == BL_ERR_SHAPE);
    float wz[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    CHECK(bitlinear_weight_quant(wz, 1, 4, tq, &s) == BL_OK && s == (float)(1.0 / 1e-5));
    for (int code = -9; code <= 1; ++code) CHECK(bitlinear_strerror(code) != nullptr);
    CHECK(bitlinear_abi_version() >= 1);
    puts("ok");
    return 0;
}
