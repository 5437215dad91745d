// host.cpp -- host-side part of the C ABI: status text, the ternary packer and
// weight_quant. Plain C++; touches no device memory.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "../../include/bitlinear.h"

extern "C" {

int bitlinear_abi_version(void) { return 1; }

const char* bitlinear_strerror(int status)
{
    switch (status) {
    case BL_OK: return "ok";
    case BL_ERR_NULL: return "a required pointer is NULL";
    case BL_ERR_SHAPE: return "unsupported or inconsistent sizes";
    case BL_ERR_ALIGN: return "a pointer is not aligned as the call requires";
    case BL_ERR_VALUE: return "a value is out of range";
    case BL_ERR_WORKSPACE: return "workspace too small";
    case BL_ERR_LAUNCH: return "kernel launch failed";
    case BL_ERR_DEVICE: return "no usable gfx950 device or HIP runtime error";
    default: return "unknown status";
    }
}

// TQ2_0 packing: four 2-bit codes (t + 1) per byte, first weight in the low
// bits. The whole input is checked before anything is written.
int bitlinear_pack(const int8_t* t, int64_t n, int64_t k, uint8_t* packed)
{
    if (!t || !packed) return BL_ERR_NULL;
    if (n <= 0 || k <= 0 || (k & 3) != 0) return BL_ERR_SHAPE;
    const int64_t total = n * k;
    for (int64_t i = 0; i < total; ++i) {
        const int v = t[i];
        if (v < -1 || v > 1) return BL_ERR_VALUE;
    }
    // Rows are contiguous in both layouts, so the packed stream is simply the
    // weight stream taken four at a time.
    const int64_t nbytes = total / 4;
    for (int64_t b = 0; b < nbytes; ++b) {
        const int8_t* w = t + 4 * b;
        packed[b] = (uint8_t)((uint32_t)(w[0] + 1) | ((uint32_t)(w[1] + 1) << 2) |
                              ((uint32_t)(w[2] + 1) << 4) | ((uint32_t)(w[3] + 1) << 6));
    }
    return BL_OK;
}

// Absmean ternary weight quantization: one fp32 scale for the whole tensor.
int bitlinear_weight_quant(const float* w, int64_t n, int64_t k, int8_t* t, float* w_scale)
{
    if (!w || !t || !w_scale) return BL_ERR_NULL;
    if (n <= 0 || k <= 0) return BL_ERR_SHAPE;
    const int64_t total = n * k;
    double abs_sum = 0.0;
    for (int64_t i = 0; i < total; ++i) {
        const float v = w[i];
        if (!isfinite(v)) return BL_ERR_VALUE;
        abs_sum += fabs((double)v);
    }
    double mean = abs_sum / (double)total;
    if (!(mean >= 1e-5)) mean = 1e-5;
    const float scale = (float)(1.0 / mean);
    for (int64_t i = 0; i < total; ++i) {
        const float r = nearbyintf(w[i] * scale);
        t[i] = (int8_t)(r > 1.0f ? 1 : (r < -1.0f ? -1 : (int)r));
    }
    *w_scale = scale;
    return BL_OK;
}

// Rotary-embedding table: theta_i = base^(-2i / hd), angle pos * theta_i, cos
// and sin in fp64, each rounded once to fp32; row pos holds hd / 2 entries.
int bitnet_rope_table(double base, int64_t head_dim, int64_t max_pos, float* cos_out, float* sin_out)
{
    if (!cos_out || !sin_out) return BL_ERR_NULL;
    if (head_dim <= 0 || head_dim % 2 != 0 || max_pos <= 0) return BL_ERR_SHAPE;
    if (!(base > 1.0) || !(base < INFINITY)) return BL_ERR_VALUE;
    const int64_t half = head_dim / 2;
    for (int64_t i = 0; i < half; ++i) {
        const double theta = pow(base, -(double)(2 * i) / (double)head_dim);
        for (int64_t p = 0; p < max_pos; ++p) {
            const double ang = (double)p * theta;
            cos_out[p * half + i] = (float)cos(ang);
            sin_out[p * half + i] = (float)sin(ang);
        }
    }
    return BL_OK;
}

}  // extern "C"
