// wave_quant.h -- [RMSNorm +] per-token absmax activation quant of one row
// (RMSNorm in front of every BitLinear, "Add Support for BitNet Architecture
// Inference", candle PR 2664; activation_quant of the same PR) by one wave, for
// rows of up to 64 * 4 * V values, or by one 512-thread workgroup. Used by the
// quant kernels and by the fused quant + GEMV kernels, so all of them compute
// the same q, s_a and sum(q) with the same operations in the same order.
//
// Lane t loads the float4 chunks t, t + 64, ... (coalesced), so no LDS and no
// barrier is needed. The fixed order of the sum of squares still holds: chunk
// u of lane t holds x[4 t + c + 256 u] (c = 0..3), i.e. members of partials
// 4 t + c (u even) and 256 + 4 t + c (u odd), accumulated in ascending u --
// ascending k within each partial. The butterfly over the 512 partials then
// runs with offsets 1 and 2 inside the lane, 4 .. 128 across lanes (xor 1 ..
// 32) and 256 inside the lane again, in that (ascending) order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wave.h"

namespace bl {

__device__ __forceinline__ int quant_one(float y, float scale)
{
    const float r = rintf(y * scale);
    return (int)fminf(fmaxf(r, -128.0f), 127.0f);
}

// Loads lane's share of row xrow[0..k) (and of the gains when kNorm).
template <bool kNorm, int V>
__device__ __forceinline__ void wave_quant_load(const float* __restrict__ xrow, const float* __restrict__ gain, int k,
                                                int lane, float4 (&xv)[V], float4 (&gv)[V])
{
    const int k4 = k >> 2;  // float4 chunks per row
    const float4* xr = reinterpret_cast<const float4*>(xrow);
    const float4* gr = reinterpret_cast<const float4*>(gain);
#pragma unroll
    for (int u = 0; u < V; ++u) {
        const int i = lane + 64 * u;
        xv[u] = i < k4 ? xr[i] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        if (kNorm) gv[u] = i < k4 ? gr[i] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
}

// Quantizes the loaded row (gains applied when kNorm) into qr (natural order,
// or 4x4 byte-transposed per 16 values when kPerm); every lane returns s_a
// (scale_out) and sum(q) (sum_out). qr may point to global memory or LDS.
template <bool kNorm, bool kPerm, int V>
__device__ __forceinline__ void wave_quant_compute(const float4 (&xv)[V], const float4 (&gv)[V], float eps, int k,
                                                   int lane, int8_t* qr, float& scale_out, int& sum_out)
{
    const int k4 = k >> 2;  // float4 chunks per row

    float r = 1.0f;
    if (kNorm) {
        double s[2][4] = {{0.0, 0.0, 0.0, 0.0}, {0.0, 0.0, 0.0, 0.0}};  // [u odd][c]
#pragma unroll
        for (int u = 0; u < V; ++u) {
            const float4 v = xv[u];
            const double a = v.x, b = v.y, c = v.z, d = v.w;
            s[u & 1][0] += a * a;  // exact squares; zero beyond k
            s[u & 1][1] += b * b;
            s[u & 1][2] += c * c;
            s[u & 1][3] += d * d;
        }
        double h[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const double p01 = s[hh][0] + s[hh][1];  // offset 1
            const double p23 = s[hh][2] + s[hh][3];
            h[hh] = wave_butterfly_sum(p01 + p23);  // offset 2, then 4 .. 128
        }
        const double ss = h[0] + h[1];  // offset 256
        r = (float)(1.0 / sqrt(ss / (double)k + (double)eps));
    }

    auto normed = [&](int u) __attribute__((always_inline)) {
        float4 y = xv[u];
        if (kNorm) {
            y.x = (y.x * r) * gv[u].x;
            y.y = (y.y * r) * gv[u].y;
            y.z = (y.z * r) * gv[u].z;
            y.w = (y.w * r) * gv[u].w;
        }
        return y;
    };
    float amax = 0.0f;
#pragma unroll
    for (int u = 0; u < V; ++u) {
        const float4 y = normed(u);
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(y.x), fabsf(y.y)), fmaxf(fabsf(y.z), fabsf(y.w))));
    }
    amax = wave_max(amax);
    const float scale = 127.0f / fmaxf(amax, 1e-5f);

    int sum = 0;
#pragma unroll
    for (int u = 0; u < V; ++u) {
        const int i = lane + 64 * u;
        if (i < k4) {
            const float4 y = normed(u);
            const int q0 = quant_one(y.x, scale), q1 = quant_one(y.y, scale);
            const int q2 = quant_one(y.z, scale), q3 = quant_one(y.w, scale);
            sum += q0 + q1 + q2 + q3;
            if (kPerm) {
                // within each 16 values, byte 4 j + g holds value 4 g + j
                int8_t* b = qr + ((4 * i) & ~15) + (i & 3);
                b[0] = (int8_t)q0;
                b[4] = (int8_t)q1;
                b[8] = (int8_t)q2;
                b[12] = (int8_t)q3;
            } else {
                const uint32_t packed = (uint32_t)(q0 & 0xff) | ((uint32_t)(q1 & 0xff) << 8) |
                                        ((uint32_t)(q2 & 0xff) << 16) | ((uint32_t)(q3 & 0xff) << 24);
                *reinterpret_cast<uint32_t*>(qr + 4 * i) = packed;
            }
        }
    }
    scale_out = scale;
    sum_out = wave_sum(sum);
}

template <bool kNorm, bool kPerm, int V>
__device__ __forceinline__ void wave_quant_row(const float* __restrict__ xrow, const float* __restrict__ gain,
                                               float eps, int k, int lane, int8_t* qr, float& scale_out,
                                               int& sum_out)
{
    float4 xv[V], gv[V];
    wave_quant_load<kNorm, V>(xrow, gain, k, lane, xv, gv);
    wave_quant_compute<kNorm, kPerm, V>(xv, gv, eps, k, lane, qr, scale_out, sum_out);
}

// The same quant by a 512-thread workgroup, for rows of up to 512 * NPT values:
// thread t holds x[t + 512 j] (one load per value) and forms partial t of the
// fixed order itself (ascending k); the butterfly runs over offsets 1 .. 32
// inside each wave and 64, 128, 256 across the 8 waves. Three barriers.
struct BlockQuantShared {
    double wsum_d[8];
    float wmax[8];
    int wsum[8];
};

template <bool kNorm, int NPT>
__device__ __forceinline__ void block_quant_load(const float* __restrict__ xr, const float* __restrict__ gain, int k,
                                                 float (&xv)[NPT], float (&gv)[NPT])
{
    const int t = threadIdx.x;
#pragma unroll
    for (int j = 0; j < NPT; ++j) {
        const int i = t + j * 512;
        xv[j] = i < k ? xr[i] : 0.0f;
        gv[j] = kNorm && i < k ? gain[i] : 0.0f;
    }
}

// Quantizes the loaded row into qr (natural or perm16 order; global memory or
// LDS); every thread returns s_a (scale_out) and sum(q) (sum_out). All 512
// threads of the workgroup must call it.
template <bool kNorm, bool kPerm, int NPT>
__device__ __forceinline__ void block_quant_compute(const float (&xv)[NPT], const float (&gv)[NPT], float eps, int k,
                                                    int8_t* qr, BlockQuantShared& sh, float& scale_out, int& sum_out)
{
    constexpr int kThreads = 512, kWaves = 8;
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;
    float r = 1.0f;
    if (kNorm) {
        double p = 0.0;
#pragma unroll
        for (int j = 0; j < NPT; ++j) {
            const double v = (double)xv[j];
            if (t + j * kThreads < k) p += v * v;
        }
        p = wave_butterfly_sum(p);
        if (lane == 0) sh.wsum_d[wave] = p;
        __syncthreads();
        r = (float)(1.0 / sqrt(cross_wave_sum8(sh.wsum_d) / (double)k + (double)eps));
    }

    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < NPT; ++j) {
        const float y = kNorm ? (xv[j] * r) * gv[j] : xv[j];
        if (t + j * kThreads < k) amax = fmaxf(amax, fabsf(y));
    }
    amax = wave_max(amax);
    if (lane == 0) sh.wmax[wave] = amax;
    __syncthreads();
    amax = sh.wmax[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) amax = fmaxf(amax, sh.wmax[w]);
    const float scale = 127.0f / fmaxf(amax, 1e-5f);

    int sum = 0;
#pragma unroll
    for (int j = 0; j < NPT; ++j) {
        const int i = t + j * kThreads;
        if (i < k) {
            const float y = kNorm ? (xv[j] * r) * gv[j] : xv[j];
            const int qv = quant_one(y, scale);
            sum += qv;
            // perm16: value 4 g + j' of each 16 sits at byte 4 j' + g
            qr[kPerm ? (i & ~15) + 4 * (i & 3) + ((i >> 2) & 3) : i] = (int8_t)qv;
        }
    }
    sum = wave_sum(sum);
    if (lane == 0) sh.wsum[wave] = sum;
    __syncthreads();
    int total = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) total += sh.wsum[w];
    scale_out = scale;
    sum_out = total;
}

}  // namespace bl
