// quant.hip -- fused RMSNorm + per-token absmax activation quant.
//
// RMSNorm in front of every BitLinear ("Add Support for BitNet Architecture
// Inference", candle PR 2664) and the per-token absmax int8 quantizer of the
// b1.58 method that the same PR names activation_quant. One 512-thread
// workgroup per token:
//   pass 1 (with a gain): thread t accumulates x[k]^2 in fp64 for k = t, t+512,
//          ... in ascending k (512 partials), then the partials are combined by
//          an xor-butterfly with offsets 1, 2, ..., 32 inside each wave and 64,
//          128, 256 across the 8 waves -- the fixed order every implementation
//          of this ABI uses; r = fl32(1 / sqrt(ss / k + eps)) in fp64.
//   pass 2: y = fl32(fl32(x * r) * g) and absmax over the row.
//   pass 3: s_a = fl32(127 / max(absmax, 1e-5)), q = clamp(rne(y * s_a)), sum(q).
//          Optionally q is written with each 16 values 4x4 byte-transposed, the
//          order in which the MFMA kernels unpack ternary weights (an internal
//          layout of the batched layer stream).
// Rows of up to 4096 values (8192 without a gain) run one wave per row
// (quant_act_wave_kernel); rows up to 16384 values are held in the registers
// of a 512-thread workgroup (one load per value); for longer rows passes 2 and
// 3 each re-read the row (an L2 hit after pass 1) and recompute y identically.
#include <algorithm>

#include "internal.h"
#include "prefetch.h"
#include "wave.h"
#include "wave_quant.h"

namespace bl {
namespace {

constexpr int kThreads = 512;  // = the number of RMSNorm partial sums
constexpr int kWaveRowsMin = 256;   // rows from which the one-wave-per-row kernel runs
constexpr int kMaxWaveChunks = 32;  // float4 chunks per lane it holds at most
constexpr int kWaves = kThreads / 64;


template <bool kNorm>
__device__ __forceinline__ float4 normed(const float* xr, const float* gain, float r, int i)
{
    const float4 xv = *reinterpret_cast<const float4*>(xr + i);
    if (!kNorm) return xv;
    const float4 gv = *reinterpret_cast<const float4*>(gain + i);
    float4 y;
    y.x = (xv.x * r) * gv.x;
    y.y = (xv.y * r) * gv.y;
    y.z = (xv.z * r) * gv.z;
    y.w = (xv.w * r) * gv.w;
    return y;
}

template <bool kNorm, bool kPerm>
__global__ __launch_bounds__(kThreads) void quant_act_kernel(const float* __restrict__ x,
                                                             const float* __restrict__ gain, float eps, int k,
                                                             int8_t* __restrict__ q, float* __restrict__ act_scale,
                                                             int32_t* __restrict__ act_sum)
{
    const int row = blockIdx.x;
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;
    const float* xr = x + (size_t)row * k;
    __shared__ double wsum_d[kWaves];
    __shared__ float wmax[kWaves];
    __shared__ int wsum[kWaves];

    float r = 1.0f;
    if (kNorm) {
        double p = 0.0;
        for (int i = t; i < k; i += kThreads) {
            const double v = (double)xr[i];
            p += v * v;  // exact square; any fusion rounds the same way
        }
        p = wave_butterfly_sum(p);
        if (lane == 0) wsum_d[wave] = p;
        __syncthreads();
        r = (float)(1.0 / sqrt(cross_wave_sum8(wsum_d) / (double)k + (double)eps));
    }

    float amax = 0.0f;
    for (int i = 4 * t; i < k; i += 4 * kThreads) {
        const float4 y = normed<kNorm>(xr, gain, r, i);
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(y.x), fabsf(y.y)), fmaxf(fabsf(y.z), fabsf(y.w))));
    }
    amax = wave_max(amax);
    if (lane == 0) wmax[wave] = amax;
    __syncthreads();
    amax = wmax[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) amax = fmaxf(amax, wmax[w]);
    const float scale = 127.0f / fmaxf(amax, 1e-5f);

    int sum = 0;
    int8_t* qr = q + (size_t)row * k;
    for (int i = 4 * t; i < k; i += 4 * kThreads) {
        const float4 y = normed<kNorm>(xr, gain, r, i);
        const int q0 = quant_one(y.x, scale), q1 = quant_one(y.y, scale);
        const int q2 = quant_one(y.z, scale), q3 = quant_one(y.w, scale);
        sum += q0 + q1 + q2 + q3;
        if (kPerm) {
            // within each 16 values, byte 4 j + g holds value 4 g + j (k = i + j
            // sits at (i & ~15) + 4 j + ((i >> 2) & 3))
            int8_t* b = qr + (i & ~15) + ((i >> 2) & 3);
            b[0] = (int8_t)q0;
            b[4] = (int8_t)q1;
            b[8] = (int8_t)q2;
            b[12] = (int8_t)q3;
        } else {
            const uint32_t packed = (uint32_t)(q0 & 0xff) | ((uint32_t)(q1 & 0xff) << 8) |
                                    ((uint32_t)(q2 & 0xff) << 16) | ((uint32_t)(q3 & 0xff) << 24);
            *reinterpret_cast<uint32_t*>(qr + i) = packed;
        }
    }
    sum = wave_sum(sum);
    if (lane == 0) wsum[wave] = sum;
    __syncthreads();
    if (t == 0) {
        act_scale[row] = scale;
        int total = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) total += wsum[w];
        if (act_sum) act_sum[row] = total;
    }
}

// The same three steps with the row held in registers: thread t loads x[k]
// (and g[k]) for k = t, t + 512, ... < NPT * 512 once, up front, so the row
// costs one trip to memory instead of three. The sum of squares runs over the
// same values in the same order as above, and y is recomputed identically.
// Workgroups past the last row (if any) only prefetch the weight lines of pf.
template <bool kNorm, bool kPerm, int NPT>
__global__ __launch_bounds__(kThreads) void quant_act_reg_kernel(const float* __restrict__ x,
                                                                 const float* __restrict__ gain, float eps, int k,
                                                                 int8_t* __restrict__ q, float* __restrict__ act_scale,
                                                                 int32_t* __restrict__ act_sum, int rows, Prefetch pf)
{
    const int row = blockIdx.x;
    if (row >= rows) {  // the whole workgroup: no barrier is skipped
        __shared__ uint32_t trash[64];
        prefetch_chunks(pf, row, row - rows, (int)gridDim.x - rows, kThreads, (uint32_t)(uintptr_t)&trash[0]);
        return;
    }
    __shared__ BlockQuantShared sh;
    float xv[NPT], gv[NPT];
    block_quant_load<kNorm, NPT>(x + (size_t)row * k, gain, k, xv, gv);
    float scale;
    int total;
    block_quant_compute<kNorm, kPerm, NPT>(xv, gv, eps, k, q + (size_t)row * k, sh, scale, total);
    if (threadIdx.x == 0) {
        act_scale[row] = scale;
        if (act_sum) act_sum[row] = total;
    }
}

// The norm + quant launch behind a product whose K was split over KS
// workgroups (SkinnyArgs::part): it first finishes that product for its row.
// Element i: acc = the KS partial sums of codes x q added up (exact, any order)
// minus sum(q) of the product's input, y = fl(fl(acc) * fl(1 / fl(s_a s_w))),
// x = fl(x + y) -- the operations, in the order, of the product's own
// epilogue with a residual -- and x is written back; the row then goes
// through the same register-resident norm + quant as quant_act_reg_kernel.
struct ReduceIn {
    const int32_t* part;  // [KS][rows][k]
    const int32_t* qs;    // sum(q) per row of the product's input
    const float* sa;      // s_a per row of the product's input
    const float* sw;      // the product's weight scale (device)
};

template <int NPT, int KS>
__global__ __launch_bounds__(kThreads) void quant_reduce_kernel(float* __restrict__ x, const float* __restrict__ gain,
                                                                float eps, int k, ReduceIn rin,
                                                                int8_t* __restrict__ q, float* __restrict__ act_scale,
                                                                int32_t* __restrict__ act_sum, int rows, Prefetch pf)
{
    const int row = blockIdx.x;
    if (row >= rows) {  // the whole workgroup: no barrier is skipped
        __shared__ uint32_t trash[64];
        prefetch_chunks(pf, row, row - rows, (int)gridDim.x - rows, kThreads, (uint32_t)(uintptr_t)&trash[0]);
        return;
    }
    __shared__ BlockQuantShared sh;
    const int t = threadIdx.x;
    float* xr = x + (size_t)row * k;
    float xv[NPT], gv[NPT];
    int acc[NPT];
#pragma unroll
    for (int j = 0; j < NPT; ++j) {
        const int i = min(t + j * kThreads, k - 1);
        xv[j] = xr[i];
        gv[j] = gain[i];
        acc[j] = 0;
#pragma unroll
        for (int p = 0; p < KS; ++p) acc[j] += rin.part[((size_t)p * rows + row) * k + i];
    }
    const float inv = 1.0f / (rin.sa[row] * *rin.sw);
    const int qs = rin.qs[row];
#pragma unroll
    for (int j = 0; j < NPT; ++j) {
        const int i = t + j * kThreads;
        if (i < k) {
            xv[j] = xv[j] + (float)(acc[j] - qs) * inv;
            xr[i] = xv[j];
        } else {
            xv[j] = 0.0f;
            gv[j] = 0.0f;
        }
    }
    float scale;
    int total;
    block_quant_compute<true, true, NPT>(xv, gv, eps, k, q + (size_t)row * k, sh, scale, total);
    if (t == 0) {
        act_scale[row] = scale;
        act_sum[row] = total;
    }
}

// One wave per row, for rows of up to 64 * 4 * V values (wave_quant_row).
template <bool kNorm, bool kPerm, int V>
__global__ __launch_bounds__(256) void quant_act_wave_kernel(const float* __restrict__ x,
                                                             const float* __restrict__ gain, float eps, int k, int m,
                                                             int8_t* __restrict__ q, float* __restrict__ act_scale,
                                                             int32_t* __restrict__ act_sum)
{
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= m) return;  // no barriers in this kernel
    float scale;
    int sum;
    wave_quant_row<kNorm, kPerm, V>(x + (size_t)row * k, gain, eps, k, lane, q + (size_t)row * k, scale, sum);
    if (lane == 0) {
        act_scale[row] = scale;
        if (act_sum) act_sum[row] = sum;
    }
}

template <bool kNorm, bool kPerm>
void launch_kind(const float* x, const float* gain, float eps, int m, int k, int8_t* q, float* act_scale,
                 int32_t* act_sum, hipStream_t s, const Prefetch& pf, int pf_blocks)
{
    // Many rows: one wave per row where a lane can hold its share of the row (x
    // and gains in registers) -- 4.15 vs 3.63 TB/s at 2048 x 2560. Few rows run
    // faster on a 512-thread workgroup per row (more lanes per reduction).
    int v = (k / 4 + 63) / 64;  // float4 chunks per lane
    const int wave_blocks = (m + 3) / 4;
    if (m < kWaveRowsMin) v = kMaxWaveChunks + 1;
#define BL_QWAVE(V)                                                                                         \
    quant_act_wave_kernel<kNorm, kPerm, V><<<wave_blocks, 256, 0, s>>>(x, gain, eps, k, m, q, act_scale, \
                                                                       act_sum)
    if (v <= 2) {
        BL_QWAVE(2);
        return;
    }
    if (v <= 4) {
        BL_QWAVE(4);
        return;
    }
    if (v <= 8) {
        BL_QWAVE(8);
        return;
    }
    if (v <= 10) {
        BL_QWAVE(10);
        return;
    }
    if (v <= 16) {
        BL_QWAVE(16);
        return;
    }
    if constexpr (!kNorm) {  // without gains a lane has room for twice the chunks
        if (v <= 32) {
            BL_QWAVE(32);
            return;
        }
    }
#undef BL_QWAVE
    const int per = (k + kThreads - 1) / kThreads;  // values per thread
#define BL_QREG(N)                                                                         \
    quant_act_reg_kernel<kNorm, kPerm, N><<<m + pf_blocks, kThreads, 0, s>>>(x, gain, eps, k, q, act_scale, \
                                                                              act_sum, m, pf)
    if (per <= 4)
        BL_QREG(4);
    else if (per <= 8)
        BL_QREG(8);
    else if (per <= 16)
        BL_QREG(16);
    else if (per <= 20)
        BL_QREG(20);
    else if (per <= 32)
        BL_QREG(32);
    else
        quant_act_kernel<kNorm, kPerm><<<m, kThreads, 0, s>>>(x, gain, eps, k, q, act_scale, act_sum);
#undef BL_QREG
}

// One extra workgroup per chunk of the next launch (a multiple of 8, at most
// 256); spans that are not 4-byte aligned are not prefetched.
Prefetch prefetch_plan(const Prefetch* pf, int& pf_blocks)
{
    Prefetch p = {{nullptr, nullptr}, {0u, 0u}, 0u};
    pf_blocks = 0;
    if (pf && pf->chunk && (pf->chunk & 3) == 0) {
        for (int i = 0; i < 2; ++i)
            if (pf->p[i] && pf->bytes[i] && (reinterpret_cast<uintptr_t>(pf->p[i]) & 3) == 0 && (pf->bytes[i] & 3) == 0) {
                p.p[i] = pf->p[i];
                p.bytes[i] = pf->bytes[i];
            }
        p.chunk = pf->chunk;
        const uint64_t top = std::max(p.bytes[0], p.bytes[1]);
        const uint64_t chunks = (top + p.chunk - 1) / p.chunk;
        pf_blocks = (int)std::min<uint64_t>(256, (chunks + 7) / 8 * 8);
    }
    return p;
}

}  // namespace

int launch_quant_reduce(float* x, const float* gain, float eps, int m, int k, const int32_t* part, int ksplit,
                        const int32_t* qs_in, const float* sa_in, const float* sw, int8_t* q, float* act_scale,
                        int32_t* act_sum, hipStream_t s, const Prefetch* pf)
{
    int pf_blocks;
    const Prefetch p = prefetch_plan(pf, pf_blocks);
    const ReduceIn rin = {part, qs_in, sa_in, sw};
    const int per = (k + kThreads - 1) / kThreads;  // values per thread
    const dim3 grid(m + pf_blocks);
#define BL_QRED(N, KS) \
    quant_reduce_kernel<N, KS><<<grid, kThreads, 0, s>>>(x, gain, eps, k, rin, q, act_scale, act_sum, m, p)
    if (ksplit == 2 && per <= 4)
        BL_QRED(4, 2);
    else if (ksplit == 2 && per <= 8)
        BL_QRED(8, 2);
    else if (ksplit == 2 && per <= 16)
        BL_QRED(16, 2);
    else if (ksplit == 4 && per <= 4)
        BL_QRED(4, 4);
    else if (ksplit == 4 && per <= 8)
        BL_QRED(8, 4);
    else if (ksplit == 4 && per <= 16)
        BL_QRED(16, 4);
    else
        return BL_ERR_SHAPE;
#undef BL_QRED
    return hipGetLastError() == hipSuccess ? BL_OK : BL_ERR_LAUNCH;
}

int launch_quant_act(const float* x, const float* gain, float eps, int m, int k, int8_t* q, float* act_scale,
                     int32_t* act_sum, hipStream_t s, bool perm16, const Prefetch* pf)
{
    int pf_blocks;
    const Prefetch p = prefetch_plan(pf, pf_blocks);
    if (perm16) {
        if (gain)
            launch_kind<true, true>(x, gain, eps, m, k, q, act_scale, act_sum, s, p, pf_blocks);
        else
            launch_kind<false, true>(x, gain, eps, m, k, q, act_scale, act_sum, s, p, pf_blocks);
    } else if (gain) {
        launch_kind<true, false>(x, gain, eps, m, k, q, act_scale, act_sum, s, p, pf_blocks);
    } else {
        launch_kind<false, false>(x, gain, eps, m, k, q, act_scale, act_sum, s, p, pf_blocks);
    }
    return hipGetLastError() == hipSuccess ? BL_OK : BL_ERR_LAUNCH;
}

}  // namespace bl
