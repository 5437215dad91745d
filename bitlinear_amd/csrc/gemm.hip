// gemm.hip -- BitLinear GEMM on int8 matrix cores (prefill, batched decode, and
// the ternary LM head with a fused per-row argmax).
//
// acc[m][n] = sum_k q[m][k] * t[n][k] is a dense int8 contraction, so it runs on
// v_mfma_i32_32x32x32_i8 (32x32 output tile, 32-deep K per instruction, exact
// int32 accumulation). The weights stay 2-bit packed in HBM and in LDS; each
// wave unpacks its B operand in registers: the packed dword of 16 consecutive
// weights of column n gives, through (w >> 2j) & 0x03030303 for j = 0..3, the
// codes c = t + 1 of weights {j, 4+j, 8+j, 12+j}. The activation tile is staged
// in LDS already transposed into that order (4x4 byte transpose per 16 bytes),
// so the K index of every (lane, byte) slot agrees between the two operands.
// The correction sum_k t q = sum_k c q - sum_k q and the fp32 rescale
// 1/(s_a s_w) are applied per row in the epilogue.
//
// Greedy decoding takes the argmax of the last logits ("BitNet Model - Complete
// Inference Pipeline", Hesper API, "Greedy Decoding"); the page's argmaxKernel
// reduces over the vocabulary and returns only the index ("GPU Argmax"). Here the
// argmax is fused into the LM-head epilogue: every wave reduces its columns to
// one 64-bit key per row, (acc + 2^31) << 32 | (2^32 - 1 - n), and merges it with
// a 64-bit atomicMax, so equal accumulators resolve to the lowest n.
#include "internal.h"

namespace bl {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr uint32_t kCodeMask = 0x03030303u;
constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kThreads = 256;
constexpr int kWaveM = 64, kWaveN = 64;       // wave tile
constexpr int kTM = kWaveM / 32, kTN = kWaveN / 32;
constexpr int kStrideA = kBK + 16;             // bytes per A row in LDS (padding against bank conflicts)
constexpr int kStrideB = kBK / 4 + 4;          // bytes per packed B row in LDS

__device__ __forceinline__ uint4 permute16(const uint4 v)
{
    const uint32_t t01lo = __builtin_amdgcn_perm(v.y, v.x, 0x05010400u);
    const uint32_t t01hi = __builtin_amdgcn_perm(v.y, v.x, 0x07030602u);
    const uint32_t t23lo = __builtin_amdgcn_perm(v.w, v.z, 0x05010400u);
    const uint32_t t23hi = __builtin_amdgcn_perm(v.w, v.z, 0x07030602u);
    uint4 o;
    o.x = __builtin_amdgcn_perm(t23lo, t01lo, 0x05040100u);
    o.y = __builtin_amdgcn_perm(t23lo, t01lo, 0x07060302u);
    o.z = __builtin_amdgcn_perm(t23hi, t01hi, 0x05040100u);
    o.w = __builtin_amdgcn_perm(t23hi, t01hi, 0x07060302u);
    return o;
}

__global__ __launch_bounds__(kThreads) void gemm_kernel(const uint8_t* __restrict__ packed, float w_scale,
                                                        const float* __restrict__ w_scale_ptr, int n, int k,
                                                        const int8_t* __restrict__ q,
                                                        const float* __restrict__ act_scale,
                                                        const int32_t* __restrict__ act_sum, int m,
                                                        const float* residual, float* y, int ldy,
                                                        int32_t* __restrict__ acc_out,
                                                        unsigned long long* __restrict__ keys)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds_a[kBM * kStrideA];
    __shared__ __attribute__((aligned(16))) uint8_t lds_b[kBN * kStrideB];
    __shared__ float lds_inv[kBM];
    __shared__ int lds_qsum[kBM];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = (wave >> 1) * kWaveM;   // wave row offset inside the block tile
    const int wn = (wave & 1) * kWaveN;    // wave column offset
    const int n0 = blockIdx.x * kBN;
    const int m0 = blockIdx.y * kBM;
    const size_t kb = (size_t)k / 4;

    const float ws = w_scale_ptr ? *w_scale_ptr : w_scale;
    if (tid < kBM) {
        const int row = m0 + tid;
        lds_inv[tid] = row < m ? 1.0f / (act_scale[row] * ws) : 0.0f;
        lds_qsum[tid] = row < m ? act_sum[row] : 0;
    }

    v16i acc[kTM][kTN];
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int j = 0; j < kTN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

    for (int k0 = 0; k0 < k; k0 += kBK) {
        // stage A: kBM rows x 64 bytes = 512 chunks of 16 bytes, 2 per thread
#pragma unroll
        for (int c = 0; c < (kBM * kBK / 16) / kThreads; ++c) {
            const int chunk = tid + c * kThreads;
            const int row = chunk >> 2, kg = chunk & 3;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (m0 + row < m) v = *reinterpret_cast<const uint4*>(q + (size_t)(m0 + row) * k + k0 + kg * 16);
            *reinterpret_cast<uint4*>(lds_a + row * kStrideA + kg * 16) = permute16(v);
        }
        // stage B: kBN packed rows x 16 bytes
        if (tid < kBN) {
            const int col = n0 + tid;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (col < n) v = *reinterpret_cast<const uint4*>(packed + (size_t)col * kb + k0 / 4);
            uint32_t* dst = reinterpret_cast<uint32_t*>(lds_b + tid * kStrideB);
            dst[0] = v.x;
            dst[1] = v.y;
            dst[2] = v.z;
            dst[3] = v.w;
        }
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < kBK / 32; ++ks) {
            const int kofs = ks * 32 + (lane >> 5) * 16;  // this lane's 16 K values
            v4i a[kTM], b[kTN];
#pragma unroll
            for (int i = 0; i < kTM; ++i) {
                const uint4 v =
                    *reinterpret_cast<const uint4*>(lds_a + (wm + i * 32 + (lane & 31)) * kStrideA + kofs);
                a[i] = v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
            }
#pragma unroll
            for (int j = 0; j < kTN; ++j) {
                const uint32_t p =
                    *reinterpret_cast<const uint32_t*>(lds_b + (wn + j * 32 + (lane & 31)) * kStrideB + kofs / 4);
                b[j] = v4i{(int)(p & kCodeMask), (int)((p >> 2) & kCodeMask), (int)((p >> 4) & kCodeMask),
                           (int)((p >> 6) & kCodeMask)};
            }
#pragma unroll
            for (int i = 0; i < kTM; ++i)
#pragma unroll
                for (int j = 0; j < kTN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        __syncthreads();
    }

    // epilogue: lane holds column (lane & 31) of each 32x32 tile; register r
    // holds row 8 (r / 4) + 4 (lane / 32) + (r % 4).
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int lrow = wm + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            const int row = m0 + lrow;
            const int qs = lds_qsum[lrow];
            const float inv = lds_inv[lrow];
            unsigned long long best = 0;
#pragma unroll
            for (int j = 0; j < kTN; ++j) {
                const int col = n0 + wn + j * 32 + (lane & 31);
                const int total = acc[i][j][r] - qs;
                if (row < m && col < n) {
                    const size_t o = (size_t)row * ldy + col;
                    if (y) {
                        float v = (float)total * inv;
                        if (residual) v = residual[o] + v;
                        y[o] = v;
                    }
                    if (acc_out) acc_out[o] = total;
                    if (keys) {
                        const unsigned long long key =
                            ((unsigned long long)((uint32_t)total ^ 0x80000000u) << 32) |
                            (unsigned long long)(0xFFFFFFFFu - (uint32_t)col);
                        best = key > best ? key : best;
                    }
                }
            }
            if (keys) {
#pragma unroll
                for (int off = 16; off >= 1; off >>= 1) {
                    const unsigned long long other = __shfl_xor(best, off, 64);
                    best = other > best ? other : best;
                }
                if ((lane & 31) == 0 && row < m && best != 0) atomicMax(keys + row, best);
            }
        }
    }
}

__global__ void argmax_init_kernel(unsigned long long* keys, int m)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < m) keys[i] = 0ull;
}

__global__ void argmax_finish_kernel(const unsigned long long* keys, int m, int32_t* idx)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < m) idx[i] = (int32_t)(0xFFFFFFFFu - (uint32_t)(keys[i] & 0xFFFFFFFFull));
}

__global__ void relu2_mul_kernel(const float* __restrict__ gate, const float* __restrict__ up, int64_t count,
                                 float* __restrict__ h)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += (int64_t)gridDim.x * blockDim.x) {
        const float g = gate[i] > 0.0f ? gate[i] : 0.0f;
        const float g2 = g * g;
        h[i] = g2 * up[i];
    }
}

}  // namespace

int launch_gemm(const uint8_t* packed, float w_scale, const float* w_scale_ptr, int n, int k, const int8_t* q,
                const float* act_scale, const int32_t* act_sum, int m, const float* residual, float* y, int ldy,
                int32_t* acc_out, int32_t* row_argmax, unsigned long long* key_ws, hipStream_t s)
{
    unsigned long long* keys = row_argmax ? key_ws : nullptr;
    if (keys) {
        argmax_init_kernel<<<(m + 255) / 256, 256, 0, s>>>(keys, m);
        if (hipGetLastError() != hipSuccess) return BL_ERR_LAUNCH;
    }
    dim3 grid((n + kBN - 1) / kBN, (m + kBM - 1) / kBM);
    gemm_kernel<<<grid, kThreads, 0, s>>>(packed, w_scale, w_scale_ptr, n, k, q, act_scale, act_sum, m, residual, y,
                                          ldy, acc_out, keys);
    if (hipGetLastError() != hipSuccess) return BL_ERR_LAUNCH;
    if (keys) {
        argmax_finish_kernel<<<(m + 255) / 256, 256, 0, s>>>(keys, m, row_argmax);
        if (hipGetLastError() != hipSuccess) return BL_ERR_LAUNCH;
    }
    return BL_OK;
}

int launch_relu2_mul(const float* gate, const float* up, int64_t count, float* h, hipStream_t s)
{
    int64_t blocks = (count + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    relu2_mul_kernel<<<(int)blocks, 256, 0, s>>>(gate, up, count, h);
    return hipGetLastError() == hipSuccess ? BL_OK : BL_ERR_LAUNCH;
}

}  // namespace bl
