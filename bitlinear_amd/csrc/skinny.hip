// skinny.hip -- BitLinear products for a few tokens (m <= 32) on int8 matrix
// cores: the batched-decode projections of a layer, including the fused
// gate/up with the relu(gate)^2 * up epilogue ("Transformer Block", Hesper
// API, "Forward Pass"; the FFN of "Memory Layout").
//
// At m <= 32 a projection is a pure weight stream of a few MB, so its time is
// set by how many dependent trips to memory a wave makes, not by bandwidth:
// every wave issues all of its loads at once and there is no loop-carried
// wait. A workgroup owns 16 output columns (weight rows) for all tokens, as the
// two 16-row tiles of v_mfma_i32_16x16x64_i8 (A: tokens, B: weight rows); its
// S waves split K into runs of KW super-steps of 256 inputs, and the exact
// int32 partials meet in LDS (integer sums, so the order does not matter).
//
// Within a super-step lane (n, b) = (lane % 16, lane / 16) takes inputs
// 64 b .. 64 b + 63: one 16-byte load of packed weights (64 weights of row n)
// and, per token tile, four 16-byte loads of activations. MFMA t (of 4) uses
// inputs 64 b + 16 t .. +15 of every lane; the packed dword t unpacks with
// (w >> 2 j) & 0x03030303 into the codes c = t + 1 of weights {j, 4+j, 8+j,
// 12+j} of the 16, which is why the activations come in the perm16 layout
// (each 16 values 4x4 byte-transposed). The code offset is removed with sum(q),
// and the fp32 dequant 1 / (s_a s_w) is applied per token.
#include "internal.h"

namespace bl {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
constexpr uint32_t kCodeMask = 0x03030303u;
constexpr int kMaxWaves = 16;  // waves per workgroup (K split)

__device__ __forceinline__ v4i codes(uint32_t p)
{
    return v4i{(int)(p & kCodeMask), (int)((p >> 2) & kCodeMask), (int)((p >> 4) & kCodeMask),
               (int)((p >> 6) & kCodeMask)};
}

__device__ __forceinline__ v4i as_v4i(const uint4 v) { return v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w}; }

// Operands of one super-step for one lane: the packed weights of NB rows
// (gate and up in the paired mode) and the activations of both token tiles.
template <int NB>
struct Ops {
    uint4 w[NB];
    uint4 a[2][4];
};

// PAIR = false: y = dequant(W q) (+ residual) for the rows of w0.
// PAIR = true: rows of w0 (gate) and w1 (up) together, y = relu(gate)^2 * up.
// Wave w of S takes super-steps (round * S + w) * KW + i, i < KW.
template <bool PAIR, int KW>
__global__ __launch_bounds__(64 * kMaxWaves) void skinny_kernel(const uint8_t* __restrict__ w0,
                                                                 const uint8_t* __restrict__ w1,
                                                                 const float* __restrict__ w_scale_ptr,
                                                                 int n_per_scale, int n, int k,
                                                                 const int8_t* __restrict__ q,
                                                                 const float* __restrict__ act_scale,
                                                                 const int32_t* __restrict__ act_sum, int m,
                                                                 const float* residual, float* y, int ldy)
{
    constexpr int NB = PAIR ? 2 : 1;
    extern __shared__ int red[];  // [S][NB * 8][64] int32 partials
    const int lane = threadIdx.x & 63;
    const int S = blockDim.x >> 6;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n0 = blockIdx.x * 16;
    const int ln = lane & 15, b = lane >> 4;
    const size_t kb = (size_t)k / 4;
    const int row = min(n0 + ln, n - 1);
    const uint8_t* wr0 = w0 + (size_t)row * kb + 16 * b;
    const uint8_t* wr1 = PAIR ? w1 + (size_t)row * kb + 16 * b : nullptr;
    const int8_t* ar0 = q + (size_t)min(ln, m - 1) * k + 64 * b;       // token tile 0
    const int8_t* ar1 = q + (size_t)min(16 + ln, m - 1) * k + 64 * b;  // token tile 1
    const int nss = (k + 255) / 256;                                   // the last may be partial

    v4i acc[NB][2];
#pragma unroll
    for (int i = 0; i < NB; ++i) acc[i][0] = acc[i][1] = v4i{0, 0, 0, 0};
    for (int base = wave * KW; base < nss; base += S * KW) {
        Ops<NB> o[KW];
        const uint4 z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < KW; ++i) {
            const int ss = base + i;
#pragma unroll
            for (int j = 0; j < NB; ++j) o[i].w[j] = z;
#pragma unroll
            for (int t = 0; t < 4; ++t) o[i].a[0][t] = o[i].a[1][t] = z;
            // k is a multiple of 64, so a lane's 64 inputs are all in range or none
            if (ss * 256 + 64 * b < k) {
                o[i].w[0] = *reinterpret_cast<const uint4*>(wr0 + (size_t)ss * 64);
                if (PAIR) o[i].w[NB - 1] = *reinterpret_cast<const uint4*>(wr1 + (size_t)ss * 64);
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    o[i].a[0][t] = *reinterpret_cast<const uint4*>(ar0 + (size_t)ss * 256 + 16 * t);
                    o[i].a[1][t] = *reinterpret_cast<const uint4*>(ar1 + (size_t)ss * 256 + 16 * t);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < KW; ++i) {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    const uint4& w = o[i].w[j];
                    const uint32_t p = t == 0 ? w.x : t == 1 ? w.y : t == 2 ? w.z : w.w;
                    const v4i bw = codes(p);
                    acc[j][0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(as_v4i(o[i].a[0][t]), bw, acc[j][0], 0, 0, 0);
                    acc[j][1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(as_v4i(o[i].a[1][t]), bw, acc[j][1], 0, 0, 0);
                }
            }
        }
    }

    // slot (tt, r): C row 4 b + r of token tile tt, column ln (MFMA C layout)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[(wave * NB * 8 + (j * 2 + tt) * 4 + r) * 64 + lane] = acc[j][tt][r];
    __syncthreads();

    const int col = n0 + ln;
    for (int slot = wave; slot < 8; slot += S) {
        const int tt = slot >> 2, r = slot & 3;
        const int tok = 16 * tt + 4 * b + r;
        int tot[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            int sum = 0;
            for (int w = 0; w < S; ++w) sum += red[(w * NB * 8 + j * 8 + slot) * 64 + lane];
            tot[j] = sum;
        }
        if (tok >= m || col >= n) continue;
        const int qs = act_sum[tok];
        const float sa = act_scale[tok];
        const size_t o = (size_t)tok * ldy + col;
        if (PAIR) {
            const float gate = (float)(tot[0] - qs) * (1.0f / (sa * w_scale_ptr[0]));
            const float up = (float)(tot[NB - 1] - qs) * (1.0f / (sa * w_scale_ptr[1]));
            const float gp = gate > 0.0f ? gate : 0.0f;
            const float g2 = gp * gp;
            y[o] = g2 * up;
        } else {
            const float inv = 1.0f / (sa * w_scale_ptr[col / n_per_scale]);
            float v = (float)(tot[0] - qs) * inv;
            if (residual) v = residual[o] + v;
            y[o] = v;
        }
    }
}

// Super-steps per wave and waves per workgroup for a K of nss super-steps:
// up to 16 waves of one or two super-steps each (at 16 waves a lane has 128
// VGPRs, room for two super-steps of operands); a longer K takes several rounds.
struct Split {
    int kw, waves;
};

inline Split pick_split(int k)
{
    const int nss = (k + 255) / 256;
    int kw = (nss + kMaxWaves - 1) / kMaxWaves;
    if (kw > 2) kw = 2;
    int waves = (nss + kw - 1) / kw;
    if (waves > kMaxWaves) waves = kMaxWaves;
    return {kw, waves};
}

template <bool PAIR>
int launch(const uint8_t* w0, const uint8_t* w1, const float* w_scale_ptr, int n_per_scale, int n, int k,
           const int8_t* q, const float* act_scale, const int32_t* act_sum, int m, const float* residual, float* y,
           int ldy, hipStream_t s)
{
    const Split sp = pick_split(k);
    const dim3 grid((n + 15) / 16), block(64 * sp.waves);
    const size_t lds = (size_t)sp.waves * (PAIR ? 2 : 1) * 8 * 64 * sizeof(int);
#define BL_SKINNY(KW)                                                                                              \
    skinny_kernel<PAIR, KW><<<grid, block, lds, s>>>(w0, w1, w_scale_ptr, n_per_scale, n, k, q, act_scale, act_sum, \
                                                   m, residual, y, ldy)
    if (sp.kw == 1)
        BL_SKINNY(1);
    else
        BL_SKINNY(2);
#undef BL_SKINNY
    return hipGetLastError() == hipSuccess ? BL_OK : BL_ERR_LAUNCH;
}

}  // namespace

int launch_skinny(const uint8_t* packed, const float* w_scale_ptr, int n_per_scale, int n, int k, const int8_t* q,
                  const float* act_scale, const int32_t* act_sum, int m, const float* residual, float* y, int ldy,
                  hipStream_t s)
{
    return launch<false>(packed, nullptr, w_scale_ptr, n_per_scale, n, k, q, act_scale, act_sum, m, residual, y, ldy,
                         s);
}

int launch_skinny_gateup(const uint8_t* w_gate, const uint8_t* w_up, const float* scale_ptr, int f, int d,
                         const int8_t* q, const float* act_scale, const int32_t* act_sum, int m, float* h,
                         hipStream_t s)
{
    return launch<true>(w_gate, w_up, scale_ptr, f, f, d, q, act_scale, act_sum, m, nullptr, h, f, s);
}

}  // namespace bl
