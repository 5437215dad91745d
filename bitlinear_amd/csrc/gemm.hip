// gemm.hip -- BitLinear GEMM on int8 matrix cores (prefill, batched decode, and
// the ternary LM head with a fused per-row argmax).
//
// acc[m][n] = sum_k q[m][k] * t[n][k] is a dense int8 contraction, so it runs on
// int8 MFMA with exact int32 accumulation: v_mfma_i32_16x16x64_i8 for large M,
// v_mfma_i32_32x32x32_i8 for small M (m <= 32 goes to the skinny kernels of
// skinny.hip instead). Tiles are staged through double-buffered LDS; the global
// loads run two K steps ahead (two register staging sets), so each has a whole
// step to land, and one barrier per K step separates the LDS buffers. The weights stay 2-bit packed
// in HBM and in LDS; each wave unpacks its B operand in registers: the packed dword of 16 consecutive
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
#include "ternary.h"
#include "wave.h"

namespace bl {
namespace {

constexpr int cdiv(int a, int b) { return (a + b - 1) / b; }

// Tile configuration: a BM x BN block tile, WAVES_M x WAVES_N waves, each
// owning a (BM/WAVES_M) x (BN/WAVES_N) wave tile of MT x MT MFMA tiles; BK-deep
// K steps. MT = 32: v_mfma_i32_32x32x32_i8 (32 inputs per instruction); MT = 16:
// v_mfma_i32_16x16x64_i8 (64 inputs). Either way lane l of an operand holds the
// 16 inputs 16 (l / MT) .. +15 of row / column l % MT, so the packed weight tile
// holds BK/4 bytes per row and every lane unpacks one packed dword per operand.
template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int BK_, int MT_>
struct Cfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, MT = MT_;
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    static constexpr int kThreads = 64 * WAVES_M * WAVES_N;
    static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    static constexpr int TM = WM / MT, TN = WN / MT;
    static constexpr int KT = 1024 / MT;   // inputs per MFMA
    static constexpr int NACC = MT * MT / 64;  // accumulator registers per tile and lane
    static constexpr int SA = BK + 16;     // LDS bytes per activation row (padded against bank conflicts)
    static constexpr int SB = BK / 4 + 4;  // LDS bytes per packed weight row (5 dwords: conflict-free reads)
    static constexpr int A_CHUNKS = BM * BK / 16, B_CHUNKS = BN * BK / 64;  // 16-byte chunks per K step
    static constexpr int A_PER_T = cdiv(A_CHUNKS, kThreads), B_PER_T = cdiv(B_CHUNKS, kThreads);
    static_assert(MT == 16 || MT == 32, "MFMA shape");
    static_assert(WM % MT == 0 && WN % MT == 0 && BK % 64 == 0 && BK % KT == 0, "tile shape");
};

template <int MT>
struct Mfma;
template <>
struct Mfma<32> {
    typedef v16i acc_t;
    static __device__ __forceinline__ acc_t run(v4i a, v4i b, acc_t c)
    {
        return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
    }
    // register r of lane l holds row 8 (r / 4) + 4 (l / 32) + r % 4 of the tile
    static __device__ __forceinline__ int row(int lane, int r) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }
};
template <>
struct Mfma<16> {
    typedef v4i acc_t;
    static __device__ __forceinline__ acc_t run(v4i a, v4i b, acc_t c)
    {
        return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
    }
    // register r of lane l holds row 4 (l / 16) + r of the tile
    static __device__ __forceinline__ int row(int lane, int r) { return 4 * (lane >> 4) + r; }
};

// Large M (prefill): 128 x 320 tiles -- 512 tiles for 2048 x 10240, two per CU.
// The four waves split the columns (128 x 80 each, 8 x 5 tiles of 16x16x64),
// so every packed weight column is unpacked by one wave only.
using CfgLarge = Cfg<128, 320, 1, 4, 64, 16>;
// Large M with few columns (fewer than two 128 x 320 tiles per CU, e.g. the FFN's
// down projection 2048 x 10240 -> 2560: 128 tiles): 64 x 160 tiles, 2 x 2
// waves of 32 x 80, 128-deep K steps (half the barriers per K), four times the
// tiles -- measured 69 us there, against 90 us for 128 x 160 tiles with 64-deep
// steps and 125 us for 128 x 320. Rows of K % 128 == 64 take the 64-deep form.
using CfgMid = Cfg<64, 160, 2, 2, 128, 16>;
using CfgMid64 = Cfg<128, 160, 2, 2, 64, 16>;
// Small M (up to 64 tokens; fewer run the skinny kernels): 32 x 256 tiles.
using CfgSmall = Cfg<32, 256, 1, 4, 64, 32>;

// Workgroup barrier over LDS only: this wave's LDS accesses complete, then
// s_barrier. Unlike __syncthreads it does not wait for outstanding global
// loads, so the loads issued for later K steps stay in flight across it.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt unconstrained
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// PAIR mode (the FFN's gate and up projections in one product): n is the
// number of output columns and every MT-row group of the B tile holds MT/2
// rows of W_gate followed by the same MT/2 rows of W_up, so in each MFMA
// output tile lane c (c < MT/2) holds gate and lane c + MT/2 holds up of one
// output column; the epilogue pairs them with one lane exchange and writes
// y = relu(gate)^2 * up ("Transformer Block", section "Feed-Forward Network
// (FFN)"; the fusedGateUpRelu dispatch of "Per-Layer Fused PreparedDispatch
// Refs"). acc_out / acc_up receive the exact gate / up accumulators.
template <class C, bool PAIR>
__global__ __launch_bounds__(C::kThreads) __attribute__((amdgpu_waves_per_eu(2))) void gemm_kernel(
    const uint8_t* __restrict__ packed, float w_scale, const float* __restrict__ w_scale_ptr, int n, int k,
    const int8_t* __restrict__ q, const float* __restrict__ act_scale, const int32_t* __restrict__ act_sum, int m,
    const float* residual, float* y, int ldy, int32_t* __restrict__ acc_out, unsigned long long* __restrict__ keys,
    const uint8_t* __restrict__ packed_up, float up_scale, int32_t* __restrict__ acc_up)
{
    using M = Mfma<C::MT>;
    constexpr int MT = C::MT;
    constexpr int HALF = MT / 2;
    __shared__ __attribute__((aligned(16))) uint8_t lds_a[2][C::BM * C::SA];
    __shared__ __attribute__((aligned(16))) uint8_t lds_b[2][C::BN * C::SB];
    __shared__ float lds_inv[C::BM];
    __shared__ float lds_inv_up[PAIR ? C::BM : 1];
    __shared__ int lds_qsum[C::BM];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = (wave / C::WAVES_N) * C::WM;  // wave row offset inside the block tile
    const int wn = (wave % C::WAVES_N) * C::WN;  // wave column offset
    const int n0 = blockIdx.x * C::BN;           // first B row of the block tile
    const int c0 = PAIR ? blockIdx.x * (C::BN / 2) : n0;  // first output column
    const int m0 = blockIdx.y * C::BM;
    const size_t kb = (size_t)k / 4;
    const int nk = k / C::BK;

    const float ws = w_scale_ptr ? *w_scale_ptr : w_scale;
    const float ws_up = PAIR ? (w_scale_ptr ? w_scale_ptr[1] : up_scale) : 0.0f;
    for (int r = tid; r < C::BM; r += C::kThreads) {
        const int row = m0 + r;
        lds_inv[r] = row < m ? 1.0f / (act_scale[row] * ws) : 0.0f;
        if constexpr (PAIR) lds_inv_up[r] = row < m ? 1.0f / (act_scale[row] * ws_up) : 0.0f;
        lds_qsum[r] = row < m ? act_sum[row] : 0;
    }

    // Global -> register staging of one K step: activation chunks (16 bytes of
    // one row) and packed weight chunks (16 bytes of one weight row). Rows past
    // m / n read row 0 (in bounds); their results are never stored.
    uint4 ga[2][C::A_PER_T], gb[2][C::B_PER_T];  // two K steps in flight
    // st: the staging set (a constant at every call, so the arrays stay in registers)
    auto load_global = [&](int s, int st) __attribute__((always_inline)) {
        const int k0 = s * C::BK;
#pragma unroll
        for (int c = 0; c < C::A_PER_T; ++c) {
            const int chunk = tid + c * C::kThreads;
            const int row = chunk / (C::BK / 16), kg = chunk % (C::BK / 16);
            const int grow = (chunk < C::A_CHUNKS && m0 + row < m) ? m0 + row : 0;
            ga[st][c] = *reinterpret_cast<const uint4*>(q + (size_t)grow * k + k0 + kg * 16);
        }
#pragma unroll
        for (int c = 0; c < C::B_PER_T; ++c) {
            const int chunk = tid + c * C::kThreads;
            const int row = chunk / (C::BK / 64), kg = chunk % (C::BK / 64);
            if constexpr (PAIR) {
                // B row -> (gate | up, output column); columns past n read row 0
                const int within = row % MT;
                const int col = c0 + HALF * (row / MT) + (within % HALF);
                const int gcol = (chunk < C::B_CHUNKS && col < n) ? col : 0;
                const uint8_t* src = within < HALF ? packed : packed_up;
                gb[st][c] = *reinterpret_cast<const uint4*>(src + (size_t)gcol * kb + k0 / 4 + kg * 16);
            } else {
                const int gcol = (chunk < C::B_CHUNKS && n0 + row < n) ? n0 + row : 0;
                gb[st][c] = *reinterpret_cast<const uint4*>(packed + (size_t)gcol * kb + k0 / 4 + kg * 16);
            }
        }
    };
    auto store_lds = [&](int buf, int st) __attribute__((always_inline)) {
#pragma unroll
        for (int c = 0; c < C::A_PER_T; ++c) {
            const int chunk = tid + c * C::kThreads;
            if (C::A_CHUNKS % C::kThreads == 0 || chunk < C::A_CHUNKS) {
                const int row = chunk / (C::BK / 16), kg = chunk % (C::BK / 16);
                *reinterpret_cast<uint4*>(lds_a[buf] + row * C::SA + kg * 16) = permute16(ga[st][c]);
            }
        }
#pragma unroll
        for (int c = 0; c < C::B_PER_T; ++c) {
            const int chunk = tid + c * C::kThreads;
            if (C::B_CHUNKS % C::kThreads == 0 || chunk < C::B_CHUNKS) {
                const int row = chunk / (C::BK / 64), kg = chunk % (C::BK / 64);
                uint32_t* dst = reinterpret_cast<uint32_t*>(lds_b[buf] + row * C::SB + kg * 16);
                dst[0] = gb[st][c].x;
                dst[1] = gb[st][c].y;
                dst[2] = gb[st][c].z;
                dst[3] = gb[st][c].w;
            }
        }
    };

    typename M::acc_t acc[C::TM][C::TN];
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
#pragma unroll
            for (int r = 0; r < C::NACC; ++r) acc[i][j][r] = 0;

    // One K step: loads for step s + 2 go out, the MFMAs of step s run from LDS
    // buffer s & 1, and step s + 1 (loaded one step earlier) is stored into the
    // other buffer. Steps alternate staging sets and buffers, so the loop is
    // unrolled by two with constant set indices.
    auto k_step = [&](int s, int cur) __attribute__((always_inline)) {
        if (s + 2 < nk) load_global(s + 2, cur);  // two steps ahead: a whole step to land
#pragma unroll
        for (int ks = 0; ks < C::BK / C::KT; ++ks) {
            const int kofs = ks * C::KT + (lane / MT) * 16;  // this lane's 16 K values
            v4i a[C::TM], b[C::TN];
#pragma unroll
            for (int i = 0; i < C::TM; ++i) {
                const uint4 v =
                    *reinterpret_cast<const uint4*>(lds_a[cur] + (wm + i * MT + (lane % MT)) * C::SA + kofs);
                a[i] = v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
            }
#pragma unroll
            for (int j = 0; j < C::TN; ++j) {
                const uint32_t p =
                    *reinterpret_cast<const uint32_t*>(lds_b[cur] + (wn + j * MT + (lane % MT)) * C::SB + kofs / 4);
                b[j] = ternary_codes(p);
            }
#pragma unroll
            for (int i = 0; i < C::TM; ++i)
#pragma unroll
                for (int j = 0; j < C::TN; ++j) acc[i][j] = M::run(a[i], b[j], acc[i][j]);
        }
        // the other buffer was last read before the previous barrier
        if (s + 1 < nk) store_lds(cur ^ 1, cur ^ 1);
        lds_barrier();
    };
    load_global(0, 0);
    if (nk > 1) load_global(1, 1);
    store_lds(0, 0);
    __syncthreads();
    // pairs of steps, then an odd last one: one path through the loop, so the
    // accumulators stay in place (a conditional second step made the compiler
    // copy all of them at the back edge)
    int s = 0;
    for (; s + 1 < nk; s += 2) {
        k_step(s, 0);
        k_step(s + 1, 1);
    }
    if (s < nk) k_step(s, 0);

    // epilogue: lane holds column lane % MT of each tile, register r the row
    // M::row(lane, r).
    if constexpr (PAIR) {
        // lane c < HALF: gate of column c0 + (wn + j MT) / 2 + c; lane c + HALF: its up
        const int cl = lane % MT;
        if (!acc_out && !acc_up && m0 + C::BM <= m && c0 + C::BN / 2 <= n) {
            // An interior tile that only writes y: no per-element bounds or
            // pointer checks (the lanes of gate columns store)
            float* yb = y + (size_t)(m0 + wm) * ldy + c0 + wn / 2 + cl;
#pragma unroll
            for (int i = 0; i < C::TM; ++i) {
#pragma unroll
                for (int r = 0; r < C::NACC; ++r) {
                    const int lrow = wm + i * MT + M::row(lane, r);
                    const int qs = lds_qsum[lrow];
                    const float inv_g = lds_inv[lrow];
                    const float inv_u = lds_inv_up[lrow];
                    float* yr = yb + (size_t)(i * MT + M::row(lane, r)) * ldy;
#pragma unroll
                    for (int j = 0; j < C::TN; ++j) {
                        const int total = acc[i][j][r] - qs;
                        const int other = xor_lane<HALF>(total);
                        const float gate = (float)total * inv_g;
                        const float up = (float)other * inv_u;
                        const float gp = gate > 0.0f ? gate : 0.0f;
                        const float g2 = gp * gp;
                        if (cl < HALF) yr[j * HALF] = g2 * up;
                    }
                }
            }
            return;
        }
#pragma unroll
        for (int i = 0; i < C::TM; ++i) {
#pragma unroll
            for (int r = 0; r < C::NACC; ++r) {
                const int lrow = wm + i * MT + M::row(lane, r);
                const int row = m0 + lrow;
                const int qs = lds_qsum[lrow];
                const float inv_g = lds_inv[lrow];
                const float inv_u = lds_inv_up[lrow];
#pragma unroll
                for (int j = 0; j < C::TN; ++j) {
                    const int total = acc[i][j][r] - qs;
                    const int other = xor_lane<HALF>(total);
                    const int col = c0 + (wn + j * MT) / 2 + (cl % HALF);
                    if (cl < HALF && row < m && col < n) {
                        const size_t o = (size_t)row * ldy + col;
                        const float gate = (float)total * inv_g;
                        const float up = (float)other * inv_u;
                        const float gp = gate > 0.0f ? gate : 0.0f;
                        const float g2 = gp * gp;
                        y[o] = g2 * up;
                        if (acc_out) acc_out[o] = total;
                        if (acc_up) acc_up[o] = other;
                    }
                }
            }
        }
        return;
    }
    // An interior tile that only writes y takes a path with no per-element
    // bounds or pointer checks (they are uniform there; the general path below
    // unrolls into hundreds of branches).
    if (y && !residual && !acc_out && !keys && m0 + C::BM <= m && n0 + C::BN <= n) {
        float* yb = y + (size_t)(m0 + wm) * ldy + n0 + wn + (lane % MT);
#pragma unroll
        for (int i = 0; i < C::TM; ++i) {
#pragma unroll
            for (int r = 0; r < C::NACC; ++r) {
                const int lrow = wm + i * MT + M::row(lane, r);
                const int qs = lds_qsum[lrow];
                const float inv = lds_inv[lrow];
                float* yr = yb + (size_t)(i * MT + M::row(lane, r)) * ldy;
#pragma unroll
                for (int j = 0; j < C::TN; ++j) yr[j * MT] = (float)(acc[i][j][r] - qs) * inv;
            }
        }
        return;
    }
    // General path; for the argmax, the MT lanes of a row reduce their keys.
#pragma unroll
    for (int i = 0; i < C::TM; ++i) {
#pragma unroll
        for (int r = 0; r < C::NACC; ++r) {
            const int lrow = wm + i * MT + M::row(lane, r);
            const int row = m0 + lrow;
            const int qs = lds_qsum[lrow];
            const float inv = lds_inv[lrow];
            unsigned long long best = 0;
#pragma unroll
            for (int j = 0; j < C::TN; ++j) {
                const int col = n0 + wn + j * MT + (lane % MT);
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
                        const unsigned long long key = argmax_key(total, col);
                        best = key > best ? key : best;
                    }
                }
            }
            if (keys) {
#pragma unroll
                for (int off = MT / 2; off >= 1; off >>= 1) {
                    const unsigned long long other = __shfl_xor(best, off, 64);
                    best = other > best ? other : best;
                }
                if ((lane % MT) == 0 && row < m && best != 0) atomicMax(keys + row, best);
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
    if (m <= 2 * CfgSmall::BM) {
        dim3 grid((n + CfgSmall::BN - 1) / CfgSmall::BN, (m + CfgSmall::BM - 1) / CfgSmall::BM);
        gemm_kernel<CfgSmall, false><<<grid, CfgSmall::kThreads, 0, s>>>(
            packed, w_scale, w_scale_ptr, n, k, q, act_scale, act_sum, m, residual, y, ldy, acc_out, keys, nullptr,
            0.0f, nullptr);
    } else if ((int64_t)cdiv(n, CfgLarge::BN) * cdiv(m, CfgLarge::BM) < 2 * 256 && k % CfgMid::BK == 0) {
        dim3 grid((n + CfgMid::BN - 1) / CfgMid::BN, (m + CfgMid::BM - 1) / CfgMid::BM);
        gemm_kernel<CfgMid, false><<<grid, CfgMid::kThreads, 0, s>>>(
            packed, w_scale, w_scale_ptr, n, k, q, act_scale, act_sum, m, residual, y, ldy, acc_out, keys, nullptr,
            0.0f, nullptr);
    } else if ((int64_t)cdiv(n, CfgLarge::BN) * cdiv(m, CfgLarge::BM) < 2 * 256) {
        dim3 grid((n + CfgMid64::BN - 1) / CfgMid64::BN, (m + CfgMid64::BM - 1) / CfgMid64::BM);
        gemm_kernel<CfgMid64, false><<<grid, CfgMid64::kThreads, 0, s>>>(
            packed, w_scale, w_scale_ptr, n, k, q, act_scale, act_sum, m, residual, y, ldy, acc_out, keys, nullptr,
            0.0f, nullptr);
    } else {
        dim3 grid((n + CfgLarge::BN - 1) / CfgLarge::BN, (m + CfgLarge::BM - 1) / CfgLarge::BM);
        gemm_kernel<CfgLarge, false><<<grid, CfgLarge::kThreads, 0, s>>>(
            packed, w_scale, w_scale_ptr, n, k, q, act_scale, act_sum, m, residual, y, ldy, acc_out, keys, nullptr,
            0.0f, nullptr);
    }
    if (hipGetLastError() != hipSuccess) return BL_ERR_LAUNCH;
    if (keys) {
        argmax_finish_kernel<<<(m + 255) / 256, 256, 0, s>>>(keys, m, row_argmax);
        if (hipGetLastError() != hipSuccess) return BL_ERR_LAUNCH;
    }
    return BL_OK;
}

int launch_gemm_gateup(const uint8_t* w_gate, float s_gate, const uint8_t* w_up, float s_up, const float* scale_ptr,
                       int f, int d, const int8_t* q, const float* act_scale, const int32_t* act_sum, int m, float* h,
                       int32_t* acc_gate, int32_t* acc_up, hipStream_t s)
{
    // B-row space: 2 f rows (gate and up interleaved by half tiles)
    if (m <= 2 * CfgSmall::BM) {
        dim3 grid((2 * f + CfgSmall::BN - 1) / CfgSmall::BN, (m + CfgSmall::BM - 1) / CfgSmall::BM);
        gemm_kernel<CfgSmall, true><<<grid, CfgSmall::kThreads, 0, s>>>(w_gate, s_gate, scale_ptr, f, d, q, act_scale,
                                                                        act_sum, m, nullptr, h, f, acc_gate, nullptr,
                                                                        w_up, s_up, acc_up);
    } else {
        dim3 grid((2 * f + CfgLarge::BN - 1) / CfgLarge::BN, (m + CfgLarge::BM - 1) / CfgLarge::BM);
        gemm_kernel<CfgLarge, true><<<grid, CfgLarge::kThreads, 0, s>>>(w_gate, s_gate, scale_ptr, f, d, q, act_scale,
                                                                        act_sum, m, nullptr, h, f, acc_gate, nullptr,
                                                                        w_up, s_up, acc_up);
    }
    return hipGetLastError() == hipSuccess ? BL_OK : BL_ERR_LAUNCH;
}

}  // namespace bl
