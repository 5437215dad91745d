// gemv.hip -- decode BitLinear GEMV (a few tokens) on packed ternary weights.
//
// The decode step of a BitNet layer is a weight stream: every packed byte of a
// BitLinear is read once per token ("Transformer Block", Hesper API, "Memory
// Layout": ~26 MB of TQ2_0 weights per BitNet-3B layer). Each group of L lanes
// owns one output row; lane j of the group reads the row's 16-byte chunks
// j, j+L, j+2L, ... with 128-bit loads (a chunk is 64 weights), so a load
// instruction of the wave covers 64/L rows x L consecutive chunks.
//
// Unpack: a packed dword holds the codes c = t+1 of 16 consecutive weights,
// field j of byte b being weight 4b+j. (w >> 2j) & 0x03030303 therefore yields
// the codes of weights {j, 4+j, 8+j, 12+j} as four bytes, which one
// v_dot4_i32_i8 multiplies with the activations taken in the same order. The
// activations are put in that order once per lane (a 4x4 byte transpose with
// v_perm_b32), so the inner loop is 3 shifts, 4 ANDs and 4 dot4 per 16 weights.
// Since c = t + 1, sum_k t*q = sum_k c*q - sum_k q: the act_sum of the token is
// subtracted once per row. The partial sums are reduced across the L lanes with
// xor shuffles, and the group's first lane applies the single fp32 rescale.
#include "internal.h"
#include "ternary.h"
#include "wave_quant.h"

namespace bl {
namespace {

constexpr int kMaxChunksPerLane = 8;
constexpr int kFwdMaxK = 4096;         // longest row of the one-wave quant + GEMV
constexpr int kFwdBlockMaxK = 16384;   // ... and of the 512-thread form
constexpr int kFwdBlockGrid = 256;     // workgroups of the 512-thread form: one per CU

// 4x4 byte transpose of 16 activations a[0..15] (given as 4 dwords, natural
// order) into the order the shifted code masks produce: out[j] holds
// a[j], a[4+j], a[8+j], a[12+j].
__device__ __forceinline__ void permute16(const uint4 v, uint32_t out[4])
{
    const uint32_t t01lo = __builtin_amdgcn_perm(v.y, v.x, 0x05010400u);  // a0 a4 a1 a5
    const uint32_t t01hi = __builtin_amdgcn_perm(v.y, v.x, 0x07030602u);  // a2 a6 a3 a7
    const uint32_t t23lo = __builtin_amdgcn_perm(v.w, v.z, 0x05010400u);  // a8 a12 a9 a13
    const uint32_t t23hi = __builtin_amdgcn_perm(v.w, v.z, 0x07030602u);  // a10 a14 a11 a15
    out[0] = __builtin_amdgcn_perm(t23lo, t01lo, 0x05040100u);            // a0 a4 a8 a12
    out[1] = __builtin_amdgcn_perm(t23lo, t01lo, 0x07060302u);            // a1 a5 a9 a13
    out[2] = __builtin_amdgcn_perm(t23hi, t01hi, 0x05040100u);            // a2 a6 a10 a14
    out[3] = __builtin_amdgcn_perm(t23hi, t01hi, 0x07060302u);            // a3 a7 a11 a15
}

// The 64 activations of chunk `ch` of token row qr, permuted (16 dwords).
__device__ __forceinline__ void load_q_chunk(const int8_t* qr, int ch, uint32_t out[16])
{
    const uint4* src = reinterpret_cast<const uint4*>(qr + (size_t)ch * 64);
#pragma unroll
    for (int g = 0; g < 4; ++g) permute16(src[g], out + 4 * g);
}

// sum over one 16-byte chunk (64 weights) of code * activation.
__device__ __forceinline__ int dot_chunk(const uint4 w, const uint32_t* qp, int acc)
{
    const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int g = 0; g < 4; ++g) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t c = (wd[g] >> (2 * j)) & kCodeMask;
            acc = __builtin_amdgcn_sdot4((int)c, (int)qp[4 * g + j], acc, false);
        }
    }
    return acc;
}

template <int L>
__device__ __forceinline__ int group_sum(int v)
{
#pragma unroll
    for (int off = L / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

__device__ __forceinline__ float dequant(int acc, int qsum, float inv) { return (float)(acc - qsum) * inv; }

// Loads of one packed row: lane j of the group takes chunks j, j+L, ...
template <int L>
__device__ __forceinline__ void load_row(const uint8_t* rowp, bool valid, int lane_in_group, int chunks,
                                         uint4 w[kMaxChunksPerLane])
{
#pragma unroll
    for (int c = 0; c < kMaxChunksPerLane; ++c) {
        const int ch = lane_in_group + c * L;
        w[c] = (valid && ch < chunks) ? *reinterpret_cast<const uint4*>(rowp + (size_t)ch * 16) : make_uint4(0, 0, 0, 0);
    }
}

// Per-lane partial sums of code * activation over the loaded chunks, for all
// m tokens. For m == 1 the activations live in registers (qreg, loaded once
// per lane); otherwise they are read and permuted per row.
template <int L, int M>
__device__ __forceinline__ void dot_row(const uint4 w[kMaxChunksPerLane], int lane_in_group, int chunks,
                                        const int8_t* q, int k, const uint32_t (*qreg)[16], int acc[M])
{
#pragma unroll
    for (int mm = 0; mm < M; ++mm) acc[mm] = 0;
#pragma unroll
    for (int c = 0; c < kMaxChunksPerLane; ++c) {
        const int ch = lane_in_group + c * L;
        if (ch < chunks) {
            if (M == 1) {
                acc[0] = dot_chunk(w[c], qreg[c], acc[0]);
            } else {
#pragma unroll
                for (int mm = 0; mm < M; ++mm) {
                    uint32_t qp[16];
                    load_q_chunk(q + (size_t)mm * k, ch, qp);
                    acc[mm] = dot_chunk(w[c], qp, acc[mm]);
                }
            }
        }
    }
}

// load_row with a fixed number of loads: the row index is clamped to the last
// row and the chunk index to the last chunk (those lanes re-read a line that is
// being fetched anyway; dot_row_one skips their chunks), so no load sits under a
// branch and a later wait can name exactly the loads it needs.
template <int L, int CPL>
__device__ __forceinline__ void load_row_fixed(const uint8_t* rowp, int lane_in_group, int chunks,
                                               uint4 w[kMaxChunksPerLane])
{
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const int ch = min(lane_in_group + c * L, chunks - 1);
        w[c] = *reinterpret_cast<const uint4*>(rowp + (size_t)ch * 16);
    }
}

// dot_row for one token with the activations in registers.
template <int L, int CPL>
__device__ __forceinline__ int dot_row_one(const uint4 w[kMaxChunksPerLane], int lane_in_group, int chunks,
                                           const uint32_t (*qreg)[16])
{
    int acc = 0;
#pragma unroll
    for (int c = 0; c < CPL; ++c)
        if (lane_in_group + c * L < chunks) acc = dot_chunk(w[c], qreg[c], acc);
    return acc;
}

template <int L, int M>
__device__ __forceinline__ void load_qreg(const int8_t* q, int lane_in_group, int chunks, uint32_t qreg[][16])
{
    if (M != 1) return;
#pragma unroll
    for (int c = 0; c < kMaxChunksPerLane; ++c) {
        const int ch = lane_in_group + c * L;
        if (ch < chunks) load_q_chunk(q, ch, qreg[c]);
    }
}

// ---- single matrix ---------------------------------------------------------
template <int L, int M>
__global__ __launch_bounds__(64) void gemv_kernel(const uint8_t* __restrict__ packed, float w_scale,
                                                  const float* __restrict__ w_scale_ptr, int n, int k,
                                                  const int8_t* __restrict__ q, const float* __restrict__ act_scale,
                                                  const int32_t* __restrict__ act_sum,
                                                  const float* residual, float* y, int32_t* __restrict__ acc_out)
{
    constexpr int R = 64 / L;
    const int lane = threadIdx.x;
    const int g = lane / L, j = lane % L;
    const int chunks = k / 64;
    const size_t row_bytes = (size_t)k / 4;
    uint32_t qreg[M == 1 ? kMaxChunksPerLane : 1][16];
    load_qreg<L, M>(q, j, chunks, qreg);
    const float ws = w_scale_ptr ? *w_scale_ptr : w_scale;
    for (int base = blockIdx.x * R; base < n; base += gridDim.x * R) {
        const int row = base + g;
        const bool valid = row < n;
        uint4 w[kMaxChunksPerLane];
        load_row<L>(packed + (size_t)row * row_bytes, valid, j, chunks, w);
        int acc[M];
        dot_row<L, M>(w, j, chunks, q, k, qreg, acc);
#pragma unroll
        for (int mm = 0; mm < M; ++mm) acc[mm] = group_sum<L>(acc[mm]);
        if (valid && j == 0) {
#pragma unroll
            for (int mm = 0; mm < M; ++mm) {
                const int total = acc[mm] - act_sum[mm];
                const float inv = 1.0f / (act_scale[mm] * ws);
                float v = (float)total * inv;
                const size_t o = (size_t)mm * n + row;
                if (residual) v = residual[o] + v;
                y[o] = v;
                if (acc_out) acc_out[o] = total;
            }
        }
    }
}

// ---- the LM head of one token with the repetition penalty and greedy keys ---
// gemv_kernel's product with the greedy head's epilogue ("BitNet Model -
// Complete Inference Pipeline", "GPU Argmax": repetition penalty, then the
// argmax): the logit (acc - sum q) / (s_a s_w) of a column whose bit is set in
// the penalty bitmap becomes l / penalty if positive, else l * penalty; each
// workgroup writes the largest fp32 argmax key of its columns to tile_keys
// (reduced by tile_argmax_kernel), and the logits to y if given. One token:
// the weights stream at the GEMV's rate, where the MFMA skinny product uses one
// of its 32 rows.
template <int L>
__global__ __launch_bounds__(64) void head_gemv_kernel(const uint8_t* __restrict__ packed, float w_scale, int n, int k,
                                                       const int8_t* __restrict__ q,
                                                       const float* __restrict__ act_scale,
                                                       const int32_t* __restrict__ act_sum,
                                                       const uint32_t* __restrict__ pen_bits, float penalty,
                                                       float* __restrict__ y, unsigned long long* __restrict__ tile_keys)
{
    constexpr int R = 64 / L;
    const int lane = threadIdx.x;
    const int g = lane / L, j = lane % L;
    const int chunks = k / 64;
    const size_t row_bytes = (size_t)k / 4;
    uint32_t qreg[kMaxChunksPerLane][16];
    load_qreg<L, 1>(q, j, chunks, qreg);
    const float inv = 1.0f / (act_scale[0] * w_scale);
    const int qs = act_sum[0];
    unsigned long long best = 0;
    for (int base = blockIdx.x * R; base < n; base += gridDim.x * R) {
        const int row = base + g;
        const bool valid = row < n;
        uint4 w[kMaxChunksPerLane];
        load_row<L>(packed + (size_t)row * row_bytes, valid, j, chunks, w);
        int acc[1];
        dot_row<L, 1>(w, j, chunks, q, k, qreg, acc);
        acc[0] = group_sum<L>(acc[0]);
        if (valid && j == 0) {
            float v = (float)(acc[0] - qs) * inv;
            if (pen_bits && ((pen_bits[row >> 5] >> (row & 31)) & 1u)) v = v > 0.0f ? v / penalty : v * penalty;
            if (y) y[row] = v;
            const unsigned long long key = argmax_key_f32(v, row);
            best = key > best ? key : best;
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const unsigned long long other = __shfl_xor(best, off, 64);
        best = other > best ? other : best;
    }
    if (lane == 0) tile_keys[blockIdx.x] = best;
}

// head_gemv_kernel with the final RMSNorm + quant of the token fused in, one
// 512-thread workgroup per CU on a block of rpb consecutive rows: the
// workgroup quantizes x once with the workgroup quant (block_quant_compute:
// the same q, s_a and sum(q) as the quant kernel) into LDS while its first
// rows stream in; its 8 waves then take 64 rows at a time, 8 lanes per row
// (wave w rows w, w + 8, ... of each 64), with the next 64 rows' loads issued
// before the current ones' dot products. Each workgroup writes the largest
// fp32 argmax key of its rows to tile_keys[blockIdx.x].
template <int NPT>
__global__ __launch_bounds__(512) void head_block_kernel(const float* __restrict__ x, const float* __restrict__ gain,
                                                         float eps, const uint8_t* __restrict__ packed, float w_scale,
                                                         int n, int k, const uint32_t* __restrict__ pen_bits,
                                                         float penalty, float* __restrict__ y,
                                                         unsigned long long* __restrict__ tile_keys, int rpb)
{
    constexpr int L = 8;
    constexpr int CPL = NPT;  // chunks per lane: k <= 512 NPT, 8 NPT chunks over 8 lanes
    static_assert(CPL <= kMaxChunksPerLane, "row size");
    __shared__ __attribute__((aligned(16))) int8_t qs[512 * NPT];
    __shared__ BlockQuantShared sh;
    __shared__ unsigned long long wbest[8];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane / L, j = lane % L;
    const int chunks = k / 64;
    const size_t row_bytes = (size_t)k / 4;

    float xv[NPT], gv[NPT];
    block_quant_load<true, NPT>(x, gain, k, xv, gv);  // first: a wave's loads complete in issue order
    const int r1 = min(blockIdx.x * rpb + rpb, n);     // this workgroup's rows end here
    int row = blockIdx.x * rpb + wave + 8 * g;
    // slots past the block's last row load that row again (from cache), not another block's
    uint4 wa[kMaxChunksPerLane], wb[kMaxChunksPerLane];
    load_row_fixed<L, CPL>(packed + (size_t)min(row, r1 - 1) * row_bytes, j, chunks, wa);
    load_row_fixed<L, CPL>(packed + (size_t)min(row + 64, r1 - 1) * row_bytes, j, chunks, wb);
    __builtin_amdgcn_sched_barrier(0);  // keep the weight loads ahead of the quant
    float s_a;
    int qsum;
    block_quant_compute<true, false, NPT>(xv, gv, eps, k, qs, sh, s_a, qsum);  // ends with a barrier

    uint32_t qreg[kMaxChunksPerLane][16];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const int ch = j + c * L;
        if (ch < chunks) load_q_chunk(qs, ch, qreg[c]);
    }
    const float inv = 1.0f / (s_a * w_scale);
    unsigned long long best = 0;
    auto emit = [&](int acc, int r) __attribute__((always_inline)) {
        if (r < r1 && j == 0) {
            float v = (float)(acc - qsum) * inv;
            if (pen_bits && ((pen_bits[r >> 5] >> (r & 31)) & 1u)) v = v > 0.0f ? v / penalty : v * penalty;
            if (y) y[r] = v;
            const unsigned long long key = argmax_key_f32(v, r);
            best = key > best ? key : best;
        }
    };
    // two register sets in turn: the loads of the rows after next go out
    // before the dot products of the current ones
    for (;;) {
        emit(group_sum<L>(dot_row_one<L, CPL>(wa, j, chunks, qreg)), row);
        row += 64;
        if (__builtin_amdgcn_readfirstlane(row - 8 * g) >= r1) break;
        load_row_fixed<L, CPL>(packed + (size_t)min(row + 64, r1 - 1) * row_bytes, j, chunks, wa);
        emit(group_sum<L>(dot_row_one<L, CPL>(wb, j, chunks, qreg)), row);
        row += 64;
        if (__builtin_amdgcn_readfirstlane(row - 8 * g) >= r1) break;
        load_row_fixed<L, CPL>(packed + (size_t)min(row + 64, r1 - 1) * row_bytes, j, chunks, wb);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const unsigned long long other = __shfl_xor(best, off, 64);
        best = other > best ? other : best;
    }
    if (lane == 0) wbest[wave] = best;
    __syncthreads();
    if (threadIdx.x == 0) {
#pragma unroll
        for (int w = 1; w < 8; ++w) best = wbest[w] > best ? wbest[w] : best;
        tile_keys[blockIdx.x] = best;
    }
}

// ---- [RMSNorm +] quant + GEMV of one token in one launch -------------------
// Every workgroup (one wave) quantizes the whole input row itself with the
// one-wave quant (wave_quant_row: the same operations in the same order as
// the quant kernel, so every workgroup holds the same q, s_a and sum(q)) into
// LDS, and then runs its rows as gemv_kernel does. The input row is read by
// every workgroup, from L2 after the first; the workgroup's first weight rows
// are loaded right behind it, so their fetch overlaps the quant. Workgroup 0
// also writes q, s_a and sum(q) where asked.
template <int V, bool kNorm>
__global__ __launch_bounds__(64) void fwd_kernel(const float* __restrict__ x, const float* __restrict__ gain, float eps,
                                                 const uint8_t* __restrict__ packed, float w_scale, int n, int k,
                                                 float* __restrict__ y, int8_t* __restrict__ q_out,
                                                 float* __restrict__ scale_out, int32_t* __restrict__ sum_out)
{
    constexpr int L = 8, R = 64 / L;
    static_assert(64 * 4 * V <= kFwdMaxK, "row held in LDS");
    __shared__ __attribute__((aligned(16))) int8_t qs[kFwdMaxK];
    const int lane = threadIdx.x;
    const int g = lane / L, j = lane % L;
    const int chunks = k / 64;
    const size_t row_bytes = (size_t)k / 4;

    // x first: a wave's loads complete in issue order, so the quant waits
    // only for x while the weight rows stream in behind it
    float4 xv[V], gv[V];
    wave_quant_load<kNorm, V>(x, gain, k, lane, xv, gv);
    constexpr int CPL = (V + 1) / 2;  // chunks per lane: k <= 256 V
    uint4 w[kMaxChunksPerLane];
    int base = blockIdx.x * R;
    load_row_fixed<L, CPL>(packed + (size_t)min(base + g, n - 1) * row_bytes, j, chunks, w);
    __builtin_amdgcn_sched_barrier(0);  // keep the weight loads ahead of the quant
    float s_a;
    int qsum;
    wave_quant_compute<kNorm, false, V>(xv, gv, eps, k, lane, qs, s_a, qsum);
    __syncthreads();  // q complete in LDS

    uint32_t qreg[kMaxChunksPerLane][16];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const int ch = j + c * L;
        if (ch < chunks) load_q_chunk(qs, ch, qreg[c]);
    }
    if (blockIdx.x == 0) {
        if (q_out)
            for (int i = lane; i < k / 16; i += 64)
                reinterpret_cast<uint4*>(q_out)[i] = reinterpret_cast<const uint4*>(qs)[i];
        if (lane == 0) {
            if (scale_out) *scale_out = s_a;
            if (sum_out) *sum_out = qsum;
        }
    }
    const float inv = 1.0f / (s_a * w_scale);
    for (;;) {
        const int row = base + g;
        int acc = 0;
        const int acc0 = dot_row_one<L, CPL>(w, j, chunks, qreg);
        acc = group_sum<L>(acc0);
        if (row < n && j == 0) y[row] = (float)(acc - qsum) * inv;
        base += gridDim.x * R;
        if (base >= n) break;
        load_row_fixed<L, CPL>(packed + (size_t)min(base + g, n - 1) * row_bytes, j, chunks, w);
    }
}

// fwd_kernel for rows longer than one wave can hold (4096 < k <= 512 NPT): a
// 512-thread workgroup quantizes x with the workgroup quant of the quant kernel
// (block_quant_compute: same operations, same order, so every workgroup holds
// the same q, s_a and sum(q)) into LDS, then its waves run its rpb consecutive
// rows (wave w rows w, w + 8, ...) with all 64 lanes each. Optional residual
// (may alias y) and exact accumulators, as gemv_kernel.
template <int NPT, bool kNorm>
__global__ __launch_bounds__(512) void fwd_block_kernel(const float* __restrict__ x, const float* __restrict__ gain,
                                                        float eps, const uint8_t* __restrict__ packed, float w_scale,
                                                        const float* __restrict__ w_scale_ptr, int n, int k,
                                                        const float* residual, float* y, int32_t* __restrict__ acc_out,
                                                        int8_t* __restrict__ q_out, float* __restrict__ scale_out,
                                                        int32_t* __restrict__ sum_out, int rpb)
{
    constexpr int L = 64, RW = 8;                // a row per wave at a time
    constexpr int CPL = (8 * NPT + L - 1) / L;   // chunks per lane: k <= 512 NPT
    static_assert(CPL <= kMaxChunksPerLane && 512 * NPT <= kFwdBlockMaxK, "row size");
    __shared__ __attribute__((aligned(16))) int8_t qs[512 * NPT];
    __shared__ BlockQuantShared sh;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int chunks = k / 64;
    const size_t row_bytes = (size_t)k / 4;

    float xv[NPT], gv[NPT];
    block_quant_load<kNorm, NPT>(x, gain, k, xv, gv);  // first: a wave's loads complete in issue order
    uint4 w[kMaxChunksPerLane];
    const int r1 = min(blockIdx.x * rpb + rpb, n);  // this workgroup's rows end here
    int row = blockIdx.x * rpb + wave;
    load_row_fixed<L, CPL>(packed + (size_t)min(row, n - 1) * row_bytes, lane, chunks, w);
    __builtin_amdgcn_sched_barrier(0);  // keep the weight loads ahead of the quant
    float s_a;
    int qsum;
    block_quant_compute<kNorm, false, NPT>(xv, gv, eps, k, qs, sh, s_a, qsum);  // ends with a barrier

    uint32_t qreg[kMaxChunksPerLane][16];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const int ch = lane + c * L;
        if (ch < chunks) load_q_chunk(qs, ch, qreg[c]);
    }
    if (blockIdx.x == 0) {
        if (q_out)
            for (int i = threadIdx.x; i < k / 16; i += 512)
                reinterpret_cast<uint4*>(q_out)[i] = reinterpret_cast<const uint4*>(qs)[i];
        if (threadIdx.x == 0) {
            if (scale_out) *scale_out = s_a;
            if (sum_out) *sum_out = qsum;
        }
    }
    const float ws = w_scale_ptr ? *w_scale_ptr : w_scale;
    const float inv = 1.0f / (s_a * ws);
    for (;;) {
        const int acc = group_sum<L>(dot_row_one<L, CPL>(w, lane, chunks, qreg));
        if (row < r1 && lane == 0) {
            const int total = acc - qsum;
            float v = (float)total * inv;
            if (residual) v = residual[row] + v;
            y[row] = v;
            if (acc_out) acc_out[row] = total;
        }
        row += RW;
        if (row >= r1) break;
        load_row_fixed<L, CPL>(packed + (size_t)row * row_bytes, lane, chunks, w);
    }
}

// ---- several matrices of equal shape sharing the activations (q, k, v) ----
struct MultiPtrs {
    const uint8_t* p[4];
};

template <int L, int M>
__global__ __launch_bounds__(64) void gemv_multi_kernel(MultiPtrs mats, int count, const float* __restrict__ w_scale_ptr,
                                                        int n, int k, const int8_t* __restrict__ q,
                                                        const float* __restrict__ act_scale,
                                                        const int32_t* __restrict__ act_sum, float* __restrict__ y,
                                                        int ldy)
{
    constexpr int R = 64 / L;
    const int lane = threadIdx.x;
    const int g = lane / L, j = lane % L;
    const int chunks = k / 64;
    const size_t row_bytes = (size_t)k / 4;
    const int total_rows = n * count;
    uint32_t qreg[M == 1 ? kMaxChunksPerLane : 1][16];
    load_qreg<L, M>(q, j, chunks, qreg);
    for (int base = blockIdx.x * R; base < total_rows; base += gridDim.x * R) {
        const int r = base + g;
        const bool valid = r < total_rows;
        const int mat = valid ? r / n : 0;
        const int row = valid ? r - mat * n : 0;
        const uint8_t* P = mats.p[0];
#pragma unroll
        for (int i = 1; i < 4; ++i)
            if (mat == i) P = mats.p[i];
        uint4 w[kMaxChunksPerLane];
        load_row<L>(P + (size_t)row * row_bytes, valid, j, chunks, w);
        int acc[M];
        dot_row<L, M>(w, j, chunks, q, k, qreg, acc);
#pragma unroll
        for (int mm = 0; mm < M; ++mm) acc[mm] = group_sum<L>(acc[mm]);
        if (valid && j == 0) {
            const float ws = w_scale_ptr[mat];
#pragma unroll
            for (int mm = 0; mm < M; ++mm) {
                const float inv = 1.0f / (act_scale[mm] * ws);
                y[(size_t)mm * ldy + (size_t)mat * n + row] = dequant(acc[mm], act_sum[mm], inv);
            }
        }
    }
}

// ---- fused gate/up with relu(gate)^2 * up --------------------------------------
template <int L, int M>
__global__ __launch_bounds__(64) void gateup_kernel(const uint8_t* __restrict__ w_gate, float s_gate,
                                                    const uint8_t* __restrict__ w_up, float s_up,
                                                    const float* __restrict__ scale_ptr, int f, int d,
                                                    const int8_t* __restrict__ q, const float* __restrict__ act_scale,
                                                    const int32_t* __restrict__ act_sum, float* __restrict__ h,
                                                    int32_t* __restrict__ acc_gate, int32_t* __restrict__ acc_up)
{
    constexpr int R = 64 / L;
    const int lane = threadIdx.x;
    const int g = lane / L, j = lane % L;
    const int chunks = d / 64;
    const size_t row_bytes = (size_t)d / 4;
    uint32_t qreg[M == 1 ? kMaxChunksPerLane : 1][16];
    load_qreg<L, M>(q, j, chunks, qreg);
    const float sg = scale_ptr ? scale_ptr[0] : s_gate;
    const float su = scale_ptr ? scale_ptr[1] : s_up;
    for (int base = blockIdx.x * R; base < f; base += gridDim.x * R) {
        const int row = base + g;
        const bool valid = row < f;
        uint4 wg[kMaxChunksPerLane], wu[kMaxChunksPerLane];
        load_row<L>(w_gate + (size_t)row * row_bytes, valid, j, chunks, wg);
        load_row<L>(w_up + (size_t)row * row_bytes, valid, j, chunks, wu);
        int ag[M], au[M];
        dot_row<L, M>(wg, j, chunks, q, d, qreg, ag);
        dot_row<L, M>(wu, j, chunks, q, d, qreg, au);
#pragma unroll
        for (int mm = 0; mm < M; ++mm) {
            ag[mm] = group_sum<L>(ag[mm]);
            au[mm] = group_sum<L>(au[mm]);
        }
        if (valid && j == 0) {
#pragma unroll
            for (int mm = 0; mm < M; ++mm) {
                const int tg = ag[mm] - act_sum[mm], tu = au[mm] - act_sum[mm];
                const float gate = (float)tg * (1.0f / (act_scale[mm] * sg));
                const float up = (float)tu * (1.0f / (act_scale[mm] * su));
                const float gp = gate > 0.0f ? gate : 0.0f;
                const float g2 = gp * gp;
                const size_t o = (size_t)mm * f + row;
                h[o] = g2 * up;
                if (acc_gate) acc_gate[o] = tg;
                if (acc_up) acc_up[o] = tu;
            }
        }
    }
}

// gateup_kernel for one token with the [RMSNorm +] quant of its input fused
// in, one 512-thread workgroup per CU: it quantizes x once with the workgroup
// quant (block_quant_compute: the same q, s_a and sum(q) as the quant kernel)
// into LDS while its first gate and up rows stream in, and its 8 waves run its
// rpb consecutive rows, 8 lanes per row (wave w takes rows w, w + 8, ... of
// the block): x is read once per CU.
template <int NPT, bool kNorm>
__global__ __launch_bounds__(512) void fwd_gateup_block_kernel(
    const float* __restrict__ x, const float* __restrict__ gain, float eps, const uint8_t* __restrict__ w_gate,
    float s_gate, const uint8_t* __restrict__ w_up, float s_up, const float* __restrict__ scale_ptr, int f, int d,
    float* __restrict__ h, int8_t* __restrict__ q_out, float* __restrict__ scale_out, int32_t* __restrict__ sum_out,
    int32_t* __restrict__ acc_gate, int32_t* __restrict__ acc_up, int rpb)
{
    constexpr int L = 8;               // 8 lanes per row, 8 rows per wave at a time
    constexpr int CPL = NPT;           // chunks per lane: d <= 512 NPT, 8 NPT chunks over 8 lanes
    static_assert(CPL <= kMaxChunksPerLane, "row size");
    __shared__ __attribute__((aligned(16))) int8_t qs[512 * NPT];
    __shared__ BlockQuantShared sh;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane / L, j = lane % L;
    const int chunks = d / 64;
    const size_t row_bytes = (size_t)d / 4;

    float xv[NPT], gv[NPT];
    block_quant_load<kNorm, NPT>(x, gain, d, xv, gv);  // first: a wave's loads complete in issue order
    uint4 wg[kMaxChunksPerLane], wu[kMaxChunksPerLane];
    const int r1 = min(blockIdx.x * rpb + rpb, f);  // this workgroup's rows end here
    int row = blockIdx.x * rpb + wave + 8 * g;      // 8 waves x 8 groups: 64 rows at a time
    // slots past the block's last row load that row again (from cache), not another block's
    load_row_fixed<L, CPL>(w_gate + (size_t)min(row, r1 - 1) * row_bytes, j, chunks, wg);
    load_row_fixed<L, CPL>(w_up + (size_t)min(row, r1 - 1) * row_bytes, j, chunks, wu);
    __builtin_amdgcn_sched_barrier(0);  // keep the weight loads ahead of the quant
    float s_a;
    int qsum;
    block_quant_compute<kNorm, false, NPT>(xv, gv, eps, d, qs, sh, s_a, qsum);  // ends with a barrier

    uint32_t qreg[kMaxChunksPerLane][16];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const int ch = j + c * L;
        if (ch < chunks) load_q_chunk(qs, ch, qreg[c]);
    }
    if (blockIdx.x == 0) {
        if (q_out)
            for (int i = threadIdx.x; i < d / 16; i += 512)
                reinterpret_cast<uint4*>(q_out)[i] = reinterpret_cast<const uint4*>(qs)[i];
        if (threadIdx.x == 0) {
            if (scale_out) *scale_out = s_a;
            if (sum_out) *sum_out = qsum;
        }
    }
    const float sg = scale_ptr ? scale_ptr[0] : s_gate;
    const float su = scale_ptr ? scale_ptr[1] : s_up;
    for (;;) {
        const int ag = group_sum<L>(dot_row_one<L, CPL>(wg, j, chunks, qreg));
        const int au = group_sum<L>(dot_row_one<L, CPL>(wu, j, chunks, qreg));
        if (row < r1 && j == 0) {
            const int tg = ag - qsum, tu = au - qsum;
            const float gate = (float)tg * (1.0f / (s_a * sg));
            const float up = (float)tu * (1.0f / (s_a * su));
            const float gp = gate > 0.0f ? gate : 0.0f;
            const float g2 = gp * gp;
            h[row] = g2 * up;
            if (acc_gate) acc_gate[row] = tg;
            if (acc_up) acc_up[row] = tu;
        }
        // the next 64 rows of the block; the wave stops when none of its rows is left
        row += 64;
        if (__builtin_amdgcn_readfirstlane(row - 8 * g) >= r1) break;
        load_row_fixed<L, CPL>(w_gate + (size_t)min(row, r1 - 1) * row_bytes, j, chunks, wg);
        load_row_fixed<L, CPL>(w_up + (size_t)min(row, r1 - 1) * row_bytes, j, chunks, wu);
    }
}

// Lanes per row so that every lane holds at most kMaxChunksPerLane chunks.
inline int pick_lanes(int k)
{
    const int chunks = k / 64;
    if (chunks <= 8 * kMaxChunksPerLane) return 8;
    if (chunks <= 16 * kMaxChunksPerLane) return 16;
    if (chunks <= 32 * kMaxChunksPerLane) return 32;
    return 64;
}

inline int grid_for(int rows, int lanes)
{
    const int per_block = 64 / lanes;
    const int blocks = (rows + per_block - 1) / per_block;
    return blocks < 8192 ? blocks : 8192;
}

#define BL_DISPATCH_M(MACRO, LVAL)                     \
    switch (m) {                                      \
    case 1: MACRO(LVAL, 1); break;                    \
    case 2: MACRO(LVAL, 2); break;                    \
    case 3: MACRO(LVAL, 3); break;                    \
    case 4: MACRO(LVAL, 4); break;                    \
    case 5: MACRO(LVAL, 5); break;                    \
    case 6: MACRO(LVAL, 6); break;                    \
    case 7: MACRO(LVAL, 7); break;                    \
    default: MACRO(LVAL, 8); break;                   \
    }

#define BL_DISPATCH_L(MACRO)                           \
    switch (lanes) {                                  \
    case 8: BL_DISPATCH_M(MACRO, 8); break;            \
    case 16: BL_DISPATCH_M(MACRO, 16); break;          \
    case 32: BL_DISPATCH_M(MACRO, 32); break;          \
    default: BL_DISPATCH_M(MACRO, 64); break;          \
    }

}  // namespace

int gemv_rows_per_block(int k) { return 64 / pick_lanes(k); }

bool fwd_fits(int m, int k) { return m == 1 && k >= 64 && k <= kFwdMaxK && k % 64 == 0 && pick_lanes(k) == 8; }

bool fwd_block_fits(int m, int k) { return m == 1 && k > kFwdMaxK && k <= kFwdBlockMaxK && k % 64 == 0; }

int launch_gemv(const uint8_t* packed, float w_scale, const float* w_scale_ptr, int n, int k, const int8_t* q,
                const float* act_scale, const int32_t* act_sum, int m, const float* residual, float* y,
                int32_t* acc_out, hipStream_t s)
{
    const int lanes = pick_lanes(k);
    const int grid = grid_for(n, lanes);
#define BL_LAUNCH(LV, MV)                                                                                    \
    gemv_kernel<LV, MV><<<grid, 64, 0, s>>>(packed, w_scale, w_scale_ptr, n, k, q, act_scale, act_sum, residual, \
                                            y, acc_out)
    BL_DISPATCH_L(BL_LAUNCH)
#undef BL_LAUNCH
    return hipGetLastError() == hipSuccess ? BL_OK : BL_ERR_LAUNCH;
}

int launch_head_gemv(const uint8_t* packed, float w_scale, int n, int k, const int8_t* q, const float* act_scale,
                     const int32_t* act_sum, const uint32_t* pen_bits, float penalty, float* y,
                     unsigned long long* tile_keys, int max_tiles, int* tiles, hipStream_t s)
{
    const int lanes = pick_lanes(k);
    int grid = grid_for(n, lanes);
    if (grid > max_tiles) grid = max_tiles;
    *tiles = grid;
#define BL_HEAD(LV)                                                                                          \
    head_gemv_kernel<LV><<<grid, 64, 0, s>>>(packed, w_scale, n, k, q, act_scale, act_sum, pen_bits, penalty, y, \
                                             tile_keys)
    switch (lanes) {
    case 8: BL_HEAD(8); break;
    case 16: BL_HEAD(16); break;
    case 32: BL_HEAD(32); break;
    default: BL_HEAD(64); break;
    }
#undef BL_HEAD
    return hipGetLastError() == hipSuccess ? BL_OK : BL_ERR_LAUNCH;
}

int launch_head_block(const float* x, const float* gain, float eps, const uint8_t* packed, float w_scale, int n,
                      int k, const uint32_t* pen_bits, float penalty, float* y, unsigned long long* tile_keys,
                      int max_tiles, int* tiles, hipStream_t s)
{
    if (!fwd_fits(1, k) || n < 1) return BL_ERR_SHAPE;
    // one 512-thread workgroup per CU on a block of consecutive rows
    const int grid_max = max_tiles < kFwdBlockGrid ? max_tiles : kFwdBlockGrid;
    const int rpb = (n + grid_max - 1) / grid_max, grid = (n + rpb - 1) / rpb;
    *tiles = grid;
    const int npt = (k + 511) / 512;
#define BL_HEADB(NPT)                                                                                       \
    head_block_kernel<NPT><<<grid, 512, 0, s>>>(x, gain, eps, packed, w_scale, n, k, pen_bits, penalty, y, \
                                                tile_keys, rpb)
    if (npt <= 1)
        BL_HEADB(1);
    else if (npt <= 2)
        BL_HEADB(2);
    else if (npt <= 4)
        BL_HEADB(4);
    else if (npt <= 5)
        BL_HEADB(5);
    else
        BL_HEADB(8);
#undef BL_HEADB
    return hipGetLastError() == hipSuccess ? BL_OK : BL_ERR_LAUNCH;
}

int launch_fwd(const float* x, const float* gain, float eps, const uint8_t* packed, float w_scale, int n, int k,
               float* y, int8_t* q_out, float* scale_out, int32_t* sum_out, hipStream_t s)
{
    if (!fwd_fits(1, k)) return BL_ERR_SHAPE;
    const int grid = grid_for(n, 8);
    const int v = (k / 4 + 63) / 64;  // float4 chunks per lane
#define BL_FWD(V)                                                                                          \
    (gain ? fwd_kernel<V, true><<<grid, 64, 0, s>>>(x, gain, eps, packed, w_scale, n, k, y, q_out, scale_out, \
                                                     sum_out)                                              \
          : fwd_kernel<V, false><<<grid, 64, 0, s>>>(x, gain, eps, packed, w_scale, n, k, y, q_out, scale_out, \
                                                      sum_out))
    if (v <= 2)
        BL_FWD(2);
    else if (v <= 4)
        BL_FWD(4);
    else if (v <= 8)
        BL_FWD(8);
    else if (v <= 10)
        BL_FWD(10);
    else
        BL_FWD(16);
#undef BL_FWD
    return hipGetLastError() == hipSuccess ? BL_OK : BL_ERR_LAUNCH;
}

int launch_fwd_block(const float* x, const float* gain, float eps, const uint8_t* packed, float w_scale,
                     const float* w_scale_ptr, int n, int k, const float* residual, float* y, int32_t* acc_out,
                     int8_t* q_out, float* scale_out, int32_t* sum_out, hipStream_t s)
{
    if (!fwd_block_fits(1, k)) return BL_ERR_SHAPE;
    // one workgroup per CU, each on a block of consecutive rows (it reads x once)
    const int rpb = (n + kFwdBlockGrid - 1) / kFwdBlockGrid, grid = (n + rpb - 1) / rpb;
    const int per = (k + 511) / 512;  // values per thread
#define BL_FWDB(N, G)                                                                                              \
    fwd_block_kernel<N, G><<<grid, 512, 0, s>>>(x, gain, eps, packed, w_scale, w_scale_ptr, n, k, residual, y, acc_out, \
                                                q_out, scale_out, sum_out, rpb)
#define BL_FWDB_N(N)      \
    if (gain)             \
        BL_FWDB(N, true); \
    else                  \
        BL_FWDB(N, false)
    if (per <= 16) {
        BL_FWDB_N(16);
    } else if (per <= 20) {
        BL_FWDB_N(20);
    } else {
        BL_FWDB_N(32);
    }
#undef BL_FWDB_N
#undef BL_FWDB
    return hipGetLastError() == hipSuccess ? BL_OK : BL_ERR_LAUNCH;
}

int launch_gemv_multi(int count, const uint8_t* const* packed, const float* w_scale_ptr, int n_each, int k,
                      const int8_t* q, const float* act_scale, const int32_t* act_sum, int m, float* y, int ldy,
                      hipStream_t s)
{
    MultiPtrs mats{};
    for (int i = 0; i < 4; ++i) mats.p[i] = packed[i < count ? i : 0];
    const int lanes = pick_lanes(k);
    const int grid = grid_for(n_each * count, lanes);
#define BL_LAUNCH(LV, MV)                                                                                 \
    gemv_multi_kernel<LV, MV><<<grid, 64, 0, s>>>(mats, count, w_scale_ptr, n_each, k, q, act_scale, act_sum, \
                                                  y, ldy)
    BL_DISPATCH_L(BL_LAUNCH)
#undef BL_LAUNCH
    return hipGetLastError() == hipSuccess ? BL_OK : BL_ERR_LAUNCH;
}

int launch_gateup(const uint8_t* w_gate, float s_gate, const uint8_t* w_up, float s_up, const float* scale_ptr, int f,
                  int d, const int8_t* q, const float* act_scale, const int32_t* act_sum, int m, float* h,
                  int32_t* acc_gate, int32_t* acc_up, hipStream_t s)
{
    const int lanes = pick_lanes(d);
    const int grid = grid_for(f, lanes);
#define BL_LAUNCH(LV, MV)                                                                                    \
    gateup_kernel<LV, MV><<<grid, 64, 0, s>>>(w_gate, s_gate, w_up, s_up, scale_ptr, f, d, q, act_scale, act_sum, \
                                              h, acc_gate, acc_up)
    BL_DISPATCH_L(BL_LAUNCH)
#undef BL_LAUNCH
    return hipGetLastError() == hipSuccess ? BL_OK : BL_ERR_LAUNCH;
}

int launch_fwd_gateup(const float* x, const float* gain, float eps, const uint8_t* w_gate, float s_gate,
                      const uint8_t* w_up, float s_up, const float* scale_ptr, int f, int d, float* h,
                      int8_t* q_out, float* scale_out, int32_t* sum_out, int32_t* acc_gate, int32_t* acc_up,
                      hipStream_t s)
{
    if (!fwd_fits(1, d)) return BL_ERR_SHAPE;
    {
        // one 512-thread workgroup per CU on a block of consecutive rows
        const int rpb = (f + kFwdBlockGrid - 1) / kFwdBlockGrid, grid = (f + rpb - 1) / rpb;
        const int npt = (d + 511) / 512;
#define BL_FWDGUB(NPT, N)                                                                                            \
    fwd_gateup_block_kernel<NPT, N><<<grid, 512, 0, s>>>(x, gain, eps, w_gate, s_gate, w_up, s_up, scale_ptr, f, d, h, \
                                                        q_out, scale_out, sum_out, acc_gate, acc_up, rpb)
#define BL_FWDGUB_N(NPT)      \
    if (gain)                 \
        BL_FWDGUB(NPT, true); \
    else                      \
        BL_FWDGUB(NPT, false)
        if (npt <= 1) {
            BL_FWDGUB_N(1);
        } else if (npt <= 2) {
            BL_FWDGUB_N(2);
        } else if (npt <= 4) {
            BL_FWDGUB_N(4);
        } else if (npt <= 5) {
            BL_FWDGUB_N(5);
        } else {
            BL_FWDGUB_N(8);
        }
#undef BL_FWDGUB_N
#undef BL_FWDGUB
    }
    return hipGetLastError() == hipSuccess ? BL_OK : BL_ERR_LAUNCH;
}

}  // namespace bl
