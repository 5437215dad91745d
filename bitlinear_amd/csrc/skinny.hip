// skinny.hip -- BitLinear products for a few tokens (m <= 32) on int8 matrix
// cores: the batched-decode projections, the fused gate/up with the
// relu(gate)^2 * up epilogue ("Transformer Block", Hesper API, "Forward Pass";
// the FFN of "Memory Layout") and the ternary LM head with its per-token argmax
// ("BitNet Model - Complete Inference Pipeline", Hesper API, "Greedy Decoding").
//
// At m <= 32 a projection is a pure weight stream of a few MB, so its time is
// set by how many dependent trips to memory a wave makes, not by bandwidth:
// every wave issues all of its loads at once and there is no loop-carried
// wait. All 32 tokens are the 32 rows of one v_mfma_i32_32x32x32_i8 A tile; a
// wave holds NB B tiles of 32 weight rows (consecutive rows, or the gate and
// up rows of the same 32 outputs). The S waves of a workgroup split K into runs
// of KW super-steps of 128 inputs, and their exact int32 partials meet through
// LDS integer atomics (so the order does not matter).
//
// Within a super-step lane (c, h) = (lane % 32, lane / 32) takes inputs
// 64 h .. 64 h + 63: one 16-byte load of packed weights per B tile (64 weights
// of row c) and, for MFMA t (of 4), inputs 64 h + 16 t .. +15 of token c.
// Packed dword t unpacks into the 4x4-transposed code order (ternary_codes),
// and the activations meet it in the same order -- stored that way by the
// quantizer (perm16), or transposed in registers when they come in natural
// order. The activations are loaded row-contiguous (eight lanes cover a
// token's 128 bytes, so a load touches 8 cache lines instead of 32) and pass
// through the wave's own LDS rows into operand order. The code offset is
// removed with sum(q), and the fp32 dequant 1 / (s_a s_w) is applied per
// token.
#include "internal.h"
#include "ternary.h"

namespace bl {
namespace {

constexpr int kMaxWaves = 16;  // waves per workgroup (K split)
constexpr int kPreSlots = 1;   // epilogue slots per wave whose inputs are loaded up front

// Operands of one super-step for one lane: the packed weights of its B tiles,
// and 4 x 16 bytes of the activations in the row-contiguous load order (lane l
// of load u holds bytes 16 (l % 8) .. +15 of token 8 u + l / 8).
template <int NB>
struct Ops {
    uint4 w[NB];
    uint4 a[4];
};

// Activations of one super-step in LDS, per wave: 32 token rows of 128 bytes,
// rows 144 bytes apart so the 16-byte operand reads of a wave fall in distinct
// banks.
constexpr int kRowA = 144;
constexpr int kStageA = 32 * kRowA;

// register r of lane l holds token 8 (r / 4) + 4 (l / 32) + r % 4 of the tile
__device__ __forceinline__ int tile_row(int lane, int r) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// Wave w of S takes super-steps (round * S + w) * KW + i, i < KW.
template <int NB, bool PAIR, int KW, bool NAT>
__global__ __launch_bounds__(64 * kMaxWaves) void skinny_kernel(SkinnyArgs a)
{
    static_assert(!PAIR || NB == 2, "paired mode: gate and up tiles");
    extern __shared__ int red[];  // [NB][16][64] int32 totals, then the waves' activation rows
    constexpr int COLS = PAIR ? 32 : 32 * NB;
    const int lane = threadIdx.x & 63;
    const int S = blockDim.x >> 6;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // K split: workgroup b takes part b mod ksplit of tile b / ksplit, so the
    // workgroups of one part run on the same XCDs and share its activations in L2
    const bool split = a.part != nullptr;
    const int kp = split ? (int)blockIdx.x % a.ksplit : 0;
    const int tile = split ? (int)blockIdx.x / a.ksplit : (int)blockIdx.x;
    const int kr = split ? a.k / a.ksplit : a.k;  // inputs of this workgroup, from kp * kr
    const int n0 = tile * COLS;
    const int lc = lane & 31, h = lane >> 5;
    const size_t kb = (size_t)a.k / 4;
    const uint8_t* wr[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        const int row = min(PAIR ? n0 + lc : n0 + 32 * j + lc, a.n - 1);
        wr[j] = (PAIR && j == 1 ? a.w1 : a.w0) + (size_t)row * kb + (size_t)(kp * kr) / 4 + 16 * h;
    }
    // row-contiguous activation loads: lane l of load u reads 16 bytes of token 8 u + l / 8
    const int c8 = lane & 7;
    const int8_t* ar[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
        ar[u] = a.q + (size_t)min(8 * u + (lane >> 3), a.m - 1) * a.k + (size_t)kp * kr + 16 * c8;
    int8_t* stage = reinterpret_cast<int8_t*>(red + NB * 16 * 64) + wave * kStageA;
    const int nss = (kr + 127) / 128;  // the last may be partial

    for (int i = threadIdx.x; i < NB * 16 * 64; i += blockDim.x) red[i] = 0;

    // Epilogue inputs of this wave's slots, loaded with the operands when a
    // wave has at most kPreSlots slots (16 / S): they travel in the same trip.
    int pre_qs[kPreSlots];
    float pre_sa[kPreSlots], pre_sw[kPreSlots][NB], pre_res[kPreSlots][NB];
    if (S * kPreSlots >= 16 && !split) {
#pragma unroll
        for (int i = 0; i < kPreSlots; ++i) {
            const int r = min(wave + S * i, 15);  // slots past 15 load slot 15 again (unused)
            const int tok = tile_row(lane, r);
            const int tokc = min(tok, a.m - 1);
            pre_qs[i] = a.act_sum[tokc];
            pre_sa[i] = a.act_scale[tokc];
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const int col = PAIR ? n0 + lc : n0 + 32 * j + lc;
                if (PAIR)
                    pre_sw[i][j] = a.w_scale_ptr ? a.w_scale_ptr[j] : (j == 0 ? a.w_scale0 : a.w_scale1);
                else
                    pre_sw[i][j] = a.w_scale_ptr ? a.w_scale_ptr[min(col, a.n - 1) / a.n_per_scale] : a.w_scale0;
                pre_res[i][j] = (!PAIR && a.residual && a.y && tok < a.m && col < a.n)
                                    ? a.residual[(size_t)tok * a.ldy + col]
                                    : 0.0f;
            }
        }
    }

    v16i acc[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][r] = 0;
    for (int base = wave * KW; base < nss; base += S * KW) {
        Ops<NB> o[KW];
        const uint4 z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < KW; ++i) {
            const int ss = base + i;
#pragma unroll
            for (int j = 0; j < NB; ++j) o[i].w[j] = z;
#pragma unroll
            for (int u = 0; u < 4; ++u) o[i].a[u] = z;
            // kr is a multiple of 64, so a lane's 64 weights are all in range or none
            if (ss * 128 + 64 * h < kr) {
#pragma unroll
                for (int j = 0; j < NB; ++j) o[i].w[j] = *reinterpret_cast<const uint4*>(wr[j] + (size_t)ss * 32);
            }
            if (ss * 128 + 16 * c8 < kr) {
#pragma unroll
                for (int u = 0; u < 4; ++u) o[i].a[u] = *reinterpret_cast<const uint4*>(ar[u] + (size_t)ss * 128);
            }
        }
#pragma unroll
        for (int i = 0; i < KW; ++i) {
            // through this wave's LDS rows into the operand order: lane (c, h)
            // takes bytes 64 h + 16 t .. +15 of token c for MFMA t. A wave's LDS
            // accesses complete in order, so the rows are reused without a wait.
#pragma unroll
            for (int u = 0; u < 4; ++u)
                *reinterpret_cast<uint4*>(stage + (8 * u + (lane >> 3)) * kRowA + 16 * c8) = o[i].a[u];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const uint4 raw = *reinterpret_cast<const uint4*>(stage + lc * kRowA + 64 * h + 16 * t);
                const v4i av = as_v4i(NAT ? permute16(raw) : raw);
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    const uint4& w = o[i].w[j];
                    const uint32_t p = t == 0 ? w.x : t == 1 ? w.y : t == 2 ? w.z : w.w;
                    acc[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, ternary_codes(p), acc[j], 0, 0, 0);
                }
            }
        }
    }

    __syncthreads();  // the zeroed totals are visible
    if (wave * KW < nss) {
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) atomicAdd(&red[(j * 16 + r) * 64 + lane], acc[j][r]);
    }
    __syncthreads();

    if (split) {  // uniform: the part's raw totals, no epilogue
        for (int r = wave; r < 16; r += S) {
            const int tok = tile_row(lane, r);
            const int col = n0 + lc;
            if (tok < a.m && col < a.n)
                a.part[((size_t)kp * a.m + tok) * a.n + col] = red[r * 64 + lane];
        }
        return;
    }
    const int tiles = gridDim.x;
    // Epilogue of slot r (C row 4 b + r of the tile, see tile_row) with the
    // slot's per-token and per-column inputs.
    auto emit = [&](int r, int qs, float sa, const float* sw, const float* res) __attribute__((always_inline)) {
        const int tok = tile_row(lane, r);
        int tot[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j) tot[j] = red[(j * 16 + r) * 64 + lane] - qs;
        if (PAIR) {
            const int col = n0 + lc;
            if (tok < a.m && col < a.n) {
                const float gate = (float)tot[0] * (1.0f / (sa * sw[0]));
                const float up = (float)tot[1] * (1.0f / (sa * sw[1]));
                const float gp = gate > 0.0f ? gate : 0.0f;
                const float g2 = gp * gp;
                const size_t o = (size_t)tok * a.ldy + col;
                a.y[o] = g2 * up;
                if (a.acc0) a.acc0[o] = tot[0];
                if (a.acc1) a.acc1[o] = tot[1];
            }
        } else {
            unsigned long long best = 0;
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const int col = n0 + 32 * j + lc;
                if (tok < a.m && col < a.n) {
                    const size_t o = (size_t)tok * a.ldy + col;
                    unsigned long long key;
                    if (a.pen_bits) {
                        // the repetition penalty on this token's logit, then an fp32 key
                        float v = (float)tot[j] * (1.0f / (sa * sw[j]));
                        if ((a.pen_bits[(size_t)tok * a.pen_words + (col >> 5)] >> (col & 31)) & 1u)
                            v = v > 0.0f ? v / a.penalty : v * a.penalty;
                        if (a.y) a.y[o] = v;
                        key = argmax_key_f32(v, col);
                    } else {
                        if (a.y) {
                            float v = (float)tot[j] * (1.0f / (sa * sw[j]));
                            if (a.residual) v = res[j] + v;
                            a.y[o] = v;
                        }
                        key = argmax_key(tot[j], col);
                    }
                    if (a.acc0) a.acc0[o] = tot[j];
                    best = key > best ? key : best;
                }
            }
            if (a.tile_keys) {  // uniform branch: every lane takes part in the exchange
#pragma unroll
                for (int off = 16; off >= 1; off >>= 1) {
                    const unsigned long long other = __shfl_xor(best, off, 64);
                    best = other > best ? other : best;
                }
                if (lc == 0 && tok < a.m) a.tile_keys[(size_t)tok * tiles + blockIdx.x] = best;
            }
        }
    };
    // the slot's inputs: sum(q), s_a of its token, the weight scale and the
    // residual of its columns
    auto fetch = [&](int r, int& qs, float& sa, float* sw, float* res) __attribute__((always_inline)) {
        const int tok = tile_row(lane, r);
        const int tokc = min(tok, a.m - 1);
        qs = a.act_sum[tokc];
        sa = a.act_scale[tokc];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const int col = PAIR ? n0 + lc : n0 + 32 * j + lc;
            if (PAIR)
                sw[j] = a.w_scale_ptr ? a.w_scale_ptr[j] : (j == 0 ? a.w_scale0 : a.w_scale1);
            else
                sw[j] = a.w_scale_ptr ? a.w_scale_ptr[min(col, a.n - 1) / a.n_per_scale] : a.w_scale0;
            res[j] = (!PAIR && a.residual && a.y && tok < a.m && col < a.n) ? a.residual[(size_t)tok * a.ldy + col]
                                                                          : 0.0f;
        }
    };
    if (S * kPreSlots >= 16) {
        // at most kPreSlots slots per wave: their inputs were loaded with the
        // operands (pre_* below), one trip to memory fewer
#pragma unroll
        for (int i = 0; i < kPreSlots; ++i)
            if (wave + S * i < 16) emit(wave + S * i, pre_qs[i], pre_sa[i], pre_sw[i], pre_res[i]);
    } else {
        for (int r = wave; r < 16; r += S) {
            int qs;
            float sa, sw[NB], res[NB];
            fetch(r, qs, sa, sw, res);
            emit(r, qs, sa, sw, res);
        }
    }
}

// Per token, the largest of the workgroups' keys; its low word gives the column.
// With hist, the chosen column also joins the token's history.
__global__ __launch_bounds__(256) void tile_argmax_kernel(const unsigned long long* __restrict__ keys, int tiles,
                                                          int32_t* __restrict__ idx, int32_t* __restrict__ hist,
                                                          int stride, int32_t* __restrict__ hist_len)
{
    __shared__ unsigned long long wbest[4];
    const int tok = blockIdx.x;
    unsigned long long best = 0;
    for (int i = threadIdx.x; i < tiles; i += 256) {
        const unsigned long long v = keys[(size_t)tok * tiles + i];
        best = v > best ? v : best;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const unsigned long long other = __shfl_xor(best, off, 64);
        best = other > best ? other : best;
    }
    if ((threadIdx.x & 63) == 0) wbest[threadIdx.x >> 6] = best;
    __syncthreads();
    if (threadIdx.x == 0) {
#pragma unroll
        for (int w = 1; w < 4; ++w) best = wbest[w] > best ? wbest[w] : best;
        const int32_t c = (int32_t)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFull));
        idx[tok] = c;
        if (hist && hist_len) {
            const int len = hist_len[tok];
            if (len >= 0 && len < stride) {
                hist[(size_t)tok * stride + len] = c;
                hist_len[tok] = len + 1;
            }
        }
    }
}

struct Split {
    int kw, waves;
};

// Super-steps per wave (1, 2 or 4) and waves per workgroup for nss
// super-steps: up to max_waves waves of as few super-steps as fit in one round,
// at most kw_max each (the
// operands of a lane at 16 waves must fit its 128 VGPRs); a longer K takes
// several rounds.
inline Split pick_split(int k, int kw_max, int max_waves)
{
    const int nss = (k + 127) / 128;
    int kw = (nss + max_waves - 1) / max_waves;
    if (kw == 3) kw = 4;
    if (kw > kw_max) kw = kw_max;
    if (kw < 1) kw = 1;
    int waves = (nss + kw - 1) / kw;
    if (waves > max_waves) waves = max_waves;
    return {kw, waves};
}

template <int NB, bool PAIR, bool NAT>
int launch_nb(const SkinnyArgs& a, hipStream_t s)
{
    constexpr int cols = PAIR ? 32 : 32 * NB;
    constexpr int kw_max = NB == 1 ? 4 : 2;
    const int tiles = (a.n + cols - 1) / cols;
    const int parts = a.part ? a.ksplit : 1;
    // More workgroups than CUs (the LM head): at most 8 waves each, so two fit
    // on a CU (LDS and registers) and the grid runs in fewer rounds.
    const Split sp = pick_split(a.k / parts, kw_max, tiles * parts > 256 ? kMaxWaves / 2 : kMaxWaves);
    const dim3 grid(tiles * parts), block(64 * sp.waves);
    const size_t lds = (size_t)NB * 16 * 64 * sizeof(int) + (size_t)sp.waves * kStageA;
    if (sp.kw == 1)
        skinny_kernel<NB, PAIR, 1, NAT><<<grid, block, lds, s>>>(a);
    else if (sp.kw == 2)
        skinny_kernel<NB, PAIR, 2, NAT><<<grid, block, lds, s>>>(a);
    else
        skinny_kernel<NB, PAIR, kw_max, NAT><<<grid, block, lds, s>>>(a);
    return hipGetLastError() == hipSuccess ? BL_OK : BL_ERR_LAUNCH;
}

// Two 32-row tiles per wave where that still leaves a workgroup per CU.
inline bool two_tiles(int n) { return n >= 64 * 256; }

}  // namespace

int skinny_tiles(int n, bool pair)
{
    if (pair) return (n + 31) / 32;
    return two_tiles(n) ? (n + 63) / 64 : (n + 31) / 32;
}

int skinny_rows_per_tile(int n, bool pair) { return pair || !two_tiles(n) ? 32 : 64; }

int launch_skinny(const SkinnyArgs& a, bool natural_q, hipStream_t s)
{
    if (a.part) {  // K split: one matrix of 32-row tiles, each part a whole number of 64-input chunks
        if (a.w1 || two_tiles(a.n) || a.ksplit < 1 || a.k % (64 * a.ksplit) != 0) return BL_ERR_SHAPE;
        return natural_q ? launch_nb<1, false, true>(a, s) : launch_nb<1, false, false>(a, s);
    }
    if (a.w1) return natural_q ? launch_nb<2, true, true>(a, s) : launch_nb<2, true, false>(a, s);
    if (two_tiles(a.n)) return natural_q ? launch_nb<2, false, true>(a, s) : launch_nb<2, false, false>(a, s);
    return natural_q ? launch_nb<1, false, true>(a, s) : launch_nb<1, false, false>(a, s);
}

int launch_tile_argmax(const unsigned long long* tile_keys, int tiles, int m, int32_t* idx, hipStream_t s,
                       int32_t* hist, int stride, int32_t* hist_len)
{
    tile_argmax_kernel<<<m, 256, 0, s>>>(tile_keys, tiles, idx, hist, stride, hist_len);
    return hipGetLastError() == hipSuccess ? BL_OK : BL_ERR_LAUNCH;
}

}  // namespace bl
