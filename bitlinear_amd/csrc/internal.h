// internal.h -- shared declarations of the HIP library (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/bitlinear.h"

namespace bl {

// Launchers (defined in the .hip files). They assume validated arguments and
// return BL_OK or BL_ERR_LAUNCH.

struct Prefetch;

// [RMSNorm +] activation quant, one workgroup per token. With perm16, q is
// written with each 16 values 4x4 byte-transposed (byte 4 j + g of a group
// holds value 4 g + j), the operand order of the skinny MFMA kernels. With pf
// (and fewer rows than the one-wave-per-row kernel takes), extra workgroups of
// the same launch pull the weight lines of pf toward the CUs for the kernel that
// follows; they change no result.
int launch_quant_act(const float* x, const float* gain, float eps, int m, int k, int8_t* q,
                     float* act_scale, int32_t* act_sum, hipStream_t s, bool perm16 = false,
                     const Prefetch* pf = nullptr);
// RMSNorm + quant (perm16 order) of x[m][k] after first finishing the K-split
// product whose ksplit (2 or 4) partial sums part[ksplit][m][k] it adds up:
// x += dequant(sum - qs_in, sa_in, *sw) in that product's epilogue order, x is
// written back, then quantized as launch_quant_act does. k <= 8192.
int launch_quant_reduce(float* x, const float* gain, float eps, int m, int k, const int32_t* part, int ksplit,
                        const int32_t* qs_in, const float* sa_in, const float* sw, int8_t* q, float* act_scale,
                        int32_t* act_sum, hipStream_t s, const Prefetch* pf);

// Weight rows read by workgroup b of a GEMV-family launch over k inputs (rows
// [b R, (b + 1) R) of the stacked matrices), and by workgroup b of a skinny
// launch over n outputs (rows [b R, (b + 1) R) of each of its matrices).
int gemv_rows_per_block(int k);
int skinny_rows_per_tile(int n, bool pair);

// [RMSNorm +] quant + GEMV of one token in one launch (fwd_fits(m, k): m == 1,
// 64 <= k <= 4096, k % 64 == 0). q_out, scale_out, sum_out may be null.
bool fwd_fits(int m, int k);
int launch_fwd(const float* x, const float* gain, float eps, const uint8_t* packed, float w_scale, int n, int k,
               float* y, int8_t* q_out, float* scale_out, int32_t* sum_out, hipStream_t s);

// The same for longer rows (fwd_block_fits(m, k): m == 1, 4096 < k <= 16384,
// k % 64 == 0), with an optional residual (may alias y) and exact accumulators.
bool fwd_block_fits(int m, int k);
int launch_fwd_block(const float* x, const float* gain, float eps, const uint8_t* packed, float w_scale,
                     const float* w_scale_ptr, int n, int k, const float* residual, float* y, int32_t* acc_out,
                     int8_t* q_out, float* scale_out, int32_t* sum_out, hipStream_t s);

// launch_gateup for one token with the [RMSNorm +] quant of x fused in (fwd_fits(1, d)).
int launch_fwd_gateup(const float* x, const float* gain, float eps, const uint8_t* w_gate, float s_gate,
                      const uint8_t* w_up, float s_up, const float* scale_ptr, int f, int d, float* h,
                      int8_t* q_out, float* scale_out, int32_t* sum_out, int32_t* acc_gate, int32_t* acc_up,
                      hipStream_t s);

// Decode GEMV, m in [1, 8]. The weight scale is read from w_scale_ptr when it
// is non-null, else w_scale is used.
int launch_gemv(const uint8_t* packed, float w_scale, const float* w_scale_ptr, int n, int k, const int8_t* q,
                const float* act_scale, const int32_t* act_sum, int m, const float* residual, float* y,
                int32_t* acc_out, hipStream_t s);

// Several GEMVs sharing one activation vector, in one launch (used for q/k/v):
// matrix j has n_rows[j] rows starting at packed[j]; outputs go to
// y + j * n_rows[0] (row stride ldy per token).
int launch_gemv_multi(int count, const uint8_t* const* packed, const float* w_scale_ptr, int n_each, int k,
                      const int8_t* q, const float* act_scale, const int32_t* act_sum, int m, float* y,
                      int ldy, hipStream_t s);

// Fused gate/up GEMV with the relu(gate)^2 * up epilogue, m in [1, 8].
int launch_gateup(const uint8_t* w_gate, float s_gate, const uint8_t* w_up, float s_up,
                  const float* scale_ptr /* [2] or null */, int f, int d, const int8_t* q,
                  const float* act_scale, const int32_t* act_sum, int m, float* h, int32_t* acc_gate,
                  int32_t* acc_up, hipStream_t s);

// MFMA GEMM. y, residual and acc_out have row stride ldy (>= n). key_ws: m
// uint64 argmax keys (only with row_argmax).
int launch_gemm(const uint8_t* packed, float w_scale, const float* w_scale_ptr, int n, int k, const int8_t* q,
                const float* act_scale, const int32_t* act_sum, int m, const float* residual, float* y, int ldy,
                int32_t* acc_out, int32_t* row_argmax, unsigned long long* key_ws, hipStream_t s);

// Persistent one-token layer stream (stream.hip). fits() tells whether the
// shapes and the device suit it; ll_region holds stream_ll_words(d, f) 64-bit
// words and ctrl two 32-bit words, all zero before the first call. With attn
// the stand-in z is unused and every layer runs single-token attention with
// RoPE and the caches of one sequence ([n_layers][heads][max_seq][hd]).
constexpr int kStreamAttnMaxChunks = 32;  // chunk partials per head the persistent attention keeps
struct StreamAttn {
    int heads, max_seq, pos;
    const float *rope_cos, *rope_sin;  // full tables [max_seq][hd / 2]
    float *k_cache, *v_cache;
    float* attn;  // [n_layers][d] or null
    void* part;   // 8-byte words [heads][kStreamAttnMaxChunks][hd + 2]
};
bool stream_persistent_fits(int m, int d, int f, const StreamAttn* attn);
size_t stream_ll_words(int d, int f);
int launch_stream_persistent(const uint8_t* weights, const float* scales, const float* gains, const float* z,
                             int n_layers, int d, int f, float eps, float* x, float* qkv, long long qkv_stride,
                             void* ll_region, uint32_t* ctrl, const StreamAttn* attn, hipStream_t s);

// Skinny MFMA products for m <= 32 tokens (skinny.hip). Without w1:
// y[m][n] = [residual +] (acc - act_sum) / (act_scale * s_w), with s_w =
// w_scale_ptr[col / n_per_scale] (stacked matrices) or w_scale0; acc0 gets the
// exact acc - act_sum; tile_keys, if set, gets per token and workgroup the
// argmax key of its columns ([m][skinny_tiles(n, false)]), reduced by
// launch_tile_argmax. With w1 (paired mode): w0 / w1 are the gate / up
// matrices (scales w_scale_ptr[0..1] or w_scale0 / w_scale1), y = relu(gate)^2
// * up, acc0 / acc1 the exact gate / up accumulators. y, residual, acc0 and
// acc1 share the row stride ldy. q is in the perm16 layout, or in natural
// order when natural_q is set.
struct SkinnyArgs {
    const uint8_t* w0 = nullptr;
    const uint8_t* w1 = nullptr;
    const float* w_scale_ptr = nullptr;
    float w_scale0 = 0.0f, w_scale1 = 0.0f;
    int n_per_scale = 1, n = 0, k = 0;
    const int8_t* q = nullptr;
    const float* act_scale = nullptr;
    const int32_t* act_sum = nullptr;
    int m = 0;
    const float* residual = nullptr;
    float* y = nullptr;
    int ldy = 0;
    int32_t* acc0 = nullptr;
    int32_t* acc1 = nullptr;
    unsigned long long* tile_keys = nullptr;
    // Repetition penalty (LM head only, not with w1 or residual): bit col of
    // pen_bits[tok * pen_words ...] set means that token's logit of column col
    // is divided by penalty if positive, else multiplied by it; y (if set)
    // receives the penalised logits and the argmax keys order fp32 values.
    const uint32_t* pen_bits = nullptr;
    int pen_words = 0;
    float penalty = 1.0f;
    // K split over workgroups (one matrix, not with w1, the head or the
    // epilogue outputs): with part set, workgroup (tile, p) of ksplit covers
    // inputs [p k / ksplit, (p + 1) k / ksplit) and writes its exact sums of
    // codes x q, sum(q) not yet removed, to part[(p m + tok) n + col]; the
    // reader adds the ksplit partials (quant_reduce).
    int32_t* part = nullptr;
    int ksplit = 1;
};
int launch_skinny(const SkinnyArgs& a, bool natural_q, hipStream_t s);
int skinny_tiles(int n, bool pair);
// The LM head of one token (m == 1) with the repetition penalty (pen_bits: the
// sequence's bitmap, or null) as a GEMV: each of the *tiles (<= max_tiles)
// workgroups writes its largest penalised fp32 argmax key to tile_keys, and
// the logits go to y if given (gemv.hip).
int launch_head_gemv(const uint8_t* packed, float w_scale, int n, int k, const int8_t* q, const float* act_scale,
                     const int32_t* act_sum, const uint32_t* pen_bits, float penalty, float* y,
                     unsigned long long* tile_keys, int max_tiles, int* tiles, hipStream_t s);
// launch_head_gemv with the final RMSNorm(gain, eps) + quant of the token x
// fused in (k <= 4096): one 512-thread workgroup per CU on a block of rows,
// each writing one key (*tiles <= min(max_tiles, 256) of them).
int launch_head_block(const float* x, const float* gain, float eps, const uint8_t* packed, float w_scale, int n,
                      int k, const uint32_t* pen_bits, float penalty, float* y, unsigned long long* tile_keys,
                      int max_tiles, int* tiles, hipStream_t s);
// Per token the column of the largest key; with hist, the chosen token is
// also appended to its sequence's history (hist[r][hist_len[r]], hist_len[r]
// + 1, while there is room).
int launch_tile_argmax(const unsigned long long* tile_keys, int tiles, int m, int32_t* idx, hipStream_t s,
                       int32_t* hist = nullptr, int stride = 0, int32_t* hist_len = nullptr);

// The FFN's gate and up projections as one MFMA GEMM over the stacked weights,
// with h[m][f] = relu(gate)^2 * up in the epilogue (any m; used above 32
// tokens). scale_ptr: [s_gate, s_up] or null (then s_gate / s_up).
int launch_gemm_gateup(const uint8_t* w_gate, float s_gate, const uint8_t* w_up, float s_up, const float* scale_ptr,
                       int f, int d, const int8_t* q, const float* act_scale, const int32_t* act_sum, int m, float* h,
                       int32_t* acc_gate, int32_t* acc_up, hipStream_t s);


// Greedy decoding around the stream (greedy.hip). penalty_words(n): 32-bit
// words of one sequence's bitmap over n vocabulary entries.
inline int penalty_words(int n) { return (n + 31) / 32; }
// The penalty bitmaps of the sequences' histories (bits: m rows of
// penalty_words(vocab) words), built by launch_embed's workgroups when given.
struct PenaltyRows {
    const int32_t* hist;
    int stride;
    const int32_t* hist_len;
    uint32_t* bits;
};
int launch_embed(const uint8_t* table, float s_e, int vocab, int d, const int32_t* tokens, int m, float* x,
                 hipStream_t s, const PenaltyRows* pen = nullptr);
int launch_penalty_bits(const int32_t* hist, int stride, const int32_t* hist_len, int n, int m, uint32_t* bits,
                        hipStream_t s);

// Top-k (topp false, k) or nucleus (topp true, p) sampling of m rows of n
// logits with the caller's uniforms u (sample.hip); workspace:
// sample_workspace_bytes(m, n) bytes, 256-aligned.
size_t sample_workspace_bytes(int m, int n);
int launch_sample(bool topp, const float* logits, int m, int n, int k, float p, float temperature, const double* u,
                  int32_t* out, void* workspace, hipStream_t s);

// Single-token attention of m sequences at position pos (attn.hip): RoPE of q
// and k from qkv rows [q | k | v] (row stride ldq), k and v appended to the
// caches ([m][heads][max_seq][hd]), attention over 0 .. pos into out (row
// stride ldo). q_rot: m * d floats; part: m * heads * attn_chunks(max_seq) *
// (hd + 2) floats.
int attn_chunks(int max_seq);
int launch_attention(const float* qkv, int ldq, int m, int d, int heads, const float* rope_cos, const float* rope_sin,
                     int max_seq, int pos, float* k_cache, float* v_cache, float* q_rot, float* part, float* out,
                     int ldo, hipStream_t s);

inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace bl
