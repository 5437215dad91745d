// greedy.hip -- the device side of greedy decoding around the BitLinear stream
// ("BitNet Model - Complete Inference Pipeline", Hesper API):
//   - the ternary embedding lookup (section "Architecture": the embedding layer
//     is TQ2_0 quantized; "Memory Footprint": 50000 x 2560 x 0.25 bytes);
//   - the repetition penalty of section "GPU Argmax" (repetitionPenaltyKernel,
//     appendPenaltyToken, gpuArgmaxWithPenalty): the previous tokens of each
//     sequence are set in a per-sequence bitmap over the vocabulary, which the
//     LM-head epilogue (skinny.hip) reads to penalise those logits before it
//     forms its argmax keys, so penalty and argmax take one pass and no logits
//     need to be written. The embedding launch of a greedy step builds these
//     bitmaps too, and the argmax key reduction (skinny.hip) appends the
//     chosen token to each sequence's history on the device.
#include "internal.h"

namespace bl {
namespace {

constexpr int kEmbedThreads = 256;

// Per sequence r: clear its bitmap of words 32-bit words, then set the bit of
// every history id in [0, n) (hist_len clamped to [0, stride]). All threads
// of the workgroup (kThreads of them) take part.
template <int kThreads>
__device__ __forceinline__ void penalty_bits_row(int r, const int32_t* __restrict__ hist, int stride,
                                                 const int32_t* __restrict__ hist_len, int n, int words,
                                                 uint32_t* __restrict__ bits)
{
    uint32_t* b = bits + (size_t)r * words;
    for (int i = threadIdx.x; i < words; i += kThreads) b[i] = 0u;
    __syncthreads();  // the clears are done before any bit is set
    int len = stride > 0 ? hist_len[r] : 0;
    len = len < 0 ? 0 : (len > stride ? stride : len);
    for (int i = threadIdx.x; i < len; i += kThreads) {
        const int v = hist[(size_t)r * stride + i];
        if (v >= 0 && v < n) atomicOr(b + (v >> 5), 1u << (v & 31));
    }
}

// Row tokens[r] of the packed table, dequantized: t / s_e, i.e. +inv, -inv or
// +0 with inv = fl32(1 / s_e) (the correctly rounded quotient of +-1 by s_e is
// +-inv). Each thread expands one 16-byte chunk (64 values) per step. A token
// outside [0, vocab) gives a zero row. With bits, the same workgroup also
// builds sequence r's penalty bitmap (the history does not change before the
// LM head reads it), which saves the head a launch.
__global__ __launch_bounds__(kEmbedThreads) void embed_kernel(const uint8_t* __restrict__ table, float s_e,
                                                              int vocab, int d, const int32_t* __restrict__ tokens,
                                                              float* __restrict__ x, const int32_t* __restrict__ hist,
                                                              int stride, const int32_t* __restrict__ hist_len,
                                                              int words, uint32_t* __restrict__ bits)
{
    const int r = blockIdx.x;
    const int tok = tokens[r];
    float* xr = x + (size_t)r * d;
    const int chunks = d / 64;
    if (bits) penalty_bits_row<kEmbedThreads>(r, hist, stride, hist_len, vocab, words, bits);
    if (tok < 0 || tok >= vocab) {
        for (int i = threadIdx.x; i < d / 4; i += kEmbedThreads)
            reinterpret_cast<float4*>(xr)[i] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        return;
    }
    const float inv = 1.0f / s_e;
    const uint4* row = reinterpret_cast<const uint4*>(table + (size_t)tok * (d / 4));
    for (int c = threadIdx.x; c < chunks; c += kEmbedThreads) {
        const uint4 p = row[c];
        const uint32_t w[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            // dword q holds values 16 q .. 16 q + 15 of the chunk, value i at bits 2 i
            float v[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const uint32_t code = (w[q] >> (2 * i)) & 3u;  // code 3 never appears (treated as 0)
                v[i] = code == 2u ? inv : (code == 0u ? -inv : 0.0f);
            }
            float4* dst = reinterpret_cast<float4*>(xr + 64 * c + 16 * q);
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
        }
    }
}

__global__ __launch_bounds__(256) void penalty_bits_kernel(const int32_t* __restrict__ hist, int stride,
                                                           const int32_t* __restrict__ hist_len, int n, int words,
                                                           uint32_t* __restrict__ bits)
{
    penalty_bits_row<256>(blockIdx.x, hist, stride, hist_len, n, words, bits);
}

}  // namespace

int launch_embed(const uint8_t* table, float s_e, int vocab, int d, const int32_t* tokens, int m, float* x,
                 hipStream_t s, const PenaltyRows* pen)
{
    embed_kernel<<<m, kEmbedThreads, 0, s>>>(table, s_e, vocab, d, tokens, x, pen ? pen->hist : nullptr,
                                             pen ? pen->stride : 0, pen ? pen->hist_len : nullptr,
                                             penalty_words(vocab), pen ? pen->bits : nullptr);
    return hipGetLastError() == hipSuccess ? BL_OK : BL_ERR_LAUNCH;
}

int launch_penalty_bits(const int32_t* hist, int stride, const int32_t* hist_len, int n, int m, uint32_t* bits,
                        hipStream_t s)
{
    penalty_bits_kernel<<<m, 256, 0, s>>>(hist, stride, hist_len, n, penalty_words(n), bits);
    return hipGetLastError() == hipSuccess ? BL_OK : BL_ERR_LAUNCH;
}

}  // namespace bl
