// attn.hip -- single-token attention with a KV cache and rotary position
// embedding, for the decode step ("BitNet Model - Complete Inference
// Pipeline", Hesper API: "KV Cache State", forwardSingleToken; "Transformer
// Block": "Forward Pass with KV Cache", forwardWithCache; Config: numHeads,
// headDim, ropeBase).
//
// Head h of H owns columns h hd .. h hd + hd - 1 of q, k and v (hd = d / H).
//   rope_append : q and k of the new token turn pairwise -- (x[2i], x[2i+1]) by
//                 pos * theta_i, with the caller's fp32 cos / sin table row of
//                 position pos, four products then a difference and a sum,
//                 each rounded on its own -- and k, v join the caches at
//                 position pos; the rotated q goes to a scratch vector.
//   attention   : per (sequence, head), positions 0 .. pos split into chunks of
//                 256, one workgroup per chunk: one thread per position forms
//                 the score q . k_j / sqrt(hd), the chunk's maximum and sum of
//                 e^(s_j - max) and, one thread per head element, the weighted
//                 sum of v_j; the partials (max, sum, hd sums) go to a workspace.
//   combine     : per (sequence, head) the chunks are merged with the usual
//                 rescaling by e^(max_c - max) and divided by the total.
// Scores, exponentials and sums are fp32 (the hardware's expf); the result
// differs from an exact evaluation by a small multiple of fp32 rounding.
#include "internal.h"

namespace bl {
namespace {

constexpr int kChunk = 256;  // positions per attention workgroup (one per thread)

__global__ void rope_append_kernel(const float* __restrict__ qkv, int ldq, int d, int heads, int hd,
                                   const float* __restrict__ cos_row, const float* __restrict__ sin_row, int max_seq,
                                   int pos, float* __restrict__ q_rot, float* __restrict__ k_cache,
                                   float* __restrict__ v_cache)
{
    const int r = blockIdx.x / heads, h = blockIdx.x % heads;
    const float* src = qkv + (size_t)r * ldq + h * hd;
    const size_t cache_row = ((size_t)(r * heads + h) * max_seq + pos) * hd;
    for (int i = threadIdx.x; i < hd / 2; i += blockDim.x) {
        const float c = cos_row[i], s = sin_row[i];
        {
            const float a = src[2 * i], b = src[2 * i + 1];
            const float ac = a * c, bs = b * s, as = a * s, bc = b * c;
            q_rot[(size_t)r * d + h * hd + 2 * i] = ac - bs;
            q_rot[(size_t)r * d + h * hd + 2 * i + 1] = as + bc;
        }
        {
            const float a = src[d + 2 * i], b = src[d + 2 * i + 1];
            const float ac = a * c, bs = b * s, as = a * s, bc = b * c;
            k_cache[cache_row + 2 * i] = ac - bs;
            k_cache[cache_row + 2 * i + 1] = as + bc;
        }
        v_cache[cache_row + 2 * i] = src[2 * d + 2 * i];
        v_cache[cache_row + 2 * i + 1] = src[2 * d + 2 * i + 1];
    }
}

__device__ __forceinline__ float block_reduce(float v, float* red, bool is_max)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const float o = __shfl_xor(v, off, 64);
        v = is_max ? fmaxf(v, o) : v + o;
    }
    __syncthreads();  // red is free
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float t = red[0];
    for (int w = 1; w < (int)(blockDim.x >> 6); ++w) t = is_max ? fmaxf(t, red[w]) : t + red[w];
    return t;
}

// Partials of chunk c of (sequence r, head h): [max, sum, acc[hd]].
__global__ __launch_bounds__(kChunk) void attn_partial_kernel(const float* __restrict__ q_rot, int d, int heads,
                                                              int hd, const float* __restrict__ k_cache,
                                                              const float* __restrict__ v_cache, int max_seq, int pos,
                                                              int chunks, float* __restrict__ part)
{
    __shared__ float e[kChunk];
    __shared__ float red[kChunk / 64];
    __shared__ float qs[256];
    const int rh = blockIdx.x / chunks, c = blockIdx.x % chunks;
    const int r = rh / heads, h = rh % heads;
    const int t = threadIdx.x;
    const int j0 = c * kChunk, cnt = min(kChunk, pos + 1 - j0);
    const size_t base = (size_t)rh * max_seq * hd;
    for (int i = t; i < hd; i += kChunk) qs[i] = q_rot[(size_t)r * d + h * hd + i];
    __syncthreads();
    const float scale = 1.0f / sqrtf((float)hd);
    float s = -INFINITY;
    if (t < cnt) {
        const float* kj = k_cache + base + (size_t)(j0 + t) * hd;
        float dot = 0.0f;
        for (int i = 0; i < hd; i += 4) {
            const float4 kv = *reinterpret_cast<const float4*>(kj + i);
            dot += qs[i] * kv.x;
            dot += qs[i + 1] * kv.y;
            dot += qs[i + 2] * kv.z;
            dot += qs[i + 3] * kv.w;
        }
        s = dot * scale;
    }
    const float mx = block_reduce(s, red, true);
    const float ev = t < cnt ? expf(s - mx) : 0.0f;
    e[t] = ev;
    const float sum = block_reduce(ev, red, false);  // its barriers also publish e[]
    float* out = part + (size_t)blockIdx.x * (hd + 2);
    for (int i = t; i < hd; i += kChunk) {
        float acc = 0.0f;
        const float* vi = v_cache + base + (size_t)j0 * hd + i;
        for (int j = 0; j < cnt; ++j) acc += e[j] * vi[(size_t)j * hd];
        out[2 + i] = acc;
    }
    if (t == 0) {
        out[0] = mx;
        out[1] = sum;
    }
}

__global__ void attn_combine_kernel(const float* __restrict__ part, int heads, int hd, int chunks,
                                    float* __restrict__ out, int ldo)
{
    const int rh = blockIdx.x, r = rh / heads, h = rh % heads;
    const float* p = part + (size_t)rh * chunks * (hd + 2);
    float mx = -INFINITY;
    for (int c = 0; c < chunks; ++c) mx = fmaxf(mx, p[(size_t)c * (hd + 2)]);
    float den = 0.0f;
    for (int c = 0; c < chunks; ++c) den += p[(size_t)c * (hd + 2) + 1] * expf(p[(size_t)c * (hd + 2)] - mx);
    for (int i = threadIdx.x; i < hd; i += blockDim.x) {
        float acc = 0.0f;
        for (int c = 0; c < chunks; ++c) acc += p[(size_t)c * (hd + 2) + 2 + i] * expf(p[(size_t)c * (hd + 2)] - mx);
        out[(size_t)r * ldo + h * hd + i] = acc / den;
    }
}

}  // namespace

int attn_chunks(int max_seq) { return (max_seq + kChunk - 1) / kChunk; }

int launch_attention(const float* qkv, int ldq, int m, int d, int heads, const float* rope_cos, const float* rope_sin,
                     int max_seq, int pos, float* k_cache, float* v_cache, float* q_rot, float* part, float* out,
                     int ldo, hipStream_t s)
{
    const int hd = d / heads;
    const int half = hd / 2;
    rope_append_kernel<<<m * heads, half < 64 ? 64 : (half < 128 ? 128 : 256), 0, s>>>(
        qkv, ldq, d, heads, hd, rope_cos + (size_t)pos * half, rope_sin + (size_t)pos * half, max_seq, pos, q_rot,
        k_cache, v_cache);
    if (hipGetLastError() != hipSuccess) return BL_ERR_LAUNCH;
    const int chunks = (pos + 1 + kChunk - 1) / kChunk;
    attn_partial_kernel<<<m * heads * chunks, kChunk, 0, s>>>(q_rot, d, heads, hd, k_cache, v_cache, max_seq, pos,
                                                              chunks, part);
    if (hipGetLastError() != hipSuccess) return BL_ERR_LAUNCH;
    attn_combine_kernel<<<m * heads, 128, 0, s>>>(part, heads, hd, chunks, out, ldo);
    return hipGetLastError() == hipSuccess ? BL_OK : BL_ERR_LAUNCH;
}

}  // namespace bl
