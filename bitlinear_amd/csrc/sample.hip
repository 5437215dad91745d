// sample.hip -- top-k and nucleus (top-p) sampling of logits on the device
// ("BitNet Model - Complete Inference Pipeline", Hesper API, section "Text
// Generation": Top-k Sampling, Nucleus (Top-p) Sampling; sampleTopK and
// sampleNucleus take a temperature and a random number generator).
//
// The caller draws the random numbers: u[r] uniform in [0, 1), one per row.
// Tokens are taken in the pages' sorted order (descending logit, the lower
// index first among equal logits), i.e. in descending order of the 64-bit key
// (order-preserving logit bits, then 2^32 - 1 - index). Token i weighs
// e^((l_i - l_max) / T), computed in fp64 and rounded to a fixed-point integer
// with 40 fractional bits, so every sum of weights is exact and independent of
// the order in which the workgroup adds it. Then:
//   top-k   : the first min(k, n) tokens are kept;
//   nucleus : the shortest sorted prefix whose weight reaches ceil(p * Z) is
//             kept (Z the total weight);
//   draw    : r = floor(u * M), M the kept weight; the first kept token whose
//             cumulative weight exceeds r is chosen.
// Nothing is sorted. Each "first token in sorted order whose cumulative
// weight reaches a target" is found by a most-significant-digit radix
// selection over the keys, 8 bits per pass: a pass sums the (exact, int64)
// weights of the candidates per digit value in LDS, and one wave finds the
// digit at which the running total crosses the target.
//
// The exponential is written out here (fp64, valid on [-32, 0]): Cody-Waite
// range reduction x = k ln2 + r with ln2 split into a 32-significant-bit head
// (k * head is exact) and a tail, e^r from its Taylor series through r^13/13!
// by Horner's rule, then the exact scaling by 2^k. Every operation is a single
// IEEE-rounded fp64 operation (no contraction), so its value does not depend
// on the hardware's own exp.
#include "internal.h"

namespace bl {
namespace {

constexpr int kT = 1024;
constexpr int kWaves = kT / 64;

__device__ __forceinline__ double exp_neg(double x)
{
    constexpr double kLn2Head = 0x1.62e42fee00000p-1;
    constexpr double kLn2Tail = 0x1.a39ef35793c76p-33;
    constexpr double kInvLn2 = 0x1.71547652b82fep+0;
    if (x < -32.0) return 0.0;
    const double k = rint(x * kInvLn2);
    const double r = (x - k * kLn2Head) - k * kLn2Tail;
    double poly = 1.0 / 6227020800.0;  // 1 / 13!
    poly = poly * r + 1.0 / 479001600.0;
    poly = poly * r + 1.0 / 39916800.0;
    poly = poly * r + 1.0 / 3628800.0;
    poly = poly * r + 1.0 / 362880.0;
    poly = poly * r + 1.0 / 40320.0;
    poly = poly * r + 1.0 / 5040.0;
    poly = poly * r + 1.0 / 720.0;
    poly = poly * r + 1.0 / 120.0;
    poly = poly * r + 1.0 / 24.0;
    poly = poly * r + 1.0 / 6.0;
    poly = poly * r + 1.0 / 2.0;
    poly = poly * r + 1.0;
    poly = poly * r + 1.0;
    return ldexp(poly, (int)k);
}

// Sort key of token i: larger keys come first in the pages' order.
__device__ __forceinline__ unsigned long long sort_key(float l, int i)
{
    uint32_t b = __float_as_uint(l);
    if ((b << 1) == 0u) b = 0u;  // -0 sorts with +0
    const uint32_t ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    return ((unsigned long long)ord << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)i);
}

struct Shared {
    unsigned long long hist[256];
    long long red[kWaves];
    float redf[kWaves];
    int sel_digit;
    long long sel_above;
};

__device__ __forceinline__ long long wave_sum_i64(long long v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// Workgroup sum of an int64 (exact), returned to every thread.
__device__ long long block_sum_i64(long long v, Shared& sh)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    v = wave_sum_i64(v);
    __syncthreads();  // sh.red is free
    if (lane == 0) sh.red[wave] = v;
    __syncthreads();
    long long t = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) t += sh.red[w];
    return t;
}

__device__ float block_max(float v, Shared& sh)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    if (lane == 0) sh.redf[wave] = v;
    __syncthreads();
    float t = sh.redf[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) t = fmaxf(t, sh.redf[w]);
    return t;
}

// The largest key kappa whose tokens with keys >= kappa weigh at least target
// (unit weights when COUNT): the token at which the cumulative weight, in
// sorted order, first reaches target. Needs 1 <= target <= the total weight.
template <bool COUNT>
__device__ unsigned long long select_key(const float* __restrict__ l, const long long* __restrict__ w, int n,
                                         long long target, Shared& sh)
{
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    unsigned long long prefix = 0, mask = 0;
    long long above = 0;  // weight of the keys above the candidates
    for (int level = 7; level >= 0; --level) {
        const int shift = 8 * level;
        if (t < 256) sh.hist[t] = 0ull;
        __syncthreads();
        for (int i = t; i < n; i += kT) {
            const unsigned long long key = sort_key(l[i], i);
            if ((key & mask) == prefix) {
                const long long wi = COUNT ? 1 : w[i];
                if (wi != 0) atomicAdd(&sh.hist[(key >> shift) & 255ull], (unsigned long long)wi);
            }
        }
        __syncthreads();
        if (wave == 0) {
            // lane l holds digits 255 - 4 l .. 252 - 4 l (descending)
            long long b[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = (long long)sh.hist[255 - 4 * lane - j];
            const long long s4 = b[0] + b[1] + b[2] + b[3];
            long long incl = s4;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const long long v = __shfl_up(incl, off, 64);
                if (lane >= off) incl += v;
            }
            long long run = above + (incl - s4);
            int found = -1;
            long long before = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (found < 0 && run + b[j] >= target) {
                    found = 255 - 4 * lane - j;
                    before = run;
                }
                run += b[j];
            }
            const unsigned long long ballot = __ballot(found >= 0);
            const int first = ballot ? __ffsll((long long)ballot) - 1 : 0;
            if (lane == first) {
                sh.sel_digit = found < 0 ? 0 : found;  // found exists when target is in range
                sh.sel_above = before;
            }
        }
        __syncthreads();
        prefix |= (unsigned long long)sh.sel_digit << shift;
        mask |= 255ull << shift;
        above = sh.sel_above;
        __syncthreads();  // every thread has read the selection before the next clear
    }
    return prefix;
}

template <bool TOPP>
__global__ __launch_bounds__(kT) void sample_kernel(const float* __restrict__ logits, int n, int k, float p, float temp,
                                                    const double* __restrict__ u, int32_t* __restrict__ out,
                                                    long long* __restrict__ wbuf)
{
    __shared__ Shared sh;
    const int row = blockIdx.x, t = threadIdx.x;
    const float* l = logits + (size_t)row * n;
    long long* w = wbuf + (size_t)row * n;

    float lm = -INFINITY;
    for (int i = t; i < n; i += kT) lm = fmaxf(lm, l[i]);
    const float lmax = block_max(lm, sh);

    long long part = 0;
    for (int i = t; i < n; i += kT) {
        const double x = ((double)l[i] - (double)lmax) / (double)temp;
        const long long q = (long long)rint(ldexp(exp_neg(x), 40));
        w[i] = q;
        part += q;
    }
    const long long total = block_sum_i64(part, sh);  // its barriers also publish w to the workgroup

    unsigned long long kappa;
    if (TOPP) {
        const double tg = ceil((double)p * (double)total);
        long long target = tg > (double)total ? total : (long long)tg;
        if (target < 1) target = 1;
        kappa = select_key<false>(l, w, n, target, sh);
    } else {
        kappa = select_key<true>(l, w, n, k < n ? k : n, sh);
    }
    long long kept = 0;
    for (int i = t; i < n; i += kT)
        if (sort_key(l[i], i) >= kappa) kept += w[i];
    const long long mass = block_sum_i64(kept, sh);
    const double rd = floor(u[row] * (double)mass);
    const long long r = rd < 0.0 ? 0 : (rd >= (double)mass ? mass - 1 : (long long)rd);
    // the kept tokens are a prefix of the sorted order, so the first token
    // whose cumulative weight reaches r + 1 (<= mass) is a kept one
    const unsigned long long chosen = select_key<false>(l, w, n, r + 1, sh);
    if (t == 0) out[row] = (int32_t)(0xFFFFFFFFu - (uint32_t)(chosen & 0xFFFFFFFFull));
}

}  // namespace

int launch_sample(bool topp, const float* logits, int m, int n, int k, float p, float temperature, const double* u,
                  int32_t* out, long long* wbuf, hipStream_t s)
{
    if (topp)
        sample_kernel<true><<<m, kT, 0, s>>>(logits, n, k, p, temperature, u, out, wbuf);
    else
        sample_kernel<false><<<m, kT, 0, s>>>(logits, n, k, p, temperature, u, out, wbuf);
    return hipGetLastError() == hipSuccess ? BL_OK : BL_ERR_LAUNCH;
}

}  // namespace bl
