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
// selection over the keys in six digits (12, 10, 10, 11, 11, 10 bits): a
// level sums the (exact, int64) weights and the counts of the candidates per
// digit value in LDS; each wave totals a block of digit values, and one wave
// finds the block and then the digit at which the running total crosses the
// target (lane prefix sums by DPP row shifts and broadcasts; the sums are
// integers, so their order does not matter). The first level's sums come
// from the launch that computes the weights (up to 64 workgroups per row, each
// on a slice, their histograms and totals added into the row's by exact
// integer atomics) and serve both selections; the
// twelve-bit first digit (sign, exponent, three mantissa bits of the logit)
// spreads logits of a few units over many bins, which keeps the LDS atomics
// of that pass from piling onto a handful of addresses. Once a level's
// candidates number at most 2048, the pass that reads them also copies their
// keys and weights into LDS, and the deeper levels (and the second selection,
// while its candidates are among them) run from that list; the first
// selection's second level copies every token whose first digit is at least
// the chosen one, when they fit, so that the draw (always a kept token) runs
// from the list too. The kept weight M
// is read off the first selection (the weight above the kept boundary plus
// the boundary token's own).
//
// The exponential is written out here (fp64, valid on [-32, 0]): Cody-Waite
// range reduction x = k ln2 + r with ln2 split into a 32-significant-bit head
// (k * head is exact) and a tail, e^r from its Taylor series through r^13/13!
// by Horner's rule, then the exact scaling by 2^k. Every operation is a single
// IEEE-rounded fp64 operation (no contraction), so its value does not depend
// on the hardware's own exp.
#include <algorithm>

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

// Radix digits of the key from the top: 12 bits (sign, exponent and three
// mantissa bits of the logit, so that logits of a few units spread over many
// bins), then 10, 10, 11, 11, 10.
constexpr int kLevels = 6;
__device__ __forceinline__ int digit_width(int lv) { return lv == 0 ? 12 : (lv == 3 || lv == 4) ? 11 : 10; }
__device__ __forceinline__ int digit_shift(int lv)
{
    return lv == 0 ? 52 : lv == 1 ? 42 : lv == 2 ? 32 : lv == 3 ? 21 : lv == 4 ? 10 : 0;
}
constexpr int kBins0 = 4096;  // first level
constexpr int kBins = 2048;   // deeper levels
constexpr int kCap = 2048;    // candidates held in LDS
constexpr int kB = 8;         // logits per thread whose loads a pass issues together

struct Shared {
    unsigned long long h0w[kBins0];  // first level over all tokens: weight sums
    unsigned int h0c[kBins0];        //                               counts
    unsigned long long hw[kBins];    // deeper levels
    unsigned int hc[kBins];
    unsigned long long ck[kCap];     // the candidate list: keys
    long long cw[kCap];              //                     weights
    long long red[kWaves][3];
    float redf[kWaves];
    unsigned int ncand;
    int sel_digit;
    long long sel_above_t, sel_above_w, sel_bin_w;
    unsigned int sel_above_c, sel_bin_c;
};

__device__ __forceinline__ long long wave_sum_i64(long long v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}



// Lane i receives lane i - n's value of its row of 16 (n = 1, 2, 4, 8), or a
// row broadcast (lane 15 into rows 1 and 3, then lane 31 into rows 2 and 3);
// 0 where there is none. Integer sums, exact in any order.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ long long dpp64(long long v)
{
    const int lo = __builtin_amdgcn_update_dpp(0, (int)(unsigned int)(unsigned long long)v, CTRL, ROW_MASK, 0xF, true);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)((unsigned long long)v >> 32), CTRL, ROW_MASK, 0xF, true);
    return (long long)(((unsigned long long)(unsigned int)hi << 32) | (unsigned long long)(unsigned int)lo);
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ long long lane_scan(long long v)
{
    v += dpp64<0x111, 0xF>(v);  // row_shr:1
    v += dpp64<0x112, 0xF>(v);  // row_shr:2
    v += dpp64<0x114, 0xF>(v);  // row_shr:4
    v += dpp64<0x118, 0xF>(v);  // row_shr:8
    v += dpp64<0x142, 0xA>(v);  // row_bcast:15
    v += dpp64<0x143, 0xC>(v);  // row_bcast:31
    return v;
}

// Result of a selection: the key, and the weight and count of the tokens
// above it, and its own weight.
struct Pick {
    unsigned long long key;
    long long above_w, own_w;
};

// The largest key kappa whose tokens with keys >= kappa weigh at least target
// (unit weights when COUNT): the token at which the cumulative weight, in
// sorted order, first reaches target. Needs 1 <= target <= the total. Level 0
// reads the first-level histogram built with the weights; a deeper level sums
// its candidates (the tokens matching the digits chosen so far) per digit in
// LDS, exact in any order, read from the candidate list when it holds them
// all, else from the logits and weights -- the pass that finds at most kCap
// candidates also copies them into the list.
template <bool COUNT>
__device__ Pick select_key(const float* __restrict__ l, const long long* __restrict__ w, int n, long long target,
                           Shared& sh, unsigned long long& lmask, unsigned long long& lprefix, int& lfloor,
                           bool first)
{
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    unsigned long long prefix = 0, mask = 0;
    long long above_t = 0, above_w = 0;
    unsigned int above_c = 0;
    unsigned int cand = 0xFFFFFFFFu;  // candidates at this level (unknown at level 0)
    Pick out{0ull, 0, 0};
    for (int lv = 0; lv < kLevels; ++lv) {
        const int width = digit_width(lv), shift = digit_shift(lv), bins = 1 << width;
        const unsigned long long dmask = (unsigned long long)(bins - 1);
        const unsigned long long* hw = lv == 0 ? sh.h0w : sh.hw;
        const unsigned int* hc = lv == 0 ? sh.h0c : sh.hc;
        if (lv > 0) {
            for (int i = t; i < bins; i += kT) {
                sh.hw[i] = 0ull;
                sh.hc[i] = 0u;
            }
            // the list holds every token whose first digit is at least lfloor
            // (lfloor >= 0), or every token matching lprefix under lmask
            const bool in_list = lfloor >= 0 ? (int)(prefix >> 52) >= lfloor
                                             : (mask & lmask) == lmask && (prefix & lmask) == lprefix;
            // the first selection's second level keeps every token at or above
            // its first digit when they fit: the draw is among them
            const bool fill_floor = !in_list && first && lv == 1 && above_c + cand <= (unsigned int)kCap;
            const bool fill = !in_list && (fill_floor || cand <= (unsigned int)kCap);
            const unsigned long long floor_key = prefix & (0xFFFull << 52);
            if (fill && t == 0) sh.ncand = 0u;
            __syncthreads();
            if (in_list) {
                const int nc = (int)sh.ncand;
                for (int i = t; i < nc; i += kT) {
                    const unsigned long long key = sh.ck[i];
                    if ((key & mask) == prefix) {
                        const int d = (int)((key >> shift) & dmask);
                        atomicAdd(&sh.hw[d], (unsigned long long)sh.cw[i]);
                        atomicAdd(&sh.hc[d], 1u);
                    }
                }
            } else {
                // batches of kB logits per thread, their loads issued together
                for (int i0 = t; i0 < n; i0 += kB * kT) {
                    float lv[kB];
#pragma unroll
                    for (int u = 0; u < kB; ++u) lv[u] = i0 + u * kT < n ? l[i0 + u * kT] : 0.0f;
                    unsigned long long key[kB];
#pragma unroll
                    for (int u = 0; u < kB; ++u) key[u] = sort_key(lv[u], i0 + u * kT);
                    if (fill) {
                        // the kept tokens (at most kCap) go to the list with their
                        // index; their weights are gathered below in one round
#pragma unroll
                        for (int u = 0; u < kB; ++u) {
                            const int i = i0 + u * kT;
                            if (i < n && (fill_floor ? key[u] >= floor_key : (key[u] & mask) == prefix)) {
                                const unsigned int slot = atomicAdd(&sh.ncand, 1u);
                                sh.ck[slot] = key[u];
                                sh.cw[slot] = i;
                            }
                        }
                    } else {
                        long long wv[kB];
#pragma unroll
                        for (int u = 0; u < kB; ++u) {
                            const int i = i0 + u * kT;
                            const bool hit = i < n && (key[u] & mask) == prefix;
                            wv[u] = hit ? w[i] : -1;  // -1: not a candidate (weights are >= 0)
                        }
#pragma unroll
                        for (int u = 0; u < kB; ++u) {
                            if (wv[u] >= 0) {
                                const int d = (int)((key[u] >> shift) & dmask);
                                atomicAdd(&sh.hw[d], (unsigned long long)wv[u]);
                                atomicAdd(&sh.hc[d], 1u);
                            }
                        }
                    }
                }
                if (fill) {
                    __syncthreads();
                    const int nc = (int)sh.ncand;
                    for (int i = t; i < nc; i += kT) {
                        const long long wv = w[(int)sh.cw[i]];
                        sh.cw[i] = wv;
                        const unsigned long long key = sh.ck[i];
                        if ((key & mask) == prefix) {  // this level's candidates
                            const int d = (int)((key >> shift) & dmask);
                            atomicAdd(&sh.hw[d], (unsigned long long)wv);
                            atomicAdd(&sh.hc[d], 1u);
                        }
                    }
                    lmask = mask;
                    lprefix = prefix;
                    lfloor = fill_floor ? (int)(prefix >> 52) : -1;
                }
            }
            __syncthreads();
        }
        // the digit at which the running total (digits in descending order)
        // reaches target. Wave w totals the block of bins / 16 digits
        // bins - 1 - w B .. bins - (w + 1) B (lane j its digits j, j + 64, ...
        // of the block); wave 0 then finds the block where the total crosses
        // target, and the digit inside it 64 digits at a time.
        const int B = bins / kWaves;
        {
            long long s0 = 0, s1 = 0, s2 = 0;  // target units, weight, count
            for (int i = lane; i < B; i += 64) {
                const int d = bins - 1 - B * wave - i;
                const long long bw = (long long)hw[d], bc = (long long)hc[d];
                s0 += COUNT ? bc : bw;
                s1 += bw;
                s2 += bc;
            }
            s0 = lane_scan(s0);
            s1 = lane_scan(s1);
            s2 = lane_scan(s2);
            if (lv == 0) __syncthreads();  // sh.red is free (the total's reduction read it last)
            if (lane == 63) {
                sh.red[wave][0] = s0;
                sh.red[wave][1] = s1;
                sh.red[wave][2] = s2;
            }
        }
        __syncthreads();
        if (wave == 0) {
            const long long b0 = lane < kWaves ? sh.red[lane][0] : 0, b1 = lane < kWaves ? sh.red[lane][1] : 0;
            const long long b2 = lane < kWaves ? sh.red[lane][2] : 0;
            const long long i0 = lane_scan(b0), i1 = lane_scan(b1), i2 = lane_scan(b2);
            const bool cross = lane < kWaves && above_t + i0 - b0 < target && above_t + i0 >= target;
            // one block (1 <= target <= total); block 0 should there be none
            const int W = max(__ffsll((unsigned long long)__ballot(cross)) - 1, 0);
            long long rt = above_t + __shfl(i0 - b0, W, 64), rw = above_w + __shfl(i1 - b1, W, 64);
            long long rc = (long long)above_c + __shfl(i2 - b2, W, 64);
            for (int i0b = 0; i0b < B; i0b += 64) {
                const int i = i0b + lane;
                const int d = bins - 1 - B * W - i;
                const long long bw = i < B ? (long long)hw[d] : 0, bc = i < B ? (long long)hc[d] : 0;
                const long long bt = COUNT ? bc : bw;
                const long long f0 = lane_scan(bt), f1 = lane_scan(bw), f2 = lane_scan(bc);
                const bool hit = i < B && rt + f0 - bt < target && rt + f0 >= target;
                if (hit) {
                    sh.sel_digit = d;
                    sh.sel_above_t = rt + f0 - bt;
                    sh.sel_above_w = rw + f1 - bw;
                    sh.sel_above_c = (unsigned int)(rc + f2 - bc);
                    sh.sel_bin_w = bw;
                    sh.sel_bin_c = (unsigned int)bc;
                }
                if (__ballot(hit)) break;
                rt += __shfl(f0, 63, 64);
                rw += __shfl(f1, 63, 64);
                rc += __shfl(f2, 63, 64);
            }
        }
        __syncthreads();
        const int d = sh.sel_digit;
        prefix |= (unsigned long long)d << shift;
        mask |= dmask << shift;
        above_t = sh.sel_above_t;
        above_w = sh.sel_above_w;
        above_c = sh.sel_above_c;
        cand = sh.sel_bin_c;
        out.own_w = sh.sel_bin_w;  // at the last level: the one token with this key
        __syncthreads();  // every thread has read the selection before it is written again
    }
    out.key = prefix;
    out.above_w = above_w;
    return out;
}

// ---- the row maximum, the weights and the first-level histogram over P
// workgroups per row (P = splits: a slice of about n / P tokens each) -----------
// The fp64 weights (about fifty fp64 instructions per token) dominate a row;
// spread over P CUs they take a P-th of the time. Maxima and the integer sums
// are exact in any order, so the result does not depend on P.
constexpr int kMaxSplits = 64;

struct SampleWs {
    float* maxp;                // [m][kMaxSplits] slice maxima
    unsigned long long* h0w;    // [m][kBins0] first-level weight sums
    unsigned int* h0c;          // [m][kBins0] first-level counts
    long long* total;           // [m] total weight
};

// Slice maxima; each workgroup also zeroes its share of its row's histogram.
__global__ __launch_bounds__(256) void sample_max_kernel(const float* __restrict__ logits, int n, int splits,
                                                         SampleWs ws)
{
    __shared__ float red[4];
    const int row = blockIdx.x / splits, sp = blockIdx.x - row * splits, t = threadIdx.x;
    const int per = (n + splits - 1) / splits, i0 = sp * per, i1 = min(i0 + per, n);
    const float* l = logits + (size_t)row * n;
    float lm = -INFINITY;
    for (int i = i0 + t; i < i1; i += 256) lm = fmaxf(lm, l[i]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) lm = fmaxf(lm, __shfl_xor(lm, off, 64));
    if ((t & 63) == 0) red[t >> 6] = lm;
    __syncthreads();
    if (t == 0) ws.maxp[(size_t)row * kMaxSplits + sp] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const int bper = (kBins0 + splits - 1) / splits, b0 = sp * bper, b1 = min(b0 + bper, kBins0);
    for (int b = b0 + t; b < b1; b += 256) {
        ws.h0w[(size_t)row * kBins0 + b] = 0ull;
        ws.h0c[(size_t)row * kBins0 + b] = 0u;
    }
    if (sp == 0 && t == 0) ws.total[row] = 0;
}

__device__ __forceinline__ float row_max(const SampleWs& ws, int row, int splits)
{
    float m = -INFINITY;
    for (int j = 0; j < splits; ++j) m = fmaxf(m, ws.maxp[(size_t)row * kMaxSplits + j]);
    return m;
}

struct WeightsShared {
    unsigned long long h0w[kBins0];
    unsigned int h0c[kBins0];
    long long red[kWaves];
};

// A slice's weights (stored), its first-level histogram (in LDS, then added to
// the row's) and its total weight.
__global__ __launch_bounds__(kT) void sample_weights_kernel(const float* __restrict__ logits, int n, int splits,
                                                            float temp, long long* __restrict__ wbuf, SampleWs ws)
{
    __shared__ WeightsShared sh;
    const int row = blockIdx.x / splits, sp = blockIdx.x - row * splits, t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int per = (n + splits - 1) / splits, i0 = sp * per, i1 = min(i0 + per, n);
    const float* l = logits + (size_t)row * n;
    long long* w = wbuf + (size_t)row * n;
    for (int i = t; i < kBins0; i += kT) {
        sh.h0w[i] = 0ull;
        sh.h0c[i] = 0u;
    }
    const float lmax = row_max(ws, row, splits);
    __syncthreads();
    long long part = 0;
    for (int ib = i0 + t; ib < i1; ib += kB * kT) {
        float lv[kB];
#pragma unroll
        for (int u = 0; u < kB; ++u) lv[u] = ib + u * kT < i1 ? l[ib + u * kT] : 0.0f;
#pragma unroll
        for (int u = 0; u < kB; ++u) {
            const int i = ib + u * kT;
            if (i < i1) {
                const double x = ((double)lv[u] - (double)lmax) / (double)temp;
                const long long q = (long long)rint(ldexp(exp_neg(x), 40));
                w[i] = q;
                part += q;
                const int d = (int)(sort_key(lv[u], i) >> 52);
                atomicAdd(&sh.h0w[d], (unsigned long long)q);
                atomicAdd(&sh.h0c[d], 1u);
            }
        }
    }
    part = wave_sum_i64(part);
    if (lane == 0) sh.red[wave] = part;
    __syncthreads();
    if (t == 0) {
        long long tot = 0;
        for (int j = 0; j < kWaves; ++j) tot += sh.red[j];
        atomicAdd(reinterpret_cast<unsigned long long*>(ws.total + row), (unsigned long long)tot);
    }
    for (int b = t; b < kBins0; b += kT) {
        const unsigned int c = sh.h0c[b];
        if (c) {
            atomicAdd(ws.h0w + (size_t)row * kBins0 + b, sh.h0w[b]);
            atomicAdd(ws.h0c + (size_t)row * kBins0 + b, c);
        }
    }
}

template <bool TOPP>
__global__ __launch_bounds__(kT) void sample_kernel(const float* __restrict__ logits, int n, int splits, int k,
                                                    float p, const double* __restrict__ u, int32_t* __restrict__ out,
                                                    long long* __restrict__ wbuf, SampleWs ws)
{
    __shared__ Shared sh;
    const int row = blockIdx.x, t = threadIdx.x;
    const float* l = logits + (size_t)row * n;
    const long long* w = wbuf + (size_t)row * n;
    for (int i = t; i < kBins0; i += kT) {
        sh.h0w[i] = ws.h0w[(size_t)row * kBins0 + i];
        sh.h0c[i] = ws.h0c[(size_t)row * kBins0 + i];
    }
    const long long total = ws.total[row];
    __syncthreads();

    unsigned long long lmask = ~0ull, lprefix = 0ull;  // the candidate list: empty
    int lfloor = -1;
    Pick kept;
    if (TOPP) {
        // min(Z, ceil(p Z)) compared exactly: fl64(Z) may round above Z, and a
        // target above Z would have no crossing digit
        const double tg = ceil((double)p * (double)total);
        long long target = tg < 9.0e18 ? (long long)tg : total;
        if (target > total) target = total;
        if (target < 1) target = 1;
        kept = select_key<false>(l, w, n, target, sh, lmask, lprefix, lfloor, true);
    } else {
        kept = select_key<true>(l, w, n, k < n ? k : n, sh, lmask, lprefix, lfloor, true);
    }
    // the kept tokens (keys >= kappa) weigh the tokens above kappa plus kappa's own
    const long long mass = kept.above_w + kept.own_w;
    const double rd = floor(u[row] * (double)mass);
    const long long r = rd < 0.0 ? 0 : (rd >= (double)mass ? mass - 1 : (long long)rd);
    // the kept tokens are a prefix of the sorted order, so the first token
    // whose cumulative weight reaches r + 1 (<= mass) is a kept one
    const Pick chosen = select_key<false>(l, w, n, r + 1, sh, lmask, lprefix, lfloor, false);
    if (t == 0) out[row] = (int32_t)(0xFFFFFFFFu - (uint32_t)(chosen.key & 0xFFFFFFFFull));
}

}  // namespace

// Workspace of launch_sample: the weights, then the slice maxima, the first-level
// histograms and the totals (each part 256-aligned).
size_t sample_workspace_bytes(int m, int n)
{
    auto al = [](size_t b) { return (b + 255) / 256 * 256; };
    return al((size_t)m * n * 8) + al((size_t)m * kMaxSplits * 4) + al((size_t)m * kBins0 * 8) +
           al((size_t)m * kBins0 * 4) + al((size_t)m * 8);
}

int launch_sample(bool topp, const float* logits, int m, int n, int k, float p, float temperature, const double* u,
                  int32_t* out, void* workspace, hipStream_t s)
{
    auto al = [](size_t b) { return (b + 255) / 256 * 256; };
    char* base = static_cast<char*>(workspace);
    long long* wbuf = reinterpret_cast<long long*>(base);
    size_t off = al((size_t)m * n * 8);
    SampleWs ws;
    ws.maxp = reinterpret_cast<float*>(base + off);
    off += al((size_t)m * kMaxSplits * 4);
    ws.h0w = reinterpret_cast<unsigned long long*>(base + off);
    off += al((size_t)m * kBins0 * 8);
    ws.h0c = reinterpret_cast<unsigned int*>(base + off);
    off += al((size_t)m * kBins0 * 4);
    ws.total = reinterpret_cast<long long*>(base + off);
    // workgroups per row: the rows over about 256 CUs, at least 1024 tokens each
    int splits = std::max(1, std::min(kMaxSplits, 256 / std::max(m, 1)));
    splits = std::max(1, std::min(splits, (n + kT - 1) / kT));
    const int g = m * splits;
    sample_max_kernel<<<g, 256, 0, s>>>(logits, n, splits, ws);
    sample_weights_kernel<<<g, kT, 0, s>>>(logits, n, splits, temperature, wbuf, ws);
    if (topp)
        sample_kernel<true><<<m, kT, 0, s>>>(logits, n, splits, k, p, u, out, wbuf, ws);
    else
        sample_kernel<false><<<m, kT, 0, s>>>(logits, n, splits, k, p, u, out, wbuf, ws);
    return hipGetLastError() == hipSuccess ? BL_OK : BL_ERR_LAUNCH;
}

}  // namespace bl
