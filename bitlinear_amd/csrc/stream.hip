// stream.hip -- persistent kernel for the decoder-layer BitLinear stream at
// one token.
//
// Per layer the stream has four dependent steps ("Transformer Block", Hesper
// API, "Forward Pass"; the seven projections of "Memory Layout"):
//   P1  q, k, v  = BitLinear(quant(rmsnorm(x, g_attn)))              3d rows, K = d
//   P2  x'       = x + BitLinear_o(quant(rmsnorm(z, g_attn_sub)))    d rows,  K = d
//   P3  h        = relu(gate)^2 * up, gate/up = BitLinear(quant(rmsnorm(x', g_ffn)))
//                                                                     f row pairs, K = d
//   P4  x''      = x' + BitLinear_down(quant(rmsnorm(h, g_ffn_sub)))  d rows, K = f
// P2 waits for every workgroup to finish P1, as the o projection waits for
// attention over all heads in the full model. The kernels with ATTN (a decode
// step of one sequence) run that attention: P1 publishes q, k, v, a phase PA
// computes single-token attention with RoPE and the KV caches, and P2 waits
// for its published output instead of the stand-in z.
//
// At one token every step is a short weight stream (1.6 to 13 MB) whose input
// is a vector produced by all CUs in the step before. Launching a kernel per
// step pays the kernel start and the HBM latency ramp 128 times per token. Here
// one workgroup per CU (256 on an MI355X) stays resident for the whole token:
//   - each workgroup owns fixed output rows of every step and issues the loads
//     of those weight rows (and of the step's RMSNorm gains) before it waits
//     for the step's input, so the weight fetch overlaps the hand-over. The
//     rows go straight into registers in the layout of the MFMA B operand;
//   - a wave's loads complete in issue order, so a wait for a hand-over also
//     waits for every weight row issued before it, and a step whose rows come
//     from HBM (13 MB for gate/up) holds its wait until they have streamed
//     in. Each workgroup therefore pulls its rows of a later step into L2
//     one step or two ahead, right after a wait has ended, while HBM is
//     otherwise idle: gate/up after P2's wait, down and the next layer's o
//     rows after P3's, the next layer's q/k/v rows after P4's. The prefetch
//     is one dword per 128-byte line, loaded straight into a scratch area of
//     LDS (global_load_lds_dword), so it needs no register, and the compiler,
//     which does not see it, adds no wait for it; the wave's next poll waits
//     for it like for any older load. Every prefetch is followed by a poll
//     before the workgroup can leave, so none is in flight at the end;
//   - a step's output vector is published as fp32 words written with
//     device-scope atomic stores, the word's value doubling as its flag: 0
//     (+0.0) means "not written yet" (+0.0 itself is published as -0.0).
//     Each vector has two copies that alternate by layer; a producer clears
//     its words of the other copy when it writes, which every consumer has
//     finished reading by then. A consumer loads all words of the vector it
//     needs in one batch and repeats until none reads 0. Value and flag
//     travel in one single-copy-atomic store, so no fence or separate
//     barrier is needed, and a poll moves 4 bytes per value (an epoch-tagged
//     8-byte word measured 4 % slower: the hand-overs are sensitive to the
//     poll traffic). P2's wait uses epoch-tagged 8-byte flags, one per
//     workgroup, four per 128-byte line (one per line doubles the poll
//     traffic, sixteen per line makes the writers contend);
//   - every workgroup then computes the RMSNorm + activation quant of the full
//     vector itself, so no extra round trip is spent on broadcasting q. The
//     sum of squares keeps the fixed fp64 order of quant.hip: thread t sums
//     x[k]^2 for k = t, t + 512, ... in ascending k, and an xor-butterfly
//     combines the 512 partials (offsets 1..32 with exact lane exchanges,
//     64..256 through LDS). P2's input stands in for the attention output,
//     so its norm + quant runs after the wait for P1, where the real one
//     would become available;
//   - dot products: v_mfma_i32_16x16x64_i8 with the token in row 0 of A and
//     16 weight rows as the columns of B (rows 1..15 of A are zero). A lane
//     of B holds 16 weights of one row; from a packed 16-byte chunk (64
//     weights) the masks 0x03, 0x0C, 0x30 per byte select the codes of weights
//     4i+0, 4i+1, 4i+2 scaled by 1, 4, 16, and (w >> 2) & 0x30 those of 4i+3
//     scaled by 16, so one AND (two for the last class) yields each operand.
//     The activation vector sits in LDS in the matching byte order. The
//     scaled accumulators are exact multiples of their scales and are shifted
//     back exactly; the code offset (c = t + 1) is removed with sum(q).
// A workgroup has 512 threads (8 waves, 2 per SIMD).
// The P2/P4 rows of a workgroup are the same, so the residual x of its rows
// stays in registers across the whole stream.
//
// Termination: every wait is bounded by a wall-clock limit of 2 s from the
// start of that wait (s_memrealtime, 100 MHz) and by a shared status word; a
// workgroup that gives up sets the status, every other one sees it and leaves,
// so the grid always drains.
#include <type_traits>

#include "internal.h"
#include "prefetch.h"
#include "wave.h"

namespace bl {
namespace {

constexpr int kT = 512;      // threads per workgroup: 8 waves, 2 per SIMD; also the
                             // number of RMSNorm partial sums of the fixed order
constexpr int kGrid = 256;   // workgroups: one per CU of an MI355X
constexpr uint32_t kCodeMask = 0x03030303u;
constexpr long long kTimeoutTicks = 200000000LL;  // 2 s at 100 MHz
constexpr int kMaxK = 10240;
constexpr int kFlagStride = 4;   // words between the "P1 finished" flags: four per 128-byte line

constexpr int cdiv(int a, int b) { return (a + b - 1) / b; }

typedef int v4i __attribute__((ext_vector_type(4)));

// One step: N output rows per stacked matrix (MATS matrices), K inputs. A
// workgroup owns R consecutive rows of each matrix, RT = MATS * R in all. Its
// dot products are ITEMS items (tile, s): rows 16 tile .. +15 against inputs
// 256 s .. +255; wave w takes the contiguous items [w P, (w + 1) P).
template <int N, int K, int MATS>
struct Step {
    static constexpr int R = N / kGrid;
    static constexpr int RT = MATS * R;
    static constexpr int TILES = cdiv(RT, 16);
    static constexpr int KSTEPS = K / 256;
    static constexpr int ITEMS = TILES * KSTEPS;
    static constexpr int P = cdiv(ITEMS, kT / 64);
    static_assert(N % kGrid == 0 && R >= 1, "rows per workgroup");
    static_assert(K % 256 == 0 && K <= kMaxK, "K");
    static_assert(RT <= 128, "LDS accumulators");
};

struct StreamArgs {
    const uint8_t* weights;
    const float* scales;
    const float* gains;
    const float* z;
    float* x;
    float* qkv;
    long long qkv_layer_stride;  // elements between layers (0: scratch reused)
    uint32_t* xa;                // x at layer start (published by P4), two copies
    uint32_t* xb;                // x after the o residual (published by P2), two copies
    uint32_t* hh;                // h (published by P3), two copies
    unsigned long long* done;    // per-workgroup "P1 finished" flags
    uint32_t* ctrl;              // [0] epoch base, [1] status
    int n_layers;
    float eps;
    // attention (the kernels with ATTN only)
    uint32_t* qq;                // q, k, v (published by P1), two copies of 3d words
    uint32_t* ao;                // attention output (published by PA), two copies of d words
    const float* rope_cos;       // row pos of the rotary table [hd / 2]
    const float* rope_sin;
    float* k_cache;              // [n_layers][heads][max_seq][hd]
    float* v_cache;
    float* attn;                 // [n_layers][d] or null
    unsigned long long* apart;   // per head and chunk: epoch-tagged [max, sum, hd weighted sums]
    int heads, hd, max_seq, pos, chunks_max;
};

__device__ __forceinline__ void ll_store(unsigned long long* p, float v, uint32_t e)
{
    const unsigned long long w = ((unsigned long long)e << 32) | (unsigned long long)__float_as_uint(v);
    __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ unsigned long long ll_load(const unsigned long long* p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Published vector words are plain fp32 bit patterns with 0x00000000 (+0.0)
// meaning "not written yet": a producer publishes +0.0 as -0.0 (the values
// are only squared, scaled and rounded by the consumer, where the two agree)
// and clears its word of the vector's other copy, which is read again only
// two hand-overs later, after every consumer has finished with it.
__device__ __forceinline__ void val_store(uint32_t* p, float v)
{
    const uint32_t b = __float_as_uint(v);
    __hip_atomic_store(p, b == 0u ? 0x80000000u : b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void val_clear(uint32_t* p)
{
    __hip_atomic_store(p, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t status_load(const uint32_t* ctrl)
{
    return __hip_atomic_load(ctrl + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Workgroup barrier for LDS: this wave's LDS accesses complete, then
// s_barrier; global loads in flight stay in flight.
__device__ __forceinline__ void lds_sync()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt unconstrained
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Workgroup-wide OR of failed with one barrier: lane 0 of each wave stores its
// wave's ballot in its own word of vote[kT / 64], and every thread reads all
// of them after the barrier. The words are written again only at the next
// wait, which lies behind further barriers (the norm + quant's), so no thread
// can read a later vote.
__device__ __forceinline__ bool block_any(bool failed, uint32_t* vote)
{
    const uint32_t wv = __ballot(failed) != 0ull ? 1u : 0u;
    if ((threadIdx.x & 63) == 0) vote[threadIdx.x >> 6] = wv;
    lds_sync();
    uint32_t any = 0u;
#pragma unroll
    for (int i = 0; i < kT / 64; ++i) any |= vote[i];
    return any != 0u;
}

// Loads the words k = t, t + 512, ... < N of buf until every one carries epoch
// e (all loads of a round are issued before any is checked); v receives the
// fp32 payloads. Returns false, for the whole workgroup, on a timeout (2 s from
// the start of this wait) or when another workgroup gave up.
template <int N, int STRIDE = 1>
__device__ bool poll_vec(const unsigned long long* buf, uint32_t e, float* v, uint32_t* ctrl, uint32_t* vote)
{
    constexpr int NI = cdiv(N, kT);
    const int t = threadIdx.x;
    const long long t_start = (long long)__builtin_amdgcn_s_memrealtime();
    unsigned long long w[NI];
    bool failed = false;
    for (int spin = 0;; ++spin) {
        // every load is unconditional (clamped address) so that the whole batch
        // is in flight before the first wait
#pragma unroll
        for (int i = 0; i < NI; ++i) w[i] = ll_load(buf + STRIDE * min(t + kT * i, N - 1));
        bool ready = true;
#pragma unroll
        for (int i = 0; i < NI; ++i) ready = ready && (uint32_t)(w[i] >> 32) == e;
        if (ready) break;
        if ((spin & 15) == 15 &&
            (status_load(ctrl) != 0 || (long long)__builtin_amdgcn_s_memrealtime() - t_start > kTimeoutTicks)) {
            failed = true;
            break;
        }
        __builtin_amdgcn_s_sleep(3);  // about 190 cycles between rounds
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) v[i] = (t + kT * i < N) ? __uint_as_float((uint32_t)w[i]) : 0.0f;
    if (block_any(failed, vote)) {
        if (t == 0) __hip_atomic_fetch_or(ctrl + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return false;
    }
    return true;
}

// As poll_vec for a published fp32 vector: repeats until no word reads 0.
template <int N>
__device__ bool poll_val(const uint32_t* buf, float* v, uint32_t* ctrl, uint32_t* vote)
{
    constexpr int NI = cdiv(N, kT);
    const int t = threadIdx.x;
    const long long t_start = (long long)__builtin_amdgcn_s_memrealtime();
    uint32_t w[NI];
    bool failed = false;
    for (int spin = 0;; ++spin) {
#pragma unroll
        for (int i = 0; i < NI; ++i)
            w[i] = __hip_atomic_load(buf + min(t + kT * i, N - 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        bool ready = true;
#pragma unroll
        for (int i = 0; i < NI; ++i) ready = ready && w[i] != 0u;
        if (ready) break;
        if ((spin & 15) == 15 &&
            (status_load(ctrl) != 0 || (long long)__builtin_amdgcn_s_memrealtime() - t_start > kTimeoutTicks)) {
            failed = true;
            break;
        }
        __builtin_amdgcn_s_sleep(3);  // about 190 cycles between rounds
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) v[i] = (t + kT * i < N) ? __uint_as_float(w[i]) : 0.0f;
    if (block_any(failed, vote)) {
        if (t == 0) __hip_atomic_fetch_or(ctrl + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return false;
    }
    return true;
}

template <int N>
__device__ __forceinline__ void load_strided(const float* src, float* out)
{
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < cdiv(N, kT); ++i) out[i] = src[min(t + kT * i, N - 1)];
#pragma unroll
    for (int i = 0; i < cdiv(N, kT); ++i)
        if (t + kT * i >= N) out[i] = 0.0f;
}

// The code rne(fl32(y * scale)) from one more fp32 add: the rounded product
// plus 1.5 * 2^23 lands in [2^23, 2^24), where consecutive floats are one
// apart, so the add rounds it to an integer, to nearest even as rintf does; the
// bit pattern is then 0x4B400000 + code, whose low byte is the code's int8 byte.
// With scale = 127 / max(absmax, 1e-5) no |y * scale| exceeds 127 (1 + 2^-23),
// so the quantizer's clamp to [-128, 127] never acts and is left out. (The
// library builds with -ffp-contract=off: the product is rounded on its own.)
__device__ __forceinline__ uint32_t quant_bits(float y, float scale)
{
    const float p = y * scale;
    return __float_as_uint(p + 12582912.0f);
}
constexpr uint32_t kQuantBias = 0x4B400000u;  // bit pattern of 1.5 * 2^23

// Byte position of activation k in LDS: within each 64 values, the 16 bytes at
// 16 j hold k = 16 g + 4 i + j at byte 4 g + i (the order of the B operand
// built from mask class j).
__device__ __forceinline__ int q_pos(int k)
{
    return (k & ~63) | ((k & 3) << 4) | (((k >> 4) & 3) << 2) | ((k >> 2) & 3);
}

struct Shared {
    __attribute__((aligned(16))) uint8_t q[kMaxK];  // quantized input vector (q_pos order)
    __attribute__((aligned(16))) uint8_t zero[64];  // A rows 1..15
    double red_d[kT / 64];
    float red_f[kT / 64];
    int red_i[kT / 64];
    int acc[128];  // per-row accumulators of a step (gate rows, then up rows)
    uint32_t trash[64];  // written by the L2 prefetch loads, never read
    uint32_t vote[kT / 64];  // per-wave failure votes of a wait
};

// Every 128-byte line of [p, p + BYTES), one per thread. BYTES is a multiple
// of 64 (whole packed rows, K % 256 == 0), so the dword read at the start of
// the last line lies inside the span.
template <int BYTES>
__device__ __forceinline__ void prefetch_span(const uint8_t* p, uint32_t lds_off)
{
    static_assert(BYTES % 64 == 0, "whole 64-byte chunks");
    for (int i = threadIdx.x; i < cdiv(BYTES, 128); i += kT) prefetch_line(p + 128 * i, lds_off);
}

// RMSNorm (gains g[i] = gain[t + 512 i]) + activation quant of the N values
// held as v[i] = x[t + 512 i] into the permuted int8 vector sh.q; returns s_a
// and sum(q) to every thread. Thread t's own values form partial t of the sum
// of squares (k = t, t + 512, ... ascending); the butterfly then runs inside
// each wave (offsets 1..32) and across the 8 waves (64, 128, 256).
template <int N>
__device__ void norm_quant(const float* v, const float* g, float eps, Shared& sh, float& s_out, int& qsum_out)
{
    static_assert(kT == 512, "the sum of squares is defined over 512 partials");
    constexpr int NI = cdiv(N, kT);
    constexpr int W = kT / 64;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    double p = 0.0;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const double xv = (double)v[i];
        p += xv * xv;  // v is zero beyond N
    }
    p = wave_butterfly_sum(p);
    if (lane == 0) sh.red_d[wave] = p;
    __syncthreads();
    const float r = (float)(1.0 / sqrt(cross_wave_sum8(sh.red_d) / (double)N + (double)eps));

    float y[NI];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        y[i] = (v[i] * r) * g[i];
        amax = fmaxf(amax, fabsf(y[i]));
    }
    amax = wave_max(amax);
    if (lane == 0) sh.red_f[wave] = amax;
    __syncthreads();
    amax = sh.red_f[0];
#pragma unroll
    for (int i = 1; i < W; ++i) amax = fmaxf(amax, sh.red_f[i]);
    const float scale = 127.0f / fmaxf(amax, 1e-5f);
    int sum = 0;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int k = t + kT * i;
        if (k < N) {
            const uint32_t qb = quant_bits(y[i], scale);
            sum += (int)(qb - kQuantBias);
            sh.q[q_pos(k)] = (uint8_t)qb;
        }
    }
    sum = wave_sum(sum);
    if (lane == 0) sh.red_i[wave] = sum;
    __syncthreads();
    s_out = scale;
    int total = 0;
#pragma unroll
    for (int i = 0; i < W; ++i) total += sh.red_i[i];
    qsum_out = total;
}

__device__ __forceinline__ v4i mask4(const uint4 p, uint32_t m)
{
    return v4i{(int)(p.x & m), (int)(p.y & m), (int)(p.z & m), (int)(p.w & m)};
}

// Loads the B operands of this wave's items: lane (n, b) = (lane % 16,
// lane / 16) takes bytes 64 s + 16 b .. +15 of slot row 16 tile + n (clamped to
// the last row; items past the end repeat the last one, so every load is
// unconditional and all issue before the first wait). row_ptr(r) is the
// packed row r of the step.
template <class S, class RowPtr>
__device__ __forceinline__ void load_items(uint4* wr, RowPtr row_ptr)
{
    const int lane = threadIdx.x & 63, n = lane & 15, b = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
    for (int j = 0; j < S::P; ++j) {
        const int it = min(wave * S::P + j, S::ITEMS - 1);
        const int tile = it / S::KSTEPS, s = it - tile * S::KSTEPS;
        const int row = min(16 * tile + n, S::RT - 1);
        wr[j] = *reinterpret_cast<const uint4*>(row_ptr(row) + 64 * s + 16 * b);
    }
}

// The wave's items: one MFMA accumulator per mask class; when the tile
// changes, and at the end, the row sums of codes x q (row 0 of C: lanes 0..15,
// register 0) go to acc[] through LDS atomics, exact in any order.
template <class S>
__device__ __forceinline__ void dots(const uint4* wr, const uint8_t* q, const uint8_t* zero, int* acc)
{
    const int lane = threadIdx.x & 63, n = lane & 15, b = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint8_t* a_base = n == 0 ? q + 64 * b : zero;
    const int a_step = n == 0 ? 256 : 0;
    const v4i zc = {0, 0, 0, 0};
    v4i c0 = zc, c1 = zc, c2 = zc, c3 = zc;
    int tile = -1;
    auto flush = [&]() {
        const int v = c0[0] + (c1[0] >> 2) + ((c2[0] + c3[0]) >> 4);
        if (lane < 16 && 16 * tile + lane < S::RT) atomicAdd(acc + 16 * tile + lane, v);
        c0 = zc;
        c1 = zc;
        c2 = zc;
        c3 = zc;
    };
#pragma unroll
    for (int j = 0; j < S::P; ++j) {
        const int it = wave * S::P + j;
        if (it < S::ITEMS) {
            const int tl = it / S::KSTEPS, s = it - tl * S::KSTEPS;
            if (tl != tile) {
                if (tile >= 0) flush();
                tile = tl;
            }
            const uint8_t* ap = a_base + a_step * s;
            const v4i a0 = *reinterpret_cast<const v4i*>(ap);
            const v4i a1 = *reinterpret_cast<const v4i*>(ap + 16);
            const v4i a2 = *reinterpret_cast<const v4i*>(ap + 32);
            const v4i a3 = *reinterpret_cast<const v4i*>(ap + 48);
            const uint4 p = wr[j];
            const uint4 p3 = make_uint4(p.x >> 2, p.y >> 2, p.z >> 2, p.w >> 2);
            c0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, mask4(p, kCodeMask), c0, 0, 0, 0);
            c1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, mask4(p, kCodeMask << 2), c1, 0, 0, 0);
            c2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a2, mask4(p, kCodeMask << 4), c2, 0, 0, 0);
            c3 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a3, mask4(p3, kCodeMask << 4), c3, 0, 0, 0);
        }
    }
    if (tile >= 0) flush();
}

// ---- single-token attention inside the stream --------------------------------
// Phase PA of the kernels with ATTN ("Transformer Block", "Forward Pass with
// KV Cache"; "BitNet Model - Complete Inference Pipeline", "KV Cache State").
// Positions 0 .. pos of a head split into chunks (attn_chunk_len); G = 256 /
// heads workgroups serve each head, workgroup (h, split) taking the chunks
// c = split, split + G, ... Each waits for the 3 hd published words of q, k
// and v of its head, turns q and k by RoPE (the one holding position pos also
// appends k and v to the caches), and per chunk forms the scores
// q . k_j / sqrt(hd), the chunk's maximum and sum of e^(s - max), and the
// weighted sums of v (512 / (hd / 4) groups of hd / 4 threads, a thread
// holding four columns, each group over every (512 / (hd / 4))-th position,
// then the groups in order). A score is the sum, in
// order, of the dot products of q and k_j over the hd / 4 runs of four
// values. Split 0 merges the chunks by rescaling with e^(max_c - max), as the
// launch path's merge kernel does, and publishes the head's output for P2.
// Scores, exponentials and sums are fp32.
//
// One CU pulls cache rows from HBM at only a few tens of GB/s, so the rows of
// a head are spread over all of its workgroups (attn_chunk_len), and each
// workgroup issues a chunk's K and V loads together, right after the wait for
// q, k and v, as float4s: K in row-major order (thread t takes t, t + 512,
// ...), V in the layout of the weighted sums (indices past the chunk's rows
// are clamped to its last row, so that every load is unconditional). The
// barriers between the loads and their use wait for LDS only (__syncthreads
// would also wait for the loads in flight).
constexpr int kAttnChunk = 256;
constexpr int kAttnMinChunk = 16;
constexpr int kAttnCutFrom = 224;  // positions 0 .. pos with pos below this are one chunk
constexpr int kMaxAttnChunks = kStreamAttnMaxChunks;  // 32: max_seq <= 8192
constexpr int kMaxHd = 256;
constexpr int kAttnKB = 8;   // K float4s per thread and round: 204 positions of hd = 80
constexpr int kAttnVB = 7;   // V float4s per thread and round: 175 positions of hd = 80
// (larger rounds spill registers)

// Positions per chunk for position pos and G workgroups per head: 256 once a
// head has at least min(G, 32) such chunks; below that the positions are cut
// into up to min(G, 32) chunks of a multiple of 8, at least 16, so that every
// workgroup of the head pulls a share of the cache rows -- except up to 224
// positions, which stay one chunk: there the merge's hand-over costs more
// than the split saves.
__device__ __forceinline__ int attn_chunk_len(int pos, int G)
{
    const int gm = min(G, kMaxAttnChunks);
    const int n256 = (pos + kAttnChunk) / kAttnChunk;
    if (n256 >= gm || pos < kAttnCutFrom) return kAttnChunk;
    const int len = (((pos + gm) / gm) + 7) & ~7;  // ceil((pos + 1) / gm), up to a multiple of 8
    return max(len, kAttnMinChunk);
}

struct AttnShared {
    __attribute__((aligned(16))) float q[kMaxHd];  // rotated q, rotated k and v of position pos
    __attribute__((aligned(16))) float k[kMaxHd];
    __attribute__((aligned(16))) float v[kMaxHd];
    float e[kAttnChunk];                    // e^(s_j - max) of the chunk's positions
    float kp[kAttnChunk * (kMaxHd / 4)];    // q . k over each run of four values, row-major
    __attribute__((aligned(16))) float part[4 * kT];  // per-group partial sums of the weighted values
    float red[kT / 64];
    float chunk[kMaxAttnChunks][kMaxHd + 2];  // per chunk: max, sum, weighted sums
    uint32_t vote;  // the epoch of a phase whose q/k/v wait failed (0 at kernel start)
    uint32_t merge_vote[2][kT / 64];  // per-wave flags of the merge wait's rounds, by round parity
};
struct NoAttnShared {};

__device__ __forceinline__ float block_max_f(float v, float* red)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    v = wave_max(v);
    lds_sync();  // red is free
    if (lane == 0) red[wave] = v;
    lds_sync();
    float m = red[0];
#pragma unroll
    for (int i = 1; i < kT / 64; ++i) m = fmaxf(m, red[i]);
    return m;
}

__device__ __forceinline__ float block_sum_f(float v, float* red)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    lds_sync();
    if (lane == 0) red[wave] = v;
    lds_sync();
    float s = red[0];
#pragma unroll
    for (int i = 1; i < kT / 64; ++i) s += red[i];
    return s;
}

// Attention work of workgroup (h, split) in layer l: head h's chunks c with
// c % G == split (G workgroups per head). The workgroup that holds position
// pos (the last chunk) appends k and v to the caches. Split 0 merges: its own
// chunks' partials stay in LDS, the others' arrive as epoch-tagged words
// (epoch E2, so no copy needs clearing), and it publishes the head's output.
// False (for the whole workgroup) when a wait gave up. D: the model width (q,
// k, v are the 3 consecutive D-word rows of qq).
template <int D>
__device__ bool attention_split(const StreamArgs& a, int l, int h, int split, int G, uint32_t E2,
                                const uint32_t* qq_cur, uint32_t* ao_cur, uint32_t* ao_old, AttnShared& s)
{
    const int t = threadIdx.x;
    const int hd = a.hd, half = hd / 2, pos = a.pos, h4 = hd / 4;
    const int len = attn_chunk_len(pos, G);
    const int nch = (pos + len) / len;
    const int last = (nch - 1) % G;  // the split that holds position pos
    const float* kbase = a.k_cache + ((size_t)l * a.heads + h) * a.max_seq * hd;
    const float* vbase = a.v_cache + ((size_t)l * a.heads + h) * a.max_seq * hd;
    // V: thread (g, c4v) takes float4 column c4v of positions g, g + groups, ...
    const int groups = kT / h4, g = t / h4, c4v = t - g * h4;
    const size_t vstep = (size_t)groups * h4;  // float4s between a thread's V positions

    // One round of a chunk's cache rows (lim >= 1 rows from position j0): K
    // float4s f0 + t + 512 i, V positions g + groups (u0 + u) of float4 column
    // c4v, indices clamped to the last row (threads without V positions read
    // row j0).
    float4 kr[kAttnKB];
    float4 vr[kAttnVB];
    auto load_k = [&](int j0, int lim, int f0) {
        const float4* kb4 = reinterpret_cast<const float4*>(kbase + (size_t)j0 * hd);
        const int nf = lim * (hd / 4);
#pragma unroll
        for (int i = 0; i < kAttnKB; ++i) kr[i] = kb4[min(f0 + t + kT * i, nf - 1)];
    };
    auto load_v = [&](int j0, int lim, int u0) {
        const bool has = g < groups && lim > g;  // else: row j0 only
        const int mine = has ? (lim - g + groups - 1) / groups : 1;
        const float4* vp = reinterpret_cast<const float4*>(vbase + (size_t)(j0 + (has ? g : 0)) * hd) + c4v;
#pragma unroll
        for (int u = 0; u < kAttnVB; ++u) vr[u] = vp[(size_t)min(u0 + u, mine - 1) * vstep];
    };

    // RoPE factors first: loads complete in issue order, so a load issued after
    // the cache rows' would wait for all of them
    const float rc = t < half ? a.rope_cos[t] : 0.0f, rsn = t < half ? a.rope_sin[t] : 0.0f;
    // the 3 hd words of this head: q, then k, then v. The waves that hold none
    // of them issue their loads of the first chunk's cache rows (which do not
    // depend on this step's q, k, v) before the wait; the polling waves after
    // it, since a poll issued behind those loads would wait for them. The
    // failure vote is an LDS word read after the next LDS-only barrier, which
    // unlike __syncthreads leaves the early loads in flight.
    const int n = 3 * hd;
    const bool poller = (t >> 6) * 64 < n;  // uniform in a wave
    const int lim0 = min(len, pos - split * len);
    if (!poller && lim0 > 0) {
        load_k(split * len, lim0, 0);
        load_v(split * len, lim0, 0);
    }
    const long long t_start = (long long)__builtin_amdgcn_s_memrealtime();
    uint32_t w[2] = {0u, 0u};
    bool failed = false;
    if (poller) {
        for (int spin = 0;; ++spin) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int u = min(t + kT * i, n - 1);
                const int seg = u / hd;
                w[i] = __hip_atomic_load(qq_cur + seg * D + h * hd + (u - seg * hd), __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
            }
            if (w[0] != 0u && w[1] != 0u) break;
            if ((spin & 15) == 15 &&
                (status_load(a.ctrl) != 0 ||
                 (long long)__builtin_amdgcn_s_memrealtime() - t_start > kTimeoutTicks)) {
                failed = true;
                break;
            }
            __builtin_amdgcn_s_sleep(3);
        }
    }
    if (failed) {
        s.vote = E2;
        __hip_atomic_fetch_or(a.ctrl + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (poller && lim0 > 0) {
        load_k(split * len, lim0, 0);
        load_v(split * len, lim0, 0);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int u = t + kT * i;
        if (u < n) {
            // q, k, v are (acc - sum q) / (s_a s_w) with a positive divisor and so
            // never -0.0: the word -0.0 is the published +0.0
            const float x = w[i] == 0x80000000u ? 0.0f : __uint_as_float(w[i]);
            const int seg = u / hd, i_ = u - seg * hd;
            (seg == 0 ? s.q : seg == 1 ? s.k : s.v)[i_] = x;
        }
    }
    lds_sync();
    if (s.vote == E2) return false;  // a poller's wait failed (uniform: one LDS word)
    // RoPE of q and k (each thread its own pair); the split of the last chunk
    // writes k and v at position pos of the caches
    if (t < half) {
        const float c = rc, sn = rsn;
        {
            const float x0 = s.q[2 * t], x1 = s.q[2 * t + 1];
            const float ac = x0 * c, bs = x1 * sn, as = x0 * sn, bc = x1 * c;
            s.q[2 * t] = ac - bs;
            s.q[2 * t + 1] = as + bc;
        }
        {
            const float x0 = s.k[2 * t], x1 = s.k[2 * t + 1];
            const float ac = x0 * c, bs = x1 * sn, as = x0 * sn, bc = x1 * c;
            s.k[2 * t] = ac - bs;
            s.k[2 * t + 1] = as + bc;
        }
        if (split == last) {
            float* krow = a.k_cache + (((size_t)l * a.heads + h) * a.max_seq + pos) * hd;
            float* vrow = a.v_cache + (((size_t)l * a.heads + h) * a.max_seq + pos) * hd;
            krow[2 * t] = s.k[2 * t];
            krow[2 * t + 1] = s.k[2 * t + 1];
            vrow[2 * t] = s.v[2 * t];
            vrow[2 * t + 1] = s.v[2 * t + 1];
        }
    }
    lds_sync();
    const float scale = 1.0f / sqrtf((float)hd);
    // run of float4 f = t + 512 i within its row: f mod h4, advanced by 512 mod h4 per i
    const int c4_first = t % h4, c4_step = kT % h4;
    for (int c = split; c < nch; c += G) {
        const int j0 = c * len, cnt = min(len, pos + 1 - j0);
        const int lim = min(len, pos - j0);  // cache rows of the chunk (position pos is not one)
        const int nf = lim * h4;
        if (c != split && lim > 0) {
            load_k(j0, lim, 0);
            load_v(j0, lim, 0);
        }
        // q . k over each run of four values of the cache rows
        int c4 = c4_first;
        for (int f0 = 0; f0 < nf; f0 += kT * kAttnKB) {
            if (f0 > 0) load_k(j0, lim, f0);
#pragma unroll
            for (int i = 0; i < kAttnKB; ++i) {
                const int f = f0 + t + kT * i;
                if (f < nf) {
                    const float4 qv = *reinterpret_cast<const float4*>(s.q + 4 * c4);
                    s.kp[f] = ((qv.x * kr[i].x + qv.y * kr[i].y) + qv.z * kr[i].z) + qv.w * kr[i].w;
                }
                c4 += c4_step;
                if (c4 >= h4) c4 -= h4;
            }
        }
        if (lim < cnt && t < h4) {
            // position pos (row lim of the chunk), from LDS: its cache row is being written now
            const float4 qv = *reinterpret_cast<const float4*>(s.q + 4 * t);
            const float4 kv = *reinterpret_cast<const float4*>(s.k + 4 * t);
            s.kp[nf + t] = ((qv.x * kv.x + qv.y * kv.y) + qv.z * kv.z) + qv.w * kv.w;
        }
        lds_sync();
        float sc = -INFINITY;
        if (t < cnt) {
            float dot = 0.0f;
            const float* pr = s.kp + t * h4;
#pragma unroll 8
            for (int m = 0; m < h4; ++m) dot += pr[m];
            sc = dot * scale;
        }
        const float mx = block_max_f(sc, s.red);
        if (t < kAttnChunk) s.e[t] = t < cnt ? expf(sc - mx) : 0.0f;
        const float sum = block_sum_f(t < cnt ? s.e[t] : 0.0f, s.red);  // its barriers also publish e[]
        // positions j0 + jj, jj = g, g + groups, ... ascending: the cache rows,
        // then position pos (always the last one) from LDS
        const int mine = (g < groups && lim > g) ? (lim - g + groups - 1) / groups : 0;
        float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        for (int u0 = 0; u0 < mine; u0 += kAttnVB) {
            if (u0 > 0) load_v(j0, lim, u0);
#pragma unroll
            for (int u = 0; u < kAttnVB; ++u)
                if (u0 + u < mine) {
                    const float e = s.e[g + (u0 + u) * groups];
                    acc.x += e * vr[u].x;
                    acc.y += e * vr[u].y;
                    acc.z += e * vr[u].z;
                    acc.w += e * vr[u].w;
                }
        }
        if (g < groups) {
            const int jj = g + mine * groups;  // my first position not in the cache rows
            if (jj == pos - j0 && jj < cnt) {  // pos lies in this chunk
                const float e = s.e[jj];
                const float4 vv = *reinterpret_cast<const float4*>(s.v + 4 * c4v);
                acc.x += e * vv.x;
                acc.y += e * vv.y;
                acc.z += e * vv.z;
                acc.w += e * vv.w;
            }
            *reinterpret_cast<float4*>(s.part + g * hd + 4 * c4v) = acc;
        }
        lds_sync();
        float* cp = s.chunk[split == 0 ? c : 0];
        if (t < hd) {
            float acc2 = 0.0f;
            for (int q = 0; q < groups; ++q) acc2 += s.part[q * hd + t];
            cp[2 + t] = acc2;
        }
        if (t == 0) {
            cp[0] = mx;
            cp[1] = sum;
        }
        if (split != 0) {
            // publish the chunk's partials: [max, sum, hd weighted sums]
            lds_sync();
            unsigned long long* dst = a.apart + ((size_t)h * a.chunks_max + c) * (hd + 2);
            if (t < hd + 2) ll_store(dst + t, cp[t], E2);
        }
        // the next chunk's first writes (kp[], e[], part[], the chunk slot) follow
        // at least one barrier after this chunk's last reads of them
    }
    if (split != 0) return true;
    // split 0: the other chunks' partials, then the merge and the head's output
    const int others = nch - (nch + G - 1) / G;  // chunks held by splits 1 .. G-1
    if (others > 0) {
        // word u of the chunks c % G != 0, in chunk order; each round issues
        // all of its loads before it checks any
        const int nw = others * (hd + 2);
        constexpr int kMW = 4;
        const long long t0 = (long long)__builtin_amdgcn_s_memrealtime();
        for (int spin = 0;; ++spin) {
            bool ready = true;
            for (int u0 = 0; u0 < nw; u0 += kT * kMW) {
                unsigned long long v[kMW];
#pragma unroll
                for (int i = 0; i < kMW; ++i) {
                    const int u = min(u0 + t + kT * i, nw - 1);
                    const int oc = u / (hd + 2), wi = u - oc * (hd + 2);
                    const int c = oc + oc / (G - 1) + 1;
                    v[i] = ll_load(a.apart + ((size_t)h * a.chunks_max + c) * (hd + 2) + wi);
                }
#pragma unroll
                for (int i = 0; i < kMW; ++i) {
                    const int u = u0 + t + kT * i;
                    if (u < nw) {
                        const int oc = u / (hd + 2), wi = u - oc * (hd + 2);
                        const int c = oc + oc / (G - 1) + 1;
                        if ((uint32_t)(v[i] >> 32) != E2)
                            ready = false;
                        else
                            s.chunk[c][wi] = __uint_as_float((uint32_t)v[i]);
                    }
                }
            }
            // one vote per round, bit 0: a word not yet written, bit 1: gave up.
            // Lane 0 of each wave stores its wave's flags in this round's words
            // (alternating by round: a wave writes a round's words again only
            // after the next round's barrier, which every wave reaches after
            // reading them); all ready ends the wait even if a thread gave up.
            const bool gave_up = (spin & 15) == 15 && (status_load(a.ctrl) != 0 ||
                                 (long long)__builtin_amdgcn_s_memrealtime() - t0 > kTimeoutTicks);
            uint32_t* words = s.merge_vote[spin & 1];
            const uint32_t wf = (__ballot(!ready) != 0ull ? 1u : 0u) | (__ballot(gave_up) != 0ull ? 2u : 0u);
            if ((t & 63) == 0) words[t >> 6] = wf;
            lds_sync();
            uint32_t any = 0u;
#pragma unroll
            for (int i = 0; i < kT / 64; ++i) any |= words[i];
            if (!(any & 1u)) break;
            if (any & 2u) {
                if (t == 0) __hip_atomic_fetch_or(a.ctrl + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                return false;
            }
            __builtin_amdgcn_s_sleep(3);
        }
    }
    __syncthreads();
    if (t < hd) {
        float mx = -INFINITY;
        for (int c = 0; c < nch; ++c) mx = fmaxf(mx, s.chunk[c][0]);
        float den = 0.0f, acc = 0.0f;
        for (int c = 0; c < nch; ++c) den += s.chunk[c][1] * expf(s.chunk[c][0] - mx);
        for (int c = 0; c < nch; ++c) acc += s.chunk[c][2 + t] * expf(s.chunk[c][0] - mx);
        const float out = acc / den;
        val_store(ao_cur + h * hd + t, out);
        val_clear(ao_old + h * hd + t);
        if (a.attn) a.attn[(size_t)l * D + h * hd + t] = out;
    }
    return true;
}

// With ON, keeps v computed where this stands: an empty asm that claims to
// read and write it, so the compiler does not sink the computation (a
// correctly rounded division) into an epilogue behind the next barrier, where
// it would sit on the path to the published words; placed before the dot
// products, it overlaps them. The form with attention, whose registers are at
// the limit, came out slower with it and leaves it off.
template <bool ON, class T>
__device__ __forceinline__ void pin(T& v)
{
    if constexpr (ON) asm volatile("" : "+v"(v));
}

template <int D, int F, bool ATTN>
__global__ __launch_bounds__(kT) void stream_kernel(StreamArgs a)
{
    using S1 = Step<3 * D, D, 1>;  // q, k, v stacked
    using S2 = Step<D, D, 1>;      // o (and the rows of x this workgroup owns)
    using S3 = Step<F, D, 2>;      // gate rows, then up rows
    using S4 = Step<D, F, 1>;      // down
    static_assert(S2::R == S4::R, "o and down share their rows");
    constexpr int ND = cdiv(D, kT), NF = cdiv(F, kT);
    constexpr size_t dd = (size_t)D * D / 4, fd = (size_t)F * D / 4;
    constexpr size_t blob = 4 * dd + 3 * fd;

    __shared__ Shared sh;
    __shared__ std::conditional_t<ATTN, AttnShared, NoAttnShared> ash;
    const int w = blockIdx.x, t = threadIdx.x;

    const uint32_t base = __hip_atomic_load(a.ctrl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (status_load(a.ctrl) != 0) return;  // a failed call left stale flags: the workspace must be re-zeroed
    if ((unsigned long long)base + 4ull * (unsigned long long)a.n_layers + 8ull >= 0x80000000ull) {
        if (w == 0 && t == 0) __hip_atomic_fetch_or(a.ctrl + 1, 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }

    const int r1 = w * S1::R, r2 = w * S2::R, r3 = w * S3::R;
    // epilogue thread t < R owns row t of the step
    const bool e1 = t < S1::R, e2 = t < S2::R, e3 = t < S3::R;
    if (t < 16) reinterpret_cast<uint32_t*>(sh.zero)[t] = 0u;  // visible after the first barrier
    if constexpr (ATTN) {
        if (t == 0) ash.vote = 0u;  // likewise, long before the first attention phase
    }

    float xres = e2 ? a.x[r2 + t] : 0.0f;  // residual x of this workgroup's rows
    float s_a;
    int qsum;

    // The weight rows, gains and stand-in input of a step are loaded when the
    // step starts, before its wait: the fetch overlaps the hand-over. A wave's
    // loads complete in issue order, so a poll also waits for every load issued
    // before it: loading P3's or P4's rows into registers a step earlier
    // measured slower; their lines are prefetched into L2 instead (pf*).
    uint4 w1[S1::P], w2[S2::P], w3[S3::P], w4[S4::P];
    float g1[ND], g2[ND], g3[ND], g4[NF], zv[ND];
    auto fetch2 = [&](int l) {
        const uint8_t* W = a.weights + (size_t)l * blob + 3 * dd + (size_t)r2 * (D / 4);
        load_items<S2>(w2, [&](int r) { return W + (size_t)r * (D / 4); });
    };
    auto fetch1 = [&](int l) {
        // q, k, v are consecutive D x D/4 matrices: stacked row r is at r * D/4
        const uint8_t* W = a.weights + (size_t)l * blob + (size_t)r1 * (D / 4);
        load_items<S1>(w1, [&](int r) { return W + (size_t)r * (D / 4); });
        load_strided<D>(a.gains + (size_t)l * (3 * D + F), g1);
        // P2's gains and stand-in input (its norm + quant follows the wait for P1)
        load_strided<D>(a.gains + (size_t)l * (3 * D + F) + D, g2);
        if constexpr (!ATTN) load_strided<D>(a.z + (size_t)l * D, zv);
    };
    auto fetch3 = [&](int l) {
        const uint8_t* W = a.weights + (size_t)l * blob + 4 * dd + (size_t)r3 * (D / 4);
        load_items<S3>(w3, [&](int r) {
            return r < S3::R ? W + (size_t)r * (D / 4) : W + fd + (size_t)(r - S3::R) * (D / 4);
        });
        load_strided<D>(a.gains + (size_t)l * (3 * D + F) + 2 * D, g3);
    };
    auto fetch4 = [&](int l) {
        const uint8_t* W = a.weights + (size_t)l * blob + 4 * dd + 2 * fd + (size_t)r2 * (F / 4);
        load_items<S4>(w4, [&](int r) { return W + (size_t)r * (F / 4); });
        load_strided<F>(a.gains + (size_t)l * (3 * D + F) + 3 * D, g4);
    };
    const uint32_t trash = (uint32_t)(uintptr_t)&sh.trash[0];
    auto pf1q = [&](int l) {  // q, k, v rows of layer l
        prefetch_span<S1::R * (D / 4)>(a.weights + (size_t)l * blob + (size_t)r1 * (D / 4), trash);
    };
    auto pf1o = [&](int l) {  // o rows of layer l
        prefetch_span<S2::R * (D / 4)>(a.weights + (size_t)l * blob + 3 * dd + (size_t)r2 * (D / 4), trash);
    };
    auto pf3 = [&](int l) {  // gate and up rows of layer l
        const uint8_t* W = a.weights + (size_t)l * blob + 4 * dd + (size_t)r3 * (D / 4);
        prefetch_span<S3::R * (D / 4)>(W, trash);
        prefetch_span<S3::R * (D / 4)>(W + fd, trash);
    };
    auto pf4 = [&](int l) {  // down rows of layer l
        prefetch_span<S4::R * (F / 4)>(a.weights + (size_t)l * blob + 4 * dd + 2 * fd + (size_t)r2 * (F / 4), trash);
    };
    for (int l = 0; l < a.n_layers; ++l) {
        [[maybe_unused]] const uint32_t E = base + 4u * (uint32_t)l;
        float sw[7];  // this layer's weight scales
#pragma unroll
        for (int i = 0; i < 7; ++i) sw[i] = a.scales[7 * l + i];
        float* qkv = a.qkv + (size_t)l * a.qkv_layer_stride;
        // copy of the published vectors written in this layer (the phase
        // counter makes the alternation continue across calls)
        const int cp = (int)(((base >> 2) + (uint32_t)l) & 1u);
        uint32_t* xa_in = a.xa + (cp ^ 1) * D;  // written by the previous layer's P4
        uint32_t* xa_out = a.xa + cp * D;
        uint32_t* xb_cur = a.xb + cp * D;
        uint32_t* xb_old = a.xb + (cp ^ 1) * D;
        uint32_t* hh_cur = a.hh + cp * F;
        uint32_t* hh_old = a.hh + (cp ^ 1) * F;
        uint32_t* qq_cur = a.qq + cp * 3 * D;
        uint32_t* qq_old = a.qq + (cp ^ 1) * 3 * D;
        uint32_t* ao_cur = a.ao + cp * D;
        uint32_t* ao_old = a.ao + (cp ^ 1) * D;

        // ---- P1: q, k, v ----
        {
            if (t < S1::R) sh.acc[t] = 0;
            fetch1(l);
            float v[ND];
            if (l == 0) {
                load_strided<D>(a.x, v);
            } else if (!poll_val<D>(xa_in, v, a.ctrl, sh.vote)) {
                return;
            }
            norm_quant<D>(v, g1, a.eps, sh, s_a, qsum);
            const int mat1 = (r1 + t) / D;
            float inv = 1.0f / (s_a * (mat1 == 0 ? sw[0] : (mat1 == 1 ? sw[1] : sw[2])));
            pin<!ATTN>(inv);
            pin<!ATTN>(qsum);
            dots<S1>(w1, sh.q, sh.zero, sh.acc);
            __syncthreads();
            if (e1) {
                const int row = r1 + t;
                const float val = (float)(sh.acc[t] - qsum) * inv;
                qkv[row] = val;
                if constexpr (ATTN) {
                    val_store(qq_cur + row, val);
                    val_clear(qq_old + row);
                }
            }
            if constexpr (!ATTN) {
                if (t == 0) ll_store(a.done + kFlagStride * w, 0.0f, E + 1);
            }
        }
        // ---- PA: attention, G = 256 / heads workgroups per head ----
        if constexpr (ATTN) {
            const int G = kGrid / a.heads, len = attn_chunk_len(a.pos, G), nch = (a.pos + len) / len;
            if (w < a.heads * G && w % G < nch &&
                !attention_split<D>(a, l, w / G, w % G, G, E + 2, qq_cur, ao_cur, ao_old, ash))
                return;
        }
        // ---- P2: o projection of the stand-in z, residual ----
        {
            // z stands in for the attention output, which exists only once
            // every workgroup has finished P1: its norm + quant follows the wait
            if (t < S2::R) sh.acc[t] = 0;
            fetch2(l);
            float ov[ND];
            if constexpr (ATTN) {
                // the attention output of every head (each head's inputs came
                // from P1 rows of many workgroups, so every workgroup has
                // published P1, and read the base, by now)
                if (!poll_val<D>(ao_cur, ov, a.ctrl, sh.vote)) return;
            } else {
                float fl[1];
                if (!poll_vec<kGrid, kFlagStride>(a.done, E + 1, fl, a.ctrl, sh.vote)) return;
            }
            pf3(l);
            if (l == 0 && w == 0 && t == 0)  // every workgroup has read the base by now
                __hip_atomic_store(a.ctrl, base + 4u * (uint32_t)a.n_layers, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            if constexpr (ATTN)
                norm_quant<D>(ov, g2, a.eps, sh, s_a, qsum);
            else
                norm_quant<D>(zv, g2, a.eps, sh, s_a, qsum);
            float inv = 1.0f / (s_a * sw[3]);
            pin<!ATTN>(inv);
            pin<!ATTN>(qsum);
            dots<S2>(w2, sh.q, sh.zero, sh.acc);
            __syncthreads();
            if (e2) {
                xres = xres + (float)(sh.acc[t] - qsum) * inv;
                val_store(xb_cur + r2 + t, xres);
                val_clear(xb_old + r2 + t);
            }
        }
        // ---- P3: gate/up with relu(gate)^2 * up ----
        {
            if (t < S3::R) {
                sh.acc[t] = 0;
                sh.acc[S3::R + t] = 0;
            }
            fetch3(l);
            float v[ND];
            if (!poll_val<D>(xb_cur, v, a.ctrl, sh.vote)) return;
            pf4(l);
            if (l + 1 < a.n_layers) pf1o(l + 1);
            norm_quant<D>(v, g3, a.eps, sh, s_a, qsum);
            float inv_g = 1.0f / (s_a * sw[4]), inv_u = 1.0f / (s_a * sw[5]);
            pin<!ATTN>(inv_g);
            pin<!ATTN>(inv_u);
            pin<!ATTN>(qsum);
            dots<S3>(w3, sh.q, sh.zero, sh.acc);
            __syncthreads();
            if (e3) {
                const float gate = (float)(sh.acc[t] - qsum) * inv_g;
                const float up = (float)(sh.acc[S3::R + t] - qsum) * inv_u;
                const float gp = gate > 0.0f ? gate : 0.0f;
                const float g2v = gp * gp;
                val_store(hh_cur + r3 + t, g2v * up);
                val_clear(hh_old + r3 + t);
            }
        }
        // ---- P4: down projection of h, residual ----
        {
            if (t < S4::R) sh.acc[t] = 0;
            fetch4(l);
            float v[NF];
            if (!poll_val<F>(hh_cur, v, a.ctrl, sh.vote)) return;
            if (l + 1 < a.n_layers) pf1q(l + 1);
            norm_quant<F>(v, g4, a.eps, sh, s_a, qsum);
            float inv = 1.0f / (s_a * sw[6]);
            pin<!ATTN>(inv);
            pin<!ATTN>(qsum);
            dots<S4>(w4, sh.q, sh.zero, sh.acc);
            __syncthreads();
            if (e2) {
                xres = xres + (float)(sh.acc[t] - qsum) * inv;
                val_store(xa_out + r2 + t, xres);
                val_clear(xa_in + r2 + t);
                if (l == a.n_layers - 1) a.x[r2 + t] = xres;
            }
        }
    }
}

using StreamFn = void (*)(StreamArgs);

// Shapes with a compiled kernel: BitNet-3B, BitNet-1.3B and a small test shape.
StreamFn stream_fn(int d, int f, bool attn)
{
    if (d == 2560 && f == 10240) return attn ? stream_kernel<2560, 10240, true> : stream_kernel<2560, 10240, false>;
    if (d == 2048 && f == 8192) return attn ? stream_kernel<2048, 8192, true> : stream_kernel<2048, 8192, false>;
    if (d == 256 && f == 1024) return attn ? stream_kernel<256, 1024, true> : stream_kernel<256, 1024, false>;
    return nullptr;
}

struct DeviceInfo {
    int cus = 0;
};

DeviceInfo device_info()
{
    static DeviceInfo cache[64];
    static bool have[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return DeviceInfo{};
    if (!have[dev]) {
        DeviceInfo info;
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess) info.cus = v;
        cache[dev] = info;
        have[dev] = true;
    }
    return cache[dev];
}

// Whether every CU can hold one workgroup of the kernel (registers, LDS, waves).
bool one_per_cu(StreamFn fn)
{
    int blocks = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, reinterpret_cast<const void*>(fn), kT, 0) !=
        hipSuccess)
        return false;
    return blocks >= 1;
}

}  // namespace

bool stream_persistent_fits(int m, int d, int f, const StreamAttn* attn)
{
    if (m != 1) return false;
    if (attn && (attn->heads < 1 || attn->heads > kGrid || d % attn->heads != 0 || (d / attn->heads) % 4 != 0 ||
                 d / attn->heads > kMaxHd || attn->max_seq > kMaxAttnChunks * kAttnChunk))
        return false;
    const StreamFn fn = stream_fn(d, f, attn != nullptr);
    if (!fn) return false;
    const DeviceInfo info = device_info();
    return info.cus >= kGrid && one_per_cu(fn);
}

int launch_stream_persistent(const uint8_t* weights, const float* scales, const float* gains, const float* z,
                             int n_layers, int d, int f, float eps, float* x, float* qkv, long long qkv_stride,
                             void* ll_region, uint32_t* ctrl, const StreamAttn* attn, hipStream_t s)
{
    const StreamFn fn = stream_fn(d, f, attn != nullptr);
    if (!fn) return BL_ERR_SHAPE;
    StreamArgs a;
    a.weights = weights;
    a.scales = scales;
    a.gains = gains;
    a.z = z;
    a.x = x;
    a.qkv = qkv;
    a.qkv_layer_stride = qkv_stride;
    // 8-byte flag words first, then two copies of each published vector
    unsigned long long* ll = static_cast<unsigned long long*>(ll_region);
    a.done = ll;
    uint32_t* vec = reinterpret_cast<uint32_t*>(ll + (size_t)kGrid * kFlagStride);
    a.xa = vec;
    a.xb = vec + 2 * d;
    a.hh = vec + 4 * d;
    a.qq = vec + 4 * d + 2 * f;
    a.ao = vec + 10 * d + 2 * f;
    a.ctrl = ctrl;
    a.n_layers = n_layers;
    a.eps = eps;
    a.rope_cos = a.rope_sin = nullptr;
    a.k_cache = a.v_cache = a.attn = nullptr;
    a.apart = nullptr;
    a.heads = a.hd = a.max_seq = a.pos = a.chunks_max = 0;
    if (attn) {
        const int hd = d / attn->heads;
        a.rope_cos = attn->rope_cos + (size_t)attn->pos * (hd / 2);
        a.rope_sin = attn->rope_sin + (size_t)attn->pos * (hd / 2);
        a.k_cache = attn->k_cache;
        a.v_cache = attn->v_cache;
        a.attn = attn->attn;
        a.heads = attn->heads;
        a.hd = hd;
        a.max_seq = attn->max_seq;
        a.pos = attn->pos;
        a.apart = static_cast<unsigned long long*>(attn->part);
        a.chunks_max = kMaxAttnChunks;
    }
    // A plain launch: with at least kGrid CUs that each fit one workgroup, all
    // kGrid workgroups are resident together on a device that runs nothing
    // else. Should one not become resident (another queue holding CUs), the
    // others' waits time out and set the status word: the kernel ends early
    // and never hangs. (A cooperative launch would make residency a launch
    // condition, but its runtime state made profiled processes crash at exit.)
    fn<<<dim3(kGrid), dim3(kT), 0, s>>>(a);
    return hipGetLastError() == hipSuccess ? BL_OK : BL_ERR_LAUNCH;
}

// 8-byte words: the flags, then two copies each of x (twice), h, q/k/v and the
// attention output as 4-byte words
size_t stream_ll_words(int d, int f) { return (size_t)6 * d + f + (size_t)kGrid * kFlagStride; }

}  // namespace bl
