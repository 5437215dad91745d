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
// attention over all heads in the full model.
//
// At one token every step is a short weight stream (1.6 to 13 MB) whose input
// is a vector produced by all CUs in the step before. Launching a kernel per
// step pays the kernel start and the HBM latency ramp 128 times per token. Here
// one workgroup per CU (256 on an MI355X) stays resident for the whole token:
//   - each workgroup owns fixed output rows of every step and issues the loads
//     of those weight rows (and of the step's RMSNorm gains) before it waits
//     for the step's input, so the weight fetch overlaps the hand-over;
//   - a step's output vector is published as 64-bit words {fp32 value, epoch}
//     written with device-scope atomic stores; a consumer loads all words of
//     the vector it needs in one batch and repeats until every epoch matches.
//     Value and flag travel in one single-copy-atomic store, so no fence or
//     separate barrier is needed;
//   - every workgroup then computes the RMSNorm + activation quant of the full
//     vector itself, so no extra round trip is spent on broadcasting q. The
//     sum of squares keeps the fixed fp64 order of quant.hip: with the vector
//     staged in LDS, thread l < 256 sums x[k]^2 for k = l, l+256, ... in
//     ascending k, then an xor-butterfly combines the 256 partials (offsets 128
//     and 64 through LDS, 32..1 with exact lane exchanges);
//   - the dot products are those of gemv.hip (dot4 on shifted code masks
//     against activations permuted once into LDS). Each row of a step gets
//     floor(1024 / rows) lanes, and the lanes' partial sums meet in LDS through
//     int32 atomic adds, which are exact in any order.
// A workgroup has 1024 threads (4 waves per SIMD), so the vector work of a step
// is spread over 4x the lanes of a one-wave-per-SIMD layout and its latencies
// overlap.
// The P2/P4 rows of a workgroup are the same, so the residual x of its rows
// stays in registers across the whole stream.
//
// Termination: every wait is bounded by a wall-clock limit (s_memrealtime,
// 100 MHz) and by a shared status word; a workgroup that gives up sets the
// status, every other one sees it and leaves, so the grid always drains.
#include "internal.h"
#include "wave.h"

namespace bl {
namespace {

constexpr int kT = 512;      // threads per workgroup: 8 waves, 2 per SIMD; also the
                             // number of RMSNorm partial sums of the fixed order
constexpr int kGrid = 256;   // workgroups: one per CU of an MI355X
constexpr uint32_t kCodeMask = 0x03030303u;
constexpr long long kTimeoutTicks = 200000000LL;  // 2 s at 100 MHz
constexpr int kMaxK = 10240;

constexpr int cdiv(int a, int b) { return (a + b - 1) / b; }

// Geometry of one step: N output rows of K inputs spread over kGrid
// workgroups; lanes per row and 16-byte chunks per lane.
template <int N, int K>
struct Step {
    static constexpr int R = cdiv(N, kGrid);  // rows per workgroup
    static constexpr int Lr = kT / R;         // lanes per row
    static constexpr int C = K / 64;          // chunks per row
    static constexpr int CL = cdiv(C, Lr);    // chunks per lane
    static_assert(R >= 1 && R <= 64, "rows per workgroup");
    static_assert(Lr >= 1, "lanes per row");
    static_assert(K % 64 == 0 && K <= kMaxK, "K");
};

struct StreamArgs {
    const uint8_t* weights;
    const float* scales;
    const float* gains;
    const float* z;
    float* x;
    float* qkv;
    long long qkv_layer_stride;  // elements between layers (0: scratch reused)
    unsigned long long* xa;      // x at layer start (published by P4)
    unsigned long long* xb;      // x after the o residual (published by P2)
    unsigned long long* hh;      // h (published by P3)
    unsigned long long* done;    // per-workgroup "P1 finished" flags
    uint32_t* ctrl;              // [0] epoch base, [1] status
    int n_layers;
    float eps;
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

__device__ __forceinline__ uint32_t status_load(const uint32_t* ctrl)
{
    return __hip_atomic_load(ctrl + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Loads the words k = t, t + 1024, ... < N of buf until every one carries epoch
// e (all loads of a round are issued before any is checked); v receives the
// fp32 payloads. Returns false, for the whole workgroup, on a timeout or when
// another workgroup gave up.
template <int N>
__device__ bool poll_vec(const unsigned long long* buf, uint32_t e, float* v, uint32_t* ctrl, long long t_start)
{
    constexpr int NI = cdiv(N, kT);
    const int t = threadIdx.x;
    unsigned long long w[NI];
    bool failed = false;
    for (int spin = 0;; ++spin) {
        // every load is unconditional (clamped address) so that the whole batch
        // is in flight before the first wait
#pragma unroll
        for (int i = 0; i < NI; ++i) w[i] = ll_load(buf + min(t + kT * i, N - 1));
        bool ready = true;
#pragma unroll
        for (int i = 0; i < NI; ++i) ready = ready && (uint32_t)(w[i] >> 32) == e;
        if (ready) break;
        if ((spin & 15) == 15 &&
            (status_load(ctrl) != 0 || (long long)__builtin_amdgcn_s_memrealtime() - t_start > kTimeoutTicks)) {
            failed = true;
            break;
        }
        __builtin_amdgcn_s_sleep(2);
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) v[i] = (t + kT * i < N) ? __uint_as_float((uint32_t)w[i]) : 0.0f;
    if (__syncthreads_or(failed ? 1 : 0)) {
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

__device__ __forceinline__ int quant_one(float y, float scale)
{
    const float r = rintf(y * scale);
    return (int)fminf(fmaxf(r, -128.0f), 127.0f);
}

// Byte position of activation k in the permuted LDS layout (per 16 values,
// dword j holds k0+j, k0+4+j, k0+8+j, k0+12+j).
__device__ __forceinline__ int perm_pos(int k) { return (k & ~15) | ((k & 3) << 2) | ((k >> 2) & 3); }

struct Shared {
    __attribute__((aligned(16))) uint8_t q[kMaxK];  // quantized input vector, permuted
    double red_d[kT / 64];
    float red_f[kT / 64];
    int red_i[kT / 64];
    int acc[128];  // per-row accumulators of a step (gate rows, then up rows)
};

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
            const int qv = quant_one(y[i], scale);
            sum += qv;
            sh.q[perm_pos(k)] = (uint8_t)(qv & 0xff);
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

__device__ __forceinline__ int dot16(uint32_t p, const uint4 q, int acc)
{
    acc = __builtin_amdgcn_sdot4((int)(p & kCodeMask), (int)q.x, acc, false);
    acc = __builtin_amdgcn_sdot4((int)((p >> 2) & kCodeMask), (int)q.y, acc, false);
    acc = __builtin_amdgcn_sdot4((int)((p >> 4) & kCodeMask), (int)q.z, acc, false);
    acc = __builtin_amdgcn_sdot4((int)((p >> 6) & kCodeMask), (int)q.w, acc, false);
    return acc;
}

// One lane's part of a step: row ri = t / Lr of the workgroup's rows, chunks
// j, j + Lr, ... of that row (j = t % Lr).
template <class S>
struct Lane {
    int ri, j;
    bool active;
    __device__ Lane(int row0, int n_rows)
    {
        ri = threadIdx.x / S::Lr;
        j = threadIdx.x % S::Lr;
        active = ri < S::R && row0 + ri < n_rows;
    }
};

// rowp must point at a valid row even for inactive lanes (the caller clamps
// the row); chunks past the row end re-read its last chunk. Loads are
// unconditional so that they all issue before the first wait; dot_row ignores
// what inactive lanes and excess chunks loaded.
template <class S>
__device__ __forceinline__ void load_row(const uint8_t* rowp, const Lane<S>& ln, uint4* w)
{
#pragma unroll
    for (int c = 0; c < S::CL; ++c) {
        const int ch = min(ln.j + c * S::Lr, S::C - 1);
        w[c] = *reinterpret_cast<const uint4*>(rowp + (size_t)ch * 16);
    }
}

template <class S>
__device__ __forceinline__ int dot_row(const uint4* w, const Lane<S>& ln, const uint8_t* q)
{
    int acc = 0;
#pragma unroll
    for (int c = 0; c < S::CL; ++c) {
        const int ch = ln.j + c * S::Lr;
        if (S::CL * S::Lr <= S::C || ch < S::C) {  // the test folds away when every lane's chunks exist
            const uint4* qp = reinterpret_cast<const uint4*>(q + (size_t)ch * 64);
            acc = dot16(w[c].x, qp[0], acc);
            acc = dot16(w[c].y, qp[1], acc);
            acc = dot16(w[c].z, qp[2], acc);
            acc = dot16(w[c].w, qp[3], acc);
        }
    }
    return acc;
}

template <int D, int F>
__global__ __launch_bounds__(kT) void stream_kernel(StreamArgs a)
{
    using S1 = Step<3 * D, D>;  // q, k, v
    using S2 = Step<D, D>;      // o (and the rows of x this workgroup owns)
    using S3 = Step<F, D>;      // gate / up
    using S4 = Step<D, F>;      // down
    static_assert(S2::R == S4::R, "o and down share their rows");
    static_assert(2 * S3::R <= 128 && S1::R <= 128, "LDS accumulators");
    constexpr int ND = cdiv(D, kT), NF = cdiv(F, kT);
    constexpr size_t dd = (size_t)D * D / 4, fd = (size_t)F * D / 4;
    constexpr size_t blob = 4 * dd + 3 * fd;

    __shared__ Shared sh;
    const int w = blockIdx.x, t = threadIdx.x;
    const long long t_start = (long long)__builtin_amdgcn_s_memrealtime();

    const uint32_t base = __hip_atomic_load(a.ctrl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (status_load(a.ctrl) != 0) return;  // a failed call left stale flags: the workspace must be re-zeroed
    if ((unsigned long long)base + 4ull * (unsigned long long)a.n_layers + 8ull >= 0x80000000ull) {
        if (w == 0 && t == 0) __hip_atomic_fetch_or(a.ctrl + 1, 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }

    const int r1 = w * S1::R, r2 = w * S2::R, r3 = w * S3::R;
    const Lane<S1> l1(r1, 3 * D);
    const Lane<S2> l2(r2, D);
    const Lane<S3> l3(r3, F);
    const Lane<S4> l4(r2, D);
    // epilogue thread t < R owns row t of the step
    const bool e1 = t < S1::R && r1 + t < 3 * D, e2 = t < S2::R && r2 + t < D, e3 = t < S3::R && r3 + t < F;

    float xres = e2 ? a.x[r2 + t] : 0.0f;  // residual x of this workgroup's rows
    float s_a;
    int qsum;

    // The weight rows, gains and stand-in input of a step are loaded when the
    // step starts, before its wait: the fetch overlaps the hand-over. (Loading
    // a step earlier does not pay: a wave's loads complete in issue order, so
    // every later wait would also wait for the early loads.)
    uint4 w1[S1::CL], w2[S2::CL], wg[S3::CL], wu[S3::CL], w4[S4::CL];
    float g1[ND], g2[ND], g3[ND], g4[NF], zv[ND];
    auto fetch1 = [&](int l) {
        const uint8_t* W = a.weights + (size_t)l * blob;
        const int row = l1.active ? r1 + l1.ri : 0;
        const int mat = row / D, rin = row - mat * D;
        load_row<S1>(W + mat * dd + (size_t)rin * (D / 4), l1, w1);
        load_strided<D>(a.gains + (size_t)l * (3 * D + F), g1);
        // P2's gains and stand-in input: its norm + quant runs right after P1
        load_strided<D>(a.gains + (size_t)l * (3 * D + F) + D, g2);
        load_strided<D>(a.z + (size_t)l * D, zv);
    };
    auto fetch2 = [&](int l) {
        const uint8_t* W = a.weights + (size_t)l * blob;
        load_row<S2>(W + 3 * dd + (size_t)(l2.active ? r2 + l2.ri : 0) * (D / 4), l2, w2);
    };
    auto fetch3 = [&](int l) {
        const uint8_t* W = a.weights + (size_t)l * blob;
        const size_t ro = (size_t)(l3.active ? r3 + l3.ri : 0) * (D / 4);
        load_row<S3>(W + 4 * dd + ro, l3, wg);
        load_row<S3>(W + 4 * dd + fd + ro, l3, wu);
        load_strided<D>(a.gains + (size_t)l * (3 * D + F) + 2 * D, g3);
    };
    auto fetch4 = [&](int l) {
        const uint8_t* W = a.weights + (size_t)l * blob;
        load_row<S4>(W + 4 * dd + 2 * fd + (size_t)(l4.active ? r2 + l4.ri : 0) * (F / 4), l4, w4);
        load_strided<F>(a.gains + (size_t)l * (3 * D + F) + 3 * D, g4);
    };
    for (int l = 0; l < a.n_layers; ++l) {
        const uint32_t E = base + 4u * (uint32_t)l;
        float sw[7];  // this layer's weight scales
#pragma unroll
        for (int i = 0; i < 7; ++i) sw[i] = a.scales[7 * l + i];
        float* qkv = a.qkv + (size_t)l * a.qkv_layer_stride;

        // ---- P1: q, k, v ----
        {
            if (t < S1::R) sh.acc[t] = 0;
            fetch1(l);
            float v[ND];
            if (l == 0) {
                load_strided<D>(a.x, v);
            } else if (!poll_vec<D>(a.xa, E, v, a.ctrl, t_start)) {
                return;
            }
            norm_quant<D>(v, g1, a.eps, sh, s_a, qsum);
            const int acc = dot_row<S1>(w1, l1, sh.q);
            if (l1.active) atomicAdd(&sh.acc[l1.ri], acc);
            __syncthreads();
            if (e1) {
                const int row = r1 + t, mat = row / D;
                const float inv = 1.0f / (s_a * (mat == 0 ? sw[0] : (mat == 1 ? sw[1] : sw[2])));
                qkv[row] = (float)(sh.acc[t] - qsum) * inv;
            }
            if (t == 0) ll_store(a.done + w, 0.0f, E + 1);
        }
        // ---- P2: o projection of the stand-in z, residual ----
        {
            // z does not depend on the stream: its norm + quant runs before the
            // wait for P1 to finish everywhere
            norm_quant<D>(zv, g2, a.eps, sh, s_a, qsum);
            if (t < S2::R) sh.acc[t] = 0;
            fetch2(l);
            float fl[1];
            if (!poll_vec<kGrid>(a.done, E + 1, fl, a.ctrl, t_start)) return;
            if (l == 0 && w == 0 && t == 0)  // every workgroup has read the base by now
                __hip_atomic_store(a.ctrl, base + 4u * (uint32_t)a.n_layers, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            const int acc = dot_row<S2>(w2, l2, sh.q);
            if (l2.active) atomicAdd(&sh.acc[l2.ri], acc);
            __syncthreads();
            if (e2) {
                const float inv = 1.0f / (s_a * sw[3]);
                xres = xres + (float)(sh.acc[t] - qsum) * inv;
                ll_store(a.xb + r2 + t, xres, E + 2);
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
            if (!poll_vec<D>(a.xb, E + 2, v, a.ctrl, t_start)) return;
            norm_quant<D>(v, g3, a.eps, sh, s_a, qsum);
            const int ag = dot_row<S3>(wg, l3, sh.q);
            const int au = dot_row<S3>(wu, l3, sh.q);
            if (l3.active) {
                atomicAdd(&sh.acc[l3.ri], ag);
                atomicAdd(&sh.acc[S3::R + l3.ri], au);
            }
            __syncthreads();
            if (e3) {
                const float gate = (float)(sh.acc[t] - qsum) * (1.0f / (s_a * sw[4]));
                const float up = (float)(sh.acc[S3::R + t] - qsum) * (1.0f / (s_a * sw[5]));
                const float gp = gate > 0.0f ? gate : 0.0f;
                const float g2v = gp * gp;
                ll_store(a.hh + r3 + t, g2v * up, E + 3);
            }
        }
        // ---- P4: down projection of h, residual ----
        {
            if (t < S4::R) sh.acc[t] = 0;
            fetch4(l);
            float v[NF];
            if (!poll_vec<F>(a.hh, E + 3, v, a.ctrl, t_start)) return;
            norm_quant<F>(v, g4, a.eps, sh, s_a, qsum);
            const int acc = dot_row<S4>(w4, l4, sh.q);
            if (l4.active) atomicAdd(&sh.acc[l4.ri], acc);
            __syncthreads();
            if (e2) {
                const float inv = 1.0f / (s_a * sw[6]);
                xres = xres + (float)(sh.acc[t] - qsum) * inv;
                ll_store(a.xa + r2 + t, xres, E + 4);
                if (l == a.n_layers - 1) a.x[r2 + t] = xres;
            }
        }
    }
}

using StreamFn = void (*)(StreamArgs);

// Shapes with a compiled kernel: BitNet-3B, BitNet-1.3B and a small test shape.
StreamFn stream_fn(int d, int f)
{
    if (d == 2560 && f == 10240) return stream_kernel<2560, 10240>;
    if (d == 2048 && f == 8192) return stream_kernel<2048, 8192>;
    if (d == 256 && f == 1024) return stream_kernel<256, 1024>;
    return nullptr;
}

struct DeviceInfo {
    int cus = 0;
    bool coop = false;
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
        v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeCooperativeLaunch, dev) == hipSuccess) info.coop = v != 0;
        cache[dev] = info;
        have[dev] = true;
    }
    return cache[dev];
}

}  // namespace

bool stream_persistent_fits(int m, int d, int f)
{
    if (m != 1 || !stream_fn(d, f)) return false;
    const DeviceInfo info = device_info();
    return info.coop && info.cus >= kGrid;
}

int launch_stream_persistent(const uint8_t* weights, const float* scales, const float* gains, const float* z,
                             int n_layers, int d, int f, float eps, float* x, float* qkv, long long qkv_stride,
                             void* ll_region, uint32_t* ctrl, hipStream_t s)
{
    const StreamFn fn = stream_fn(d, f);
    if (!fn) return BL_ERR_SHAPE;
    StreamArgs a;
    a.weights = weights;
    a.scales = scales;
    a.gains = gains;
    a.z = z;
    a.x = x;
    a.qkv = qkv;
    a.qkv_layer_stride = qkv_stride;
    unsigned long long* ll = static_cast<unsigned long long*>(ll_region);
    a.xa = ll;
    a.xb = ll + d;
    a.hh = ll + 2 * d;
    a.done = ll + 2 * d + f;
    a.ctrl = ctrl;
    a.n_layers = n_layers;
    a.eps = eps;
    void* args[] = {&a};
    const hipError_t e =
        hipLaunchCooperativeKernel(reinterpret_cast<const void*>(fn), dim3(kGrid), dim3(kT), args, 0, s);
    return e == hipSuccess ? BL_OK : BL_ERR_LAUNCH;
}

size_t stream_ll_words(int d, int f) { return (size_t)2 * d + f + kGrid; }

}  // namespace bl
