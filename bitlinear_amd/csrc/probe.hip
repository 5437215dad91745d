// probe.hip -- roofline probes: the measured ceilings that the benchmark
// reports beside the nominal MI355X peaks (8 TB/s HBM, 5.0 POP/s dense int8).
//
//   read probe: every byte of a caller buffer is read once with 16-byte loads,
//     eight loads in flight per thread, two 1024-thread workgroups per CU;
//     the loaded words are folded into one word per workgroup and
//     xor-ed into a sink, so the loads cannot be dropped.
//   MFMA probe: waves that issue only v_mfma_i32_16x16x64_i8 on register
//     operands, eight independent accumulators per wave (enough to cover the
//     instruction's latency), two waves per SIMD on every CU.
// Neither touches anything but its arguments; both are plain launches on the
// caller's stream.
#include <algorithm>

#include "internal.h"
#include "ternary.h"

namespace bl {
namespace {

constexpr int kReadThreads = 1024;
constexpr int kReadUnroll = 8;

__global__ __launch_bounds__(kReadThreads) void read_probe_kernel(const uint4* __restrict__ p, uint64_t n16,
                                                                  uint32_t* sink)
{
    const uint64_t stride = (uint64_t)gridDim.x * kReadThreads;
    uint64_t i = (uint64_t)blockIdx.x * kReadThreads + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (kReadUnroll - 1) * stride < n16; i += kReadUnroll * stride) {
        uint4 v[kReadUnroll];
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) v[u] = p[i + u * stride];
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += stride) {
        const uint4 v = p[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    // fold the workgroup into one word
    for (int off = 32; off >= 1; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
    __shared__ uint32_t part[kReadThreads / 64];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t t = 0;
        for (int w = 0; w < kReadThreads / 64; ++w) t ^= part[w];
        atomicXor(sink, t);
    }
}

constexpr int kMfmaThreads = 256;
constexpr int kMfmaChains = 8;

// One MFMA accumulating in place: the compiler's own form of a loop-carried
// accumulator is moved between registers every iteration, which the probe
// would then measure instead of the matrix cores.
#define BL_MFMA_INPLACE(c, a, b) asm volatile("v_mfma_i32_16x16x64_i8 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b))

// A 32-bit mix of x (the murmur3 finaliser), for operand bytes that look random.
__device__ __forceinline__ int mix32(uint32_t x)
{
    x ^= x >> 16;
    x *= 0x85ebca6bu;
    x ^= x >> 13;
    x *= 0xc2b2ae35u;
    x ^= x >> 16;
    return (int)x;
}

// DENSE = false: one operand pair of small values (mostly zero bytes) for every
// MFMA. DENSE = true: each chain its own pair of random-looking bytes, so
// consecutive MFMAs see different operands with every bit toggling, as in a
// GEMM on real data; the matrix cores then draw more power and the clock can
// drop, which this form measures.
template <bool DENSE>
__global__ __launch_bounds__(kMfmaThreads) void mfma_probe_kernel(int64_t iters, uint32_t* sink)
{
    const int lane = threadIdx.x & 63;
    v4i a[8], b[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        if (DENSE) {
            const uint32_t s = (uint32_t)(blockIdx.x * 4096 + threadIdx.x * 16 + j * 2);
            a[j] = v4i{mix32(8 * s), mix32(8 * s + 1), mix32(8 * s + 2), mix32(8 * s + 3)};
            b[j] = v4i{mix32(8 * s + 4), mix32(8 * s + 5), mix32(8 * s + 6), mix32(8 * s + 7)};
        } else {
            a[j] = v4i{lane, lane * 3, lane * 5, lane * 7};
            b[j] = v4i{lane ^ 1, lane ^ 2, lane ^ 3, lane ^ 4};
        }
    }
    // eight independent chains: each MFMA reads an accumulator written eight
    // instructions earlier
    v4i c0 = {0, 0, 0, 0}, c1 = {1, 0, 0, 0}, c2 = {2, 0, 0, 0}, c3 = {3, 0, 0, 0};
    v4i c4 = {4, 0, 0, 0}, c5 = {5, 0, 0, 0}, c6 = {6, 0, 0, 0}, c7 = {7, 0, 0, 0};
    for (int64_t it = 0; it < iters; ++it) {
        BL_MFMA_INPLACE(c0, a[0], b[0]);
        BL_MFMA_INPLACE(c1, a[1], b[1]);
        BL_MFMA_INPLACE(c2, a[2], b[2]);
        BL_MFMA_INPLACE(c3, a[3], b[3]);
        BL_MFMA_INPLACE(c4, a[4], b[4]);
        BL_MFMA_INPLACE(c5, a[5], b[5]);
        BL_MFMA_INPLACE(c6, a[6], b[6]);
        BL_MFMA_INPLACE(c7, a[7], b[7]);
    }
    const v4i r = c0 ^ c1 ^ c2 ^ c3 ^ c4 ^ c5 ^ c6 ^ c7;
    const uint32_t acc = (uint32_t)(r[0] ^ r[1] ^ r[2] ^ r[3]);
    if (acc == 0x9e3779b9u) atomicXor(sink, acc);  // practically never taken; keeps the chains alive
}

#undef BL_MFMA_INPLACE

int cu_count()
{
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    return cus;
}

}  // namespace
}  // namespace bl

extern "C" {

int bitlinear_probe_read(const void* buf, size_t bytes, uint32_t* sink, void* stream)
{
    if (!buf || !sink) return BL_ERR_NULL;
    if (bytes == 0 || bytes % 16 != 0) return BL_ERR_SHAPE;
    if (!bl::aligned(buf, 16) || !bl::aligned(sink, 4)) return BL_ERR_ALIGN;
    const int cus = bl::cu_count();
    if (cus <= 0) return BL_ERR_DEVICE;
    const uint64_t n16 = bytes / 16;
    // two 1024-thread workgroups per CU, but no more workgroups than 16-byte words
    const uint64_t want = (uint64_t)cus * 2;
    const uint64_t grid = std::min<uint64_t>(want, (n16 + bl::kReadThreads - 1) / bl::kReadThreads);
    bl::read_probe_kernel<<<(unsigned)grid, bl::kReadThreads, 0, reinterpret_cast<hipStream_t>(stream)>>>(
        static_cast<const uint4*>(buf), n16, sink);
    return hipGetLastError() == hipSuccess ? BL_OK : BL_ERR_LAUNCH;
}

int64_t bitlinear_probe_mfma_ops(int64_t iters)
{
    const int cus = bl::cu_count();
    if (iters <= 0 || cus <= 0) return 0;
    // waves x MFMAs per wave x (16 x 16 x 64 multiply-adds = 32768 ops)
    return (int64_t)cus * 8 * iters * bl::kMfmaChains * 32768;
}

namespace {
int probe_mfma(bool dense, int64_t iters, uint32_t* sink, void* stream)
{
    if (!sink) return BL_ERR_NULL;
    if (iters <= 0 || iters > ((int64_t)1 << 40)) return BL_ERR_SHAPE;
    if (!bl::aligned(sink, 4)) return BL_ERR_ALIGN;
    const int cus = bl::cu_count();
    if (cus <= 0) return BL_ERR_DEVICE;
    // two waves per SIMD: 8 waves per CU, as 2 workgroups of 4 waves
    const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (dense)
        bl::mfma_probe_kernel<true><<<cus * 2, bl::kMfmaThreads, 0, s>>>(iters, sink);
    else
        bl::mfma_probe_kernel<false><<<cus * 2, bl::kMfmaThreads, 0, s>>>(iters, sink);
    return hipGetLastError() == hipSuccess ? BL_OK : BL_ERR_LAUNCH;
}
}  // namespace

int bitlinear_probe_mfma_i8(int64_t iters, uint32_t* sink, void* stream)
{
    return probe_mfma(false, iters, sink, stream);
}

int bitlinear_probe_mfma_i8_dense(int64_t iters, uint32_t* sink, void* stream)
{
    return probe_mfma(true, iters, sink, stream);
}

}  // extern "C"
