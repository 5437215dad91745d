// wave.h -- exact lane exchanges inside a 64-lane wavefront on gfx950.
//
// xor_lane<M>(v) returns the value of lane (lane ^ M). The exchanges move bits
// unchanged (DPP moves and the gfx950 permlane swaps are VALU instructions, no
// LDS round trip), so an xor-butterfly built from them combines exactly the
// same operands, in the same order, as the butterfly written out on the CPU:
//   M = 1, 2  : DPP quad_perm [1,0,3,2] / [2,3,0,1]
//   M = 4, 8  : DPP row_shl:M (from lane + M) or row_shr:M (from lane - M),
//               selected by bit M of the lane id (both stay inside a 16-lane row)
//   M = 16    : v_permlane16_swap (rows 0<->1 and 2<->3)
//   M = 32    : v_permlane32_swap (lanes 0..31 <-> 32..63)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bl {

template <int M>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v)
{
    static_assert(M == 1 || M == 2 || M == 4 || M == 8 || M == 16 || M == 32, "xor mask inside one wave");
    if constexpr (M == 1) {
        return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
    } else if constexpr (M == 2) {
        return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);
    } else if constexpr (M == 4 || M == 8) {
        const uint32_t up = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x100 | M, 0xF, 0xF, false);
        const uint32_t dn = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x110 | M, 0xF, 0xF, false);
        return (__lane_id() & M) ? dn : up;
    } else if constexpr (M == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        return ((__lane_id() >> 4) & 1) ? r[0] : r[1];
    } else {
        const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        return (__lane_id() >> 5) ? r[0] : r[1];
    }
}

template <int M>
__device__ __forceinline__ int xor_lane(int v)
{
    return (int)xor_lane<M>((uint32_t)v);
}

template <int M>
__device__ __forceinline__ float xor_lane(float v)
{
    return __uint_as_float(xor_lane<M>(__float_as_uint(v)));
}

template <int M>
__device__ __forceinline__ double xor_lane(double v)
{
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = xor_lane<M>((uint32_t)b), hi = xor_lane<M>((uint32_t)(b >> 32));
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// p + p(lane ^ M) for M = 1, 2, ..., 32: the in-wave part of the fixed
// xor-butterfly over the RMSNorm partial sums (every lane ends with the sum
// of its wave, combined in exactly this order).
__device__ __forceinline__ double wave_butterfly_sum(double p)
{
    p = p + xor_lane<1>(p);
    p = p + xor_lane<2>(p);
    p = p + xor_lane<4>(p);
    p = p + xor_lane<8>(p);
    p = p + xor_lane<16>(p);
    p = p + xor_lane<32>(p);
    return p;
}

// The cross-wave part of the butterfly over 8 wave sums s[0..7] (offsets 64,
// 128, 256 between partials): ((s0+s1)+(s2+s3)) + ((s4+s5)+(s6+s7)).
__device__ __forceinline__ double cross_wave_sum8(const double* s)
{
    return ((s[0] + s[1]) + (s[2] + s[3])) + ((s[4] + s[5]) + (s[6] + s[7]));
}

__device__ __forceinline__ float wave_max(float v)
{
    v = fmaxf(v, xor_lane<32>(v));
    v = fmaxf(v, xor_lane<16>(v));
    v = fmaxf(v, xor_lane<8>(v));
    v = fmaxf(v, xor_lane<4>(v));
    v = fmaxf(v, xor_lane<2>(v));
    v = fmaxf(v, xor_lane<1>(v));
    return v;
}

__device__ __forceinline__ int wave_sum(int v)
{
    v += xor_lane<32>(v);
    v += xor_lane<16>(v);
    v += xor_lane<8>(v);
    v += xor_lane<4>(v);
    v += xor_lane<2>(v);
    v += xor_lane<1>(v);
    return v;
}

// Sum over aligned groups of L lanes (L a power of two <= 64).
template <int L>
__device__ __forceinline__ int group_sum(int v)
{
    if constexpr (L >= 64) v += xor_lane<32>(v);
    if constexpr (L >= 32) v += xor_lane<16>(v);
    if constexpr (L >= 16) v += xor_lane<8>(v);
    if constexpr (L >= 8) v += xor_lane<4>(v);
    if constexpr (L >= 4) v += xor_lane<2>(v);
    if constexpr (L >= 2) v += xor_lane<1>(v);
    return v;
}

}  // namespace bl
