// ternary.h -- operand helpers shared by the int8 MFMA kernels.
//
// Packed ternary weights hold four 2-bit codes c = t + 1 per byte, weight i of
// a row at bits 2 (i % 4) of byte i / 4. The pages give TQ2_0 only its name and
// its size of 0.25 byte per weight ("BitNet Model - Complete Inference
// Pipeline", section "Memory Footprint (BitNet-3B with TQ2_0)"); this layout is
// the one the ABI header states. A dword holds weights 0..15 of a 16-run.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bl {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr uint32_t kCodeMask = 0x03030303u;

// The 16 codes of one packed dword as an MFMA operand: (p >> 2 j) & 0x03030303
// puts the codes of weights j, 4 + j, 8 + j, 12 + j in the bytes of dword j,
// i.e. byte 4 j + g holds weight 4 g + j (a 4x4 byte transpose of the natural
// order). The activations meet them in the same order.
__device__ __forceinline__ v4i ternary_codes(uint32_t p)
{
    return v4i{(int)(p & kCodeMask), (int)((p >> 2) & kCodeMask), (int)((p >> 4) & kCodeMask),
               (int)((p >> 6) & kCodeMask)};
}

// 4x4 byte transpose of 16 int8 values: byte 4 j + g of the result is byte
// 4 g + j of v, the order of ternary_codes.
__device__ __forceinline__ uint4 permute16(const uint4 v)
{
    const uint32_t t01lo = __builtin_amdgcn_perm(v.y, v.x, 0x05010400u);
    const uint32_t t01hi = __builtin_amdgcn_perm(v.y, v.x, 0x07030602u);
    const uint32_t t23lo = __builtin_amdgcn_perm(v.w, v.z, 0x05010400u);
    const uint32_t t23hi = __builtin_amdgcn_perm(v.w, v.z, 0x07030602u);
    uint4 o;
    o.x = __builtin_amdgcn_perm(t23lo, t01lo, 0x05040100u);
    o.y = __builtin_amdgcn_perm(t23lo, t01lo, 0x07060302u);
    o.z = __builtin_amdgcn_perm(t23hi, t01hi, 0x05040100u);
    o.w = __builtin_amdgcn_perm(t23hi, t01hi, 0x07060302u);
    return o;
}

__device__ __forceinline__ v4i as_v4i(const uint4 v) { return v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w}; }

// Argmax key of an fp32 value: its bits mapped to an unsigned order that
// matches the float order (-0 taken as +0, so equal values tie), then lower
// columns first. Non-finite values do not occur.
__device__ __forceinline__ unsigned long long argmax_key_f32(float v, int col)
{
    uint32_t b = __float_as_uint(v);
    if ((b << 1) == 0u) b = 0u;
    const uint32_t ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    return ((unsigned long long)ord << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)col);
}

// Argmax key of an exact accumulator: larger totals first, then lower columns.
__device__ __forceinline__ unsigned long long argmax_key(int total, int col)
{
    return ((unsigned long long)((uint32_t)total ^ 0x80000000u) << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)col);
}

}  // namespace bl
