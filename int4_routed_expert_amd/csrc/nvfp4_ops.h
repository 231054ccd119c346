// NVFP4 expert arithmetic shared by the GEMV kernels and the decode launch
// (Flint NVFP4 repack, kekzle/Flint-NVFP4, rows "Layout per Linear" and
// "Declaration"): E2M1 codes two per byte (even K in the low nibble), one
// E4M3 block scale per 16 columns of K, one fp32 tensor scale per Linear;
// gfx950 converts two E2M1 codes to an exact fp16 pair in one instruction
// (v_cvt_scalef32_pk_f16_fp4, scale 1), products are exact in
// v_dot2_f32_f16 and summed in fp32 per 16-element block.
#pragma once

#include "common.h"

namespace moe_w4 {

constexpr int kNvBlock = 16;
constexpr uint32_t kNvScaleGate = (uint32_t)kI * kH / kNvBlock;                    // 65,536 bytes
constexpr uint32_t kNvScaleGu = 2 * kNvScaleGate;                                  // 131,072
constexpr uint32_t kNvScalePerExpert = kNvScaleGu + (uint32_t)kH * kI / kNvBlock;  // 196,608

// Eight codes (byte b: element 2b in the low nibble, 2b + 1 in the high one)
// -> four fp16 pairs h[b] = (value 2b, value 2b + 1).
__device__ __forceinline__ void e2m1x8_to_half(uint32_t w, uint32_t (&h)[4]) {
    h[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0));
    h[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1));
    h[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2));
    h[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3));
}

// One lane's 32 codes (word i: elements 8i .. 8i + 7) as fp16 pairs
// h[4i + b] = (value 8i + 2b, value 8i + 2b + 1).
__device__ __forceinline__ void conv32_nv(const uint4 c, uint32_t (&h)[16]) {
    uint32_t q[4];
    e2m1x8_to_half(c.x, q);
    h[0] = q[0]; h[1] = q[1]; h[2] = q[2]; h[3] = q[3];
    e2m1x8_to_half(c.y, q);
    h[4] = q[0]; h[5] = q[1]; h[6] = q[2]; h[7] = q[3];
    e2m1x8_to_half(c.z, q);
    h[8] = q[0]; h[9] = q[1]; h[10] = q[2]; h[11] = q[3];
    e2m1x8_to_half(c.w, q);
    h[12] = q[0]; h[13] = q[1]; h[14] = q[2]; h[15] = q[3];
}
// Those against the operand words xs[4i + b] = (x[8i + 2b], x[8i + 2b + 1]):
// s0 * (sum over elements 0..15) + s1 * (sum over elements 16..31).
__device__ __forceinline__ float dot32h_nv(const uint32_t (&h)[16], const uint32_t (&xs)[16], float s0, float s1) {
    float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) a0 = dot2h(h[k], xs[k], a0);
#pragma unroll
    for (int k = 8; k < 16; ++k) a1 = dot2h(h[k], xs[k], a1);
    return a0 * s0 + a1 * s1;
}
__device__ __forceinline__ float dot32_nv(const uint4 c, const uint32_t (&xs)[16], float s0, float s1) {
    uint32_t h[4];
    float a0 = 0.0f, a1 = 0.0f;
    e2m1x8_to_half(c.x, h);
#pragma unroll
    for (int k = 0; k < 4; ++k) a0 = dot2h(h[k], xs[k], a0);
    e2m1x8_to_half(c.y, h);
#pragma unroll
    for (int k = 0; k < 4; ++k) a0 = dot2h(h[k], xs[4 + k], a0);
    e2m1x8_to_half(c.z, h);
#pragma unroll
    for (int k = 0; k < 4; ++k) a1 = dot2h(h[k], xs[8 + k], a1);
    e2m1x8_to_half(c.w, h);
#pragma unroll
    for (int k = 0; k < 4; ++k) a1 = dot2h(h[k], xs[12 + k], a1);
    return a0 * s0 + a1 * s1;
}

}  // namespace moe_w4
