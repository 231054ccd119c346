// Device routines of the int4 GEMVs shared by the decode kernels: operand
// loads, the mask conversion of 32 codes per lane, and the gate/up row-pair
// loads (rows of 1 KiB, lane l owning K [32l, 32l+32), one scale per lane).
#pragma once

#include "common.h"

namespace moe_w4 {

__device__ __forceinline__ uint4 ldg4(const void *p) { return *reinterpret_cast<const uint4 *>(p); }
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Load one lane's 32 stored activations (16 half2 words) and their offset.
__device__ __forceinline__ float load_operand32(const uint32_t *src, uint32_t (&xs)[16]) {
    float off = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint4 v = ldg4(src + 4 * i);
        xs[4 * i] = v.x; xs[4 * i + 1] = v.y; xs[4 * i + 2] = v.z; xs[4 * i + 3] = v.w;
        off = q_offset(v.x, v.y, v.z, v.w, off);
    }
    return off;
}

// sum_k c_k x_k over one lane's 32-element slice: 16 dot2 on mask-converted codes.
__device__ __forceinline__ float dot_slice(const Q4 (&q)[4], const uint32_t (&xs)[16], float acc) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        acc = dot2h(q[d].q0, xs[4 * d + 0], acc);
        acc = dot2h(q[d].q1, xs[4 * d + 1], acc);
        acc = dot2h(q[d].q2, xs[4 * d + 2], acc);
        acc = dot2h(q[d].q3, xs[4 * d + 3], acc);
    }
    return acc;
}

__device__ __forceinline__ void convert16(const uint4 w, Q4 (&q)[4]) {
    q[0] = int4x8_to_q(w.x);
    q[1] = int4x8_to_q(w.y);
    q[2] = int4x8_to_q(w.z);
    q[3] = int4x8_to_q(w.w);
}

__device__ __forceinline__ float silu_f(float v) { return v / (1.0f + expf(-v)); }

constexpr int kGuPairs = 4;   // row pairs per batch

struct GuRows {
    uint4 g[kGuPairs], u[kGuPairs];
    uint16_t sg[kGuPairs], su[kGuPairs];   // bf16 bits of the gate and up scales
};

template <bool RELOAD>
__device__ __forceinline__ void gu_load_pair(GuRows &R, int i, rsrc_t cg, rsrc_t sp, uint32_t cv, uint32_t sv, int r) {
    if (RELOAD) {
        R.g[i] = bload16_nt_reload(cg, cv, r * (kH / 2));
        R.u[i] = bload16_nt_reload(cg, cv, kPlaneGateBytes + r * (kH / 2));
        R.sg[i] = bload2_nt_reload(sp, sv, 2 * r * (kH / kG));
        R.su[i] = bload2_nt_reload(sp, sv, 2 * (kScalesGate + r * (kH / kG)));
    } else {
        R.g[i] = bload16_nt(cg, cv, r * (kH / 2));
        R.u[i] = bload16_nt(cg, cv, kPlaneGateBytes + r * (kH / 2));
        R.sg[i] = bload2_nt(sp, sv, 2 * r * (kH / kG));
        R.su[i] = bload2_nt(sp, sv, 2 * (kScalesGate + r * (kH / kG)));
    }
}

// One assignment's a = silu(g)*u (512 fp32) -> the fp16 operands of the down
// projection, by one wave: Hadamard on each 128-block (lane l owns 8 values of
// block l/16), a power-of-two prescale per block (largest magnitude in
// [2^13, 2^14)), stored in the int4x8_to_q operand order.  at: 256 words,
// at_scale: the 4 block multipliers 2^sh.
// (a0, a1: the lane's 8 values of a, K [8 lane, 8 lane + 8).)
__device__ __forceinline__ void rotate_act_wave(float4 a0, float4 a1, int lane, uint32_t *at, float *at_scale) {
    float v[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
    fwht128_lanes16(v, lane);
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
    for (int m = 1; m <= 8; m <<= 1) amax = fmaxf(amax, shfl_xor_f(amax, m));
    int sh = 0;
    if (amax > 0.0f && isfinite(amax)) {
        int ex;
        frexpf(amax, &ex);
        sh = ex - 14;   // largest magnitude in [2^13, 2^14): exact scaling, far from fp16 overflow
    }
    uint4 w;
    w.x = pack_half2(ldexpf(v[0], -sh), ldexpf(v[4], -sh));
    w.y = pack_half2(ldexpf(v[1], -sh - 4), ldexpf(v[5], -sh - 4));
    w.z = pack_half2(ldexpf(v[2], -sh), ldexpf(v[6], -sh));
    w.w = pack_half2(ldexpf(v[3], -sh - 4), ldexpf(v[7], -sh - 4));
    reinterpret_cast<uint4 *>(at)[lane] = w;
    at_scale[lane >> 4] = ldexpf(1.0f, sh);   // the 16 lanes of a block store the same value
}

}  // namespace moe_w4
