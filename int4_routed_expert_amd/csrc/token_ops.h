// Per-token device routines shared by the routing kernels and the fused
// decode kernel: top-6 selection of one token's logits, the normalised
// 128-point Hadamard of x, and the fp16 operand layout of the int4 GEMVs.
#pragma once

#include "common.h"

namespace moe_w4 {

// ---------------------------------------------------------------------------
// Top-6 of one token's 256 logits, one wave per token.  Keys order floats
// monotonically as unsigned integers; ties go to the lower expert index.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t order_key(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Normalised 128-point Sylvester Hadamard on a 128-block spread over 4 lanes
// (lane & 3 selects the 32-element quarter).  Five butterfly stages run inside
// the lane, the strides 32 and 64 go across lanes.
__device__ __forceinline__ void fwht128_4lanes(float (&v)[32], int lane) {
#pragma unroll
    for (int h = 1; h < 32; h <<= 1) {
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            if ((i & h) == 0) {
                const float a = v[i], b = v[i + h];
                v[i] = a + b;
                v[i + h] = a - b;
            }
        }
    }
#pragma unroll
    for (int m = 1; m <= 2; m <<= 1) {
        const bool upper = (lane & m) != 0;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            const float p = shfl_xor_f(v[i], m);
            v[i] = upper ? (p - v[i]) : (v[i] + p);
        }
    }
    const float inv = 0.08838834764831845f;   // 1/sqrt(128)
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] *= inv;
}

// Store 32 consecutive rotated values as fp16 in the operand order of
// int4x8_to_q: per 8-group (x0,x4) (x1/16,x5/16) (x2,x6) (x3/16,x7/16), after
// multiplying by 2^-sh (a power-of-two prescale chosen per token or block).
__device__ __forceinline__ void store_operand32(const float (&v)[32], int sh, uint32_t *dst) {
    uint32_t w[16];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const float *q = v + 8 * g;
        w[4 * g + 0] = pack_half2(ldexpf(q[0], -sh), ldexpf(q[4], -sh));
        w[4 * g + 1] = pack_half2(ldexpf(q[1], -sh - 4), ldexpf(q[5], -sh - 4));
        w[4 * g + 2] = pack_half2(ldexpf(q[2], -sh), ldexpf(q[6], -sh));
        w[4 * g + 3] = pack_half2(ldexpf(q[3], -sh - 4), ldexpf(q[7], -sh - 4));
    }
    uint4 *d = reinterpret_cast<uint4 *>(dst);
#pragma unroll
    for (int i = 0; i < 4; ++i) d[i] = make_uint4(w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]);
}

// Power-of-two prescale: the largest magnitude lands in [2^13, 2^14), well
// inside fp16, whatever the input scale (the NInfer README of Flint, section
// "Quality", scales rows by exact powers of two against fp16 overflow).
__device__ __forceinline__ int prescale_shift(float amax) {
    if (!(amax > 0.0f) || !isfinite(amax)) return 0;
    int ex;
    frexpf(amax, &ex);   // amax = f * 2^ex, f in [0.5, 1)
    return ex - 14;
}

// Top-6 of one token's 256 logits by one wave (lane l holds logits 4l..4l+3).
// Every lane ends with the six experts in slot order (descending logit, ties
// to the lower index) and their weights sigmoid(l_j) / max(sum sigmoid, 2^-14).
struct Top6 {
    int e[kTopK];
    float w[kTopK];
};

// Largest value over the wave, left in lane 63 by DPP steps (a running
// maximum over row shifts 1, 2, 4, 8, then the two row broadcasts) and read
// from there: no LDS round trips, unlike a butterfly of lane shuffles.  Lanes
// that read outside their row take 0, which never wins.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false));   // row_shr:1
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false));   // row_shr:2
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false));   // row_shr:4
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false));   // row_shr:8
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false));   // row_bcast:15
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false));   // row_bcast:31
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// (key, index) order of the selection: larger key first, equal keys by the
// lower expert index.
__device__ __forceinline__ bool ahead(uint32_t ka, int ia, uint32_t kb, int ib) {
    return ka > kb || (ka == kb && ia < ib);
}

// Router policy (bloomery issue #632, design thread and its host-policy
// slice: the router rule distinguishes no normalisation, the legacy selected
// sum and the selected sum with the 2^-14 floor, and a bias that is absent or
// used for selection only).  flags: bits 0-1 the normalisation (kNormFloor,
// kNormSum, kNormNone), bit 2 kBiasSelectOnly.  bias: fp32 [256] or null.
constexpr int kNormFloor = 0, kNormSum = 1, kNormNone = 2, kBiasSelectOnly = 4;
struct RouterPolicy {
    const float *bias;
    int flags;
};

__device__ __forceinline__ Top6 top6_wave(float4 lv, int lane, RouterPolicy rp) {
    // the choice is made on the fp32 logit plus the bias, if any
    float4 kv = lv;
    if (rp.bias) {
        const float4 b = reinterpret_cast<const float4 *>(rp.bias)[lane];
        kv.x += b.x; kv.y += b.y; kv.z += b.z; kv.w += b.w;
    }
    // each lane sorts its 4 (key, expert) pairs (a 5-comparator network on the
    // total order above), then six rounds take the largest head over the wave
    uint32_t k[4] = {order_key(kv.x), order_key(kv.y), order_key(kv.z), order_key(kv.w)};
    int ix[4] = {4 * lane, 4 * lane + 1, 4 * lane + 2, 4 * lane + 3};
    auto cswap = [&](int a, int b) {
        if (ahead(k[b], ix[b], k[a], ix[a])) {
            const uint32_t tk = k[a]; k[a] = k[b]; k[b] = tk;
            const int ti = ix[a]; ix[a] = ix[b]; ix[b] = ti;
        }
    };
    cswap(0, 1); cswap(2, 3); cswap(0, 2); cswap(1, 3); cswap(1, 2);
    Top6 r;
    uint32_t sel_k[kTopK];
    int head = 0;   // entries of this lane's list already taken
#pragma unroll
    for (int j = 0; j < kTopK; ++j) {
        // an exhausted list offers 0, below the key of every non-NaN logit
        const uint32_t hk = head == 0 ? k[0] : head == 1 ? k[1] : head == 2 ? k[2] : head == 3 ? k[3] : 0u;
        const int hi = head == 0 ? ix[0] : head == 1 ? ix[1] : head == 2 ? ix[2] : ix[3];
        const uint32_t K = wave_max_u32(hk);
        // among equal heads the lowest lane holds the lowest expert index
        const int L = (int)__builtin_ctzll(__ballot(hk == K));
        r.e[j] = __builtin_amdgcn_readlane(hi, L);
        sel_k[j] = K;
        if (lane == L) ++head;
    }
    // sigmoids side by side (lane j < 6), summed in slot order; the sigmoid
    // takes the selection key, or with a selection-only bias the logit itself
    uint32_t mine = sel_k[0];
    int mine_e = r.e[0];
#pragma unroll
    for (int j = 1; j < kTopK; ++j)
        if (lane == j) {
            mine = sel_k[j];
            mine_e = r.e[j];
        }
    float lw = key_value(mine);
    if (rp.flags & kBiasSelectOnly) {
        const int src = mine_e >> 2, q = mine_e & 3;   // lane src holds logits 4 src .. 4 src + 3
        const float c0 = __shfl(lv.x, src, kWave), c1 = __shfl(lv.y, src, kWave);
        const float c2 = __shfl(lv.z, src, kWave), c3 = __shfl(lv.w, src, kWave);
        lw = q == 0 ? c0 : q == 1 ? c1 : q == 2 ? c2 : c3;
    }
    const float sig = 1.0f / (1.0f + expf(-lw));
    float ssum = 0.0f;
#pragma unroll
    for (int j = 0; j < kTopK; ++j) ssum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sig), j));
    const int norm = rp.flags & 3;
    const float denom = norm == kNormFloor ? fmaxf(ssum, 6.103515625e-05f)   // 2^-14
                        : norm == kNormSum ? ssum : 1.0f;
    const float w = sig / denom;
#pragma unroll
    for (int j = 0; j < kTopK; ++j) r.w[j] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), j));
    return r;
}

// Rotated x of one token by one wave: lane l holds K [32l, 32l+32) of the bf16
// row (four 16-byte words), so lanes 4b..4b+3 hold Hadamard block b.  Writes the
// lane's 16 operand words to dst and returns the token's prescale shift sh
// (operands are x_rot * 2^-sh).
__device__ __forceinline__ int rotate_x_wave(const uint4 (&xq)[4], int lane, uint32_t *dst) {
    float v[32];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint4 q = xq[i];
        v[8 * i + 0] = bf16lo(q.x); v[8 * i + 1] = bf16hi(q.x);
        v[8 * i + 2] = bf16lo(q.y); v[8 * i + 3] = bf16hi(q.y);
        v[8 * i + 4] = bf16lo(q.z); v[8 * i + 5] = bf16hi(q.z);
        v[8 * i + 6] = bf16lo(q.w); v[8 * i + 7] = bf16hi(q.w);
    }
    fwht128_4lanes(v, lane);
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = wave_max(amax);
    const int sh = prescale_shift(amax);
    store_operand32(v, sh, dst);
    return sh;
}

// x of one token by one wave as natural-order fp16 operands (the NVFP4
// experts' basis: no Hadamard): lane l holds K [32l, 32l+32) of the bf16 row
// and writes words (x[2i], x[2i+1]) * 2^-sh to dst[0..15]; returns the
// token's prescale shift sh (largest magnitude in [2^13, 2^14), bf16 values
// times a power of two: exact in fp16 unless they fall below its normal range).
__device__ __forceinline__ int natural_x_wave(const uint4 (&xq)[4], int lane, uint32_t *dst) {
    float v[32];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint4 q = xq[i];
        v[8 * i + 0] = bf16lo(q.x); v[8 * i + 1] = bf16hi(q.x);
        v[8 * i + 2] = bf16lo(q.y); v[8 * i + 3] = bf16hi(q.y);
        v[8 * i + 4] = bf16lo(q.z); v[8 * i + 5] = bf16hi(q.z);
        v[8 * i + 6] = bf16lo(q.w); v[8 * i + 7] = bf16hi(q.w);
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = wave_max(amax);
    const int sh = prescale_shift(amax);
    uint4 *d = reinterpret_cast<uint4 *>(dst);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float *q = v + 8 * i;
        d[i] = make_uint4(pack_half2(ldexpf(q[0], -sh), ldexpf(q[1], -sh)), pack_half2(ldexpf(q[2], -sh), ldexpf(q[3], -sh)),
                          pack_half2(ldexpf(q[4], -sh), ldexpf(q[5], -sh)), pack_half2(ldexpf(q[6], -sh), ldexpf(q[7], -sh)));
    }
    (void)lane;
    return sh;
}

}  // namespace moe_w4
