// The packer: bf16 expert weights -> the library's int4 expert format, the
// step right before the layer (how its codes arise).  Format: Flint model
// card (Aijuus/flint-w4exp), table row "weights": signed int4 codes, one bf16
// scale per 128 of K, in a basis rotated by a 128-wide Hadamard transform
// (fwht128).  The card quotes the format's error, 11.7% relative Frobenius
// per expert plane ("Why the linears stay bf16"), but not the quantiser; the
// reading here is scale = bf16(absmax / 7) over the 128 rotated values of a
// group, code = clamp(round-half-even(w / scale), -8, 7), 0 for a zero group.
//
// Every expert is gate [512][2048], up [512][2048], down [2048][512] bf16, in
// that order, and its codes and scales follow the same row order, so the
// whole bank is one sequence of independent 128-element groups: group G
// reads bf16 elements [128 G, 128 G + 128) and writes code bytes [64 G,
// 64 G + 64) and scale G.  A group is 4 lanes: lane q holds elements
// [32q, 32q + 32), rotates them with its 3 neighbours (the fwht128 butterfly
// in fp32: strides 1 .. 16 inside the lane, 32 and 64 across, then the
// 1/sqrt(128) factor), takes the group's absmax and writes its 32 codes as 16
// bytes, so a wave reads 4 KiB and writes 1 KiB contiguously.
//
// Each code takes fp32(w / scale) rounded half to even.  The division runs as
// a multiplication by the hardware reciprocal, whose quotient is within 3e-6
// of the correctly rounded one; only a lane with a quotient within 1e-4 of a
// half-integer (where the two could round apart) repeats its divisions with
// the correctly rounded fp32 division, so every code is the one the exact
// fp32 quotient gives.  Clamping to [-8, 7] before rounding gives the same
// code as rounding first: the bounds are integers.
#include "common.h"
#include "launch.h"

namespace moe_w4 {

namespace {

constexpr int kPackGroupsPerWg = 64;   // 256 threads, 4 lanes per group
constexpr float kRoundMagic = 0x1.8p23f;   // q + 1.5*2^23 holds round-half-even(q) in its low mantissa bits

__global__ __launch_bounds__(256) void k_pack_groups(const uint16_t *__restrict__ w, int64_t n_groups,
                                                     uint8_t *__restrict__ codes, uint16_t *__restrict__ scales) {
    const int lane = threadIdx.x & 63, q = lane & 3;
    const int64_t g = (int64_t)blockIdx.x * kPackGroupsPerWg + (threadIdx.x >> 2);
    const bool valid = g < n_groups;
    const int64_t gg = valid ? g : n_groups - 1;   // past the end: the last group again (not stored)
    const uint4 *src = reinterpret_cast<const uint4 *>(w + 128 * gg + 32 * q);
    float v[32];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint4 raw = src[i];
        v[8 * i + 0] = bf16lo(raw.x); v[8 * i + 1] = bf16hi(raw.x);
        v[8 * i + 2] = bf16lo(raw.y); v[8 * i + 3] = bf16hi(raw.y);
        v[8 * i + 4] = bf16lo(raw.z); v[8 * i + 5] = bf16hi(raw.z);
        v[8 * i + 6] = bf16lo(raw.w); v[8 * i + 7] = bf16hi(raw.w);
    }
    // fwht128: strides 1..16 inside the lane, 32 and 64 across the group's
    // lanes as one fma by +-1 each (a + b below, a - b above; one rounding,
    // the same value as the add or subtract), then the 1/sqrt(128) factor
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
        const float sgn = (lane & m) ? -1.0f : 1.0f;
#pragma unroll
        for (int i = 0; i < 32; ++i) v[i] = fmaf(v[i], sgn, shfl_xor_f(v[i], m));
    }
    const float kInvSqrt = 0.08838834764831845f;   // 1/sqrt(128)
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        v[i] *= kInvSqrt;
        amax = fmaxf(amax, fabsf(v[i]));
    }
    amax = fmaxf(amax, shfl_xor_f(amax, 1));
    amax = fmaxf(amax, shfl_xor_f(amax, 2));
    const uint16_t sb = f32_to_bf16(__fdiv_rn(amax, 7.0f));
    const float s = bf16_to_f32(sb);
    const float inv = __builtin_amdgcn_rcpf(s);
    // fast quotients: within 3e-6 of the correctly rounded ones, so their
    // round-half-even is the same unless one lies within 1e-4 of a half-integer
    uint32_t t[32];
    float dmax = s >= 0x1p-100f ? 0.0f : 1.0f;   // a zero or tiny scale: the exact path
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        const float qc = __builtin_amdgcn_fmed3f(v[i] * inv, -8.0f, 7.0f);
        const float r = qc + kRoundMagic;
        dmax = fmaxf(dmax, fabsf(qc - (r - kRoundMagic)));
        t[i] = __float_as_uint(r);
    }
    if (dmax > 0.4999f) {
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            const float qe = s > 0.0f ? __fdiv_rn(v[i], s) : 0.0f;
            t[i] = __float_as_uint(__builtin_amdgcn_fmed3f(qe, -8.0f, 7.0f) + kRoundMagic);
        }
    }
    uint32_t packed[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 32; ++i)   // element 32q + i: low nibble when even; two's complement
        packed[i >> 3] |= (t[i] & 15u) << (4 * (i & 7));
    if (valid) {
        reinterpret_cast<uint4 *>(codes + 64 * g)[q] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
        if (q == 0) scales[g] = sb;
    }
}

}  // namespace

void launch_pack_experts(const uint16_t *w, int64_t n_experts, uint8_t *codes, uint16_t *scales, hipStream_t s) {
    const int64_t n_groups = n_experts * (int64_t)kScalesPerExpert;
    const int64_t grid = (n_groups + kPackGroupsPerWg - 1) / kPackGroupsPerWg;
    if (grid > 0) hipLaunchKernelGGL(k_pack_groups, dim3((unsigned)grid), dim3(256), 0, s, w, n_groups, codes, scales);
}

}  // namespace moe_w4
