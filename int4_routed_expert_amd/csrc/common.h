// Shared constants and device helpers of the moe_w4 kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe_w4 {

constexpr int kH = 2048;            // model width
constexpr int kE = 256;             // routed experts
constexpr int kTopK = 6;            // experts per token
constexpr int kI = 512;             // routed expert width
constexpr int kIS = 1024;           // shared expert width
constexpr int kDenseInter = 6144;   // width of the dense SwiGLU MLP blocks
constexpr int kG = 128;             // K per scale == Hadamard block
constexpr int kWave = 64;

constexpr size_t kPlaneGateBytes = (size_t)kI * kH / 2;                // 524,288
constexpr size_t kCodeBytesGu = 2 * kPlaneGateBytes;                   // 1,048,576
constexpr size_t kCodeBytesPerExpert = kCodeBytesGu + (size_t)kH * kI / 2;  // 1,572,864
constexpr size_t kScalesGate = (size_t)kI * (kH / kG);                 // 8,192
constexpr size_t kScalesGu = 2 * kScalesGate;                          // 16,384
constexpr size_t kScalesPerExpert = kScalesGu + (size_t)kH * (kI / kG);  // 24,576
constexpr size_t kSharedGateElems = (size_t)kIS * kH;                  // 2,097,152

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));

// bf16 halves of a packed 32-bit word, widened exactly to fp32.
__device__ __forceinline__ float bf16lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

// fp32 -> bf16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t pack_half2(float lo, float hi) {
    _Float16 a = (_Float16)lo, b = (_Float16)hi;   // v_cvt_f16_f32, round to nearest even
    return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}
__device__ __forceinline__ float half_lo(uint32_t v) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xffffu)); }
__device__ __forceinline__ float half_hi(uint32_t v) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16)); }

// v_dot2_f32_f16: acc + a.lo*b.lo + a.hi*b.hi with fp32 accumulation.
__device__ __forceinline__ float dot2h(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), acc, false);
}
// v_dot2_f32_bf16: acc + a.lo*b.lo + a.hi*b.hi (bf16 products are exact in fp32).
__device__ __forceinline__ float dot2b(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, a), __builtin_bit_cast(bf162_t, b), acc, false);
}

// OCP E4M3 ("FN") byte -> fp32, exact: sign, 4 exponent bits (bias 7), 3
// mantissa bits, exponent 0 subnormal (m * 2^-9), no infinities, S.1111.111 NaN.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
    const uint32_t e = (b >> 3) & 15u, m = b & 7u;
    float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
    if (e == 15u && m == 7u) mag = __uint_as_float(0x7fc00000u);
    return (b & 0x80u) ? -mag : mag;
}

// ---------------------------------------------------------------------------
// int4 -> fp16 operands without a per-nibble conversion.
//
// Eight signed int4 codes c0..c7 sit in one dword (c_i in bits 4i..4i+3).
// XOR with 0x88888888 turns each into u_i = c_i + 8 in [0, 15].  OR-ing a
// nibble into the mantissa of the fp16 1024.0 (0x6400) gives 1024 + u exactly;
// a nibble in bits 4..7 of a half gives 1024 + 16u.  So four masks give four
// half2 words, each exact:
//   q0 = (1024+u0, 1024+u4)   q1 = (1024+16u1, 1024+16u5)
//   q2 = (1024+u2, 1024+u6)   q3 = (1024+16u3, 1024+16u7)
// They pair with activations stored as (x0, x4), (x1/16, x5/16), (x2, x6),
// (x3/16, x7/16).  Then sum(q . xs) = sum_k c_k x_k + 1032*sum_even(xs) + 1152*sum_odd(xs),
// where xs are the stored fp16 activations; the second part (the "offset") is
// known per activation slice and is subtracted once, by starting the fp32
// accumulator at its negative.
// ---------------------------------------------------------------------------
struct Q4 { uint32_t q0, q1, q2, q3; };

// (w ^ B) on the mask bits A, B elsewhere: with B = 0x6400 | the nibble's sign
// bit, this is the XOR-by-8, AND and OR above in one three-input bit op
// (v_bitop3_b32), so eight codes cost one shift and four bit ops.
__device__ __forceinline__ uint32_t nib_to_half(uint32_t w, uint32_t A, uint32_t B) { return (A & (w ^ B)) | (~A & B); }

__device__ __forceinline__ Q4 int4x8_to_q(uint32_t w) {
    const uint32_t t = w >> 8;
    Q4 r;
    r.q0 = nib_to_half(w, 0x000f000fu, 0x64086408u);
    r.q1 = nib_to_half(w, 0x00f000f0u, 0x64806480u);
    r.q2 = nib_to_half(t, 0x000f000fu, 0x64086408u);
    r.q3 = nib_to_half(t, 0x00f000f0u, 0x64806480u);
    return r;
}

// Offset of one stored 8-group (four half2 words in the order above), added to
// acc: 1032 * (even-position values) + 1152 * (odd-position values), on the
// same dot2 unit as the products (fp16 1032.0 = 0x6408, 1152.0 = 0x6480).
__device__ __forceinline__ float q_offset(uint32_t x0, uint32_t x1, uint32_t x2, uint32_t x3, float acc) {
    acc = dot2h(x0, 0x64086408u, acc);
    acc = dot2h(x1, 0x64806480u, acc);
    acc = dot2h(x2, 0x64086408u, acc);
    acc = dot2h(x3, 0x64806480u, acc);
    return acc;
}

// ---------------------------------------------------------------------------
// Wave-level helpers (wave64).
// ---------------------------------------------------------------------------
// Raw buffer loads: a wave-uniform descriptor (base, size) in SGPRs, one VGPR
// byte offset per lane and a wave-uniform SGPR offset, so runs of row loads
// need no per-row VGPR addresses; reads past `bytes` return zero.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_buf(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint16_t bload2(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
}
__device__ __forceinline__ uint32_t bload4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}
// Non-temporal variants (cache policy "nt") for data read once, such as the
// weight streams: on MI355X a plain streaming read of 2 GiB reaches ~6.3 TB/s
// with nt loads against ~5.8 TB/s without.
constexpr int kCachePolicyNT = 2;
__device__ __forceinline__ uint4 bload16_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kCachePolicyNT);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint16_t bload2_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, kCachePolicyNT);
}
// Same loads marked volatile (bit 31 of the cache-policy operand): a reload
// of data already in registers that the compiler must not merge with the
// first load (which would make everything derived from it loop-invariant).
constexpr int kVolatileLoad = (int)(1u << 31);
__device__ __forceinline__ uint4 bload16_nt_reload(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kCachePolicyNT | kVolatileLoad);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint16_t bload2_nt_reload(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, kCachePolicyNT | kVolatileLoad);
}

// Order point for register pressure: an empty asm that "reads" `after` and
// "rewrites" `next`, so the compiler cannot start work on `next` (e.g. the
// int4 -> fp16 conversion of the next row) before `after` is computed.  The
// instruction scheduler barrier alone does not stop the earlier
// instruction-selection scheduling from converting every row up front.
__device__ __forceinline__ void order_after(uint4 &next, float after) {
    asm volatile("" : "+v"(next.x), "+v"(next.y), "+v"(next.z), "+v"(next.w) : "v"(after));
}

// Mark a value the compiler cannot prove wave-uniform as uniform (SGPR), so
// addresses built from it use scalar bases and loads through it are scalar.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int wave_id() { return uniform(threadIdx.x >> 6); }

// v of lane (lane ^ m).  For the partners inside a row of 16 lanes (m = 1, 2,
// 4, 8, known at compile time after unrolling) this is a DPP move (quad
// permutes and row rotations) instead of an LDS crossbar round trip; other
// distances use ds_bpermute.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float shfl_xor_f(float v, int m) {
    if (__builtin_constant_p(m)) {
        if (m == 1) return dpp_move<0xb1>(v);   // quad_perm [1, 0, 3, 2]
        if (m == 2) return dpp_move<0x4e>(v);   // quad_perm [2, 3, 0, 1]
        if (m == 4) {
            // row_ror:r gives lane i the value of lane (i - r) mod 16 of its row
            const float from_below = dpp_move<0x124>(v);   // lane i - 4
            const float from_above = dpp_move<0x12c>(v);   // lane i + 4
            return (threadIdx.x & 4) ? from_below : from_above;
        }
        if (m == 8) return dpp_move<0x128>(v);  // row_ror:8: lane i ^ 8
    }
    return __shfl_xor(v, m, kWave);
}

// fwht128 of the 128-blocks held by 16-lane groups (lane j of a group holds
// elements [8j, 8j + 8) of its block), in fp32: the Sylvester butterfly, each
// stage replacing (a, b) at distance h by (a + b, a - b), h = 1, 2, 4 inside
// a lane and 8, 16, 32, 64 across lanes, then the 1/sqrt(128) factor.
__device__ __forceinline__ void fwht128_lanes16(float (&v)[8], int lane) {
#pragma unroll
    for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if ((i & h) == 0) {
                const float a = v[i], b = v[i + h];
                v[i] = a + b;
                v[i + h] = a - b;
            }
        }
    }
#pragma unroll
    for (int m = 1; m <= 8; m <<= 1) {   // strides 8..64: lanes of the same block
        const bool upper = (lane & m) != 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float q = shfl_xor_f(v[i], m);
            v[i] = upper ? (q - v[i]) : (v[i] + q);
        }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] *= 0.08838834764831845f;   // 1/sqrt(128)
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += shfl_xor_f(v, m);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, shfl_xor_f(v, m));
    return v;
}

// Sum V values over the `span` lanes that differ in the low log2(span) bits of
// the lane id, leaving value i = (lane & (span-1)) >> (log2(span) - log2(V)) on
// each lane (V <= span, both powers of two).  Each halving step exchanges half
// of the remaining values with the partner lane, so the cost is about V
// shuffles instead of V*log2(span).
// Lane-dependent choice between two register values as bit operations: a
// plain `cond ? v[i] : v[i + half]` is turned by the compiler into a select
// of addresses, i.e. dynamic indexing of v, which costs a compare and a
// select per element of v.
__device__ __forceinline__ float pick_bits(uint32_t mask, float if_set, float if_clear) {
    return __uint_as_float((__float_as_uint(if_set) & mask) | (__float_as_uint(if_clear) & ~mask));
}

template <int V, int SPAN>
__device__ __forceinline__ float transpose_reduce(float (&v)[V]) {
    const int lane = threadIdx.x & (kWave - 1);
    constexpr int kSteps = __builtin_ctz(V);
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
        const int m = SPAN >> (s + 1);          // partner distance
        const int half = V >> (s + 1);          // values kept after this step
        const uint32_t upper = (lane & m) ? 0xffffffffu : 0u;
#pragma unroll
        for (int i = 0; i < half; ++i) {
            const float a = v[i], b = v[i + half];
            const float send = pick_bits(upper, a, b);
            const float keep = pick_bits(upper, b, a);
            v[i] = keep + shfl_xor_f(send, m);
        }
    }
    float r = v[0];
#pragma unroll
    for (int m = (SPAN >> kSteps) >> 1; m >= 1; m >>= 1) r += shfl_xor_f(r, m);
    return r;
}

}  // namespace moe_w4
