// Routed experts at decode sizes: grouped, HBM-streaming GEMV over int4 codes.
//
// Format (Flint model card, Aijuus/flint-w4exp, table row "weights"): signed
// int4 codes, one bf16 scale per 128 of K, in a fwht128-rotated basis.  Bank
// layout (NInfer README of Flint, "What is inside"): per expert, gate rows
// then up rows (2 x 512, K = 2048) and 2,048 down rows (K = 512).
//
// Each workgroup takes one expert that has tokens and a slice of its rows;
// the codes of those rows are read from HBM once and applied to every token
// routed to that expert.  Codes are turned into exact fp16 operands by bit
// masks (see int4x8_to_q) and multiplied on v_dot2_f32_f16 with fp32
// accumulation; the bf16 group scale is applied per lane, since each lane's
// 32-element K slice lies inside one 128-group.
#include "common.h"
#include "launch.h"

namespace moe_w4 {

__device__ __forceinline__ uint4 ldg4(const void *p) { return *reinterpret_cast<const uint4 *>(p); }

// Load one lane's 32 stored activations (16 half2 words) and their offset.
__device__ __forceinline__ float load_operand32(const uint32_t *src, uint32_t (&xs)[16]) {
    float off = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint4 v = ldg4(src + 4 * i);
        xs[4 * i] = v.x; xs[4 * i + 1] = v.y; xs[4 * i + 2] = v.z; xs[4 * i + 3] = v.w;
        off += q_offset(v.x, v.y, v.z, v.w);
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

// ---------------------------------------------------------------------------
// gate/up: for expert e, wave rows r0..r0+P of gate and of up; lane l owns
// K [32l, 32l+32).  act[p][r] = silu(g) * u for every sorted position p of e.
// ---------------------------------------------------------------------------
template <int P, int NT>
__global__ __launch_bounds__(256) void k_gateup_gemv(const uint8_t *__restrict__ codes,
                                                     const uint16_t *__restrict__ scales,
                                                     const uint32_t *__restrict__ xt,
                                                     const float *__restrict__ xt_scale,
                                                     const int *__restrict__ offsets,
                                                     const int *__restrict__ perm,
                                                     const int *__restrict__ n_active,
                                                     const int *__restrict__ active,
                                                     float *__restrict__ act) {
    constexpr int V = 2 * P * NT;
    constexpr int kLogV = __builtin_ctz(V);
    static_assert((V & (V - 1)) == 0 && V <= 64, "V must be a power of two <= 64");
    if ((int)blockIdx.x >= *n_active) return;
    const int e = active[blockIdx.x];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r0 = (blockIdx.y * 4 + wave) * P;
    const int p_begin = offsets[e], p_end = offsets[e + 1];

    const uint8_t *cg = codes + (size_t)e * kCodeBytesPerExpert + (size_t)r0 * (kH / 2) + lane * 16;
    const uint16_t *sg = scales + (size_t)e * kScalesPerExpert + r0 * (kH / kG) + (lane >> 2);
    uint4 wg[P], wu[P];
    float s_g[P], s_u[P];
#pragma unroll
    for (int i = 0; i < P; ++i) {
        wg[i] = ldg4(cg + i * (kH / 2));
        wu[i] = ldg4(cg + kPlaneGateBytes + i * (kH / 2));
        s_g[i] = bf16_to_f32(sg[i * (kH / kG)]);
        s_u[i] = bf16_to_f32(sg[kScalesGate + i * (kH / kG)]);
    }

    for (int p0 = p_begin; p0 < p_end; p0 += NT) {
        uint32_t xs[NT][16];
        float off[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            const int p = min(p0 + n, p_end - 1);
            const int t = perm[p] / kTopK;
            off[n] = load_operand32(xt + (size_t)t * (kH / 2) + lane * 16, xs[n]);
        }
        float v[V];
#pragma unroll
        for (int i = 0; i < P; ++i) {
            Q4 qg[4], qu[4];
            convert16(wg[i], qg);
            convert16(wu[i], qu);
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                v[(i * NT + n) * 2 + 0] = dot_slice(qg, xs[n], -off[n]) * s_g[i];
                v[(i * NT + n) * 2 + 1] = dot_slice(qu, xs[n], -off[n]) * s_u[i];
            }
        }
        const float r = transpose_reduce<V, 64>(v);
        // value index vi = lane >> (6 - kLogV); its gate/up partner is vi ^ 1
        const float other = shfl_xor_f(r, 1 << (6 - kLogV));
        const int vi = lane >> (6 - kLogV);
        const int i = vi / (2 * NT), n = (vi >> 1) % NT;
        const int p = p0 + n;
        if ((vi & 1) == 0 && (lane & ((1 << (6 - kLogV)) - 1)) == 0 && p < p_end) {
            const float sc = xt_scale[perm[p] / kTopK];
            const float g = r * sc, u = other * sc;
            act[(size_t)p * kI + r0 + i] = silu_f(g) * u;
        }
    }
}

void launch_gateup_gemv(const uint8_t *codes, const uint16_t *scales, const uint32_t *xt,
                        const float *xt_scale, const int *offsets, const int *perm,
                        const int *n_active, const int *active, int T, float *act, hipStream_t s) {
    constexpr int P = 4, NT = 4;
    const int max_active = min(kE, kTopK * T);
    dim3 grid(max_active, kI / (4 * P));
    hipLaunchKernelGGL((k_gateup_gemv<P, NT>), grid, dim3(256), 0, s, codes, scales, xt, xt_scale,
                       offsets, perm, n_active, active, act);
}

// ---------------------------------------------------------------------------
// a -> fp16 operands of the down projection: Hadamard on each of the four
// 128-blocks of a (one wave per assignment, lane l owns 8 values), a
// power-of-two prescale per block, stored in the int4x8_to_q operand order.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_rotate_act(const float *__restrict__ act, int n_rows,
                                                    uint32_t *__restrict__ at,
                                                    float *__restrict__ at_scale) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int p = blockIdx.x * 4 + wave;
    if (p >= n_rows) return;
    const float4 *src = reinterpret_cast<const float4 *>(act + (size_t)p * kI + lane * 8);
    const float4 a0 = src[0], a1 = src[1];
    float v[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
    // strides 1, 2, 4 inside the lane; 8..64 across lanes (lane & 15 = position in block)
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
    for (int m = 1; m <= 8; m <<= 1) {
        const bool upper = (lane & m) != 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float q = shfl_xor_f(v[i], m);
            v[i] = upper ? (q - v[i]) : (v[i] + q);
        }
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        v[i] *= 0.08838834764831845f;
        amax = fmaxf(amax, fabsf(v[i]));
    }
#pragma unroll
    for (int m = 1; m <= 8; m <<= 1) amax = fmaxf(amax, shfl_xor_f(amax, m));
    int sh = 0;
    if (amax > 0.0f && isfinite(amax)) {
        int ex;
        frexpf(amax, &ex);
        sh = ex - 14;
    }
    uint4 w;
    w.x = pack_half2(ldexpf(v[0], -sh), ldexpf(v[4], -sh));
    w.y = pack_half2(ldexpf(v[1], -sh - 4), ldexpf(v[5], -sh - 4));
    w.z = pack_half2(ldexpf(v[2], -sh), ldexpf(v[6], -sh));
    w.w = pack_half2(ldexpf(v[3], -sh - 4), ldexpf(v[7], -sh - 4));
    reinterpret_cast<uint4 *>(at + (size_t)p * (kI / 2))[lane] = w;
    if ((lane & 15) == 0) at_scale[(size_t)p * (kI / kG) + (lane >> 4)] = ldexpf(1.0f, sh);
}

void launch_rotate_act(const float *act, int T, uint32_t *at, float *at_scale, hipStream_t s) {
    const int n = kTopK * T;
    hipLaunchKernelGGL(k_rotate_act, dim3((n + 3) / 4), dim3(256), 0, s, act, n, at, at_scale);
}

// ---------------------------------------------------------------------------
// down: rows of 256 B (K = 512).  16 lanes per row, lane j = lane & 15 owns
// K [32j, 32j+32) (inside block j/4); one wave load covers 4 rows; a wave does
// Q loads.  o[p][n] for every sorted position p of the expert.
// ---------------------------------------------------------------------------
template <int Q, int NT>
__global__ __launch_bounds__(256) void k_down_gemv(const uint8_t *__restrict__ codes,
                                                   const uint16_t *__restrict__ scales,
                                                   const uint32_t *__restrict__ at,
                                                   const float *__restrict__ at_scale,
                                                   const int *__restrict__ offsets,
                                                   const int *__restrict__ n_active,
                                                   const int *__restrict__ active,
                                                   float *__restrict__ o) {
    constexpr int V = Q * NT;
    constexpr int kLogV = __builtin_ctz(V);
    static_assert((V & (V - 1)) == 0 && V <= 16, "V must be a power of two <= 16");
    if ((int)blockIdx.x >= *n_active) return;
    const int e = active[blockIdx.x];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int j = lane & 15, rsub = lane >> 4;
    const int n_base = (blockIdx.y * 4 + wave) * 4 * Q;
    const int p_begin = offsets[e], p_end = offsets[e + 1];

    const uint8_t *cd = codes + (size_t)e * kCodeBytesPerExpert + kCodeBytesGu + (size_t)(n_base + rsub) * (kI / 2) + j * 16;
    const uint16_t *sd = scales + (size_t)e * kScalesPerExpert + kScalesGu + (n_base + rsub) * (kI / kG) + (j >> 2);
    uint4 w[Q];
    float s[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        w[q] = ldg4(cd + (size_t)q * 4 * (kI / 2));
        s[q] = bf16_to_f32(sd[q * 4 * (kI / kG)]);
    }
    for (int p0 = p_begin; p0 < p_end; p0 += NT) {
        uint32_t xs[NT][16];
        float off[NT], mult[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            const int p = min(p0 + n, p_end - 1);
            off[n] = load_operand32(at + (size_t)p * (kI / 2) + j * 16, xs[n]);
            mult[n] = at_scale[(size_t)p * (kI / kG) + (j >> 2)];
        }
        float v[V];
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            Q4 qq[4];
            convert16(w[q], qq);
#pragma unroll
            for (int n = 0; n < NT; ++n) v[q * NT + n] = dot_slice(qq, xs[n], -off[n]) * (s[q] * mult[n]);
        }
        const float r = transpose_reduce<V, 16>(v);
        const int vi = j >> (4 - kLogV);
        const int q = vi / NT, n = vi % NT;
        const int p = p0 + n;
        if ((j & ((1 << (4 - kLogV)) - 1)) == 0 && p < p_end)
            o[(size_t)p * kH + n_base + 4 * q + rsub] = r;
    }
}

void launch_down_gemv(const uint8_t *codes, const uint16_t *scales, const uint32_t *at,
                      const float *at_scale, const int *offsets, const int *n_active,
                      const int *active, int T, float *o, hipStream_t s) {
    constexpr int Q = 4, NT = 4;
    const int max_active = min(kE, kTopK * T);
    dim3 grid(max_active, kH / (4 * 4 * Q));
    hipLaunchKernelGGL((k_down_gemv<Q, NT>), grid, dim3(256), 0, s, codes, scales, at, at_scale,
                       offsets, n_active, active, o);
}

}  // namespace moe_w4
