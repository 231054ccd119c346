// Routed experts at decode sizes: grouped, HBM-streaming GEMV over int4 codes.
//
// Format (Flint model card, Aijuus/flint-w4exp, table row "weights"): signed
// int4 codes, one bf16 scale per 128 of K, in a fwht128-rotated basis.  Bank
// layout (NInfer README of Flint, "What is inside"): per expert, gate rows
// then up rows (2 x 512, K = 2048) and 2,048 down rows (K = 512).
//
// Work is split into wave-sized items: (expert with tokens, a run of rows).
// A wave streams its rows in batches of 8 KB with the next batch's loads in
// flight while the current one is multiplied, so the whole grid keeps
// hundreds of KB per CU outstanding.  Codes become exact fp16 operands by bit
// masks (int4x8_to_q) and meet the activations on v_dot2_f32_f16 with fp32
// sums; each lane's 32-element K slice lies inside one 128-group, so the bf16
// scale is applied once per lane and row.  The codes of a row are read from
// HBM once for all tokens routed to that expert.
#include "common.h"
#include "launch.h"

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

template <int N>
__device__ __forceinline__ float pick(const float (&a)[N], int i) {
    float r = a[0];
#pragma unroll
    for (int k = 1; k < N; ++k) r = (i == k) ? a[k] : r;
    return r;
}

// =========================================================================
// gate/up.  A wave item is (active expert slot, gate rows [r0, r0+RPI) and
// the same up rows).  Lane l owns K [32l, 32l+32) of every row.  Rows are
// consumed in pairs (gate r, up r); the loads of the pair four ahead are
// issued into the registers a pair frees, so 8 KB per wave stay in flight
// without a second buffer.  At most two tokens are held in registers; an
// expert with more tokens is streamed again per pair of tokens (the rows are
// then L2 hits).
// =========================================================================
template <int NT>
__device__ __forceinline__ void gu_tokens(const uint32_t *__restrict__ xt, const float *__restrict__ xt_scale,
                                          const int *__restrict__ perm, int p0, int n_valid, int lane,
                                          uint32_t (&xs)[NT][16], float (&off)[NT], float (&sc)[NT]) {
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        const int p = p0 + min(n, n_valid - 1);
        const int t = uniform(perm[p]) / kTopK;
        off[n] = load_operand32(xt + (size_t)t * (kH / 2) + lane * 16, xs[n]);
        sc[n] = __builtin_bit_cast(float, uniform(__builtin_bit_cast(int, xt_scale[t])));
    }
}

template <int NT, int RPI>
__device__ __forceinline__ void gu_stream(rsrc_t cg, rsrc_t sp, uint32_t cv, uint32_t sv, int r0,
                                          const uint32_t *__restrict__ xt, const float *__restrict__ xt_scale,
                                          const int *__restrict__ perm, int p0, int n_valid, int lane,
                                          float *__restrict__ act) {
    constexpr int kDepth = 4;   // row pairs in flight
    constexpr int V = 2 * kDepth * NT;
    constexpr int kLogV = __builtin_ctz(V);
    uint4 rg[kDepth], ru[kDepth];
    uint16_t sg[kDepth], su[kDepth];   // bf16 bits of the gate and up scales
#pragma unroll
    for (int i = 0; i < kDepth; ++i) {
        rg[i] = bload16(cg, cv, (r0 + i) * (kH / 2));
        ru[i] = bload16(cg, cv, kPlaneGateBytes + (r0 + i) * (kH / 2));
        sg[i] = bload2(sp, sv, 2 * (r0 + i) * (kH / kG));
        su[i] = bload2(sp, sv, 2 * (kScalesGate + (r0 + i) * (kH / kG)));
    }
    uint32_t xs[NT][16];
    float off[NT], sc[NT];
    gu_tokens<NT>(xt, xt_scale, perm, p0, n_valid, lane, xs, off, sc);
#pragma unroll
    for (int b = 0; b < RPI / kDepth; ++b) {
        float v[V];
#pragma unroll
        for (int i = 0; i < kDepth; ++i) {
            const int r = r0 + kDepth * b + i;
            const bool more = kDepth * (b + 1) < RPI;
            {
                Q4 q[4];
                convert16(rg[i], q);
                const float sc_row = bf16_to_f32(sg[i]);
                if (more) {
                    rg[i] = bload16(cg, cv, (r + kDepth) * (kH / 2));
                    sg[i] = bload2(sp, sv, 2 * (r + kDepth) * (kH / kG));
                }
#pragma unroll
                for (int n = 0; n < NT; ++n) v[(i * NT + n) * 2 + 0] = dot_slice(q, xs[n], -off[n]) * sc_row;
            }
            {
                Q4 q[4];
                convert16(ru[i], q);
                const float sc_row = bf16_to_f32(su[i]);
                if (more) {
                    ru[i] = bload16(cg, cv, kPlaneGateBytes + (r + kDepth) * (kH / 2));
                    su[i] = bload2(sp, sv, 2 * (kScalesGate + (r + kDepth) * (kH / kG)));
                }
#pragma unroll
                for (int n = 0; n < NT; ++n) v[(i * NT + n) * 2 + 1] = dot_slice(q, xs[n], -off[n]) * sc_row;
            }
            __builtin_amdgcn_sched_barrier(0);   // keep the ring: no hoisting of later loads
        }
        const float red = transpose_reduce<V, 64>(v);
        const float other = shfl_xor_f(red, 1 << (6 - kLogV));
        const int vi = lane >> (6 - kLogV);
        const int i = vi / (2 * NT), n = (vi >> 1) % NT;
        if ((vi & 1) == 0 && (lane & ((1 << (6 - kLogV)) - 1)) == 0 && n < n_valid) {
            const float s = pick(sc, n);
            const float g = red * s, u = other * s;
            act[(size_t)(p0 + n) * kI + r0 + kDepth * b + i] = silu_f(g) * u;
        }
    }
}

template <int RPI>
__global__ __launch_bounds__(256) void k_gateup_dec(const uint8_t *__restrict__ codes,
                                                    const uint16_t *__restrict__ scales,
                                                    const uint32_t *__restrict__ xt,
                                                    const float *__restrict__ xt_scale,
                                                    const int *__restrict__ offsets,
                                                    const int *__restrict__ perm,
                                                    const int *__restrict__ n_active,
                                                    const int *__restrict__ active,
                                                    float *__restrict__ act) {
    constexpr int kItems = kI / RPI;   // items per expert
    const int lane = threadIdx.x & 63;
    const int item = blockIdx.x * 4 + wave_id();
    const int slot = item / kItems;
    if (slot >= uniform(*n_active)) return;
    const int e = uniform(active[slot]);
    const int r0 = (item % kItems) * RPI;
    const rsrc_t cg = make_buf(codes + (size_t)e * kCodeBytesPerExpert, kCodeBytesGu);
    const rsrc_t sp = make_buf(scales + (size_t)e * kScalesPerExpert, 2 * kScalesGu);
    const uint32_t cv = lane * 16, sv = (lane >> 2) * 2;
    const int p_begin = uniform(offsets[e]), p_end = uniform(offsets[e + 1]);
    for (int p0 = p_begin; p0 < p_end; p0 += 2) {
        if (p_end - p0 == 1) gu_stream<1, RPI>(cg, sp, cv, sv, r0, xt, xt_scale, perm, p0, 1, lane, act);
        else gu_stream<2, RPI>(cg, sp, cv, sv, r0, xt, xt_scale, perm, p0, 2, lane, act);
    }
}

// =========================================================================
// down.  A wave item is (active expert slot, rows [n0, n0+RPI)).  The wave
// first rotates a = silu(g)*u of the expert's tokens (Hadamard per 128-block,
// power-of-two prescale per block, fp16 operands) through its own LDS slot,
// then streams its rows: 16 lanes per row (lane j = lane & 15 owns K
// [32j, 32j+32), inside block j/4), one 1 KiB wave load = 4 rows.
// =========================================================================
constexpr int kDownNT = 4;
struct DownLds {
    uint32_t at[kDownNT][kI / 2];   // fp16 operands, 1 KiB per token
    float mult[kDownNT][kI / kG];   // 2^shift per block
};

// Rotate token p's a (fp32 [512]) into the wave's LDS slot n.
__device__ __forceinline__ void rotate_into_lds(const float *__restrict__ act, int p, int n, int lane, DownLds &L) {
    const float4 *src = reinterpret_cast<const float4 *>(act + (size_t)p * kI + lane * 8);
    const float4 a0 = src[0], a1 = src[1];
    float v[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
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
        sh = ex - 14;   // largest magnitude in [2^13, 2^14): exact, far from fp16 overflow
    }
    uint4 w;
    w.x = pack_half2(ldexpf(v[0], -sh), ldexpf(v[4], -sh));
    w.y = pack_half2(ldexpf(v[1], -sh - 4), ldexpf(v[5], -sh - 4));
    w.z = pack_half2(ldexpf(v[2], -sh), ldexpf(v[6], -sh));
    w.w = pack_half2(ldexpf(v[3], -sh - 4), ldexpf(v[7], -sh - 4));
    reinterpret_cast<uint4 *>(L.at[n])[lane] = w;
    if ((lane & 15) == 0) L.mult[n][lane >> 4] = ldexpf(1.0f, sh);
}

template <int NT, int RPI>
__device__ __forceinline__ void dn_stream(rsrc_t cd, rsrc_t sp, uint32_t cv, uint32_t sv, int n0,
                                          const DownLds &L, int slot0, int p0, int n_valid, int lane,
                                          float *__restrict__ o) {
    constexpr int kDepth = 4;          // wave loads (4 rows each) in flight
    constexpr int V = kDepth * NT;
    constexpr int kLogV = __builtin_ctz(V);
    const int j = lane & 15, rsub = lane >> 4;
    uint4 w[kDepth];
    uint16_t s[kDepth];
#pragma unroll
    for (int q = 0; q < kDepth; ++q) {
        w[q] = bload16(cd, cv, (n0 + 4 * q) * (kI / 2));
        s[q] = bload2(sp, sv, 2 * (n0 + 4 * q) * (kI / kG));
    }
    uint32_t xs[NT][16];
    float off[NT], mult[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        const int nn = slot0 + min(n, n_valid - 1);   // LDS slot of this token
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint4 q = reinterpret_cast<const uint4 *>(L.at[nn] + 16 * j)[i];
            xs[n][4 * i] = q.x; xs[n][4 * i + 1] = q.y; xs[n][4 * i + 2] = q.z; xs[n][4 * i + 3] = q.w;
            acc = q_offset(q.x, q.y, q.z, q.w, acc);
        }
        off[n] = acc;
        mult[n] = L.mult[nn][j >> 2];
    }
#pragma unroll
    for (int b = 0; b < RPI / (4 * kDepth); ++b) {
        float v[V];
#pragma unroll
        for (int q = 0; q < kDepth; ++q) {
            const int r = n0 + 4 * (kDepth * b + q);
            Q4 qq[4];
            convert16(w[q], qq);
            const float scale_row = bf16_to_f32(s[q]);
            if (4 * kDepth * (b + 1) < RPI) {
                w[q] = bload16(cd, cv, (r + 4 * kDepth) * (kI / 2));
                s[q] = bload2(sp, sv, 2 * (r + 4 * kDepth) * (kI / kG));
            }
#pragma unroll
            for (int n = 0; n < NT; ++n) v[q * NT + n] = dot_slice(qq, xs[n], -off[n]) * (scale_row * mult[n]);
            __builtin_amdgcn_sched_barrier(0);
        }
        const float red = transpose_reduce<V, 16>(v);
        const int vi = j >> (4 - kLogV);
        const int q = vi / NT, n = vi % NT;
        if ((j & ((1 << (4 - kLogV)) - 1)) == 0 && n < n_valid)
            o[(size_t)(p0 + n) * kH + n0 + 4 * (kDepth * b + q) + rsub] = red;
    }
}

template <int RPI>
__global__ __launch_bounds__(256) void k_down_dec(const uint8_t *__restrict__ codes,
                                                  const uint16_t *__restrict__ scales,
                                                  const float *__restrict__ act,
                                                  const int *__restrict__ offsets,
                                                  const int *__restrict__ n_active,
                                                  const int *__restrict__ active,
                                                  float *__restrict__ o) {
    __shared__ DownLds lds[4];
    constexpr int kItems = kH / RPI;
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int item = blockIdx.x * 4 + wave;
    const int slot = item / kItems;
    if (slot >= uniform(*n_active)) return;
    const int e = uniform(active[slot]);
    const int n0 = (item % kItems) * RPI;
    const int j = lane & 15, rsub = lane >> 4;
    const rsrc_t cd = make_buf(codes + (size_t)e * kCodeBytesPerExpert + kCodeBytesGu, kCodeBytesPerExpert - kCodeBytesGu);
    const rsrc_t sp = make_buf(scales + (size_t)e * kScalesPerExpert + kScalesGu, 2 * (kScalesPerExpert - kScalesGu));
    const uint32_t cv = rsub * (kI / 2) + j * 16, sv = 2 * (rsub * (kI / kG) + (j >> 2));
    const int p_begin = uniform(offsets[e]), p_end = uniform(offsets[e + 1]);
    DownLds &L = lds[wave];
    for (int p0 = p_begin; p0 < p_end; p0 += kDownNT) {
        const int nv = min(kDownNT, p_end - p0);
        for (int n = 0; n < nv; ++n) rotate_into_lds(act, p0 + n, n, lane, L);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        for (int c = 0; c < nv; c += 2) {
            if (nv - c == 1) dn_stream<1, RPI>(cd, sp, cv, sv, n0, L, c, p0 + c, 1, lane, o);
            else dn_stream<2, RPI>(cd, sp, cv, sv, n0, L, c, p0 + c, 2, lane, o);
        }
        __builtin_amdgcn_wave_barrier();
    }
}

// ------------------------------------------------------------------ launchers
void launch_gateup_gemv(const uint8_t *codes, const uint16_t *scales, const uint32_t *xt,
                        const float *xt_scale, const int *offsets, const int *perm,
                        const int *n_active, const int *active, int T, float *act, hipStream_t s) {
    const int max_active = min(kE, kTopK * T);
    if (T <= 8) {
        constexpr int RPI = 4;
        const int waves = max_active * (kI / RPI);
        hipLaunchKernelGGL((k_gateup_dec<RPI>), dim3((waves + 3) / 4), dim3(256), 0, s, codes, scales, xt,
                           xt_scale, offsets, perm, n_active, active, act);
    } else {
        constexpr int RPI = 16;
        const int waves = max_active * (kI / RPI);
        hipLaunchKernelGGL((k_gateup_dec<RPI>), dim3((waves + 3) / 4), dim3(256), 0, s, codes, scales, xt,
                           xt_scale, offsets, perm, n_active, active, act);
    }
}

void launch_down_gemv(const uint8_t *codes, const uint16_t *scales, const float *act, const int *offsets,
                      const int *n_active, const int *active, int T, float *o, hipStream_t s) {
    const int max_active = min(kE, kTopK * T);
    if (T <= 8) {
        constexpr int RPI = 16;
        const int waves = max_active * (kH / RPI);
        hipLaunchKernelGGL((k_down_dec<RPI>), dim3((waves + 3) / 4), dim3(256), 0, s, codes, scales, act,
                           offsets, n_active, active, o);
    } else {
        constexpr int RPI = 64;
        const int waves = max_active * (kH / RPI);
        hipLaunchKernelGGL((k_down_dec<RPI>), dim3((waves + 3) / 4), dim3(256), 0, s, codes, scales, act,
                           offsets, n_active, active, o);
    }
}

}  // namespace moe_w4
