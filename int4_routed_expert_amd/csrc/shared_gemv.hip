// Ungated bf16 shared expert: z = Wsd (silu(Wsg x) * (Wsu x)), width 1024.
//
// Flint model card (Aijuus/flint-w4exp), introduction: top-6 routed experts
// plus an ungated shared expert; table row "weights": the shared expert stays
// bf16 (section "Why the linears stay bf16": quantising it kills the model).
// NInfer README of Flint, "What is inside": shared expert (1024) with gate and
// up rows.  The shared expert sees x itself, not the rotated x.
//
// bf16 weights times bf16 activations on v_dot2_f32_bf16 (exact products,
// fp32 sums).  The intermediate h = silu(g)*u is rounded to bf16 once, as the
// operand of the down projection.
#include "common.h"
#include "launch.h"

namespace moe_w4 {

__device__ __forceinline__ uint4 ldg4s(const void *p) { return *reinterpret_cast<const uint4 *>(p); }

// gate/up: wave owns P pairs (gate row r, up row r); lane l owns K [32l, 32l+32).
template <int P, int NT, int TT>
__global__ __launch_bounds__(256) void k_shared_gateup(const uint16_t *__restrict__ w,
                                                       const uint16_t *__restrict__ x, int T,
                                                       uint16_t *__restrict__ hs) {
    constexpr int V = 2 * P * NT;
    constexpr int kLogV = __builtin_ctz(V);
    static_assert((V & (V - 1)) == 0 && V <= 64, "V must be a power of two <= 64");
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r0 = (blockIdx.x * 4 + wave) * P;
    const int t_begin = blockIdx.y * TT, t_end = min(t_begin + TT, T);
    uint32_t wg[P][16], wu[P][16];
#pragma unroll
    for (int i = 0; i < P; ++i) {
        const uint16_t *g = w + (size_t)(r0 + i) * kH + lane * 32;
        const uint16_t *u = g + kSharedGateElems;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint4 a = ldg4s(g + 8 * c), b = ldg4s(u + 8 * c);
            wg[i][4 * c] = a.x; wg[i][4 * c + 1] = a.y; wg[i][4 * c + 2] = a.z; wg[i][4 * c + 3] = a.w;
            wu[i][4 * c] = b.x; wu[i][4 * c + 1] = b.y; wu[i][4 * c + 2] = b.z; wu[i][4 * c + 3] = b.w;
        }
    }
    for (int t0 = t_begin; t0 < t_end; t0 += NT) {
        uint32_t xs[NT][16];
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            const int t = min(t0 + n, t_end - 1);
            const uint16_t *xp = x + (size_t)t * kH + lane * 32;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint4 a = ldg4s(xp + 8 * c);
                xs[n][4 * c] = a.x; xs[n][4 * c + 1] = a.y; xs[n][4 * c + 2] = a.z; xs[n][4 * c + 3] = a.w;
            }
        }
        float v[V];
#pragma unroll
        for (int i = 0; i < P; ++i) {
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                float ag = 0.0f, au = 0.0f;
#pragma unroll
                for (int d = 0; d < 16; ++d) {
                    ag = dot2b(wg[i][d], xs[n][d], ag);
                    au = dot2b(wu[i][d], xs[n][d], au);
                }
                v[(i * NT + n) * 2 + 0] = ag;
                v[(i * NT + n) * 2 + 1] = au;
            }
        }
        const float r = transpose_reduce<V, 64>(v);
        const float other = shfl_xor_f(r, 1 << (6 - kLogV));
        const int vi = lane >> (6 - kLogV);
        const int i = vi / (2 * NT), n = (vi >> 1) % NT;
        const int t = t0 + n;
        if ((vi & 1) == 0 && (lane & ((1 << (6 - kLogV)) - 1)) == 0 && t < t_end) {
            const float h = r / (1.0f + expf(-r)) * other;
            hs[(size_t)t * kIS + r0 + i] = f32_to_bf16(h);
        }
    }
}

// down: rows of 1024 bf16 (2 KB); 32 lanes per row, lane owns K [32(l&31), +32);
// one wave load covers 2 rows; Q loads per wave.
template <int Q, int NT, int TT>
__global__ __launch_bounds__(256) void k_shared_down(const uint16_t *__restrict__ w,
                                                     const uint16_t *__restrict__ hs, int T,
                                                     float *__restrict__ z) {
    constexpr int V = Q * NT;
    constexpr int kLogV = __builtin_ctz(V);
    static_assert((V & (V - 1)) == 0 && V <= 32, "V must be a power of two <= 32");
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int j = lane & 31, rsub = lane >> 5;
    const int n_base = (blockIdx.x * 4 + wave) * 2 * Q;
    const int t_begin = blockIdx.y * TT, t_end = min(t_begin + TT, T);
    const uint16_t *wd = w + 2 * kSharedGateElems + (size_t)(n_base + rsub) * kIS + j * 32;
    uint32_t wr[Q][16];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint4 a = ldg4s(wd + (size_t)q * 2 * kIS + 8 * c);
            wr[q][4 * c] = a.x; wr[q][4 * c + 1] = a.y; wr[q][4 * c + 2] = a.z; wr[q][4 * c + 3] = a.w;
        }
    }
    for (int t0 = t_begin; t0 < t_end; t0 += NT) {
        uint32_t hsv[NT][16];
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            const int t = min(t0 + n, t_end - 1);
            const uint16_t *hp = hs + (size_t)t * kIS + j * 32;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint4 a = ldg4s(hp + 8 * c);
                hsv[n][4 * c] = a.x; hsv[n][4 * c + 1] = a.y; hsv[n][4 * c + 2] = a.z; hsv[n][4 * c + 3] = a.w;
            }
        }
        float v[V];
#pragma unroll
        for (int q = 0; q < Q; ++q) {
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                float acc = 0.0f;
#pragma unroll
                for (int d = 0; d < 16; ++d) acc = dot2b(wr[q][d], hsv[n][d], acc);
                v[q * NT + n] = acc;
            }
        }
        const float r = transpose_reduce<V, 32>(v);
        const int vi = j >> (5 - kLogV);
        const int q = vi / NT, n = vi % NT;
        const int t = t0 + n;
        if ((j & ((1 << (5 - kLogV)) - 1)) == 0 && t < t_end) z[(size_t)t * kH + n_base + 2 * q + rsub] = r;
    }
}

void launch_shared_gateup(const uint16_t *w, const uint16_t *x, int T, uint16_t *hs, hipStream_t s) {
    constexpr int P = 2, NT = 4, TT = 64;
    dim3 grid(kIS / (4 * P), (T + TT - 1) / TT);
    hipLaunchKernelGGL((k_shared_gateup<P, NT, TT>), grid, dim3(256), 0, s, w, x, T, hs);
}

void launch_shared_down(const uint16_t *w, const uint16_t *hs, int T, float *z, hipStream_t s) {
    constexpr int Q = 4, NT = 4, TT = 64;
    dim3 grid(kH / (4 * 2 * Q), (T + TT - 1) / TT);
    hipLaunchKernelGGL((k_shared_down<Q, NT, TT>), grid, dim3(256), 0, s, w, hs, T, z);
}

}  // namespace moe_w4
