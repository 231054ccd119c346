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
#include "gemv_ops.h"

namespace moe_w4 {

// =========================================================================
// gate/up.  A wave item is (active expert slot, gate rows [r0, r0 + 4*NB)
// and the same up rows), streamed as NB batches of 4 row pairs (8 KB): the
// loads of batch b+1 go into the registers batch b frees, so 8 KB per wave
// stay in flight.  The first batch is requested as soon as the expert is
// known, before the tokens are read.  Lane l owns K [32l, 32l+32) of every
// row.  One or two tokens per pass; more tokens re-read the rows (L2 hits).
// =========================================================================
// NB batches of 4 row pairs for NT tokens (1 or 2; n_valid <= NT).  On entry
// R holds the first batch; the next batch is loaded into the registers each
// row frees.
template <int NB, int NT>
__device__ __forceinline__ void gu_compute(GuRows &R, rsrc_t cg, rsrc_t sp, uint32_t cv, uint32_t sv, int r0,
                                           const uint32_t *__restrict__ xt, const float *__restrict__ xt_scale,
                                           int t_a, int t_b, int p0, int n_valid, int lane,
                                           float *__restrict__ act) {
    constexpr int V = 2 * kGuPairs * NT;
    constexpr int kLogV = __builtin_ctz(V);
    uint32_t xs[NT][16];
    float off[NT], sc[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        const int t = n ? t_b : t_a;
        off[n] = load_operand32(xt + (size_t)t * (kH / 2) + lane * 16, xs[n]);
        sc[n] = __builtin_bit_cast(float, uniform(__builtin_bit_cast(int, xt_scale[t])));
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const int rb = r0 + kGuPairs * b;
        float v[V];
#pragma unroll
        for (int i = 0; i < kGuPairs; ++i) {
            const int rn = rb + kGuPairs + i;   // same pair of the next batch
#pragma unroll
            for (int h = 0; h < 2; ++h) {      // gate row, then up row
                Q4 q[4];
                convert16(h ? R.u[i] : R.g[i], q);
                const float sr = bf16_to_f32(h ? R.su[i] : R.sg[i]);
                if (b + 1 < NB) {   // refill the freed registers with the next batch
                    if (h) {
                        R.u[i] = bload16_nt(cg, cv, kPlaneGateBytes + rn * (kH / 2));
                        R.su[i] = bload2_nt(sp, sv, 2 * (kScalesGate + rn * (kH / kG)));
                    } else {
                        R.g[i] = bload16_nt(cg, cv, rn * (kH / 2));
                        R.sg[i] = bload2_nt(sp, sv, 2 * rn * (kH / kG));
                    }
                }
#pragma unroll
                for (int n = 0; n < NT; ++n) v[(i * NT + n) * 2 + h] = dot_slice(q, xs[n], -off[n]) * sr;
                __builtin_amdgcn_sched_barrier(0);   // one row at a time (register pressure)
            }
        }
        const float red = transpose_reduce<V, 64>(v);
        const float other = shfl_xor_f(red, 1 << (6 - kLogV));
        const int vi = lane >> (6 - kLogV);
        const int i = vi / (2 * NT), n = (vi >> 1) % NT;
        if ((vi & 1) == 0 && (lane & ((1 << (6 - kLogV)) - 1)) == 0 && n < n_valid) {
            const float s = n ? sc[NT - 1] : sc[0];
            const float g = red * s, u = other * s;
            act[(size_t)(p0 + n) * kI + rb + i] = silu_f(g) * u;
        }
    }
}

template <int NB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void k_gateup_dec(
    const uint8_t *__restrict__ codes, const uint16_t *__restrict__ scales, const uint32_t *__restrict__ xt,
    const float *__restrict__ xt_scale, const int *__restrict__ perm, const int *__restrict__ slots,
    float *__restrict__ act) {
    constexpr int kRows = kGuPairs * NB;
    constexpr int kItems = kI / kRows;   // items per expert
    const int lane = threadIdx.x & 63;
    const int item = blockIdx.x * 4 + wave_id();
    const int *rec = slots + 8 * (item / kItems);   // {expert, p_begin, n, t0, t1}
    const int e = rec[0];
    if (e < 0) return;   // slot without an expert
    const int p_begin = rec[1], n = rec[2], t0 = rec[3], t1 = rec[4];
    const int r0 = (item % kItems) * kRows;
    const rsrc_t cg = make_buf(codes + (size_t)e * kCodeBytesPerExpert, kCodeBytesGu);
    const rsrc_t sp = make_buf(scales + (size_t)e * kScalesPerExpert, 2 * kScalesGu);
    const uint32_t cv = lane * 16, sv = (lane >> 2) * 2;
    GuRows R;
    if (n == 1) {
        // the common decode case: one token, no second operand set
#pragma unroll
        for (int i = 0; i < kGuPairs; ++i) gu_load_pair<false>(R, i, cg, sp, cv, sv, r0 + i);
        gu_compute<NB, 1>(R, cg, sp, cv, sv, r0, xt, xt_scale, t0, t0, p_begin, 1, lane, act);
        return;
    }
    // Two or more tokens, two at a time through one call site.  Later pairs
    // re-read the rows (L2 hits) with volatile loads, which the compiler cannot
    // merge with the first ones (that would make every row's conversion
    // loop-invariant and hold all of them in registers).
#pragma unroll
    for (int i = kGuPairs - 1; i >= 0; --i) gu_load_pair<true>(R, i, cg, sp, cv, sv, r0 + i);
    const int p_end = p_begin + n;
    int ta = t0, tb = t1;
    for (int p0 = p_begin;;) {
        gu_compute<NB, 2>(R, cg, sp, cv, sv, r0, xt, xt_scale, ta, tb, p0, min(2, p_end - p0), lane, act);
        p0 += 2;
        if (p0 >= p_end) break;
#pragma unroll
        for (int i = kGuPairs - 1; i >= 0; --i) gu_load_pair<true>(R, i, cg, sp, cv, sv, r0 + i);
        ta = perm[p0] / kTopK;
        tb = perm[min(p0 + 1, p_end - 1)] / kTopK;
    }
}

// =========================================================================
// down.  A wave item is (active expert slot, rows [n0, n0 + 4*kDnLoads)):
// 8 KB of codes in kDnLoads wave loads (4 rows each; 16 lanes per row, lane
// j = lane & 15 owns K [32j, 32j+32), inside block j/4), all requested as
// soon as the expert is known.  The four waves of a workgroup share one
// expert; while their codes are in flight they turn up to four of its
// assignments' a = silu(g)*u into fp16 operands in LDS (wave w: assignment
// w; Hadamard per 128-block and a power-of-two prescale per block, as the
// down projection's rotated basis needs).
// =========================================================================
constexpr int kDnLoads = 8;

struct DnRows {
    uint4 w[kDnLoads];
    uint16_t s[kDnLoads];
};

template <bool RELOAD>
__device__ __forceinline__ void dn_load(DnRows &R, rsrc_t cd, rsrc_t sp, uint32_t cv, uint32_t sv, int n0) {
#pragma unroll
    for (int q = 0; q < kDnLoads; ++q) {
        if (RELOAD) {
            R.w[q] = bload16_nt_reload(cd, cv, (n0 + 4 * q) * (kI / 2));
            R.s[q] = bload2_nt_reload(sp, sv, 2 * (n0 + 4 * q) * (kI / kG));
        } else {
            R.w[q] = bload16_nt(cd, cv, (n0 + 4 * q) * (kI / 2));
            R.s[q] = bload2_nt(sp, sv, 2 * (n0 + 4 * q) * (kI / kG));
        }
    }
}

// at, at_scale: the NT assignments' operands in LDS (rows of kI/2 words and
// kI/kG block multipliers); p0: the sorted position of the first.
template <int NT>
__device__ __forceinline__ void dn_compute(DnRows &R, int n0, const uint32_t *at, const float *at_scale, int p0,
                                           int n_valid, int lane, float *__restrict__ o) {
    constexpr int kPerRed = 2;                 // wave loads per reduction
    constexpr int V = kPerRed * NT;
    constexpr int kLogV = __builtin_ctz(V);
    const int j = lane & 15, rsub = lane >> 4;
    uint32_t xs[NT][16];
    float off[NT], mult[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        const int q = min(n, n_valid - 1);
        off[n] = load_operand32(at + q * (kI / 2) + j * 16, xs[n]);
        mult[n] = at_scale[q * (kI / kG) + (j >> 2)];
    }
#pragma unroll
    for (int q0 = 0; q0 < kDnLoads; q0 += kPerRed) {
        float v[V];
#pragma unroll
        for (int k = 0; k < kPerRed; ++k) {
            Q4 qq[4];
            convert16(R.w[q0 + k], qq);
            const float scale_row = bf16_to_f32(R.s[q0 + k]);
#pragma unroll
            for (int n = 0; n < NT; ++n) v[k * NT + n] = dot_slice(qq, xs[n], -off[n]) * (scale_row * mult[n]);
            if (q0 + k + 1 < kDnLoads) order_after(R.w[q0 + k + 1], v[k * NT]);
        }
        const float red = transpose_reduce<V, 16>(v);
        const int vi = j >> (4 - kLogV);
        const int k = vi / NT, n = vi % NT;
        if ((j & ((1 << (4 - kLogV)) - 1)) == 0 && n < n_valid)
            o[(size_t)(p0 + n) * kH + n0 + 4 * (q0 + k) + rsub] = red;
    }
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void k_down_dec(
    const uint8_t *__restrict__ codes, const uint16_t *__restrict__ scales, const float *__restrict__ act,
    const int *__restrict__ slots, float *__restrict__ o) {
    constexpr int kRows = 4 * kDnLoads;
    constexpr int kItems = kH / kRows;
    static_assert(kItems % 4 == 0, "the four waves of a workgroup must share one expert");
    __shared__ uint32_t at[4][kI / 2];
    __shared__ float at_scale[4][kI / kG];
    const int wave = wave_id();
    const int lane = threadIdx.x & 63;
    const int item = blockIdx.x * 4 + wave;
    const int *rec = slots + 8 * (item / kItems);   // {expert, p_begin, n, ...}
    const int e = rec[0];
    if (e < 0) return;
    const int p_begin = rec[1], n = rec[2];
    const int n0 = (item % kItems) * kRows;
    const int j = lane & 15, rsub = lane >> 4;
    const rsrc_t cd = make_buf(codes + (size_t)e * kCodeBytesPerExpert + kCodeBytesGu, kCodeBytesPerExpert - kCodeBytesGu);
    const rsrc_t sp = make_buf(scales + (size_t)e * kScalesPerExpert + kScalesGu, 2 * (kScalesPerExpert - kScalesGu));
    const uint32_t cv = rsub * (kI / 2) + j * 16, sv = 2 * (rsub * (kI / kG) + (j >> 2));
    // a of the assignment p (wave w: p = c + w), requested before the codes so
    // that the rotation waits only for it; its operands go to LDS slot w
    float4 a0, a1;
    auto load_a = [&](int p) {
        const rsrc_t ab = make_buf(act + (size_t)p * kI, kI * 4);
        a0 = __builtin_bit_cast(float4, bload16(ab, lane * 32, 0));
        a1 = __builtin_bit_cast(float4, bload16(ab, lane * 32 + 16, 0));
    };
    auto rotate = [&]() { rotate_act_wave(a0, a1, lane, at[wave], at_scale[wave]); };
    DnRows R;
    if (n == 1) {   // the common decode case
        if (wave == 0) load_a(p_begin);
        dn_load<false>(R, cd, sp, cv, sv, n0);
        if (wave == 0) rotate();
        __syncthreads();
        dn_compute<1>(R, n0, at[0], at_scale[0], p_begin, 1, lane, o);
        return;
    }
    // two or more tokens: four assignments per round of operands, two at a
    // time through one call site; volatile reloads (L2 hits) keep the rows
    // loop-variant
    const int p_end = p_begin + n;
    for (int c = p_begin; c < p_end; c += 4) {
        const bool mine = c + wave < p_end;
        if (mine) load_a(c + wave);
        dn_load<true>(R, cd, sp, cv, sv, n0);
        if (c != p_begin) __syncthreads();   // every wave is done with the last round's operands
        if (mine) rotate();
        __syncthreads();
        const int m = min(4, p_end - c);
        for (int q = 0; q < m; q += 2) {
            if (q) dn_load<true>(R, cd, sp, cv, sv, n0);
            dn_compute<2>(R, n0, at[q], at_scale[q], c + q, min(2, m - q), lane, o);
        }
    }
}

// ------------------------------------------------------------------ launchers
void launch_gateup_gemv(const uint8_t *codes, const uint16_t *scales, const uint32_t *xt,
                        const float *xt_scale, const int *perm, const int *slots, int T, float *act,
                        hipStream_t s) {
    const int max_active = min(kE, kTopK * T);
    const int waves = max_active * (kI / kGuPairs);
    hipLaunchKernelGGL((k_gateup_dec<1>), dim3((waves + 3) / 4), dim3(256), 0, s, codes, scales, xt, xt_scale,
                       perm, slots, act);
}

void launch_down_gemv(const uint8_t *codes, const uint16_t *scales, const float *act, const int *slots, int T,
                      float *o, hipStream_t s) {
    const int max_active = min(kE, kTopK * T);
    const int waves = max_active * (kH / (4 * kDnLoads));   // 64 items per expert
    hipLaunchKernelGGL(k_down_dec, dim3((waves + 3) / 4), dim3(256), 0, s, codes, scales, act, slots, o);
}

}  // namespace moe_w4
