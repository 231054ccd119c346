// Routed experts in the NVFP4 container (Flint NVFP4 repack, kekzle/Flint-NVFP4,
// rows "Layout per Linear" and "Declaration"): per Linear, E2M1 codes two per
// byte, one E4M3 block scale per 16 columns of K and one fp32 tensor scale;
// the weights are in the original basis (no Hadamard) and the activations are
// not quantised (W4A16).  The experts run as streaming GEMVs at every token
// count, driven by the slot records of the sort like the int4 GEMVs.
//
// Arithmetic: gfx950 converts two E2M1 codes (one byte) to an exact fp16 pair
// in one instruction (v_cvt_scalef32_pk_f16_fp4, scale 1).  The activations
// become fp16 with a power-of-two prescale (largest magnitude in [2^13,
// 2^14)), products are exact in v_dot2_f32_f16 and summed in fp32 per
// 16-element block, the block's E4M3 scale (exact in fp32) multiplies that
// block sum, and the tensor scale and the prescale multiply the row sum.
//
// Library layout per expert e (rows in the int4 layout's order):
//   codes   e * 1,572,864 B: gate [512][1024 B], up [512][1024 B], down [2048][256 B]
//           (two codes per byte, even K in the low nibble)
//   scales  e * 196,608 B:   gate [512][128], up [512][128], down [2048][32] (E4M3)
//   tensor  e * 3 floats:    gate, up, down
#include "common.h"
#include "gemv_ops.h"
#include "launch.h"
#include "nvfp4_ops.h"
#include "token_ops.h"

namespace moe_w4 {

namespace {

// Empty asm that "rewrites" a register quad, so that the conversion of codes
// reused for several tokens is redone per token instead of being hoisted out
// of the token loop (all converted rows would not fit in registers).
__device__ __forceinline__ void refresh(uint4 &v) {
    asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
}

// =========================================================================
// gate/up.  A wave item is (active expert slot, gate rows [r0, r0 + 4) and
// the same up rows): 8 rows of 1 KiB, lane l owning K [32l, 32l + 32) of each
// (16 bytes of codes, the 2 scale bytes of blocks 2l and 2l + 1), all
// requested as soon as the expert is known.  The four waves of a workgroup
// share the expert: while their codes are in flight they turn up to four of
// its tokens' x into fp16 operands in LDS (wave w: token w of the round; the
// whole row is in one wave, so the prescale needs no other wave).  Codes are
// converted once per pair of tokens; a = silu(g) * u goes to act.
// =========================================================================
constexpr int kNvGuPairs = 4;
constexpr int kNvRows = 2 * kNvGuPairs;   // rows 0-3: gate r0 + i; 4-7: up r0 + i - 4

// NT tokens (operands xo rows, multipliers xm) against the item's 8 rows.
template <int NT>
__device__ __forceinline__ void nv_gu_compute(const uint4 (&c)[kNvRows], const float (&s0)[kNvRows],
                                              const float (&s1)[kNvRows], const uint32_t *xo, const float *xm,
                                              float tg, float tu, int r0, int p0, int n_valid, int lane,
                                              float *__restrict__ act) {
    constexpr int V = kNvRows * NT;
    constexpr int kSpan = kWave / V;   // lanes that end with one value
    uint32_t xs[NT][16];
    float mult[NT];
#pragma unroll
    for (int nn = 0; nn < NT; ++nn) {
        const int q = min(nn, n_valid - 1);
        const uint4 *src = reinterpret_cast<const uint4 *>(xo + q * (kH / 2) + lane * 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint4 w = src[i];
            xs[nn][4 * i] = w.x; xs[nn][4 * i + 1] = w.y; xs[nn][4 * i + 2] = w.z; xs[nn][4 * i + 3] = w.w;
        }
        mult[nn] = xm[q];
    }
    float r[V];
#pragma unroll
    for (int i = 0; i < kNvRows; ++i) {
        uint4 ci = c[i];
        refresh(ci);
        uint32_t h[16];
        conv32_nv(ci, h);
#pragma unroll
        for (int nn = 0; nn < NT; ++nn) r[i * NT + nn] = dot32h_nv(h, xs[nn], s0[i], s1[i]);
    }
    const float red = transpose_reduce<V, kWave>(r);   // value v = i * NT + nn on lanes kSpan*v ..
    const float up = shfl_xor_f(red, 32);               // row i + 4: lanes 32 apart
    const int v = lane / kSpan, i = v / NT, nn = v % NT;
    if (lane < 32 && lane % kSpan == 0 && nn < n_valid) {
        const float g = red * tg * mult[nn], u = up * tu * mult[nn];
        act[(size_t)(p0 + nn) * kI + r0 + i] = silu_f(g) * u;
    }
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void k_gateup_nv(const uint8_t *__restrict__ codes, const uint8_t *__restrict__ scales,
                                                   const float *__restrict__ tscales, const uint16_t *__restrict__ x,
                                                   const int *__restrict__ perm, const int *__restrict__ slots,
                                                   float *__restrict__ act) {
    constexpr int kItems = kI / kNvGuPairs;   // 128 per expert
    static_assert(kItems % 4 == 0, "the four waves of a workgroup must share one expert");
    __shared__ uint32_t xo[4][kH / 2];
    __shared__ float xm[4];
    const int lane = threadIdx.x & 63;
    const int wave = wave_id();
    const int item = blockIdx.x * 4 + wave;
    const int *rec = slots + 8 * (item / kItems);   // {expert, p_begin, n, ...}
    const int e = rec[0];
    if (e < 0) return;
    const int p_begin = rec[1], n = rec[2];
    const int r0 = (item % kItems) * kNvGuPairs;
    const rsrc_t cres = make_buf(codes + (size_t)e * kCodeBytesPerExpert, (uint32_t)kCodeBytesGu);
    const rsrc_t sres = make_buf(scales + (size_t)e * kNvScalePerExpert, kNvScaleGu);
    // x of the round's token for this wave, requested before the codes
    uint4 xq[4];
    auto load_x = [&](int p) {
        const int t = uniform(perm[p] / kTopK);
        const uint4 *xp = reinterpret_cast<const uint4 *>(x + (size_t)t * kH + 32 * lane);
#pragma unroll
        for (int i = 0; i < 4; ++i) xq[i] = xp[i];
    };
    auto stage_x = [&]() {
        float v[32];
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint4 q = xq[i];
            v[8 * i + 0] = bf16lo(q.x); v[8 * i + 1] = bf16hi(q.x);
            v[8 * i + 2] = bf16lo(q.y); v[8 * i + 3] = bf16hi(q.y);
            v[8 * i + 4] = bf16lo(q.z); v[8 * i + 5] = bf16hi(q.z);
            v[8 * i + 6] = bf16lo(q.w); v[8 * i + 7] = bf16hi(q.w);
        }
#pragma unroll
        for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
        const int sh = prescale_shift(wave_max(amax));
        uint4 *dst = reinterpret_cast<uint4 *>(xo[wave] + lane * 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float *q = v + 8 * i;
            dst[i] = make_uint4(pack_half2(ldexpf(q[0], -sh), ldexpf(q[1], -sh)),
                                pack_half2(ldexpf(q[2], -sh), ldexpf(q[3], -sh)),
                                pack_half2(ldexpf(q[4], -sh), ldexpf(q[5], -sh)),
                                pack_half2(ldexpf(q[6], -sh), ldexpf(q[7], -sh)));
        }
        xm[wave] = ldexpf(1.0f, sh);   // every lane stores the same value
    };
    const int p_end = p_begin + n;
    if (wave < n) load_x(p_begin + wave);
    uint4 c[kNvRows];
    uint16_t sb[kNvRows];
#pragma unroll
    for (int i = 0; i < kNvRows; ++i) {
        const int r = r0 + (i % kNvGuPairs);
        const uint32_t coff = (i < kNvGuPairs ? 0u : (uint32_t)kPlaneGateBytes) + (uint32_t)r * (kH / 2);
        const uint32_t soff = (i < kNvGuPairs ? 0u : kNvScaleGate) + (uint32_t)r * (kH / kNvBlock);
        c[i] = bload16_nt(cres, lane * 16, coff);
        sb[i] = bload2_nt(sres, lane * 2, soff);
    }
    const float tg = tscales[3 * e], tu = tscales[3 * e + 1];
    if (wave < n) stage_x();
    __syncthreads();
    float s0[kNvRows], s1[kNvRows];
#pragma unroll
    for (int i = 0; i < kNvRows; ++i) {
        s0[i] = e4m3_to_f32(sb[i] & 0xffu);
        s1[i] = e4m3_to_f32(sb[i] >> 8);
    }
    if (n == 1) {   // the common decode case
        nv_gu_compute<1>(c, s0, s1, xo[0], xm, tg, tu, r0, p_begin, 1, lane, act);
        return;
    }
    for (int cb = p_begin;;) {
        const int m = min(4, p_end - cb);
        for (int q = 0; q < m; q += 2)
            nv_gu_compute<2>(c, s0, s1, xo[q], xm + q, tg, tu, r0, cb + q, min(2, m - q), lane, act);
        cb += 4;
        if (cb >= p_end) break;
        __syncthreads();   // every wave is done with this round's operands
        if (cb + wave < p_end) {
            load_x(cb + wave);
            stage_x();
        }
        __syncthreads();
    }
}

// =========================================================================
// down.  A wave item is (active expert slot, rows [n0, n0 + 32)) in 8 wave
// loads of 4 rows (16 lanes per row, lane j = lane & 15 owning K [32j,
// 32j + 32): 16 bytes of codes, the scale bytes of blocks 2j and 2j + 1).
// The four waves of a workgroup share the expert; while their codes are in
// flight they turn up to four of its assignments' a into fp16 operands in
// LDS (one prescale per assignment).
// =========================================================================
constexpr int kNvDnLoads = 8;

struct NvDnRows {
    uint4 c[kNvDnLoads];
    uint16_t s[kNvDnLoads];
};

template <bool RELOAD>
__device__ __forceinline__ void nv_dn_load(NvDnRows &R, rsrc_t cd, rsrc_t sd, uint32_t cv, uint32_t sv, int n0) {
#pragma unroll
    for (int q = 0; q < kNvDnLoads; ++q) {
        if (RELOAD) {
            R.c[q] = bload16_nt_reload(cd, cv, (n0 + 4 * q) * (kI / 2));
            R.s[q] = bload2_nt_reload(sd, sv, (n0 + 4 * q) * (kI / kNvBlock));
        } else {
            R.c[q] = bload16_nt(cd, cv, (n0 + 4 * q) * (kI / 2));
            R.s[q] = bload2_nt(sd, sv, (n0 + 4 * q) * (kI / kNvBlock));
        }
    }
}

// at, at_mult: the NT assignments' operands in LDS (rows of kI/2 words) and
// their 2^sh; p0: the sorted position of the first.
template <int NT>
__device__ __forceinline__ void nv_dn_compute(const NvDnRows &R, int n0, const uint32_t *at, const float *at_mult,
                                              float tdown, int p0, int n_valid, int lane, float *__restrict__ o) {
    constexpr int kPerRed = 2;   // wave loads per reduction
    constexpr int V = kPerRed * NT;
    constexpr int kLogV = __builtin_ctz(V);
    const int j = lane & 15, rsub = lane >> 4;
    uint32_t xs[NT][16];
    float mult[NT];
#pragma unroll
    for (int nn = 0; nn < NT; ++nn) {
        const int q = min(nn, n_valid - 1);
        const uint4 *src = reinterpret_cast<const uint4 *>(at + q * (kI / 2) + j * 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint4 w = src[i];
            xs[nn][4 * i] = w.x; xs[nn][4 * i + 1] = w.y; xs[nn][4 * i + 2] = w.z; xs[nn][4 * i + 3] = w.w;
        }
        mult[nn] = at_mult[q] * tdown;
    }
#pragma unroll
    for (int q0 = 0; q0 < kNvDnLoads; q0 += kPerRed) {
        float v[V];
#pragma unroll
        for (int k = 0; k < kPerRed; ++k) {
            const uint16_t s = R.s[q0 + k];
            const float s0 = e4m3_to_f32(s & 0xffu), s1 = e4m3_to_f32(s >> 8);
#pragma unroll
            for (int nn = 0; nn < NT; ++nn) v[k * NT + nn] = dot32_nv(R.c[q0 + k], xs[nn], s0, s1) * mult[nn];
        }
        const float red = transpose_reduce<V, 16>(v);
        const int vi = j >> (4 - kLogV);
        const int k = vi / NT, nn = vi % NT;
        if ((j & ((1 << (4 - kLogV)) - 1)) == 0 && nn < n_valid)
            o[(size_t)(p0 + nn) * kH + n0 + 4 * (q0 + k) + rsub] = red;
    }
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void k_down_nv(
    const uint8_t *__restrict__ codes, const uint8_t *__restrict__ scales, const float *__restrict__ tscales,
    const float *__restrict__ act, const int *__restrict__ slots, float *__restrict__ o) {
    constexpr int kRows = 4 * kNvDnLoads;
    constexpr int kItems = kH / kRows;
    static_assert(kItems % 4 == 0, "the four waves of a workgroup must share one expert");
    __shared__ uint32_t at[4][kI / 2];
    __shared__ float at_mult[4];
    const int wave = wave_id();
    const int lane = threadIdx.x & 63;
    const int item = blockIdx.x * 4 + wave;
    const int *rec = slots + 8 * (item / kItems);   // {expert, p_begin, n, ...}
    const int e = rec[0];
    if (e < 0) return;
    const int p_begin = rec[1], n = rec[2];
    const int n0 = (item % kItems) * kRows;
    const int j = lane & 15, rsub = lane >> 4;
    const rsrc_t cd = make_buf(codes + (size_t)e * kCodeBytesPerExpert + kCodeBytesGu,
                               (uint32_t)(kCodeBytesPerExpert - kCodeBytesGu));
    const rsrc_t sd = make_buf(scales + (size_t)e * kNvScalePerExpert + kNvScaleGu, kNvScalePerExpert - kNvScaleGu);
    const uint32_t cv = rsub * (kI / 2) + j * 16, sv = rsub * (kI / kNvBlock) + j * 2;
    const float tdown = tscales[3 * e + 2];
    // a of the assignment p (wave w: p = c + w), requested before the codes so
    // that staging waits only for it; lane l holds a[8l .. 8l + 8)
    float4 a0, a1;
    auto load_a = [&](int p) {
        const rsrc_t ab = make_buf(act + (size_t)p * kI, kI * 4);
        a0 = __builtin_bit_cast(float4, bload16(ab, lane * 32, 0));
        a1 = __builtin_bit_cast(float4, bload16(ab, lane * 32 + 16, 0));
    };
    auto stage = [&]() {
        const float v[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
        const int sh = prescale_shift(wave_max(amax));
        uint4 w;
        w.x = pack_half2(ldexpf(v[0], -sh), ldexpf(v[1], -sh));
        w.y = pack_half2(ldexpf(v[2], -sh), ldexpf(v[3], -sh));
        w.z = pack_half2(ldexpf(v[4], -sh), ldexpf(v[5], -sh));
        w.w = pack_half2(ldexpf(v[6], -sh), ldexpf(v[7], -sh));
        reinterpret_cast<uint4 *>(at[wave])[lane] = w;
        at_mult[wave] = ldexpf(1.0f, sh);   // every lane stores the same value
    };
    NvDnRows R;
    if (n == 1) {   // the common decode case
        if (wave == 0) load_a(p_begin);
        nv_dn_load<false>(R, cd, sd, cv, sv, n0);
        if (wave == 0) stage();
        __syncthreads();
        nv_dn_compute<1>(R, n0, at[0], at_mult, tdown, p_begin, 1, lane, o);
        return;
    }
    // two or more tokens: four assignments per round of operands, two at a
    // time through one call site; volatile reloads (L2 hits) keep the rows
    // loop-variant
    const int p_end = p_begin + n;
    for (int c = p_begin; c < p_end; c += 4) {
        const bool mine = c + wave < p_end;
        if (mine) load_a(c + wave);
        nv_dn_load<true>(R, cd, sd, cv, sv, n0);
        if (c != p_begin) __syncthreads();   // every wave is done with the last round's operands
        if (mine) stage();
        __syncthreads();
        const int m = min(4, p_end - c);
        for (int q = 0; q < m; q += 2) {
            if (q) nv_dn_load<true>(R, cd, sd, cv, sv, n0);
            nv_dn_compute<2>(R, n0, at[q], at_mult + q, tdown, c + q, min(2, m - q), lane, o);
        }
    }
}

}  // namespace

void launch_gateup_nvfp4(const uint8_t *codes, const uint8_t *scales, const float *tscales, const uint16_t *x,
                         const int *perm, const int *slots, int T, float *act, hipStream_t s) {
    const int max_active = min(kE, kTopK * T);
    const int waves = max_active * (kI / kNvGuPairs);
    hipLaunchKernelGGL(k_gateup_nv, dim3((waves + 3) / 4), dim3(256), 0, s, codes, scales, tscales, x, perm, slots,
                       act);
}

void launch_down_nvfp4(const uint8_t *codes, const uint8_t *scales, const float *tscales, const float *act,
                       const int *slots, int T, float *o, hipStream_t s) {
    const int max_active = min(kE, kTopK * T);
    const int waves = max_active * (kH / (4 * kNvDnLoads));
    hipLaunchKernelGGL(k_down_nv, dim3((waves + 3) / 4), dim3(256), 0, s, codes, scales, tscales, act, slots, o);
}

}  // namespace moe_w4
