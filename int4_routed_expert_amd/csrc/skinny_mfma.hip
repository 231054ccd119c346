// bf16 x bf16 products with few rows on the MFMA units: the router logits
// and the shared expert.
//
//   router:        logits[t][e] = x_t . R_e (+ bias_e)          (256 columns)
//   shared gate/up h[t][r]      = silu(x_t . Wg_r) * (x_t . Wu_r)  (1024 x 2 columns)
//   shared down    z[t][n]      = h_t . Wd_n                       (2048 columns)
//
// Router rows are bf16 widened exactly to fp32 with fp32 sums (NInfer README
// of Flint, "What is inside"); the shared expert is an ungated bf16 SwiGLU of
// width 1024 on the unrotated x (Flint model card, Aijuus/flint-w4exp,
// introduction and table row "weights").  bf16 products are exact and the
// MFMA sums in fp32.  h is rounded to bf16 once, as the operand of the down
// projection.
//
// Why MFMA here: with T tokens the shared expert does 2T flops per weight
// byte.  At T = 32 that is 64 flop/B, above what the VALU sustains at HBM
// speed, so the product is a real (skinny) contraction; at T = 1 the MFMA
// simply runs mostly empty while the weights stream.
//
// Tiling: a workgroup owns 16 output columns (for SwiGLU: 8 gate rows and the
// same 8 up rows) and all tokens; its KS waves split K, each accumulating
// 16x16 tiles of v_mfma_f32_16x16x32_bf16, and reduce through LDS.  Lane
// (r = l % 16, g = l / 16) loads 32 consecutive K of weight row r and of
// token row r, so every lane load is 64 contiguous bytes and the K order
// inside an MFMA is the same for both operands.
#include "common.h"
#include "launch.h"

namespace moe_w4 {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

enum { kEpiStoreF32 = 0, kEpiSwiglu = 1 };

__device__ __forceinline__ f32x4_t mfma16(uint4 a, uint4 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                   0, 0, 0);
}

// MT: 16-row token tiles held at once (tokens are walked in chunks of 16*MT).
// KS: waves per workgroup, splitting K.
template <int MT, int KS, int EPI>
__global__ __launch_bounds__(64 * KS) void k_skinny(const uint16_t *__restrict__ A, int M, int K,
                                                    const uint16_t *__restrict__ B, int b_rows, int b_split,
                                                    const float *__restrict__ bias, void *__restrict__ out,
                                                    int ldo) {
    __shared__ f32x4_t red[KS][MT][64];
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int r = lane & 15, g = lane >> 4;
    const int c0 = blockIdx.x * 16;   // first output column of the workgroup
    // weight row of this lane's column
    int brow;
    if (EPI == kEpiSwiglu) brow = (r < 8) ? (c0 / 2 + r) : (b_split + c0 / 2 + r - 8);
    else brow = c0 + r;
    const int kw = K / KS;
    const int k_begin = wave * kw;
    // one wave-uniform descriptor over the weight matrix; the row is in the lane offset
    const __amdgpu_buffer_rsrc_t bres = make_buf(B, (uint32_t)(b_rows * K * 2));
    const uint32_t brow_off = (uint32_t)brow * K * 2;

    for (int m0 = 0; m0 < M; m0 += 16 * MT) {
        f32x4_t acc[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        for (int k0 = k_begin; k0 < k_begin + kw; k0 += 128) {
            uint4 b[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) b[s] = bload16_nt(bres, brow_off + (uint32_t)(k0 + 32 * g + 8 * s) * 2, 0);
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                const int m = min(m0 + 16 * t + r, M - 1);
                const uint4 *ap = reinterpret_cast<const uint4 *>(A + (size_t)m * K + k0 + 32 * g);
                uint4 a[4];
#pragma unroll
                for (int s = 0; s < 4; ++s) a[s] = ap[s];
#pragma unroll
                for (int s = 0; s < 4; ++s) acc[t] = mfma16(a[s], b[s], acc[t]);
            }
        }
        // The accumulators are read right after the last MFMA of the loop; give
        // the MFMA pipeline its wait states explicitly (the hazard is not always
        // covered at the loop exit).
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" ::: "memory");
#pragma unroll
        for (int t = 0; t < MT; ++t) red[wave][t][lane] = acc[t];
        __syncthreads();
        // wave t (< MT) finishes token tile t
        for (int t = wave; t < MT; t += KS) {
            f32x4_t s = red[0][t][lane];
#pragma unroll
            for (int w = 1; w < KS; ++w) s += red[w][t][lane];
            // lane holds rows m0 + 16t + 4g + i of column c0 + r
            if (EPI == kEpiStoreF32) {
                const float bcol = bias ? bias[c0 + r] : 0.0f;
                float *o = static_cast<float *>(out);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int m = m0 + 16 * t + 4 * g + i;
                    if (m < M) o[(size_t)m * ldo + c0 + r] = s[i] + bcol;
                }
            } else {
                uint16_t *o = static_cast<uint16_t *>(out);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float up = __shfl_xor(s[i], 8, kWave);   // column r+8 holds the up row
                    const int m = m0 + 16 * t + 4 * g + i;
                    if (r < 8 && m < M) {
                        const float gv = s[i];
                        o[(size_t)m * ldo + c0 / 2 + r] = f32_to_bf16(gv / (1.0f + expf(-gv)) * up);
                    }
                }
            }
        }
        __syncthreads();
    }
}

template <int KS, int EPI>
static void launch_skinny(const uint16_t *A, int M, int K, const uint16_t *B, int n_cols, int b_split,
                          const float *bias, void *out, int ldo, hipStream_t s) {
    dim3 grid(n_cols / 16), block(64 * KS);
    const int b_rows = n_cols;   // weight rows the columns read
    if (M <= 16)
        hipLaunchKernelGGL((k_skinny<1, KS, EPI>), grid, block, 0, s, A, M, K, B, b_rows, b_split, bias, out, ldo);
    else if (M <= 32)
        hipLaunchKernelGGL((k_skinny<2, KS, EPI>), grid, block, 0, s, A, M, K, B, b_rows, b_split, bias, out, ldo);
    else
        hipLaunchKernelGGL((k_skinny<4, KS, EPI>), grid, block, 0, s, A, M, K, B, b_rows, b_split, bias, out, ldo);
}

void launch_router_logits(const uint16_t *x, const uint16_t *router_w, const float *bias, int T,
                          float *logits, hipStream_t s) {
    launch_skinny<8, kEpiStoreF32>(x, T, kH, router_w, kE, 0, bias, logits, kE, s);
}

void launch_shared_gateup(const uint16_t *w, const uint16_t *x, int T, uint16_t *hs, hipStream_t s) {
    // columns: 16-wide tiles of (8 gate rows, the same 8 up rows); up rows start at row 1024
    launch_skinny<8, kEpiSwiglu>(x, T, kH, w, 2 * kIS, kIS, nullptr, hs, kIS, s);
}

void launch_shared_down(const uint16_t *w, const uint16_t *hs, int T, float *z, hipStream_t s) {
    launch_skinny<8, kEpiStoreF32>(hs, T, kIS, w + 2 * kSharedGateElems, kH, 0, nullptr, z, kH, s);
}

}  // namespace moe_w4
