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
// Tiling: a workgroup owns CW output columns (for SwiGLU: CW/2 gate rows and
// the same CW/2 up rows) and all tokens; its KS waves split K, each accumulating
// 16x16 tiles of v_mfma_f32_16x16x32_bf16, and reduce through LDS.  MFMA s of
// a 128-wide K block takes K [32s, 32s + 32) of the block, lane (r = l % 16,
// g = l / 16) holding K [32s + 8g, 32s + 8g + 8) of weight row r % CW and of
// token row r: the four lanes of a row read 64 contiguous bytes in one load
// (whole half lines, not 16-byte pieces spread over two lines), and the K
// order inside an MFMA is the same for both operands.
#include "common.h"
#include "launch.h"
#include "token_ops.h"

namespace moe_w4 {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

enum { kEpiStoreF32 = 0, kEpiSwiglu = 1, kEpiCombine = 2, kEpiStoreBf16 = 3 };

// One job of a launch: a weight matrix, its output and its epilogue.  A launch
// runs up to two jobs side by side (workgroups [0, n_blocks0) do job 0, the
// rest job 1), so independent products share one launch and overlap.
struct SkinnyJob {
    const uint16_t *B;      // weight rows, K contiguous
    int b_rows;             // rows of B the job reads
    int b_split;            // SwiGLU: first up row (gate rows start at 0)
    int n_blocks;           // workgroups of the job (CW output columns each)
    int epi;                // kEpi*
    const float *bias;      // kEpiStoreF32: added per column, or null
    void *out;              // f32 [M][ldo] (store, combine: bf16), bf16 [M][ldo] (SwiGLU)
    int ldo;
    // kEpiCombine: y = bf16(acc + sum_j w[t][j] * o[pos[6t+j]][col])
    const float *topk_w;
    const int *pos;
    const float *o;
};

struct SkinnyJobs {
    SkinnyJob job[2];
    // optional third role, workgroups past the two jobs: the Hadamard-rotated
    // fp16 copy of x (rotate_x_wave), one wave per token
    const uint16_t *rot_x;
    int rot_tokens;
    uint32_t *xt;
    float *xt_scale;
    // completion counter replicas cleared by workgroup 0 for the next launch
    // (kFusedCounters of them, kFusedCounterStride apart), or null
    int *clear_counters;
};

__device__ __forceinline__ f32x4_t mfma16(uint4 a, uint4 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                   0, 0, 0);
}

// MT: 16-row token tiles held at once (tokens are walked in chunks of 16*MT).
// KS: waves per workgroup, splitting K; KB: 128-wide K blocks per wave
// (K = 128 * KS * KB).  CW: output columns per workgroup, 16 or 8.  With 8,
// lanes r and r + 8 read the same weight row, which doubles the workgroups of
// a small matrix (the 1024-row shared down projection would otherwise leave
// half the CUs idle); the MFMA units have ample room for the duplicate columns.
template <int MT, int KS, int KB, int CW>
__global__ __launch_bounds__(64 * KS) void k_skinny(const uint16_t *__restrict__ A, int M, SkinnyJobs jobs) {
    constexpr int K = 128 * KS * KB;
    // Activations through LDS (KB <= 2): each wave stages its own K slice of
    // the token tiles with whole-line direct loads (one wave instruction reads
    // 1 KiB: 4 / KB rows x KB * 256 contiguous bytes) and reads the MFMA
    // operands back from LDS.  Loading them straight into the operand layout
    // (16 rows x 64 bytes per instruction) runs ~3.5x slower per CU, and every
    // workgroup reads all of x.  Slot P of row R holds 16-byte chunk
    // P ^ (R & 15) of the row's slice, so the 16 rows of an operand read hit
    // 16 different 4-bank groups.  The reduction buffer reuses the wave's own
    // staging area.  KB = 6 (the dense block's down projection) would not fit:
    // it loads the operands directly.
    constexpr bool kLds = KB <= 2;
    constexpr int kRowBytes = KB * 256;              // one token's K slice of one wave
    constexpr int kTileBytes = 16 * kRowBytes;
    constexpr int kWaveBytes = kLds ? MT * kTileBytes : MT * 64 * 16;
    static_assert(!kLds || kWaveBytes >= MT * 64 * 16, "the reduction fits the staging area");
    __shared__ __attribute__((aligned(16))) uint8_t xs[KS][kWaveBytes];
    auto red_at = [&](int w, int t) -> f32x4_t * { return reinterpret_cast<f32x4_t *>(xs[w]) + t * 64; };
    if (jobs.clear_counters && blockIdx.x == 0 && threadIdx.x < kFusedCounters)
        jobs.clear_counters[threadIdx.x * kFusedCounterStride] = 0;
    const int bx = (int)blockIdx.x;
    // both jobs' fields are read (in parallel, at fixed kernel-argument
    // offsets) and then selected: indexing the argument by the job number
    // would make every field a dependent scalar load
    const SkinnyJob j0 = jobs.job[0], j1 = jobs.job[1];
    if (bx >= j0.n_blocks + j1.n_blocks) {
        const int lane = threadIdx.x & 63;
        const int t = (bx - j0.n_blocks - j1.n_blocks) * KS + wave_id();
        if (t >= jobs.rot_tokens) return;
        uint4 xq[4];
        const uint4 *xp = reinterpret_cast<const uint4 *>(jobs.rot_x + (size_t)t * kH + lane * 32);
#pragma unroll
        for (int i = 0; i < 4; ++i) xq[i] = xp[i];
        const int sh = rotate_x_wave(xq, lane, jobs.xt + (size_t)t * (kH / 2) + lane * 16);
        if (lane == 0) jobs.xt_scale[t] = ldexpf(1.0f, sh);
        return;
    }
    const bool second = bx >= j0.n_blocks;
    SkinnyJob J;
    J.B = second ? j1.B : j0.B;
    J.b_rows = second ? j1.b_rows : j0.b_rows;
    J.b_split = second ? j1.b_split : j0.b_split;
    J.n_blocks = second ? j1.n_blocks : j0.n_blocks;
    J.epi = second ? j1.epi : j0.epi;
    J.bias = second ? j1.bias : j0.bias;
    J.out = second ? j1.out : j0.out;
    J.ldo = second ? j1.ldo : j0.ldo;
    J.topk_w = second ? j1.topk_w : j0.topk_w;
    J.pos = second ? j1.pos : j0.pos;
    J.o = second ? j1.o : j0.o;
    const int blk = second ? bx - j0.n_blocks : bx;
    const int epi = J.epi;
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int r = lane & 15, g = lane >> 4;
    constexpr int HC = CW / 2;
    const int c = r & (CW - 1);   // column of this lane inside the workgroup's CW
    const int c0 = blk * CW;      // first output column of the workgroup
    // weight row of this lane's column: SwiGLU tiles are (CW/2 gate rows, the same CW/2 up rows)
    const int brow = (epi == kEpiSwiglu) ? ((c < HC) ? (c0 / 2 + c) : (J.b_split + c0 / 2 + c - HC)) : (c0 + c);
    const int k_begin = wave * (K / KS);
    // one wave-uniform descriptor over the weight matrix; the row is in the lane offset
    const __amdgpu_buffer_rsrc_t bres = make_buf(J.B, (uint32_t)(J.b_rows * K * 2));
    const uint32_t brow_off = (uint32_t)brow * K * 2;
    uint4 b[KB][4];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int s = 0; s < 4; ++s)
            b[kb][s] = bload16_nt(bres, brow_off + (uint32_t)(k_begin + 128 * kb + 32 * s + 8 * g) * 2, 0);
    // combine: the weights and expert rows of the first token tiles do not
    // depend on the product and are requested now (wave t finishes tile t)
    float pw[4][kTopK], po[4][kTopK];
    const bool pre = epi == kEpiCombine && wave < MT && r < CW;
    if (pre) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = min(16 * wave + 4 * g + i, M - 1);
#pragma unroll
            for (int j = 0; j < kTopK; ++j) {
                pw[i][j] = J.topk_w[(size_t)m * kTopK + j];
                po[i][j] = J.o[(size_t)J.pos[(size_t)m * kTopK + j] * kH + c0 + c];
            }
        }
    }

    for (int m0 = 0; m0 < M; m0 += 16 * MT) {
        f32x4_t acc[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        if constexpr (kLds) {
            // instruction i of tile t: rows 4i/KB + l / (16 KB) of the tile, slot l % (16 KB)
            constexpr int kCpr = KB * 16, kRpi = 4 / KB, kInstr = 16 / kRpi;
            const int rr = lane / kCpr, slot = lane % kCpr;
#pragma unroll
            for (int t = 0; t < MT; ++t)
#pragma unroll
                for (int i = 0; i < kInstr; ++i) {
                    const int R = kRpi * i + rr;
                    const int m = min(m0 + 16 * t + R, M - 1);
                    const uint16_t *src = A + (size_t)m * K + k_begin + 8 * (slot ^ (R & 15));
                    __builtin_amdgcn_global_load_lds(src, (lds_void_t *)(xs[wave] + t * kTileBytes + i * 1024), 16,
                                                     0, 0);
                }
            __builtin_amdgcn_s_waitcnt(0);   // the staged rows (and the weights) have arrived
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                uint4 a[KB][4];
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        const int cq = 16 * kb + 4 * s + g;   // 16-byte group of the row
                        a[kb][s] = *reinterpret_cast<const uint4 *>(xs[wave] + t * kTileBytes + r * kRowBytes +
                                                                    16 * (cq ^ r));
                    }
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int s = 0; s < 4; ++s) acc[t] = mfma16(a[kb][s], b[kb][s], acc[t]);
            }
        } else {
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                const int m = min(m0 + 16 * t + r, M - 1);
                const uint4 *ap = reinterpret_cast<const uint4 *>(A + (size_t)m * K + k_begin + 8 * g);
                uint4 a[KB][4];
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int s = 0; s < 4; ++s) a[kb][s] = ap[16 * kb + 4 * s];
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int s = 0; s < 4; ++s) acc[t] = mfma16(a[kb][s], b[kb][s], acc[t]);
            }
        }
        // The accumulators are read right after the last MFMA; give the MFMA
        // pipeline its wait states explicitly (the hazard is not always
        // covered by the compiler at a loop exit).
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" ::: "memory");
#pragma unroll
        for (int t = 0; t < MT; ++t) red_at(wave, t)[lane] = acc[t];
        __syncthreads();
        // wave t (< MT) finishes token tile t; lanes with r < CW own the columns
        for (int t = wave; t < MT; t += KS) {
            f32x4_t sum = red_at(0, t)[lane];
#pragma unroll
            for (int w = 1; w < KS; ++w) sum += red_at(w, t)[lane];
            // lane holds rows m0 + 16t + 4g + i of column c0 + c
            if (epi == kEpiStoreBf16) {
                uint16_t *o = static_cast<uint16_t *>(J.out);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int m = m0 + 16 * t + 4 * g + i;
                    if (r < CW && m < M) o[(size_t)m * J.ldo + c0 + c] = f32_to_bf16(sum[i]);
                }
            } else if (epi == kEpiStoreF32) {
                const float bcol = J.bias ? J.bias[c0 + c] : 0.0f;
                float *o = static_cast<float *>(J.out);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int m = m0 + 16 * t + 4 * g + i;
                    if (r < CW && m < M) o[(size_t)m * J.ldo + c0 + c] = sum[i] + bcol;
                }
            } else if (epi == kEpiSwiglu) {
                uint16_t *o = static_cast<uint16_t *>(J.out);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float up = __shfl_xor(sum[i], HC, kWave);   // column c + CW/2 holds the up row
                    const int m = m0 + 16 * t + 4 * g + i;
                    if (r < HC && m < M) {
                        const float gv = sum[i];
                        o[(size_t)m * J.ldo + c0 / 2 + c] = f32_to_bf16(gv / (1.0f + expf(-gv)) * up);
                    }
                }
            } else {   // combine with the routed experts, in slot order
                uint16_t *y = static_cast<uint16_t *>(J.out);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int m = m0 + 16 * t + 4 * g + i;
                    if (r < CW && m < M) {
                        float acc_y = sum[i];
                        if (m0 == 0) {
#pragma unroll
                            for (int j = 0; j < kTopK; ++j) acc_y = fmaf(pw[i][j], po[i][j], acc_y);
                        } else {
#pragma unroll
                            for (int j = 0; j < kTopK; ++j) {
                                const float w = J.topk_w[(size_t)m * kTopK + j];
                                const int p = J.pos[(size_t)m * kTopK + j];
                                acc_y = fmaf(w, J.o[(size_t)p * kH + c0 + c], acc_y);
                            }
                        }
                        y[(size_t)m * J.ldo + c0 + c] = f32_to_bf16(acc_y);
                    }
                }
            }
        }
        __syncthreads();
    }
}

template <int KB, int CW>
static void launch_skinny_k(const uint16_t *A, int M, const SkinnyJobs &jobs, hipStream_t s) {
    constexpr int KS = 8;
    dim3 grid(jobs.job[0].n_blocks + jobs.job[1].n_blocks + (jobs.rot_tokens + KS - 1) / KS), block(64 * KS);
    if (M <= 16)
        hipLaunchKernelGGL((k_skinny<1, KS, KB, CW>), grid, block, 0, s, A, M, jobs);
    else
        hipLaunchKernelGGL((k_skinny<2, KS, KB, CW>), grid, block, 0, s, A, M, jobs);
}

static SkinnyJob no_job() { return SkinnyJob{nullptr, 0, 0, 0, kEpiStoreF32, nullptr, nullptr, 0, nullptr, nullptr, nullptr}; }

static SkinnyJobs no_jobs() {
    SkinnyJobs jobs;
    jobs.job[0] = jobs.job[1] = no_job();
    jobs.rot_x = nullptr;
    jobs.rot_tokens = 0;
    jobs.xt = nullptr;
    jobs.xt_scale = nullptr;
    jobs.clear_counters = nullptr;
    return jobs;
}

void launch_router_and_shared_gateup(const uint16_t *x, int T, const uint16_t *router_w, const float *bias,
                                     float *logits, const uint16_t *shared_w, uint16_t *hs, uint32_t *xt,
                                     float *xt_scale, int *clear_counters, hipStream_t s) {
    SkinnyJobs jobs = no_jobs();
    jobs.rot_x = x;
    jobs.rot_tokens = xt ? T : 0;
    jobs.xt = xt;
    jobs.xt_scale = xt_scale;
    jobs.clear_counters = clear_counters;
    jobs.job[0] = SkinnyJob{router_w, kE, 0, kE / 16, kEpiStoreF32, bias, logits, kE, nullptr, nullptr, nullptr};
    // columns: 16-wide tiles of (8 gate rows, the same 8 up rows); up rows start at row 1024
    jobs.job[1] = SkinnyJob{shared_w, 2 * kIS, kIS, 2 * kIS / 16, kEpiSwiglu, nullptr, hs, kIS, nullptr, nullptr, nullptr};
    launch_skinny_k<kH / (128 * 8), 16>(x, T, jobs, s);
}

void launch_shared_down_combine(const uint16_t *shared_w, const uint16_t *hs, int T, const float *topk_w,
                                const int *pos, const float *o, uint16_t *y, hipStream_t s) {
    SkinnyJobs jobs = no_jobs();
    jobs.job[0] = SkinnyJob{shared_w + 2 * kSharedGateElems, kH, 0, kH / 8, kEpiCombine, nullptr, y, kH, topk_w, pos, o};
    jobs.job[1] = no_job();
    launch_skinny_k<kIS / (128 * 8), 8>(hs, T, jobs, s);
}


// Dense SwiGLU MLP block of width 6144 (NInfer README of Flint, "What is
// inside": blocks 0 and 1; bf16 like every linear of the model card): the
// gate/up job as for the shared expert, 16-column tiles of (8 gate rows, the
// same 8 up rows); the down projection over K = 6144, 8 waves splitting K.
void launch_dense_mlp_gateup_skinny(const uint16_t *x, int T, const uint16_t *w, uint16_t *h, hipStream_t s) {
    SkinnyJobs jobs = no_jobs();
    jobs.job[0] = SkinnyJob{w, 2 * kDenseInter, kDenseInter, 2 * kDenseInter / 16, kEpiSwiglu, nullptr, h, kDenseInter,
                            nullptr, nullptr, nullptr};
    jobs.job[1] = no_job();
    launch_skinny_k<kH / (128 * 8), 16>(x, T, jobs, s);
}

void launch_dense_mlp_down_skinny(const uint16_t *w, const uint16_t *h, int T, uint16_t *y, hipStream_t s) {
    SkinnyJobs jobs = no_jobs();
    jobs.job[0] = SkinnyJob{w + 2 * (size_t)kDenseInter * kH, kH, 0, kH / 8, kEpiStoreBf16, nullptr, y, kH, nullptr,
                            nullptr, nullptr};
    jobs.job[1] = no_job();
    launch_skinny_k<kDenseInter / (128 * 8), 8>(h, T, jobs, s);
}

}  // namespace moe_w4
