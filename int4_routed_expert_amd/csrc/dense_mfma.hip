// bf16 x bf16 products with many rows (prefill sizes) on the MFMA units:
// the router logits and the shared expert, the same contractions as the
// few-row kernels of skinny_mfma.hip (router rows bf16 widened exactly with
// fp32 sums, NInfer README of Flint, "What is inside"; ungated bf16 SwiGLU
// shared expert of width 1024, Flint model card, Aijuus/flint-w4exp,
// introduction and table row "weights").  bf16 products are exact and
// v_mfma_f32_32x32x16_bf16 sums them in fp32.
//
// Tiling: a workgroup computes a 128 x 128 output tile with 4 waves (2 x 2,
// 64 x 64 each: 2 x 2 MFMA tiles).  K advances 64 at a time: operands are
// loaded into registers kPrefetch steps ahead and written to a double-buffered
// LDS tile one step ahead; rows of 64 bf16 (128 bytes) are stored with the
// 16-byte group position swizzled by bits 1..3 of the row, so the MFMA reads
// of 16 consecutive rows hit 16 distinct 4-bank slots.
//
// Epilogues: fp32 store (+ per-column bias) for the logits and the shared
// down projection z; SwiGLU for the shared gate/up, whose 128-column tile is
// 64 gate rows and the same 64 up rows (each wave's two 32-column MFMA tiles
// are a gate tile and its up tile, so silu(g) * u pairs registers of one
// lane).  The layer's combine follows as its own pass (k_combine).
#include "common.h"
#include "launch.h"

namespace moe_w4 {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kTile = 128;
constexpr int kStepK = 64;                       // bf16 per row per LDS slot (128 bytes, 8 groups)
constexpr int kRowBytes = kStepK * 2;
constexpr int kChunksPerRow = kRowBytes / 16;
constexpr int kSlotBytes = kTile * kRowBytes;    // 16 KB per operand per slot
constexpr int kStageLoads = kTile * kChunksPerRow / 256;   // 16-byte loads per thread per operand per step
constexpr int kPrefetch = 2;                     // steps whose operands are in flight in registers
constexpr int kXcds = 8;

enum { kEpiStore = 0, kEpiSwiglu = 1, kEpiStoreBf16 = 2 };

struct DenseJob {
    const uint16_t *B;   // weight rows, K contiguous
    int n_tiles;         // 128-column tiles of the job
    int epi;
    int up_row;          // SwiGLU: first up row (gate rows start at 0)
    const float *bias;   // kEpiStore: per column, or null
    void *out;           // f32 (store) or bf16 (SwiGLU, bf16 store) [M][ldo]
    int ldo;
};
struct DenseJobs {
    DenseJob job[2];
    int *clear;    // n_clear ints zeroed by the first workgroups (256 each), or null
    int n_clear;
    // RT (router folded into the shared gate/up tiles): tile nt of job 0 also
    // computes router columns [kRtCols nt, kRtCols nt + kRtCols) of its rows
    const uint16_t *router_w;
    const float *router_bias;   // per column, or null
    float *logits;              // [M][256] fp32
};
constexpr int kRtCols = 16;   // router columns per shared tile (16 tiles x 16 = 256)

__device__ __forceinline__ f32x16_t mfma_bf16(uint4 a, uint4 b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                   0, 0, 0);
}

__device__ __forceinline__ void mfma_drain() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" ::: "memory");
}

}  // namespace

// A: [M][K] bf16 rows.  Work item: (m tile, job n tile).
// RT: the router's 256 columns ride along the 16 shared gate/up tiles, 16 per
// tile (B gets 16 more rows in LDS; wave (wm, wn) multiplies the 32 A rows
// 64 wm + 32 wn .. of its own operands by them, the 16 columns padded to the
// MFMA's 32 by repeating them).  A launch of 256 tiles then fills the 256 CUs
// once; the router as tiles of its own made 288, and the 32 CUs that ran two
// set the launch's time (42 -> 31 us at T = 2048 without the router tiles).
template <int K, bool RT>
__global__ __launch_bounds__(256) void k_dense_mfma(const uint16_t *__restrict__ A, int M, int m_tiles,
                                                    DenseJobs jobs) {
    constexpr int kSteps = K / kStepK;
    static_assert(kSteps >= 3, "pipeline prologue");
    constexpr int kSlotBytesB = kSlotBytes + (RT ? kRtCols * kRowBytes : 0);
    __shared__ __attribute__((aligned(16))) uint8_t sa[2][kSlotBytes], sb[2][kSlotBytesB];
    if (jobs.clear) {
        const int i = (int)blockIdx.x * 256 + (int)threadIdx.x;
        if (i < jobs.n_clear) jobs.clear[i] = 0;
    }

    // work item: XCD-aware when there are enough m tiles (each XCD keeps a
    // few m tiles' A rows in its L2 and walks all n tiles), else linear
    const int n_total = jobs.job[0].n_tiles + jobs.job[1].n_tiles;
    int mt, nt;
    if (m_tiles >= kXcds) {
        const int b = blockIdx.x, xcd = b % kXcds, k = b / kXcds;
        mt = xcd + kXcds * (k / n_total);
        nt = k % n_total;
    } else {
        mt = blockIdx.x / n_total;
        nt = blockIdx.x % n_total;
    }
    if (mt >= m_tiles) return;
    // both jobs' fields are read in parallel and then selected (indexing the
    // kernel argument by the job number would chain dependent scalar loads)
    const DenseJob j0 = jobs.job[0], j1 = jobs.job[1];
    const bool second = nt >= j0.n_tiles;
    DenseJob J;
    J.B = second ? j1.B : j0.B;
    J.n_tiles = second ? j1.n_tiles : j0.n_tiles;
    J.epi = second ? j1.epi : j0.epi;
    J.up_row = second ? j1.up_row : j0.up_row;
    J.bias = second ? j1.bias : j0.bias;
    J.out = second ? j1.out : j0.out;
    J.ldo = second ? j1.ldo : j0.ldo;
    if (second) nt -= j0.n_tiles;

    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
    const int n = lane & 31, g = lane >> 5;
    const int wm = wave >> 1, wn = wave & 1;
    const int m0 = mt * kTile;

    // B rows of this tile: tile column c (0..127) -> weight row.  SwiGLU:
    // wave column half wn covers tile columns [64wn, 64wn+64): 32 gate rows
    // then the same 32 up rows
    auto b_row = [&](int c) -> int {
        if (J.epi != kEpiSwiglu) return nt * kTile + c;
        const int half = c >> 6, cc = c & 63;
        const int r = nt * 64 + 32 * half + (cc & 31);
        return (cc < 32) ? r : J.up_row + r;
    };

    // staging: per step each thread moves 16-byte chunks c = tid + 256 i of A
    // and of B (row c / 8, position c % 8 holding group (c % 8) ^ ((row >> 1) & 7));
    // raw buffer loads keep their program order, two steps ahead.  The A
    // descriptor starts at the tile's first row, so its 32-bit offsets stay
    // below 128 rows (1.5 MiB at K = 6144) whatever M is; B offsets are below
    // the weight matrix's size (at most 6144 rows of K = 6144)
    const __amdgpu_buffer_rsrc_t ares = make_buf(A + (size_t)m0 * K, 0xffffffffu);
    const __amdgpu_buffer_rsrc_t bres = make_buf(J.B, 0xffffffffu);
    uint32_t aoff[kStageLoads], boff[kStageLoads];
    int ldst[kStageLoads];
    // RT: threads 0..127 also move the 16 router rows' chunk tid (row kTile + tid / 8)
    const bool rt_stager = RT && tid < kRtCols * kChunksPerRow;
    const __amdgpu_buffer_rsrc_t rres = make_buf(RT ? jobs.router_w : J.B, 0xffffffffu);
    uint32_t rt_off = 0;
    int rt_ldst = 0;
    if (rt_stager) {
        const int r = kTile + tid / kChunksPerRow, pos = tid % kChunksPerRow;
        const int grp = pos ^ ((r >> 1) & 7);
        rt_off = (uint32_t)(nt * kRtCols + tid / kChunksPerRow) * (K * 2) + grp * 16;
        rt_ldst = r * kRowBytes + pos * 16;
    }
#pragma unroll
    for (int i = 0; i < kStageLoads; ++i) {
        const int c = tid + 256 * i, r = c / kChunksPerRow, pos = c % kChunksPerRow;
        const int grp = pos ^ ((r >> 1) & 7);
        aoff[i] = (uint32_t)(min(m0 + r, M - 1) - m0) * (K * 2) + grp * 16;
        boff[i] = (uint32_t)b_row(r) * (K * 2) + grp * 16;
        ldst[i] = r * kRowBytes + pos * 16;
    }
    uint4 stg[kPrefetch][2 * kStageLoads + (RT ? 1 : 0)];
    auto load = [&](int set, int step) {
#pragma unroll
        for (int i = 0; i < kStageLoads; ++i) {
            stg[set][i] = bload16(ares, aoff[i] + step * kRowBytes, 0);
            stg[set][kStageLoads + i] = bload16(bres, boff[i] + step * kRowBytes, 0);
        }
        if constexpr (RT) {
            if (rt_stager) stg[set][2 * kStageLoads] = bload16(rres, rt_off + step * kRowBytes, 0);
        }
    };
    auto store = [&](int set, int slot) {
#pragma unroll
        for (int i = 0; i < kStageLoads; ++i) {
            *reinterpret_cast<uint4 *>(sa[slot] + ldst[i]) = stg[set][i];
            *reinterpret_cast<uint4 *>(sb[slot] + ldst[i]) = stg[set][kStageLoads + i];
        }
        if constexpr (RT) {
            if (rt_stager) *reinterpret_cast<uint4 *>(sb[slot] + rt_ldst) = stg[set][2 * kStageLoads];
        }
    };

    f32x16_t acc[2][2], acc_r;
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[x][y][i] = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc_r[i] = 0.0f;

    // step k's operands live in register set k % 2 until stored to LDS slot
    // k % 2: step 0 is stored before the loop, step s + 1 during step s
#pragma unroll
    for (int d = 0; d < kPrefetch; ++d) load(d, d);
    store(0, 0);
    load(0, 2);
    __syncthreads();

    // fully unrolled up to K = 2048; longer K in pairs of steps (a full unroll
    // of 96 steps holds enough addresses live to fall to one wave per SIMD)
    constexpr int kUnroll = kSteps <= 32 ? kSteps : 2;
#pragma unroll kUnroll
    for (int s = 0; s < kSteps; ++s) {
        const int slot = s & 1;
        // every operand of the step is requested from LDS first, so the MFMAs
        // below wait for the LDS latency once per step, not once per k-slice
        uint4 a[kChunksPerRow / 2][2], b[kChunksPerRow / 2][2], br[kChunksPerRow / 2];
#pragma unroll
        for (int j = 0; j < kChunksPerRow / 2; ++j) {
            const int grp = (kChunksPerRow / 2) * g + j;
            if constexpr (RT) {   // router row n % 16 (lanes n and n + 16 alike)
                const int r = kTile + (n & (kRtCols - 1));
                br[j] = *reinterpret_cast<const uint4 *>(sb[slot] + r * kRowBytes + ((grp ^ ((r >> 1) & 7)) * 16));
            }
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                const int r = 64 * wm + 32 * x + n;
                a[j][x] = *reinterpret_cast<const uint4 *>(sa[slot] + r * kRowBytes + ((grp ^ ((r >> 1) & 7)) * 16));
            }
#pragma unroll
            for (int y = 0; y < 2; ++y) {
                const int r = 64 * wn + 32 * y + n;
                b[j][y] = *reinterpret_cast<const uint4 *>(sb[slot] + r * kRowBytes + ((grp ^ ((r >> 1) & 7)) * 16));
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        // step s + 1 (loaded two steps ago) into the other slot, whose readers
        // all passed the previous barrier; its registers then take step s + 3
        if (s + 1 < kSteps) store((s + 1) % kPrefetch, slot ^ 1);
        if (s + 3 < kSteps) load((s + 1) % kPrefetch, s + 3);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < kChunksPerRow / 2; ++j) {
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int y = 0; y < 2; ++y) acc[x][y] = mfma_bf16(a[j][x], b[j][y], acc[x][y]);
            if constexpr (RT) {
                // the wave's rows 32 wn .. of its 64: a component-wise select
                // (an index by wn would move the operands to scratch)
                const uint4 lo = a[j][0], hi = a[j][1];
                const uint4 ar = make_uint4(wn ? hi.x : lo.x, wn ? hi.y : lo.y, wn ? hi.z : lo.z, wn ? hi.w : lo.w);
                acc_r = mfma_bf16(ar, br[j], acc_r);
            }
        }
        __syncthreads();
    }
    mfma_drain();

    // epilogue: lane holds rows 64wm + 32x + 8(i/4) + 4g + (i%4), column 64wn + 32y + n
    if constexpr (RT) {
        // router columns: rows 64wm + 32wn + 8(i/4) + 4g + (i%4), column n < 16
        if (n < kRtCols) {
            const int c = nt * kRtCols + n;
            const float bc = jobs.router_bias ? jobs.router_bias[c] : 0.0f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int m = m0 + 64 * wm + 32 * wn + 8 * (i >> 2) + 4 * g + (i & 3);
                if (m < M) jobs.logits[(size_t)m * kE + c] = acc_r[i] + bc;
            }
        }
    }
    float bcol[2] = {0.0f, 0.0f};
    if (J.epi == kEpiStore && J.bias) {
        bcol[0] = J.bias[nt * kTile + 64 * wn + n];
        bcol[1] = J.bias[nt * kTile + 64 * wn + 32 + n];
    }
#pragma unroll
    for (int x = 0; x < 2; ++x) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int m = m0 + 64 * wm + 32 * x + 8 * (i >> 2) + 4 * g + (i & 3);
            if (m >= M) continue;
            if (J.epi == kEpiStore) {
                float *o = static_cast<float *>(J.out);
#pragma unroll
                for (int y = 0; y < 2; ++y) {
                    const int c = nt * kTile + 64 * wn + 32 * y + n;
                    o[(size_t)m * J.ldo + c] = acc[x][y][i] + bcol[y];
                }
            } else if (J.epi == kEpiStoreBf16) {
                uint16_t *o = static_cast<uint16_t *>(J.out);
#pragma unroll
                for (int y = 0; y < 2; ++y) {
                    const int c = nt * kTile + 64 * wn + 32 * y + n;
                    o[(size_t)m * J.ldo + c] = f32_to_bf16(acc[x][y][i]);
                }
            } else {   // kEpiSwiglu
                const float gv = acc[x][0][i], uv = acc[x][1][i];
                const int r = nt * 64 + 32 * wn + n;
                // silu with the hardware exp and reciprocal (relative error ~1e-7)
                static_cast<uint16_t *>(J.out)[(size_t)m * J.ldo + r] =
                    f32_to_bf16(gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * uv);
            }
        }
    }
}

// Compute units of the current device (queried once per process).
static int cu_count() {
    static const int n = [] {
        int dev = 0, v = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
            v = 256;
        return v;
    }();
    return n;
}

static DenseJob no_dense_job() { return DenseJob{nullptr, 0, kEpiStore, 0, nullptr, nullptr, 0}; }

template <int K, bool RT = false>
static void launch_dense(const uint16_t *A, int M, const DenseJobs &jobs, hipStream_t s) {
    const int m_tiles = (M + kTile - 1) / kTile;
    const int n_total = jobs.job[0].n_tiles + jobs.job[1].n_tiles;
    const int grid = (m_tiles >= kXcds) ? kXcds * ((m_tiles + kXcds - 1) / kXcds) * n_total : m_tiles * n_total;
    hipLaunchKernelGGL((k_dense_mfma<K, RT>), dim3(grid), dim3(256), 0, s, A, M, m_tiles, jobs);
}

void launch_router_and_shared_gateup_dense(const uint16_t *x, int T, const uint16_t *router_w, const float *bias,
                                           float *logits, const uint16_t *shared_w, uint16_t *hs, hipStream_t s,
                                           int *clear, int n_clear) {
    DenseJobs jobs = {};
    jobs.clear = clear;
    jobs.n_clear = n_clear;
    // the shared gate/up in 16 tiles of 64 gate + 64 up rows per 128 tokens;
    // the router either as 2 tiles of its own per 128 tokens, or folded into
    // the shared tiles (16 columns each) when its own tiles would take the
    // launch past one round of the CUs and the folded ones fit in it (15-16
    // token tiles, 1793-2048 tokens on 256 CUs); elsewhere the fold only
    // lengthens every tile
    static_assert((kIS / 64) * kRtCols == kE, "the router's columns spread over the shared tiles");
    const int m_tiles = (T + kTile - 1) / kTile, cus = cu_count();
    const bool fold = m_tiles * (kIS / 64) <= cus && m_tiles * (kIS / 64 + kE / kTile) > cus;
    jobs.job[0] = DenseJob{shared_w, kIS / 64, kEpiSwiglu, kIS, nullptr, hs, kIS};
    if (fold) {
        jobs.job[1] = no_dense_job();
        jobs.router_w = router_w;
        jobs.router_bias = bias;
        jobs.logits = logits;
        launch_dense<kH, true>(x, T, jobs, s);
    } else {
        jobs.job[1] = DenseJob{router_w, kE / kTile, kEpiStore, 0, bias, logits, kE};
        launch_dense<kH>(x, T, jobs, s);
    }
}

void launch_shared_down_dense(const uint16_t *shared_w, const uint16_t *hs, int T, float *z, hipStream_t s) {
    DenseJobs jobs = {};
    jobs.job[0] = DenseJob{shared_w + 2 * kSharedGateElems, kH / kTile, kEpiStore, 0, nullptr, z, kH};
    jobs.job[1] = no_dense_job();
    launch_dense<kIS>(hs, T, jobs, s);
}

// Dense SwiGLU MLP block (NInfer README of Flint, "What is inside": blocks 0
// and 1 are dense SwiGLU MLPs of width 6144; the model card keeps every
// linear bf16): h = bf16(silu(x Wg^T) * (x Wu^T)), then y = bf16(h Wd^T).
void launch_dense_mlp_gateup_dense(const uint16_t *x, int T, const uint16_t *w, uint16_t *h, hipStream_t s) {
    DenseJobs jobs = {};
    jobs.job[0] = DenseJob{w, kDenseInter / 64, kEpiSwiglu, kDenseInter, nullptr, h, kDenseInter};
    jobs.job[1] = no_dense_job();
    launch_dense<kH>(x, T, jobs, s);
}

void launch_dense_mlp_down_dense(const uint16_t *w, const uint16_t *h, int T, uint16_t *y, hipStream_t s) {
    DenseJobs jobs = {};
    jobs.job[0] = DenseJob{w + 2 * (size_t)kDenseInter * kH, kH / kTile, kEpiStoreBf16, 0, nullptr, y, kH};
    jobs.job[1] = no_dense_job();
    launch_dense<kDenseInter>(h, T, jobs, s);
}

// y[t] = bf16(z[t] + sum_j w[t][j] o[pos[6t + j]]), slots in order, with o the
// grouped down kernel's rows: fp16 times a per-row multiplier (HALF) or fp32
// (the NVFP4 experts' rows): a wave per token, lane l owns columns [32l,
// 32l + 32); every load of the token is in flight at once (the gathers of an
// epilogue inside the GEMM tile were latency-bound).
template <bool HALF>
__global__ __launch_bounds__(256) void k_combine(const float *__restrict__ z, const float *__restrict__ topk_w,
                                                 const int *__restrict__ pos, const void *__restrict__ o,
                                                 const float *__restrict__ o_scale, int T, uint16_t *__restrict__ y) {
    const int t = blockIdx.x * 4 + wave_id();
    if (t >= T) return;
    const int lane = threadIdx.x & 63;
    float w[kTopK];
    int p[kTopK];
#pragma unroll
    for (int j = 0; j < kTopK; ++j) {
        w[j] = __builtin_bit_cast(float, uniform(__builtin_bit_cast(int, topk_w[(size_t)t * kTopK + j])));
        p[j] = uniform(pos[(size_t)t * kTopK + j]);
    }
    const float4 *zr = reinterpret_cast<const float4 *>(z + (size_t)t * kH) + 8 * lane;
    float4 acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = zr[i];
    if (HALF) {
        float ws[kTopK];
        uint4 h[kTopK][4];
#pragma unroll
        for (int j = 0; j < kTopK; ++j) {
            ws[j] = w[j] * __builtin_bit_cast(float, uniform(__builtin_bit_cast(int, o_scale[p[j]])));
            const uint4 *orow = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(o) + (size_t)p[j] * kH) +
                                4 * lane;
#pragma unroll
            for (int i = 0; i < 4; ++i) h[j][i] = orow[i];
        }
#pragma unroll
        for (int j = 0; j < kTopK; ++j) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t q[4] = {h[j][i].x, h[j][i].y, h[j][i].z, h[j][i].w};
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    float4 &a = acc[2 * i + k];
                    a.x = fmaf(ws[j], half_lo(q[2 * k]), a.x);
                    a.y = fmaf(ws[j], half_hi(q[2 * k]), a.y);
                    a.z = fmaf(ws[j], half_lo(q[2 * k + 1]), a.z);
                    a.w = fmaf(ws[j], half_hi(q[2 * k + 1]), a.w);
                }
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < kTopK; ++j) {
            const float4 *orow = reinterpret_cast<const float4 *>(static_cast<const float *>(o) + (size_t)p[j] * kH) +
                                 8 * lane;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float4 v = orow[i];
                acc[i].x = fmaf(w[j], v.x, acc[i].x);
                acc[i].y = fmaf(w[j], v.y, acc[i].y);
                acc[i].z = fmaf(w[j], v.z, acc[i].z);
                acc[i].w = fmaf(w[j], v.w, acc[i].w);
            }
        }
    }
    uint32_t packed[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        packed[2 * i] = (uint32_t)f32_to_bf16(acc[i].x) | ((uint32_t)f32_to_bf16(acc[i].y) << 16);
        packed[2 * i + 1] = (uint32_t)f32_to_bf16(acc[i].z) | ((uint32_t)f32_to_bf16(acc[i].w) << 16);
    }
    uint4 *yr = reinterpret_cast<uint4 *>(y + (size_t)t * kH) + 4 * lane;
#pragma unroll
    for (int i = 0; i < 4; ++i) yr[i] = make_uint4(packed[4 * i], packed[4 * i + 1], packed[4 * i + 2], packed[4 * i + 3]);
}

void launch_combine(const float *z, const float *topk_w, const int *pos, const float *o, int T, uint16_t *y,
                    hipStream_t s) {
    hipLaunchKernelGGL(k_combine<false>, dim3((T + 3) / 4), dim3(256), 0, s, z, topk_w, pos,
                       static_cast<const void *>(o), nullptr, T, y);
}

void launch_combine_half(const float *z, const float *topk_w, const int *pos, const uint16_t *o,
                         const float *o_scale, int T, uint16_t *y, hipStream_t s) {
    hipLaunchKernelGGL(k_combine<true>, dim3((T + 3) / 4), dim3(256), 0, s, z, topk_w, pos,
                       static_cast<const void *>(o), o_scale, T, y);
}

}  // namespace moe_w4
