// Decode sizes (1..8 tokens): the layer in two launches.
//
// At these sizes every step of the layer moves little data, so the layer is
// bound by the latency of its dependent steps rather than by bandwidth: a
// launch per step (router, top-6, sort, gate/up, rotation of a, down, combine)
// costs a few microseconds each.  The first launch computes the router logits
// (one wave per router row; fp32 sums of exact bf16 products, NInfer README of
// Flint, "What is inside").  In a layer of a stack it also computes x itself
// from the residual stream (rmsnorm), and the second launch adds y to the
// residual stream, so a stack layer is two launches as well.  The second
// launch runs all the rest, with three roles of workgroups:
//
//   gate/up workgroups (the first 256): the routing of all tokens from the
//       logits (wave t: top-6 of token t, model card, introduction: 256
//       experts, top-6; weights sigmoid / max(sum, 2^-14), bloomery issue
//       #632, design thread), then a stable sort of the <= 48 assignments in
//       LDS; x is rotated in LDS (fwht128 per 128-block, model card, table row
//       "weights"; one task per 512-wide quarter of a token, dealt from the
//       last wave down so that it runs beside the top-6 of the first waves; one
//       power-of-two prescale per block), then wave batches of 2 (gate, up) row
//       pairs of an active expert for all of its tokens, a = silu(g) * u in
//       fp32 (sorted-position order), the next batch's codes in flight while
//       one is multiplied;
//   shared workgroups (the next 256): the shared expert's h =
//       bf16(silu(x Wsg^T) * (x Wsu^T)) (ungated bf16 SwiGLU of width 1024,
//       Flint model card, introduction; four columns of h per workgroup, waves
//       0-3 the gate rows, 4-7 the up rows), streamed beside the routed
//       experts' codes;
//   down workgroups (the last 256): each owns 8 output features.  It requests
//       the shared down weights of its features, routes as the gate/up
//       workgroups do and requests its down codes for every active expert;
//       once h is complete it computes the shared down projection z of its
//       features, and once a is complete it rotates a of every assignment in
//       LDS, finishes the routed down products and writes y = bf16(z + sum_j
//       w_j o_j) in slot order.
//
// h and a cross between workgroups through device-scope stores and loads
// (cache policy sc0 sc1: written through to, and read from, the level shared
// by all XCDs), so neither side needs a whole-L2 writeback or invalidate, and
// through two completion counters (h done, a done) that the first launch sets
// to zero.  Each counter is kept in 16 replicas on separate lines (every
// producing workgroup adds 1 to each, one atomic per lane) and each down
// workgroup polls one replica: 256 pollers of a single line crowd its memory
// channel, and code loads that land on the same channel wait behind them.
// Only the down workgroups wait, and only for gate/up and shared workgroups,
// which have lower indices and never wait, so they were dispatched first and
// finish whatever else is resident; the waits are also bounded in time (5 ms
// by default), and a down workgroup that gives up writes NaN to its outputs
// (y, and in a stack layer the residual stream, so that every later layer's
// output is NaN too) and sets the workspace's error word, so a failure cannot
// hang the device and cannot go unnoticed.
//
// The same launch serves the experts in the NVFP4 container (template
// argument NV; Flint NVFP4 repack, kekzle/Flint-NVFP4, rows "Layout per
// Linear" and "Declaration"): x and a enter as natural-order fp16 with one
// power-of-two prescale per token or assignment (no Hadamard), the E2M1 codes
// times their E4M3 block scales are exact products against them
// (nvfp4_ops.h), and the fp32 tensor scales multiply the row sums.
#include "common.h"
#include "gemv_ops.h"
#include "handoff.h"
#include "launch.h"
#include "nvfp4_ops.h"
#include "token_ops.h"

namespace moe_w4 {

namespace {

constexpr int kFuThreads = 512;
constexpr int kFuWaves = kFuThreads / kWave;        // 8
constexpr int kFuGuWgs = 256;                       // gate/up workgroups
constexpr int kFuShWgs = kIS / 4;                   // shared gate/up workgroups (4 columns of h each)
constexpr int kFuDnWgs = 256;                       // down workgroups
constexpr int kFuDn0 = kFuGuWgs + kFuShWgs;         // first down workgroup
constexpr int kFuCols = kH / kFuDnWgs;              // 8 output features per down workgroup
constexpr int kFuPairs = 2;                         // (gate, up) row pairs per wave batch
constexpr int kFuBatchesPerExpert = kI / kFuPairs;  // 256

static_assert(kFuWaves == kFuCols, "a down wave owns one feature of the shared projection");
static_assert(kFuWaves >= kFusedMaxTokens, "one wave per token for the routing");


template <int T>
struct FuRouting {
    static constexpr int N = kTopK * T;
    int e[N];       // expert of assignment a = 6t + j
    float w[N];     // its weight
    int pos[N];     // sorted position of assignment a
    int perm[N];    // assignment at sorted position p
    int se[N];      // expert at sorted position p
    int act_e[N];   // active experts, ascending
    int act_begin[N];
    int act_n[N];
    int n_act;
};

template <int T>
struct FuGateUp {
    uint32_t xt[T][kH / 2];         // rotated x, fp16 operand order
    float xsc[T][kH / kG];          // 2^sh of each (token, block)
};

template <int T>
struct FuDown {
    static constexpr int N = kTopK * T;
    uint32_t at[N][kI / 2];         // rotated a per sorted position
    float atsc[N][kI / kG];
    float o[N][kFuCols];            // routed outputs of this workgroup's features
    float z[T][kFuCols];            // shared expert outputs
    int fail_h, fail_a;             // a wait gave up
};

template <int T>
struct FuShared {
    uint4 xl[T][kH / 8];            // x, bf16
    float part[8][8];               // [wave][token] row sums
};

template <int T>
union FuWork {
    FuGateUp<T> gu;
    FuDown<T> dn;
    FuShared<T> sh;
};

// Empty asm that "rewrites" a register quad: the mask conversion of codes that
// are reused for several tokens is then redone per token instead of being
// hoisted out of the token loop (all converted rows would not fit in registers).
__device__ __forceinline__ void refresh(uint4 &v) {
    asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
}

__device__ __forceinline__ float4 bf16x4_lo(uint4 q) {
    return make_float4(bf16lo(q.x), bf16hi(q.x), bf16lo(q.y), bf16hi(q.y));
}
__device__ __forceinline__ float4 bf16x4_hi(uint4 q) {
    return make_float4(bf16lo(q.z), bf16hi(q.z), bf16lo(q.w), bf16hi(q.w));
}

// One wave batch of gate/up codes: 2 row pairs, lane l owning K [32l, 32l+32).
struct GuBatch {
    uint4 g[kFuPairs], u[kFuPairs];
    uint16_t sg[kFuPairs], su[kFuPairs];
};

// Row . x_t for every token, by one wave (load i of lane l takes K
// [512i + 8l, 512i + 8l + 8) of the bf16 row, so each load reads 1 KB
// contiguous; x from LDS in the same layout); token t's sum ends on lanes
// 8t..8t+7 (all of them).  The row is requested first (row_load), so that
// its loads are in flight while x is staged.
__device__ __forceinline__ void row_load(const uint16_t *row, int lane, uint4 (&w)[4]) {
    const __amdgpu_buffer_rsrc_t rb = make_buf(row, kH * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = bload16_nt(rb, lane * 16 + 1024 * i, 0);
}
template <int T>
__device__ __forceinline__ float row_dot_tokens(const uint4 (&w)[4], const uint4 (*xl)[kH / 8], int lane) {
    float v[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        float acc = 0.0f;
        if (t < T) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint4 xv = xl[t][64 * i + lane];
                acc = dot2b(xv.x, w[i].x, acc);
                acc = dot2b(xv.y, w[i].y, acc);
                acc = dot2b(xv.z, w[i].z, acc);
                acc = dot2b(xv.w, w[i].w, acc);
            }
        }
        v[t] = acc;
    }
    return transpose_reduce<8, kWave>(v);
}

// ---------------------------------------------------------------------------
// Launch 1: the router logits.  32 workgroups of 8 waves, one router row per
// wave (fp32 sums of exact bf16 products, NInfer README of Flint, "What is
// inside": router rows widened exactly from bf16).  x is staged in LDS once
// per workgroup; in a stack layer (RESID) it is computed there from the fp32
// residual stream as bf16(resid / sqrt(mean(resid^2) + 1e-6)) (wave t: token
// t; every workgroup sums in the same order, so all agree bit for bit) and
// workgroup 0 writes it out.  Workgroup 0 also clears the counters of the
// second launch and, if `error` is not null, the error word.
// ---------------------------------------------------------------------------
constexpr int kRouterWgs = kE / 8;

// Stage x [T][2048] bf16 in LDS, from x itself or (RESID) as the bf16 RMS
// norm of the residual stream; workgroup 0 of the launch writes that x out.
template <int T, bool RESID>
__device__ __forceinline__ void stage_x(const uint16_t *__restrict__ x, const float *__restrict__ resid,
                                        uint16_t *__restrict__ x_out, uint4 (*xl)[kH / 8], int tid, int lane,
                                        int wave) {
    if (!RESID) {
#pragma unroll
        for (int i = 0; i < (T * (kH / 8) + 511) / 512; ++i) {
            const int q = tid + 512 * i;
            if (q < T * (kH / 8)) (&xl[0][0])[q] = reinterpret_cast<const uint4 *>(x)[q];
        }
    } else if (wave < T) {
        // lane l: values 8l .. 8l+7 of each 512-wide quarter (16-byte words 64i + l)
        const int t = wave;
        float4 r[4][2];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float4 *rp = reinterpret_cast<const float4 *>(resid + (size_t)t * kH + 512 * i + 8 * lane);
            r[i][0] = rp[0];
            r[i][1] = rp[1];
        }
        float ss = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                ss += r[i][h].x * r[i][h].x + r[i][h].y * r[i][h].y + r[i][h].z * r[i][h].z + r[i][h].w * r[i][h].w;
        const float inv = 1.0f / sqrtf(wave_sum(ss) / (float)kH + 1e-6f);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float4 a = r[i][0], b = r[i][1];
            uint4 q;
            q.x = (uint32_t)f32_to_bf16(a.x * inv) | ((uint32_t)f32_to_bf16(a.y * inv) << 16);
            q.y = (uint32_t)f32_to_bf16(a.z * inv) | ((uint32_t)f32_to_bf16(a.w * inv) << 16);
            q.z = (uint32_t)f32_to_bf16(b.x * inv) | ((uint32_t)f32_to_bf16(b.y * inv) << 16);
            q.w = (uint32_t)f32_to_bf16(b.z * inv) | ((uint32_t)f32_to_bf16(b.w * inv) << 16);
            xl[t][64 * i + lane] = q;
            if (blockIdx.x == 0) reinterpret_cast<uint4 *>(x_out + (size_t)t * kH + 512 * i + 8 * lane)[0] = q;
        }
    }
}

template <int T, bool RESID>
__global__ __launch_bounds__(512) void k_router_small(const uint16_t *__restrict__ x, const float *__restrict__ resid,
                                                      uint16_t *__restrict__ x_out,
                                                      const uint16_t *__restrict__ router_w,
                                                      const float *__restrict__ bias, float *__restrict__ logits,
                                                      int *__restrict__ counters, int *__restrict__ error) {
    __shared__ uint4 xl[T][kH / 8];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    // both counters of the second launch (a done, h done) and the error word
    if (blockIdx.x == 0 && tid < 2 * kFusedCounters) counters[tid * kFusedCounterStride] = 0;
    if (blockIdx.x == 0 && tid == 2 * kFusedCounters && error) *error = 0;
    // this wave's router row, requested before x is staged
    const int e = 8 * (int)blockIdx.x + wave;
    uint4 w[4];
    row_load(router_w + (size_t)e * kH, lane, w);
    stage_x<T, RESID>(x, resid, x_out, xl, tid, lane, wave);
    __syncthreads();
    const int t = lane >> 3;
    const float sum = row_dot_tokens<T>(w, xl, lane);
    if ((lane & 7) == 0 && t < T) logits[(size_t)t * kE + e] = sum + (bias ? bias[e] : 0.0f);
}

// ---------------------------------------------------------------------------
// Launch 2: everything else (one instance per token count, so that every loop
// over tokens, assignments and down slots has a compile-time trip count and
// the loads of a phase are all issued before the first of them is waited for).
// ---------------------------------------------------------------------------
// NV: NVFP4 experts (nvfp4_ops.h) instead of the int4 ones: x and a as
// natural-order fp16 operands with one power-of-two prescale per token or
// assignment (no Hadamard), E2M1 codes times their E4M3 block scales, and the
// tensor scales applied to the row sums.
template <int T, bool NV>
__global__ __launch_bounds__(kFuThreads) __attribute__((amdgpu_waves_per_eu(4))) void k_decode_fused(FusedDecodeArgs A) {
    constexpr int N = kTopK * T;                              // assignments
    constexpr int kSlots = (N + kFuWaves - 1) / kFuWaves;     // down experts (or positions) per wave at most
    __shared__ FuRouting<T> R;
    __shared__ FuWork<T> U;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = wave_id();
    const bool gu_role = blockIdx.x < kFuGuWgs;

    if ((int)blockIdx.x >= kFuGuWgs && (int)blockIdx.x < kFuDn0) {
        // ---- shared role: 4 columns c0 .. c0+3 of h for every token; this
        // wave's gate (waves 0-3) or up (4-7) row requested before x is staged
        const int c0 = ((int)blockIdx.x - kFuGuWgs) * 4;
        uint4 w[4];
        row_load(A.shared_gu + (size_t)((wave < 4 ? 0 : kIS) + c0 + (wave & 3)) * kH, lane, w);
        stage_x<T, false>(A.x, nullptr, nullptr, U.sh.xl, tid, lane, wave);
        __syncthreads();
        const float sum = row_dot_tokens<T>(w, U.sh.xl, lane);
        if ((lane & 7) == 0) U.sh.part[wave][lane >> 3] = sum;
        __syncthreads();
        if (tid < 4 * T) {
            const int tt = tid >> 2, c = tid & 3;
            const uint16_t hv = f32_to_bf16(silu_f(U.sh.part[c][tt]) * U.sh.part[4 + c][tt]);
            __builtin_amdgcn_raw_buffer_store_b16(hv, make_buf(A.hs, (uint32_t)(T * kIS * 2)),
                                                  2 * (tt * kIS + c0 + c), 0, kHandOff);
        }
        // count this workgroup done once its stores of h are complete
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (wave == 0) count_done(A.counters_h, lane);
        return;
    }

    // ---- work that depends on nothing: the loads of the logits and of x
    // (gate/up role), or of the shared down weights of this workgroup's
    // features (down role: load i of lane l takes K [512i + 8l, 512i + 8l + 8)
    // of row c0 + wave) ----
    float4 lv = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (wave < T) lv = reinterpret_cast<const float4 *>(A.logits + (size_t)wave * kE)[lane];
    constexpr int kRotTasks = (4 * T + kFuWaves - 1) / kFuWaves;   // x quarters per wave
    uint4 xq[kRotTasks];
    uint4 xn[4];   // NV: wave t < T holds x[t][32 lane .. 32 lane + 32)
    uint4 wsd0 = make_uint4(0, 0, 0, 0), wsd1 = wsd0;
    if (NV && gu_role) {
        if (wave < T) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                xn[i] = reinterpret_cast<const uint4 *>(A.x + (size_t)wave * kH + 32 * lane + 8 * i)[0];
        }
    } else if (gu_role) {
        // task k = (token k / 4, 512-wide quarter k % 4), dealt from the last wave down
#pragma unroll
        for (int i = 0; i < kRotTasks; ++i) {
            const int k = min(kFuWaves - 1 - wave + kFuWaves * i, 4 * T - 1);
            xq[i] = reinterpret_cast<const uint4 *>(A.x + (size_t)(k >> 2) * kH + (k & 3) * 512)[lane];
        }
    } else {
        const int c0 = ((int)blockIdx.x - kFuDn0) * kFuCols;
        const __amdgpu_buffer_rsrc_t wb = make_buf(A.shared_down + (size_t)(c0 + wave) * kIS, kIS * 2);
        wsd0 = bload16_nt(wb, lane * 16, 0);
        wsd1 = bload16_nt(wb, lane * 16 + 1024, 0);
    }

    // ---- routing: wave t selects token t's six experts ----
    if (wave < T) {
        const int t = wave;
        const Top6 sel = top6_wave(lv, lane, RouterPolicy{A.router_bias, A.router_policy});
#pragma unroll
        for (int j = 0; j < kTopK; ++j) {
            if (lane == j) {
                R.e[kTopK * t + j] = sel.e[j];
                R.w[kTopK * t + j] = sel.w[j];
            }
        }
    }
    if (NV && gu_role) {
        // x as natural-order fp16 operands, one prescale per token
        if (wave < T) {
            const int sh = natural_x_wave(xn, lane, &U.gu.xt[wave][16 * lane]);
            if (lane == 0) U.gu.xsc[wave][0] = ldexpf(1.0f, sh);
        }
    } else if (gu_role) {
        // rotated x, 4 blocks per task, beside the top-6 (waves from the first up)
#pragma unroll
        for (int i = 0; i < kRotTasks; ++i) {
            const int k = kFuWaves - 1 - wave + kFuWaves * i;
            if (k < 4 * T) {
                const int t = k >> 2, qq = k & 3;
                rotate_act_wave(bf16x4_lo(xq[i]), bf16x4_hi(xq[i]), lane, &U.gu.xt[t][qq * 256], &U.gu.xsc[t][qq * 4]);
            }
        }
    }
    __syncthreads();
    // stable sort of the N <= 48 assignments by expert (rank = number of
    // assignments with a smaller expert, or the same expert and a smaller index)
    if (wave == 0) {
        const int ei = lane < N ? R.e[lane] : 0x7fffffff;
        int rank = 0;
#pragma unroll
        for (int k = 0; k < N; ++k) {
            const int ek = __builtin_amdgcn_readlane(ei, k);
            rank += (ek < ei) || (ek == ei && k < lane);
        }
        if (lane < N) {
            R.pos[lane] = rank;
            R.perm[rank] = lane;
            R.se[rank] = ei;
        }
    }
    __syncthreads();
    if (wave == 0) {
        const int r = lane;
        const int er = r < N ? R.se[r] : -1;
        const bool first = r < N && (r == 0 || R.se[r - 1] != er);
        const uint64_t fb = __ballot(first);
        if (first) {
            const int ai = __popcll(fb & ((1ull << r) - 1ull));
            const uint64_t above = fb >> (r + 1);   // r < 48
            const int next = above ? r + 1 + __builtin_ctzll(above) : N;
            R.act_e[ai] = er;
            R.act_begin[ai] = r;
            R.act_n[ai] = next - r;
        }
        if (lane == 0) R.n_act = __popcll(fb);
    }
    __syncthreads();
    const int n_act = R.n_act;

    // the routing results of the call (one workgroup writes them)
    if (blockIdx.x == 0) {
        if (tid < N) {
            A.topk_idx[tid] = R.e[tid];
            A.topk_w[tid] = R.w[tid];
            A.pos[tid] = R.pos[tid];
            A.perm[tid] = R.perm[tid];
        }
        if (tid <= kE) {
            int c = 0;
            for (int k = 0; k < N; ++k) c += R.se[k] < tid;
            A.offsets[tid] = c;
        }
        if (tid < kE) {
            int4 *rec = reinterpret_cast<int4 *>(A.slots + 8 * tid);
            if (tid < n_act) {
                const int b = R.act_begin[tid], n = R.act_n[tid];
                const int t0 = R.perm[b] / kTopK, t1 = n > 1 ? R.perm[b + 1] / kTopK : t0;
                rec[0] = make_int4(R.act_e[tid], b, n, t0);
                rec[1] = make_int4(t1, 0, 0, 0);
                A.chunks[tid] = make_int4(R.act_e[tid], b, n, 0);   // <= 8 rows: one chunk per expert
            } else {
                rec[0] = make_int4(-1, 0, 0, 0);
                rec[1] = make_int4(0, 0, 0, 0);
            }
        }
        if (tid == 0) {
            *A.n_active = n_act;
            *A.n_chunks = n_act;
        }
    }

    if (gu_role) {
        // ---- routed gate/up: wave batches of 2 row pairs of one active expert,
        // dealt workgroup-major (consecutive batches on different CUs), the
        // next batch's loads in flight while one is multiplied ----
        const int nb = n_act * kFuBatchesPerExpert;
        const rsrc_t act_buf = make_buf(A.act, (uint32_t)(N * kI * 4));
        const uint32_t cv = lane * 16, sv = (lane >> 2) * 2;
        constexpr int kStride = kFuGuWgs * kFuWaves;
        auto load = [&](GuBatch &G, int bb) {
            const int ai = bb / kFuBatchesPerExpert, r0 = (bb % kFuBatchesPerExpert) * kFuPairs;
            const int e = uniform(R.act_e[ai]);
            const rsrc_t cg = make_buf(A.codes + (size_t)e * kCodeBytesPerExpert, kCodeBytesGu);
            const rsrc_t sp = NV ? make_buf(A.nv_scales + (size_t)e * kNvScalePerExpert, kNvScaleGu)
                                 : make_buf(A.scales + (size_t)e * kScalesPerExpert, 2 * kScalesGu);
#pragma unroll
            for (int i = 0; i < kFuPairs; ++i) {
                const int r = r0 + i;
                G.g[i] = bload16_nt(cg, cv, r * (kH / 2));
                G.u[i] = bload16_nt(cg, cv, kPlaneGateBytes + r * (kH / 2));
                if constexpr (NV) {   // the E4M3 scales of blocks 2 lane, 2 lane + 1
                    G.sg[i] = bload2_nt(sp, 2 * lane, r * (kH / kNvBlock));
                    G.su[i] = bload2_nt(sp, 2 * lane, kNvScaleGate + r * (kH / kNvBlock));
                } else {
                    G.sg[i] = bload2_nt(sp, sv, 2 * r * (kH / kG));
                    G.su[i] = bload2_nt(sp, sv, 2 * (kScalesGate + r * (kH / kG)));
                }
            }
        };
        // a batch's products for every token of its expert (codes in G)
        auto compute = [&](GuBatch &G, int bb) {
            const int ai = bb / kFuBatchesPerExpert, r0 = (bb % kFuBatchesPerExpert) * kFuPairs;
            const int p0 = uniform(R.act_begin[ai]), n = uniform(R.act_n[ai]);
            float tg = 1.0f, tu = 1.0f;   // NV: the gate and up tensor scales
            if constexpr (NV) {
                const int e = uniform(R.act_e[ai]);
                tg = A.tscales[3 * e];
                tu = A.tscales[3 * e + 1];
            }
            for (int k = 0; k < n; ++k) {
                const int p = p0 + k;
                const int t = R.perm[p] / kTopK;
#pragma unroll
                for (int i = 0; i < kFuPairs; ++i) {
                    refresh(G.g[i]);
                    refresh(G.u[i]);
                }
                uint32_t xs[16];
                float v[2 * kFuPairs];
                if constexpr (NV) {
                    const uint4 *src = reinterpret_cast<const uint4 *>(&U.gu.xt[t][lane * 16]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint4 w = src[i];
                        xs[4 * i] = w.x; xs[4 * i + 1] = w.y; xs[4 * i + 2] = w.z; xs[4 * i + 3] = w.w;
                    }
                    const float xm = U.gu.xsc[t][0];
#pragma unroll
                    for (int i = 0; i < kFuPairs; ++i) {
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            const uint16_t sc = h ? G.su[i] : G.sg[i];
                            v[2 * i + h] = dot32_nv(h ? G.u[i] : G.g[i], xs, e4m3_to_f32(sc & 0xffu),
                                                    e4m3_to_f32(sc >> 8)) * xm;
                        }
                    }
                } else {
                    const float off = load_operand32(&U.gu.xt[t][lane * 16], xs);
                    const float xsc = U.gu.xsc[t][lane >> 2];
#pragma unroll
                    for (int i = 0; i < kFuPairs; ++i) {
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            Q4 q[4];
                            convert16(h ? G.u[i] : G.g[i], q);
                            v[2 * i + h] = dot_slice(q, xs, -off) * (bf16_to_f32(h ? G.su[i] : G.sg[i]) * xsc);
                        }
                    }
                }
                // value 2i (gate row r0+i) ends on lanes 32i..32i+15, its up row on the next 16
                const float red = transpose_reduce<2 * kFuPairs, kWave>(v);
                const float other = shfl_xor_f(red, 16);
                if ((lane & 31) == 0)
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(silu_f(red * tg) * (other * tu)), act_buf,
                                                          4 * (p * kI + r0 + (lane >> 5)), 0, kHandOff);
            }
        };
        // two register sets in turn (no copies, so the loads of one stay in
        // flight while the other is multiplied); past the end a set re-reads
        // the wave's last batch (in bounds, unused)
        int b = wave * kFuGuWgs + (int)blockIdx.x;
        if (b < nb) {
            GuBatch G0, G1;
            load(G0, b);
            for (;;) {
                load(G1, min(b + kStride, nb - 1));
                compute(G0, b);
                b += kStride;
                if (b >= nb) break;
                load(G0, min(b + kStride, nb - 1));
                compute(G1, b);
                b += kStride;
                if (b >= nb) break;
            }
        }
        // count this workgroup done once every wave's stores of a are complete
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (wave == 0) count_done(A.counters, lane);
        return;
    }

    // ---- down role ----
    const int c0 = ((int)blockIdx.x - kFuDn0) * kFuCols;
    const int replica = ((int)blockIdx.x % kFusedCounters) * kFusedCounterStride;
    // down codes of this workgroup's 8 features for every active expert this
    // wave handles (experts wave, wave + 8, ...): lane l takes row l / 8 and,
    // in half h, K [256h + 32 (l % 8), 256h + 32 (l % 8) + 32) (inside block
    // 2h + (l % 8) / 4), so each load reads 128 contiguous bytes per row
    const int rr = lane >> 3, kq = lane & 7;
    uint4 dw[kSlots][2];
    uint16_t ds[kSlots][2];
#pragma unroll
    for (int s = 0; s < kSlots; ++s) {
        // slots past the last active expert re-read its rows (in bounds, unused),
        // so that every load is issued before any is waited for
        const int ai = min(wave + kFuWaves * s, n_act - 1);
        const int e = uniform(R.act_e[ai]);
        const rsrc_t cd = make_buf(A.codes + (size_t)e * kCodeBytesPerExpert + kCodeBytesGu + (size_t)c0 * (kI / 2),
                                   kFuCols * (kI / 2));
        const rsrc_t sd =
            NV ? make_buf(A.nv_scales + (size_t)e * kNvScalePerExpert + kNvScaleGu + (size_t)c0 * (kI / kNvBlock),
                          kFuCols * (kI / kNvBlock))
               : make_buf(A.scales + (size_t)e * kScalesPerExpert + kScalesGu + (size_t)c0 * (kI / kG),
                          kFuCols * (kI / kG) * 2);
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            dw[s][hf] = bload16_nt(cd, rr * (kI / 2) + 128 * hf + kq * 16, 0);
            // NV: the E4M3 scales of blocks 16 hf + 2 kq, +1; else the bf16 scale of block 2 hf + kq / 4
            ds[s][hf] = NV ? bload2_nt(sd, rr * (kI / kNvBlock) + 16 * hf + 2 * kq, 0)
                           : bload2_nt(sd, 2 * (rr * (kI / kG) + 2 * hf + (kq >> 2)), 0);
        }
    }

    // NaN outputs for this workgroup's features (and in the residual stream of
    // a stack layer), and the error word: a wait gave up
    auto give_up = [&]() {
        if (tid < T * kFuCols) {
            const size_t i = (size_t)(tid / kFuCols) * kH + c0 + tid % kFuCols;
            A.y[i] = 0x7fc0;
            if (A.resid) A.resid[i] = __builtin_nanf("");
        }
        if (tid == 0) __hip_atomic_store(A.error, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };

    // the shared down projection once every shared workgroup is done (bounded):
    // z[t][c0 + wave] = h_t . Wsd[c0 + wave]
    if (tid == 0) U.dn.fail_h = !wait_count(A.counters_h + replica, kFuShWgs, A.wait_ticks);
    __syncthreads();
    if (U.dn.fail_h) {
        give_up();
        return;
    }
    {
        const rsrc_t hb = make_buf(A.hs, (uint32_t)(T * kIS * 2));
        float v[8];
        // four tokens at a time (the down codes in flight hold many registers)
#pragma unroll
        for (int t0 = 0; t0 < 8; t0 += 4) {
            uint4 hq[4][2];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (t0 + i < T) {
                    const int ho = (t0 + i) * kIS * 2;
                    hq[i][0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(hb, lane * 16, ho,
                                                                                               kHandOff));
                    hq[i][1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(hb, lane * 16 + 1024,
                                                                                               ho, kHandOff));
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float acc = 0.0f;
                if (t0 + i < T) {
                    acc = dot2b(hq[i][0].x, wsd0.x, acc); acc = dot2b(hq[i][0].y, wsd0.y, acc);
                    acc = dot2b(hq[i][0].z, wsd0.z, acc); acc = dot2b(hq[i][0].w, wsd0.w, acc);
                    acc = dot2b(hq[i][1].x, wsd1.x, acc); acc = dot2b(hq[i][1].y, wsd1.y, acc);
                    acc = dot2b(hq[i][1].z, wsd1.z, acc); acc = dot2b(hq[i][1].w, wsd1.w, acc);
                }
                v[t0 + i] = acc;
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        const float sum = transpose_reduce<8, kWave>(v);   // token lane / 8
        if ((lane & 7) == 0 && (lane >> 3) < T) U.dn.z[lane >> 3][wave] = sum;
    }

    // wait until every gate/up workgroup is done (bounded)
    if (tid == 0) U.dn.fail_a = !wait_count(A.counters + replica, kFuGuWgs + A.wait_target_extra, A.wait_ticks);
    __syncthreads();
    if (U.dn.fail_a) {
        give_up();
        return;
    }

    // rotated a of every assignment (wave per sorted position), all loads first
    {
        const rsrc_t act_buf = make_buf(A.act, (uint32_t)(N * kI * 4));
        u32x4_t a[kSlots][2];
#pragma unroll
        for (int i = 0; i < kSlots; ++i) {
            const int p = min(wave + kFuWaves * i, N - 1);
            a[i][0] = __builtin_amdgcn_raw_buffer_load_b128(act_buf, 4 * (p * kI + lane * 8), 0, kHandOff);
            a[i][1] = __builtin_amdgcn_raw_buffer_load_b128(act_buf, 4 * (p * kI + lane * 8 + 4), 0, kHandOff);
        }
#pragma unroll
        for (int i = 0; i < kSlots; ++i) {
            const int p = wave + kFuWaves * i;
            if (p < N) {
                if constexpr (NV) {
                    // natural-order fp16 operands, one prescale per assignment
                    const float4 a0 = __builtin_bit_cast(float4, a[i][0]), a1 = __builtin_bit_cast(float4, a[i][1]);
                    const float v[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
                    float amax = 0.0f;
#pragma unroll
                    for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(v[k]));
                    const int sh = prescale_shift(wave_max(amax));
                    uint4 w;
                    w.x = pack_half2(ldexpf(v[0], -sh), ldexpf(v[1], -sh));
                    w.y = pack_half2(ldexpf(v[2], -sh), ldexpf(v[3], -sh));
                    w.z = pack_half2(ldexpf(v[4], -sh), ldexpf(v[5], -sh));
                    w.w = pack_half2(ldexpf(v[6], -sh), ldexpf(v[7], -sh));
                    reinterpret_cast<uint4 *>(&U.dn.at[p][0])[lane] = w;
                    if (lane == 0) U.dn.atsc[p][0] = ldexpf(1.0f, sh);
                } else {
                    rotate_act_wave(__builtin_bit_cast(float4, a[i][0]), __builtin_bit_cast(float4, a[i][1]), lane,
                                    &U.dn.at[p][0], &U.dn.atsc[p][0]);
                }
            }
        }
    }
    __syncthreads();

    // routed down: o[p][c0 + rr] for every sorted position p of the wave's experts
#pragma unroll
    for (int s = 0; s < kSlots; ++s) {
        const int ai = wave + kFuWaves * s;
        if (ai < n_act) {
            const int p0 = uniform(R.act_begin[ai]), n = uniform(R.act_n[ai]);
            const float tsd = NV ? A.tscales[3 * uniform(R.act_e[ai]) + 2] : 1.0f;   // NV: down tensor scale
            for (int k = 0; k < n; ++k) {
                const int p = p0 + k;
                // operands of K [256h + 32 kq, +32): words 128h + 16 kq .. +15
                float acc = 0.0f;
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    refresh(dw[s][hf]);
                    uint32_t xs[16];
                    if constexpr (NV) {
                        const uint4 *src = reinterpret_cast<const uint4 *>(&U.dn.at[p][128 * hf + 16 * kq]);
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const uint4 w = src[i];
                            xs[4 * i] = w.x; xs[4 * i + 1] = w.y; xs[4 * i + 2] = w.z; xs[4 * i + 3] = w.w;
                        }
                        acc += dot32_nv(dw[s][hf], xs, e4m3_to_f32(ds[s][hf] & 0xffu), e4m3_to_f32(ds[s][hf] >> 8));
                    } else {
                        Q4 q[4];
                        convert16(dw[s][hf], q);
                        const float off = load_operand32(&U.dn.at[p][128 * hf + 16 * kq], xs);
                        acc += dot_slice(q, xs, -off) *
                               (bf16_to_f32(ds[s][hf]) * U.dn.atsc[p][2 * hf + (kq >> 2)]);
                    }
                }
                if constexpr (NV) acc *= U.dn.atsc[p][0] * tsd;
                acc += shfl_xor_f(acc, 1);
                acc += shfl_xor_f(acc, 2);
                acc += shfl_xor_f(acc, 4);
                if (kq == 0) U.dn.o[p][rr] = acc;
            }
        }
    }
    __syncthreads();

    // combine in slot order: y = bf16(z + sum_j w_j o_j)
    if (tid < T * kFuCols) {
        const int t = tid / kFuCols, c = tid % kFuCols;
        float acc = U.dn.z[t][c];
#pragma unroll
        for (int j = 0; j < kTopK; ++j) acc = fmaf(R.w[kTopK * t + j], U.dn.o[R.pos[kTopK * t + j]][c], acc);
        const uint16_t yb = f32_to_bf16(acc);
        A.y[(size_t)t * kH + c0 + c] = yb;
        if (A.resid) A.resid[(size_t)t * kH + c0 + c] += bf16_to_f32(yb);   // stack layer: resid += y
    }
}

}  // namespace

#define MOE_FUSED_DISPATCH2(KERNEL, B, ...)                                      \
    switch (T) {                                                                 \
    case 1: hipLaunchKernelGGL((KERNEL<1, B>), __VA_ARGS__); break;              \
    case 2: hipLaunchKernelGGL((KERNEL<2, B>), __VA_ARGS__); break;              \
    case 3: hipLaunchKernelGGL((KERNEL<3, B>), __VA_ARGS__); break;              \
    case 4: hipLaunchKernelGGL((KERNEL<4, B>), __VA_ARGS__); break;              \
    case 5: hipLaunchKernelGGL((KERNEL<5, B>), __VA_ARGS__); break;              \
    case 6: hipLaunchKernelGGL((KERNEL<6, B>), __VA_ARGS__); break;              \
    case 7: hipLaunchKernelGGL((KERNEL<7, B>), __VA_ARGS__); break;              \
    case 8: hipLaunchKernelGGL((KERNEL<8, B>), __VA_ARGS__); break;              \
    default: break;                                                              \
    }

void launch_router_small(const uint16_t *x, const float *resid, uint16_t *x_out, int T, const uint16_t *router_w,
                         const float *bias, float *logits, int *counters, int *error, hipStream_t s) {
    if (resid) {
        MOE_FUSED_DISPATCH2(k_router_small, true, dim3(kRouterWgs), dim3(512), 0, s, x, resid, x_out, router_w, bias,
                            logits, counters, error)
    } else {
        MOE_FUSED_DISPATCH2(k_router_small, false, dim3(kRouterWgs), dim3(512), 0, s, x, resid, x_out, router_w, bias,
                            logits, counters, error)
    }
}

void launch_decode_fused(const FusedDecodeArgs &args, hipStream_t s) {
    const int T = args.T;
    if (args.nv_scales) {
        MOE_FUSED_DISPATCH2(k_decode_fused, true, dim3(kFuDn0 + kFuDnWgs), dim3(kFuThreads), 0, s, args)
    } else {
        MOE_FUSED_DISPATCH2(k_decode_fused, false, dim3(kFuDn0 + kFuDnWgs), dim3(kFuThreads), 0, s, args)
    }
}

#undef MOE_FUSED_DISPATCH2


}  // namespace moe_w4
