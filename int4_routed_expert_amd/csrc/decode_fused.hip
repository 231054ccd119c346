// Decode sizes (1..8 tokens): the layer in two launches.
//
// At these sizes every step of the layer moves little data, so the layer is
// bound by the latency of its dependent steps rather than by bandwidth: a
// launch per step (router, top-6, sort, gate/up, rotation of a, down, combine)
// costs a few microseconds each.  Here the first launch computes everything
// that needs only x: the router logits (one wave per router row) and the
// shared expert's h = bf16(silu(x Wsg^T) * (x Wsu^T)) (ungated bf16 SwiGLU of
// width 1024, Flint model card, Aijuus/flint-w4exp, introduction; four
// columns of h per workgroup).  In a layer of a stack it also computes x
// itself from the residual stream (rmsnorm), and the second launch adds y to
// the residual stream, so a stack layer is two launches as well.  The second
// launch runs all the rest, with two roles of workgroups:
//
//   every workgroup: the routing of all tokens from the logits (wave t: top-6
//       of token t, model card, introduction: 256 experts, top-6; weights
//       sigmoid / max(sum, 2^-14), bloomery issue #632, design thread), then a
//       stable sort of the <= 48 assignments in LDS;
//   gate/up workgroups (the first 256): x is rotated in LDS (fwht128 per
//       128-block, model card, table row "weights"; one task per 512-wide
//       quarter of a token, dealt from the last wave down so that it runs
//       beside the top-6 of the first waves; one power-of-two prescale per
//       block), then wave batches
//       of 2 (gate, up) row pairs of an active expert for all of its tokens,
//       a = silu(g) * u in fp32 (sorted-position order), the next batch's codes
//       in flight while one is multiplied;
//   down workgroups (the other 256): each owns 8 output features.  Before
//       waiting it computes the shared down projection z of its features and
//       requests the down codes of its features for every active expert; once
//       a is complete it rotates a of every assignment in LDS, finishes the
//       routed down products and writes y = bf16(z + sum_j w_j o_j) in slot
//       order.
//
// a crosses between workgroups through device-scope stores and loads (cache
// policy sc0 sc1: written through to, and read from, the level shared by all
// XCDs), so neither side needs a whole-L2 writeback or invalidate, and through
// a completion counter that the first launch sets to zero.  The counter is
// kept in 16 replicas on separate lines (every gate/up workgroup adds 1 to
// each, one atomic per lane) and each down workgroup polls one replica: 256
// pollers of a single line crowd its memory channel, and code loads that land
// on the same channel wait behind them.  Only the down workgroups wait, and
// only for gate/up workgroups, which have lower indices and never wait, so
// they were dispatched first and finish whatever else is resident; the wait
// is also bounded in time (5 ms by default), and a down workgroup that gives
// up writes NaN to its outputs (y, and in a stack layer the residual stream,
// so that every later layer's output is NaN too) and sets the workspace's
// error word, so a failure cannot hang the device and cannot go unnoticed.
#include "common.h"
#include "gemv_ops.h"
#include "launch.h"
#include "token_ops.h"

namespace moe_w4 {

namespace {

constexpr int kFuThreads = 512;
constexpr int kFuWaves = kFuThreads / kWave;        // 8
constexpr int kFuGuWgs = 256;                       // gate/up workgroups
constexpr int kFuDnWgs = 256;                       // down workgroups
constexpr int kFuCols = kH / kFuDnWgs;              // 8 output features per down workgroup
constexpr int kFuPairs = 2;                         // (gate, up) row pairs per wave batch
constexpr int kFuBatchesPerExpert = kI / kFuPairs;  // 256

static_assert(kFuWaves == kFuCols, "a down wave owns one feature of the shared projection");
static_assert(kFuWaves >= kFusedMaxTokens, "one wave per token for the routing");

// Cache policy of the a hand-off: device scope (sc1) plus the volatile
// bit, which keeps the accesses in program order around the counter and
// barriers (the compiler adds sc0: system scope, also coherent across XCDs).
constexpr int kHandOff = 16 | (int)(1u << 31);

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
    int fail;
};

template <int T>
union FuWork {
    FuGateUp<T> gu;
    FuDown<T> dn;
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

// Poll one replica of a completion counter until it reaches `target` or
// `ticks` of the 100 MHz real-time clock pass; returns whether it was reached.
__device__ __forceinline__ bool wait_count(const int *counter, int target, uint32_t ticks) {
    const uint64_t t_start = __builtin_amdgcn_s_memrealtime();
    for (;;) {
        if (__hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= target) return true;
        if (__builtin_amdgcn_s_memrealtime() - t_start > ticks) return false;
        __builtin_amdgcn_s_sleep(8);
    }
}

// Add 1 to every replica of a counter (lanes 0..15 of the calling wave).
__device__ __forceinline__ void count_done(int *counters, int lane) {
    if (lane < kFusedCounters)
        __hip_atomic_fetch_add(counters + lane * kFusedCounterStride, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
// Launch 1: what needs only x.  Workgroups of 8 waves, one weight row per
// wave: the first 32 compute router logits (fp32 sums of exact bf16
// products, NInfer README of Flint, "What is inside": router rows widened
// exactly from bf16), the other 256 four columns c of h each (waves 0-3 the
// gate rows, 4-7 the up rows).  x is staged in LDS once per workgroup; in a
// stack layer (RESID) it is computed there from the fp32 residual stream as
// bf16(resid / sqrt(mean(resid^2) + 1e-6)) (wave t: token t; every
// workgroup sums in the same order, so all agree bit for bit) and workgroup 0
// writes it out.  Workgroup 0 also clears the counters of the second launch
// and, if `error` is not null, the error word.
// ---------------------------------------------------------------------------
constexpr int kRouterWgs = kE / 8;
constexpr int kSharedWgs = kIS / 4;

template <int T, bool RESID>
__global__ __launch_bounds__(512) void k_router_shared_small(const uint16_t *__restrict__ x,
                                                             const float *__restrict__ resid,
                                                             uint16_t *__restrict__ x_out,
                                                             const uint16_t *__restrict__ router_w,
                                                             const float *__restrict__ bias,
                                                             const uint16_t *__restrict__ shared_gu,
                                                             float *__restrict__ logits, uint16_t *__restrict__ hs,
                                                             int *__restrict__ counters, int *__restrict__ error) {
    __shared__ uint4 xl[T][kH / 8];
    __shared__ float part[8][8];   // shared role: [wave][token]
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    if (blockIdx.x == 0 && tid < kFusedCounters) counters[tid * kFusedCounterStride] = 0;
    if (blockIdx.x == 0 && tid == kFusedCounters && error) *error = 0;
    // this wave's weight row (router row e, or gate (waves 0-3) / up (4-7) row
    // c0 + (wave & 3) of the shared expert), requested before x is staged
    const bool router = (int)blockIdx.x < kRouterWgs;
    const int e = 8 * (int)blockIdx.x + wave;
    const int c0 = ((int)blockIdx.x - kRouterWgs) * 4;
    uint4 w[4];
    row_load(router ? router_w + (size_t)e * kH : shared_gu + (size_t)((wave < 4 ? 0 : kIS) + c0 + (wave & 3)) * kH,
             lane, w);
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
    __syncthreads();
    const int t = lane >> 3;
    const float sum = row_dot_tokens<T>(w, xl, lane);
    if (router) {
        if ((lane & 7) == 0 && t < T) logits[(size_t)t * kE + e] = sum + (bias ? bias[e] : 0.0f);
        return;
    }
    if ((lane & 7) == 0) part[wave][t] = sum;
    __syncthreads();
    if (tid < 4 * T) {
        const int tt = tid >> 2, c = tid & 3;
        hs[(size_t)tt * kIS + c0 + c] = f32_to_bf16(silu_f(part[c][tt]) * part[4 + c][tt]);
    }
}

// ---------------------------------------------------------------------------
// Launch 2: everything else (one instance per token count, so that every loop
// over tokens, assignments and down slots has a compile-time trip count and
// the loads of a phase are all issued before the first of them is waited for).
// ---------------------------------------------------------------------------
template <int T>
__global__ __launch_bounds__(kFuThreads) __attribute__((amdgpu_waves_per_eu(4))) void k_decode_fused(FusedDecodeArgs A) {
    constexpr int N = kTopK * T;                              // assignments
    constexpr int kSlots = (N + kFuWaves - 1) / kFuWaves;     // down experts (or positions) per wave at most
    __shared__ FuRouting<T> R;
    __shared__ FuWork<T> U;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = wave_id();
    const bool gu_role = blockIdx.x < kFuGuWgs;

    // ---- work that depends on nothing: the loads of the logits and of x
    // (gate/up role), or the shared down projection of this workgroup's
    // features, z[t][c0 + wave] = h_t . Wsd[c0 + wave], load i of lane l taking
    // K [512i + 8l, 512i + 8l + 8) (down role) ----
    float4 lv = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (wave < T) lv = reinterpret_cast<const float4 *>(A.logits + (size_t)wave * kE)[lane];
    constexpr int kRotTasks = (4 * T + kFuWaves - 1) / kFuWaves;   // x quarters per wave
    uint4 xq[kRotTasks];
    if (gu_role) {
        // task k = (token k / 4, 512-wide quarter k % 4), dealt from the last wave down
#pragma unroll
        for (int i = 0; i < kRotTasks; ++i) {
            const int k = min(kFuWaves - 1 - wave + kFuWaves * i, 4 * T - 1);
            xq[i] = reinterpret_cast<const uint4 *>(A.x + (size_t)(k >> 2) * kH + (k & 3) * 512)[lane];
        }
    } else {
        const int c0 = ((int)blockIdx.x - kFuGuWgs) * kFuCols;
        const __amdgpu_buffer_rsrc_t wb = make_buf(A.shared_down + (size_t)(c0 + wave) * kIS, kIS * 2);
        const __amdgpu_buffer_rsrc_t hb = make_buf(A.hs, (uint32_t)(T * kIS * 2));
        const uint4 w0 = bload16_nt(wb, lane * 16, 0), w1 = bload16_nt(wb, lane * 16 + 1024, 0);
        uint4 hq[T][2];
#pragma unroll
        for (int t = 0; t < T; ++t) {
            hq[t][0] = bload16(hb, lane * 16, t * kIS * 2);
            hq[t][1] = bload16(hb, lane * 16 + 1024, t * kIS * 2);
        }
        float v[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            float acc = 0.0f;
            if (t < T) {
                acc = dot2b(hq[t][0].x, w0.x, acc); acc = dot2b(hq[t][0].y, w0.y, acc);
                acc = dot2b(hq[t][0].z, w0.z, acc); acc = dot2b(hq[t][0].w, w0.w, acc);
                acc = dot2b(hq[t][1].x, w1.x, acc); acc = dot2b(hq[t][1].y, w1.y, acc);
                acc = dot2b(hq[t][1].z, w1.z, acc); acc = dot2b(hq[t][1].w, w1.w, acc);
            }
            v[t] = acc;
        }
        const float sum = transpose_reduce<8, kWave>(v);   // token lane / 8
        if ((lane & 7) == 0 && (lane >> 3) < T) U.dn.z[lane >> 3][wave] = sum;
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
    if (gu_role) {
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
            const rsrc_t sp = make_buf(A.scales + (size_t)e * kScalesPerExpert, 2 * kScalesGu);
#pragma unroll
            for (int i = 0; i < kFuPairs; ++i) {
                const int r = r0 + i;
                G.g[i] = bload16_nt(cg, cv, r * (kH / 2));
                G.u[i] = bload16_nt(cg, cv, kPlaneGateBytes + r * (kH / 2));
                G.sg[i] = bload2_nt(sp, sv, 2 * r * (kH / kG));
                G.su[i] = bload2_nt(sp, sv, 2 * (kScalesGate + r * (kH / kG)));
            }
        };
        // a batch's products for every token of its expert (codes in G)
        auto compute = [&](GuBatch &G, int bb) {
            const int ai = bb / kFuBatchesPerExpert, r0 = (bb % kFuBatchesPerExpert) * kFuPairs;
            const int p0 = uniform(R.act_begin[ai]), n = uniform(R.act_n[ai]);
            for (int k = 0; k < n; ++k) {
                const int p = p0 + k;
                const int t = R.perm[p] / kTopK;
#pragma unroll
                for (int i = 0; i < kFuPairs; ++i) {
                    refresh(G.g[i]);
                    refresh(G.u[i]);
                }
                uint32_t xs[16];
                const float off = load_operand32(&U.gu.xt[t][lane * 16], xs);
                const float xsc = U.gu.xsc[t][lane >> 2];
                float v[2 * kFuPairs];
#pragma unroll
                for (int i = 0; i < kFuPairs; ++i) {
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        Q4 q[4];
                        convert16(h ? G.u[i] : G.g[i], q);
                        v[2 * i + h] = dot_slice(q, xs, -off) * (bf16_to_f32(h ? G.su[i] : G.sg[i]) * xsc);
                    }
                }
                // value 2i (gate row r0+i) ends on lanes 32i..32i+15, its up row on the next 16
                const float red = transpose_reduce<2 * kFuPairs, kWave>(v);
                const float other = shfl_xor_f(red, 16);
                if ((lane & 31) == 0)
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(silu_f(red) * other), act_buf,
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
    const int c0 = ((int)blockIdx.x - kFuGuWgs) * kFuCols;
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
        const rsrc_t sd = make_buf(A.scales + (size_t)e * kScalesPerExpert + kScalesGu + (size_t)c0 * (kI / kG),
                                   kFuCols * (kI / kG) * 2);
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            dw[s][hf] = bload16_nt(cd, rr * (kI / 2) + 128 * hf + kq * 16, 0);
            ds[s][hf] = bload2_nt(sd, 2 * (rr * (kI / kG) + 2 * hf + (kq >> 2)), 0);
        }
    }

    // wait until every gate/up workgroup is done (bounded)
    if (tid == 0) U.dn.fail = !wait_count(A.counters + replica, kFuGuWgs + A.wait_target_extra, A.wait_ticks);
    __syncthreads();
    if (U.dn.fail) {
        // NaN outputs for this workgroup's features (and in the residual
        // stream of a stack layer), and the error word
        if (tid < T * kFuCols) {
            const size_t i = (size_t)(tid / kFuCols) * kH + c0 + tid % kFuCols;
            A.y[i] = 0x7fc0;
            if (A.resid) A.resid[i] = __builtin_nanf("");
        }
        if (tid == 0) __hip_atomic_store(A.error, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
            if (p < N)
                rotate_act_wave(__builtin_bit_cast(float4, a[i][0]), __builtin_bit_cast(float4, a[i][1]), lane,
                                &U.dn.at[p][0], &U.dn.atsc[p][0]);
        }
    }
    __syncthreads();

    // routed down: o[p][c0 + rr] for every sorted position p of the wave's experts
#pragma unroll
    for (int s = 0; s < kSlots; ++s) {
        const int ai = wave + kFuWaves * s;
        if (ai < n_act) {
            const int p0 = uniform(R.act_begin[ai]), n = uniform(R.act_n[ai]);
            for (int k = 0; k < n; ++k) {
                const int p = p0 + k;
                // operands of K [256h + 32 kq, +32): words 128h + 16 kq .. +15
                float acc = 0.0f;
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    refresh(dw[s][hf]);
                    Q4 q[4];
                    convert16(dw[s][hf], q);
                    uint32_t xs[16];
                    const float off = load_operand32(&U.dn.at[p][128 * hf + 16 * kq], xs);
                    acc += dot_slice(q, xs, -off) *
                           (bf16_to_f32(ds[s][hf]) * U.dn.atsc[p][2 * hf + (kq >> 2)]);
                }
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

#define MOE_FUSED_DISPATCH(KERNEL, ...)                                          \
    switch (T) {                                                                 \
    case 1: hipLaunchKernelGGL(KERNEL<1>, __VA_ARGS__); break;                   \
    case 2: hipLaunchKernelGGL(KERNEL<2>, __VA_ARGS__); break;                   \
    case 3: hipLaunchKernelGGL(KERNEL<3>, __VA_ARGS__); break;                   \
    case 4: hipLaunchKernelGGL(KERNEL<4>, __VA_ARGS__); break;                   \
    case 5: hipLaunchKernelGGL(KERNEL<5>, __VA_ARGS__); break;                   \
    case 6: hipLaunchKernelGGL(KERNEL<6>, __VA_ARGS__); break;                   \
    case 7: hipLaunchKernelGGL(KERNEL<7>, __VA_ARGS__); break;                   \
    case 8: hipLaunchKernelGGL(KERNEL<8>, __VA_ARGS__); break;                   \
    default: break;                                                              \
    }

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

void launch_router_shared_small(const uint16_t *x, const float *resid, uint16_t *x_out, int T,
                                const uint16_t *router_w, const float *bias, const uint16_t *shared_w, float *logits,
                                uint16_t *hs, int *counters, int *error, hipStream_t s) {
    if (resid) {
        MOE_FUSED_DISPATCH2(k_router_shared_small, true, dim3(kRouterWgs + kSharedWgs), dim3(512), 0, s, x, resid, x_out,
                            router_w, bias, shared_w, logits, hs, counters, error)
    } else {
        MOE_FUSED_DISPATCH2(k_router_shared_small, false, dim3(kRouterWgs + kSharedWgs), dim3(512), 0, s, x, resid, x_out,
                            router_w, bias, shared_w, logits, hs, counters, error)
    }
}

#undef MOE_FUSED_DISPATCH2

void launch_decode_fused(const FusedDecodeArgs &args, hipStream_t s) {
    const int T = args.T;
    MOE_FUSED_DISPATCH(k_decode_fused, dim3(kFuGuWgs + kFuDnWgs), dim3(kFuThreads), 0, s, args)
}

#undef MOE_FUSED_DISPATCH

}  // namespace moe_w4
