// Decode sizes (1..8 tokens): everything after the router in one launch.
//
// At these sizes every step of the layer moves little data, so the layer is
// bound by the latency of its dependent steps rather than by bandwidth: a
// launch per step (top-6, sort, gate/up, rotation of a, down, combine) costs
// a few microseconds each.  Here one launch runs them all, with two roles of
// workgroups and one dependency between them:
//
//   every workgroup: the routing of all tokens from the logits (wave t: top-6
//       of token t, Flint model card, Aijuus/flint-w4exp, introduction: 256
//       experts, top-6; weights sigmoid / max(sum, 2^-14), bloomery issue #632,
//       design thread), then a stable sort of the <= 48 assignments in LDS;
//   gate/up workgroups (the first kFuGuWgs): rotated x in LDS (fwht128, model
//       card, table row "weights"), then wave batches of 4 (gate, up) row pairs
//       of an active expert for all of its tokens, a = silu(g) * u stored in
//       fp32 (sorted-position order); then each workgroup counts itself done;
//   down workgroups (the rest): each owns 8 output features.  Before waiting
//       it computes the shared expert's down projection for its features (h is
//       complete: the router launch wrote it) and requests the down codes of
//       its features for every active expert.  Once every gate/up workgroup
//       has counted itself done it rotates a of every assignment in LDS,
//       finishes the routed down products and writes y = bf16(z + sum_j w_j o_j)
//       in slot order.
//
// The dependency is a device-scope completion counter that the router launch
// sets to zero.  It is kept in 16 replicas on separate 256-byte lines (every
// gate/up workgroup adds 1 to each, with one atomic per lane of a wave) and
// each down workgroup polls one of them: 256 pollers of a single line crowd
// that line's memory channel, and the gate/up code loads that land on the
// same channel wait behind them (measured: 3 us loads became 8-13 us).  a crosses between the
// workgroups with device-scope stores and loads (cache policy sc0 sc1: written
// through to, and read from, the level shared by all XCDs), so neither side
// needs a whole-L2 writeback or invalidate (a fence at device scope costs one
// of those per workgroup, and with 512 workgroups they dominated the launch):
// a gate/up workgroup waits until its stores are complete, then counts
// itself done.  The down workgroups only ever wait for gate/up workgroups,
// which have lower indices and never wait, so they were dispatched first and
// finish whatever else is resident; the wait is also bounded in time, and a
// down workgroup that gives up writes NaN to its outputs, so a failure cannot
// hang the device and cannot go unnoticed.
#include "common.h"
#include "gemv_ops.h"
#include "launch.h"
#include "token_ops.h"

namespace moe_w4 {

namespace {

constexpr int kFuMaxA = kTopK * kFusedMaxTokens;   // 48 assignments at most
constexpr int kFuThreads = 512;
constexpr int kFuWaves = kFuThreads / kWave;        // 8
constexpr int kFuGuWgs = 256;                       // gate/up workgroups
constexpr int kFuDnWgs = 256;                       // down workgroups
constexpr int kFuCols = kH / kFuDnWgs;              // 8 output features per down workgroup
constexpr int kFuBatchesPerExpert = kI / kGuPairs;  // 128 batches of 4 row pairs
constexpr uint64_t kFuWaitTicks = 500000;           // 5 ms of the 100 MHz s_memrealtime clock

static_assert(kFuWaves == kFuCols, "a down wave owns one feature of the shared projection");
static_assert(kFuWaves >= kFusedMaxTokens, "one wave per token for the routing");

struct FuRouting {
    int e[kFuMaxA];       // expert of assignment a = 6t + j
    float w[kFuMaxA];     // its weight
    int pos[kFuMaxA];     // sorted position of assignment a
    int perm[kFuMaxA];    // assignment at sorted position p
    int se[kFuMaxA];      // expert at sorted position p
    int act_e[kFuMaxA];   // active experts, ascending
    int act_begin[kFuMaxA];
    int act_n[kFuMaxA];
    int n_act;
};

struct FuGateUp {
    uint32_t xt[kFusedMaxTokens][kH / 2];   // rotated x, fp16 operand order
    float xsc[kFusedMaxTokens];             // 2^sh of each token
};

struct FuDown {
    uint32_t at[kFuMaxA][kI / 2];           // rotated a per sorted position
    float atsc[kFuMaxA][kI / kG];
    float o[kFuMaxA][kFuCols];              // routed outputs of this workgroup's features
    float z[kFusedMaxTokens][kFuCols];      // shared expert outputs
    int fail;
};

union FuWork {
    FuGateUp gu;
    FuDown dn;
};

// Cache policy of the a hand-off: device scope (sc1) plus the volatile bit,
// which keeps the accesses in program order around the counter and barrier
// (the compiler adds sc0: system scope, also coherent across the XCDs).
constexpr int kHandOff = 16 | (int)(1u << 31);

// Empty asm that "rewrites" a register quad: the mask conversion of codes that
// are reused for several tokens is then redone per token instead of being
// hoisted out of the token loop (all converted rows would not fit in registers).
__device__ __forceinline__ void refresh(uint4 &v) {
    asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
}

// One instance per token count: every loop over tokens, assignments and
// down slots has a compile-time trip count, so the loads of a phase are all
// issued before the first of them is waited for.
template <int T>
__global__ __launch_bounds__(kFuThreads) __attribute__((amdgpu_waves_per_eu(4))) void k_decode_fused(FusedDecodeArgs A) {
    constexpr int N = kTopK * T;                       // assignments
    constexpr int kSlots = (N + kFuWaves - 1) / kFuWaves;   // down experts per wave at most
    __shared__ FuRouting R;
    __shared__ FuWork U;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = wave_id();
    const bool gu_role = blockIdx.x < kFuGuWgs;
    const int c0 = ((int)blockIdx.x - kFuGuWgs) * kFuCols;   // down role: first output feature

    // ---- work that depends on nothing: the loads of x (gate/up role), or
    // the shared expert's down projection for this workgroup's features (down
    // role): z[t][c0 + wave] = h_t . Wsd[c0 + wave], lane l owning K [16l, 16l+16)
    float4 lv = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (wave < T) lv = reinterpret_cast<const float4 *>(A.logits + (size_t)wave * kE)[lane];
    uint4 xq[4];
    if (gu_role) {
        if (wave < T) {
            const uint4 *xp = reinterpret_cast<const uint4 *>(A.x + (size_t)wave * kH + lane * 32);
#pragma unroll
            for (int i = 0; i < 4; ++i) xq[i] = xp[i];
        }
    } else {
        const __amdgpu_buffer_rsrc_t wb = make_buf(A.shared_down + (size_t)(c0 + wave) * kIS, kIS * 2);
        const uint4 w0 = bload16_nt(wb, lane * 32, 0), w1 = bload16_nt(wb, lane * 32 + 16, 0);
        const __amdgpu_buffer_rsrc_t hb = make_buf(A.hs, (uint32_t)(T * kIS * 2));
        uint4 h[T][2];
#pragma unroll
        for (int t = 0; t < T; ++t) {
            h[t][0] = bload16(hb, lane * 32, t * kIS * 2);
            h[t][1] = bload16(hb, lane * 32 + 16, t * kIS * 2);
        }
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const uint4 h0 = h[t][0], h1 = h[t][1];
            float acc = 0.0f;
            acc = dot2b(h0.x, w0.x, acc); acc = dot2b(h0.y, w0.y, acc);
            acc = dot2b(h0.z, w0.z, acc); acc = dot2b(h0.w, w0.w, acc);
            acc = dot2b(h1.x, w1.x, acc); acc = dot2b(h1.y, w1.y, acc);
            acc = dot2b(h1.z, w1.z, acc); acc = dot2b(h1.w, w1.w, acc);
            acc = wave_sum(acc);
            if (lane == 0) U.dn.z[t][wave] = acc;
        }
    }

    // ---- routing: wave t selects token t's six experts ----
    if (wave < T) {
        const int t = wave;
        const Top6 sel = top6_wave(lv, lane);
#pragma unroll
        for (int j = 0; j < kTopK; ++j) {
            if (lane == j) {
                R.e[kTopK * t + j] = sel.e[j];
                R.w[kTopK * t + j] = sel.w[j];
            }
        }
        if (gu_role) {
            const int sh = rotate_x_wave(xq, lane, &U.gu.xt[t][lane * 16]);
            if (lane == 0) U.gu.xsc[t] = ldexpf(1.0f, sh);
        }
    }
    __syncthreads();
    // stable sort of the N <= 48 assignments by expert (rank = number of
    // assignments with a smaller expert, or the same expert and a smaller index)
    if (wave == 0) {
        const int ei = lane < N ? R.e[lane] : 0x7fffffff;
        int rank = 0;
        for (int k = 0; k < N; ++k) {
            const int ek = R.e[k];
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
        // ---- gate/up: wave batches of 4 row pairs of one active expert ----
        const int nb = n_act * kFuBatchesPerExpert;
        const rsrc_t act_buf = make_buf(A.act, (uint32_t)(N * kI * 4));
        const uint32_t cv = lane * 16, sv = (lane >> 2) * 2;
        for (int b = (int)blockIdx.x * kFuWaves + wave; b < nb; b += kFuGuWgs * kFuWaves) {
            const int ai = b / kFuBatchesPerExpert;
            const int r0 = (b % kFuBatchesPerExpert) * kGuPairs;
            const int e = uniform(R.act_e[ai]), p0 = uniform(R.act_begin[ai]), n = uniform(R.act_n[ai]);
            const rsrc_t cg = make_buf(A.codes + (size_t)e * kCodeBytesPerExpert, kCodeBytesGu);
            const rsrc_t sp = make_buf(A.scales + (size_t)e * kScalesPerExpert, 2 * kScalesGu);
            GuRows G;
#pragma unroll
            for (int i = 0; i < kGuPairs; ++i) gu_load_pair<false>(G, i, cg, sp, cv, sv, r0 + i);
            for (int k = 0; k < n; ++k) {
                const int p = p0 + k;
                const int t = R.perm[p] / kTopK;
#pragma unroll
                for (int i = 0; i < kGuPairs; ++i) {
                    refresh(G.g[i]);
                    refresh(G.u[i]);
                }
                uint32_t xs[16];
                const float off = load_operand32(&U.gu.xt[t][lane * 16], xs);
                const float sc = U.gu.xsc[t];
                float v[2 * kGuPairs];
#pragma unroll
                for (int i = 0; i < kGuPairs; ++i) {
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        Q4 q[4];
                        convert16(h ? G.u[i] : G.g[i], q);
                        v[2 * i + h] = dot_slice(q, xs, -off) * bf16_to_f32(h ? G.su[i] : G.sg[i]);
                    }
                }
                // value 2i (gate row r0+i) and 2i+1 (its up row) end on lanes 8*(2i)..
                const float red = transpose_reduce<2 * kGuPairs, kWave>(v);
                const float other = shfl_xor_f(red, 8);
                const int vi = lane >> 3;
                if ((vi & 1) == 0 && (lane & 7) == 0)
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(silu_f(red * sc) * (other * sc)), act_buf,
                                                          4 * (p * kI + r0 + (vi >> 1)), 0, kHandOff);
            }
        }
        // count this workgroup done once every wave's stores of a are complete
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tid < kFusedCounters)
            __hip_atomic_fetch_add(A.counters + tid * kFusedCounterStride, 1, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        return;
    }

    // ---- down role ----
    // down codes of this workgroup's 8 features for every active expert this
    // wave handles (experts wave, wave + 8, ...): lane l takes row l / 8 and
    // K [64 (l % 8), 64 (l % 8) + 64), inside block (l % 8) / 2
    const int rr = lane >> 3, kq = lane & 7;
    uint4 dw[kSlots][2];
    uint16_t ds[kSlots];
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
        dw[s][0] = bload16_nt(cd, rr * (kI / 2) + kq * 32, 0);
        dw[s][1] = bload16_nt(cd, rr * (kI / 2) + kq * 32 + 16, 0);
        ds[s] = bload2_nt(sd, 2 * (rr * (kI / kG) + (kq >> 1)), 0);
    }

    // wait until every gate/up workgroup is done (bounded)
    if (tid == 0) {
        const int *counter = A.counters + (blockIdx.x % kFusedCounters) * kFusedCounterStride;
        const uint64_t t_start = __builtin_amdgcn_s_memrealtime();
        int ok = 0;
        for (;;) {
            if (__hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= kFuGuWgs) {
                ok = 1;
                break;
            }
            if (__builtin_amdgcn_s_memrealtime() - t_start > kFuWaitTicks) break;
            __builtin_amdgcn_s_sleep(8);
        }
        U.dn.fail = !ok;
    }
    __syncthreads();
    if (U.dn.fail) {
        if (tid < T * kFuCols) A.y[(size_t)(tid / kFuCols) * kH + c0 + tid % kFuCols] = 0x7fc0;   // NaN
        return;
    }

    // rotated a of every assignment (wave per sorted position)
    const rsrc_t act_buf = make_buf(A.act, (uint32_t)(N * kI * 4));
#pragma unroll
    for (int p = wave; p < N; p += kFuWaves) {
        const u32x4_t a0 = __builtin_amdgcn_raw_buffer_load_b128(act_buf, 4 * (p * kI + lane * 8), 0, kHandOff);
        const u32x4_t a1 = __builtin_amdgcn_raw_buffer_load_b128(act_buf, 4 * (p * kI + lane * 8 + 4), 0, kHandOff);
        rotate_act_wave(__builtin_bit_cast(float4, a0), __builtin_bit_cast(float4, a1), lane, &U.dn.at[p][0],
                        &U.dn.atsc[p][0]);
    }
    __syncthreads();

    // routed down: o[p][c0 + rr] for every sorted position p of the wave's experts
#pragma unroll
    for (int s = 0; s < kSlots; ++s) {
        const int ai = wave + kFuWaves * s;
        if (ai < n_act) {
            const int p0 = uniform(R.act_begin[ai]), n = uniform(R.act_n[ai]);
            const float srow = bf16_to_f32(ds[s]);
            for (int k = 0; k < n; ++k) {
                const int p = p0 + k;
                // operands of K [64 kq, 64 kq + 64): words 32 kq .. 32 kq + 31,
                // one 32-code half at a time
                float acc = 0.0f;
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    refresh(dw[s][hf]);
                    Q4 q[4];
                    convert16(dw[s][hf], q);
                    uint32_t xs[16];
                    const float off = load_operand32(&U.dn.at[p][32 * kq + 16 * hf], xs);
                    acc = dot_slice(q, xs, acc - off);
                }
                acc *= srow * U.dn.atsc[p][kq >> 1];
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
        A.y[(size_t)t * kH + c0 + c] = f32_to_bf16(acc);
    }
}

}  // namespace

void launch_decode_fused(const FusedDecodeArgs &args, hipStream_t s) {
    const dim3 grid(kFuGuWgs + kFuDnWgs), block(kFuThreads);
    switch (args.T) {
    case 1: hipLaunchKernelGGL(k_decode_fused<1>, grid, block, 0, s, args); break;
    case 2: hipLaunchKernelGGL(k_decode_fused<2>, grid, block, 0, s, args); break;
    case 3: hipLaunchKernelGGL(k_decode_fused<3>, grid, block, 0, s, args); break;
    case 4: hipLaunchKernelGGL(k_decode_fused<4>, grid, block, 0, s, args); break;
    case 5: hipLaunchKernelGGL(k_decode_fused<5>, grid, block, 0, s, args); break;
    case 6: hipLaunchKernelGGL(k_decode_fused<6>, grid, block, 0, s, args); break;
    case 7: hipLaunchKernelGGL(k_decode_fused<7>, grid, block, 0, s, args); break;
    default: hipLaunchKernelGGL(k_decode_fused<8>, grid, block, 0, s, args); break;
    }
}

}  // namespace moe_w4
