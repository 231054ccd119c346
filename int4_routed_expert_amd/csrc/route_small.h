// Routing of a few tokens (up to kRouteSmallMaxTokens) in one launch of
// ceil(T / 8) workgroups of 8 waves: wave w of workgroup b selects the top-6
// of token 8b + w (model card, introduction: 256 experts, top-6; weights
// sigmoid / max(sum, 2^-14), bloomery issue #632, design thread), all tokens
// side by side; the selections are handed to workgroup 0 through the
// workspace (coherent stores and a completion counter that the launch before
// clears), and workgroup 0 sorts the <= 288 assignments by expert in LDS
// (a stable counting sort, the algorithm of k_sort) and writes offsets,
// perm, pos, the slot records and the chunk list.  One token per wave: the
// selection is a chain of ~450 dependent instructions (~1.2 us), which one
// workgroup walking four tokens per wave paid four times.
#pragma once

#include "common.h"
#include "handoff.h"
#include "launch.h"
#include "token_ops.h"

namespace moe_w4 {

struct RouteSmallArgs {
    const float *logits;   // [T][256], without the bias
    int T;
    RouterPolicy rp;
    int *topk_idx;
    float *topk_w;
    int *offsets;
    int *perm;
    int *pos;
    int *n_active;
    int *slots;
    int4 *chunks;
    int *n_chunks;
    int *error_clear;      // cleared at the start, or null (keep an earlier failure visible)
    int *error;            // set to 1 if the hand-off wait gives up
    float *o;              // expert rows [6T][2048] fp32 (filled with NaN if the wait gives up)
    int *counters;         // completion counter replicas (zero on entry)
    int wait_target_extra; // added to the wait target (tests of the failure path)
    uint32_t wait_ticks;
};

constexpr int kRouteWaves = 8;
constexpr int kRouteMaxChunks = (kTopK * kRouteSmallMaxTokens + 63) / 64;
static_assert(kRouteWaves >= kRouteMaxChunks, "one wave per 64 assignments in the ranking");

// The hand-off wait gave up: routing that no kernel after it can misuse (no
// active expert, pos and perm the identity), NaN expert rows so that every y
// the combine writes is NaN, and the error word set.
__device__ __forceinline__ void route_give_up(const RouteSmallArgs &A, int tid) {
    const int N = kTopK * A.T;
    for (int i = tid; i <= kE; i += 64 * kRouteWaves) A.offsets[i] = 0;
    for (int i = tid; i < kE; i += 64 * kRouteWaves) {
        int4 *rec = reinterpret_cast<int4 *>(A.slots + 8 * i);
        rec[0] = make_int4(-1, 0, 0, 0);
        rec[1] = make_int4(0, 0, 0, 0);
    }
    for (int a = tid; a < N; a += 64 * kRouteWaves) {
        A.pos[a] = a;
        A.perm[a] = a;
    }
    for (size_t i = tid; i < (size_t)N * kH; i += 64 * kRouteWaves) A.o[i] = __builtin_nanf("");
    if (tid == 0) {
        *A.n_active = 0;
        *A.n_chunks = 0;
        *A.error = 1;
    }
}

// (router.hip is the one translation unit that includes this file)
__global__ __launch_bounds__(64 * kRouteWaves) void k_route_par(RouteSmallArgs A) {
    constexpr int NW = kRouteWaves;
    constexpr int kMaxChunks = kRouteMaxChunks;
    __shared__ int sel[kTopK * kRouteSmallMaxTokens];     // expert of assignment a
    __shared__ int sperm[kTopK * kRouteSmallMaxTokens];   // assignment at sorted position p
    __shared__ int cnt[kMaxChunks][kE];                   // per chunk: count, then base of each expert
    __shared__ int tot[kE];
    __shared__ int offs[kE + 1];
    __shared__ int act_rank[kE];                          // active experts below e (-1: e not active)
    __shared__ int act_list[kE];                          // active expert of each slot
    __shared__ int n_act_s;
    __shared__ int fail;
    const int T = A.T;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int N = kTopK * T;
    const int G = (int)gridDim.x;

    // ---- top-6 of token t: one wave each ----
    const int t = NW * (int)blockIdx.x + wave;
    if (t < T) {
        const float4 lv = reinterpret_cast<const float4 *>(A.logits + (size_t)t * kE)[lane];
        const Top6 r = top6_wave(lv, lane, A.rp);
        const __amdgpu_buffer_rsrc_t ib = make_buf(A.topk_idx, (uint32_t)(4 * N));
#pragma unroll
        for (int j = 0; j < kTopK; ++j) {
            if (lane == j) {
                __builtin_amdgcn_raw_buffer_store_b32(r.e[j], ib, 4 * (kTopK * t + j), 0, kHandOff);
                A.topk_w[(size_t)t * kTopK + j] = r.w[j];
                sel[kTopK * t + j] = r.e[j];
            }
        }
    }
    if (blockIdx.x != 0) {
        // count this workgroup done once every wave's selections are stored
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (wave == 0) count_done(A.counters, lane);
        return;
    }

    // ---- workgroup 0: wait for the other selections, then sort ----
    for (int i = tid; i < kMaxChunks * kE; i += 64 * NW) (&cnt[0][0])[i] = 0;
    if (tid == 0 && A.error_clear) *A.error_clear = 0;
    if (tid == 0) fail = G > 1 && !wait_count(A.counters, G - 1 + A.wait_target_extra, A.wait_ticks);
    __syncthreads();
    if (fail) {
        route_give_up(A, tid);
        return;
    }
    {
        const __amdgpu_buffer_rsrc_t ib = make_buf(A.topk_idx, (uint32_t)(4 * N));
        for (int a = kTopK * NW + tid; a < N; a += 64 * NW)
            sel[a] = (int)__builtin_amdgcn_raw_buffer_load_b32(ib, 4 * a, 0, kHandOff);
    }
    __syncthreads();

    // stable counting sort: chunk c = assignments [64c, 64c + 64) belongs to
    // wave c; equal experts inside a chunk are ranked with ballots, and the
    // counts of earlier chunks and of smaller experts give the base
    const int n_chunks_a = (N + 63) >> 6;
    int e_mine = -1, within = 0;
    if (wave < n_chunks_a) {
        const int a = 64 * wave + lane;
        const bool valid = a < N;
        e_mine = valid ? sel[a] : 0;
        uint64_t same = __ballot(valid);
#pragma unroll
        for (int bit = 0; bit < 8; ++bit) {
            const uint64_t bal = __ballot((e_mine >> bit) & 1);
            same &= ((e_mine >> bit) & 1) ? bal : ~bal;
        }
        const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
        within = __popcll(same & below);
        // the lowest lane of each group of equal experts records the group size
        if (valid && (same & below) == 0) cnt[wave][e_mine] = __popcll(same);
        if (!valid) e_mine = -1;
    }
    __syncthreads();
    // per expert: base of each chunk, total (thread e < 256)
    if (tid < kE) {
        int run = 0;
        for (int c = 0; c < n_chunks_a; ++c) {
            const int v = cnt[c][tid];
            cnt[c][tid] = run;
            run += v;
        }
        tot[tid] = run;
    }
    __syncthreads();
    // exclusive scan of the totals (wave 0, 4 per lane) -> offsets; flags of
    // the non-empty experts -> slot of each active expert
    if (wave == 0) {
        int c4[4], f[4], sc = 0, sf = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            c4[i] = tot[4 * lane + i];
            f[i] = c4[i] > 0;
            sc += c4[i];
            sf += f[i];
        }
        int ic = sc, jf = sf;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int pc = __shfl_up(ic, d, kWave), pf = __shfl_up(jf, d, kWave);
            if (lane >= d) { ic += pc; jf += pf; }
        }
        int ec = ic - sc, ef = jf - sf;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = 4 * lane + i;
            offs[e] = ec;
            A.offsets[e] = ec;
            act_rank[e] = f[i] ? ef : -1;
            ec += c4[i];
            ef += f[i];
        }
        if (lane == 63) {
            offs[kE] = ec;
            A.offsets[kE] = ec;
            *A.n_active = ef;
            *A.n_chunks = ef;
            n_act_s = ef;
        }
    }
    __syncthreads();
    if (e_mine >= 0) {
        const int a = 64 * wave + lane;
        const int dest = offs[e_mine] + cnt[wave][e_mine] + within;
        A.pos[a] = dest;
        A.perm[dest] = a;
        sperm[dest] = a;
    }
    if (tid < kE && act_rank[tid] >= 0) act_list[act_rank[tid]] = tid;
    __syncthreads();
    // slot records {expert, first sorted position, count, first token, second
    // token}, records past n_active hold expert -1; chunks {expert, first
    // position, rows, 0} (rows <= 48 < 96: one chunk per active expert)
    if (tid < kE) {
        int4 *rec = reinterpret_cast<int4 *>(A.slots + 8 * tid);
        if (tid < n_act_s) {
            const int e = act_list[tid], b = offs[e], n = offs[e + 1] - offs[e];
            const int t0 = sperm[b] / kTopK, t1 = n > 1 ? sperm[b + 1] / kTopK : t0;
            rec[0] = make_int4(e, b, n, t0);
            rec[1] = make_int4(t1, 0, 0, 0);
            A.chunks[tid] = make_int4(e, b, n, 0);
        } else {
            rec[0] = make_int4(-1, 0, 0, 0);
            rec[1] = make_int4(0, 0, 0, 0);
        }
    }
}

}  // namespace moe_w4
