// Top-6 and the stable token->expert sort of a few tokens (up to
// kRouteSmallMaxTokens) in one workgroup of NW waves: wave w selects tokens
// w, w + NW, ... (all their logit loads issued first; model card, introduction:
// 256 experts, top-6; weights sigmoid / max(sum, 2^-14), bloomery issue #632,
// design thread); then a stable counting sort of the <= 288 assignments in LDS
// (the algorithm of k_sort, with the chosen experts never leaving the
// workgroup).  Used by the routing launch and by the launch that routes beside
// the shared expert's gate/up.
#pragma once

#include "common.h"
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
    int *error;            // cleared (this launch sequence cannot fail), or null
};

template <int NW>
__device__ __forceinline__ void route_small_block(const RouteSmallArgs &A) {
    constexpr int kPerWave = (kRouteSmallMaxTokens + NW - 1) / NW;
    constexpr int kMaxChunks = (kTopK * kRouteSmallMaxTokens + 63) / 64;
    static_assert(NW >= kMaxChunks, "one wave per 64 assignments in the ranking");
    __shared__ int sel[kTopK * kRouteSmallMaxTokens];     // expert of assignment a
    __shared__ int sperm[kTopK * kRouteSmallMaxTokens];   // assignment at sorted position p
    __shared__ int cnt[kMaxChunks][kE];                   // per chunk: count, then base of each expert
    __shared__ int tot[kE];
    __shared__ int offs[kE + 1];
    __shared__ int act_rank[kE];                          // active experts below e (-1: e not active)
    __shared__ int act_list[kE];                          // active expert of each slot
    __shared__ int n_act_s;
    const int T = A.T;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int N = kTopK * T;
    for (int i = tid; i < kMaxChunks * kE; i += 64 * NW) (&cnt[0][0])[i] = 0;
    if (tid == 0 && A.error) *A.error = 0;

    float4 lv[kPerWave];
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
        const int t = min(wave + NW * i, T - 1);   // past the end: token T-1 again (unused)
        lv[i] = reinterpret_cast<const float4 *>(A.logits + (size_t)t * kE)[lane];
    }
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
        const int t = wave + NW * i;
        if (t < T) {
            const Top6 r = top6_wave(lv[i], lane, A.rp);
#pragma unroll
            for (int j = 0; j < kTopK; ++j) {
                if (lane == j) {
                    A.topk_idx[(size_t)t * kTopK + j] = r.e[j];
                    A.topk_w[(size_t)t * kTopK + j] = r.w[j];
                    sel[kTopK * t + j] = r.e[j];
                }
            }
        }
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
