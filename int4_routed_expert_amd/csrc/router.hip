// Router (sigmoid, top-6, renormalised with a 2^-14 floor), rotation of x,
// and the stable token->expert counting sort.
//
// Follows: bloomery issue #632 ("model: Flint ..."), design thread — unbiased
// sigmoid router over 256 experts, top-6, weights = score / max(sum, 2^-14),
// six (index, fp32 weight) slots per token; NInfer README of Flint, section
// "What is inside" — router rows are bf16 widened exactly to fp32; Flint
// model card (Aijuus/flint-w4exp), table row "weights" — experts are stored in
// a fwht128-rotated basis, so x is rotated per 128-block before the experts.
#include "common.h"
#include "launch.h"
#include "token_ops.h"

namespace moe_w4 {

__global__ __launch_bounds__(256) void k_topk_rotate(const float *__restrict__ logits,
                                                     const uint16_t *__restrict__ x, int T,
                                                     int *__restrict__ topk_idx,
                                                     float *__restrict__ topk_w,
                                                     uint32_t *__restrict__ xt,
                                                     float *__restrict__ xt_scale, RouterPolicy rp) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + wave;
    if (t >= T) return;

    // x is independent of the logits: its loads go out first, so the two
    // memory round trips overlap
    uint4 xq[4];
    {
        const uint4 *xp = reinterpret_cast<const uint4 *>(x + (size_t)t * kH + lane * 32);
#pragma unroll
        for (int i = 0; i < 4; ++i) xq[i] = xp[i];
    }
    const float4 lv = reinterpret_cast<const float4 *>(logits + (size_t)t * kE)[lane];
    const Top6 sel = top6_wave(lv, lane, rp);
#pragma unroll
    for (int j = 0; j < kTopK; ++j) {
        if (lane == j) {
            topk_idx[(size_t)t * kTopK + j] = sel.e[j];
            topk_w[(size_t)t * kTopK + j] = sel.w[j];
        }
    }
    const int sh = rotate_x_wave(xq, lane, xt + (size_t)t * (kH / 2) + lane * 16);
    if (lane == 0) xt_scale[t] = ldexpf(1.0f, sh);
}

void launch_topk_rotate(const float *logits, const uint16_t *x, int T, const float *bias, int policy,
                        int *topk_idx, float *topk_w, uint32_t *xt, float *xt_scale, hipStream_t s) {
    hipLaunchKernelGGL(k_topk_rotate, dim3((T + 3) / 4), dim3(256), 0, s, logits, x, T, topk_idx,
                       topk_w, xt, xt_scale, RouterPolicy{bias, policy});
}

// ---------------------------------------------------------------------------
// Stable counting sort of the assignments a = 6t + j by expert, in one
// workgroup of 16 waves.  Wave w owns a contiguous range of assignments.
//   1. per-wave histograms;  2. per-(wave, expert) bases = expert offset +
//   counts of earlier waves;  3. each wave walks its range in order, 64 at a
//   time, ranking equal experts inside the chunk with ballots.
// The result depends only on topk_idx: offsets, perm and pos are exact.
// ---------------------------------------------------------------------------
constexpr int kSortWaves = 16;
constexpr int kSortBatch = 8;        // chunks of 64 assignments whose loads are issued together
constexpr int kSortKeep = 16;        // chunks per wave kept in registers between the two passes
constexpr int kSortChunkRows = 96;   // rows of one chunk of the MFMA grouped kernels

__global__ __launch_bounds__(1024) void k_sort(const int *__restrict__ topk_idx, int T,
                                               int *__restrict__ offsets, int *__restrict__ perm,
                                               int *__restrict__ pos, int *__restrict__ n_active,
                                               int *__restrict__ slots, int4 *__restrict__ chunks,
                                               int *__restrict__ n_chunks, int *__restrict__ error) {
    __shared__ int cnt[kSortWaves][kE];
    __shared__ int tot[kE];
    __shared__ int offs[kE + 1];
    __shared__ int first2[kE][2];   // tokens at the first two sorted positions of each expert
    __shared__ int slot_e[kE + 1];  // expert of each active slot; [kE] = number of slots
    __shared__ int chunk0[kE];      // first chunk of each expert
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int N = kTopK * T;
    const int per = ((N + kSortWaves * 64 - 1) / (kSortWaves * 64)) * 64;
    const int a0 = wave * per, a1 = min(a0 + per, N);

    for (int i = tid; i < kSortWaves * kE; i += blockDim.x) (&cnt[0][0])[i] = 0;
    if (tid == 0 && error) *error = 0;   // this launch sequence cannot fail on the device
    // up to kSortKeep chunks of 64 per wave (6 * T <= 16384) are loaded once,
    // all in flight together, and stay in registers for the ranking pass
    const bool keep = per <= 64 * kSortKeep;
    int kv[kSortKeep];
    if (keep) {
#pragma unroll
        for (int u = 0; u < kSortKeep; ++u) {
            const int a = a0 + 64 * u + lane;
            kv[u] = a < a1 ? topk_idx[a] : -1;
        }
    }
    __syncthreads();
    if (keep) {
#pragma unroll
        for (int u = 0; u < kSortKeep; ++u)
            if (kv[u] >= 0) atomicAdd(&cnt[wave][kv[u]], 1);
    }
    // otherwise the wave's assignments are read kSortBatch chunks of 64 at a
    // time, all loads of a batch in flight together
    for (int c0 = a0; !keep && c0 < a1; c0 += 64 * kSortBatch) {
        int ev[kSortBatch];
#pragma unroll
        for (int u = 0; u < kSortBatch; ++u) {
            const int a = c0 + 64 * u + lane;
            ev[u] = a < a1 ? topk_idx[a] : -1;
        }
#pragma unroll
        for (int u = 0; u < kSortBatch; ++u)
            if (ev[u] >= 0) atomicAdd(&cnt[wave][ev[u]], 1);
    }
    __syncthreads();
    if (tid < kE) {
        int run = 0;
        for (int w = 0; w < kSortWaves; ++w) {
            const int c = cnt[w][tid];
            cnt[w][tid] = run;   // becomes the wave's base inside the expert
            run += c;
        }
        tot[tid] = run;
    }
    __syncthreads();
    if (wave == 0) {
        // exclusive scans of the 256 totals (4 per lane), of the non-empty
        // flags and of the chunk counts (kChunkRows assignments per chunk)
        int c[4], f[4], k[4], sc = 0, sf = 0, sk = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            c[i] = tot[4 * lane + i];
            f[i] = c[i] > 0;
            k[i] = (c[i] + kSortChunkRows - 1) / kSortChunkRows;
            sc += c[i];
            sf += f[i];
            sk += k[i];
        }
        int ic = sc, jf = sf, jk = sk;   // inclusive scans over lanes
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int pc = __shfl_up(ic, d, kWave);
            const int pf = __shfl_up(jf, d, kWave);
            const int pk = __shfl_up(jk, d, kWave);
            if (lane >= d) { ic += pc; jf += pf; jk += pk; }
        }
        int ec = ic - sc, ef = jf - sf, ek = jk - sk;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = 4 * lane + i;
            offs[e] = ec;
            offsets[e] = ec;
            chunk0[e] = ek;
            if (f[i]) slot_e[ef] = e;
            ec += c[i];
            ef += f[i];
            ek += k[i];
        }
        if (lane == 63) {
            offs[kE] = ec;
            offsets[kE] = ec;
            *n_active = ef;
            *n_chunks = ek;
            slot_e[kE] = ef;
        }
    }
    __syncthreads();
    for (int i = tid; i < kSortWaves * kE; i += blockDim.x) (&cnt[0][0])[i] += offs[i % kE];
    // chunk list of the MFMA grouped path: {expert, first sorted position, rows, 0}
    if (tid < kE) {
        const int n = tot[tid];
        for (int r = 0, q = chunk0[tid]; r < n; r += kSortChunkRows, ++q)
            chunks[q] = make_int4(tid, offs[tid] + r, min(kSortChunkRows, n - r), 0);
    }
    __syncthreads();
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    // stable rank of each assignment of chunk [c0, c0 + 64) (expert e) in its expert
    auto rank_chunk = [&](int c0, int e) {
        const int a = c0 + lane;
        const bool valid = a < a1;
        uint64_t same = __ballot(valid);
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const uint64_t bal = __ballot((e >> b) & 1);
            same &= ((e >> b) & 1) ? bal : ~bal;
        }
        if (valid) {
            const int base = cnt[wave][e];
            const int dest = base + __popcll(same & below);
            perm[dest] = a;
            pos[a] = dest;
            if (dest - offs[e] < 2) first2[e][dest - offs[e]] = a / kTopK;
            if ((same >> lane) == 1ull) cnt[wave][e] = base + __popcll(same);
        }
    };
    if (keep) {
#pragma unroll
        for (int u = 0; u < kSortKeep; ++u) {
            if (a0 + 64 * u >= a1) break;
            rank_chunk(a0 + 64 * u, kv[u] < 0 ? 0 : kv[u]);
        }
    }
    for (int cb = a0; !keep && cb < a1; cb += 64 * kSortBatch) {
        int ev[kSortBatch];
#pragma unroll
        for (int u = 0; u < kSortBatch; ++u) {
            const int a = cb + 64 * u + lane;
            ev[u] = a < a1 ? topk_idx[a] : 0;
        }
#pragma unroll
        for (int u = 0; u < kSortBatch; ++u) {
            if (cb + 64 * u >= a1) break;
            rank_chunk(cb + 64 * u, ev[u]);
        }
    }
    __syncthreads();
    // One 32-byte record per active slot, so a grouped kernel gets its expert,
    // token range and first two tokens with a single scalar load; slots past
    // n_active hold expert -1.
    if (tid < kE) {
        int4 *rec = reinterpret_cast<int4 *>(slots + 8 * tid);
        if (tid < slot_e[kE]) {
            const int e = slot_e[tid];
            const int n = offs[e + 1] - offs[e];
            rec[0] = make_int4(e, offs[e], n, first2[e][0]);
            rec[1] = make_int4(n > 1 ? first2[e][1] : first2[e][0], 0, 0, 0);
        } else {
            rec[0] = make_int4(-1, 0, 0, 0);
            rec[1] = make_int4(0, 0, 0, 0);
        }
    }
}

// ---------------------------------------------------------------------------
// Top-6 and sort of a few tokens (up to kRouteSmallMaxTokens) in one
// workgroup of 16 waves: wave w selects tokens w, w + 16, ... (all their logit
// loads issued first); then a stable counting sort of the <= 288 assignments
// in LDS (the algorithm of k_sort, with the chosen experts never leaving the
// workgroup).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void k_route_small(const float *__restrict__ logits, int T,
                                                      int *__restrict__ topk_idx, float *__restrict__ topk_w,
                                                      int *__restrict__ offsets, int *__restrict__ perm,
                                                      int *__restrict__ pos, int *__restrict__ n_active,
                                                      int *__restrict__ slots, int4 *__restrict__ chunks,
                                                      int *__restrict__ n_chunks, int *__restrict__ error,
                                                      RouterPolicy rp) {
    constexpr int kPerWave = (kRouteSmallMaxTokens + kSortWaves - 1) / kSortWaves;
    constexpr int kMaxChunks = (kTopK * kRouteSmallMaxTokens + 63) / 64;
    __shared__ int sel[kTopK * kRouteSmallMaxTokens];     // expert of assignment a
    __shared__ int sperm[kTopK * kRouteSmallMaxTokens];   // assignment at sorted position p
    __shared__ int cnt[kMaxChunks][kE];                   // per chunk: count, then base of each expert
    __shared__ int tot[kE];
    __shared__ int offs[kE + 1];
    __shared__ int act_rank[kE];                          // active experts below e (-1: e not active)
    __shared__ int act_list[kE];                          // active expert of each slot
    __shared__ int n_act_s;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int N = kTopK * T;
    for (int i = tid; i < kMaxChunks * kE; i += blockDim.x) (&cnt[0][0])[i] = 0;
    if (tid == 0 && error) *error = 0;   // this launch sequence cannot fail on the device

    float4 lv[kPerWave];
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
        const int t = min(wave + kSortWaves * i, T - 1);   // past the end: token T-1 again (unused)
        lv[i] = reinterpret_cast<const float4 *>(logits + (size_t)t * kE)[lane];
    }
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
        const int t = wave + kSortWaves * i;
        if (t < T) {
            const Top6 r = top6_wave(lv[i], lane, rp);
#pragma unroll
            for (int j = 0; j < kTopK; ++j) {
                if (lane == j) {
                    topk_idx[(size_t)t * kTopK + j] = r.e[j];
                    topk_w[(size_t)t * kTopK + j] = r.w[j];
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
            offsets[e] = ec;
            act_rank[e] = f[i] ? ef : -1;
            ec += c4[i];
            ef += f[i];
        }
        if (lane == 63) {
            offs[kE] = ec;
            offsets[kE] = ec;
            *n_active = ef;
            *n_chunks = ef;
            n_act_s = ef;
        }
    }
    __syncthreads();
    if (e_mine >= 0) {
        const int a = 64 * wave + lane;
        const int dest = offs[e_mine] + cnt[wave][e_mine] + within;
        pos[a] = dest;
        perm[dest] = a;
        sperm[dest] = a;
    }
    if (tid < kE && act_rank[tid] >= 0) act_list[act_rank[tid]] = tid;
    __syncthreads();
    // slot records {expert, first sorted position, count, first token, second
    // token}, records past n_active hold expert -1; chunks {expert, first
    // position, rows, 0} (rows <= 48 < 96: one chunk per active expert)
    if (tid < kE) {
        int4 *rec = reinterpret_cast<int4 *>(slots + 8 * tid);
        if (tid < n_act_s) {
            const int e = act_list[tid], b = offs[e], n = offs[e + 1] - offs[e];
            const int t0 = sperm[b] / kTopK, t1 = n > 1 ? sperm[b + 1] / kTopK : t0;
            rec[0] = make_int4(e, b, n, t0);
            rec[1] = make_int4(t1, 0, 0, 0);
            chunks[tid] = make_int4(e, b, n, 0);
        } else {
            rec[0] = make_int4(-1, 0, 0, 0);
            rec[1] = make_int4(0, 0, 0, 0);
        }
    }
}

void launch_route_small(const float *logits, int T, const float *bias, int policy, int *topk_idx, float *topk_w,
                        int *offsets, int *perm, int *pos, int *n_active, int *slots, int *chunks, int *n_chunks,
                        int *error, hipStream_t s) {
    hipLaunchKernelGGL(k_route_small, dim3(1), dim3(1024), 0, s, logits, T, topk_idx, topk_w, offsets, perm, pos,
                       n_active, slots, reinterpret_cast<int4 *>(chunks), n_chunks, error, RouterPolicy{bias, policy});
}

void launch_sort(const int *topk_idx, int T, int *offsets, int *perm, int *pos, int *n_active,
                 int *slots, int *chunks, int *n_chunks, int *error, hipStream_t s) {
    hipLaunchKernelGGL(k_sort, dim3(1), dim3(1024), 0, s, topk_idx, T, offsets, perm, pos, n_active,
                       slots, reinterpret_cast<int4 *>(chunks), n_chunks, error);
}

}  // namespace moe_w4
