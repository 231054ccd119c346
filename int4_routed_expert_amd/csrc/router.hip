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
#include "route_small.h"
#include "token_ops.h"

namespace moe_w4 {

constexpr int kSortWaves = 16;
constexpr int kSortWgAssign = kSortWaves * 64;   // assignments per workgroup of the wide sort

// ROTATE: xt gets the fwht128-rotated x in the int4 experts' operand order;
// otherwise x itself as natural-order fp16 (the NVFP4 experts' operands).
template <bool ROTATE>
__global__ __launch_bounds__(512) void k_topk_rotate(const float *__restrict__ logits,
                                                     const uint16_t *__restrict__ x, int T,
                                                     int *__restrict__ topk_idx,
                                                     float *__restrict__ topk_w,
                                                     uint32_t *__restrict__ xt,
                                                     float *__restrict__ xt_scale, RouterPolicy rp,
                                                     int *__restrict__ hist) {
    // two waves per token, side by side: waves 0-3 select the top-6 of tokens
    // 4b .. 4b+3, waves 4-7 turn the same tokens' x into operands (the two
    // are independent; one wave doing both ran the chains back to back)
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (wave & 3);
    if (t >= T) return;
    if (wave < 4) {
        const float4 lv = reinterpret_cast<const float4 *>(logits + (size_t)t * kE)[lane];
        const Top6 sel = top6_wave(lv, lane, rp);
#pragma unroll
        for (int j = 0; j < kTopK; ++j) {
            if (lane == j) {
                topk_idx[(size_t)t * kTopK + j] = sel.e[j];
                topk_w[(size_t)t * kTopK + j] = sel.w[j];
                // the wide sort's count of expert e in the workgroup of
                // assignment 6t + j (a sum: the order of the adds is free)
                if (hist) atomicAdd(&hist[(size_t)((kTopK * t + j) / kSortWgAssign) * kE + sel.e[j]], 1);
            }
        }
        return;
    }
    uint4 xq[4];
    const uint4 *xp = reinterpret_cast<const uint4 *>(x + (size_t)t * kH + lane * 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) xq[i] = xp[i];
    const int sh = ROTATE ? rotate_x_wave(xq, lane, xt + (size_t)t * (kH / 2) + lane * 16)
                          : natural_x_wave(xq, lane, xt + (size_t)t * (kH / 2) + lane * 16);
    if (lane == 0) xt_scale[t] = ldexpf(1.0f, sh);
}

void launch_topk_rotate(const float *logits, const uint16_t *x, int T, const float *bias, int policy,
                        int *topk_idx, float *topk_w, uint32_t *xt, float *xt_scale, hipStream_t s, bool rotate,
                        int *hist) {
    if (rotate)
        hipLaunchKernelGGL(k_topk_rotate<true>, dim3((T + 3) / 4), dim3(512), 0, s, logits, x, T, topk_idx, topk_w,
                           xt, xt_scale, RouterPolicy{bias, policy}, hist);
    else
        hipLaunchKernelGGL(k_topk_rotate<false>, dim3((T + 3) / 4), dim3(512), 0, s, logits, x, T, topk_idx,
                           topk_w, xt, xt_scale, RouterPolicy{bias, policy}, hist);
}

// ---------------------------------------------------------------------------
// Stable counting sort of the assignments a = 6t + j by expert, in one
// workgroup of 16 waves.  Wave w owns a contiguous range of assignments.
//   1. per-wave histograms;  2. per-(wave, expert) bases = expert offset +
//   counts of earlier waves;  3. each wave walks its range in order, 64 at a
//   time, ranking equal experts inside the chunk with ballots.
// The result depends only on topk_idx: offsets, perm and pos are exact.
// ---------------------------------------------------------------------------
constexpr int kSortBatch = 8;        // chunks of 64 assignments whose loads are issued together
constexpr int kSortKeep = 16;        // chunks per wave kept in registers between the two passes

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
        // flags and of the chunk counts (chunk_count)
        int c[4], f[4], k[4], sc = 0, sf = 0, sk = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            c[i] = tot[4 * lane + i];
            f[i] = c[i] > 0;
            k[i] = chunk_count(c[i], T);
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
        for (int r = 0, q = chunk0[tid], st = chunk_step(n, T); r < n; r += st, ++q)
            chunks[q] = make_int4(tid, offs[tid] + r, min(st, n - r), 0);
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
// The same stable counting sort spread over many workgroups (prefill sizes):
// workgroup b owns assignments [1024 b, 1024 b + 1024), wave w of it the 64
// from 1024 b + 64 w.
//   1. the top-6 launch before it adds each selection into the histogram of
//      its workgroup over the experts, hist[b][e] (zeroed by the launch before
//      that; a sum, so the order of the adds is free).
//   2. k_sort_place: every workgroup reads all histograms: per expert the
//      total (-> offsets) and the counts of the workgroups before it (its base
//      inside the expert); inside the workgroup, per-wave counts and ballots
//      rank its assignments exactly as k_sort does.  Workgroup 0 writes the
//      offsets, the chunk list and the slot records; the workgroup that places
//      an expert's first (second) sorted assignment writes its first (second)
//      token into the expert's record.
// The result is that of k_sort bit for bit: stable in the assignment index.
// ---------------------------------------------------------------------------

int sort_hist_blocks(int T) { return (kTopK * T + kSortWgAssign - 1) / kSortWgAssign; }

__global__ __launch_bounds__(1024) void k_sort_place(const int *__restrict__ topk_idx, int N, int nb,
                                                     const int *__restrict__ hist, int *__restrict__ offsets,
                                                     int *__restrict__ perm, int *__restrict__ pos,
                                                     int *__restrict__ n_active, int *__restrict__ slots,
                                                     int4 *__restrict__ chunks, int *__restrict__ n_chunks,
                                                     int *__restrict__ error) {
    __shared__ int cnt[kSortWaves][kE];   // per wave: count, then base of each expert
    __shared__ int base[kE];              // this workgroup's first sorted position of each expert
    __shared__ int tot[kE];
    __shared__ int offs[kE + 1];
    __shared__ int act_rank[kE];          // active experts below e (-1: e not active)
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int b = blockIdx.x;
    for (int i = tid; i < kSortWaves * kE; i += blockDim.x) (&cnt[0][0])[i] = 0;
    if (b == 0 && tid == 0 && error) *error = 0;   // this launch sequence cannot fail on the device
    // this thread's assignment and the histograms of every workgroup (thread e < 256)
    const int a = b * kSortWgAssign + tid;
    const bool valid = a < N;
    const int e_mine = valid ? topk_idx[a] : 0;
    if (tid < kE) {
        int before = 0, total = 0;
        for (int k = 0; k < nb; ++k) {
            const int c = hist[(size_t)k * kE + tid];
            before += k < b ? c : 0;
            total += c;
        }
        base[tid] = before;
        tot[tid] = total;
    }
    __syncthreads();
    if (valid) atomicAdd(&cnt[wave][e_mine], 1);
    // exclusive scans of the totals (offsets), of the non-empty flags (slot
    // of each active expert) and of the chunk counts (wave 0, 4 per lane)
    if (wave == 0) {
        int c[4], f[4], k[4], sc = 0, sf = 0, sk = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            c[i] = tot[4 * lane + i];
            f[i] = c[i] > 0;
            k[i] = chunk_count(c[i], N / kTopK);
            sc += c[i];
            sf += f[i];
            sk += k[i];
        }
        int ic = sc, jf = sf, jk = sk;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int pc = __shfl_up(ic, d, kWave), pf = __shfl_up(jf, d, kWave), pk = __shfl_up(jk, d, kWave);
            if (lane >= d) { ic += pc; jf += pf; jk += pk; }
        }
        int ec = ic - sc, ef = jf - sf, ek = jk - sk;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = 4 * lane + i;
            offs[e] = ec;
            act_rank[e] = f[i] ? ef : -1;
            if (b == 0) {
                offsets[e] = ec;
                if (f[i]) {
                    // the expert's record (its tokens are written where they are placed)
                    int *rec = slots + 8 * ef;
                    rec[0] = e;
                    rec[1] = ec;
                    rec[2] = c[i];
                    rec[5] = 0;
                    rec[6] = 0;
                    rec[7] = 0;
                }
                for (int r = 0, q = ek, st = chunk_step(c[i], N / kTopK); r < c[i]; r += st, ++q)
                    chunks[q] = make_int4(e, ec + r, min(st, c[i] - r), 0);
            }
            ec += c[i];
            ef += f[i];
            ek += k[i];
        }
        if (lane == 63) {
            offs[kE] = ec;
            if (b == 0) {
                offsets[kE] = ec;
                *n_active = ef;
                *n_chunks = ek;
            }
        }
        // records past the active experts
        if (b == 0) {
            const int n_act = __shfl(jf, 63, kWave);
            for (int r = n_act + lane; r < kE; r += kWave) {
                int4 *rec = reinterpret_cast<int4 *>(slots + 8 * r);
                rec[0] = make_int4(-1, 0, 0, 0);
                rec[1] = make_int4(0, 0, 0, 0);
            }
        }
    }
    __syncthreads();
    // per-wave bases: offset of the expert + this workgroup's base + the counts
    // of the earlier waves of the workgroup (thread e < 256)
    if (tid < kE) {
        int run = offs[tid] + base[tid];
        for (int w = 0; w < kSortWaves; ++w) {
            const int c = cnt[w][tid];
            cnt[w][tid] = run;
            run += c;
        }
    }
    __syncthreads();
    // stable rank inside the wave's 64 assignments: equal experts ranked by
    // lane through the ballots of the expert's bits
    uint64_t same = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
        const uint64_t bal = __ballot((e_mine >> bit) & 1);
        same &= ((e_mine >> bit) & 1) ? bal : ~bal;
    }
    if (valid) {
        const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
        const int dest = cnt[wave][e_mine] + __popcll(same & below);
        perm[dest] = a;
        pos[a] = dest;
        // the expert's first and second tokens into its record
        const int r = dest - offs[e_mine];
        const int n_e = offs[e_mine + 1] - offs[e_mine];
        int *rec = slots + 8 * act_rank[e_mine];
        if (r == 0) {
            rec[3] = a / kTopK;
            if (n_e == 1) rec[4] = a / kTopK;
        } else if (r == 1) {
            rec[4] = a / kTopK;
        }
    }
}

// Top-6 and sort of a few tokens (up to kRouteSmallMaxTokens): one wave per
// token, then workgroup 0 sorts (route_small.h).
void launch_route_par(const float *logits, int T, const float *bias, int policy, int *topk_idx, float *topk_w,
                      int *offsets, int *perm, int *pos, int *n_active, int *slots, int *chunks, int *n_chunks,
                      float *o, int *counters, int *error_clear, int *error, int wait_target_extra,
                      uint32_t wait_ticks, hipStream_t s) {
    const RouteSmallArgs A{logits, T, RouterPolicy{bias, policy}, topk_idx, topk_w, offsets, perm, pos, n_active,
                           slots, reinterpret_cast<int4 *>(chunks), n_chunks, error_clear, error, o, counters,
                           wait_target_extra, wait_ticks};
    hipLaunchKernelGGL(k_route_par, dim3((T + kRouteWaves - 1) / kRouteWaves), dim3(64 * kRouteWaves), 0, s, A);
}

void launch_sort_wide(const int *topk_idx, int T, const int *hist, int *offsets, int *perm, int *pos,
                      int *n_active, int *slots, int *chunks, int *n_chunks, int *error, hipStream_t s) {
    const int nb = sort_hist_blocks(T), N = kTopK * T;
    hipLaunchKernelGGL(k_sort_place, dim3(nb), dim3(1024), 0, s, topk_idx, N, nb, hist, offsets, perm, pos, n_active,
                       slots, reinterpret_cast<int4 *>(chunks), n_chunks, error);
}

void launch_sort(const int *topk_idx, int T, int *offsets, int *perm, int *pos, int *n_active,
                 int *slots, int *chunks, int *n_chunks, int *error, hipStream_t s) {
    hipLaunchKernelGGL(k_sort, dim3(1), dim3(1024), 0, s, topk_idx, T, offsets, perm, pos, n_active,
                       slots, reinterpret_cast<int4 *>(chunks), n_chunks, error);
}

}  // namespace moe_w4
