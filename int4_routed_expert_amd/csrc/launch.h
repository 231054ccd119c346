// Host-side launchers of the moe_w4 kernels (one per kernel family).
// Every launcher only enqueues on `stream`; the caller checks hipGetLastError.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe_w4 {

// One launch: router logits[T][256] = x R^T (+ bias), and the shared expert's
// h[T][1024] = bf16(silu(x Wsg^T) * (x Wsu^T)); if xt is not null, also the
// rotated fp16 copy of x (xt, xt_scale, as launch_topk_rotate writes them);
// if clear_counters is not null, workgroup 0 clears those counter replicas
// (kFusedCounters of them) for launch_route_par.
void launch_router_and_shared_gateup(const uint16_t *x, int T, const uint16_t *router_w, const float *bias,
                                     float *logits, const uint16_t *shared_w, uint16_t *hs, uint32_t *xt,
                                     float *xt_scale, int *clear_counters, hipStream_t s);

// Decode sizes (1..kFusedMaxTokens tokens): one launch for the router logits
// (it also clears the counters of the launch after it), then the whole rest
// of the layer in one launch (top-6, sort, rotation of x, routed gate/up, the
// shared expert's gate/up, rotation of a, routed and shared down, combine).
constexpr int kFusedMaxTokens = 8;
constexpr int kFusedCounters = 16;        // replicas of each completion counter,
constexpr int kFusedCounterStride = 64;   // one per 256 bytes of `counters`
// bytes of the counters: a done, then h done (16 replicas each)
constexpr int kFusedSyncBytes = 2 * kFusedCounters * kFusedCounterStride * 4;
struct FusedDecodeArgs {
    const uint16_t *x;
    const float *logits;           // without the router bias
    const float *router_bias;      // fp32 [256] or null
    int router_policy;             // MOE_W4_ROUTER_* flags
    const uint8_t *codes;
    const uint16_t *scales;        // int4 experts: bf16 group scales (null for NVFP4)
    const uint8_t *nv_scales;      // NVFP4 experts: E4M3 block scales (null for int4)
    const float *tscales;          // NVFP4 experts: fp32 tensor scales [256][3]
    const uint16_t *shared_gu;     // [2048][2048] bf16: gate rows, then up rows
    const uint16_t *shared_down;   // [2048][1024] bf16
    uint16_t *hs;                  // [T][1024] bf16 scratch: the shared expert's h
    int T;
    int *topk_idx;
    float *topk_w;
    int *offsets;
    int *perm;
    int *pos;
    int *n_active;
    int *slots;
    int4 *chunks;
    int *n_chunks;
    float *act;                    // [6T][512] fp32 scratch, sorted-position order
    uint16_t *y;
    float *resid;                  // stack layer: resid += y (else null)
    int *counters;                 // a done: 4096 bytes, zero at launch (the first launch clears them)
    int *counters_h;               // h done: the next 4096 bytes, likewise
    int *error;                    // set to 1 by a down workgroup whose wait gave up
    int wait_target_extra;         // added to the count the wait needs (0; > 0 only to test the failure path)
    uint32_t wait_ticks;           // bound of the wait, in ticks of the 100 MHz real-time clock
};
// The wait bound and the extra count of the fused launch (process-wide;
// moe_w4_set_fused_wait in the ABI).
void fused_wait_params(uint32_t &ticks, int &extra);
// With resid (a stack layer), x is computed as bf16(rmsnorm(resid)) and also
// written to x_out, and the second launch adds y to resid.  counters:
// kFusedSyncBytes, cleared by this launch; error: the workspace's error word,
// cleared by this launch when non-null.
void launch_router_small(const uint16_t *x, const float *resid, uint16_t *x_out, int T, const uint16_t *router_w,
                         const float *bias, float *logits, int *counters, int *error, hipStream_t s);
void launch_decode_fused(const FusedDecodeArgs &args, hipStream_t s);

// Per token: top-6 of the logits (+ bias, if any), the sigmoid weights
// normalised as the router policy says (bias, policy: MOE_W4_ROUTER_* flags),
// and the Hadamard-rotated fp16 copy of x (with its power-of-two scale).  The
// router launches write the logits without the bias.
// rotate = false: xt gets x itself as natural-order fp16 with the same
// per-token prescale (the operands of the NVFP4 experts' MFMA form).
// hist (or null): the wide sort's int[sort_hist_blocks(T)][256] histograms,
// zero on entry, which the selections are counted into.
void launch_topk_rotate(const float *logits, const uint16_t *x, int T, const float *bias, int policy,
                        int *topk_idx, float *topk_w, uint32_t *xt, float *xt_scale, hipStream_t s,
                        bool rotate = true, int *hist = nullptr);
// Chunks of the MFMA grouped kernels: an expert's sorted assignments are cut
// into chunks of kChunkRows (two 32-row MFMA tiles; the down kernel stages
// 64 rows of A, 64 x 1 KB fitting in LDS twice per CU).  From
// kChunkMaxRowsMinT tokens on, an expert with at most kChunkMaxRows is one
// chunk instead (three tiles; the down kernel takes 65-96 rows in two
// passes): one chunk per expert keeps the number of workgroups at the number
// of touched experts (T = 2048 with uniform routing: 256 chunks, 1024 gate/up
// workgroups, two full rounds of the 512 slots, where 64-row chunks made 261
// and a tail).  Below that size no expert usually passes 64 rows and the
// lighter two-tile kernels are faster.
constexpr int kChunkRows = 64;
constexpr int kChunkMaxRows = 96;
constexpr int kChunkMaxRowsMinT = 1536;
__host__ __device__ constexpr bool chunk_long(int T) { return T >= kChunkMaxRowsMinT; }
// rows between the chunks of an expert with n sorted assignments (T tokens)
__host__ __device__ constexpr int chunk_step(int n, int T) {
    return chunk_long(T) && n <= kChunkMaxRows ? kChunkMaxRows : kChunkRows;
}
__host__ __device__ constexpr int chunk_count(int n, int T) { return (n + chunk_step(n, T) - 1) / chunk_step(n, T); }
// Stable counting sort of the 6T assignments by expert (one workgroup).
// slots: int[256][8] records {expert, first sorted position, count, first
// token, second token, 0, 0, 0}, one per expert with tokens, then expert -1.
// chunks: int[max_chunks(T)][4] records {expert, first sorted position, rows
// (see chunk_step), 0} covering every expert's assignments; *n_chunks of them.
// The same result from many workgroups, for prefill sizes: hist is
// int[sort_hist_blocks(T)][256], the experts' counts per workgroup of 1024
// assignments, which the top-6 launch before it filled (launch_topk_rotate).
int sort_hist_blocks(int T);
void launch_sort_wide(const int *topk_idx, int T, const int *hist, int *offsets, int *perm, int *pos,
                      int *n_active, int *slots, int *chunks, int *n_chunks, int *error, hipStream_t s);
// error (or null): the workspace's error word, cleared (this sequence cannot fail).
void launch_sort(const int *topk_idx, int T, int *offsets, int *perm, int *pos, int *n_active,
                 int *slots, int *chunks, int *n_chunks, int *error, hipStream_t s);
// Top-6 of up to kRouteSmallMaxTokens tokens, one wave per token over
// ceil(T/8) workgroups, handed to workgroup 0, which sorts the assignments
// in LDS (offsets, perm, pos, slot records, chunk list).  counters: replicas
// that the launch before cleared (launch_router_and_shared_gateup);
// error_clear (or null) is cleared; if the hand-off wait gives up after
// wait_ticks of the 100 MHz clock (target raised by wait_target_extra, for
// tests), error is set to 1, no expert is active and o[6T][2048] is NaN.
constexpr int kRouteSmallMaxTokens = 48;
void launch_route_par(const float *logits, int T, const float *bias, int policy, int *topk_idx, float *topk_w,
                      int *offsets, int *perm, int *pos, int *n_active, int *slots, int *chunks, int *n_chunks,
                      float *o, int *counters, int *error_clear, int *error, int wait_target_extra,
                      uint32_t wait_ticks, hipStream_t s);

// Routed experts, GEMV form (few tokens per expert), driven by the slot records.
void launch_gateup_gemv(const uint8_t *codes, const uint16_t *scales, const uint32_t *xt,
                        const float *xt_scale, const int *perm, const int *slots, int T, float *act,
                        hipStream_t s);
// Down projection of a = silu(g)*u (act, fp32, sorted positions); the launch
// itself turns a into rotated fp16 operands (+ per-block power-of-two scales).
void launch_down_gemv(const uint8_t *codes, const uint16_t *scales, const float *act, const int *slots, int T,
                      float *o, hipStream_t s);

// Routed experts, MFMA form (prefill): chunks of <= kChunkMaxRows assignments
// of one expert against tiles of weight rows.  gate/up writes the rotated
// fp16 operands of the down projection directly (at, at_scale).
int max_chunks(int T);
void launch_gateup_mfma(const uint8_t *codes, const uint16_t *scales, const uint32_t *xt, const float *xt_scale,
                        const int *perm, const int *chunks, const int *n_chunks, int T, uint32_t *at,
                        float *at_scale, hipStream_t s);
// o: fp16 rows [6T][2048]; o_scale: fp32 [6T], the multiplier of each row.
void launch_down_mfma(const uint8_t *codes, const uint16_t *scales, const uint32_t *at, const float *at_scale,
                      const int *chunks, const int *n_chunks, int T, uint16_t *o, float *o_scale, hipStream_t s);

// The same two kernels for NVFP4 experts (E2M1 codes, E4M3 scales per 16 of
// K, fp32 tensor scales [256][3]; original basis): xn, xn_scale are x as
// natural-order fp16 with a per-token prescale (launch_topk_rotate with rotate
// = false); gate/up writes a (an, an_scale) in natural order without a
// rotation; down writes fp32 rows o [6T][2048].
void launch_gateup_mfma_nvfp4(const uint8_t *codes, const uint8_t *scales, const float *tscales, const uint32_t *xn,
                              const float *xn_scale, const int *perm, const int *chunks, const int *n_chunks, int T,
                              uint32_t *an, float *an_scale, hipStream_t s);
void launch_down_mfma_nvfp4(const uint8_t *codes, const uint8_t *scales, const float *tscales, const uint32_t *an,
                            const float *an_scale, const int *chunks, const int *n_chunks, int T, float *o,
                            hipStream_t s);

// Shared expert down projection fused with the combine:
// y = bf16(h Wsd^T + sum_j w_j o[pos[6t+j]]), slots in order.
void launch_shared_down_combine(const uint16_t *shared_w, const uint16_t *hs, int T, const float *topk_w,
                                const int *pos, const float *o, uint16_t *y, hipStream_t s);

// The same two launches for many tokens (prefill sizes): LDS-tiled MFMA GEMMs.
// clear (or null): n_clear ints zeroed by the launch (the wide sort's
// histograms, which the top-6 launch after it counts into).
void launch_router_and_shared_gateup_dense(const uint16_t *x, int T, const uint16_t *router_w, const float *bias,
                                           float *logits, const uint16_t *shared_w, uint16_t *hs, hipStream_t s,
                                           int *clear = nullptr, int n_clear = 0);
// shared down projection z = h Wsd^T (fp32), then the combine as its own pass
void launch_shared_down_dense(const uint16_t *shared_w, const uint16_t *hs, int T, float *z, hipStream_t s);
void launch_combine(const float *z, const float *topk_w, const int *pos, const float *o, int T, uint16_t *y,
                    hipStream_t s);
// the same with fp16 rows o times o_scale[row] (the grouped down kernel's output)
void launch_combine_half(const float *z, const float *topk_w, const int *pos, const uint16_t *o,
                         const float *o_scale, int T, uint16_t *y, hipStream_t s);

// The packer: n_experts experts of bf16 weights (gate [512][2048], up
// [512][2048], down [2048][512] each) -> int4 codes and bf16 scales in the
// library layout (fwht128 on K, scale = bf16(absmax / 7) per 128-group).
void launch_pack_experts(const uint16_t *w, int64_t n_experts, uint8_t *codes, uint16_t *scales, hipStream_t s);

// Dense SwiGLU MLP block (width kDenseInter): w = bf16 gate [6144][2048], up
// [6144][2048], down [2048][6144]; h bf16 [T][6144]; y bf16 [T][2048].  Skinny
// kernels below kPrefillMinTokens tokens, LDS-tiled MFMA GEMMs from there on.
void launch_dense_mlp_gateup_skinny(const uint16_t *x, int T, const uint16_t *w, uint16_t *h, hipStream_t s);
void launch_dense_mlp_down_skinny(const uint16_t *w, const uint16_t *h, int T, uint16_t *y, hipStream_t s);
void launch_dense_mlp_gateup_dense(const uint16_t *x, int T, const uint16_t *w, uint16_t *h, hipStream_t s);
void launch_dense_mlp_down_dense(const uint16_t *w, const uint16_t *h, int T, uint16_t *y, hipStream_t s);

// Routed experts in the NVFP4 container (E2M1 codes, E4M3 scales per 16 of
// K, fp32 tensor scales [256][3]; original basis), GEMV form at every token
// count, driven by the slot records: gate/up writes a = silu(g) * u (fp32,
// sorted positions); down reads it and writes the expert rows o.
void launch_gateup_nvfp4(const uint8_t *codes, const uint8_t *scales, const float *tscales, const uint16_t *x,
                         const int *perm, const int *slots, int T, float *act, hipStream_t s);
void launch_down_nvfp4(const uint8_t *codes, const uint8_t *scales, const float *tscales, const float *act,
                       const int *slots, int T, float *o, hipStream_t s);

// Stack glue: x_bf16 = bf16(rmsnorm(resid)); resid += f32(y).
void launch_rmsnorm_bf16(const float *resid, int T, uint16_t *x, hipStream_t s);
void launch_residual_add(float *resid, const uint16_t *y, int T, hipStream_t s);

// Seeded generator.
void launch_gen_normal_bf16(uint64_t key, int64_t n, float mult, int absval, uint16_t *out, hipStream_t s);
void launch_gen_codes(uint64_t key, int rows, int k, int experts, int64_t expert_elems,
                      int64_t expert_stride_bytes, uint8_t *out, hipStream_t s);
void launch_gen_scales(uint64_t key, int groups_per_row, int rows, int experts, int64_t expert_stride,
                       float mult, uint16_t *out, hipStream_t s);

}  // namespace moe_w4
