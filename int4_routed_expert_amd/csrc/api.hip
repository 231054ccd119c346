// C ABI of the moe_w4 library: validation, workspace layout, launch order.
// The declarations and their contracts are in include/moe_w4.h.
#include <math.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "common.h"
#include "launch.h"
#include "moe_w4.h"
#include "token_ops.h"

static_assert(MOE_W4_EXPERT_WEIGHTS == 2 * moe_w4::kCodeBytesPerExpert, "two int4 codes per byte");
static_assert(MOE_W4_NVFP4_CODE_BYTES == moe_w4::kCodeBytesPerExpert &&
                  MOE_W4_NVFP4_SCALE_BYTES == 3 * moe_w4::kI * moe_w4::kH / 16,
              "NVFP4 expert layout");
static_assert(MOE_W4_DENSE_INTER == moe_w4::kDenseInter && MOE_W4_DENSE_WEIGHTS == 3 * moe_w4::kDenseInter * moe_w4::kH,
              "dense MLP shape");
static_assert(MOE_W4_ROUTER_NORM_FLOOR == moe_w4::kNormFloor && MOE_W4_ROUTER_NORM_SUM == moe_w4::kNormSum &&
                  MOE_W4_ROUTER_NORM_NONE == moe_w4::kNormNone &&
                  MOE_W4_ROUTER_BIAS_SELECT_ONLY == moe_w4::kBiasSelectOnly,
              "router policy flags of the header and the kernels agree");

using namespace moe_w4;

namespace {

thread_local int g_last_device_error = 0;

// Diagnostics of the two-launch form's bounded wait (moe_w4_set_fused_wait).
constexpr uint32_t kDefaultWaitTicks = 500000;   // 5 ms of the 100 MHz real-time clock
std::atomic<uint32_t> g_wait_ticks{kDefaultWaitTicks};
std::atomic<int> g_wait_extra{0};

constexpr size_t kAlignWs = 256;
size_t align_up(size_t v) { return (v + kAlignWs - 1) & ~(kAlignWs - 1); }

bool t_in_range(int64_t T) { return T >= 0 && T <= MOE_W4_MAX_TOKENS; }

moe_w4_ws_layout make_layout(int64_t T) {
    moe_w4_ws_layout L;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = align_up(off + bytes);
        return at;
    };
    const size_t t = (size_t)T, a = (size_t)kTopK * T;
    L.logits = take(4 * kE * t);
    L.topk_idx = take(4 * a);
    L.topk_w = take(4 * a);
    L.offsets = take(4 * (kE + 1));
    L.perm = take(4 * a);
    L.pos = take(4 * a);
    L.n_active = take(4);
    L.active = take(4 * 8 * kE);
    L.xt = take(2 * kH * t);
    L.xt_scale = take(4 * t);
    L.act = take(4 * kI * a);
    L.at = take(2 * kI * a);
    L.at_scale = take(4 * (kI / kG) * a);
    L.hs = take(2 * kIS * t);
    L.o = take(4 * kH * a);
    L.z = take(4 * kH * t);
    L.chunks = take(16 * (size_t)max_chunks((int)T));
    L.n_chunks = take(4);
    L.sync = take(kFusedSyncBytes);
    L.error = take(4);
    L.hist = take(4 * (size_t)kE * sort_hist_blocks((int)T));
    L.total = off;
    return L;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool overlap(const void *a, size_t na, const void *b, size_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

int device_status(hipError_t err) {
    if (err == hipSuccess) return MOE_W4_OK;
    g_last_device_error = (int)err;
    return MOE_W4_EDEVICE;
}

int validate_forward(const void *x, const void *router_w, const void *codes, const void *scales,
                     const void *shared_w, int64_t T, const void *y, const float *bias,
                     const void *ws, size_t ws_bytes) {
    if (!t_in_range(T)) return MOE_W4_EINVAL;
    if (T == 0) return MOE_W4_OK;
    if (!x || !router_w || !codes || !scales || !shared_w || !y || !ws) return MOE_W4_EINVAL;
    const void *ptrs[] = {x, router_w, codes, scales, shared_w, y, ws};
    for (const void *p : ptrs)
        if (!aligned(p, MOE_W4_ALIGN)) return MOE_W4_EINVAL;
    if (bias && !aligned(bias, 4)) return MOE_W4_EINVAL;
    if (ws_bytes < make_layout(T).total) return MOE_W4_EWORKSPACE;
    const size_t act_bytes = (size_t)T * kH * 2;
    if (overlap(y, act_bytes, x, act_bytes) || overlap(y, act_bytes, ws, ws_bytes)) return MOE_W4_EINVAL;
    return MOE_W4_OK;
}

const char *kStageNames[] = {"router_shared_gateup", "topk_sort", "routed_gateup", "rotate_act", "routed_down",
                             "shared_down_combine"};
constexpr int kStages = sizeof(kStageNames) / sizeof(kStageNames[0]);

// From this many tokens on, the routed experts run as MFMA grouped products
// (chunks of up to 64 tokens per expert) and the router and shared expert as
// LDS-tiled GEMMs; below it, as streaming GEMVs and few-row MFMA products.
constexpr int kPrefillMinTokens = 128;

template <class T_>
T_ *ws_at(void *ws, size_t off) { return reinterpret_cast<T_ *>(static_cast<char *>(ws) + off); }

// resid (stack layers of 1-8 tokens only): x_ is then written, as
// bf16(rmsnorm(resid)), by the first launch, and the last adds y to resid.
// keep_error: leave the workspace's error word as it is (the later layers of a
// stack call, so that a failure of any layer stays visible).
int run_forward(const void *x_, const void *router_w_, const void *codes_, const void *scales_,
                const void *shared_w_, int64_t T64, void *y_, const float *bias, void *ws,
                hipStream_t s, void *const *events, int n_events, float *resid = nullptr, int policy = 0,
                bool keep_error = false) {
    const int T = (int)T64;
    const moe_w4_ws_layout L = make_layout(T64);
    const uint16_t *x = static_cast<const uint16_t *>(x_);
    const uint16_t *router_w = static_cast<const uint16_t *>(router_w_);
    const uint8_t *codes = static_cast<const uint8_t *>(codes_);
    const uint16_t *scales = static_cast<const uint16_t *>(scales_);
    const uint16_t *shared_w = static_cast<const uint16_t *>(shared_w_);
    uint16_t *y = static_cast<uint16_t *>(y_);

    float *logits = ws_at<float>(ws, L.logits);
    int *topk_idx = ws_at<int>(ws, L.topk_idx);
    float *topk_w = ws_at<float>(ws, L.topk_w);
    int *offsets = ws_at<int>(ws, L.offsets);
    int *perm = ws_at<int>(ws, L.perm);
    int *pos = ws_at<int>(ws, L.pos);
    int *n_active = ws_at<int>(ws, L.n_active);
    int *active = ws_at<int>(ws, L.active);
    uint32_t *xt = ws_at<uint32_t>(ws, L.xt);
    float *xt_scale = ws_at<float>(ws, L.xt_scale);
    float *act = ws_at<float>(ws, L.act);
    uint32_t *at = ws_at<uint32_t>(ws, L.at);
    float *at_scale = ws_at<float>(ws, L.at_scale);
    uint16_t *hs = ws_at<uint16_t>(ws, L.hs);
    float *o = ws_at<float>(ws, L.o);
    float *z = ws_at<float>(ws, L.z);
    int *chunks = ws_at<int>(ws, L.chunks);
    int *n_chunks = ws_at<int>(ws, L.n_chunks);
    const bool grouped = T >= kPrefillMinTokens;
    const bool fused = T <= kFusedMaxTokens;
    const bool small_route = !grouped && T <= kRouteSmallMaxTokens;
    int *counters = ws_at<int>(ws, L.sync);
    int *error = ws_at<int>(ws, L.error);
    int *error_clear = keep_error ? nullptr : error;

    int stage = 0;
    auto mark = [&](void) -> int {
        if (events && stage < n_events) {
            hipError_t e = hipEventRecord(static_cast<hipEvent_t>(events[stage]), s);
            if (e != hipSuccess) return device_status(e);
        }
        ++stage;
        return MOE_W4_OK;
    };
    auto check = [&](void) -> int { return device_status(hipGetLastError()); };
    int rc;
#define MOE_STEP(call)                        \
    do {                                      \
        call;                                 \
        if ((rc = check()) != MOE_W4_OK) return rc; \
    } while (0)
#define MOE_MARK()                            \
    do {                                      \
        if ((rc = mark()) != MOE_W4_OK) return rc; \
    } while (0)

    (void)hipGetLastError();   // clear a stale error so it is not blamed on this call
    MOE_MARK();
    if (fused) {
        // two launches: the router logits (which also clear the counters),
        // then the rest of the layer; the other stages are empty.  The logits
        // are written without the bias; the routing adds it
        MOE_STEP(launch_router_small(x, resid, const_cast<uint16_t *>(x), T, router_w, nullptr, logits, counters,
                                     error_clear, s));
        MOE_MARK();
        MOE_MARK();
        FusedDecodeArgs fa;
        fa.x = x;
        fa.logits = logits;
        fa.router_bias = bias;
        fa.router_policy = policy;
        fa.codes = codes;
        fa.scales = scales;
        fa.nv_scales = nullptr;
        fa.tscales = nullptr;
        fa.shared_gu = shared_w;
        fa.shared_down = shared_w + 2 * kSharedGateElems;
        fa.hs = hs;
        fa.T = T;
        fa.topk_idx = topk_idx;
        fa.topk_w = topk_w;
        fa.offsets = offsets;
        fa.perm = perm;
        fa.pos = pos;
        fa.n_active = n_active;
        fa.slots = active;
        fa.chunks = reinterpret_cast<int4 *>(chunks);
        fa.n_chunks = n_chunks;
        fa.act = act;
        fa.y = y;
        fa.resid = resid;
        fa.counters = counters;
        fa.counters_h = counters + kFusedCounters * kFusedCounterStride;
        fa.error = error;
        fa.wait_target_extra = g_wait_extra.load(std::memory_order_relaxed);
        fa.wait_ticks = g_wait_ticks.load(std::memory_order_relaxed);
        MOE_STEP(launch_decode_fused(fa, s));
        for (int i = 0; i < 4; ++i) MOE_MARK();
        return MOE_W4_OK;
    }
    if (grouped)
        // (it also zeroes the sort's histograms, which the top-6 launch fills)
        MOE_STEP(launch_router_and_shared_gateup_dense(x, T, router_w, nullptr, logits, shared_w, hs, s,
                                                       ws_at<int>(ws, L.hist), kE * sort_hist_blocks(T)));
    else if (small_route)
        // up to kRouteSmallMaxTokens tokens: the router, the shared gate/up
        // and the rotation of x in one launch, which also clears the counter
        // of the routing launch after it
        MOE_STEP(launch_router_and_shared_gateup(x, T, router_w, nullptr, logits, shared_w, hs, xt, xt_scale,
                                                 counters, s));
    else
        MOE_STEP(launch_router_and_shared_gateup(x, T, router_w, nullptr, logits, shared_w, hs, nullptr, xt_scale,
                                                 nullptr, s));
    MOE_MARK();
    if (small_route) {
        MOE_STEP(launch_route_par(logits, T, bias, policy, topk_idx, topk_w, offsets, perm, pos, n_active, active,
                                  chunks, n_chunks, o, counters, error_clear, error,
                                  g_wait_extra.load(std::memory_order_relaxed),
                                  g_wait_ticks.load(std::memory_order_relaxed), s));
    } else {
        MOE_STEP(launch_topk_rotate(logits, x, T, bias, policy, topk_idx, topk_w, xt, xt_scale, s, true,
                                    grouped ? ws_at<int>(ws, L.hist) : nullptr));
        if (grouped)   // many workgroups
            MOE_STEP(launch_sort_wide(topk_idx, T, ws_at<int>(ws, L.hist), offsets, perm, pos, n_active, active,
                                      chunks, n_chunks, error_clear, s));
        else
            MOE_STEP(launch_sort(topk_idx, T, offsets, perm, pos, n_active, active, chunks, n_chunks, error_clear,
                                 s));
    }
    MOE_MARK();
    if (grouped) {
        // gate/up also rotates a: the rotate_act stage is empty on this path
        MOE_STEP(launch_gateup_mfma(codes, scales, xt, xt_scale, perm, chunks, n_chunks, T, at, at_scale, s));
        MOE_MARK();
        MOE_MARK();
        // fp16 rows in the first half of the o region, their multipliers behind them
        MOE_STEP(launch_down_mfma(codes, scales, at, at_scale, chunks, n_chunks, T, reinterpret_cast<uint16_t *>(o),
                                  o + (size_t)kTopK * T * kH / 2, s));
        MOE_MARK();
    } else {
        MOE_STEP(launch_gateup_gemv(codes, scales, xt, xt_scale, perm, active, T, act, s));
        MOE_MARK();
        // the down launch rotates a itself: the rotate_act stage is empty
        MOE_MARK();
        MOE_STEP(launch_down_gemv(codes, scales, act, active, T, o, s));
        MOE_MARK();
    }
    if (grouped) {
        MOE_STEP(launch_shared_down_dense(shared_w, hs, T, z, s));
        MOE_STEP(launch_combine_half(z, topk_w, pos, reinterpret_cast<const uint16_t *>(o),
                                     o + (size_t)kTopK * T * kH / 2, T, y, s));
    } else
        MOE_STEP(launch_shared_down_combine(shared_w, hs, T, topk_w, pos, o, y, s));
    MOE_MARK();
#undef MOE_STEP
#undef MOE_MARK
    return MOE_W4_OK;
}

// The layer with NVFP4 experts: the router, the shared expert, the routing
// and the combine of the int4 path (no rotated x is needed), the experts as
// NVFP4 GEMVs at every token count.  Stage marks as in run_forward (the
// rotate_act stage is empty).
int run_forward_nvfp4(const void *x_, const void *router_w_, const void *codes_, const void *scales_,
                      const float *tscales, const void *shared_w_, int64_t T64, void *y_, const float *bias,
                      void *ws, hipStream_t s, void *const *events, int n_events) {
    const int T = (int)T64;
    const moe_w4_ws_layout L = make_layout(T64);
    const uint16_t *x = static_cast<const uint16_t *>(x_);
    const uint16_t *router_w = static_cast<const uint16_t *>(router_w_);
    const uint8_t *codes = static_cast<const uint8_t *>(codes_);
    const uint8_t *scales = static_cast<const uint8_t *>(scales_);
    const uint16_t *shared_w = static_cast<const uint16_t *>(shared_w_);
    uint16_t *y = static_cast<uint16_t *>(y_);
    float *logits = ws_at<float>(ws, L.logits);
    int *topk_idx = ws_at<int>(ws, L.topk_idx);
    float *topk_w = ws_at<float>(ws, L.topk_w);
    int *offsets = ws_at<int>(ws, L.offsets);
    int *perm = ws_at<int>(ws, L.perm);
    int *pos = ws_at<int>(ws, L.pos);
    int *n_active = ws_at<int>(ws, L.n_active);
    int *active = ws_at<int>(ws, L.active);
    uint32_t *xt = ws_at<uint32_t>(ws, L.xt);
    float *xt_scale = ws_at<float>(ws, L.xt_scale);
    float *act = ws_at<float>(ws, L.act);
    uint16_t *hs = ws_at<uint16_t>(ws, L.hs);
    float *o = ws_at<float>(ws, L.o);
    float *z = ws_at<float>(ws, L.z);
    int *chunks = ws_at<int>(ws, L.chunks);
    int *n_chunks = ws_at<int>(ws, L.n_chunks);
    int *error = ws_at<int>(ws, L.error);
    int *counters = ws_at<int>(ws, L.sync);
    const bool dense = T >= kPrefillMinTokens;
    const bool small_route = T <= kRouteSmallMaxTokens;

    int stage = 0;
    int rc;
    auto mark = [&](void) -> int {
        if (events && stage < n_events) {
            hipError_t e = hipEventRecord(static_cast<hipEvent_t>(events[stage]), s);
            if (e != hipSuccess) return device_status(e);
        }
        ++stage;
        return MOE_W4_OK;
    };
#define NV_STEP(call)                                                          \
    do {                                                                       \
        call;                                                                  \
        if ((rc = device_status(hipGetLastError())) != MOE_W4_OK) return rc;   \
    } while (0)
#define NV_MARK()                                  \
    do {                                           \
        if ((rc = mark()) != MOE_W4_OK) return rc; \
    } while (0)
    (void)hipGetLastError();
    NV_MARK();
    if (T <= kFusedMaxTokens) {
        // the two launches of the int4 layer's fused form, with the NVFP4
        // experts' codes and scales
        NV_STEP(launch_router_small(x, nullptr, nullptr, T, router_w, nullptr, logits, counters, error, s));
        NV_MARK();
        NV_MARK();
        FusedDecodeArgs fa;
        fa.x = x;
        fa.logits = logits;
        fa.router_bias = bias;
        fa.router_policy = 0;
        fa.codes = codes;
        fa.scales = nullptr;
        fa.nv_scales = scales;
        fa.tscales = tscales;
        fa.shared_gu = shared_w;
        fa.shared_down = shared_w + 2 * kSharedGateElems;
        fa.hs = hs;
        fa.T = T;
        fa.topk_idx = topk_idx;
        fa.topk_w = topk_w;
        fa.offsets = offsets;
        fa.perm = perm;
        fa.pos = pos;
        fa.n_active = n_active;
        fa.slots = active;
        fa.chunks = reinterpret_cast<int4 *>(chunks);
        fa.n_chunks = n_chunks;
        fa.act = act;
        fa.y = y;
        fa.resid = nullptr;
        fa.counters = counters;
        fa.counters_h = counters + kFusedCounters * kFusedCounterStride;
        fa.error = error;
        fa.wait_target_extra = g_wait_extra.load(std::memory_order_relaxed);
        fa.wait_ticks = g_wait_ticks.load(std::memory_order_relaxed);
        NV_STEP(launch_decode_fused(fa, s));
        for (int i = 0; i < 4; ++i) NV_MARK();
        return MOE_W4_OK;
    }
    if (dense)
        NV_STEP(launch_router_and_shared_gateup_dense(x, T, router_w, nullptr, logits, shared_w, hs, s,
                                                      ws_at<int>(ws, L.hist), kE * sort_hist_blocks(T)));
    else
        NV_STEP(launch_router_and_shared_gateup(x, T, router_w, nullptr, logits, shared_w, hs, nullptr, xt_scale,
                                                small_route ? counters : nullptr, s));
    NV_MARK();
    if (small_route) {
        NV_STEP(launch_route_par(logits, T, bias, 0, topk_idx, topk_w, offsets, perm, pos, n_active, active, chunks,
                                 n_chunks, o, counters, error, error, g_wait_extra.load(std::memory_order_relaxed),
                                 g_wait_ticks.load(std::memory_order_relaxed), s));
    } else {
        // from 128 tokens on x as natural-order fp16 for the MFMA experts (the
        // GEMVs below that read x itself)
        NV_STEP(launch_topk_rotate(logits, x, T, bias, 0, topk_idx, topk_w, xt, xt_scale, s, false,
                                   dense ? ws_at<int>(ws, L.hist) : nullptr));
        if (dense)
            NV_STEP(launch_sort_wide(topk_idx, T, ws_at<int>(ws, L.hist), offsets, perm, pos, n_active, active,
                                     chunks, n_chunks, error, s));
        else
            NV_STEP(launch_sort(topk_idx, T, offsets, perm, pos, n_active, active, chunks, n_chunks, error, s));
    }
    NV_MARK();
    if (dense) {
        // MFMA tiles over chunks of up to 64 assignments of one expert
        NV_STEP(launch_gateup_mfma_nvfp4(codes, scales, tscales, xt, xt_scale, perm, chunks, n_chunks, T,
                                         ws_at<uint32_t>(ws, L.at), ws_at<float>(ws, L.at_scale), s));
        NV_MARK();
        NV_MARK();
        NV_STEP(launch_down_mfma_nvfp4(codes, scales, tscales, ws_at<uint32_t>(ws, L.at), ws_at<float>(ws, L.at_scale),
                                       chunks, n_chunks, T, o, s));
        NV_MARK();
    } else {
        NV_STEP(launch_gateup_nvfp4(codes, scales, tscales, x, perm, active, T, act, s));
        NV_MARK();
        NV_MARK();
        NV_STEP(launch_down_nvfp4(codes, scales, tscales, act, active, T, o, s));
        NV_MARK();
    }
    if (dense) {
        NV_STEP(launch_shared_down_dense(shared_w, hs, T, z, s));
        NV_STEP(launch_combine(z, topk_w, pos, o, T, y, s));
    } else
        NV_STEP(launch_shared_down_combine(shared_w, hs, T, topk_w, pos, o, y, s));
    NV_MARK();
#undef NV_STEP
#undef NV_MARK
    return MOE_W4_OK;
}

uint64_t host_mix64(uint64_t z) {
    z ^= z >> 30;
    z *= 0xBF58476D1CE4E5B9ull;
    z ^= z >> 27;
    z *= 0x94D049BB133111EBull;
    z ^= z >> 31;
    return z;
}
uint64_t stream_key(uint64_t seed, int layer, int kind) {
    return host_mix64(seed * 0x9E3779B97F4A7C15ull + (uint64_t)(64 * (int64_t)layer + kind));
}
float normal_mult(double sigma) { return (float)(sigma * sqrt(3.0) / 65536.0); }

// One layer of a stack on validated arguments: x_buf = bf16(rmsnorm(resid)),
// y_buf = layer(x_buf), resid += f32(y_buf).  keep_error: see run_forward.
int run_stack_layer(float *resid, const void *router_w, const void *codes, const void *scales,
                    const void *shared_w, int64_t T, void *x_buf, void *y_buf, void *ws, hipStream_t s,
                    bool keep_error) {
    (void)hipGetLastError();
    if (T <= kFusedMaxTokens)   // rmsnorm and residual add inside the two launches
        return run_forward(x_buf, router_w, codes, scales, shared_w, T, y_buf, nullptr, ws, s, nullptr, 0, resid, 0,
                           keep_error);
    launch_rmsnorm_bf16(resid, (int)T, static_cast<uint16_t *>(x_buf), s);
    int rc = device_status(hipGetLastError());
    if (rc != MOE_W4_OK) return rc;
    rc = run_forward(x_buf, router_w, codes, scales, shared_w, T, y_buf, nullptr, ws, s, nullptr, 0, nullptr, 0,
                     keep_error);
    if (rc != MOE_W4_OK) return rc;
    launch_residual_add(resid, static_cast<const uint16_t *>(y_buf), (int)T, s);
    return device_status(hipGetLastError());
}

// The stack's workspace: a forward workspace, then one layer's x and y (used
// when no trace is given).
struct StackWs {
    size_t x, y, total;
};
StackWs stack_ws_parts(int64_t T) {
    StackWs P;
    P.x = make_layout(T).total;
    P.y = align_up(P.x + (size_t)T * kH * 2);
    P.total = align_up(P.y + (size_t)T * kH * 2);
    return P;
}

// ---------------------------------------------------------------------------
// The forward without allocation (moe_w4_forward_static): its workspace is
// this file-scope device array, one copy per GPU, held until the process
// ends.  The array's name in host code is only a handle for the runtime; the
// device address of each GPU's copy comes from hipGetSymbolAddress, taken
// once per device with that device current, and only that address reaches
// the kernels.  Every call on a GPU shares its copy: nothing in it needs to
// be initialised (each call writes what it reads, and clears its own
// counters), but calls that overlap on one GPU race on it.
// ---------------------------------------------------------------------------
constexpr size_t kStaticScratchBytes = 11u << 20;   // the workspace of MOE_W4_STATIC_MAX_TOKENS tokens fits
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// The device address of the current GPU's copy of `scratch`.
int static_scratch(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return device_status(e);
    if (dev < 0 || dev >= kMaxDevices) return device_status(hipErrorInvalidDevice);
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return device_status(e);
            if (!p || make_layout(MOE_W4_STATIC_MAX_TOKENS).total > kStaticScratchBytes)
                return device_status(hipErrorInvalidSymbol);
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return MOE_W4_OK;
}

}  // namespace

extern "C" {

size_t moe_w4_workspace_bytes(int64_t T) { return t_in_range(T) ? make_layout(T).total : 0; }

int moe_w4_workspace_layout(int64_t T, moe_w4_ws_layout *out) {
    if (!out || !t_in_range(T)) return MOE_W4_EINVAL;
    *out = make_layout(T);
    return MOE_W4_OK;
}

int moe_w4_forward(const void *x, const void *router_w, const void *codes, const void *scales,
                   const void *shared_w, int64_t T, void *y, const float *router_bias,
                   void *workspace, size_t workspace_bytes, void *stream) {
    int rc = validate_forward(x, router_w, codes, scales, shared_w, T, y, router_bias, workspace, workspace_bytes);
    if (rc != MOE_W4_OK || T == 0) return rc;
    return run_forward(x, router_w, codes, scales, shared_w, T, y, router_bias, workspace,
                       static_cast<hipStream_t>(stream), nullptr, 0);
}

int moe_w4_forward_policy(const void *x, const void *router_w, const void *codes, const void *scales,
                          const void *shared_w, int64_t T, void *y, const float *router_bias, int router_policy,
                          void *workspace, size_t workspace_bytes, void *stream) {
    if ((router_policy & ~(MOE_W4_ROUTER_NORM_MASK | MOE_W4_ROUTER_BIAS_SELECT_ONLY)) != 0 ||
        (router_policy & MOE_W4_ROUTER_NORM_MASK) > MOE_W4_ROUTER_NORM_NONE)
        return MOE_W4_EINVAL;
    int rc = validate_forward(x, router_w, codes, scales, shared_w, T, y, router_bias, workspace, workspace_bytes);
    if (rc != MOE_W4_OK || T == 0) return rc;
    return run_forward(x, router_w, codes, scales, shared_w, T, y, router_bias, workspace,
                       static_cast<hipStream_t>(stream), nullptr, 0, nullptr, router_policy);
}

int moe_w4_forward_static(const void *x, const void *router_w, const void *codes, const void *scales,
                          const void *shared_w, int64_t T, void *y, const float *router_bias, void *stream) {
    if (!t_in_range(T)) return MOE_W4_EINVAL;
    if (T > MOE_W4_STATIC_MAX_TOKENS) return MOE_W4_EWORKSPACE;
    if (T == 0) return MOE_W4_OK;
    void *ws = nullptr;
    int rc = static_scratch(&ws);
    if (rc != MOE_W4_OK) return rc;
    rc = validate_forward(x, router_w, codes, scales, shared_w, T, y, router_bias, ws, kStaticScratchBytes);
    if (rc != MOE_W4_OK) return rc;
    return run_forward(x, router_w, codes, scales, shared_w, T, y, router_bias, ws, static_cast<hipStream_t>(stream),
                       nullptr, 0);
}

int moe_w4_profile_points(void) { return kStages + 1; }

const char *moe_w4_profile_point_name(int i) {
    if (i == 0) return "start";
    if (i < 1 || i > kStages) return nullptr;
    return kStageNames[i - 1];
}

int moe_w4_forward_profiled(const void *x, const void *router_w, const void *codes,
                            const void *scales, const void *shared_w, int64_t T, void *y,
                            const float *router_bias, void *workspace, size_t workspace_bytes,
                            void *stream, void *const *events, int n_events) {
    if (n_events < 0 || (n_events > 0 && !events)) return MOE_W4_EINVAL;
    int rc = validate_forward(x, router_w, codes, scales, shared_w, T, y, router_bias, workspace, workspace_bytes);
    if (rc != MOE_W4_OK || T == 0) return rc;
    return run_forward(x, router_w, codes, scales, shared_w, T, y, router_bias, workspace,
                       static_cast<hipStream_t>(stream), events, n_events);
}

int moe_w4_forward_nvfp4_profiled(const void *x, const void *router_w, const void *codes, const void *scales,
                                  const float *tensor_scales, const void *shared_w, int64_t T, void *y,
                                  const float *router_bias, void *workspace, size_t workspace_bytes, void *stream,
                                  void *const *events, int n_events) {
    if (n_events < 0 || (n_events > 0 && !events)) return MOE_W4_EINVAL;
    int rc = validate_forward(x, router_w, codes, scales, shared_w, T, y, router_bias, workspace, workspace_bytes);
    if (rc != MOE_W4_OK || T == 0) return rc;
    if (!tensor_scales || !aligned(tensor_scales, 4)) return MOE_W4_EINVAL;
    return run_forward_nvfp4(x, router_w, codes, scales, tensor_scales, shared_w, T, y, router_bias, workspace,
                             static_cast<hipStream_t>(stream), events, n_events);
}

int moe_w4_forward_nvfp4(const void *x, const void *router_w, const void *codes, const void *scales,
                         const float *tensor_scales, const void *shared_w, int64_t T, void *y,
                         const float *router_bias, void *workspace, size_t workspace_bytes, void *stream) {
    return moe_w4_forward_nvfp4_profiled(x, router_w, codes, scales, tensor_scales, shared_w, T, y, router_bias,
                                         workspace, workspace_bytes, stream, nullptr, 0);
}

size_t moe_w4_dense_mlp_workspace_bytes(int64_t T) {
    return t_in_range(T) ? align_up((size_t)T * kDenseInter * 2) + 256 : 0;
}

int moe_w4_dense_mlp(const void *x, const void *w, int64_t T, void *y, void *workspace, size_t workspace_bytes,
                     void *stream) {
    if (!t_in_range(T)) return MOE_W4_EINVAL;
    if (T == 0) return MOE_W4_OK;
    if (!x || !w || !y || !workspace) return MOE_W4_EINVAL;
    const void *ptrs[] = {x, w, y, workspace};
    for (const void *p : ptrs)
        if (!aligned(p, MOE_W4_ALIGN)) return MOE_W4_EINVAL;
    if (workspace_bytes < moe_w4_dense_mlp_workspace_bytes(T)) return MOE_W4_EWORKSPACE;
    const size_t act_bytes = (size_t)T * kH * 2;
    if (overlap(y, act_bytes, x, act_bytes) || overlap(y, act_bytes, workspace, workspace_bytes) ||
        overlap(y, act_bytes, w, (size_t)MOE_W4_DENSE_WEIGHTS * 2))
        return MOE_W4_EINVAL;
    const int t = (int)T;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const uint16_t *xb = static_cast<const uint16_t *>(x), *wb = static_cast<const uint16_t *>(w);
    uint16_t *h = static_cast<uint16_t *>(workspace), *yb = static_cast<uint16_t *>(y);
    (void)hipGetLastError();
    if (t >= kPrefillMinTokens) {
        launch_dense_mlp_gateup_dense(xb, t, wb, h, s);
        if (hipPeekAtLastError() == hipSuccess) launch_dense_mlp_down_dense(wb, h, t, yb, s);
    } else {
        launch_dense_mlp_gateup_skinny(xb, t, wb, h, s);
        if (hipPeekAtLastError() == hipSuccess) launch_dense_mlp_down_skinny(wb, h, t, yb, s);
    }
    return device_status(hipGetLastError());
}

int moe_w4_pack_experts(const void *w, int64_t n_experts, void *codes, void *scales, void *stream) {
    if (n_experts < 0 || n_experts > MOE_W4_PACK_MAX_EXPERTS) return MOE_W4_EINVAL;
    if (n_experts == 0) return MOE_W4_OK;
    if (!w || !codes || !scales) return MOE_W4_EINVAL;
    if (!aligned(w, MOE_W4_ALIGN) || !aligned(codes, MOE_W4_ALIGN) || !aligned(scales, MOE_W4_ALIGN))
        return MOE_W4_EINVAL;
    const size_t nw = (size_t)n_experts * MOE_W4_EXPERT_WEIGHTS * 2;
    const size_t nc = (size_t)n_experts * kCodeBytesPerExpert, ns = (size_t)n_experts * kScalesPerExpert * 2;
    if (overlap(w, nw, codes, nc) || overlap(w, nw, scales, ns) || overlap(codes, nc, scales, ns))
        return MOE_W4_EINVAL;
    (void)hipGetLastError();
    launch_pack_experts(static_cast<const uint16_t *>(w), n_experts, static_cast<uint8_t *>(codes),
                        static_cast<uint16_t *>(scales), static_cast<hipStream_t>(stream));
    return device_status(hipGetLastError());
}

int moe_w4_generate_layer(uint64_t seed, int layer, void *router_w, void *codes, void *scales,
                          void *shared_w, void *stream) {
    if (layer < 0 || layer > (1 << 20)) return MOE_W4_EINVAL;
    const void *ptrs[] = {router_w, codes, scales, shared_w};
    for (const void *p : ptrs)
        if (p && !aligned(p, MOE_W4_ALIGN)) return MOE_W4_EINVAL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    const float m_w = normal_mult(0.02), m_s = normal_mult(0.01);
    if (router_w)
        launch_gen_normal_bf16(stream_key(seed, layer, 1), (int64_t)kE * kH, m_w, 0,
                               static_cast<uint16_t *>(router_w), s);
    if (codes) {
        uint8_t *c = static_cast<uint8_t *>(codes);
        const int64_t ee = (int64_t)kI * kH;
        launch_gen_codes(stream_key(seed, layer, 2), kI, kH, kE, ee, kCodeBytesPerExpert, c, s);
        launch_gen_codes(stream_key(seed, layer, 3), kI, kH, kE, ee, kCodeBytesPerExpert, c + kPlaneGateBytes, s);
        launch_gen_codes(stream_key(seed, layer, 4), kH, kI, kE, ee, kCodeBytesPerExpert, c + kCodeBytesGu, s);
    }
    if (scales) {
        uint16_t *sc = static_cast<uint16_t *>(scales);
        launch_gen_scales(stream_key(seed, layer, 5), kH / kG, kI, kE, kScalesPerExpert, m_s, sc, s);
        launch_gen_scales(stream_key(seed, layer, 6), kH / kG, kI, kE, kScalesPerExpert, m_s, sc + kScalesGate, s);
        launch_gen_scales(stream_key(seed, layer, 7), kI / kG, kH, kE, kScalesPerExpert, m_s, sc + kScalesGu, s);
    }
    if (shared_w) {
        uint16_t *w = static_cast<uint16_t *>(shared_w);
        launch_gen_normal_bf16(stream_key(seed, layer, 8), (int64_t)kSharedGateElems, m_w, 0, w, s);
        launch_gen_normal_bf16(stream_key(seed, layer, 9), (int64_t)kSharedGateElems, m_w, 0, w + kSharedGateElems, s);
        launch_gen_normal_bf16(stream_key(seed, layer, 10), (int64_t)kSharedGateElems, m_w, 0, w + 2 * kSharedGateElems, s);
    }
    return device_status(hipGetLastError());
}

int moe_w4_generate_x(uint64_t seed, int layer, int64_t T, void *x, void *stream) {
    if (!t_in_range(T) || layer < 0 || layer > (1 << 20)) return MOE_W4_EINVAL;
    if (T == 0) return MOE_W4_OK;
    if (!x || !aligned(x, MOE_W4_ALIGN)) return MOE_W4_EINVAL;
    (void)hipGetLastError();
    launch_gen_normal_bf16(stream_key(seed, layer, 0), T * kH, normal_mult(1.0), 0,
                           static_cast<uint16_t *>(x), static_cast<hipStream_t>(stream));
    return device_status(hipGetLastError());
}

int moe_w4_stack_layer(float *resid, const void *router_w, const void *codes, const void *scales,
                       const void *shared_w, int64_t T, void *x_buf, void *y_buf, void *workspace,
                       size_t workspace_bytes, void *stream) {
    if (!t_in_range(T)) return MOE_W4_EINVAL;
    if (T == 0) return MOE_W4_OK;
    if (!resid || !aligned(resid, MOE_W4_ALIGN)) return MOE_W4_EINVAL;
    int rc = validate_forward(x_buf, router_w, codes, scales, shared_w, T, y_buf, nullptr, workspace, workspace_bytes);
    if (rc != MOE_W4_OK) return rc;
    const size_t rb = (size_t)T * kH * 4, ab = (size_t)T * kH * 2;
    if (overlap(resid, rb, x_buf, ab) || overlap(resid, rb, y_buf, ab) || overlap(resid, rb, workspace, workspace_bytes))
        return MOE_W4_EINVAL;
    return run_stack_layer(resid, router_w, codes, scales, shared_w, T, x_buf, y_buf, workspace,
                           static_cast<hipStream_t>(stream), false);
}

size_t moe_w4_stack_workspace_bytes(int64_t T) {
    if (!t_in_range(T)) return 0;
    return stack_ws_parts(T).total;
}

int moe_w4_stack_forward(float *resid, const moe_w4_layer *layers, int n_layers, int64_t T, void *trace,
                         void *workspace, size_t workspace_bytes, void *stream) {
    if (!t_in_range(T) || n_layers < 0 || n_layers > MOE_W4_STACK_MAX_LAYERS) return MOE_W4_EINVAL;
    if (T == 0 || n_layers == 0) return MOE_W4_OK;
    if (!layers || !resid || !workspace) return MOE_W4_EINVAL;
    if (!aligned(resid, MOE_W4_ALIGN) || !aligned(workspace, MOE_W4_ALIGN)) return MOE_W4_EINVAL;
    if (trace && !aligned(trace, MOE_W4_ALIGN)) return MOE_W4_EINVAL;
    for (int l = 0; l < n_layers; ++l) {
        const moe_w4_layer &w = layers[l];
        const void *ptrs[] = {w.router_w, w.codes, w.scales, w.shared_w};
        for (const void *p : ptrs)
            if (!p || !aligned(p, MOE_W4_ALIGN)) return MOE_W4_EINVAL;
    }
    const StackWs P = stack_ws_parts(T);
    if (workspace_bytes < P.total) return MOE_W4_EWORKSPACE;
    const size_t rb = (size_t)T * kH * 4, ab = (size_t)T * kH * 2, tb = (size_t)n_layers * 2 * ab;
    if (overlap(resid, rb, workspace, workspace_bytes)) return MOE_W4_EINVAL;
    if (trace && (overlap(trace, tb, resid, rb) || overlap(trace, tb, workspace, workspace_bytes)))
        return MOE_W4_EINVAL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    char *ws = static_cast<char *>(workspace);
    for (int l = 0; l < n_layers; ++l) {
        const moe_w4_layer &w = layers[l];
        void *xb = trace ? static_cast<char *>(trace) + (size_t)(2 * l) * ab : ws + P.x;
        void *yb = trace ? static_cast<char *>(trace) + (size_t)(2 * l + 1) * ab : ws + P.y;
        const int rc = run_stack_layer(resid, w.router_w, w.codes, w.scales, w.shared_w, T, xb, yb, ws, s, l > 0);
        if (rc != MOE_W4_OK) return rc;
    }
    return MOE_W4_OK;
}

int moe_w4_generate_normal_bf16(uint64_t seed, uint32_t tensor_id, int64_t n, double sigma, void *out, void *stream) {
    if (n < 0 || n > MOE_W4_GENERATE_MAX_ELEMS || !(sigma >= 0.0) || !isfinite(sigma)) return MOE_W4_EINVAL;
    if (n == 0) return MOE_W4_OK;
    if (!out || !aligned(out, 2)) return MOE_W4_EINVAL;
    (void)hipGetLastError();
    const uint64_t key = host_mix64(seed * 0x9E3779B97F4A7C15ull + (uint64_t)tensor_id);
    launch_gen_normal_bf16(key, n, normal_mult(sigma), 0, static_cast<uint16_t *>(out), static_cast<hipStream_t>(stream));
    return device_status(hipGetLastError());
}

int moe_w4_set_fused_wait(int64_t max_ticks, int extra_count) {
    if (max_ticks < 0 || max_ticks > 0xffffffffLL || extra_count < 0) return MOE_W4_EINVAL;
    g_wait_ticks.store(max_ticks == 0 ? kDefaultWaitTicks : (uint32_t)max_ticks, std::memory_order_relaxed);
    g_wait_extra.store(extra_count, std::memory_order_relaxed);
    return MOE_W4_OK;
}

const char *moe_w4_status_string(int status) {
    switch (status) {
        case MOE_W4_OK: return "ok";
        case MOE_W4_EINVAL: return "invalid argument (pointer, size, alignment or aliasing)";
        case MOE_W4_EWORKSPACE: return "workspace too small";
        case MOE_W4_EDEVICE: return "HIP launch or runtime call failed";
        default: return "unknown status";
    }
}

int moe_w4_last_device_error(void) { return g_last_device_error; }

int moe_w4_version(void) { return 100; }

}  // extern "C"
