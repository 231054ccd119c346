/*
 * moe_w4 — the routed mixture-of-experts layer of Flint with four-bit experts,
 * for one AMD Instinct MI355X (gfx950).  C ABI.
 *
 * What the layer computes (the pages this follows):
 *   - Flint model card of the int4-expert container (Aijuus/flint-w4exp),
 *     introduction and table row "weights": 256 routed experts, top-6, plus an
 *     ungated shared expert; routed weights are signed int4 codes with one
 *     bf16 scale per 128 of K, stored in a basis rotated by a 128-wide
 *     Hadamard transform (fwht128); the shared expert stays bf16.
 *   - NInfer README of Flint (WaveCut/Flint-UD-Q4_K_XL-NInfer-v3), section
 *     "What is inside": sigmoid router scores renormalised over the chosen
 *     experts; per expert, gate rows then up rows (2 x 512) and 2,048 down rows;
 *     shared expert of width 1024; router rows in fp32 widened from bf16.
 *   - bloomery issue #632 ("model: Flint ..."), design thread: no router
 *     correction bias; weights w = score / max(sum of the 6 scores, 2^-14);
 *     the router hands six (index, fp32 weight) slots to the expert stage.
 *
 *   logits = R x (+ bias)         fp32 sums of exact bf16 products
 *   S      = 6 largest logits, larger first, equal logits -> lower index
 *   w_j    = sigmoid(l_j) / max(sum_j sigmoid(l_j), 2^-14)
 *   xr     = H128 applied to every 128-block of x      (H128 = normalised Sylvester Hadamard)
 *   o_j    = Wd_e H128( silu(Wg_e xr) * (Wu_e xr) ),    W = code * scale[row][k/128]
 *   z      = Wsd( silu(Wsg x) * (Wsu x) )              (bf16 weights, unrotated)
 *   y      = bf16_rne( sum_j w_j o_j + z )
 *
 * Layouts (row-major, K contiguous; all pointers are device pointers):
 *   x        bf16 [T][2048]
 *   router_w bf16 [256][2048]
 *   codes    u8   [256][1,572,864]: expert e at e*1,572,864 B holds
 *            gate [512][1024 B], up [512][1024 B], down [2048][256 B];
 *            element k of a row is the low nibble of byte k/2 when k is even,
 *            the high nibble when k is odd; two's complement, [-8, 7].
 *   scales   bf16 [256][24,576]: expert e at element e*24,576 holds
 *            gate [512][16], up [512][16], down [2048][4]; scale g of a row
 *            multiplies the codes of K in [128g, 128g+128).
 *   shared_w bf16, 6,291,456 elements: gate [1024][2048], up [1024][2048],
 *            down [2048][1024].
 *   bias     fp32 [256] added to the logits (for the choice, and by default for
 *            the sigmoid too), or NULL (Flint has none).
 *   y        bf16 [T][2048].
 *
 * Ownership and threading: the caller owns every buffer, including the
 * workspace.  The library allocates no device memory in these calls, keeps no
 * pointer after the enqueued work completes and holds no mutable global state
 * apart from the diagnostic setting of moe_w4_set_fused_wait, so calls on
 * different streams are independent if they use different workspaces.  Work is enqueued on `stream` (a hipStream_t passed as void*;
 * NULL = the default stream) and the call returns without synchronising.
 *
 * Errors: arguments are validated before any HIP call.  Asynchronous device
 * faults surface at the caller's next synchronisation.  No C++ exception
 * crosses this interface.  Non-finite inputs are not checked.
 */
#ifndef MOE_W4_H
#define MOE_W4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_W4_HIDDEN 2048
#define MOE_W4_EXPERTS 256
#define MOE_W4_TOPK 6
#define MOE_W4_INTER 512
#define MOE_W4_SHARED_INTER 1024
#define MOE_W4_GROUP 128
#define MOE_W4_CODE_BYTES_PER_EXPERT 1572864
#define MOE_W4_SCALES_PER_EXPERT 24576
#define MOE_W4_SHARED_ELEMS 6291456
/* Largest T of a call.  Every 32-bit buffer offset of the kernels stays in
 * range up to here (the largest workspace region, the expert rows o of 6T
 * assignments, is 3.2 GB at this T), and the GPU tests run this size. */
#define MOE_W4_MAX_TOKENS 65536
#define MOE_W4_ALIGN 16
/* From 1 to this many tokens a forward call is two launches (the router, then
 * the rest of the layer in one launch whose workgroups hand the routed gate/up
 * results and the shared expert's activations to the down projection through
 * device-scope counters in the workspace's `sync` region, cleared by the first
 * launch); from MOE_W4_FUSED_MAX_TOKENS + 1 tokens on, one launch per step
 * (up to 48 tokens the routing launch hands its workgroups' top-6 selections
 * to its workgroup 0 through the same counters, cleared by the launch before). */
#define MOE_W4_FUSED_MAX_TOKENS 8
/* Most layers in one moe_w4_stack_forward call. */
#define MOE_W4_STACK_MAX_LAYERS 1024
/* Most elements of one moe_w4_generate_normal_bf16 call. */
#define MOE_W4_GENERATE_MAX_ELEMS (1LL << 40)

/* Router policy of moe_w4_forward_policy (bloomery issue #632, design thread
 * and its host-policy slice: the router rule distinguishes no normalisation,
 * the legacy selected sum and the selected sum with the 2^-14 floor, and a
 * router bias that is absent or used for the selection only).  One of the
 * three normalisations, optionally OR-ed with MOE_W4_ROUTER_BIAS_SELECT_ONLY;
 * 0 is Flint's own policy, the one moe_w4_forward uses. */
#define MOE_W4_ROUTER_NORM_FLOOR 0       /* w_j = s_j / max(sum s, 2^-14)        */
#define MOE_W4_ROUTER_NORM_SUM 1         /* w_j = s_j / sum s (legacy; no floor) */
#define MOE_W4_ROUTER_NORM_NONE 2        /* w_j = s_j                            */
#define MOE_W4_ROUTER_NORM_MASK 3
#define MOE_W4_ROUTER_BIAS_SELECT_ONLY 4 /* s_j = sigmoid(R x) without the bias  */

/* status codes */
#define MOE_W4_OK 0
#define MOE_W4_EINVAL (-1)     /* bad pointer, size, alignment or aliasing      */
#define MOE_W4_EWORKSPACE (-2) /* workspace_bytes below moe_w4_workspace_bytes */
#define MOE_W4_EDEVICE (-3)    /* a HIP call or launch failed; see last_device_error */

/* Byte offsets of the routing results and intermediates inside the workspace.
 * Tests read the routing results through these after a forward call:
 *   topk_idx  i32 [T][6]  chosen experts, slot order = descending logit
 *   topk_w    f32 [T][6]  renormalised weights of those slots
 *   offsets   i32 [257]   offsets[e]..offsets[e+1] = sorted positions of expert e; offsets[256] = 6T
 *   perm      i32 [6T]    sorted position p -> assignment a = 6t + j, ordered by (expert, a)
 *   pos       i32 [6T]    inverse of perm
 *   n_active  i32 [1]     number of experts with at least one token
 *   active    i32 [256][8] one record per expert with tokens, ascending by expert:
 *                         {expert, offsets[expert], token count, first token,
 *                         second token (= first if one), 0, 0, 0}; records past
 *                         n_active hold expert -1
 *   chunks    i32 [n][4]  from T >= 128 on (MFMA grouped path): {expert, first sorted
 *                         position, rows, 0} covering each expert's sorted
 *                         positions in order, ascending by expert (chunks of
 *                         64 and a ragged last one; from T = 1536 on, one chunk
 *                         for an expert with <= 96 rows); n_chunks i32 [1]
 *                         holds n.  (Written at every T; read only on that path.)
 *   logits    f32 [T][256] router logits R x, without the bias
 *   sync      8192 bytes of counters for the hand-offs inside a launch (1-48
 *             tokens); their contents on entry do not matter (the call clears
 *             them itself).
 *   error     i32 [1]: 0 after a call that completed normally; 1 if a bounded
 *             wait of a hand-off gave up: a down workgroup of the two-launch
 *             form (1-8 tokens) waiting for the gate/up results, or the
 *             routing launch (9-48 tokens) waiting for the top-6 selections
 *             (the outputs are then NaN; see moe_w4_set_fused_wait).  A stack
 *             call keeps a failure of any of its layers.
 *   hist      scratch of the sort at prefill sizes (per-workgroup histograms). */
typedef struct moe_w4_ws_layout {
    size_t logits, topk_idx, topk_w, offsets, perm, pos, n_active, active;
    size_t xt, xt_scale, act, at, at_scale, hs, o, z, chunks, n_chunks, sync, error, hist;
    size_t total;
} moe_w4_ws_layout;

/* Bytes of workspace a forward call over T tokens needs (0 <= T <= MOE_W4_MAX_TOKENS;
 * returns 0 for an out-of-range T). */
size_t moe_w4_workspace_bytes(int64_t T);

/* Fills *out with the workspace layout for T tokens.  EINVAL for a NULL out or
 * an out-of-range T. */
int moe_w4_workspace_layout(int64_t T, moe_w4_ws_layout *out);

/* One MoE layer over T tokens: y = layer(x).  All pointers 16-byte aligned;
 * y must not overlap x or the workspace.  T == 0 returns MOE_W4_OK and
 * enqueues nothing.  Returns MOE_W4_EINVAL / MOE_W4_EWORKSPACE with nothing
 * enqueued, or MOE_W4_EDEVICE if a launch failed. */
int moe_w4_forward(const void *x, const void *router_w, const void *codes, const void *scales,
                   const void *shared_w, int64_t T, void *y, const float *router_bias,
                   void *workspace, size_t workspace_bytes, void *stream);

/* moe_w4_forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * no workspace argument; the workspace is a file-scope device array of the
 * library (11 MiB, one copy per GPU the library runs on, kept until the
 * process ends), located on the first call on each device.  The call itself
 * allocates nothing and calls no allocating routine.  Every call on a GPU
 * shares that GPU's array: calls that overlap on one GPU (on different
 * streams, or from different threads) race and must not be made; routing
 * results are not exposed.  T up to MOE_W4_STATIC_MAX_TOKENS; a larger T
 * returns MOE_W4_EWORKSPACE with nothing enqueued.  Otherwise arguments,
 * results and errors as moe_w4_forward. */
#define MOE_W4_STATIC_MAX_TOKENS 128
int moe_w4_forward_static(const void *x, const void *router_w, const void *codes, const void *scales,
                          const void *shared_w, int64_t T, void *y, const float *router_bias, void *stream);

/* moe_w4_forward with a router policy (MOE_W4_ROUTER_* above): the choice
 * is always the 6 largest of (logit + bias); router_policy selects the
 * normalisation of the sigmoid scores and whether the sigmoid sees the bias.
 * With MOE_W4_ROUTER_NORM_SUM, six scores that all underflow to 0 in fp32
 * give NaN weights (0/0).  EINVAL for an unknown policy; otherwise as
 * moe_w4_forward. */
int moe_w4_forward_policy(const void *x, const void *router_w, const void *codes, const void *scales,
                          const void *shared_w, int64_t T, void *y, const float *router_bias, int router_policy,
                          void *workspace, size_t workspace_bytes, void *stream);

/* Number of timing points moe_w4_forward_profiled records. */
int moe_w4_profile_points(void);
/* Name of timing point i (the stage that ends there), or NULL. */
const char *moe_w4_profile_point_name(int i);

/* moe_w4_forward that also records hipEvent_t events[i] (caller-created, passed
 * as void*) on `stream` at the stage boundaries: events[0] before the first
 * stage and events[i] after stage i, for i < moe_w4_profile_points().  The
 * kernels and results are those of moe_w4_forward. */
int moe_w4_forward_profiled(const void *x, const void *router_w, const void *codes,
                            const void *scales, const void *shared_w, int64_t T, void *y,
                            const float *router_bias, void *workspace, size_t workspace_bytes,
                            void *stream, void *const *events, int n_events);

/* The layer with routed experts in the NVFP4 container instead of int4 (Flint
 * NVFP4 repack, kekzle/Flint-NVFP4, rows "Layout per Linear" and
 * "Declaration": per Linear E2M1 codes two per byte, one E4M3 block scale per
 * 16 columns, one F32 tensor scale; W4A16).  Read as
 *   w[n][k] = e2m1(code[n][k]) * e4m3(scale[n][k / 16]) * tensor_scale
 * (OCP E2M1: sign, 2 exponent bits bias 1, 1 mantissa bit; OCP E4M3 "FN":
 * sign, 4 exponent bits bias 7, 3 mantissa bits, S.1111.111 NaN), weights in
 * the original basis (x and a are not rotated), activations not quantised.
 * Router, shared expert, routing and combine are those of moe_w4_forward
 * (Flint's router policy); x and the SwiGLU activations a enter the expert
 * products as fp16 with one power-of-two prescale per token or assignment,
 * and expert outputs are fp32 sums of exact products.  1-8 tokens run as the
 * two launches of moe_w4_forward's decode form (same hand-off waits, error
 * word and moe_w4_set_fused_wait).
 * codes: u8, expert e at e * MOE_W4_NVFP4_CODE_BYTES: gate [512][1024], up
 *        [512][1024], down [2048][256]; code of even k in the low nibble.
 * scales: u8 E4M3, expert e at e * MOE_W4_NVFP4_SCALE_BYTES: gate [512][128],
 *        up [512][128], down [2048][32] (block k / 16 of row n).
 * tensor_scales: f32 [256][3] (gate, up, down), 4-byte aligned device pointer.
 * Other arguments, the workspace and the errors as moe_w4_forward (EINVAL
 * also for a NULL or misaligned tensor_scales).  A NaN scale byte gives NaN
 * outputs for the tokens routed to that expert. */
#define MOE_W4_NVFP4_CODE_BYTES 1572864
#define MOE_W4_NVFP4_SCALE_BYTES 196608
int moe_w4_forward_nvfp4(const void *x, const void *router_w, const void *codes, const void *scales,
                         const float *tensor_scales, const void *shared_w, int64_t T, void *y,
                         const float *router_bias, void *workspace, size_t workspace_bytes, void *stream);
/* The same with the timing events of moe_w4_forward_profiled (the rotate_act
 * point follows routed_gateup with nothing between them). */
int moe_w4_forward_nvfp4_profiled(const void *x, const void *router_w, const void *codes, const void *scales,
                                  const float *tensor_scales, const void *shared_w, int64_t T, void *y,
                                  const float *router_bias, void *workspace, size_t workspace_bytes,
                                  void *stream, void *const *events, int n_events);

/* Seeded synthetic weights of one layer, written on the device with the
 * counter-based SplitMix64 generator (Steele, Lea and Flood, OOPSLA 2014):
 *   r(seed, tid, i) = mix64(mix64(seed*G + tid) + (i+1)*G), G = 0x9E3779B97F4A7C15,
 *   tid = 64*layer + kind (1 router, 2..4 gate/up/down codes, 5..7 their scales,
 *   8..10 shared gate/up/down); codes = (r >> 60) - 8; "normal" bf16 values are
 *   bf16_rne(f32(sum of the four 16-bit lanes of r - 131070) * f32(sigma*sqrt(3)/65536))
 *   with sigma 0.02 for router and shared weights; scales use the absolute
 *   value with sigma 0.01.  Any output pointer may be NULL to skip it. */
int moe_w4_generate_layer(uint64_t seed, int layer, void *router_w, void *codes, void *scales,
                          void *shared_w, void *stream);

/* Seeded x: bf16 [T][2048], sigma 1, tid = 64*layer + 0. */
int moe_w4_generate_x(uint64_t seed, int layer, int64_t T, void *x, void *stream);

/* Any seeded "normal" bf16 tensor of the same scheme: out[i] =
 * bf16_rne(f32(S(r(seed, tensor_id, i))) * f32(sigma*sqrt(3)/65536)) for
 * i < n, S the centred sum of the four 16-bit lanes of r (an Irwin-Hall
 * variate with the standard deviation sigma, bounded at about 3.46 sigma).
 * out: device pointer, 2-byte aligned, n bf16.  n == 0 enqueues nothing.
 * EINVAL for n outside [0, MOE_W4_GENERATE_MAX_ELEMS], a negative or
 * non-finite sigma, or a NULL / misaligned out. */
int moe_w4_generate_normal_bf16(uint64_t seed, uint32_t tensor_id, int64_t n, double sigma, void *out, void *stream);

/* One layer of a stack: the caller's residual stream stays fp32.
 *   x_in = bf16_rne( resid / sqrt(mean(resid^2) + 1e-6) )    (unit-gain RMS norm)
 *   resid += f32( moe_w4_forward(x_in) )
 * resid: f32 [T][2048] in/out.  x_buf: bf16 [T][2048] scratch that receives
 * x_in (the layer input, kept for inspection); y_buf: bf16 [T][2048] scratch
 * that receives the layer output.  Same validation as moe_w4_forward. */
int moe_w4_stack_layer(float *resid, const void *router_w, const void *codes, const void *scales,
                       const void *shared_w, int64_t T, void *x_buf, void *y_buf,
                       void *workspace, size_t workspace_bytes, void *stream);

/* The weights of one layer of a stack (device pointers, layouts of
 * moe_w4_forward). */
typedef struct moe_w4_layer {
    const void *router_w;
    const void *codes;
    const void *scales;
    const void *shared_w;
} moe_w4_layer;

/* Workspace bytes of moe_w4_stack_forward over T tokens (0 for an
 * out-of-range T): a forward workspace plus one layer's bf16 x and y. */
size_t moe_w4_stack_workspace_bytes(int64_t T);

/* A stack of MoE layers (bloomery issue #632, readiness comment: Flint has 2
 * dense and 47 routed blocks; this call runs the routed ones) over one batch:
 * for l = 0 .. n_layers-1,
 *   x_l   = bf16_rne( resid / sqrt(mean(resid^2) + 1e-6) )   (unit-gain RMS norm)
 *   y_l   = moe_w4_forward(x_l) with layers[l]
 *   resid = resid + f32(y_l)                                  (fp32 residual stream)
 * resid: f32 [T][2048] device, in/out.  layers: host array of n_layers
 * descriptors (read during the call only).  trace: NULL, or bf16
 * [n_layers][2][T][2048] device memory that receives x_l and y_l of every
 * layer (so each layer can be checked on its own input).  workspace: at least
 * moe_w4_stack_workspace_bytes(T) bytes, contents on entry irrelevant; after
 * the call its routing results (moe_w4_workspace_layout) are the last layer's
 * and its error word covers every layer.  Enqueues only kernels (no
 * allocation, no synchronisation, no memset), so it may be captured into a
 * HIP graph.  T == 0 or n_layers == 0 enqueues nothing.  EINVAL for a bad
 * T, n_layers outside [0, MOE_W4_STACK_MAX_LAYERS], a NULL or misaligned
 * pointer (16 bytes; every layer's four), or resid / trace / workspace
 * overlapping; EWORKSPACE for a short workspace; EDEVICE if a launch failed. */
int moe_w4_stack_forward(float *resid, const moe_w4_layer *layers, int n_layers, int64_t T, void *trace,
                         void *workspace, size_t workspace_bytes, void *stream);

/* Diagnostic of the bounded hand-off waits (1-48 tokens), for tests of their
 * failure path.  The down workgroups of the two-launch form (1-8 tokens) wait
 * for the gate/up results, and workgroup 0 of the routing launch (9-48
 * tokens) for the other workgroups' top-6 selections: max_ticks sets the bound
 * in ticks of the GPU's 100 MHz real-time clock (0 restores the default,
 * 500,000 = 5 ms) and extra_count a count the waits need beyond the producing
 * workgroups (default 0).  With extra_count > 0 a wait can never complete, so
 * it gives up after max_ticks: the down workgroups write NaN to their outputs
 * (and to the residual stream in a stack layer), the routing workgroup leaves
 * no expert active and NaN expert rows (so y is NaN), and the workspace's
 * error word is set; every kernel still exits normally.
 * Process-wide; read when a call enqueues its launches (a captured graph keeps
 * the values of its capture), so set it only while no other thread calls the
 * library.  EINVAL for max_ticks outside [0, 2^32) or extra_count < 0. */
int moe_w4_set_fused_wait(int64_t max_ticks, int extra_count);

/* The packer: bf16 expert weights -> this library's int4 expert format (the
 * step before the layer).  Format from the Flint model card (Aijuus/flint-w4exp),
 * table row "weights" (int4 codes, group 128, bf16 scale, fwht128 rotation);
 * its error, 11.7% relative Frobenius per expert plane, from the card's "Why
 * the linears stay bf16".  The quantiser is not printed there; it is read as:
 *   rotated row  r = every 128-block of the row times H128 (fp32 butterfly,
 *                    strides 1..64 in ascending order, then 1/sqrt(128))
 *   scale        s = bf16_rne( fp32(absmax of the block's r) / 7 )
 *   code         c = clamp( round_half_even( fp32(r / s) ), -8, 7 ), 0 if s == 0
 * w: bf16, n_experts experts of MOE_W4_EXPERT_WEIGHTS elements each: gate
 * [512][2048], up [512][2048], down [2048][512] (the row order of the codes).
 * codes, scales: the layouts of moe_w4_forward (expert e at e*1,572,864 B and
 * at element e*24,576).  All pointers 16-byte aligned device pointers; the
 * outputs must not overlap w or each other.  n_experts == 0 enqueues nothing.
 * EINVAL for a bad pointer, alignment, overlap or n_experts outside
 * [0, MOE_W4_PACK_MAX_EXPERTS]; EDEVICE if the launch failed. */
#define MOE_W4_EXPERT_WEIGHTS 3145728
#define MOE_W4_PACK_MAX_EXPERTS 65536
int moe_w4_pack_experts(const void *w, int64_t n_experts, void *codes, void *scales, void *stream);

/* Dense SwiGLU MLP block, the neighbour of the MoE blocks in the same model
 * (NInfer README of Flint, "What is inside": blocks 0 and 1 are dense SwiGLU
 * MLPs of width 6144; the model card keeps every linear bf16):
 *   y = bf16_rne( Wd( silu(Wg x) * (Wu x) ) )     fp32 sums of exact bf16 products,
 *                                                  the SwiGLU product rounded to bf16 once
 * w: bf16, MOE_W4_DENSE_WEIGHTS elements: gate [6144][2048], up [6144][2048],
 * down [2048][6144].  x, y: bf16 [T][2048].  workspace: at least
 * moe_w4_dense_mlp_workspace_bytes(T) bytes, contents on entry irrelevant.
 * Validation, T == 0 and errors as for moe_w4_forward. */
#define MOE_W4_DENSE_INTER 6144
#define MOE_W4_DENSE_WEIGHTS 37748736
size_t moe_w4_dense_mlp_workspace_bytes(int64_t T);
int moe_w4_dense_mlp(const void *x, const void *w, int64_t T, void *y, void *workspace, size_t workspace_bytes,
                     void *stream);

/* Static text for a status code. */
const char *moe_w4_status_string(int status);

/* The hipError_t behind the last MOE_W4_EDEVICE returned on this thread (0 if none). */
int moe_w4_last_device_error(void);

/* Library version, major*10000 + minor*100 + patch. */
int moe_w4_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_W4_H */
