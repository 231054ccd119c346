"""CPU oracle of the Flint int4 routed-expert MoE layer — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call this module.  The library and its Python
binding never do: they share no code, constant table or helper with it.

Everything here is plain NumPy in float64 and follows the pages step by step:

* Flint model card for the int4-expert container (Aijuus/flint-w4exp),
  introduction and table row "weights": 256 experts, 6 chosen per token, and
  one shared expert without a gate; the routed experts hold int4 codes with a
  bf16 scale for each 128 elements of K, in a basis rotated by the 128-point
  Hadamard transform (fwht128); the shared expert and the other linears are
  bf16.
* NInfer README of Flint (WaveCut/Flint-UD-Q4_K_XL-NInfer-v3), section
  "What is inside": sigmoid router scores renormalised over the 6 chosen
  experts; each expert holds gate rows then up rows (2 x 512) and 2,048 down
  rows; a shared expert of width 1024 with gate and up rows; router rows
  kept in fp32, widened exactly from bf16.  Section "Quality": fp16 sums of
  the routed experts overflow, so every sum here is at least fp32 (here fp64).
* bloomery issue #632 ("model: Flint ..."), description and the design
  thread: sigmoid router, 6 of 256 experts, no router correction bias, and
  the normalisation policy max(sum of selected scores, 2**-14) with the six
  (index, fp32 weight) slots handed to the expert stage.
* Flint NVFP4 repack (kekzle/Flint-NVFP4), rows "Layout per Linear" and
  "Declaration": the second expert container, E2M1 codes with E4M3 block
  scales per 16 columns and an F32 tensor scale, W4A16 (the section at the
  end of this module, with its readings).

Readings where the pages are silent:

* Hadamard: Sylvester order, H[i][j] = (-1)**popcount(i & j) / sqrt(128),
  no random signs; symmetric and its own inverse.
* Rotation acts on the K side of all three expert planes: x before gate/up
  (16 blocks), a = silu(g)*u before down (4 blocks).
* Dequantisation is symmetric: w = code * scale; group g of a row covers
  K in [128g, 128g+128); even K in the low nibble; two's complement codes.
* Top-6 is chosen on fp32 logits (the precision the pages give the router),
  higher logit first, equal logits to the lower expert index; the slot
  order is that order.  A token whose 6th/7th fp64 logit gap is <= 1e-3 is
  flagged as a near-tie.
* The optional router bias is added to the logit before selection and
  before the sigmoid (a synthetic skew; Flint itself has none).
* Router policy variants (bloomery issue #632, design thread and the
  follow-up host-policy slice: the router description distinguishes no
  normalisation, the legacy selected-sum and the selected-sum with the
  2**-14 floor, and a bias that is absent or used for selection only):
  norm "floor" (Flint, the default) divides by max(sum, 2**-14), "sum"
  divides by the plain sum, "none" keeps the sigmoid scores; bias_mode
  "logit" (default) adds the bias to the logit for both the choice and the
  sigmoid, "select" adds it for the choice only.
* silu(v) = v / (1 + exp(-v)); the shared expert is added with weight 1.
* The shared expert (and the dense MLP blocks) are bf16 linears: the input of
  the down linear, h = silu(g) * u, is rounded to bf16 once (g and u exact).
  The routed experts' activations are not rounded (the expert weights are
  int4; the pages give their activations no narrower format).
* A token whose 6th/7th fp64 logit gap is <= 1e-3 is a near-tie (its chosen
  set is decided by rounding); one whose chosen logits have two within 1e-3
  of each other is an order tie (their slot order is decided by rounding).
* y is rounded once, fp64 -> bf16 round-to-nearest-even.

Parity pins live in ``tests/test_oracle_*.py``.  Absolute output values on
the synthetic workloads are "parity unpinned" against the pages (they print
no worked example of the layer); the pins constrain every step instead.
"""
from __future__ import annotations

import math

import numpy as np

H = 2048
E = 256
K_TOP = 6
I_R = 512
I_S = 1024
G = 128
NEAR_TIE_GAP = 1e-3
WEIGHT_FLOOR = 2.0 ** -14
RMS_EPS = 1e-6


# ---------------------------------------------------------------- numbers
def bf16_to_f64(bits) -> np.ndarray:
    """Widen bf16 bit patterns exactly (bf16 is the top half of an fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(v) -> np.ndarray:
    """Round float64 to the nearest bf16 (ties to even), one rounding.

    bf16 keeps 8 significant bits and fp32's exponent range; below 2**-126
    the spacing is 2**-133.  Overflow goes to +-inf, NaN to a quiet NaN.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    finite = np.isfinite(a) & (a > 0)
    _, e = np.frexp(np.where(finite, a, 1.0))            # a = m * 2**e, m in [0.5, 1)
    step_exp = np.where(e - 1 >= -126, e - 8, -133)       # 8 significant bits / subnormal spacing
    q = np.ldexp(np.where(finite, a, 0.0), -step_exp)     # exact scaling by a power of two
    r = np.rint(q)                                        # round half to even
    val = np.ldexp(r, step_exp)
    over = val >= 2.0 ** 128
    with np.errstate(over="ignore"):
        bits = (val.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint32)
    bits = np.where(over | np.isinf(a), 0x7F80, bits)
    bits = np.where(a == 0, 0, bits)
    bits = bits | np.where(np.signbit(v), 0x8000, 0)
    bits = np.where(np.isnan(v), 0x7FC0, bits)
    return bits.astype(np.uint16)


def f32_round(v) -> np.ndarray:
    """Round to fp32 (IEEE round-to-nearest-even), returned as float64."""
    return np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)


def sigmoid(v):
    return 1.0 / (1.0 + np.exp(-np.asarray(v, dtype=np.float64)))


def silu(v):
    v = np.asarray(v, dtype=np.float64)
    return v / (1.0 + np.exp(-v))


# -------------------------------------------------------------- Hadamard
def hadamard(n: int = G) -> np.ndarray:
    """Normalised Sylvester Hadamard matrix of order n (a power of two).

    Built by the doubling recursion H_2m = [[H_m, H_m], [H_m, -H_m]] and
    divided by sqrt(n), so it is symmetric and orthogonal (its own inverse).
    """
    h = np.array([[1.0]])
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    assert h.shape[0] == n
    return h / math.sqrt(n)


def rotate_blocks(v: np.ndarray, block: int = G) -> np.ndarray:
    """Apply the normalised 128-point Hadamard to every 128-block of the last axis."""
    v = np.asarray(v, dtype=np.float64)
    hn = hadamard(block)
    shp = v.shape
    nb = shp[-1] // block
    return (v.reshape(shp[:-1] + (nb, block)) @ hn).reshape(shp)


# --------------------------------------------------------------- weights
def unpack_int4(packed: np.ndarray, k: int) -> np.ndarray:
    """Packed bytes [..., k/2] -> signed int4 values [..., k] (even k low nibble)."""
    p = np.asarray(packed, dtype=np.uint8)
    lo = (p & 0x0F).astype(np.int16)
    hi = (p >> 4).astype(np.int16)
    vals = np.empty(p.shape[:-1] + (k,), dtype=np.int16)
    vals[..., 0::2] = lo
    vals[..., 1::2] = hi
    vals[vals >= 8] -= 16                # two's complement
    return vals


def dequantize(packed_rows: np.ndarray, scale_bits: np.ndarray, k: int) -> np.ndarray:
    """W[n, k] = code[n, k] * scale[n, k // 128] in float64."""
    codes = unpack_int4(packed_rows, k).astype(np.float64)
    s = bf16_to_f64(scale_bits)                      # [n, k/128]
    return codes * np.repeat(s, G, axis=1)


def expert_planes(code_bytes: np.ndarray, scale_bits: np.ndarray):
    """Split one expert's blobs (library layout) into dequantised gate, up, down."""
    cb = np.asarray(code_bytes, dtype=np.uint8)
    sb = np.asarray(scale_bits, dtype=np.uint16)
    nb_gu = I_R * H // 2
    g_rows = cb[:nb_gu].reshape(I_R, H // 2)
    u_rows = cb[nb_gu:2 * nb_gu].reshape(I_R, H // 2)
    d_rows = cb[2 * nb_gu:].reshape(H, I_R // 2)
    ns = I_R * (H // G)
    sg = sb[:ns].reshape(I_R, H // G)
    su = sb[ns:2 * ns].reshape(I_R, H // G)
    sd = sb[2 * ns:].reshape(H, I_R // G)
    return dequantize(g_rows, sg, H), dequantize(u_rows, su, H), dequantize(d_rows, sd, I_R)


def shared_planes(shared_bits: np.ndarray):
    sb = bf16_to_f64(shared_bits)
    n = I_S * H
    return sb[:n].reshape(I_S, H), sb[n:2 * n].reshape(I_S, H), sb[2 * n:].reshape(H, I_S)


# ---------------------------------------------------------------- router
NORMS = ("floor", "sum", "none")
BIAS_MODES = ("logit", "select")


def route(x: np.ndarray, router_bits: np.ndarray, bias=None, norm="floor", bias_mode="logit"):
    """Sigmoid top-6 router; by default the renormaliser has the 2**-14 floor.

    x: float64 [T, K] (already widened); router_bits: bf16 bits [n_experts, K]
    (256 x 2048 for Flint; any n_experts >= 7 works).  norm / bias_mode: the
    policy variants above.  Returns a dict with the fp64 logits the choice is
    made on, their fp32 rounding, the logits the sigmoid takes (logits_w),
    topk_idx [T, 6], topk_w [T, 6] (float64), the 6th-7th gap and the
    near-tie flags, and the smallest gap between consecutive chosen logits
    (order_gap) with its flags (order_tie).
    """
    if norm not in NORMS or bias_mode not in BIAS_MODES:
        raise ValueError("unknown router policy")
    R = bf16_to_f64(router_bits)                      # [256, 2048]
    unbiased = x @ R.T                                # [T, 256]
    logits = unbiased
    if bias is not None:
        logits = logits + np.asarray(bias, dtype=np.float64)[None, :]
    logits_w = unbiased if bias_mode == "select" else logits
    l32 = f32_round(logits)
    T, n_exp = logits.shape
    idx = np.empty((T, K_TOP), dtype=np.int32)
    gap = np.empty(T, dtype=np.float64)
    order_gap = np.empty(T, dtype=np.float64)
    experts = np.arange(n_exp)
    for t in range(T):
        # higher fp32 logit first; equal logits -> lower expert index
        order = np.lexsort((experts, -l32[t]))
        idx[t] = order[:K_TOP]
        srt = np.sort(logits[t])[::-1]
        gap[t] = srt[K_TOP - 1] - srt[K_TOP]
        order_gap[t] = np.min(srt[:K_TOP - 1] - srt[1:K_TOP])
    sel = np.take_along_axis(logits_w, idx.astype(np.int64), axis=1)
    sig = sigmoid(sel)
    if norm == "floor":
        w = sig / np.maximum(sig.sum(axis=1, keepdims=True), WEIGHT_FLOOR)
    elif norm == "sum":
        w = sig / sig.sum(axis=1, keepdims=True)
    else:
        w = sig
    return dict(logits=logits, logits32=l32, logits_w=logits_w, topk_idx=idx, topk_w=w,
                gap=gap, near_tie=gap <= NEAR_TIE_GAP, order_gap=order_gap, order_tie=order_gap <= NEAR_TIE_GAP)


def sort_assignments(topk_idx: np.ndarray):
    """Counting sort of the 6T assignments a = 6t + j by expert, stable in a."""
    flat = np.asarray(topk_idx, dtype=np.int64).ravel()
    counts = np.bincount(flat, minlength=E)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    perm = np.argsort(flat, kind="stable")
    pos = np.empty_like(perm)
    pos[perm] = np.arange(perm.size)
    return dict(counts=counts.astype(np.int32), offsets=offsets.astype(np.int32),
                perm=perm.astype(np.int32), pos=pos.astype(np.int32))


# ---------------------------------------------------------------- experts
def expert_swiglu(xt: np.ndarray, wg, wu, wd) -> np.ndarray:
    """One rotated int4 expert on rotated inputs xt [n, 2048] -> [n, 2048]."""
    g = xt @ wg.T
    u = xt @ wu.T
    a = silu(g) * u
    at = rotate_blocks(a)
    return at @ wd.T


def bf16_round(v) -> np.ndarray:
    """v rounded to the nearest bf16 (ties to even), as float64."""
    return bf16_to_f64(f64_to_bf16_bits(v))


def shared_expert(x: np.ndarray, shared_bits: np.ndarray) -> np.ndarray:
    """Ungated bf16 SwiGLU of width 1024 on the unrotated input: its down
    linear takes h = silu(x Wg^T) * (x Wu^T) rounded to bf16 once."""
    sg, su, sd = shared_planes(shared_bits)
    return bf16_round(silu(x @ sg.T) * (x @ su.T)) @ sd.T


def _map_experts(fn, experts, pool):
    """[fn(e) for e in experts], evaluated by `pool` (a concurrent.futures
    executor) if one is given.  Each expert's output is computed on its own and
    the caller sums them in the order of `experts` either way, so the result
    is the same bits with or without a pool."""
    return list(pool.map(fn, experts)) if pool is not None else [fn(e) for e in experts]


def moe_layer(x_bits, router_bits, expert_blobs, shared_bits, bias=None, tokens=None, norm="floor",
              bias_mode="logit", pool=None):
    """The layer: y = bf16( sum_j w_j * E_{e_j}(x) + S(x) ).

    x_bits: bf16 bits [T, 2048]; router_bits: bf16 bits [256, 2048];
    expert_blobs(e) -> (code bytes [1572864], scale bits [24576]) in the
    library layout; shared_bits: bf16 bits [6291456]; bias: fp32 [256] or None.
    tokens: optional subset of token rows whose expert outputs and y are
    computed (routing and the sort always cover all T tokens).  norm,
    bias_mode: the router policy (see route).  pool: optional executor that
    evaluates the experts concurrently (same result).
    """
    x = bf16_to_f64(x_bits)
    T = x.shape[0]
    rt = route(x, router_bits, bias, norm, bias_mode)
    srt = sort_assignments(rt["topk_idx"])
    rows = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    xt = rotate_blocks(x[rows])
    routed = np.zeros((rows.size, H), dtype=np.float64)
    need = {}
    for r_i, t in enumerate(rows):
        for j in range(K_TOP):
            need.setdefault(int(rt["topk_idx"][t, j]), []).append((r_i, j))
    def expert_out(e):
        wg, wu, wd = expert_planes(*expert_blobs(e))
        ri = np.array([p[0] for p in need[e]])
        return expert_swiglu(xt[ri], wg, wu, wd)

    experts = sorted(need)
    for e, o in zip(experts, _map_experts(expert_out, experts, pool)):
        lst = need[e]
        ri = np.array([p[0] for p in lst])
        jj = np.array([p[1] for p in lst])
        w = rt["topk_w"][rows[ri], jj]
        for n in range(len(lst)):
            routed[ri[n]] += w[n] * o[n]
    z = shared_expert(x[rows], shared_bits)
    y = routed + z
    out = dict(rt)
    out.update(srt)
    out.update(rows=rows, routed=routed, shared=z, y=y, y_bits=f64_to_bf16_bits(y))
    return out


def moe_layer_dense(x_bits, router_bits, expert_blobs, shared_bits, bias=None):
    """Every expert evaluated, with the gate of non-selected experts set to zero."""
    x = bf16_to_f64(x_bits)
    T = x.shape[0]
    rt = route(x, router_bits, bias)
    gates = np.zeros((T, E))
    for t in range(T):
        gates[t, rt["topk_idx"][t]] = rt["topk_w"][t]
    xt = rotate_blocks(x)
    y = shared_expert(x, shared_bits)
    for e in range(E):
        wg, wu, wd = expert_planes(*expert_blobs(e))
        y = y + gates[:, e:e + 1] * expert_swiglu(xt, wg, wu, wd)
    return dict(y=y, y_bits=f64_to_bf16_bits(y), gates=gates)


# --------------------------------------------------------- dense MLP block
I_D = 6144
DENSE_WEIGHTS = 3 * I_D * H


def dense_mlp(x_bits: np.ndarray, w_bits: np.ndarray) -> dict:
    """Dense SwiGLU MLP block (NInfer README of Flint, "What is inside": blocks 0
    and 1 are dense SwiGLU MLPs of width 6144; bf16 like every linear of the
    model card): y = bf16( Wd bf16(silu(Wg x) * (Wu x)) ), fp64 otherwise (the
    down linear's input rounded to bf16 once, as in the shared expert).

    x_bits: bf16 bits [T, 2048]; w_bits: bf16 bits [DENSE_WEIGHTS], gate
    [6144][2048], up [6144][2048], down [2048][6144].
    """
    x = bf16_to_f64(x_bits)
    w = bf16_to_f64(np.asarray(w_bits, dtype=np.uint16).ravel())
    n = I_D * H
    wg, wu, wd = w[:n].reshape(I_D, H), w[n:2 * n].reshape(I_D, H), w[2 * n:].reshape(H, I_D)
    y = bf16_round(silu(x @ wg.T) * (x @ wu.T)) @ wd.T
    return dict(y=y, y_bits=f64_to_bf16_bits(y))


# ------------------------------------------------------------------ stack
def rmsnorm(x: np.ndarray) -> np.ndarray:
    """x / sqrt(mean(x^2) + 1e-6), unit gain, per row."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + RMS_EPS)


def stack_step(resid: np.ndarray, layer_inputs, pool=None):
    """x_{l+1} = x_l + moe_l(bf16(rmsnorm(x_l))) over the given layers.

    layer_inputs: iterable of (router_bits, expert_blobs, shared_bits) per layer.
    resid: fp32-valued residual [T, 2048] (float64 array holding fp32 values).
    The layer boundary is bf16 (the library's x and y); the residual is fp32.
    Returns the final residual and the bf16 inputs of every layer.
    """
    x = f32_round(resid)
    inputs = []
    for router_bits, blobs, shared_bits in layer_inputs:
        xin = f64_to_bf16_bits(rmsnorm(x))
        inputs.append(xin)
        out = moe_layer(xin, router_bits, blobs, shared_bits, pool=pool)
        x = f32_round(x + bf16_to_f64(out["y_bits"]))
    return x, inputs


# ------------------------------------------------------- test-only quantizer
def quantize_rotated(w: np.ndarray):
    """Rotate a float weight [n, k] on K, then int4-quantise per group of 128.

    The pages state the format (int4 codes, group 128, bf16 scale, fwht128
    rotation) and its error (11.7% relative Frobenius per expert plane, model
    card, "Why the linears stay bf16"), not the quantiser.  Reading used here:
    scale = bf16(absmax / 7) per group, code = clamp(rint(w_rot / scale), -8, 7).
    Returns (int4 values [n, k], scale bf16 bits [n, k/128]).
    """
    w = np.asarray(w, dtype=np.float64)
    n, k = w.shape
    wr = rotate_blocks(w)                              # W (I x Hn): the stored basis
    grp = wr.reshape(n, k // G, G)
    amax = np.abs(grp).max(axis=2)
    s_bits = f64_to_bf16_bits(amax / 7.0)
    s = bf16_to_f64(s_bits)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s[..., None] > 0, grp / s[..., None], 0.0)
    codes = np.clip(np.rint(q), -8, 7).astype(np.int16).reshape(n, k)
    return codes, s_bits


def fwht128_f32(v: np.ndarray) -> np.ndarray:
    """The fwht128 butterfly in fp32 on every 128-block of the last axis.

    The fast Walsh-Hadamard transform (Sylvester order): stages of stride
    h = 1, 2, ..., 64, each replacing (a, b) at distance h by (a + b, a - b),
    every add in fp32, then the fp32 factor 1/sqrt(128).  This is the
    rotation as a packer computes it in fp32; rotate_blocks is the same
    transform in fp64.
    """
    v = np.asarray(v, dtype=np.float32)
    shp = v.shape
    w = v.reshape(-1, G).copy()
    h = 1
    while h < G:
        q = w.reshape(-1, G // (2 * h), 2, h)
        a = q[:, :, 0, :].copy()
        b = q[:, :, 1, :].copy()
        q[:, :, 0, :] = a + b
        q[:, :, 1, :] = a - b
        w = q.reshape(-1, G)
        h *= 2
    return (w * np.float32(1.0 / math.sqrt(G))).reshape(shp)


def quantize_rotated_f32(w_bits: np.ndarray):
    """quantize_rotated with every decision taken in fp32, as the packer takes it.

    w_bits: bf16 bits [n, k].  Rotation by fwht128_f32; scale = bf16(fp32(absmax) /
    7) with the fp32 division rounded once to fp32 and then to bf16; code =
    clamp(round-half-even(fp32(w_rot / scale)), -8, 7), 0 where the scale is 0.
    Returns (int4 values [n, k], scale bf16 bits [n, k/128]).
    """
    w = bf16_to_f64(w_bits).astype(np.float32)         # exact: bf16 values are fp32 values
    n, k = w.shape
    grp = fwht128_f32(w).reshape(n, k // G, G)
    amax = np.abs(grp).max(axis=2)
    s_bits = f64_to_bf16_bits((amax / np.float32(7.0)).astype(np.float64))
    s = bf16_to_f64(s_bits).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s[..., None] > 0, grp / s[..., None], np.float32(0.0))
    codes = np.clip(np.rint(q), -8, 7).astype(np.int16).reshape(n, k)
    return codes, s_bits


def pack_int4(vals: np.ndarray) -> np.ndarray:
    """Signed int4 values [..., k] -> bytes [..., k/2]: element k in the low
    nibble of byte k/2 when k is even, two's complement (the inverse of
    unpack_int4)."""
    u = (np.asarray(vals, dtype=np.int16) & 0xF).astype(np.uint8)
    return (u[..., 0::2] | (u[..., 1::2] << 4)).astype(np.uint8)


EXPERT_WEIGHTS = 2 * I_R * H + H * I_R                 # 3,145,728 bf16 per expert


def pack_expert_bank(w_bits: np.ndarray):
    """bf16 weights of n experts [n, EXPERT_WEIGHTS] (gate [512][2048], up
    [512][2048], down [2048][512] each) -> (code bytes [n, 1572864], scale
    bits [n, 24576]) in the library layout, by quantize_rotated_f32 row by row."""
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    n = w_bits.shape[0]
    codes = np.empty((n, EXPERT_WEIGHTS // 2), dtype=np.uint8)
    scales = np.empty((n, EXPERT_WEIGHTS // G), dtype=np.uint16)
    for e in range(n):
        parts = [(w_bits[e, :2 * I_R * H].reshape(2 * I_R, H)), (w_bits[e, 2 * I_R * H:].reshape(H, I_R))]
        cb, sb = [], []
        for m in parts:
            c, sbits = quantize_rotated_f32(m)
            cb.append(pack_int4(c).ravel())
            sb.append(sbits.ravel())
        codes[e] = np.concatenate(cb)
        scales[e] = np.concatenate(sb)
    return codes, scales


def unrotated_effective(codes: np.ndarray, s_bits: np.ndarray) -> np.ndarray:
    """Effective weight in the original basis: (code * scale) (I x Hn)."""
    w = codes.astype(np.float64) * np.repeat(bf16_to_f64(s_bits), G, axis=1)
    return rotate_blocks(w)


# ------------------------------------------------------ NVFP4 expert format
# The second 4-bit expert container of the pages (Flint NVFP4 repack,
# kekzle/Flint-NVFP4, table rows "Repack", "Layout per Linear" and
# "Declaration"): per Linear, E2M1 codes two per byte, one E4M3 block scale
# per 16 columns and one F32 tensor scale, declared W4A16 (weights 4-bit,
# activations 16-bit).  Readings:
#
# * E2M1 and E4M3 are the OCP microscaling element and FP8 "FN" formats the
#   names denote: E2M1 = sign, 2 exponent bits (bias 1), 1 mantissa bit,
#   exponent 0 subnormal (0.5 * mantissa); E4M3 = sign, 4 exponent bits
#   (bias 7), 3 mantissa bits, exponent 0 subnormal (mantissa * 2**-9), no
#   infinities, S.1111.111 NaN.
# * w[n, k] = e2m1(code[n, k]) * e4m3(scale[n, k // 16]) * tensor_scale, with
#   "columns" the K (input) index of the row-major [out][in] weight; the code
#   of even k sits in the low nibble of its byte.
# * The weights stay in the original basis: no Hadamard on x or on a.
# * W4A16 is read as "the activations are not quantised": the layer is the
#   plain product with these weights, evaluated here exactly in float64
#   (no bf16 rounding of the dequantised weights).
NV_BLOCK = 16
NV_CODE_BYTES_PER_EXPERT = (2 * I_R * H + H * I_R) // 2     # 1,572,864
NV_SCALE_BYTES_PER_EXPERT = (2 * I_R * H + H * I_R) // 16   # 196,608


def e2m1_value(code) -> np.ndarray:
    """E2M1 code (0..15) -> float64."""
    c = np.asarray(code, dtype=np.int64)
    e = (c >> 1) & 3
    m = (c & 1).astype(np.float64)
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, (e - 1).astype(np.int32)))
    return np.where(c & 8, -mag, mag)


def e4m3_value(byte) -> np.ndarray:
    """E4M3 byte (0..255) -> float64 (NaN for S.1111.111)."""
    b = np.asarray(byte, dtype=np.int64)
    e = (b >> 3) & 15
    m = (b & 7).astype(np.float64)
    mag = np.where(e == 0, np.ldexp(m, -9), np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int32)))
    mag = np.where((e == 15) & ((b & 7) == 7), np.nan, mag)
    return np.where(b & 0x80, -mag, mag)


def unpack_e2m1(packed: np.ndarray, k: int) -> np.ndarray:
    """Packed bytes [..., k/2] -> E2M1 codes [..., k] (even k in the low nibble)."""
    p = np.asarray(packed, dtype=np.uint8)
    codes = np.empty(p.shape[:-1] + (k,), dtype=np.int64)
    codes[..., 0::2] = p & 0x0F
    codes[..., 1::2] = p >> 4
    return codes


def dequantize_nvfp4(packed_rows, scale_bytes, tensor_scale, k: int) -> np.ndarray:
    """W[n, k] = e2m1(code[n, k]) * e4m3(scale[n, k // 16]) * tensor_scale, float64."""
    s = e4m3_value(scale_bytes)
    return (e2m1_value(unpack_e2m1(packed_rows, k)) * np.repeat(s, NV_BLOCK, axis=-1)
            * float(np.float32(tensor_scale)))


def nvfp4_expert_planes(code_bytes, scale_bytes, tensor_scales):
    """One NVFP4 expert (library layout: codes gate [512][1024 B], up, down
    [2048][256 B]; E4M3 scales gate [512][128], up, down [2048][32]; f32
    tensor scales [gate, up, down]) -> dequantised gate, up, down."""
    cb = np.asarray(code_bytes, dtype=np.uint8)
    sb = np.asarray(scale_bytes, dtype=np.uint8)
    ts = np.asarray(tensor_scales, dtype=np.float32)
    nb = I_R * H // 2
    ns = I_R * H // NV_BLOCK
    wg = dequantize_nvfp4(cb[:nb].reshape(I_R, H // 2), sb[:ns].reshape(I_R, H // NV_BLOCK), ts[0], H)
    wu = dequantize_nvfp4(cb[nb:2 * nb].reshape(I_R, H // 2), sb[ns:2 * ns].reshape(I_R, H // NV_BLOCK), ts[1], H)
    wd = dequantize_nvfp4(cb[2 * nb:].reshape(H, I_R // 2), sb[2 * ns:].reshape(H, I_R // NV_BLOCK), ts[2], I_R)
    return wg, wu, wd


def moe_layer_nvfp4(x_bits, router_bits, expert_blobs, shared_bits, bias=None, tokens=None, pool=None):
    """The layer with NVFP4 experts: y = bf16( sum_j w_j * E_{e_j}(x) + S(x) ),
    E(x) = Wd (silu(Wg x) * (Wu x)) on the unrotated x.

    expert_blobs(e) -> (code bytes [1572864], E4M3 scale bytes [196608], f32
    tensor scales [3]); the rest as in moe_layer (Flint router policy, the
    optional pool).
    """
    x = bf16_to_f64(x_bits)
    T = x.shape[0]
    rt = route(x, router_bits, bias)
    srt = sort_assignments(rt["topk_idx"])
    rows = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    routed = np.zeros((rows.size, H), dtype=np.float64)
    need = {}
    for r_i, t in enumerate(rows):
        for j in range(K_TOP):
            need.setdefault(int(rt["topk_idx"][t, j]), []).append((r_i, j))
    def expert_out(e):
        wg, wu, wd = nvfp4_expert_planes(*expert_blobs(e))
        xe = x[rows[np.array([p[0] for p in need[e]])]]
        return (silu(xe @ wg.T) * (xe @ wu.T)) @ wd.T

    experts = sorted(need)
    for e, o in zip(experts, _map_experts(expert_out, experts, pool)):
        lst = need[e]
        ri = np.array([p[0] for p in lst])
        jj = np.array([p[1] for p in lst])
        w = rt["topk_w"][rows[ri], jj]
        for n in range(len(lst)):
            routed[ri[n]] += w[n] * o[n]
    z = shared_expert(x[rows], shared_bits)
    y = routed + z
    out = dict(rt)
    out.update(srt)
    out.update(rows=rows, routed=routed, shared=z, y=y, y_bits=f64_to_bf16_bits(y))
    return out
