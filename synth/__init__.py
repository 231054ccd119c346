"""Seeded synthetic inputs for the int4 routed-expert MoE layer.

This module is shared by the CPU oracle, the tests and the benchmark.  It
holds no arithmetic of the layer itself: it only turns (seed, tensor id,
element index) into bit patterns — int4 codes, bf16 numbers and a router
bias — in the exact memory layout the C-ABI library takes.

Generator (a published counter-based one, not taken from the pages):

* ``mix64`` is the 64-bit finaliser of SplitMix64 (Steele, Lea and Flood,
  "Fast splittable pseudorandom number generators", OOPSLA 2014; the
  constants are the "Mix13" variant that Java's SplittableRandom uses).
* ``r(seed, tid, i) = mix64(mix64(seed*G + tid) + (i + 1)*G)`` mod 2**64
  with ``G = 0x9E3779B97F4A7C15`` (the golden-ratio increment).
* An int4 code is ``(r >> 60) - 8``: uniform on [-8, 7].
* A "~N(0, sigma)" bf16 is an Irwin–Hall sum of the four 16-bit lanes of
  ``r``, centred: ``S = sum_q ((r >> 16q) & 0xFFFF) - 131070``, then
  ``bf16_rne(f32(S) * f32(sigma*sqrt(3)/65536))`` — one fp32 multiply and
  one round-to-nearest-even to bf16, with no transcendental function, so an
  independent device implementation can match it bit for bit.  The
  distribution is bounded at about +-3.46 sigma.
* ``|N(0,1)| * 0.01`` scales use ``|S|`` with sigma = 0.01.

Shapes and formats follow the Flint int4-expert model card
(Aijuus/flint-w4exp, table row "weights": int4 codes, group 128, bf16
scale, fwht128 rotation) and the NInfer README of Flint
(WaveCut/Flint-UD-Q4_K_XL-NInfer-v3, section "What is inside": each expert's
gate rows followed by its up rows, 2 x 512, and 2,048 down rows; shared
expert of 1024; router rows bf16 widened to fp32).  Because the codes are
drawn directly, they *are* the weights in the rotated basis.

Memory layout (the C-ABI layout; row-major, K contiguous):

* ``x``        bf16 [T][2048]
* ``router_w`` bf16 [256][2048]
* ``codes``    u8   [256][1,572,864]: per expert gate[512][1024 B],
  up[512][1024 B], down[2048][256 B]; element k of a row sits in the low
  nibble of byte k//2 when k is even, the high nibble when odd; two's
  complement.
* ``scales``   bf16 [256][24,576]: per expert gate[512][16], up[512][16],
  down[2048][4]; scale g covers K elements [128g, 128g+128).
* ``shared_w`` bf16: gate[1024][2048], up[1024][2048], down[2048][1024].

Tensor ids: ``tid = 64*layer + kind`` with kinds 0 x, 1 router, 2/3/4
gate/up/down codes, 5/6/7 gate/up/down scales, 8/9/10 shared
gate/up/down, 11 bias choice.  The element index is the flat index of the
element inside the tensor of that kind (int4 elements, not bytes).
"""
from __future__ import annotations

import math

import numpy as np

# ---- layer shapes -------------------------------------------------------
HIDDEN = 2048          # H: model width (K of gate/up, N of down)
N_EXPERTS = 256        # routed experts per MoE block
TOP_K = 6              # experts per token
INTER = 512            # routed expert intermediate width
SHARED_INTER = 1024    # shared expert intermediate width
GROUP = 128            # K elements per bf16 scale (and per Hadamard block)
N_MOE_LAYERS = 47      # MoE blocks of the 49-block model

GU_ROWS = 2 * INTER                                  # 1024 [gate; up] rows
CODE_BYTES_GU = GU_ROWS * HIDDEN // 2                # 1,048,576
CODE_BYTES_D = HIDDEN * INTER // 2                   # 524,288
CODE_BYTES_PER_EXPERT = CODE_BYTES_GU + CODE_BYTES_D  # 1,572,864
SCALES_GU = GU_ROWS * (HIDDEN // GROUP)              # 16,384 bf16
SCALES_D = HIDDEN * (INTER // GROUP)                 # 8,192 bf16
SCALES_PER_EXPERT = SCALES_GU + SCALES_D             # 24,576 bf16
SHARED_ELEMS = 3 * SHARED_INTER * HIDDEN             # 6,291,456 bf16

KIND_X, KIND_ROUTER = 0, 1
KIND_CODE_G, KIND_CODE_U, KIND_CODE_D = 2, 3, 4
KIND_SCALE_G, KIND_SCALE_U, KIND_SCALE_D = 5, 6, 7
KIND_SH_G, KIND_SH_U, KIND_SH_D = 8, 9, 10
KIND_BIAS = 11
KIND_NV_SCALE, KIND_NV_TSCALE = 12, 13

SIGMA_X = 1.0
SIGMA_W = 0.02
SIGMA_SCALE = 0.01

_G = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_MASK64 = (1 << 64) - 1


def tensor_id(layer: int, kind: int) -> int:
    return 64 * int(layer) + int(kind)


def mix64(z: np.ndarray) -> np.ndarray:
    """SplitMix64 finaliser on a uint64 array (wrapping arithmetic)."""
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = z ^ (z >> np.uint64(30))
        z = z * _M1
        z = z ^ (z >> np.uint64(27))
        z = z * _M2
        z = z ^ (z >> np.uint64(31))
    return z


def mix64_int(z: int) -> int:
    """Pure-Python SplitMix64 finaliser (used to pin the numpy version)."""
    z &= _MASK64
    z ^= z >> 30
    z = (z * 0xBF58476D1CE4E5B9) & _MASK64
    z ^= z >> 27
    z = (z * 0x94D049BB133111EB) & _MASK64
    z ^= z >> 31
    return z


def stream_key(seed: int, tid: int) -> int:
    return mix64_int((int(seed) * 0x9E3779B97F4A7C15 + int(tid)) & _MASK64)


def draw(seed: int, tid: int, idx) -> np.ndarray:
    """r(seed, tid, i) for an array of element indices."""
    key = np.uint64(stream_key(seed, tid))
    i = np.asarray(idx, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return mix64(key + (i + np.uint64(1)) * _G)


def draw_int(seed: int, tid: int, i: int) -> int:
    """Pure-Python r(seed, tid, i)."""
    return mix64_int(stream_key(seed, tid) + (int(i) + 1) * 0x9E3779B97F4A7C15)


# ---- value maps ---------------------------------------------------------
def irwin_hall(r: np.ndarray) -> np.ndarray:
    """Centred sum of the four 16-bit lanes of r, as int64 in [-131070, 131070]."""
    r = np.asarray(r, dtype=np.uint64)
    s = np.zeros(r.shape, dtype=np.int64)
    for q in range(4):
        s += ((r >> np.uint64(16 * q)) & np.uint64(0xFFFF)).astype(np.int64)
    return s - 131070


def normal_multiplier(sigma: float) -> np.float32:
    """f32(sigma * sqrt(3) / 65536): the one constant of the normal map."""
    return np.float32(sigma * math.sqrt(3.0) / 65536.0)


def f32_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16 bit pattern (NaN kept as quiet NaN)."""
    u = np.asarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    rounded = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) & np.uint64(0xFFFF)
    nan = np.isnan(np.asarray(v, dtype=np.float32))
    out = rounded.astype(np.uint16)
    out[nan] = 0x7FC0
    return out


def normal_bf16_bits(seed, tid, idx, sigma) -> np.ndarray:
    s = irwin_hall(draw(seed, tid, idx)).astype(np.float32)
    return f32_to_bf16_bits(s * normal_multiplier(sigma))


def abs_normal_bf16_bits(seed, tid, idx, sigma) -> np.ndarray:
    s = np.abs(irwin_hall(draw(seed, tid, idx))).astype(np.float32)
    return f32_to_bf16_bits(s * normal_multiplier(sigma))


def int4_values(seed, tid, idx) -> np.ndarray:
    """Signed int4 codes in [-8, 7] as int8."""
    r = draw(seed, tid, idx)
    return ((r >> np.uint64(60)).astype(np.int16) - 8).astype(np.int8)


def pack_int4(vals: np.ndarray) -> np.ndarray:
    """Pack int4 values along the last axis: even k -> low nibble."""
    v = np.asarray(vals, dtype=np.int8).astype(np.uint8) & np.uint8(0xF)
    return (v[..., 0::2] | (v[..., 1::2] << np.uint8(4))).astype(np.uint8)


# ---- tensors in the library's layout -------------------------------------
def gen_x(seed: int, T: int, layer: int = 0) -> np.ndarray:
    """bf16 bits [T][2048], ~N(0, 1)."""
    idx = np.arange(T * HIDDEN, dtype=np.uint64)
    return normal_bf16_bits(seed, tensor_id(layer, KIND_X), idx, SIGMA_X).reshape(T, HIDDEN)


def gen_router(seed: int, layer: int = 0) -> np.ndarray:
    """bf16 bits [256][2048], ~N(0, 0.02)."""
    idx = np.arange(N_EXPERTS * HIDDEN, dtype=np.uint64)
    return normal_bf16_bits(seed, tensor_id(layer, KIND_ROUTER), idx, SIGMA_W).reshape(N_EXPERTS, HIDDEN)


def gen_expert_codes_values(seed: int, layer: int, e: int):
    """Signed int4 values of expert e: (gate [512,2048], up [512,2048], down [2048,512])."""
    n_gu = INTER * HIDDEN
    base = np.arange(n_gu, dtype=np.uint64) + np.uint64(e * n_gu)
    g = int4_values(seed, tensor_id(layer, KIND_CODE_G), base).reshape(INTER, HIDDEN)
    u = int4_values(seed, tensor_id(layer, KIND_CODE_U), base).reshape(INTER, HIDDEN)
    d = int4_values(seed, tensor_id(layer, KIND_CODE_D), base).reshape(HIDDEN, INTER)
    return g, u, d


def gen_expert_scales_bits(seed: int, layer: int, e: int):
    """bf16 bits of expert e's scales: gate [512,16], up [512,16], down [2048,4]."""
    ng = INTER * (HIDDEN // GROUP)
    base = np.arange(ng, dtype=np.uint64) + np.uint64(e * ng)
    sg = abs_normal_bf16_bits(seed, tensor_id(layer, KIND_SCALE_G), base, SIGMA_SCALE).reshape(INTER, HIDDEN // GROUP)
    su = abs_normal_bf16_bits(seed, tensor_id(layer, KIND_SCALE_U), base, SIGMA_SCALE).reshape(INTER, HIDDEN // GROUP)
    nd = HIDDEN * (INTER // GROUP)
    based = np.arange(nd, dtype=np.uint64) + np.uint64(e * nd)
    sd = abs_normal_bf16_bits(seed, tensor_id(layer, KIND_SCALE_D), based, SIGMA_SCALE).reshape(HIDDEN, INTER // GROUP)
    return sg, su, sd


def expert_code_bytes(g: np.ndarray, u: np.ndarray, d: np.ndarray) -> np.ndarray:
    """One expert's packed codes in the library layout (1,572,864 bytes)."""
    return np.concatenate([pack_int4(g).ravel(), pack_int4(u).ravel(), pack_int4(d).ravel()])


def expert_scale_bits(sg, su, sd) -> np.ndarray:
    return np.concatenate([np.ravel(sg), np.ravel(su), np.ravel(sd)]).astype(np.uint16)


def gen_codes_scales(seed: int, layer: int = 0, experts=None):
    """Packed codes u8 [E][1572864] and scale bits u16 [E][24576] for a list of experts."""
    experts = range(N_EXPERTS) if experts is None else list(experts)
    experts = list(experts)
    codes = np.empty((len(experts), CODE_BYTES_PER_EXPERT), dtype=np.uint8)
    scales = np.empty((len(experts), SCALES_PER_EXPERT), dtype=np.uint16)
    for i, e in enumerate(experts):
        codes[i] = expert_code_bytes(*gen_expert_codes_values(seed, layer, e))
        scales[i] = expert_scale_bits(*gen_expert_scales_bits(seed, layer, e))
    return codes, scales


# ---- NVFP4 experts --------------------------------------------------------
# Codes: the same random bytes as the int4 codes of the seed (every nibble
# pattern is a valid E2M1 code, uniform over the 16).  Block scales: E4M3
# bytes with sign 0, exponent field uniform in 0..4 and any mantissa (values
# m * 2**-9 up to 1.875 * 2**-3, subnormals included).  Tensor scales: fp32
# in [0.125, 0.25).  With uniform codes (rms 2.93) the weights have rms
# about 0.03, like the int4 experts.
NV_SCALE_BYTES_PER_EXPERT = 3 * INTER * HIDDEN // 16   # 196,608


def nvfp4_scale_bytes(seed, tid, idx) -> np.ndarray:
    r = draw(seed, tid, idx)
    e = r % np.uint64(5)
    m = (r >> np.uint64(8)) & np.uint64(7)
    return ((e << np.uint64(3)) | m).astype(np.uint8)


def gen_nvfp4_scales(seed: int, layer: int = 0, experts=None) -> np.ndarray:
    """E4M3 block-scale bytes u8 [E][196608] (gate [512][128], up, down [2048][32])."""
    experts = range(N_EXPERTS) if experts is None else list(experts)
    experts = list(experts)
    out = np.empty((len(experts), NV_SCALE_BYTES_PER_EXPERT), dtype=np.uint8)
    base = np.arange(NV_SCALE_BYTES_PER_EXPERT, dtype=np.uint64)
    for i, e in enumerate(experts):
        out[i] = nvfp4_scale_bytes(seed, tensor_id(layer, KIND_NV_SCALE),
                                   base + np.uint64(e * NV_SCALE_BYTES_PER_EXPERT))
    return out


def gen_nvfp4_tensor_scales(seed: int, layer: int = 0) -> np.ndarray:
    """fp32 [256][3] tensor scales (gate, up, down) in [0.125, 0.25)."""
    r = draw(seed, tensor_id(layer, KIND_NV_TSCALE), np.arange(3 * N_EXPERTS, dtype=np.uint64))
    u = (r >> np.uint64(40)).astype(np.float64) / float(1 << 24)
    return (0.125 * (1.0 + u)).astype(np.float32).reshape(N_EXPERTS, 3)


def gen_shared(seed: int, layer: int = 0) -> np.ndarray:
    """bf16 bits of the shared expert, flat [gate 1024x2048 | up 1024x2048 | down 2048x1024]."""
    n = SHARED_INTER * HIDDEN
    idx = np.arange(n, dtype=np.uint64)
    g = normal_bf16_bits(seed, tensor_id(layer, KIND_SH_G), idx, SIGMA_W)
    u = normal_bf16_bits(seed, tensor_id(layer, KIND_SH_U), idx, SIGMA_W)
    d = normal_bf16_bits(seed, tensor_id(layer, KIND_SH_D), idx, SIGMA_W)
    return np.concatenate([g, u, d])


def skew_experts(seed: int, n_hot: int = 26, layer: int = 0) -> np.ndarray:
    """The n_hot experts with the smallest r(seed, bias-tid, e), ascending by e."""
    r = draw(seed, tensor_id(layer, KIND_BIAS), np.arange(N_EXPERTS, dtype=np.uint64))
    order = np.argsort(r, kind="stable")
    return np.sort(order[:n_hot]).astype(np.int64)


def skew_bias(seed: int, n_hot: int = 26, value: float = 3.0, layer: int = 0) -> np.ndarray:
    """fp32 [256] additive router-logit bias: `value` on the chosen experts, 0 elsewhere."""
    b = np.zeros(N_EXPERTS, dtype=np.float32)
    b[skew_experts(seed, n_hot, layer)] = np.float32(value)
    return b


# ---- the five measured workloads -----------------------------------------
# name -> (T, seed of x, seed of the weights, router bias seed or None)
CONFIGS = {
    "decode_t1": dict(T=1, x_seed=0, w_seed=0, bias_seed=None),
    "decode_t32": dict(T=32, x_seed=1, w_seed=0, bias_seed=None),
    "prefill_t2048": dict(T=2048, x_seed=2, w_seed=0, bias_seed=None),
    "prefill_t2048_skew": dict(T=2048, x_seed=3, w_seed=0, bias_seed=3),
}
STACK_SEED = 4


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
