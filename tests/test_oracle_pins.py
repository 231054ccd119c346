"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test checks one step of the layer against what the pages print, a closed
form, a textbook identity, an independent library routine (torch), brute force
on a tiny case, or an independent re-derivation written differently (the
rotation applied to the weights instead of the activations, a different int4
decode).  A dropped term, a wrong sign or index, or a transposed operand in
the oracle fails at least one of them.
"""
import itertools
import math

import numpy as np
import pytest
import torch

import synth
from oracle import moe_oracle as O
from tests.conftest import golden_constants

# ------------------------------------------------------------ helpers (tests only)
def butterfly_fwht(v):
    """In-place iterative fast Walsh-Hadamard transform on the last axis, normalised.

    Independent of the oracle's matrix construction: log2(n) add/sub stages.
    """
    v = np.array(v, dtype=np.float64, copy=True)
    n = v.shape[-1]
    h = 1
    while h < n:
        shp = v.shape[:-1] + (n // (2 * h), 2, h)
        w = v.reshape(shp)
        a = w[..., 0, :].copy()
        b = w[..., 1, :].copy()
        w[..., 0, :] = a + b
        w[..., 1, :] = a - b
        v = w.reshape(v.shape)
        h *= 2
    return v / math.sqrt(n)


def rotate_rows_blockwise(w, block=128):
    shp = w.shape
    return butterfly_fwht(w.reshape(shp[:-1] + (shp[-1] // block, block))).reshape(shp)


def decode_xor(packed, k):
    """Signed int4 decode via (nibble ^ 8) - 8, indexing bytes by k // 2."""
    ks = np.arange(k)
    b = packed[..., ks // 2].astype(np.int16)
    nib = (b >> (4 * (ks & 1))) & 0xF
    return (nib ^ 8) - 8


def bf16_exact(t):
    """A float64 tensor rounded to bf16 (nearest, ties to even) in one step,
    element by element with Python's frexp and round-half-even (torch's own
    fp64 -> bf16 conversion rounds twice, through fp32)."""
    flat = t.reshape(-1).tolist()
    out = []
    for v in flat:
        if v == 0.0 or not math.isfinite(v):
            out.append(v)
            continue
        m, e = math.frexp(v)                 # v = m 2^e, 0.5 <= |m| < 1
        out.append(math.ldexp(round(m * 256.0), e - 8))
    return torch.tensor(out, dtype=torch.float64).reshape(t.shape)


def widen(bits):
    return torch.from_numpy(np.asarray(bits, dtype=np.uint16).astype(np.int32) << 16).view(torch.float32).double()


class RandomBlobs:
    """Fast random expert blobs in the library layout (not the splitmix generator)."""

    def __init__(self, seed, zero_scales=False):
        self.seed = seed
        self.zero = zero_scales
        self.cache = {}

    def __call__(self, e):
        if e not in self.cache:
            rng = np.random.default_rng((self.seed, e))
            codes = rng.integers(0, 256, size=synth.CODE_BYTES_PER_EXPERT, dtype=np.uint8)
            if self.zero:
                scales = np.zeros(synth.SCALES_PER_EXPERT, dtype=np.uint16)
            else:
                s = np.abs(rng.standard_normal(synth.SCALES_PER_EXPERT)).astype(np.float32) * np.float32(0.01)
                scales = synth.f32_to_bf16_bits(s)
            self.cache[e] = (codes, scales)
        return self.cache[e]


def small_layer(seed, T):
    rng = np.random.default_rng(seed)
    x = synth.f32_to_bf16_bits(rng.standard_normal((T, 2048)).astype(np.float32))
    R = synth.f32_to_bf16_bits((rng.standard_normal((256, 2048)) * 0.02).astype(np.float32))
    S = synth.f32_to_bf16_bits((rng.standard_normal(synth.SHARED_ELEMS) * 0.02).astype(np.float32))
    return x, R, S


# ------------------------------------------------------------------ constants
def test_layout_constants_match_pages():
    c = golden_constants()
    assert c["n_experts"] == O.E == synth.N_EXPERTS
    assert c["top_k"] == O.K_TOP
    assert c["group"] == O.G
    assert c["expert_inter"] == O.I_R
    assert c["hidden"] == O.H
    assert c["shared_inter"] == O.I_S
    assert c["moe_layers"] == synth.N_MOE_LAYERS
    assert O.WEIGHT_FLOOR == 2.0 ** c["weight_floor_log2"]


def test_expert_bytes_closed_form_matches_pages():
    """1,622,016 B per expert; x 256 x 47 = 18.18 GiB (~18.2 GiB); 37.85 B params (37.8 B)."""
    c = golden_constants()
    per_expert = synth.CODE_BYTES_PER_EXPERT + 2 * synth.SCALES_PER_EXPERT
    assert per_expert == 1_622_016
    total = per_expert * O.E * synth.N_MOE_LAYERS
    assert round(total / 2 ** 30, 1) == c["routed_gib"]
    params = 3 * O.I_R * O.H * O.E * synth.N_MOE_LAYERS
    assert math.floor(params / 1e8) / 10 == c["routed_params_billion"]
    # 4 bits per code plus 16 bits per 128 codes
    assert per_expert * 8 / (3 * O.I_R * O.H) == pytest.approx(4.125)


# ------------------------------------------------------------------- numbers
def test_bf16_rounding_matches_torch_on_fp32_values():
    rng = np.random.default_rng(1)
    v = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(7.0),
        (rng.standard_normal(2000) * 1e-39).astype(np.float32),          # subnormals
        np.array([0.0, -0.0, 1.00390625, 1.01171875, -2.0078125, 3.3e38, 3.4e38, np.inf, -np.inf], dtype=np.float32),
    ])
    ours = O.f64_to_bf16_bits(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_bf16_rounding_brute_force_on_fp64_values():
    """Nearest bf16 by search over all finite bf16 values, ties to the even pattern."""
    allbits = np.arange(0, 0x7F80, dtype=np.uint16)
    allvals = O.bf16_to_f64(allbits)
    rng = np.random.default_rng(2)
    vals = np.concatenate([rng.standard_normal(300) * 10.0, [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -40]])
    ours = O.f64_to_bf16_bits(vals)
    for v, b in zip(vals, ours):
        d = np.abs(allvals - abs(v))
        best = np.nonzero(d == d.min())[0]
        cand = allbits[best]
        want = cand[0] if len(cand) == 1 else cand[(cand & 1) == 0][0]
        want = int(want) | (0x8000 if v < 0 else 0)
        assert int(b) == want, (v, hex(b), hex(want))


def test_silu_closed_forms():
    assert O.silu(0.0) == 0.0
    assert O.silu(40.0) == pytest.approx(40.0, rel=1e-15)
    assert abs(O.silu(-40.0)) < 1e-15
    assert O.silu(1.0) == pytest.approx(1.0 / (1.0 + math.exp(-1.0)))
    v = np.linspace(-6, 6, 101)
    np.testing.assert_allclose(O.silu(v), torch.nn.functional.silu(torch.from_numpy(v)).numpy(), rtol=1e-14, atol=1e-15)


# ------------------------------------------------------------------- Hadamard
def test_hadamard_textbook_identities():
    hn = O.hadamard(128)
    np.testing.assert_allclose(hn @ hn, np.eye(128), atol=1e-14)
    np.testing.assert_array_equal(hn, hn.T)
    i = np.arange(128)
    pc = np.vectorize(lambda v: bin(int(v)).count("1"))(i[:, None] & i[None, :])
    np.testing.assert_array_equal(hn * math.sqrt(128), (-1.0) ** pc)
    np.testing.assert_allclose(hn[0], np.full(128, 1 / math.sqrt(128)))


def test_rotation_matches_butterfly():
    rng = np.random.default_rng(3)
    v = rng.standard_normal((5, 2048))
    np.testing.assert_allclose(O.rotate_blocks(v), rotate_rows_blockwise(v), atol=1e-12)
    a = rng.standard_normal((3, 512))
    np.testing.assert_allclose(O.rotate_blocks(a), rotate_rows_blockwise(a), atol=1e-12)
    # sqrt(128) * e_0 of a block maps to all-ones, and back
    e0 = np.zeros(128)
    e0[0] = math.sqrt(128)
    np.testing.assert_allclose(O.rotate_blocks(e0[None])[0], np.ones(128), atol=1e-13)


def test_rotation_transparency():
    """W (x rotated) == (W (I x Hn)) x: the rotated basis is invisible to the product."""
    rng = np.random.default_rng(4)
    w = rng.standard_normal((64, 2048))
    x = rng.standard_normal(2048)
    lhs = w @ O.rotate_blocks(x[None])[0]
    rhs = rotate_rows_blockwise(w) @ x
    np.testing.assert_allclose(lhs, rhs, rtol=1e-11, atol=1e-11)


# --------------------------------------------------------------- quantisation
def test_int4_decode_probe_against_bitwise_reading():
    blobs = RandomBlobs(5)
    cb, sb = blobs(3)
    wg, wu, wd = O.expert_planes(cb, sb)
    rng = np.random.default_rng(6)
    nb_gu = 512 * 1024
    for _ in range(300):
        plane = int(rng.integers(0, 3))
        if plane < 2:
            n, k = int(rng.integers(0, 512)), int(rng.integers(0, 2048))
            byte = int(cb[plane * nb_gu + n * 1024 + k // 2])
            sbits = int(sb[plane * 512 * 16 + n * 16 + k // 128])
            got = (wg, wu)[plane][n, k]
        else:
            n, k = int(rng.integers(0, 2048)), int(rng.integers(0, 512))
            byte = int(cb[2 * nb_gu + n * 256 + k // 2])
            sbits = int(sb[2 * 512 * 16 + n * 4 + k // 128])
            got = wd[n, k]
        nib = (byte >> 4) if (k % 2) else (byte & 0xF)
        code = nib - 16 if nib & 0x8 else nib
        scale = np.frombuffer(np.uint32(sbits << 16).tobytes(), dtype=np.float32)[0]
        assert got == code * float(scale)


def test_unpack_matches_xor_decode():
    rng = np.random.default_rng(7)
    p = rng.integers(0, 256, size=(7, 64), dtype=np.uint8)
    np.testing.assert_array_equal(O.unpack_int4(p, 128), decode_xor(p, 128))
    vals = rng.integers(-8, 8, size=(3, 256)).astype(np.int8)
    np.testing.assert_array_equal(O.unpack_int4(synth.pack_int4(vals), 256), vals)


def test_quantize_roundtrip_within_int4_bound():
    """rotate -> quantise -> dequantise -> unrotate recovers W within int4 error."""
    c = golden_constants()
    rng = np.random.default_rng(8)
    w = rng.standard_normal((512, 2048))
    codes, s_bits = O.quantize_rotated(w)
    assert codes.min() >= -8 and codes.max() <= 7
    s = np.repeat(O.bf16_to_f64(s_bits), 128, axis=1)
    w_rot = rotate_rows_blockwise(w)
    err_rot = w_rot - codes * s
    assert np.all(np.abs(err_rot) <= s / 2 * (1 + 1e-12))
    w_back = O.unrotated_effective(codes, s_bits)
    err = w_back - w
    # orthogonal rotation: the error norm is the same in both bases
    assert np.linalg.norm(err) == pytest.approx(np.linalg.norm(err_rot), rel=1e-10)
    rel = np.linalg.norm(err) / np.linalg.norm(w)
    # the model card quotes 11.7% per expert plane; Gaussian data lands on it
    assert abs(rel - c["int4_rel_frobenius"]) < 0.01, rel


# ----------------------------------------------------------------------- packer
def test_fwht128_f32_is_the_butterfly_within_fp32_rounding():
    rng = np.random.default_rng(30)
    v = rng.standard_normal((64, 2048)).astype(np.float32)
    got = O.fwht128_f32(v).astype(np.float64)
    ref = rotate_rows_blockwise(v.astype(np.float64))
    # seven fp32 add stages and one multiply: each value within a few ulps of the block's 1-norm
    l1 = np.abs(v.astype(np.float64)).reshape(64, 16, 128).sum(axis=2)
    bound = np.repeat(l1, 128, axis=1) * 2.0 ** -21
    assert np.all(np.abs(got - ref) <= bound)
    # its own inverse up to fp32 rounding
    back = O.fwht128_f32(O.fwht128_f32(v))
    assert np.abs(back - v).max() < 1e-5 * np.abs(v).max()


def test_quantizer_f32_agrees_with_the_fp64_reading():
    """Deciding in fp32 (the packer's precision) moves a code only where the
    rotated value sits on a rounding boundary: rare, and by one step."""
    rng = np.random.default_rng(31)
    bits = synth.f32_to_bf16_bits((rng.standard_normal((512, 2048)) * 0.02).astype(np.float32))
    c32, s32 = O.quantize_rotated_f32(bits)
    c64, s64 = O.quantize_rotated(O.bf16_to_f64(bits))
    same_s = s32 == s64
    assert same_s.mean() > 0.999
    # a scale differs by at most one bf16 step
    assert np.all(np.abs(s32.astype(np.int32) - s64.astype(np.int32)) <= 1)
    rows_groups = np.repeat(same_s, 128, axis=1)
    diff = c32 != c64
    assert diff[rows_groups].mean() < 1e-4
    assert np.all(np.abs(c32.astype(np.int32) - c64)[rows_groups] <= 1)


def test_quantizer_f32_error_is_the_cards_figure():
    c = golden_constants()
    rng = np.random.default_rng(32)
    w = (rng.standard_normal((512, 2048)) * 0.02).astype(np.float32)
    bits = synth.f32_to_bf16_bits(w)
    codes, s_bits = O.quantize_rotated_f32(bits)
    assert codes.min() >= -8 and codes.max() <= 7
    w_back = O.unrotated_effective(codes, s_bits)
    wb = O.bf16_to_f64(bits)
    rel = np.linalg.norm(w_back - wb) / np.linalg.norm(wb)
    assert abs(rel - c["int4_rel_frobenius"]) < 0.01, rel
    # every rotated value within half a step of its code (no group needs the clamp)
    s = np.repeat(O.bf16_to_f64(s_bits), 128, axis=1)
    r = rotate_rows_blockwise(wb)
    assert np.all(np.abs(r - codes * s) <= s / 2 * (1 + 1e-3) + 1e-9)


def test_pack_int4_inverts_the_decoder():
    vals = np.array([[-8, -7, -1, 0, 1, 6, 7, 3, -2, 5]], dtype=np.int16)
    packed = O.pack_int4(vals)
    np.testing.assert_array_equal(decode_xor(packed, 10), vals)
    np.testing.assert_array_equal(O.unpack_int4(packed, 10), vals)
    assert packed[0, 0] == (0x8 | (0x9 << 4))       # -8 low nibble, -7 high nibble


def test_pack_bank_of_one_hot_rows():
    """A row holding 1.0 at position j of a block rotates to +-1/sqrt(128) with
    the signs of Hadamard row j, so its 16 codes of that block are
    7 * (-1)^popcount(i & j): the layout, the sign convention and the scale
    all show in one closed form."""
    w = np.zeros((2, O.EXPERT_WEIGHTS), dtype=np.uint16)
    one = synth.f32_to_bf16_bits(np.float32([1.0]))[0]
    # expert 1: gate row 3, block 5, position 77; down row 2000, block 2, position 9
    gate_off = 3 * 2048 + 5 * 128 + 77
    down_off = 2 * 512 * 2048 + 2000 * 512 + 2 * 128 + 9
    w[1, gate_off] = one
    w[1, down_off] = one
    codes, scales = O.pack_expert_bank(w)
    assert not codes[0].any() and not scales[0].any()
    vals = O.unpack_int4(codes[1], O.EXPERT_WEIGHTS)
    i = np.arange(128)
    sign77 = np.array([(-1) ** bin(k & 77).count("1") for k in i])
    sign9 = np.array([(-1) ** bin(k & 9).count("1") for k in i])
    np.testing.assert_array_equal(vals[3 * 2048 + 5 * 128: 3 * 2048 + 6 * 128], 7 * sign77)
    base = 2 * 512 * 2048 + 2000 * 512 + 2 * 128
    np.testing.assert_array_equal(vals[base: base + 128], 7 * sign9)
    assert np.count_nonzero(vals) == 256
    s = O.bf16_to_f64(scales[1])
    nz = np.nonzero(s)[0]
    assert list(nz) == [(3 * 2048 + 5 * 128) // 128, base // 128]
    np.testing.assert_allclose(s[nz], 1 / (7 * math.sqrt(128)), rtol=2 ** -8)


# ------------------------------------------------------------- dense MLP block
def test_dense_mlp_closed_form_on_one_hot_rows():
    """Gate row j = a e_k, up row j = b e_k, down column j = c e_m: the only
    nonzero output is y_m = c silu(a x_k) (b x_k)."""
    rng = np.random.default_rng(40)
    x = synth.f32_to_bf16_bits(rng.standard_normal((3, 2048)).astype(np.float32))
    w = np.zeros(O.DENSE_WEIGHTS, dtype=np.uint16)
    n = O.I_D * 2048
    j, k, m_out = 4000, 77, 1500
    a, b, c = 0.75, -1.25, 0.5
    bits = synth.f32_to_bf16_bits(np.float32([a, b, c]))
    w[j * 2048 + k] = bits[0]
    w[n + j * 2048 + k] = bits[1]
    w[2 * n + m_out * O.I_D + j] = bits[2]
    out = O.dense_mlp(x, w)
    xk = O.bf16_to_f64(x)[:, k]
    h = (a * xk / (1 + np.exp(-a * xk))) * (b * xk)
    expect = c * bf16_exact(torch.from_numpy(h)).numpy()   # the down linear's input is bf16
    np.testing.assert_allclose(out["y"][:, m_out], expect, rtol=1e-13)
    assert np.count_nonzero(out["y"]) == np.count_nonzero(expect)


def test_dense_mlp_with_zero_up_rows_is_zero():
    rng = np.random.default_rng(41)
    x = synth.f32_to_bf16_bits(rng.standard_normal((2, 2048)).astype(np.float32))
    w = synth.f32_to_bf16_bits((rng.standard_normal(O.DENSE_WEIGHTS) * 0.02).astype(np.float32))
    n = O.I_D * 2048
    w[n:2 * n] = 0
    assert not O.dense_mlp(x, w)["y"].any()


def test_dense_mlp_embeds_the_shared_expert():
    """Width-1024 weights padded with zero rows and columns to width 6144 give
    the shared expert's output (silu(0) * 0 adds nothing)."""
    x, _, S = small_layer(42, 2)
    sg, su, sd = [O.f64_to_bf16_bits(p) for p in O.shared_planes(S)]
    n = O.I_D * 2048
    w = np.zeros(O.DENSE_WEIGHTS, dtype=np.uint16)
    w[:n].reshape(O.I_D, 2048)[:1024] = sg
    w[n:2 * n].reshape(O.I_D, 2048)[:1024] = su
    w[2 * n:].reshape(2048, O.I_D)[:, :1024] = sd
    np.testing.assert_allclose(O.dense_mlp(x, w)["y"], O.shared_expert(O.bf16_to_f64(x), S), rtol=1e-12, atol=1e-15)


# ----------------------------------------------------------------------- router
def _brute_top6(l32):
    n = l32.shape[0]
    best = None
    for sub in itertools.combinations(range(n), 6):
        s = sum(float(l32[i]) for i in sub)
        key = (-s, sub)                      # max sum, then lexicographically lowest indices
        if best is None or key < best[0]:
            best = (key, sub)
    sub = best[1]
    return sorted(sub, key=lambda i: (-l32[i], i))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_top6_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    n_exp, k = 10, 32
    x = O.bf16_to_f64(synth.f32_to_bf16_bits(rng.standard_normal((4, k)).astype(np.float32)))
    R = synth.f32_to_bf16_bits(rng.standard_normal((n_exp, k)).astype(np.float32))
    rt = O.route(x, R)
    for t in range(4):
        assert list(rt["topk_idx"][t]) == _brute_top6(rt["logits32"][t])
        w = rt["topk_w"][t]
        assert w.sum() == pytest.approx(1.0, abs=1e-14)
        sig = 1.0 / (1.0 + np.exp(-rt["logits"][t, rt["topk_idx"][t]]))
        np.testing.assert_allclose(w, sig / sig.sum(), rtol=1e-14)
        assert np.all(np.diff(w) <= 0)


def test_top6_ties_go_to_lower_index():
    # integer-valued inputs: exact logits with deliberate ties
    x = np.array([[1.0, 0.0], [0.0, 0.0]])
    Rv = np.array([[1, 0], [3, 0], [2, 0], [3, 0], [2, 0], [1, 0], [2, 0], [0, 0], [2, 0], [1, 0]], dtype=np.float32)
    R = synth.f32_to_bf16_bits(Rv)
    rt = O.route(x, R)
    assert list(rt["topk_idx"][0]) == [1, 3, 2, 4, 6, 8]
    assert list(rt["topk_idx"][0]) == _brute_top6(rt["logits32"][0])
    # all logits equal: experts 0..5 with weight 1/6 each
    assert list(rt["topk_idx"][1]) == [0, 1, 2, 3, 4, 5]
    np.testing.assert_allclose(rt["topk_w"][1], np.full(6, 1 / 6), rtol=1e-15)
    assert rt["near_tie"][1] and rt["gap"][1] == 0.0


def test_router_zero_weights_pick_first_six():
    x = O.bf16_to_f64(small_layer(9, 3)[0])
    rt = O.route(x, np.zeros((256, 2048), dtype=np.uint16))
    assert np.all(rt["topk_idx"] == np.arange(6))
    np.testing.assert_allclose(rt["topk_w"], 1 / 6)


def test_weight_floor():
    """Scores summing below 2**-14 are divided by the floor, not by their sum."""
    x, R, _ = small_layer(10, 2)
    xf = O.bf16_to_f64(x)
    bias = np.full(256, -30.0, dtype=np.float32)
    rt = O.route(xf, R, bias)
    sig = 1.0 / (1.0 + np.exp(-rt["logits"][np.arange(2)[:, None], rt["topk_idx"]]))
    assert np.all(sig.sum(axis=1) < 2 ** -14)
    np.testing.assert_allclose(rt["topk_w"], sig * 2 ** 14, rtol=1e-14)
    # the bias is part of the logit: it shifts selection and weights alike
    bias2 = np.zeros(256, dtype=np.float32)
    bias2[[7, 100, 200]] = 50.0
    rt2 = O.route(xf, R, bias2)
    assert set(rt2["topk_idx"][0][:3]) == {7, 100, 200}


def _policy_case(seed, n_exp=10, k=32, T=3):
    rng = np.random.default_rng(seed)
    x = O.bf16_to_f64(synth.f32_to_bf16_bits(rng.standard_normal((T, k)).astype(np.float32)))
    R = synth.f32_to_bf16_bits(rng.standard_normal((n_exp, k)).astype(np.float32))
    # the logits recomputed here by nested loops, independent of route()
    Rw = widen(R)
    lg = np.array([[sum(x[t, i] * Rw[e, i] for i in range(k)) for e in range(n_exp)] for t in range(T)])
    return x, R, lg


def _sig(v):
    return 1.0 / (1.0 + np.exp(-np.asarray(v, dtype=np.float64)))


def test_router_policy_plain_sum_and_no_normalisation():
    """Legacy selected-sum and no normalisation (bloomery #632, host-policy
    slice): above the floor the selected-sum equals the floored one; "none"
    keeps the six sigmoid scores as they are."""
    x, R, lg = _policy_case(20)
    fl = O.route(x, R, norm="floor")
    sm = O.route(x, R, norm="sum")
    nn = O.route(x, R, norm="none")
    for t in range(x.shape[0]):
        sel = _brute_top6(O.f32_round(lg[t]))
        assert list(sm["topk_idx"][t]) == sel and list(nn["topk_idx"][t]) == sel
        s6 = _sig(lg[t, sel])
        np.testing.assert_allclose(nn["topk_w"][t], s6, rtol=1e-13)
        np.testing.assert_allclose(sm["topk_w"][t], s6 / s6.sum(), rtol=1e-13)
        assert sm["topk_w"][t].sum() == pytest.approx(1.0, abs=1e-14)
    np.testing.assert_array_equal(sm["topk_w"], fl["topk_w"])


def test_router_policy_sum_without_floor_at_tiny_scores():
    """With every logit near -30 the six scores sum below 2**-14: the floored
    policy gives weights far below 1, the legacy sum still renormalises to 1."""
    x, R, lg = _policy_case(21)
    bias = np.full(10, -30.0, dtype=np.float32)
    fl = O.route(x, R, bias, norm="floor")
    sm = O.route(x, R, bias, norm="sum")
    for t in range(x.shape[0]):
        sel = _brute_top6(O.f32_round(lg[t] - 30.0))
        s6 = _sig(lg[t, sel] - 30.0)
        assert s6.sum() < 2 ** -14
        np.testing.assert_allclose(fl["topk_w"][t], s6 * 2 ** 14, rtol=1e-12)
        np.testing.assert_allclose(sm["topk_w"][t], s6 / s6.sum(), rtol=1e-12)
        assert sm["topk_w"][t].sum() == pytest.approx(1.0, abs=1e-12)
        assert fl["topk_w"][t].sum() < 1e-3


def test_router_bias_for_selection_only():
    """A selection-only bias changes which experts are chosen, never their
    scores: a constant bias leaves the route exactly as without one, and a
    large bias on three experts puts them first with unbiased sigmoid weights."""
    x, R, lg = _policy_case(22)
    plain = O.route(x, R)
    c = np.full(10, 1.5, dtype=np.float32)
    sel_c = O.route(x, R, c, bias_mode="select")
    log_c = O.route(x, R, c, bias_mode="logit")
    np.testing.assert_array_equal(sel_c["topk_idx"], plain["topk_idx"])
    np.testing.assert_allclose(sel_c["topk_w"], plain["topk_w"], rtol=1e-14)
    assert np.abs(log_c["topk_w"] - plain["topk_w"]).max() > 1e-4   # the logit-mode bias moves the weights
    b = np.zeros(10, dtype=np.float32)
    b[[2, 5, 9]] = 50.0
    rt = O.route(x, R, b, bias_mode="select")
    for t in range(x.shape[0]):
        sel = _brute_top6(O.f32_round(lg[t] + b))
        assert list(rt["topk_idx"][t]) == sel and set(sel[:3]) == {2, 5, 9}
        s6 = _sig(lg[t, sel])
        np.testing.assert_allclose(rt["topk_w"][t], s6 / s6.sum(), rtol=1e-12)


def test_router_policy_rejects_unknown_names():
    x, R, _ = _policy_case(23)
    with pytest.raises(ValueError):
        O.route(x, R, norm="softmax")
    with pytest.raises(ValueError):
        O.route(x, R, bias_mode="both")


def test_near_tie_flag_uses_the_6th_7th_gap():
    x, R, _ = small_layer(11, 64)
    rt = O.route(O.bf16_to_f64(x), R)
    srt = -np.sort(-rt["logits"], axis=1)
    np.testing.assert_allclose(rt["gap"], srt[:, 5] - srt[:, 6])
    np.testing.assert_array_equal(rt["near_tie"], rt["gap"] <= 1e-3)


def test_order_tie_flag_uses_the_gaps_inside_the_six():
    """order_gap is the smallest difference between consecutive chosen logits
    (brute force over the six), flagged at 1e-3; a router built with two
    chosen logits 5e-4 apart flags exactly that token."""
    x, R, _ = small_layer(12, 32)
    xf = O.bf16_to_f64(x)
    rt = O.route(xf, R)
    for t in range(32):
        six = sorted(rt["logits"][t][rt["topk_idx"][t]], reverse=True)
        assert rt["order_gap"][t] == pytest.approx(min(a - b for a, b in zip(six, six[1:])), abs=1e-15)
    np.testing.assert_array_equal(rt["order_tie"], rt["order_gap"] <= 1e-3)
    # one-hot tokens: x_t = e_t picks router column t; rows 0..5 get logits
    # 6, 5, 4, 3, 2.0005, 2 on token 0 (a 5e-4 gap between its 5th and 6th)
    Rz = np.zeros((256, 2048), dtype=np.uint16)
    vals = [6.0, 5.0, 4.0, 3.0, 2.0 + 2 ** -11, 2.0]
    for e, v in enumerate(vals):
        Rz[e, 0] = synth.f32_to_bf16_bits(np.float32([v]))[0] if v != 2.0 + 2 ** -11 else 0
    xo = np.zeros((2, 2048))
    xo[0, 0] = 1.0
    bias = np.zeros(256)
    bias[4] = 2.0 + 2 ** -11     # a logit that bf16 router rows cannot hold exactly, through the bias
    r1 = O.route(xo, Rz, bias=bias)
    assert r1["order_gap"][0] == pytest.approx(2 ** -11) and r1["order_tie"][0]
    assert not r1["near_tie"][0]


# ------------------------------------------------------------------------- sort
def test_sort_against_nested_loops():
    rng = np.random.default_rng(12)
    T = 37
    idx = np.stack([rng.choice(256, 6, replace=False) for _ in range(T)]).astype(np.int32)
    idx[5] = [0, 1, 2, 3, 4, 5]
    s = O.sort_assignments(idx)
    perm = []
    for e in range(256):
        for t in range(T):
            for j in range(6):
                if idx[t, j] == e:
                    perm.append(6 * t + j)
    np.testing.assert_array_equal(s["perm"], perm)
    assert s["offsets"][0] == 0 and s["offsets"][256] == 6 * T
    for e in range(256):
        assert s["offsets"][e + 1] - s["offsets"][e] == np.sum(idx == e)
    np.testing.assert_array_equal(s["perm"][s["pos"]], np.arange(6 * T))


# ------------------------------------------------------------------- the layer
def test_layer_matches_weight_side_recomputation():
    """Independent route: unrotate the weights (butterfly), decode with XOR, SwiGLU in torch."""
    x, R, S = small_layer(13, 3)
    blobs = RandomBlobs(14)
    out = O.moe_layer(x, R, blobs, S)
    xt = widen(x)                                              # [T, 2048]
    logits = xt @ widen(R).T
    nb_gu = 512 * 1024
    for t in range(3):
        l32 = logits[t].float().double().numpy()
        sel = sorted(range(256), key=lambda i: (-l32[i], i))[:6]
        sig = torch.sigmoid(logits[t, sel])
        w = sig / sig.sum()
        acc = torch.zeros(2048, dtype=torch.float64)
        for j, e in enumerate(sel):
            cb, sb = blobs(e)
            g = decode_xor(cb[:nb_gu].reshape(512, 1024), 2048) * np.repeat(O.bf16_to_f64(sb[:8192].reshape(512, 16)), 128, 1)
            u = decode_xor(cb[nb_gu:2 * nb_gu].reshape(512, 1024), 2048) * np.repeat(O.bf16_to_f64(sb[8192:16384].reshape(512, 16)), 128, 1)
            d = decode_xor(cb[2 * nb_gu:].reshape(2048, 256), 512) * np.repeat(O.bf16_to_f64(sb[16384:].reshape(2048, 4)), 128, 1)
            ge, ue, de = (torch.from_numpy(rotate_rows_blockwise(m)) for m in (g, u, d))
            h = torch.nn.functional.silu(ge @ xt[t]) * (ue @ xt[t])
            acc += w[j] * (de @ h)
        sg = widen(S[:2048 * 1024]).reshape(1024, 2048)
        su = widen(S[2048 * 1024:4096 * 1024]).reshape(1024, 2048)
        sd = widen(S[4096 * 1024:]).reshape(2048, 1024)
        z = sd @ bf16_exact(torch.nn.functional.silu(sg @ xt[t]) * (su @ xt[t]))
        want = (acc + z).numpy()
        assert list(out["topk_idx"][t]) == sel
        np.testing.assert_allclose(out["y"][t], want, rtol=1e-9, atol=1e-9 * np.abs(want).max())


def test_zero_scales_reduce_to_shared_expert():
    x, R, S = small_layer(15, 4)
    out = O.moe_layer(x, R, RandomBlobs(16, zero_scales=True), S)
    xt = widen(x)
    sg = widen(S[:2048 * 1024]).reshape(1024, 2048)
    su = widen(S[2048 * 1024:4096 * 1024]).reshape(1024, 2048)
    sd = widen(S[4096 * 1024:]).reshape(2048, 1024)
    z = bf16_exact(torch.nn.functional.silu(xt @ sg.T) * (xt @ su.T)) @ sd.T
    np.testing.assert_allclose(out["y"], z.numpy(), rtol=1e-12, atol=1e-12)
    ref_bits = z.float().to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    # one rounding from fp64 vs torch's fp64->fp32->bf16: equal except at exact double-rounding cases
    assert np.mean(out["y_bits"] == ref_bits) > 0.999


def test_floor_case_makes_routed_part_vanish():
    x, R, S = small_layer(17, 2)
    bias = np.full(256, -30.0, dtype=np.float32)
    out = O.moe_layer(x, R, RandomBlobs(18), S, bias=bias)
    assert np.max(np.abs(out["routed"])) < 1e-6 * np.max(np.abs(out["shared"]))


def test_dense_all_expert_evaluation_equals_sparse():
    x, R, S = small_layer(19, 2)
    blobs = RandomBlobs(20)
    sparse = O.moe_layer(x, R, blobs, S)
    dense = O.moe_layer_dense(x, R, blobs, S)
    np.testing.assert_allclose(sparse["y"], dense["y"], rtol=1e-10, atol=1e-12)
    assert np.count_nonzero(dense["gates"]) == 2 * 6


def test_token_subset_matches_full():
    x, R, S = small_layer(21, 5)
    blobs = RandomBlobs(22)
    full = O.moe_layer(x, R, blobs, S)
    part = O.moe_layer(x, R, blobs, S, tokens=[4, 1])
    np.testing.assert_array_equal(part["y"], full["y"][[4, 1]])
    np.testing.assert_array_equal(part["perm"], full["perm"])


# ------------------------------------------------------------------------ stack
def test_rmsnorm_closed_form():
    x = np.array([[3.0] * 2048, [-0.5] * 2048])
    np.testing.assert_allclose(O.rmsnorm(x)[0], 3.0 / math.sqrt(9.0 + 1e-6))
    np.testing.assert_allclose(O.rmsnorm(x)[1], -0.5 / math.sqrt(0.25 + 1e-6))
    rng = np.random.default_rng(23)
    v = rng.standard_normal((3, 2048))
    ref = torch.nn.functional.rms_norm(torch.from_numpy(v), (2048,), eps=1e-6).numpy()
    np.testing.assert_allclose(O.rmsnorm(v), ref, rtol=1e-12)


def test_stack_with_shared_only_layers():
    """Zero routed scales: each layer adds bf16(shared(bf16(rmsnorm(x)))) to an fp32 residual."""
    x0, R, S = small_layer(24, 2)
    layers = [(R, RandomBlobs(25, zero_scales=True), S), (R, RandomBlobs(26, zero_scales=True), S)]
    resid0 = O.bf16_to_f64(x0) * 3.0
    out, inputs = O.stack_step(resid0, layers)
    r = torch.from_numpy(resid0).float()
    sg = widen(S[:2048 * 1024]).reshape(1024, 2048)
    su = widen(S[2048 * 1024:4096 * 1024]).reshape(1024, 2048)
    sd = widen(S[4096 * 1024:]).reshape(2048, 1024)
    for _ in range(2):
        xin = torch.nn.functional.rms_norm(r.double(), (2048,), eps=1e-6).float().to(torch.bfloat16).double()
        z = bf16_exact(torch.nn.functional.silu(xin @ sg.T) * (xin @ su.T)) @ sd.T
        r = r + z.float().to(torch.bfloat16).float()
    # equal up to the rare double-rounding difference of fp64->fp32->bf16
    np.testing.assert_allclose(out, r.double().numpy(), rtol=1e-2, atol=1e-2)
    assert np.mean(out == r.double().numpy()) > 0.99


# ------------------------------------------------------------ NVFP4 experts
# E2M1 element values of the OCP microscaling format (the format the name
# E2M1 denotes): codes 0..7 and the same magnitudes with the sign bit.
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_table():
    v = O.e2m1_value(np.arange(16))
    np.testing.assert_array_equal(v[:8], E2M1_TABLE)
    np.testing.assert_array_equal(v[8:], [-t for t in E2M1_TABLE])
    assert math.copysign(1.0, v[8]) == -1.0          # code 8 is -0


def test_e4m3_matches_torch_for_every_byte():
    b = np.arange(256)
    ours = O.e4m3_value(b)
    ref = torch.tensor(b, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    assert np.isnan(ours).sum() == 2                  # S.1111.111 only
    fin = ~np.isnan(ref)
    np.testing.assert_array_equal(ours[fin], ref[fin])


def test_e4m3_points():
    assert O.e4m3_value(0x38) == 1.0
    assert O.e4m3_value(0x7E) == 448.0                # largest finite
    assert O.e4m3_value(0x01) == 2.0 ** -9            # smallest subnormal
    assert O.e4m3_value(0x08) == 2.0 ** -6            # smallest normal
    assert O.e4m3_value(0xB8) == -1.0


def test_nvfp4_dequant_nibble_order_and_blocks():
    # one row of K = 32: code of column k is k % 16 (even k in the low nibble),
    # block scales 1.0 (0x38) and 2.0 (0x40), tensor scale 0.5
    k = np.arange(32)
    c = k % 16
    packed = (c[0::2] | (c[1::2] << 4)).astype(np.uint8)[None, :]
    w = O.dequantize_nvfp4(packed, np.array([[0x38, 0x40]], dtype=np.uint8), np.float32(0.5), 32)[0]
    table = E2M1_TABLE + [-t for t in E2M1_TABLE]
    expect = [table[ki % 16] * (1.0 if ki < 16 else 2.0) * 0.5 for ki in k]
    np.testing.assert_array_equal(w, expect)


def _nv_onehot_blob(k0, r1, cg, cu, cd, sbytes, ts):
    """Every gate/up row r has one code, cg[r] / cu[r], at column k0; every down
    row n one code cd[n] at column r1; each plane's block holding it has scale
    byte sbytes[plane]; tensor scales ts."""
    cb = np.zeros(O.NV_CODE_BYTES_PER_EXPERT, dtype=np.uint8)
    sb = np.zeros(O.NV_SCALE_BYTES_PER_EXPERT, dtype=np.uint8)
    H, I = O.H, O.I_R
    shift = 4 * (k0 & 1)
    for r in range(I):
        cb[r * (H // 2) + k0 // 2] |= np.uint8(cg[r] << shift)
        cb[I * H // 2 + r * (H // 2) + k0 // 2] |= np.uint8(cu[r] << shift)
        sb[r * (H // 16) + k0 // 16] = sbytes[0]
        sb[I * H // 16 + r * (H // 16) + k0 // 16] = sbytes[1]
    dshift = 4 * (r1 & 1)
    for n in range(H):
        cb[I * H + n * (I // 2) + r1 // 2] |= np.uint8(cd[n] << dshift)
        sb[2 * I * H // 16 + n * (I // 16) + r1 // 16] = sbytes[2]
    return cb, sb, np.asarray(ts, dtype=np.float32)


def test_nvfp4_layer_one_hot_closed_form():
    T, k0, r1 = 3, 1001, 77
    rng = np.random.default_rng(5)
    cg = rng.integers(0, 16, O.I_R)
    cu = rng.integers(0, 16, O.I_R)
    cd = rng.integers(0, 16, O.H)
    sbytes = (0x30, 0x3C, 0x28)                       # 0.5, 1.5, 0.25
    svals = (0.5, 1.5, 0.25)
    ts = (0.5, 0.25, 2.0)
    blob = _nv_onehot_blob(k0, r1, cg, cu, cd, sbytes, ts)
    x_bits = synth.gen_x(3, T)
    router, shared = synth.gen_router(3), synth.gen_shared(3)
    out = O.moe_layer_nvfp4(x_bits, router, lambda e: blob, shared)
    table = E2M1_TABLE + [-t for t in E2M1_TABLE]
    x = O.bf16_to_f64(x_bits)
    for t in range(T):
        xk = x[t, k0]
        g = table[cg[r1]] * svals[0] * ts[0] * xk
        u = table[cu[r1]] * svals[1] * ts[1] * xk
        a = g / (1.0 + math.exp(-g)) * u
        # every expert is the same; the six weights sum to 1 (sum of sigmoids > 2**-14)
        o = np.array([table[c] for c in cd]) * svals[2] * ts[2] * a
        np.testing.assert_allclose(out["routed"][t], o * out["topk_w"][t].sum(), rtol=1e-12, atol=1e-300)
        assert abs(out["topk_w"][t].sum() - 1.0) < 1e-12
    np.testing.assert_allclose(out["y"], out["routed"] + out["shared"], rtol=0, atol=0)


def test_nvfp4_layer_zero_codes_leave_the_shared_expert():
    T = 2
    blob = (np.zeros(O.NV_CODE_BYTES_PER_EXPERT, np.uint8), synth.gen_nvfp4_scales(1, 0, [0])[0],
            np.ones(3, np.float32))
    x_bits = synth.gen_x(1, T)
    out = O.moe_layer_nvfp4(x_bits, synth.gen_router(1), lambda e: blob, synth.gen_shared(1))
    assert np.all(out["routed"] == 0.0)
    z = O.shared_expert(O.bf16_to_f64(x_bits), synth.gen_shared(1))
    np.testing.assert_array_equal(out["y_bits"], O.f64_to_bf16_bits(z))


def test_nvfp4_layer_scales_with_the_down_tensor_scale():
    # the routed part is linear in the down plane's tensor scale (exact in fp64
    # for a power of two)
    T = 2
    cache = {}

    def blob(e):
        if e not in cache:
            cache[e] = (synth.gen_codes_scales(2, 0, experts=[e])[0][0], synth.gen_nvfp4_scales(2, 0, [e])[0])
        return cache[e]
    ts = synth.gen_nvfp4_tensor_scales(2)
    ts2 = ts.copy()
    ts2[:, 2] *= 4
    x_bits = synth.gen_x(2, T)
    r, sh = synth.gen_router(2), synth.gen_shared(2)
    a = O.moe_layer_nvfp4(x_bits, r, lambda e: blob(e) + (ts[e],), sh)
    b = O.moe_layer_nvfp4(x_bits, r, lambda e: blob(e) + (ts2[e],), sh)
    np.testing.assert_array_equal(b["routed"], 4 * a["routed"])
