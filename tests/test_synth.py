"""The seeded input generator: published SplitMix64 vectors, layout and statistics."""
import numpy as np
import pytest

import synth
from tests.conftest import read_golden


def test_splitmix64_published_seed0_stream():
    want = [int(v, 16) for v in read_golden("splitmix64_seed0.txt")]
    got = [int(v) for v in synth.draw(0, 0, np.arange(len(want)))]
    assert got == want
    assert [synth.draw_int(0, 0, i) for i in range(len(want))] == want


def test_vector_and_scalar_draws_agree():
    rng = np.random.default_rng(0)
    idx = rng.integers(0, 2 ** 40, size=200).astype(np.uint64)
    for seed, tid in [(0, 2), (4, 64 * 46 + 10), (3, 11)]:
        vec = synth.draw(seed, tid, idx)
        assert [int(v) for v in vec] == [synth.draw_int(seed, tid, int(i)) for i in idx]


def test_int4_codes_uniform():
    v = synth.int4_values(0, synth.tensor_id(0, synth.KIND_CODE_G), np.arange(1 << 18))
    assert v.min() == -8 and v.max() == 7
    counts = np.bincount(v.astype(np.int64) + 8, minlength=16)
    expected = (1 << 18) / 16
    chi2 = np.sum((counts - expected) ** 2 / expected)
    assert chi2 < 45  # 15 dof, p ~ 1e-4


@pytest.mark.parametrize("sigma", [1.0, 0.02])
def test_normal_moments(sigma):
    bits = synth.normal_bf16_bits(1, 0, np.arange(1 << 17), sigma)
    v = synth.bf16_bits_to_f32(bits).astype(np.float64)
    assert abs(v.mean()) < 0.02 * sigma
    assert v.std() == pytest.approx(sigma, rel=0.02)
    assert np.abs(v).max() <= 3.47 * sigma


def test_scales_are_positive_half_normal():
    bits = synth.abs_normal_bf16_bits(0, synth.tensor_id(0, synth.KIND_SCALE_G), np.arange(1 << 16), 0.01)
    v = synth.bf16_bits_to_f32(bits).astype(np.float64)
    assert v.min() >= 0
    assert v.mean() == pytest.approx(0.01 * np.sqrt(2 / np.pi), rel=0.03)


def test_expert_blob_layout():
    codes, scales = synth.gen_codes_scales(0, 0, experts=[5])
    g, u, d = synth.gen_expert_codes_values(0, 0, 5)
    cb = codes[0]
    # byte 0 of the gate plane holds k=0 (low nibble) and k=1 (high nibble) of row 0
    assert (cb[0] & 0xF) == (g[0, 0] & 0xF) and (cb[0] >> 4) == (g[0, 1] & 0xF)
    assert (cb[512 * 1024 + 1024 * 3 + 7] >> 4) == (u[3, 15] & 0xF)
    assert (cb[2 * 512 * 1024 + 256 * 100 + 2] & 0xF) == (d[100, 4] & 0xF)
    sg, su, sd = synth.gen_expert_scales_bits(0, 0, 5)
    assert scales[0][16 * 7 + 3] == sg[7, 3]
    assert scales[0][8192 + 16 * 9] == su[9, 0]
    assert scales[0][16384 + 4 * 2047 + 3] == sd[2047, 3]
    # the flat element index continues across experts
    g4 = synth.int4_values(0, synth.tensor_id(0, synth.KIND_CODE_G), np.arange(5 * 512 * 2048, 5 * 512 * 2048 + 10))
    np.testing.assert_array_equal(g.ravel()[:10], g4)


def test_skew_experts():
    hot = synth.skew_experts(3)
    assert len(hot) == 26 == len(set(hot.tolist()))
    b = synth.skew_bias(3)
    assert np.count_nonzero(b) == 26 and b.max() == np.float32(3.0)
