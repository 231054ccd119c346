"""The dense SwiGLU MLP block (width 6144) against the oracle, through the C ABI.

Seeded synthetic bf16 weights N(0, 0.02) and x N(0, 1); token counts across
the two kernel paths (skinny MFMA below 128 tokens, LDS-tiled MFMA GEMMs from
128 on), with ragged tails; the bar is the layer's (tests/parity.py): the error
beyond the bf16 rounding of y at most 2e-2 x rms, and element by element at
most Y_ELEM_TOL x rms.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import moe_oracle as O
from tests import parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    from int4_routed_expert_amd import moe_w4
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return moe_w4


@pytest.fixture(scope="module")
def weights():
    rng = np.random.default_rng(50)
    bits = synth.f32_to_bf16_bits((rng.standard_normal(O.DENSE_WEIGHTS) * 0.02).astype(np.float32))
    return bits, torch.from_numpy(bits.view(np.int16)).cuda()


def check(yg, ref, label):
    rms = float(np.sqrt(np.mean(ref ** 2)))
    err = np.abs(yg - ref)
    excess = float(((err - P.half_ulp_bf16(ref)) / rms).max())
    print(f"[parity] {label}: max_err/rms={err.max() / rms:.2e} beyond-half-ulp/rms={excess:.2e}", flush=True)
    assert np.all(np.isfinite(yg))
    assert excess <= P.Y_ELEM_TOL <= P.Y_TOL


@pytest.mark.parametrize("T", [1, 5, 16, 33, 127, 128, 300])
def test_dense_mlp_matches_oracle(m, weights, T):
    bits, w = weights
    x_bits = synth.gen_x(500 + T, T)
    x = torch.from_numpy(x_bits.view(np.int16)).cuda()
    y = torch.empty((T, 2048), dtype=torch.int16, device="cuda")
    ws = torch.full((m.moe_w4_dense_mlp_workspace_bytes(T),), 0xFF, dtype=torch.uint8, device="cuda")
    m.moe_w4_dense_mlp(x, w, y, ws)
    torch.cuda.synchronize()
    yg = O.bf16_to_f64(y.cpu().numpy().view(np.uint16))
    check(yg, O.dense_mlp(x_bits, bits)["y"], f"dense MLP T={T}")


def test_dense_mlp_largest_token_count(m, weights):
    """T = MAX_TOKENS: 512 row tiles of the GEMMs; sampled rows, the last
    tile's among them, against the oracle on those rows (rows are independent)."""
    bits, w = weights
    T = m.MAX_TOKENS
    rng = np.random.default_rng(51)
    x_bits = synth.f32_to_bf16_bits(rng.standard_normal((T, 2048)).astype(np.float32))
    x = torch.from_numpy(x_bits.view(np.int16)).cuda()
    y = torch.empty((T, 2048), dtype=torch.int16, device="cuda")
    ws = torch.empty((m.moe_w4_dense_mlp_workspace_bytes(T),), dtype=torch.uint8, device="cuda")
    m.moe_w4_dense_mlp(x, w, y, ws)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 127, 128, T - 129, T - 2, T - 1], rng.choice(T, 10, replace=False)]))
    yg = O.bf16_to_f64(y.cpu().numpy().view(np.uint16)[rows])
    check(yg, O.dense_mlp(x_bits[rows], bits)["y"], f"dense MLP T={T} (sampled rows)")


def test_dense_mlp_zero_tokens(m, weights):
    _, w = weights
    x = torch.zeros((0, 2048), dtype=torch.int16, device="cuda")
    y = torch.zeros((0, 2048), dtype=torch.int16, device="cuda")
    ws = torch.zeros(256, dtype=torch.uint8, device="cuda")
    m.moe_w4_dense_mlp(x, w, y, ws)
