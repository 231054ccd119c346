"""The dense SwiGLU MLP block (width 6144) against the oracle, through the C ABI.

Seeded synthetic bf16 weights N(0, 0.02) and x N(0, 1); token counts across
the two kernel paths (skinny MFMA below 128 tokens, LDS-tiled MFMA GEMMs from
128 on), with ragged tails; the bar is the layer's: max|err| <= 2e-2 x rms.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu
Y_TOL = 2e-2


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
    ref = O.dense_mlp(x_bits, bits)["y"]
    rms = float(np.sqrt(np.mean(ref ** 2)))
    err = float(np.abs(yg - ref).max())
    print(f"[parity] dense MLP T={T}: max_err/rms={err / rms:.2e}", flush=True)
    assert np.all(np.isfinite(yg))
    assert err <= Y_TOL * rms


def test_dense_mlp_zero_tokens(m, weights):
    _, w = weights
    x = torch.zeros((0, 2048), dtype=torch.int16, device="cuda")
    y = torch.zeros((0, 2048), dtype=torch.int16, device="cuda")
    ws = torch.zeros(256, dtype=torch.uint8, device="cuda")
    m.moe_w4_dense_mlp(x, w, y, ws)
