"""The packer (bf16 expert weights -> int4 codes and bf16 scales) against the
oracle's fp32 quantiser, through the C ABI: bit-exact codes and scales.

Inputs: seeded synthetic bf16 weights with the workload's distribution
(N(0, 0.02)), plus groups that exercise the edges (all zero, one-hot rows,
large and tiny magnitudes, a group whose absmax sits at a bf16 rounding tie).
At full size (one layer, 256 experts) sampled experts are compared exactly
and every expert's reconstruction error is checked against the model card's
11.7% figure.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import moe_oracle as O
from tests.conftest import golden_constants

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    from int4_routed_expert_amd import moe_w4
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return moe_w4


def host_weights(seed, n):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((n, O.EXPERT_WEIGHTS)) * 0.02).astype(np.float32)
    bits = synth.f32_to_bf16_bits(w)
    if n >= 2:
        e = bits[1]
        e[0:128] = 0                                            # a zero group
        e[128:256] = 0
        e[128 + 40] = synth.f32_to_bf16_bits(np.float32([1.0]))[0]   # a one-hot group
        e[256:384] = synth.f32_to_bf16_bits((rng.standard_normal(128) * 3e4).astype(np.float32))
        e[384:512] = synth.f32_to_bf16_bits((rng.standard_normal(128) * 1e-30).astype(np.float32))
        # the down plane's last group: the same value everywhere
        e[-128:] = synth.f32_to_bf16_bits(np.float32([0.75]))[0]
    return bits


def run_pack(m, bits):
    n = bits.shape[0]
    w = torch.from_numpy(bits.view(np.int16)).cuda()
    codes = torch.full((n, m.CODE_BYTES_PER_EXPERT), 0x5A, dtype=torch.uint8, device="cuda")
    scales = torch.full((n, m.SCALES_PER_EXPERT), 0x1234, dtype=torch.int16, device="cuda")
    m.moe_w4_pack_experts(w, codes, scales)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("n", [1, 3])
def test_pack_matches_oracle_bit_exact(m, n):
    bits = host_weights(40 + n, n)
    codes, scales = run_pack(m, bits)
    rc, rs = O.pack_expert_bank(bits)
    np.testing.assert_array_equal(scales, rs)
    np.testing.assert_array_equal(codes, rc)
    print(f"[pack] {n} experts: codes and scales bit-exact", flush=True)


def test_pack_zero_experts_is_a_noop(m):
    w = torch.zeros(16, dtype=torch.int16, device="cuda")
    codes = torch.full((16,), 7, dtype=torch.uint8, device="cuda")
    scales = torch.full((16,), 7, dtype=torch.int16, device="cuda")
    m.moe_w4_pack_experts(w, codes, scales, n_experts=0)
    torch.cuda.synchronize()
    assert int(codes.sum()) == 7 * 16 and int(scales.sum()) == 7 * 16


def test_pack_full_layer(m):
    """One layer's 256 experts generated on the device; two sampled experts
    bit-exact against the oracle, and the dequantised-and-unrotated weights of
    every expert within the card's relative error."""
    n = 256
    g = torch.Generator(device="cuda").manual_seed(5)
    w = (torch.randn((n, O.EXPERT_WEIGHTS), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    codes = torch.empty((n, m.CODE_BYTES_PER_EXPERT), dtype=torch.uint8, device="cuda")
    scales = torch.empty((n, m.SCALES_PER_EXPERT), dtype=torch.int16, device="cuda")
    m.moe_w4_pack_experts(w.view(torch.int16), codes, scales)
    torch.cuda.synchronize()
    for e in (0, 201):
        bits = w[e:e + 1].view(torch.int16).cpu().numpy().view(np.uint16)
        rc, rs = O.pack_expert_bank(bits)
        np.testing.assert_array_equal(scales[e].cpu().numpy().view(np.uint16), rs[0])
        np.testing.assert_array_equal(codes[e].cpu().numpy(), rc[0])
    # reconstruction error of every expert's gate/up plane, on the device:
    # decode the nibbles, scale, and compare in the rotated basis (the rotation
    # is orthogonal, so the relative error is the same in both bases)
    c = golden_constants()
    rel = []
    for e0 in range(0, n, 32):
        cb = codes[e0:e0 + 32].to(torch.int32)
        lo = (cb & 15) - ((cb & 8) << 1)
        hi = ((cb >> 4) & 15) - (((cb >> 4) & 8) << 1)
        q = torch.stack([lo, hi], dim=-1).reshape(32, -1).float()
        s = scales[e0:e0 + 32].view(torch.bfloat16).float().repeat_interleave(128, dim=1)
        deq = (q * s)[:, :2 * 512 * 2048].reshape(-1, 128)
        src = w[e0:e0 + 32, :2 * 512 * 2048].float().reshape(-1, 128)
        h = torch.from_numpy(O.hadamard(128)).float().cuda()
        rot = src @ h
        err = (deq - rot).reshape(32, -1).norm(dim=1) / rot.reshape(32, -1).norm(dim=1)
        rel.append(err.cpu().numpy())
    rel = np.concatenate(rel)
    print(f"[pack] 256 experts: relative Frobenius error of the gate/up planes {rel.min():.4f}..{rel.max():.4f}",
          flush=True)
    assert np.all(np.abs(rel - c["int4_rel_frobenius"]) < 0.01)


def test_pack_against_the_fp64_quantiser(m):
    """The packer's output against the oracle's fp64 quantiser, which shares
    no stage order with the packer's fp32 one: a scale moves by at most one
    bf16 step (rarely), and inside groups of equal scale a code moves by at
    most one step, only on rounding boundaries (the card's format; the
    quantiser is the plain reading absmax / 7 and round-half-even)."""
    bits = host_weights(61, 3)
    codes, scales = run_pack(m, bits)
    H, I, n = O.H, O.I_R, bits.shape[0]
    nb_gu, ns_gu = 2 * I * H // 2, 2 * I * H // O.G
    n_scales = n_codes = n_scale_moves = n_code_moves = 0
    for e in range(n):
        w = O.bf16_to_f64(bits[e])
        planes = ((w[:2 * I * H].reshape(2 * I, H), codes[e, :nb_gu].reshape(2 * I, H // 2), scales[e, :ns_gu]),
                  (w[2 * I * H:].reshape(H, I), codes[e, nb_gu:].reshape(H, I // 2), scales[e, ns_gu:]))
        for wp, cp, sp in planes:
            k = wp.shape[1]
            c64, s64 = O.quantize_rotated(wp)
            s_gpu = sp.reshape(s64.shape)
            ds = np.abs(s_gpu.astype(np.int32) - s64.astype(np.int32))
            assert ds.max() <= 1
            same = np.repeat(ds == 0, O.G, axis=1)
            dc = np.abs(O.unpack_int4(cp, k).astype(np.int32) - c64)
            assert dc[same].max() <= 1
            n_scales += s64.size
            n_scale_moves += int((ds != 0).sum())
            n_codes += int(same.sum())
            n_code_moves += int((dc[same] != 0).sum())
    print(f"[pack] against the fp64 quantiser: {n_scale_moves} of {n_scales} scales one step apart, "
          f"{n_code_moves} of {n_codes} codes one step apart", flush=True)
    assert n_scale_moves <= 1e-3 * n_scales
    assert n_code_moves <= 1e-4 * n_codes
