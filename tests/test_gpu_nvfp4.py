"""The layer with NVFP4 experts (moe_w4_forward_nvfp4) vs the CPU oracle.

Inputs: the seeded layer of seed 0 (router, shared expert and the code bytes,
read as E2M1 codes), seeded E4M3 block scales and fp32 tensor scales.  Sizes
cover the launch sequences the entry point uses (1-48 tokens: the one-workgroup
routing; 49-127: top-6 and sort; from 128: the dense router/shared GEMMs), with
ragged tails of the expert tiles; T = 2048 on sampled tokens.  Edge cases:
T = 0, zero codes (the routed part vanishes), scales 256 times larger, a NaN
block scale, and the same result twice.  Bar: that of tests/parity.py.
"""
import functools

import numpy as np
import pytest
import torch

import synth
from oracle import moe_oracle as O
from tests import parity as P

pytestmark = pytest.mark.gpu
SEED = 0


@pytest.fixture(scope="module")
def m():
    from int4_routed_expert_amd import moe_w4
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return moe_w4


@pytest.fixture(scope="module")
def layer0(m):
    w = m.generated_layer(SEED, 0)
    torch.cuda.synchronize()
    return w


@functools.lru_cache(maxsize=None)
def host_scales():
    return synth.gen_nvfp4_scales(SEED, 0)


@functools.lru_cache(maxsize=None)
def host_tscales():
    return synth.gen_nvfp4_tensor_scales(SEED, 0)


@pytest.fixture(scope="module")
def nv(m, layer0):
    return dict(codes=layer0["codes"],
                scales=torch.from_numpy(host_scales().ravel().copy()).cuda(),
                tscales=torch.from_numpy(host_tscales().ravel().copy()).cuda())


def blobs(scales=None, tscales=None, zero_codes=False):
    sc = host_scales() if scales is None else scales
    ts = host_tscales() if tscales is None else tscales

    def f(e):
        c = P._host_expert(SEED, 0, e)[0]
        if zero_codes:
            c = np.zeros_like(c)
        return c, sc[e], ts[e]
    return f


def oracle(x_bits, tokens=None, **kw):
    return O.moe_layer_nvfp4(x_bits, P.host_router(SEED), blobs(**kw), P.host_shared(SEED), tokens=tokens)


def report(label, s):
    print(f"[nvfp4] {label}: T={s['T']} flagged={s['flagged']} rerouted={s['rerouted']} "
          f"max_err/rms={s['ratio']:.2e}", flush=True)


@pytest.mark.parametrize("T", [1, 5, 8, 9, 32, 48, 49, 100, 130])
def test_nvfp4_layer(m, layer0, nv, T):
    print(f"[nvfp4] case T={T}", flush=True)
    x_bits = synth.gen_x(11, T)
    gpu = P.run_gpu(m, x_bits, layer0, nvfp4=nv)
    # past 48 tokens the oracle's outputs on 8 tokens (the first, the last, and
    # spread between; routing and sort still cover all of them)
    tokens = None if T <= 48 else np.unique(np.linspace(0, T - 1, 8).astype(int))
    s = P.compare(gpu, oracle(x_bits, tokens=tokens), tokens=tokens, label=f"nvfp4 T={T}")
    report(f"T={T}", s)


def test_nvfp4_full_prefill_sampled(m, layer0, nv):
    T = 2048
    print(f"[nvfp4] case T={T} sampled", flush=True)
    x_bits = synth.gen_x(12, T)
    gpu = P.run_gpu(m, x_bits, layer0, nvfp4=nv)
    tokens = np.array([0, 1, 777, 1500, 2047])
    s = P.compare(gpu, oracle(x_bits, tokens=tokens), tokens=tokens, label="nvfp4 T=2048")
    report("T=2048 sampled", s)


def test_nvfp4_zero_tokens_is_a_noop(m, layer0, nv):
    x = torch.zeros((1, 2048), dtype=torch.int16, device="cuda")
    y = torch.full((1, 2048), 7, dtype=torch.int16, device="cuda")
    ws = m.workspace(1)
    assert m.moe_w4_forward_nvfp4(x, layer0["router_w"], nv["codes"], nv["scales"], nv["tscales"],
                                  layer0["shared_w"], y, ws, T=0) == m.OK
    torch.cuda.synchronize()
    assert torch.all(y == 7)


def test_nvfp4_zero_codes_leave_the_shared_expert(m, layer0, nv):
    T = 16
    print("[nvfp4] case zero codes", flush=True)
    x_bits = synth.gen_x(13, T)
    zero = dict(nv, codes=torch.zeros_like(nv["codes"]))
    gpu = P.run_gpu(m, x_bits, layer0, nvfp4=zero)
    ref = oracle(x_bits, zero_codes=True)
    assert np.all(ref["routed"] == 0.0)
    P.compare(gpu, ref, label="nvfp4 zero codes")


def test_nvfp4_large_scales(m, layer0, nv):
    # every block scale 2^8 times larger (exponent field + 8): weights ~8,
    # expert outputs ~10^4 times the shared expert's
    T = 24
    print("[nvfp4] case large scales", flush=True)
    big = (host_scales() + np.uint8(0x40)).astype(np.uint8)
    x_bits = synth.gen_x(14, T)
    dev = dict(nv, scales=torch.from_numpy(big.ravel().copy()).cuda())
    gpu = P.run_gpu(m, x_bits, layer0, nvfp4=dev)
    s = P.compare(gpu, oracle(x_bits, scales=big), label="nvfp4 large scales")
    report("large scales", s)


def test_nvfp4_nan_scale_poisons_only_its_tokens(m, layer0, nv):
    T = 12
    print("[nvfp4] case NaN scale", flush=True)
    x_bits = synth.gen_x(15, T)
    ref = oracle(x_bits)
    e_bad = int(ref["topk_idx"][0, 0])
    sc = host_scales().copy()
    sc[e_bad, :O.I_R * O.H // O.NV_BLOCK] = 0x7F          # every gate block scale of e_bad: NaN
    dev = dict(nv, scales=torch.from_numpy(sc.ravel().copy()).cuda())
    gpu = P.run_gpu(m, x_bits, layer0, nvfp4=dev)
    y = O.bf16_to_f64(gpu["y_bits"])
    hit = np.any(gpu["topk_idx"] == e_bad, axis=1)
    assert hit[0]
    assert np.all(np.isnan(y[hit]))
    assert np.all(np.isfinite(y[~hit]))


def test_nvfp4_deterministic(m, layer0, nv):
    T = 40
    x_bits = synth.gen_x(16, T)
    a = P.run_gpu(m, x_bits, layer0, nvfp4=nv)["y_bits"]
    b = P.run_gpu(m, x_bits, layer0, nvfp4=nv, poison=True)["y_bits"]
    np.testing.assert_array_equal(a, b)
