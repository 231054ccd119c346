"""Parity helpers: run the HIP layer and the CPU oracle on the same seeded
inputs and compare them to the stated bar.

Bar (the layer's stated contract):
  * the set of chosen experts equal, for every token whose oracle 6th/7th
    logit gap exceeds 1e-3 (near-ties are flagged and counted, not failed);
    their slot order (descending logit) equal too, unless two of the chosen
    logits are within 1e-3 (an order tie, flagged the same way);
  * offsets and perm bit-exact when every token is routed identically;
    otherwise offsets must equal the histogram of the GPU's own indices and
    perm must be the stable sort of those indices;
  * topk_w within 1e-5 relative of the oracle's (fp32 sigmoid vs fp64);
  * y (bf16), over the tokens with the oracle's chosen set: the error beyond
    the rounding of the exact output to bf16, |y_gpu - y_oracle| - ulp(y_oracle)/2,
    at most 2e-2 * rms(y_oracle).  Taken literally, max |y_gpu - y_oracle| <=
    2e-2 * rms is not attainable by any bf16 output where that half ulp alone
    exceeds 2e-2 rms: outputs of |y| >= 8 with rms ~1.3, which the skewed
    prefill workload has (its correctly rounded output at 6.7 rms is 0.0267
    from the exact value, against a bar of 0.0259);
  * and element by element the same error beyond the output's rounding at most
    Y_ELEM_TOL * rms(y_oracle): the roundings of the kernels' intermediates
    (the fp16 operands of the routed experts, their fp16 expert rows on the
    MFMA path, fp32 sums in another order), which the 2e-2 bar alone would
    let hide in any output smaller than 0.02 rms.
"""
from __future__ import annotations

import concurrent.futures as cf
import functools
import os

import numpy as np
import torch

import synth
from oracle import moe_oracle as O

Y_TOL = 2e-2
Y_ELEM_TOL = 5e-3
W_RTOL = 1e-5


def half_ulp_bf16(v):
    """Half the spacing of bf16 numbers at |v| (8 significant bits; the
    subnormal spacing 2^-133 below 2^-126)."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    _, e = np.frexp(np.where(a > 0, a, 1.0))           # a in [2^(e-1), 2^e)
    return np.ldexp(1.0, np.maximum(e - 9, -134))


@functools.lru_cache(maxsize=None)
def _host_expert(seed, layer, e):
    codes, scales = synth.gen_codes_scales(seed, layer, experts=[e])
    return codes[0], scales[0]


def host_blobs(seed, layer=0, scale_mult_log2=0):
    def blobs(e):
        c, s = _host_expert(seed, layer, e)
        if scale_mult_log2:
            f = O.bf16_to_f64(s) * 2.0 ** scale_mult_log2
            s = O.f64_to_bf16_bits(f)
        return c, s
    return blobs


@functools.lru_cache(maxsize=None)
def host_router(seed, layer=0):
    return synth.gen_router(seed, layer)


@functools.lru_cache(maxsize=None)
def host_shared(seed, layer=0):
    return synth.gen_shared(seed, layer)


def to_dev_u16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def from_dev_u16(t):
    return t.cpu().numpy().view(np.uint16)


_POOL = None


def pool():
    """A thread pool for the oracle's expert evaluations (NumPy releases the
    interpreter lock in its array work), sized to this process's cores."""
    global _POOL
    if _POOL is None:
        _POOL = cf.ThreadPoolExecutor(max_workers=max(1, min(16, len(os.sched_getaffinity(0)))))
    return _POOL


def run_gpu(m, x_bits, w, bias=None, ws=None, poison=False, policy=None, nvfp4=None):
    """Run one forward; returns y bits and the routing results read from the
    workspace.  nvfp4: dict(codes, scales, tscales) of NVFP4 experts (device
    tensors) to run moe_w4_forward_nvfp4 instead of the int4 layer."""
    T = x_bits.shape[0]
    x = to_dev_u16(x_bits)
    y = torch.empty((T, 2048), dtype=torch.int16, device="cuda")
    if ws is None:
        ws = m.workspace(T)
    if poison:
        ws.fill_(0xFF)
    b = None if bias is None else torch.from_numpy(np.asarray(bias, dtype=np.float32)).cuda()
    if nvfp4 is not None:
        m.moe_w4_forward_nvfp4(x, w["router_w"], nvfp4["codes"], nvfp4["scales"], nvfp4["tscales"], w["shared_w"],
                               y, ws, router_bias=b)
    elif policy is None:
        m.moe_w4_forward(x, w["router_w"], w["codes"], w["scales"], w["shared_w"], y, ws, router_bias=b)
    else:
        m.moe_w4_forward_policy(x, w["router_w"], w["codes"], w["scales"], w["shared_w"], y, ws, router_bias=b,
                                router_policy=policy)
    torch.cuda.synchronize()
    out = dict(y_bits=from_dev_u16(y))
    out["topk_idx"] = m.ws_view(ws, T, "topk_idx", torch.int32, 6 * T).cpu().numpy().reshape(T, 6)
    out["topk_w"] = m.ws_view(ws, T, "topk_w", torch.float32, 6 * T).cpu().numpy().reshape(T, 6)
    out["offsets"] = m.ws_view(ws, T, "offsets", torch.int32, 257).cpu().numpy()
    out["perm"] = m.ws_view(ws, T, "perm", torch.int32, 6 * T).cpu().numpy()
    out["pos"] = m.ws_view(ws, T, "pos", torch.int32, 6 * T).cpu().numpy()
    out["n_active"] = int(m.ws_view(ws, T, "n_active", torch.int32, 1).cpu().numpy()[0])
    out["active"] = m.ws_view(ws, T, "active", torch.int32, 8 * 256).cpu().numpy().reshape(256, 8)
    return out


def compare(gpu, ref, tokens=None, label=""):
    """Check the bar; returns a summary dict.  `tokens`: rows of ref['y'] (None = all)."""
    T = gpu["topk_idx"].shape[0]
    flagged = ref["near_tie"]
    order_flag = ref["order_tie"]
    same_route = np.all(gpu["topk_idx"] == ref["topk_idx"], axis=1)
    same_set = np.all(np.sort(gpu["topk_idx"], axis=1) == np.sort(ref["topk_idx"], axis=1), axis=1)
    bad = ~same_set & ~flagged
    assert not bad.any(), f"{label}: chosen experts differ on unflagged tokens {np.nonzero(bad)[0][:10]}"
    bad = same_set & ~same_route & ~order_flag
    assert not bad.any(), f"{label}: slot order differs without an order tie on tokens {np.nonzero(bad)[0][:10]}"
    ok = same_set
    # weights compared expert by expert (the slot order may differ on order ties)
    go = np.argsort(gpu["topk_idx"], axis=1, kind="stable")
    ro = np.argsort(ref["topk_idx"], axis=1, kind="stable")
    np.testing.assert_allclose(np.take_along_axis(gpu["topk_w"], go, 1)[ok],
                               np.take_along_axis(ref["topk_w"], ro, 1)[ok], rtol=W_RTOL, atol=1e-7,
                               err_msg=f"{label}: topk_w")
    # sort results
    if same_route.all():
        np.testing.assert_array_equal(gpu["offsets"], ref["offsets"], err_msg=f"{label}: offsets")
        np.testing.assert_array_equal(gpu["perm"], ref["perm"], err_msg=f"{label}: perm")
        np.testing.assert_array_equal(gpu["pos"], ref["pos"], err_msg=f"{label}: pos")
    else:
        own = O.sort_assignments(gpu["topk_idx"])
        for k in ("offsets", "perm", "pos"):
            np.testing.assert_array_equal(gpu[k], own[k], err_msg=f"{label}: {k} vs the GPU's own indices")
    counts = np.diff(gpu["offsets"])
    act = np.nonzero(counts)[0]
    assert gpu["n_active"] == len(act)
    rec = gpu["active"]
    np.testing.assert_array_equal(rec[:len(act), 0], act)
    np.testing.assert_array_equal(rec[len(act):, 0], -1)
    np.testing.assert_array_equal(rec[:len(act), 1], gpu["offsets"][act])
    np.testing.assert_array_equal(rec[:len(act), 2], counts[act])
    perm = gpu["perm"]
    np.testing.assert_array_equal(rec[:len(act), 3], perm[gpu["offsets"][act]] // 6)
    second = np.where(counts[act] > 1, gpu["offsets"][act] + 1, gpu["offsets"][act])
    np.testing.assert_array_equal(rec[:len(act), 4], perm[second] // 6)
    # output
    rows = np.arange(T) if tokens is None else np.asarray(tokens)
    yr = ref["y"]                                      # fp64, rows = `rows`
    yg = O.bf16_to_f64(gpu["y_bits"][rows])
    keep = ok[rows]
    rms = float(np.sqrt(np.mean(yr ** 2)))
    err = np.abs(yg[keep] - yr[keep])
    max_err = float(err.max()) if err.size else 0.0
    assert np.all(np.isfinite(yg[keep])), f"{label}: non-finite output"
    excess = (err - half_ulp_bf16(yr[keep])) / rms if rms else np.zeros_like(err)
    elem = float(excess.max()) if excess.size else 0.0
    assert elem <= Y_TOL, f"{label}: error beyond the bf16 rounding of y {elem:.3e} * rms > {Y_TOL} * rms"
    if elem > Y_ELEM_TOL:
        i = np.unravel_index(int(np.argmax(excess)), excess.shape)
        raise AssertionError(f"{label}: element {i} of the compared rows: |err| {err[i]:.3e} exceeds half an ulp "
                             f"of {yr[keep][i]:.4e} + {Y_ELEM_TOL} * rms ({elem:.3e} * rms beyond the ulp)")
    return dict(T=T, flagged=int(flagged.sum()), rerouted=int((~same_set).sum()),
                reordered=int((same_set & ~same_route).sum()), max_err=max_err, rms=rms,
                ratio=max_err / rms if rms else 0.0, elem=elem)
