"""Throughput of the int4 routed-expert MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME] [--no-cpu]
    python bench.py --copy-calibration           # plain device copy, for HBM counter scaling
    python bench.py --pmc-summary RUN.csv ...    # per-kernel means of rocprofv3 --pmc CSVs

A step is one pass of the whole layer (router, sort, rotation, routed experts,
shared expert, combine) over one batch of seeded synthetic tokens, with
weights and inputs already resident in HBM.  Consecutive steps use different
layers' weights (generated on the device from the same seeded recipe; 24
layers at T = 1, whose 23.4 MB per layer would otherwise fit the 256 MB
Infinity Cache, 4 at larger T), so a step cannot be served from the cache
contents of the steps before it, as in a real layer stack.  Prints one JSON
line: `value` is tokens/s over exactly K back-to-back steps; `step_us` gives
the median, p10 and p90 of at least 200 steps timed one by one with HIP
events; `roofline` is that of the dominant stage.

The default workload is decode_t32: T = 32 tokens (8 sequences x (1 decoded +
3 speculative)), x seed 1, weights seed 0.  Its line also carries the
metric's other points under "points": decode_t1 (T = 1) and prefill_t2048
(T = 2048, uniform and skewed routing), each timed the same way with its own
roofline.  The stack configs run moe_w4_stack_forward over 47 layers.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16/fp16 MFMA, published

EXPERT_GU_BYTES = 1_048_576 + 32_768      # one expert's [gate; up] codes + scales
EXPERT_D_BYTES = 524_288 + 16_384         # one expert's down codes + scales
EXPERT_BYTES = EXPERT_GU_BYTES + EXPERT_D_BYTES
NV_GU_BYTES = 1_048_576 + 131_072 + 8     # one NVFP4 expert's [gate; up] codes, E4M3 scales, tensor scales
NV_D_BYTES = 524_288 + 65_536 + 4          # its down codes, scales, tensor scale
ROUTER_BYTES = 256 * 2048 * 2
SHARED_BYTES = 3 * 1024 * 2048 * 2


def roofline_entry(kernel, nbytes, flops, kernel_us, traffic):
    """The roofline of one kernel: its binding roof is the one whose peak takes
    longer for the kernel's algorithmic work (HBM bytes at 8 TB/s against
    MFMA flops at 2.5 PFLOP/s, i.e. arithmetic intensity below or above the
    ridge of 312 flop/B); both fractions are reported."""
    sec = kernel_us * 1e-6
    gbs = nbytes / sec / 1e9
    tf = flops / sec / 1e12 if flops else 0.0
    mfma_bound = flops and flops / (MFMA_BF16_PEAK_TFLOPS * 1e12) > nbytes / (HBM_PEAK_GBS * 1e9)
    r = {"bound": "mfma" if mfma_bound else "hbm", "kernel": kernel,
         "achieved": tf if mfma_bound else gbs, "peak": MFMA_BF16_PEAK_TFLOPS if mfma_bound else HBM_PEAK_GBS,
         "unit": "TFLOP/s" if mfma_bound else "GB/s"}
    r["frac"] = r["achieved"] / r["peak"]
    r["traffic"] = traffic
    r["algorithmic_bytes"] = nbytes
    if flops:
        r["algorithmic_flops"] = flops
        r["hbm_frac"] = gbs / HBM_PEAK_GBS
        r["mfma_frac"] = tf / MFMA_BF16_PEAK_TFLOPS
    r["kernel_us"] = kernel_us
    return r


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="decode_t32",
                    choices=["decode_t1", "decode_t32", "prefill_t2048", "prefill_t2048_skew", "stack_t1", "stack_t8",
                             "pack_layer", "mlp_t1", "mlp_t2048", "nvfp4_t1", "nvfp4_t32", "nvfp4_t2048"])
    ap.add_argument("--layers", type=int, default=0, help="distinct layers rotated through (0 = auto)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--eager", action="store_true",
                    help="stack configs: launch every layer from the host instead of replaying a captured graph")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="oracle baseline: seconds per thread setting (all cores, then one thread)")
    ap.add_argument("--headline-only", action="store_true",
                    help="decode_t32: skip the T = 1 and T = 2048 points of the default line")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain device-to-device copy of known size (10 x 256 MiB)")
    ap.add_argument("--traffic-lines", nargs=5,
                    metavar=("WORKLOAD", "FETCH_CSV", "WRITE_CSV", "CAL_FETCH_CSV", "CAL_WRITE_CSV"),
                    help="print profiles/hbm_traffic.txt lines for the workload's kernels from rocprofv3 "
                         "FETCH_SIZE / WRITE_SIZE runs of it and of --copy-calibration")
    ap.add_argument("--pmc-summary", nargs="+", metavar="CSV",
                    help="print per-kernel mean counter values of rocprofv3 counter_collection CSVs")
    return ap.parse_args()


# stage -> (kernel name prefix, sources that define it) for the HBM-traffic
# record, per launch sequence (1-8 tokens: two launches; 9-127: GEMVs, the
# routing in one launch of one workgroup per 8 tokens up to 48 tokens; from
# 128: MFMA tiles)
FUSED_MAX_TOKENS = 8
ROUTE_SMALL_MAX_TOKENS = 48
GROUPED_MIN_TOKENS = 128
STAGE_KERNELS_FUSED = {
    "router_shared_gateup": ("k_router_small", ["decode_fused.hip", "gemv_ops.h", "token_ops.h"]),
    "routed_gateup": ("k_decode_fused", ["decode_fused.hip", "gemv_ops.h", "token_ops.h", "nvfp4_ops.h"]),
}
STAGE_KERNELS_GEMV = {
    "router_shared_gateup": ("k_skinny", ["skinny_mfma.hip"]),
    "topk_sort": ("k_topk_rotate", ["router.hip", "token_ops.h"]),
    "routed_gateup": ("k_gateup_dec", ["experts_gemv.hip", "gemv_ops.h"]),
    "routed_down": ("k_down_dec", ["experts_gemv.hip", "gemv_ops.h"]),
    "shared_down_combine": ("k_skinny", ["skinny_mfma.hip"]),
}
STAGE_KERNELS_GROUPED = {
    "router_shared_gateup": ("k_dense_mfma<2048", ["dense_mfma.hip"]),
    "topk_sort": ("k_topk_rotate", ["router.hip", "token_ops.h"]),
    "routed_gateup": ("k_gateup_mfma", ["grouped_mfma.hip"]),
    "routed_down": ("k_down_mfma", ["grouped_mfma.hip"]),
    "shared_down_combine": ("k_dense_mfma<1024", ["dense_mfma.hip"]),
}


STAGE_KERNELS_PACK = {"pack": ("k_pack_groups", ["pack.hip"])}


STAGE_KERNELS_NVFP4 = {
    "routed_gateup": ("k_gateup_nv", ["nvfp4.hip", "nvfp4_ops.h", "gemv_ops.h", "token_ops.h"]),
    "routed_down": ("k_down_nv", ["nvfp4.hip", "nvfp4_ops.h", "gemv_ops.h", "token_ops.h"]),
}
# from 128 tokens on the NVFP4 experts run on the grouped MFMA kernels
STAGE_KERNELS_NVFP4_MFMA = {
    "routed_gateup": ("k_gateup_mfma<true", ["grouped_mfma.hip"]),
    "routed_down": ("k_down_mfma<true", ["grouped_mfma.hip"]),
}


def stage_kernels(T, workload=""):
    if T is None:   # the packer workload
        return STAGE_KERNELS_PACK
    if workload.startswith("nvfp4") and T > FUSED_MAX_TOKENS:
        return STAGE_KERNELS_NVFP4_MFMA if T >= GROUPED_MIN_TOKENS else STAGE_KERNELS_NVFP4
    if T <= FUSED_MAX_TOKENS:
        return STAGE_KERNELS_FUSED
    if T >= GROUPED_MIN_TOKENS:
        return STAGE_KERNELS_GROUPED
    if T <= ROUTE_SMALL_MAX_TOKENS:
        # the router, shared gate/up and rotation of x, then the routing launch
        return dict(STAGE_KERNELS_GEMV, topk_sort=("k_route_par", ["router.hip", "route_small.h", "handoff.h",
                                                                  "token_ops.h"]))
    return STAGE_KERNELS_GEMV


HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "int4_routed_expert_amd", "csrc")


def sources_digest(files):
    """sha256 over common.h and the kernel's source files: a recorded traffic
    figure is only valid for the kernel it was measured on."""
    import hashlib
    h = hashlib.sha256()
    for f in ["common.h"] + list(files):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload, stage, T):
    """HBM bytes per launch recorded from rocprofv3 FETCH_SIZE / WRITE_SIZE runs
    (profiles/hbm_traffic.txt), or None if absent or the kernel has changed."""
    kern, files = stage_kernels(T, workload).get(stage, (None, None))
    path = os.path.join(HERE, "profiles", "hbm_traffic.txt")
    if kern is None or not os.path.exists(path):
        return None
    digest = sources_digest(files)
    for line in open(path):
        f = line.split()
        if len(f) == 6 and not line.startswith("#") and f[0] == workload and f[1] == kern and f[5] == digest:
            return float(f[2]) + float(f[3])
    return None


def copy_calibration():
    import torch
    n = 256 << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(10):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": n, "launches": 10}), flush=True)


def pmc_summary(paths):
    import csv
    import collections
    agg = collections.defaultdict(lambda: collections.defaultdict(list))
    for path in paths:
        with open(path) as fh:
            for r in csv.DictReader(fh):
                name = r["Kernel_Name"].replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")
                agg[name][r["Counter_Name"]].append(float(r["Counter_Value"]))
    print(f"{'kernel':48s} {'dispatches':>10s}  counter means (per dispatch)")
    for name, d in sorted(agg.items()):
        n = max(len(v) for v in d.values())
        vals = "  ".join(f"{c}={sum(v) / len(v):.1f}" for c, v in sorted(d.items()))
        print(f"{name[:48]:48s} {n:10d}  {vals}")


def counter_means(path):
    """kernel name (without namespaces and arguments) -> mean counter value (KiB per dispatch)."""
    import csv
    import collections
    agg = collections.defaultdict(list)
    with open(path) as fh:
        for r in csv.DictReader(fh):
            name = r["Kernel_Name"].replace("(anonymous namespace)::", "").split("(")[0]
            name = name.replace("void ", "").split("::")[-1]
            agg[name].append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in agg.items()}


def traffic_lines(workload, fetch_csv, write_csv, cal_fetch_csv, cal_write_csv):
    """Record lines: counters scaled by what they read for a plain copy of known size."""
    import synth
    if workload == "pack_layer":
        T = None
    elif workload.startswith("nvfp4_t"):
        T = int(workload[7:])
    else:
        T = synth.CONFIGS[workload]["T"]
    copy_kib = 256 * 1024   # one calibration copy: 256 MiB read and written
    ffac = copy_kib / counter_means(cal_fetch_csv)["__amd_rocclr_copyBuffer"]
    wfac = copy_kib / counter_means(cal_write_csv)["__amd_rocclr_copyBuffer"]
    fetch, write = counter_means(fetch_csv), counter_means(write_csv)
    print(f"# {workload}: FETCH_SIZE x {ffac:.5f}, WRITE_SIZE x {wfac:.5f}")
    seen = set()
    for stage, (kern, files) in stage_kernels(T, workload).items():
        for name in sorted(fetch):
            if name.startswith(kern) and name not in seen and name in write:
                seen.add(name)
                fb, wb = fetch[name] * 1024 * ffac, write[name] * 1024 * wfac
                print(f"{workload} {kern} {fb:.0f} {wb:.0f} {fb + wb:.0f} {sources_digest(files)}")


def cpu_cores():
    """Cores this process may run on (its affinity mask)."""
    return len(os.sched_getaffinity(0))


def timed_oracle(fn, budget_s, max_reps, threads):
    """Call fn() for about budget_s seconds (at least once) with NumPy's BLAS
    pool limited to `threads`; returns (reps, seconds per rep, BLAS threads
    used).  NumPy's element-wise work is single-threaded either way."""
    from threadpoolctl import threadpool_info, threadpool_limits
    with threadpool_limits(limits=threads):
        used = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] + [1])
        reps, elapsed = 0, 0.0
        while reps == 0 or (elapsed < budget_s and reps < max_reps):
            t0 = time.perf_counter()
            fn()
            elapsed += time.perf_counter() - t0
            reps += 1
    return reps, elapsed / reps, used


def oracle_baseline(fn, units, unit, budget_s, max_reps, sample):
    """The oracle timed on all of this process's cores and on one thread:
    the cpu_baseline object (`units` of work per call of fn)."""
    reps, per, used = timed_oracle(fn, budget_s, max_reps, cpu_cores())
    reps1, per1, _ = timed_oracle(fn, budget_s, max_reps, 1)
    return {"value": units / per, "unit": unit, "cores": int(used), "kind": "oracle",
            "sample": f"{sample}; {reps} calls of {per:.2f} s on {used} BLAS threads ({cpu_cores()} cores in "
                      f"the affinity mask), {reps1} of {per1:.2f} s on one thread",
            "single_thread": {"value": units / per1, "unit": unit, "cores": 1}}


def cpu_baseline(cfg, T, x_bits, bias, budget_s):
    """The CPU oracle as it stands, on a bounded sample of the same workload."""
    import synth
    from oracle import moe_oracle as O
    R = synth.gen_router(0, 0)
    S = synth.gen_shared(0, 0)
    # the oracle routes every token; its expert work is timed on a token sample
    rt = O.route(O.bf16_to_f64(x_bits), R, bias)
    n_tok = T if T <= 32 else 8
    tokens = np.arange(n_tok)
    need = sorted(set(rt["topk_idx"][tokens].ravel().tolist()))
    blobs = {}
    for e in need:                               # input preparation, not timed
        c, s = synth.gen_codes_scales(0, 0, experts=[e])
        blobs[e] = (c[0], s[0])
    return oracle_baseline(lambda: O.moe_layer(x_bits, R, blobs.__getitem__, S, bias=bias, tokens=tokens),
                           n_tok, "tokens/s", budget_s, 50,
                           f"oracle layer calls (fp64 NumPy) on {n_tok} of the {T} tokens, the routing of all "
                           f"{T} included")


def bench_nvfp4(a, T):
    """The layer with NVFP4 experts (moe_w4_forward_nvfp4) at T tokens: the
    seeded layers of the int4 decode configs (their code bytes read as E2M1
    codes) with seeded E4M3 block scales and fp32 tensor scales.  Roofline of
    the dominant stage: HBM (the expert GEMVs stream codes and scales)."""
    import torch
    import synth
    from int4_routed_expert_amd import moe_w4 as m
    from oracle import moe_oracle as O
    cfg = synth.CONFIGS[{1: "decode_t1", 32: "decode_t32", 2048: "prefill_t2048"}[T]]
    assert cfg["T"] == T
    # at T = 1 a layer touches ~24 MB: 24 layers keep the weights a run
    # touches above the 256 MB Infinity Cache, as for the int4 layer
    n_layers = a.layers or DEFAULT_LAYERS.get(T, 4)
    log(f"config {a.config}: T={T}, {n_layers} layers with NVFP4 experts on the device")
    layers = []
    for l in range(n_layers):
        w = m.generated_layer(cfg["w_seed"], l)
        w["nv_scales"] = torch.from_numpy(synth.gen_nvfp4_scales(cfg["w_seed"], l).ravel().copy()).cuda()
        w["nv_tscales"] = torch.from_numpy(synth.gen_nvfp4_tensor_scales(cfg["w_seed"], l).ravel().copy()).cuda()
        layers.append(w)
    x_bits = synth.gen_x(cfg["x_seed"], T)
    x = torch.from_numpy(x_bits.view(np.int16)).cuda()
    y = torch.empty((T, 2048), dtype=torch.int16, device="cuda")
    ws = m.workspace(T)
    n_pts = m.moe_w4_profile_points()
    names = [m.moe_w4_profile_point_name(i) for i in range(n_pts)]

    def step(i, ev=None):
        w = layers[i % n_layers]
        if ev is None:
            m.moe_w4_forward_nvfp4(x, w["router_w"], w["codes"], w["nv_scales"], w["nv_tscales"], w["shared_w"], y, ws)
        else:
            m.moe_w4_forward_nvfp4_profiled(x, w["router_w"], w["codes"], w["nv_scales"], w["nv_tscales"],
                                            w["shared_w"], y, ws, ev)
    for i in range(a.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(a.steps):
        step(i)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / a.steps
    log(f"timed {a.steps} steps: {ms * 1e3:.1f} us/step")
    dist = step_distribution(m, step, max(a.steps, 200))
    events = m.HipEvents(a.steps * n_pts)
    for i in range(a.steps):
        step(i, events.handles[i * n_pts:(i + 1) * n_pts])
    torch.cuda.synchronize()
    stage_ms = np.zeros(n_pts - 1)
    for i in range(a.steps):
        for k in range(n_pts - 1):
            stage_ms[k] += events.elapsed_ms(i * n_pts + k, i * n_pts + k + 1)
    stage_ms /= a.steps
    events.close()
    touched = []
    for l in range(min(n_layers, a.steps)):
        step(l)
        torch.cuda.synchronize()
        touched.append(int(m.ws_view(ws, T, "n_active", torch.int32, 1).item()))
    n_touched = float(np.mean(touched))
    act = T * 2048 * 2
    layer_bytes = n_touched * (NV_GU_BYTES + NV_D_BYTES) + ROUTER_BYTES + SHARED_BYTES + 2 * act
    stage = dict(zip(names[1:], stage_ms))
    dom = max(stage, key=stage.get)
    stage_bytes = {
        "router_shared_gateup": ROUTER_BYTES + 2 * 1024 * 2048 * 2 + act + T * 256 * 4 + T * 1024 * 2,
        "topk_sort": T * 256 * 4 + T * 6 * 4 * 4 + 257 * 4 + 256 * 32,
        "routed_gateup": n_touched * NV_GU_BYTES + act + T * 6 * 512 * 4,
        "routed_down": n_touched * NV_D_BYTES + T * 6 * 512 * 4 + T * 6 * 2048 * 4,
        "shared_down_combine": 1024 * 2048 * 2 + T * 1024 * 2 + T * 6 * 2048 * 4 + act,
    }
    if T <= FUSED_MAX_TOKENS:
        # the two launches of the decode form: the router, then the rest of the
        # layer with the shared expert (recorded under routed_gateup)
        stage_bytes["router_shared_gateup"] = ROUTER_BYTES + act + T * 256 * 4
        stage_bytes["routed_gateup"] = (n_touched * (NV_GU_BYTES + NV_D_BYTES) + SHARED_BYTES + T * 256 * 4 + act
                                        + 2 * T * 1024 * 2 + act)
    dom_bytes = stage_bytes.get(dom, 0.0)
    dom_flops = 0.0
    if T >= GROUPED_MIN_TOKENS:
        dom_flops = {"routed_gateup": T * 6 * 2 * 512 * 2048 * 2, "routed_down": T * 6 * 2048 * 512 * 2}.get(dom, 0.0)
    roof = roofline_entry(dom, dom_bytes, dom_flops, stage[dom] * 1e3, recorded_traffic(a.config, dom, T))
    result = {
        "metric": "routed-MoE layer tokens/s, NVFP4 experts (W4A16)", "value": T / (ms / 1e3), "unit": "tokens/s",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "e2m1 x fp16 -> fp32",
        "data": "synthetic (seeded SplitMix64; random-init weights)",
        "config": {"workload": f"{a.config}: one MoE layer with NVFP4 experts, T={T}, x seed {cfg['x_seed']}, "
                               f"weights seed {cfg['w_seed']}", "T": T, "layers_rotated": n_layers,
                   "touched_experts": n_touched},
        "step_us": dist,
        "roofline": roof,
        "layer": {"algorithmic_bytes": layer_bytes, "hbm_gbs": layer_bytes / (ms * 1e-3) / 1e9,
                  "hbm_frac": layer_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                  "stage_us": {k: v * 1e3 for k, v in stage.items()}},
    }
    if not a.no_cpu:
        log("timing the CPU oracle baseline")
        R, S = synth.gen_router(cfg["w_seed"], 0), synth.gen_shared(cfg["w_seed"], 0)
        rt = O.route(O.bf16_to_f64(x_bits), R)
        sc, ts = synth.gen_nvfp4_scales(cfg["w_seed"], 0), synth.gen_nvfp4_tensor_scales(cfg["w_seed"], 0)
        blobs = {}
        for e in sorted(set(rt["topk_idx"][:min(T, 32)].ravel().tolist())):   # input preparation, not timed
            blobs[e] = (synth.gen_codes_scales(cfg["w_seed"], 0, experts=[e])[0][0], sc[e], ts[e])
        # past 32 tokens the expert work is timed on the first 8 tokens
        n_tok = T if T <= 32 else 8
        tokens = None if T <= 32 else np.arange(n_tok)
        result["cpu_baseline"] = oracle_baseline(
            lambda: O.moe_layer_nvfp4(x_bits, R, blobs.__getitem__, S, tokens=tokens), n_tok, "tokens/s",
            a.cpu_seconds, 50, f"oracle layer calls (fp64 NumPy) on {n_tok} of the {T} tokens, the routing of all "
                               f"{T} included")
    print(json.dumps(result), flush=True)


def bench_pack(a):
    """The packer on one layer's 256 experts: bf16 weights (seeded, N(0, 0.02)) ->
    int4 codes and bf16 scales.  A step is one moe_w4_pack_experts call over the
    whole bank; the roofline is HBM (bf16 in, codes and scales out)."""
    import torch
    from int4_routed_expert_amd import moe_w4 as m
    from oracle import moe_oracle as O
    n = 256
    g = torch.Generator(device="cuda").manual_seed(5)
    w = (torch.randn((n, m.EXPERT_WEIGHTS), generator=g, device="cuda") * 0.02).to(torch.bfloat16).view(torch.int16)
    codes = torch.empty((n, m.CODE_BYTES_PER_EXPERT), dtype=torch.uint8, device="cuda")
    scales = torch.empty((n, m.SCALES_PER_EXPERT), dtype=torch.int16, device="cuda")
    for _ in range(a.warmup):
        m.moe_w4_pack_experts(w, codes, scales)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(a.steps):
        m.moe_w4_pack_experts(w, codes, scales)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / a.steps
    nbytes = n * (m.EXPERT_WEIGHTS * 2 + m.CODE_BYTES_PER_EXPERT + m.SCALES_PER_EXPERT * 2)
    # events on the launch stream (torch's current one) around each launch
    ev = m.HipEvents(2 * a.steps)
    for i in range(a.steps):
        ev.record(2 * i)
        m.moe_w4_pack_experts(w, codes, scales)
        ev.record(2 * i + 1)
    torch.cuda.synchronize()
    kern_ms = float(np.mean([ev.elapsed_ms(2 * i, 2 * i + 1) for i in range(a.steps)]))
    ev.close()
    achieved = nbytes / (kern_ms * 1e-3) / 1e9
    result = {"metric": "packer: experts/s (bf16 experts -> fwht128 int4 codes + bf16 scales)",
              "value": n / (ms * 1e-3), "unit": "experts/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
              "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
              "data": "synthetic", "config": {"workload": "pack_layer: 256 experts of one layer, bf16 N(0, 0.02), "
                                                          "torch seed 5", "experts": n},
              "roofline": {"bound": "hbm", "kernel": "k_pack_groups", "achieved": achieved, "peak": HBM_PEAK_GBS,
                           "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                           "traffic": recorded_traffic("pack_layer", "pack", None),
                           "algorithmic_bytes": nbytes, "kernel_us": kern_ms * 1e3}}
    if not a.no_cpu:
        sample = w[:2].cpu().numpy().view(np.uint16)
        result["cpu_baseline"] = oracle_baseline(lambda: O.pack_expert_bank(sample), 2, "experts/s", a.cpu_seconds,
                                                 20, "oracle packs of 2 of the 256 experts")
    print(json.dumps(result), flush=True)


def bench_mlp(a, T):
    """The dense SwiGLU MLP block (width 6144) over T tokens: seeded bf16 weights
    N(0, 0.02) (4 sets rotated, 302 MB, beyond the Infinity Cache) and x N(0, 1).
    A step is one moe_w4_dense_mlp call (two launches); its roofline is HBM at
    T = 1 and bf16 MFMA at T = 2048, over the whole call."""
    import torch
    import synth
    from int4_routed_expert_amd import moe_w4 as m
    from oracle import moe_oracle as O
    g = torch.Generator(device="cuda").manual_seed(6)
    ws_ = [(torch.randn(m.DENSE_WEIGHTS, generator=g, device="cuda") * 0.02).to(torch.bfloat16).view(torch.int16)
           for _ in range(4)]
    x_bits = synth.gen_x(6, T)
    x = torch.from_numpy(x_bits.view(np.int16)).cuda()
    y = torch.empty((T, 2048), dtype=torch.int16, device="cuda")
    work = torch.empty(m.moe_w4_dense_mlp_workspace_bytes(T), dtype=torch.uint8, device="cuda")
    for i in range(a.warmup):
        m.moe_w4_dense_mlp(x, ws_[i % 4], y, work)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(a.steps):
        m.moe_w4_dense_mlp(x, ws_[i % 4], y, work)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / a.steps
    ev = m.HipEvents(2 * a.steps)
    for i in range(a.steps):
        ev.record(2 * i)
        m.moe_w4_dense_mlp(x, ws_[i % 4], y, work)
        ev.record(2 * i + 1)
    torch.cuda.synchronize()
    call_ms = float(np.mean([ev.elapsed_ms(2 * i, 2 * i + 1) for i in range(a.steps)]))
    ev.close()
    nbytes = m.DENSE_WEIGHTS * 2 + 2 * T * 2048 * 2
    flops = 2 * T * 3 * m.DENSE_INTER * 2048
    roof = roofline_entry("dense MLP call (gate/up + down launches)", nbytes, flops if T >= 128 else 0.0,
                          call_ms * 1e3, None)
    result = {"metric": "dense SwiGLU MLP block (width 6144) tokens/s", "value": T / (ms * 1e-3), "unit": "tokens/s",
              "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "ms_per_step": ms, "higher_is_better": True,
              "scaling": "weak", "vs_baseline": None, "dtype": "bf16 x bf16 -> fp32", "data": "synthetic",
              "config": {"workload": f"mlp_t{T}: dense SwiGLU MLP block, T={T}, x seed 6, weights torch seed 6 "
                                     f"(4 sets rotated)", "T": T},
              "roofline": roof}
    if not a.no_cpu:
        wb = ws_[0].cpu().numpy().view(np.uint16)
        n_tok = min(T, 64)
        result["cpu_baseline"] = oracle_baseline(lambda: O.dense_mlp(x_bits[:n_tok], wb), n_tok, "tokens/s",
                                                 a.cpu_seconds, 20, f"oracle calls on {n_tok} of the {T} tokens")
    print(json.dumps(result), flush=True)


def cpu_baseline_stack(T, x_bits, budget_s):
    """The CPU oracle's stack step on a bounded sample: the first two layers
    (router, shared expert and the selected experts generated on demand by the
    host generator, generation included in the time), scaled to 47 layers."""
    import synth
    from oracle import moe_oracle as O
    n_l = 2
    resid0 = O.bf16_to_f64(x_bits)

    def run():
        layers = []
        for l in range(n_l):
            cache = {}

            def blobs(e, l=l, cache=cache):
                if e not in cache:
                    c, sc = synth.gen_codes_scales(synth.STACK_SEED, l, experts=[e])
                    cache[e] = (c[0], sc[0])
                return cache[e]
            layers.append((synth.gen_router(synth.STACK_SEED, l), blobs, synth.gen_shared(synth.STACK_SEED, l)))
        O.stack_step(resid0, layers)
    # T tokens per stack step = 47 / n_l sampled runs
    return oracle_baseline(run, T * n_l / 47, "tokens/s", budget_s, 5,
                           f"oracle runs of the first {n_l} of the 47 layers at T={T} (weights of each layer and "
                           f"its selected experts generated on the host inside the timing), scaled to 47 layers")


def step_distribution(m, step, reps):
    """Per-step times from a HIP event pair around each of `reps` steps on the
    launch stream: median, p10 and p90 in microseconds."""
    import torch
    ev = m.HipEvents(2 * reps)
    for i in range(reps):
        ev.record(2 * i)
        step(i)
        ev.record(2 * i + 1)
    torch.cuda.synchronize()
    t = np.array([ev.elapsed_ms(2 * i, 2 * i + 1) for i in range(reps)]) * 1e3
    ev.close()
    return {"reps": reps, "median_us": float(np.median(t)), "p10_us": float(np.percentile(t, 10)),
            "p90_us": float(np.percentile(t, 90))}


METRIC = "routed-MoE layer tokens/s + % HBM BW (T=1,32) / % bf16 MFMA (T=2048)"
# layers rotated through by default: enough that the weights a run touches
# exceed the 256 MB Infinity Cache (T = 1 touches 23.4 MB per layer)
DEFAULT_LAYERS = {1: 24}


def bench_layer(a, name, steps, warmup, with_cpu):
    """One MoE layer (moe_w4_forward) over the workload `name`: returns the
    result object (throughput of exactly `steps` back-to-back steps, per-step
    distribution, per-stage times and the dominant stage's roofline)."""
    import torch
    import synth
    from int4_routed_expert_amd import moe_w4 as m
    cfg = synth.CONFIGS[name]
    T = cfg["T"]
    n_layers = a.layers or DEFAULT_LAYERS.get(T, 4)
    log(f"config {name}: T={T}, {n_layers} layers on the device")
    layers = [m.generated_layer(cfg["w_seed"], l) for l in range(n_layers)]
    x_bits = synth.gen_x(cfg["x_seed"], T)
    x = torch.from_numpy(x_bits.view(np.int16)).cuda()
    bias_np = None if cfg["bias_seed"] is None else synth.skew_bias(cfg["bias_seed"])
    bias = None if bias_np is None else torch.from_numpy(bias_np).cuda()
    y = torch.empty((T, 2048), dtype=torch.int16, device="cuda")
    ws = m.workspace(T)
    n_pts = m.moe_w4_profile_points()
    names = [m.moe_w4_profile_point_name(i) for i in range(n_pts)]

    def step(i, ev=None):
        w = layers[i % n_layers]
        if ev is None:
            m.moe_w4_forward(x, w["router_w"], w["codes"], w["scales"], w["shared_w"], y, ws, router_bias=bias)
        else:
            m.moe_w4_forward_profiled(x, w["router_w"], w["codes"], w["scales"], w["shared_w"], y, ws,
                                      ev, router_bias=bias)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    # timed region: exactly `steps` steps, no events inside
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    log(f"{name}: timed {steps} steps: {ms * 1e3:.1f} us/step")
    dist = step_distribution(m, step, max(steps, 200))
    # per-stage times: the same steps again with HIP events on the launch stream
    # at every stage boundary (each record adds a gap between kernels, which is
    # why the throughput above is timed without them)
    reps = max(steps, 200)
    events = m.HipEvents(reps * n_pts)
    for i in range(reps):
        step(i, events.handles[i * n_pts:(i + 1) * n_pts])
    torch.cuda.synchronize()
    stage_ms = np.zeros(n_pts - 1)
    for i in range(reps):
        for k in range(n_pts - 1):
            stage_ms[k] += events.elapsed_ms(i * n_pts + k, i * n_pts + k + 1)
    stage_ms /= reps
    events.close()

    # routing of the benchmarked layers decides the algorithmic bytes
    touched = []
    for l in range(n_layers):
        step(l)
        torch.cuda.synchronize()
        touched.append(int(m.ws_view(ws, T, "n_active", torch.int32, 1).item()))
    n_touched = float(np.mean(touched))
    layer_bytes = n_touched * EXPERT_BYTES + ROUTER_BYTES + SHARED_BYTES + 2 * T * 2048 * 2
    flops = T * (6 * 3 * 512 * 2048 * 2 + 3 * 1024 * 2048 * 2 + 256 * 2048 * 2)
    stage = dict(zip(names[1:], stage_ms))
    dom = max(stage, key=stage.get)
    # algorithmic bytes of each stage: weights and scales it must read once, plus the
    # activations it reads and writes
    act = T * 2048 * 2
    stage_bytes = {
        "router_shared_gateup": ROUTER_BYTES + 2 * 1024 * 2048 * 2 + act + T * 256 * 4 + T * 1024 * 2,
        "topk_sort": T * 256 * 4 + act + T * 6 * 4 * 4 + 257 * 4 + 256 * 32,
        "routed_gateup": n_touched * EXPERT_GU_BYTES + T * 6 * 512 * 2,
        # the GEMV down launch reads a (fp32) and rotates it itself
        "routed_down": n_touched * EXPERT_D_BYTES + T * 6 * 512 * 4 + T * 6 * 2048 * 4,
        "shared_down_combine": 1024 * 2048 * 2 + T * 1024 * 2 + T * 6 * 2048 * 4 + act,
    }
    if FUSED_MAX_TOKENS < T <= ROUTE_SMALL_MAX_TOKENS:
        # the router, the shared gate/up and the rotated x in one launch, then
        # the routing (logits in, selections and sort records out)
        stage_bytes["router_shared_gateup"] += act
        stage_bytes["topk_sort"] = T * 256 * 4 + T * 6 * 4 * 4 + 257 * 4 + 256 * 32
    if T <= FUSED_MAX_TOKENS:
        # the first launch is the router alone; the second runs the rest of the
        # layer, the shared expert included (its time is recorded under
        # routed_gateup; the later stages are empty)
        stage_bytes["router_shared_gateup"] = ROUTER_BYTES + act + T * 256 * 4
        stage_bytes["routed_gateup"] = (n_touched * EXPERT_BYTES + SHARED_BYTES + T * 256 * 4 + act
                                        + 2 * T * 1024 * 2 + act)
    dom_bytes = stage_bytes.get(dom, 0.0)
    # from 128 tokens on the routed experts and the shared expert run as MFMA
    # contractions: their flops enter the roofline beside their bytes
    stage_flops = {
        "router_shared_gateup": T * (256 + 2 * 1024) * 2048 * 2,
        "routed_gateup": T * 6 * 2 * 512 * 2048 * 2,
        "routed_down": T * 6 * 2048 * 512 * 2,
        "shared_down_combine": T * 1024 * 2048 * 2,
    }
    result = {
        "metric": METRIC, "value": T / (ms / 1e3), "unit": "tokens/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int4 x fp16/bf16 -> fp32", "data": "synthetic (seeded SplitMix64; random-init weights)",
        "config": {"workload": f"{name}: one MoE layer, T={T}, x seed {cfg['x_seed']}, weights seed "
                               f"{cfg['w_seed']}" + (", +3.0 bias on 26 experts (seed 3)" if bias is not None else ""),
                   "T": T, "layers_rotated": n_layers, "touched_experts": n_touched},
        "step_us": dist,
    }
    result["roofline"] = roofline_entry(dom, dom_bytes, stage_flops.get(dom, 0.0) if T >= GROUPED_MIN_TOKENS else 0.0,
                                        stage[dom] * 1e3, recorded_traffic(name, dom, T))
    result["layer"] = {"algorithmic_bytes": layer_bytes, "hbm_gbs": layer_bytes / (ms * 1e-3) / 1e9,
                       "hbm_frac": layer_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                       "tflops": flops / (ms * 1e-3) / 1e12,
                       "mfma_frac": flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                       "stage_us": {k: v * 1e3 for k, v in stage.items()}}
    del layers
    torch.cuda.empty_cache()
    if with_cpu:
        log(f"{name}: timing the CPU oracle baseline")
        result["cpu_baseline"] = cpu_baseline(cfg, T, x_bits, bias_np, a.cpu_seconds)
    return result


def bench_stack(a, T, with_cpu):
    """The 47-layer stack at T tokens: one moe_w4_stack_forward call per step,
    captured once as a HIP graph (checked against the eager call) and replayed."""
    import torch
    import synth
    from int4_routed_expert_amd import moe_w4 as m
    log(f"stack: T={T}, 47 layers on the device")
    layers = [m.generated_layer(synth.STACK_SEED, l) for l in range(47)]
    arr = m.stack_layers(layers)
    x_bits = synth.gen_x(synth.STACK_SEED, T)
    x = torch.from_numpy(x_bits.view(np.int16)).cuda()
    resid0 = x.view(torch.bfloat16).float()
    resid = resid0.clone()
    ws = m.stack_workspace(T)
    # algorithmic bytes of one step: each layer's touched experts, router,
    # shared expert, and the layer's x and y (routing read from a traced run)
    trace = torch.empty((47, 2, T, 2048), dtype=torch.int16, device="cuda")
    m.moe_w4_stack_forward(resid, arr, ws, trace=trace)
    torch.cuda.synchronize()
    ref = resid.clone()
    del trace
    wsl = m.workspace(T)
    yb = torch.empty((T, 2048), dtype=torch.int16, device="cuda")
    touched = 0
    resid.copy_(resid0)
    xb = torch.empty_like(yb)
    for w in layers:
        m.moe_w4_stack_layer(resid, w["router_w"], w["codes"], w["scales"], w["shared_w"], xb, yb, wsl)
        touched += int(m.ws_view(wsl, T, "n_active", torch.int32, 1).item())
    torch.cuda.synchronize()
    if not torch.equal(resid, ref):
        print("per-layer calls differ from moe_w4_stack_forward", file=sys.stderr)
        sys.exit(1)
    stack_bytes = touched * EXPERT_BYTES + 47 * (ROUTER_BYTES + SHARED_BYTES + 2 * T * 2048 * 2)
    if a.eager:
        def step(i=0):
            m.moe_w4_stack_forward(resid, arr, ws)
    else:
        graph = torch.cuda.CUDAGraph()
        resid.copy_(resid0)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            m.moe_w4_stack_forward(resid, arr, ws)
        torch.cuda.synchronize()
        for rep in range(3):
            resid.copy_(resid0)
            graph.replay()
            torch.cuda.synchronize()
            if not torch.equal(resid, ref):
                print("graph replay differs from the eager stack step", file=sys.stderr)
                sys.exit(1)
        log("graph replays match the eager step")

        def step(i=0):
            graph.replay()
    for i in range(a.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(a.steps):
        step(i)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / a.steps
    log(f"stack T={T}: timed {a.steps} steps: {ms * 1e3:.1f} us/step")
    dist = step_distribution(m, step, max(a.steps, 200))
    gbs = stack_bytes / (ms * 1e-3) / 1e9
    result = {
        "metric": METRIC, "value": T / (ms / 1e3), "unit": "tokens/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int4 x fp16/bf16 -> fp32", "data": "synthetic (seeded SplitMix64; random-init weights)",
        "config": {"workload": f"stack_t{T}: 47-layer MoE stack (moe_w4_stack_forward), T={T}, seed 4, fp32 "
                               "residual" + (", host launches" if a.eager else ", one captured graph per step"),
                   "T": T, "layers": 47, "per_layer_us": ms * 1e3 / 47},
        "step_us": dist,
        "stack": {"algorithmic_bytes": stack_bytes, "hbm_gbs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS},
        # the whole step is the unit here: 47 layers replayed as one graph
        "roofline": {"bound": "hbm", "kernel": "stack step (47 layers, one graph)", "achieved": gbs,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS, "traffic": None,
                     "algorithmic_bytes": stack_bytes, "kernel_us": ms * 1e3},
    }
    if with_cpu:
        log("timing the CPU oracle baseline")
        result["cpu_baseline"] = cpu_baseline_stack(T, x_bits, a.cpu_seconds)
    return result


POINT_KEYS = ("value", "unit", "ms_per_step", "step_us", "config", "roofline", "layer")


def main():
    a = parse()
    if a.pmc_summary:
        pmc_summary(a.pmc_summary)
        return
    if a.traffic_lines:
        traffic_lines(*a.traffic_lines)
        return
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {a.gpus} is not supported (the layer needs no "
              "collective: a multi-GPU deployment replicates it per GPU).", file=sys.stderr)
        sys.exit(2)
    if a.copy_calibration:
        copy_calibration()
        return
    if a.config == "pack_layer":
        bench_pack(a)
        return
    if a.config.startswith("mlp_t"):
        bench_mlp(a, int(a.config[5:]))
        return
    if a.config.startswith("nvfp4_t"):
        bench_nvfp4(a, int(a.config[7:]))
        return
    import torch
    torch.cuda.set_device(0)
    if a.config.startswith("stack"):
        print(json.dumps(bench_stack(a, 1 if a.config == "stack_t1" else 8, not a.no_cpu)), flush=True)
        return
    result = bench_layer(a, a.config, a.steps, a.warmup, not a.no_cpu)
    if a.config == "decode_t32" and not a.headline_only:
        # the metric's other points (T = 1 and T = 2048, uniform and skewed
        # routing), each timed the same way, under "points"
        result["points"] = {}
        for name in ("decode_t1", "prefill_t2048", "prefill_t2048_skew"):
            r = bench_layer(a, name, a.steps, a.warmup, False)
            result["points"][name] = {k: r[k] for k in POINT_KEYS}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
