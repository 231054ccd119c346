"""HIP layer vs the CPU oracle, through the C ABI, on seeded synthetic inputs.

Sizes: small and ragged T that the oracle finishes in seconds (tiles and tails
of every kernel), the four single-layer workloads at full size (T = 1, 32,
2048 uniform, 2048 skewed) with every output row compared, T = 3000 (the sort
past its register-resident size) on every row and the largest T the library
takes (65,536) with full routing and sampled rows; edge cases (one expert
taking every token, all-tie router, the 2^-14 floor, large and tiny
magnitudes, T = 0, the two-launch form's failure path forced from the host),
and invariants (determinism, batch invariance, token permutation, expert
relabelling, a poisoned workspace, the device generators against the host
ones).
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
def layer0(m):
    w = m.generated_layer(0, 0)
    torch.cuda.synchronize()
    return w


def oracle_layer(x_bits, bias=None, tokens=None, seed=0, layer=0, scale_log2=0, router=None, norm="floor",
                 bias_mode="logit"):
    R = P.host_router(seed, layer) if router is None else router
    return O.moe_layer(x_bits, R, P.host_blobs(seed, layer, scale_log2), P.host_shared(seed, layer),
                       bias=bias, tokens=tokens, norm=norm, bias_mode=bias_mode, pool=P.pool())


def report(label, s):
    print(f"[parity] {label}: T={s['T']} flagged={s['flagged']} rerouted={s['rerouted']} "
          f"reordered={s['reordered']} max_err/rms={s['ratio']:.2e} beyond-half-ulp/rms={s['elem']:.2e}", flush=True)


# ------------------------------------------------------------------ generator
def test_device_generator_matches_host(m, layer0):
    rng = np.random.default_rng(0)
    R = P.from_dev_u16(layer0["router_w"]).reshape(256, 2048)
    np.testing.assert_array_equal(R, P.host_router(0, 0))
    S = P.from_dev_u16(layer0["shared_w"])
    np.testing.assert_array_equal(S, P.host_shared(0, 0))
    codes = layer0["codes"]
    scales = layer0["scales"]
    for e in [0, 1, 77, 200, 255]:
        hc, hs = P._host_expert(0, 0, e)
        np.testing.assert_array_equal(codes[e].cpu().numpy(), hc, err_msg=f"codes of expert {e}")
        np.testing.assert_array_equal(scales[e].cpu().numpy().view(np.uint16), hs, err_msg=f"scales of expert {e}")
    # x of another seed/layer, and a second layer's tensors at sampled indices
    for seed, layer, T in [(1, 0, 32), (4, 3, 5)]:
        x = torch.empty((T, 2048), dtype=torch.int16, device="cuda")
        m.moe_w4_generate_x(seed, layer, x)
        np.testing.assert_array_equal(P.from_dev_u16(x), synth.gen_x(seed, T, layer))
    w = m.empty_layer()
    m.moe_w4_generate_layer(4, 46, w["router_w"], w["codes"], w["scales"], w["shared_w"])
    e = int(rng.integers(0, 256))
    hc, hs = synth.gen_codes_scales(4, 46, experts=[e])
    np.testing.assert_array_equal(w["codes"][e].cpu().numpy(), hc[0])
    np.testing.assert_array_equal(w["scales"][e].cpu().numpy().view(np.uint16), hs[0])
    np.testing.assert_array_equal(P.from_dev_u16(w["router_w"]).reshape(256, 2048), synth.gen_router(4, 46))


# ---------------------------------------------------------------- small / ragged
@pytest.mark.parametrize("T", [1, 2, 3, 4, 5, 6, 7, 8, 9, 16, 31, 33, 48, 49, 63, 65])
def test_layer_small_T(m, layer0, T):
    x = synth.gen_x(100 + T, T)
    g = P.run_gpu(m, x, layer0)
    ref = oracle_layer(x)
    report(f"small T={T}", P.compare(g, ref, label=f"T={T}"))


# ------------------------------------------------- MFMA grouped path (T >= 128)
# chunks of the grouped kernels (include/moe_w4.h): chunks of CHUNK_ROWS; from
# CHUNK_MAX_ROWS_MIN_T tokens on an expert with at most CHUNK_MAX_ROWS sorted
# rows is one chunk
CHUNK_ROWS = 64
CHUNK_MAX_ROWS = 96
CHUNK_MAX_ROWS_MIN_T = 1536


def expected_chunks(offsets, T):
    counts = np.diff(offsets)
    long_ok = T >= CHUNK_MAX_ROWS_MIN_T
    step = lambda n: CHUNK_MAX_ROWS if long_ok and n <= CHUNK_MAX_ROWS else CHUNK_ROWS
    return np.array([(e, offsets[e] + r, min(step(counts[e]), counts[e] - r), 0)
                     for e in np.nonzero(counts)[0]
                     for r in range(0, counts[e], step(counts[e]))]).reshape(-1, 4)


def read_chunks(m, ws, T):
    n = int(m.ws_view(ws, T, "n_chunks", torch.int32, 1).item())
    return m.ws_view(ws, T, "chunks", torch.int32, 4 * n).cpu().numpy().reshape(n, 4)


def test_grouped_path_all_tokens(m, layer0):
    """T = 128: every token against the oracle (chunks of a few rows per expert)."""
    T = 128
    x = synth.gen_x(400, T)
    ws = m.workspace(T)
    g = P.run_gpu(m, x, layer0, ws=ws)
    np.testing.assert_array_equal(read_chunks(m, ws, T), expected_chunks(g["offsets"], T))
    report("grouped T=128", P.compare(g, oracle_layer(x), label="grouped T=128"))


@pytest.mark.parametrize("T", [129, 257, 333, 2047])
def test_grouped_path_all_rows(m, layer0, T):
    print(f"[parity] case grouped T={T}", flush=True)
    x = synth.gen_x(401 + T, T)
    g = P.run_gpu(m, x, layer0)
    report(f"grouped T={T}", P.compare(g, oracle_layer(x), label=f"grouped T={T}"))


def test_grouped_chunks_of_a_hot_expert(m, layer0):
    """One expert takes all 200 tokens: chunks of 64, 64, 64 and a ragged 8."""
    T = 200
    x = synth.gen_x(402, T)
    bias = np.zeros(256, dtype=np.float32)
    bias[17] = 100.0
    ws = m.workspace(T)
    g = P.run_gpu(m, x, layer0, bias=bias, ws=ws)
    assert np.all(g["topk_idx"][:, 0] == 17)
    ch = read_chunks(m, ws, T)
    np.testing.assert_array_equal(ch, expected_chunks(g["offsets"], T))
    assert (ch[:, 0] == 17).sum() == 4 and ch[ch[:, 0] == 17][-1, 2] == 8
    tokens = np.array([0, 1, 31, 32, 63, 64, 95, 96, 127, 128, 191, 192, 199])
    report("grouped hot expert", P.compare(g, oracle_layer(x, bias=bias, tokens=tokens), tokens=tokens,
                                           label="grouped hot expert"))


def test_grouped_chunk_of_96_rows(m, layer0):
    """From 1536 tokens on an expert with at most 96 rows is one chunk: 96
    tokens steered to expert 23 (x along its router row; a -100 bias keeps
    every other token off it) make a 96-row chunk, three MFMA row tiles in
    gate/up and two passes of 64 and 32 rows in down; every row compared."""
    T, e = 1600, 23
    print(f"[parity] case T={T} expert {e} with 96 rows", flush=True)
    x = synth.gen_x(404, T).copy()
    r = O.bf16_to_f64(synth.gen_router(0, 0)[e])
    x[:96] = synth.f32_to_bf16_bits((500.0 * r).astype(np.float32))[None, :]
    bias = np.zeros(256, dtype=np.float32)
    bias[e] = -100.0
    ws = m.workspace(T)
    g = P.run_gpu(m, x, layer0, bias=bias, ws=ws)
    assert np.diff(g["offsets"])[e] == 96
    ch = read_chunks(m, ws, T)
    np.testing.assert_array_equal(ch, expected_chunks(g["offsets"], T))
    assert ch[ch[:, 0] == e].tolist() == [[e, int(g["offsets"][e]), 96, 0]]
    # the steered rows are ~50 times larger than the others (x of norm ~460):
    # each population is compared against its own rms
    for label, tokens in (("steered", np.arange(96)), ("other", np.arange(96, T))):
        s = P.compare(g, oracle_layer(x, bias=bias, tokens=tokens), tokens=tokens,
                      label=f"grouped 96-row chunk, {label} rows")
        report(f"grouped 96-row chunk, {label} rows", s)


def test_grouped_batch_invariance(m, layer0):
    """Rows do not interact on the grouped path: the first 128 tokens of a
    256-token batch give the bits of the 128-token batch."""
    x = synth.gen_x(403, 256)
    a = P.run_gpu(m, x[:128], layer0)
    b = P.run_gpu(m, x, layer0)
    np.testing.assert_array_equal(a["y_bits"], b["y_bits"][:128])


# ------------------------------------------------------------- the workloads
@pytest.mark.parametrize("name", ["decode_t1", "decode_t32"])
def test_decode_workloads(m, layer0, name):
    cfg = synth.CONFIGS[name]
    x = synth.gen_x(cfg["x_seed"], cfg["T"])
    g = P.run_gpu(m, x, layer0)
    ref = oracle_layer(x)
    report(name, P.compare(g, ref, label=name))


@pytest.mark.parametrize("name", ["prefill_t2048", "prefill_t2048_skew"])
def test_prefill_workloads_all_rows(m, layer0, name):
    cfg = synth.CONFIGS[name]
    T = cfg["T"]
    print(f"[parity] case {name}", flush=True)
    x = synth.gen_x(cfg["x_seed"], T)
    bias = None if cfg["bias_seed"] is None else synth.skew_bias(cfg["bias_seed"])
    g = P.run_gpu(m, x, layer0, bias=bias)
    ref = oracle_layer(x, bias=bias)
    s = P.compare(g, ref, label=name)
    report(name, s)
    if bias is not None:
        hot = synth.skew_experts(cfg["bias_seed"])
        share = np.isin(g["topk_idx"], hot).mean()
        print(f"[parity] {name}: share of assignments on the 26 biased experts = {share:.4f}", flush=True)
        assert share > 0.5


# ----------------------------------------------------------------- edge cases
@pytest.mark.parametrize("T", [8, 40])
def test_one_expert_takes_every_token(m, layer0, T):
    x = synth.gen_x(200, T)
    bias = np.zeros(256, dtype=np.float32)
    bias[17] = 100.0
    g = P.run_gpu(m, x, layer0, bias=bias)
    assert np.all(g["topk_idx"][:, 0] == 17)
    assert g["offsets"][18] - g["offsets"][17] == T
    report("one hot expert", P.compare(g, oracle_layer(x, bias=bias), label="one hot expert"))


@pytest.mark.parametrize("T", [8, 9])
def test_all_tie_router(m, layer0, T):
    x = synth.gen_x(201, T)
    w = dict(layer0)
    w["router_w"] = torch.zeros_like(layer0["router_w"])
    g = P.run_gpu(m, x, w)
    assert np.all(g["topk_idx"] == np.arange(6))
    np.testing.assert_allclose(g["topk_w"], 1 / 6, rtol=1e-6)
    ref = oracle_layer(x, router=np.zeros((256, 2048), dtype=np.uint16))
    report("all-tie router", P.compare(g, ref, label="all-tie router"))


# ------------------------------------------------------------ router policies
POLICIES = [("floor", "select"), ("sum", "logit"), ("sum", "select"), ("none", "logit"), ("none", "select")]


def policy_flags(m, norm, bias_mode):
    f = {"floor": m.ROUTER_NORM_FLOOR, "sum": m.ROUTER_NORM_SUM, "none": m.ROUTER_NORM_NONE}[norm]
    return f | (m.ROUTER_BIAS_SELECT_ONLY if bias_mode == "select" else 0)


@pytest.mark.parametrize("T", [3, 32, 128])
@pytest.mark.parametrize("norm,bias_mode", POLICIES)
def test_router_policies(m, layer0, T, norm, bias_mode):
    """Every router policy on each launch sequence (two launches, GEMVs, MFMA
    tiles), with a bias that favours some experts and disfavours others."""
    x = synth.gen_x(300 + T, T)
    rng = np.random.default_rng(T)
    bias = rng.normal(0.0, 1.0, 256).astype(np.float32)
    g = P.run_gpu(m, x, layer0, bias=bias, policy=policy_flags(m, norm, bias_mode))
    ref = oracle_layer(x, bias=bias, norm=norm, bias_mode=bias_mode)
    report(f"policy {norm}/{bias_mode} T={T}", P.compare(g, ref, label=f"policy {norm}/{bias_mode} T={T}"))
    if norm == "none":
        # no renormalisation: the weights are the sigmoid scores themselves
        lw = ref["logits_w"][np.arange(T)[:, None], g["topk_idx"]]
        np.testing.assert_allclose(g["topk_w"], 1.0 / (1.0 + np.exp(-lw)), rtol=1e-5)


def test_router_policy_sum_without_floor(m, layer0):
    """Below the floor the legacy selected-sum still renormalises to 1."""
    T = 5
    x = synth.gen_x(202, T)
    bias = np.full(256, -30.0, dtype=np.float32)
    g = P.run_gpu(m, x, layer0, bias=bias, policy=m.ROUTER_NORM_SUM)
    ref = oracle_layer(x, bias=bias, norm="sum")
    np.testing.assert_allclose(g["topk_w"].sum(axis=1), 1.0, rtol=1e-5)
    report("legacy sum below the floor", P.compare(g, ref, label="legacy sum below the floor"))


def test_weight_floor(m, layer0):
    T = 5
    x = synth.gen_x(202, T)
    bias = np.full(256, -30.0, dtype=np.float32)
    g = P.run_gpu(m, x, layer0, bias=bias)
    ref = oracle_layer(x, bias=bias)
    assert np.all(ref["topk_w"].sum(axis=1) < 1e-6)
    report("weight floor", P.compare(g, ref, label="weight floor"))


@pytest.mark.parametrize("x_log2,s_log2", [(12, 10), (-20, 0), (0, -12)])
def test_magnitudes(m, layer0, x_log2, s_log2):
    """Power-of-two scalings (exact in bf16) of x and of the routed scales."""
    T = 6
    xf = O.bf16_to_f64(synth.gen_x(203, T)) * 2.0 ** x_log2
    x = O.f64_to_bf16_bits(xf)
    w = dict(layer0)
    if s_log2:
        sc = layer0["scales"].view(torch.bfloat16).float() * 2.0 ** s_log2
        w["scales"] = sc.to(torch.bfloat16).view(torch.int16)
    g = P.run_gpu(m, x, w)
    ref = oracle_layer(x, scale_log2=s_log2)
    report(f"magnitude x*2^{x_log2} s*2^{s_log2}", P.compare(g, ref, label="magnitudes"))


@pytest.mark.parametrize("x_log2,s_log2", [(12, 10), (-20, 0), (0, -12)])
def test_magnitudes_grouped_path(m, layer0, x_log2, s_log2):
    """The same scalings through the MFMA path (its expert rows cross HBM as
    fp16 with a per-row multiplier), on sampled tokens."""
    T = 160
    print(f"[parity] case grouped magnitudes x*2^{x_log2} s*2^{s_log2}", flush=True)
    xf = O.bf16_to_f64(synth.gen_x(204, T)) * 2.0 ** x_log2
    x = O.f64_to_bf16_bits(xf)
    w = dict(layer0)
    if s_log2:
        sc = layer0["scales"].view(torch.bfloat16).float() * 2.0 ** s_log2
        w["scales"] = sc.to(torch.bfloat16).view(torch.int16)
    g = P.run_gpu(m, x, w)
    tokens = np.array([0, 1, 57, 100, T - 1])
    ref = oracle_layer(x, scale_log2=s_log2, tokens=tokens)
    report(f"grouped magnitude x*2^{x_log2} s*2^{s_log2}",
           P.compare(g, ref, tokens=tokens, label="grouped magnitudes"))


def test_grouped_path_uneven_down_scales(m, layer0):
    """Down rows of one expert whose scales differ by 2^24 (every odd feature's
    scales times 2^-24): the fp16 expert rows are normalised to the expert's
    largest scales, so the small features lose relative precision but not the
    bar (their outputs are 2^24 smaller)."""
    T = 160
    print("[parity] case uneven down scales", flush=True)
    sc = layer0["scales"].view(torch.bfloat16).float().reshape(256, -1).clone()
    down = sc[:, 16384:].reshape(256, 2048, 4)
    down[:, 1::2, :] *= 2.0 ** -24
    sc[:, 16384:] = down.reshape(256, -1)
    w = dict(layer0, scales=sc.to(torch.bfloat16).view(torch.int16).reshape(-1))
    base = P.host_blobs(0, 0)

    def blobs(e):
        c, s = base(e)
        f = O.bf16_to_f64(s)
        d = f[16384:].reshape(2048, 4)
        d[1::2] *= 2.0 ** -24
        f[16384:] = d.ravel()
        return c, O.f64_to_bf16_bits(f)
    x = synth.gen_x(205, T)
    g = P.run_gpu(m, x, w)
    tokens = np.array([0, 3, 80, T - 1])
    ref = O.moe_layer(x, P.host_router(0, 0), blobs, P.host_shared(0, 0), tokens=tokens)
    report("uneven down scales", P.compare(g, ref, tokens=tokens, label="uneven down scales"))


def test_zero_tokens_is_a_noop(m, layer0):
    ws = m.workspace(1)
    x = torch.empty((0, 2048), dtype=torch.int16, device="cuda")
    y = torch.full((1, 2048), 7, dtype=torch.int16, device="cuda")
    m.moe_w4_forward(x, layer0["router_w"], layer0["codes"], layer0["scales"], layer0["shared_w"], y, ws, T=0)
    torch.cuda.synchronize()
    assert torch.all(y == 7)


# ----------------------------------------------------------------- invariants
@pytest.mark.parametrize("T", [8, 48])
def test_determinism_and_poisoned_workspace(m, layer0, T):
    x = synth.gen_x(300, T)
    a = P.run_gpu(m, x, layer0)
    b = P.run_gpu(m, x, layer0, poison=True)
    np.testing.assert_array_equal(a["y_bits"], b["y_bits"])
    np.testing.assert_array_equal(a["perm"], b["perm"])


@pytest.mark.parametrize("T_full,parts", [(8, [(5, 6), (0, 3), (2, 8)]), (16, [(0, 9), (7, 16)])])
def test_batch_invariance(m, layer0, T_full, parts):
    """A token's output bits do not depend on the other tokens of the call, for
    calls that take the same launch sequence (1-8 tokens: one launch after the
    router; 9-127: the GEMV launches); across sequences the summation order
    differs and only the oracle tolerance holds."""
    x = synth.gen_x(301, T_full)
    full = P.run_gpu(m, x, layer0)
    for a, b in parts:
        part = P.run_gpu(m, x[a:b], layer0)
        np.testing.assert_array_equal(part["y_bits"], full["y_bits"][a:b])


def test_token_permutation_equivariance(m, layer0):
    x = synth.gen_x(302, 24)
    perm = np.random.default_rng(3).permutation(24)
    a = P.run_gpu(m, x, layer0)
    b = P.run_gpu(m, x[perm], layer0)
    np.testing.assert_array_equal(a["y_bits"][perm], b["y_bits"])
    np.testing.assert_array_equal(a["topk_idx"][perm], b["topk_idx"])


# ------------------------------------------------------------- large T
def test_sort_past_its_register_resident_size(m, layer0):
    """T = 3000: 18,000 assignments, more than the sort keeps in registers
    (16,384), so it streams its keys twice; every row compared."""
    T = 3000
    print(f"[parity] case T={T}", flush=True)
    x = synth.gen_x(410, T)
    ws = m.workspace(T)
    g = P.run_gpu(m, x, layer0, ws=ws)
    np.testing.assert_array_equal(read_chunks(m, ws, T), expected_chunks(g["offsets"], T))
    report(f"T={T}", P.compare(g, oracle_layer(x), label=f"T={T}"))


def gen_x_chunked(seed, T, chunk=8192):
    """synth.gen_x in pieces (the same bits; bounded host temporaries)."""
    out = np.empty((T, 2048), dtype=np.uint16)
    for t0 in range(0, T, chunk):
        idx = np.arange(t0 * 2048, min(T, t0 + chunk) * 2048, dtype=np.uint64)
        out[t0:t0 + chunk] = synth.normal_bf16_bits(seed, synth.tensor_id(0, synth.KIND_X), idx,
                                                    synth.SIGMA_X).reshape(-1, 2048)
    return out


def test_largest_token_count(m, layer0):
    """T = MAX_TOKENS (65,536): routing, offsets, perm and the chunk list of all
    393,216 assignments bit-exact; y on sampled rows (the first and last
    tokens, the rows of the first and last chunks of the busiest expert, and
    random ones)."""
    T = m.MAX_TOKENS
    print(f"[parity] case T={T}", flush=True)
    x = gen_x_chunked(411, T)
    ws = m.workspace(T)
    g = P.run_gpu(m, x, layer0, ws=ws)
    np.testing.assert_array_equal(read_chunks(m, ws, T), expected_chunks(g["offsets"], T))
    counts = np.diff(g["offsets"])
    busiest = int(np.argmax(counts))
    rows = g["perm"][[g["offsets"][busiest], g["offsets"][busiest + 1] - 1]] // 6
    rng = np.random.default_rng(11)
    tokens = np.unique(np.concatenate([[0, 1, T - 1], rows, rng.choice(T, 19, replace=False)]))
    report(f"T={T} sampled", P.compare(g, oracle_layer(x, tokens=tokens), tokens=tokens, label=f"T={T}"))


# ------------------------------------------------------- expert relabelling
@pytest.mark.parametrize("T", [5, 32, 160])
def test_expert_relabel_invariance(m, layer0, T):
    """Renumbering the experts (router rows, codes and scales together) changes
    the chosen indices by the same permutation and leaves y bit for bit (each
    assignment's arithmetic does not depend on its expert's number)."""
    pi = np.random.default_rng(500 + T).permutation(256)   # new expert k is old expert pi[k]
    ip = torch.from_numpy(pi).cuda()
    w2 = dict(layer0, router_w=layer0["router_w"][ip].contiguous(), codes=layer0["codes"][ip].contiguous(),
              scales=layer0["scales"][ip].contiguous())
    x = synth.gen_x(501, T)
    a = P.run_gpu(m, x, layer0)
    b = P.run_gpu(m, x, w2)
    np.testing.assert_array_equal(pi[b["topk_idx"]], a["topk_idx"])
    np.testing.assert_array_equal(b["topk_w"], a["topk_w"])
    np.testing.assert_array_equal(b["y_bits"], a["y_bits"])


# ------------------------------------------------------------ failure path
@pytest.mark.parametrize("T", [3, 32])
def test_fused_wait_failure_path(m, layer0, T):
    """The bounded hand-off waits, made to give up from the host (a count the
    producing workgroups never reach, a 200 us bound): at T = 3 the down
    workgroups of the two-launch form, at T = 32 workgroup 0 of the routing
    launch.  Every kernel exits normally, y and the residual stream come out
    NaN and the error word is set; with the defaults back, the same calls are
    correct again."""
    print(f"[failure path] T={T}", flush=True)
    x = synth.gen_x(210, T)
    ws = m.workspace(T)
    w = layer0
    resid0 = torch.from_numpy(O.bf16_to_f64(x).astype(np.float32)).cuda()
    xb = torch.empty((T, 2048), dtype=torch.int16, device="cuda")
    yb = torch.empty_like(xb)
    err = lambda: int(m.ws_view(ws, T, "error", torch.int32, 1).item())
    try:
        m.moe_w4_set_fused_wait(20000, 1)
        g = P.run_gpu(m, x, w, ws=ws)
        assert err() == 1
        assert np.all(np.isnan(O.bf16_to_f64(g["y_bits"])))
        resid = resid0.clone()
        m.moe_w4_stack_layer(resid, w["router_w"], w["codes"], w["scales"], w["shared_w"], xb, yb, ws)
        torch.cuda.synchronize()
        assert err() == 1 and bool(torch.isnan(resid).all())
        sws = m.stack_workspace(T)
        resid = resid0.clone()
        m.moe_w4_stack_forward(resid, [w, w], sws)
        torch.cuda.synchronize()
        assert int(m.ws_view(sws, T, "error", torch.int32, 1).item()) == 1 and bool(torch.isnan(resid).all())
    finally:
        m.moe_w4_set_fused_wait(0, 0)
    g = P.run_gpu(m, x, w, ws=ws)
    assert err() == 0
    report("after the failure path", P.compare(g, oracle_layer(x), label="after the failure path"))
    resid = resid0.clone()
    m.moe_w4_stack_layer(resid, w["router_w"], w["codes"], w["scales"], w["shared_w"], xb, yb, ws)
    torch.cuda.synchronize()
    assert err() == 0 and bool(torch.isfinite(resid).all())


# ------------------------------------------------------------ generators
@pytest.mark.parametrize("seed,tid,n,sigma", [(0, 1, 256 * 2048, 0.02), (4, 64 * 46 + 10, 2048 * 1024, 0.02),
                                              (1, 0, 32 * 2048, 1.0), (7, 1234567, 1000003, 0.5),
                                              (2 ** 64 - 1, 2 ** 32 - 1, 4097, 3.0)])
def test_generate_normal_bf16_matches_host(m, seed, tid, n, sigma):
    out = torch.full((n + 2,), 0x5555, dtype=torch.int16, device="cuda")
    m.moe_w4_generate_normal_bf16(seed, tid, out[1:], sigma, n=n)    # a 2-byte aligned start
    got = P.from_dev_u16(out)
    want = synth.normal_bf16_bits(seed, tid, np.arange(n, dtype=np.uint64), sigma)
    np.testing.assert_array_equal(got[1:n + 1], want)
    assert got[0] == 0x5555 and got[n + 1] == 0x5555
