"""The C ABI on the CPU: the library loads, exports every declared symbol, and
rejects bad arguments with the documented status before any HIP call."""
import ctypes
import os
import re
import subprocess

import pytest

from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "moe_w4.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_w4_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def m():
    from int4_routed_expert_amd import moe_w4
    return moe_w4


def test_every_declared_symbol_is_exported(m):
    names = declared_functions()
    assert len(names) >= 10
    out = subprocess.run(["nm", "-D", "--defined-only", m.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (moe_w4_\w+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    lib = ctypes.CDLL(m.LIB_PATH)
    for n in names:
        assert hasattr(lib, n)
    assert set(m.EXPORTED) == set(names)


def test_header_constants_match_the_binding(m):
    defines = dict(re.findall(r"#define MOE_W4_(\w+) \(?(-?\d+)\)?", open(HEADER).read()))
    names = ["HIDDEN", "EXPERTS", "TOPK", "INTER", "SHARED_INTER", "GROUP", "CODE_BYTES_PER_EXPERT",
             "SCALES_PER_EXPERT", "SHARED_ELEMS", "MAX_TOKENS", "FUSED_MAX_TOKENS", "ROUTER_NORM_FLOOR",
             "ROUTER_NORM_SUM", "ROUTER_NORM_NONE", "ROUTER_NORM_MASK", "ROUTER_BIAS_SELECT_ONLY", "EXPERT_WEIGHTS",
             "PACK_MAX_EXPERTS", "DENSE_INTER", "DENSE_WEIGHTS", "NVFP4_CODE_BYTES", "NVFP4_SCALE_BYTES"]
    for n in names:
        assert int(defines[n]) == getattr(m, n), n


def test_workspace_layout(m):
    assert m.moe_w4_workspace_bytes(-1) == 0
    assert m.moe_w4_workspace_bytes(m.MAX_TOKENS + 1) == 0
    for T in (0, 1, 7, 32, 2048):
        lay = m.moe_w4_workspace_layout(T)
        assert lay["total"] == m.moe_w4_workspace_bytes(T)
        offs = sorted((v, k) for k, v in lay.items() if k != "total")
        for (a, _), (b, _) in zip(offs, offs[1:]):
            assert a <= b
        assert all(v % 256 == 0 for v in lay.values())
        # regions are large enough for what the header says they hold
        assert lay["topk_w"] - lay["topk_idx"] >= 4 * 6 * T
        assert lay["perm"] - lay["offsets"] >= 4 * 257
    with pytest.raises(m.MoeW4Error):
        m.moe_w4_workspace_layout(-5)


class FakeBuf:
    """Stands in for a device tensor: only an address and a size are used."""

    def __init__(self, addr, nbytes=1 << 40):
        self.addr, self.nbytes = addr, nbytes

    def data_ptr(self):
        return self.addr

    def numel(self):
        return self.nbytes

    def element_size(self):
        return 1


class FakeX(FakeBuf):
    def __init__(self, addr, T):
        super().__init__(addr)
        self.shape = (T, 2048)


def call(m, T, x=0x10000000, r=0x20000000, c=0x30000000, s=0x40000000, sh=0x50000000, y=0x60000000,
         bias=None, ws=0x70000000, ws_bytes=None):
    lib = m._lib
    if ws_bytes is None:
        ws_bytes = m.moe_w4_workspace_bytes(max(T, 0)) if 0 <= T <= m.MAX_TOKENS else 1 << 30
    return lib.moe_w4_forward(x, r, c, s, sh, T, y, bias, ws, ws_bytes, None)


def test_validation_codes_without_device(m):
    assert call(m, 0) == m.OK                         # T == 0: nothing enqueued
    assert call(m, -1) == m.EINVAL
    assert call(m, m.MAX_TOKENS + 1) == m.EINVAL
    for k in ("x", "r", "c", "s", "sh", "y", "ws"):
        assert call(m, 4, **{k: None}) == m.EINVAL, k
        assert call(m, 4, **{k: 0x10000008 + 0x1000000}) == m.EINVAL, k    # misaligned
    assert call(m, 4, bias=0x80000002) == m.EINVAL
    assert call(m, 4, ws_bytes=m.moe_w4_workspace_bytes(4) - 1) == m.EWORKSPACE
    assert call(m, 4, y=0x10000000 + 4096) == m.EINVAL                       # y overlaps x
    assert call(m, 4, y=0x70000000 + 256) == m.EINVAL                        # y overlaps the workspace
    assert m.moe_w4_last_device_error() == 0


def test_profiled_and_stack_validation(m):
    lib = m._lib
    ev = (ctypes.c_void_p * 1)()
    assert lib.moe_w4_forward_profiled(0x1000, 0x2000, 0x3000, 0x4000, 0x5000, 4, 0x6000, None, 0x7000, 1 << 30, None, ev, -1) == m.EINVAL
    assert lib.moe_w4_forward_profiled(0x1000, 0x2000, 0x3000, 0x4000, 0x5000, 4, 0x6000, None, 0x7000, 1 << 30, None, None, 2) == m.EINVAL
    assert lib.moe_w4_forward_profiled(None, 0x2000, 0x3000, 0x4000, 0x5000, 4, 0x6000, None, 0x7000, 1 << 30, None, ev, 1) == m.EINVAL
    assert lib.moe_w4_stack_layer(None, 0x2000, 0x3000, 0x4000, 0x5000, 4, 0x6000, 0x7000, 0x8000, 1 << 30, None) == m.EINVAL
    assert lib.moe_w4_stack_layer(0x100000, 0x2000, 0x3000, 0x4000, 0x5000, 0, 0x6000, 0x7000, 0x8000, 0, None) == m.OK
    # residual overlapping the x buffer
    assert lib.moe_w4_stack_layer(0x6000, 0x2000, 0x3000, 0x4000, 0x5000, 4, 0x6000, 0x7000000, 0x8000000, 1 << 30, None) == m.EINVAL
    assert lib.moe_w4_generate_x(0, 0, -1, 0x1000, None) == m.EINVAL
    assert lib.moe_w4_generate_x(0, 0, 4, 0x1001, None) == m.EINVAL
    assert lib.moe_w4_generate_layer(0, -1, None, None, None, None, None) == m.EINVAL
    assert lib.moe_w4_generate_layer(0, 0, 0x1002, None, None, None, None) == m.EINVAL


def test_router_policy_validation(m):
    lib = m._lib
    args = (0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000)
    ws_bytes = m.moe_w4_workspace_bytes(4)
    for bad in (3, 7, 8, -1, 1 << 20):
        assert lib.moe_w4_forward_policy(*args, 4, 0x60000000, None, bad, 0x70000000, ws_bytes, None) == m.EINVAL
    for ok in (0, 1, 2, 4, 5, 6):
        # valid policies get as far as the usual checks: T == 0 returns OK
        assert lib.moe_w4_forward_policy(*args, 0, 0x60000000, None, ok, 0x70000000, ws_bytes, None) == m.OK
        assert lib.moe_w4_forward_policy(None, *args[1:], 4, 0x60000000, None, ok, 0x70000000, ws_bytes,
                                         None) == m.EINVAL


def test_pack_validation(m):
    lib = m._lib
    n = 2
    wb = n * m.EXPERT_WEIGHTS * 2
    w, c, s = 0x10000000, 0x10000000 + wb, 0x10000000 + wb + n * m.CODE_BYTES_PER_EXPERT
    assert lib.moe_w4_pack_experts(w, 0, None, None, None) == m.OK               # nothing to do
    assert lib.moe_w4_pack_experts(w, -1, c, s, None) == m.EINVAL
    assert lib.moe_w4_pack_experts(w, m.PACK_MAX_EXPERTS + 1, c, s, None) == m.EINVAL
    assert lib.moe_w4_pack_experts(None, n, c, s, None) == m.EINVAL
    assert lib.moe_w4_pack_experts(w, n, None, s, None) == m.EINVAL
    assert lib.moe_w4_pack_experts(w + 8, n, c, s, None) == m.EINVAL            # misaligned
    assert lib.moe_w4_pack_experts(w, n, w + 4096, s, None) == m.EINVAL         # codes overlap the weights
    assert lib.moe_w4_pack_experts(w, n, c, c + 16, None) == m.EINVAL           # scales overlap the codes
    assert m.moe_w4_last_device_error() == 0


def test_dense_mlp_validation(m):
    lib = m._lib
    x, w, y, ws = 0x10000000, 0x20000000, 0x60000000, 0x70000000
    nb = m.moe_w4_dense_mlp_workspace_bytes(4)
    assert nb >= 4 * m.DENSE_INTER * 2
    assert m.moe_w4_dense_mlp_workspace_bytes(-1) == 0
    assert lib.moe_w4_dense_mlp(x, w, 0, y, ws, 0, None) == m.OK
    assert lib.moe_w4_dense_mlp(x, w, -1, y, ws, nb, None) == m.EINVAL
    assert lib.moe_w4_dense_mlp(None, w, 4, y, ws, nb, None) == m.EINVAL
    assert lib.moe_w4_dense_mlp(x, w + 2, 4, y, ws, nb, None) == m.EINVAL
    assert lib.moe_w4_dense_mlp(x, w, 4, y, ws, nb - 1, None) == m.EWORKSPACE
    assert lib.moe_w4_dense_mlp(x, w, 4, x + 4096, ws, nb, None) == m.EINVAL       # y overlaps x
    assert lib.moe_w4_dense_mlp(x, w, 4, w + 4096, ws, nb, None) == m.EINVAL       # y overlaps the weights
    assert m.moe_w4_last_device_error() == 0


def test_nvfp4_validation(m):
    lib = m._lib
    x, r, c, sc, ts, sh, y, ws = (0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x48000000, 0x50000000,
                                  0x60000000, 0x70000000)
    nb = m.moe_w4_workspace_bytes(4)
    assert lib.moe_w4_forward_nvfp4(x, r, c, sc, ts, sh, 0, y, None, ws, nb, None) == m.OK    # T == 0
    assert lib.moe_w4_forward_nvfp4(x, r, c, sc, ts, sh, -1, y, None, ws, nb, None) == m.EINVAL
    assert lib.moe_w4_forward_nvfp4(x, r, c, sc, None, sh, 4, y, None, ws, nb, None) == m.EINVAL
    assert lib.moe_w4_forward_nvfp4(x, r, c, sc, ts + 2, sh, 4, y, None, ws, nb, None) == m.EINVAL
    assert lib.moe_w4_forward_nvfp4(x, r, None, sc, ts, sh, 4, y, None, ws, nb, None) == m.EINVAL
    assert lib.moe_w4_forward_nvfp4(x, r, c, sc + 8, ts, sh, 4, y, None, ws, nb, None) == m.EINVAL
    assert lib.moe_w4_forward_nvfp4(x, r, c, sc, ts, sh, 4, y, None, ws, nb - 1, None) == m.EWORKSPACE
    assert lib.moe_w4_forward_nvfp4(x, r, c, sc, ts, sh, 4, x + 4096, None, ws, nb, None) == m.EINVAL
    ev = (ctypes.c_void_p * 1)()
    assert lib.moe_w4_forward_nvfp4_profiled(x, r, c, sc, ts, sh, 4, y, None, ws, nb, None, ev, -1) == m.EINVAL
    assert lib.moe_w4_forward_nvfp4_profiled(x, r, c, sc, ts, sh, 4, y, None, ws, nb, None, None, 1) == m.EINVAL
    assert m.moe_w4_last_device_error() == 0


def test_status_strings(m):
    for st in (m.OK, m.EINVAL, m.EWORKSPACE, m.EDEVICE):
        assert m.status_string(st)
    assert m.status_string(42) == "unknown status"
    assert m.moe_w4_profile_points() == len([m.moe_w4_profile_point_name(i) for i in range(m.moe_w4_profile_points())])
    assert m.moe_w4_profile_point_name(0) == "start"
    assert m.moe_w4_profile_point_name(99) is None


def layer_array(m, n, base=0x10000000, bad=None):
    arr = (m.Layer * n)()
    for i in range(n):
        arr[i] = m.Layer(base + 0x100000 * i, base + 0x100000 * i + 0x10000, base + 0x100000 * i + 0x20000,
                         base + 0x100000 * i + 0x30000)
    if bad is not None:
        i, field, value = bad
        setattr(arr[i], field, value)
    return arr


def test_stack_forward_validation(m):
    lib = m._lib
    T = 8
    resid, trace, ws = 0x40000000, 0x50000000, 0x60000000
    nb = m.moe_w4_stack_workspace_bytes(T)
    # a forward workspace plus one layer's bf16 x and y
    assert nb >= m.moe_w4_workspace_bytes(T) + 2 * T * 2048 * 2
    assert m.moe_w4_stack_workspace_bytes(-1) == 0
    assert m.moe_w4_stack_workspace_bytes(m.MAX_TOKENS + 1) == 0
    arr = layer_array(m, 3)
    f = lib.moe_w4_stack_forward
    assert f(resid, arr, 0, T, None, ws, nb, None) == m.OK                # no layers: nothing enqueued
    assert f(resid, arr, 3, 0, None, ws, nb, None) == m.OK                # no tokens
    assert f(resid, arr, -1, T, None, ws, nb, None) == m.EINVAL
    assert f(resid, arr, m.STACK_MAX_LAYERS + 1, T, None, ws, nb, None) == m.EINVAL
    assert f(resid, arr, 3, -1, None, ws, nb, None) == m.EINVAL
    assert f(resid, arr, 3, m.MAX_TOKENS + 1, None, ws, nb, None) == m.EINVAL
    assert f(None, arr, 3, T, None, ws, nb, None) == m.EINVAL
    assert f(resid, None, 3, T, None, ws, nb, None) == m.EINVAL
    assert f(resid, arr, 3, T, None, None, nb, None) == m.EINVAL
    assert f(resid + 4, arr, 3, T, None, ws, nb, None) == m.EINVAL        # misaligned
    assert f(resid, arr, 3, T, trace + 8, ws, nb, None) == m.EINVAL
    for field in ("router_w", "codes", "scales", "shared_w"):
        assert f(resid, layer_array(m, 3, bad=(2, field, None)), 3, T, None, ws, nb, None) == m.EINVAL, field
        assert f(resid, layer_array(m, 3, bad=(1, field, 0x7000008)), 3, T, None, ws, nb, None) == m.EINVAL, field
    assert f(resid, arr, 3, T, None, ws, nb - 1, None) == m.EWORKSPACE
    assert f(ws + 256, arr, 3, T, None, ws, nb, None) == m.EINVAL         # resid inside the workspace
    assert f(resid, arr, 3, T, resid + 4096, ws, nb, None) == m.EINVAL     # trace overlaps resid
    assert f(resid, arr, 3, T, ws - 4096, ws, nb, None) == m.EINVAL        # trace runs into the workspace
    assert m.moe_w4_last_device_error() == 0


def test_generate_normal_validation(m):
    lib = m._lib
    g = lib.moe_w4_generate_normal_bf16
    assert g(0, 1, 0, 1.0, None, None) == m.OK                            # n == 0: nothing enqueued
    assert g(0, 1, -1, 1.0, 0x1000, None) == m.EINVAL
    assert g(0, 1, m.GENERATE_MAX_ELEMS + 1, 1.0, 0x1000, None) == m.EINVAL
    assert g(0, 1, 16, -0.5, 0x1000, None) == m.EINVAL
    assert g(0, 1, 16, float("nan"), 0x1000, None) == m.EINVAL
    assert g(0, 1, 16, float("inf"), 0x1000, None) == m.EINVAL
    assert g(0, 1, 16, 1.0, None, None) == m.EINVAL
    assert g(0, 1, 16, 1.0, 0x1001, None) == m.EINVAL                     # bf16 needs 2-byte alignment
    assert m.moe_w4_last_device_error() == 0


def test_fused_wait_setting(m):
    lib = m._lib
    assert lib.moe_w4_set_fused_wait(-1, 0) == m.EINVAL
    assert lib.moe_w4_set_fused_wait(1 << 32, 0) == m.EINVAL
    assert lib.moe_w4_set_fused_wait(1000, -1) == m.EINVAL
    assert lib.moe_w4_set_fused_wait(1000, 1) == m.OK
    assert lib.moe_w4_set_fused_wait(0, 0) == m.OK                        # back to the defaults


def test_workspace_error_word(m):
    for T in (1, 8, 9, 128):
        lay = m.moe_w4_workspace_layout(T)
        assert lay["sync"] + 4096 <= lay["error"] and lay["error"] + 4 <= lay["total"]
