"""Python binding of libmoe_w4 (the int4 routed-expert MoE layer for MI355X).

Argument marshalling only: every step of the layer runs in the HIP kernels of
libmoe_w4.so.  PyTorch supplies device memory and the stream.  The functions
carry the C names; the contracts are in include/moe_w4.h.  If the library is
not built, importing this package raises ImportError — there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch  # loads the HIP runtime that the library then shares

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_w4.so")

HIDDEN = 2048
EXPERTS = 256
TOPK = 6
INTER = 512
SHARED_INTER = 1024
GROUP = 128
CODE_BYTES_PER_EXPERT = 1572864
SCALES_PER_EXPERT = 24576
SHARED_ELEMS = 6291456
MAX_TOKENS = 65536
FUSED_MAX_TOKENS = 8
STACK_MAX_LAYERS = 1024
STATIC_MAX_TOKENS = 128
GENERATE_MAX_ELEMS = 1 << 40
# router policy flags of moe_w4_forward_policy (include/moe_w4.h)
ROUTER_NORM_FLOOR, ROUTER_NORM_SUM, ROUTER_NORM_NONE, ROUTER_NORM_MASK = 0, 1, 2, 3
ROUTER_BIAS_SELECT_ONLY = 4
EXPERT_WEIGHTS = 3145728       # bf16 elements of one expert's gate, up and down rows
PACK_MAX_EXPERTS = 65536
DENSE_INTER = 6144
DENSE_WEIGHTS = 37748736       # bf16 elements of a dense MLP block: gate, up [6144][2048], down [2048][6144]
NVFP4_CODE_BYTES = 1572864     # bytes of one NVFP4 expert's E2M1 codes
NVFP4_SCALE_BYTES = 196608     # E4M3 block-scale bytes of one NVFP4 expert

OK, EINVAL, EWORKSPACE, EDEVICE = 0, -1, -2, -3


class MoeW4Error(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


class WsLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in (
        "logits", "topk_idx", "topk_w", "offsets", "perm", "pos", "n_active", "active",
        "xt", "xt_scale", "act", "at", "at_scale", "hs", "o", "z", "chunks", "n_chunks", "sync", "error", "hist", "total")]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


class Layer(ctypes.Structure):
    """moe_w4_layer: the device pointers of one layer's weights."""
    _fields_ = [(n, ctypes.c_void_p) for n in ("router_w", "codes", "scales", "shared_w")]


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python -m int4_routed_expert_amd.build`")
_lib = ctypes.CDLL(LIB_PATH)

_vp, _sz, _i64, _int, _u64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int64, ctypes.c_int, ctypes.c_uint64
_sig = {
    "moe_w4_workspace_bytes": (_sz, [_i64]),
    "moe_w4_workspace_layout": (_int, [_i64, ctypes.POINTER(WsLayout)]),
    "moe_w4_forward": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp, _sz, _vp]),
    "moe_w4_forward_policy": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _int, _vp, _sz, _vp]),
    "moe_w4_forward_static": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp]),
    "moe_w4_profile_points": (_int, []),
    "moe_w4_profile_point_name": (ctypes.c_char_p, [_int]),
    "moe_w4_forward_profiled": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp, _sz, _vp,
                                       ctypes.POINTER(_vp), _int]),
    "moe_w4_forward_nvfp4": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp, _sz, _vp]),
    "moe_w4_forward_nvfp4_profiled": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp, _sz, _vp,
                                             ctypes.POINTER(_vp), _int]),
    "moe_w4_pack_experts": (_int, [_vp, _i64, _vp, _vp, _vp]),
    "moe_w4_dense_mlp_workspace_bytes": (_sz, [_i64]),
    "moe_w4_dense_mlp": (_int, [_vp, _vp, _i64, _vp, _vp, _sz, _vp]),
    "moe_w4_generate_layer": (_int, [_u64, _int, _vp, _vp, _vp, _vp, _vp]),
    "moe_w4_generate_x": (_int, [_u64, _int, _i64, _vp, _vp]),
    "moe_w4_stack_layer": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp, _sz, _vp]),
    "moe_w4_stack_workspace_bytes": (_sz, [_i64]),
    "moe_w4_stack_forward": (_int, [_vp, ctypes.POINTER(Layer), _int, _i64, _vp, _vp, _sz, _vp]),
    "moe_w4_generate_normal_bf16": (_int, [_u64, ctypes.c_uint32, _i64, ctypes.c_double, _vp, _vp]),
    "moe_w4_set_fused_wait": (_int, [_i64, _int]),
    "moe_w4_status_string": (ctypes.c_char_p, [_int]),
    "moe_w4_last_device_error": (_int, []),
    "moe_w4_version": (_int, []),
}
for _name, (_res, _args) in _sig.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args

EXPORTED = tuple(_sig)


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status, what):
    if status != OK:
        raise MoeW4Error(status, what)


def status_string(status: int) -> str:
    return _lib.moe_w4_status_string(status).decode()


moe_w4_status_string = status_string


def moe_w4_version() -> int:
    return _lib.moe_w4_version()


def moe_w4_last_device_error() -> int:
    return _lib.moe_w4_last_device_error()


def moe_w4_workspace_bytes(T: int) -> int:
    return _lib.moe_w4_workspace_bytes(T)


def moe_w4_workspace_layout(T: int) -> dict:
    lay = WsLayout()
    _check(_lib.moe_w4_workspace_layout(T, ctypes.byref(lay)), "moe_w4_workspace_layout")
    return lay.as_dict()


def moe_w4_forward(x, router_w, codes, scales, shared_w, y, workspace, router_bias=None, stream=None,
                   T=None) -> int:
    """y <- layer(x).  Tensors on the GPU; returns the status (raises on error)."""
    T = x.shape[0] if T is None else T
    st = _lib.moe_w4_forward(_ptr(x), _ptr(router_w), _ptr(codes), _ptr(scales), _ptr(shared_w), T,
                             _ptr(y), _ptr(router_bias), _ptr(workspace),
                             workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "moe_w4_forward")
    return st


def moe_w4_forward_static(x, router_w, codes, scales, shared_w, y, router_bias=None, stream=None, T=None) -> int:
    """moe_w4_forward on the library's own per-GPU device array (no workspace, no allocation)."""
    T = x.shape[0] if T is None else T
    st = _lib.moe_w4_forward_static(_ptr(x), _ptr(router_w), _ptr(codes), _ptr(scales), _ptr(shared_w), T,
                                    _ptr(y), _ptr(router_bias), _stream(stream))
    _check(st, "moe_w4_forward_static")
    return st


def moe_w4_forward_policy(x, router_w, codes, scales, shared_w, y, workspace, router_bias=None,
                          router_policy=ROUTER_NORM_FLOOR, stream=None, T=None) -> int:
    """moe_w4_forward with a router policy (ROUTER_* flags)."""
    T = x.shape[0] if T is None else T
    st = _lib.moe_w4_forward_policy(_ptr(x), _ptr(router_w), _ptr(codes), _ptr(scales), _ptr(shared_w), T,
                                    _ptr(y), _ptr(router_bias), int(router_policy), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "moe_w4_forward_policy")
    return st


def moe_w4_profile_points() -> int:
    return _lib.moe_w4_profile_points()


def moe_w4_profile_point_name(i: int):
    r = _lib.moe_w4_profile_point_name(i)
    return None if r is None else r.decode()


def moe_w4_forward_profiled(x, router_w, codes, scales, shared_w, y, workspace, events,
                            router_bias=None, stream=None) -> int:
    """moe_w4_forward recording raw hipEvent_t handles (ints) at the stage boundaries."""
    arr = (_vp * len(events))(*events)
    st = _lib.moe_w4_forward_profiled(_ptr(x), _ptr(router_w), _ptr(codes), _ptr(scales), _ptr(shared_w),
                                      x.shape[0], _ptr(y), _ptr(router_bias), _ptr(workspace),
                                      workspace.numel() * workspace.element_size(), _stream(stream),
                                      arr, len(events))
    _check(st, "moe_w4_forward_profiled")
    return st


def moe_w4_forward_nvfp4(x, router_w, codes, scales, tensor_scales, shared_w, y, workspace, router_bias=None,
                         stream=None, T=None) -> int:
    """y <- layer(x) with NVFP4 experts (codes u8, E4M3 scales u8, f32 tensor scales [256][3])."""
    T = x.shape[0] if T is None else T
    st = _lib.moe_w4_forward_nvfp4(_ptr(x), _ptr(router_w), _ptr(codes), _ptr(scales), _ptr(tensor_scales),
                                   _ptr(shared_w), T, _ptr(y), _ptr(router_bias), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "moe_w4_forward_nvfp4")
    return st


def moe_w4_forward_nvfp4_profiled(x, router_w, codes, scales, tensor_scales, shared_w, y, workspace, events,
                                  router_bias=None, stream=None) -> int:
    """moe_w4_forward_nvfp4 recording raw hipEvent_t handles at the stage boundaries."""
    arr = (_vp * len(events))(*events)
    st = _lib.moe_w4_forward_nvfp4_profiled(_ptr(x), _ptr(router_w), _ptr(codes), _ptr(scales),
                                            _ptr(tensor_scales), _ptr(shared_w), x.shape[0], _ptr(y),
                                            _ptr(router_bias), _ptr(workspace),
                                            workspace.numel() * workspace.element_size(), _stream(stream),
                                            arr, len(events))
    _check(st, "moe_w4_forward_nvfp4_profiled")
    return st


def moe_w4_generate_layer(seed, layer, router_w=None, codes=None, scales=None, shared_w=None, stream=None):
    _check(_lib.moe_w4_generate_layer(seed, layer, _ptr(router_w), _ptr(codes), _ptr(scales), _ptr(shared_w),
                                      _stream(stream)), "moe_w4_generate_layer")


def moe_w4_pack_experts(w, codes, scales, n_experts=None, stream=None):
    """bf16 expert weights (n_experts x EXPERT_WEIGHTS) -> int4 codes and bf16 scales."""
    n = w.numel() // EXPERT_WEIGHTS if n_experts is None else n_experts
    _check(_lib.moe_w4_pack_experts(_ptr(w), n, _ptr(codes), _ptr(scales), _stream(stream)), "moe_w4_pack_experts")


def moe_w4_dense_mlp_workspace_bytes(T: int) -> int:
    return _lib.moe_w4_dense_mlp_workspace_bytes(T)


def moe_w4_dense_mlp(x, w, y, workspace, stream=None, T=None):
    """y <- dense SwiGLU MLP block (width 6144) of x.  Tensors on the GPU."""
    T = x.shape[0] if T is None else T
    _check(_lib.moe_w4_dense_mlp(_ptr(x), _ptr(w), T, _ptr(y), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(stream)), "moe_w4_dense_mlp")


def moe_w4_generate_x(seed, layer, x, stream=None):
    _check(_lib.moe_w4_generate_x(seed, layer, x.shape[0], _ptr(x), _stream(stream)), "moe_w4_generate_x")


def moe_w4_stack_layer(resid, router_w, codes, scales, shared_w, x_buf, y_buf, workspace, stream=None):
    _check(_lib.moe_w4_stack_layer(_ptr(resid), _ptr(router_w), _ptr(codes), _ptr(scales), _ptr(shared_w),
                                   resid.shape[0], _ptr(x_buf), _ptr(y_buf), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), _stream(stream)),
           "moe_w4_stack_layer")


def moe_w4_stack_workspace_bytes(T: int) -> int:
    return _lib.moe_w4_stack_workspace_bytes(T)


def stack_layers(layers):
    """A ctypes array of moe_w4_layer from dicts of device tensors (router_w, codes, scales, shared_w)."""
    arr = (Layer * len(layers))()
    for i, w in enumerate(layers):
        arr[i] = Layer(_ptr(w["router_w"]), _ptr(w["codes"]), _ptr(w["scales"]), _ptr(w["shared_w"]))
    return arr


def moe_w4_stack_forward(resid, layers, workspace, trace=None, stream=None):
    """resid <- the stack of `layers` applied to resid (fp32 [T][2048]).  layers: a
    stack_layers() array (or a list of weight dicts); trace: None or bf16 device
    memory [n_layers][2][T][2048] that receives every layer's input and output."""
    arr = layers if isinstance(layers, ctypes.Array) else stack_layers(layers)
    _check(_lib.moe_w4_stack_forward(_ptr(resid), arr, len(arr), resid.shape[0], _ptr(trace), _ptr(workspace),
                                     workspace.numel() * workspace.element_size(), _stream(stream)),
           "moe_w4_stack_forward")


def moe_w4_generate_normal_bf16(seed, tensor_id, out, sigma, n=None, stream=None):
    """out[:n] <- seeded bf16 "normals" of standard deviation sigma (the scheme of the layer's inputs)."""
    n = out.numel() if n is None else n
    _check(_lib.moe_w4_generate_normal_bf16(seed, tensor_id, n, float(sigma), _ptr(out), _stream(stream)),
           "moe_w4_generate_normal_bf16")


def moe_w4_set_fused_wait(max_ticks: int = 0, extra_count: int = 0):
    """Diagnostic: bound (ticks of the 100 MHz clock; 0 = default 5 ms) and extra count of the
    two-launch form's wait; extra_count > 0 makes every such wait give up (tests of the failure path)."""
    _check(_lib.moe_w4_set_fused_wait(max_ticks, extra_count), "moe_w4_set_fused_wait")


# ---------------------------------------------------------------- allocation helpers
def empty_layer(device="cuda"):
    """Uninitialised device tensors of one layer in the library layout (as raw integer dtypes)."""
    return dict(
        router_w=torch.empty((EXPERTS, HIDDEN), dtype=torch.int16, device=device),
        codes=torch.empty((EXPERTS, CODE_BYTES_PER_EXPERT), dtype=torch.uint8, device=device),
        scales=torch.empty((EXPERTS, SCALES_PER_EXPERT), dtype=torch.int16, device=device),
        shared_w=torch.empty((SHARED_ELEMS,), dtype=torch.int16, device=device),
    )


def generated_layer(seed, layer=0, device="cuda"):
    w = empty_layer(device)
    moe_w4_generate_layer(seed, layer, w["router_w"], w["codes"], w["scales"], w["shared_w"])
    return w


def workspace(T, device="cuda"):
    return torch.empty((max(moe_w4_workspace_bytes(T), 1),), dtype=torch.uint8, device=device)


def stack_workspace(T, device="cuda"):
    return torch.empty((max(moe_w4_stack_workspace_bytes(T), 1),), dtype=torch.uint8, device=device)


def ws_view(ws, T, name, dtype, count):
    """A typed view of one workspace region (for reading routing results)."""
    off = moe_w4_workspace_layout(T)[name]
    nbytes = count * torch.empty((), dtype=dtype).element_size()
    return ws[off:off + nbytes].view(dtype)


class HipEvents:
    """Raw hipEvent_t handles from the HIP runtime torch loaded, for timing only.

    Created with hipEventDisableSystemFence: a timing event then needs no
    system-scope cache writeback and invalidation when it is recorded, which
    otherwise adds microseconds between the kernels it brackets."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, n):
        self._hip = ctypes.CDLL("libamdhip64.so.7")
        self._hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(_vp), ctypes.c_uint]
        self._hip.hipEventRecord.argtypes = [_vp, _vp]
        self._hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), _vp, _vp]
        self._hip.hipEventDestroy.argtypes = [_vp]
        self.handles = []
        for _ in range(n):
            h = _vp()
            if self._hip.hipEventCreateWithFlags(ctypes.byref(h), self.DISABLE_SYSTEM_FENCE) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            self.handles.append(h.value)

    def record(self, i, stream=None):
        if self._hip.hipEventRecord(self.handles[i], _stream(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, i, j):
        ms = ctypes.c_float()
        if self._hip.hipEventElapsedTime(ctypes.byref(ms), self.handles[i], self.handles[j]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def close(self):
        for h in self.handles:
            self._hip.hipEventDestroy(h)
        self.handles = []
