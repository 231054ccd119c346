"""moe_w4_forward_static (the forward on the library's own per-GPU device
array, for callers that cannot allocate) against moe_w4_forward.

Both run the same kernels on the same inputs, so y must agree bit for bit;
three calls in a row, each with fewer tokens than the one before (the largest
T the array takes, a GEMV-path size, a two-launch size), show that the array
keeps nothing from one call that the next one reads.  A T beyond the limit is
refused with MOE_W4_EWORKSPACE and no launch.
"""
import numpy as np
import pytest
import torch

import synth
from tests import parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    from int4_routed_expert_amd import moe_w4
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return moe_w4


def test_static_forward_matches_forward(m):
    w = m.generated_layer(0, 0)
    bias = torch.from_numpy(synth.skew_bias(3, value=0.5)).cuda()
    for T in (m.STATIC_MAX_TOKENS, 37, 5):
        print(f"[no-alloc] case T={T}", flush=True)
        x = P.to_dev_u16(synth.gen_x(600 + T, T))
        y_ref = torch.empty((T, 2048), dtype=torch.int16, device="cuda")
        ws = m.workspace(T)
        m.moe_w4_forward(x, w["router_w"], w["codes"], w["scales"], w["shared_w"], y_ref, ws, router_bias=bias)
        y = torch.full((T, 2048), 0x7FC0, dtype=torch.int16, device="cuda")
        st = m._lib.moe_w4_forward_static(x.data_ptr(), w["router_w"].data_ptr(), w["codes"].data_ptr(),
                                          w["scales"].data_ptr(), w["shared_w"].data_ptr(), T, y.data_ptr(),
                                          bias.data_ptr(), torch.cuda.current_stream().cuda_stream)
        assert st == m.OK
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), f"T={T}: static forward differs from moe_w4_forward"
        assert np.all(np.isfinite(synth.bf16_bits_to_f32(P.from_dev_u16(y))))


def test_static_forward_limit(m):
    w = m.generated_layer(0, 0)
    T = m.STATIC_MAX_TOKENS + 1
    x = torch.zeros((T, 2048), dtype=torch.int16, device="cuda")
    y = torch.full((T, 2048), 7, dtype=torch.int16, device="cuda")
    st = m._lib.moe_w4_forward_static(x.data_ptr(), w["router_w"].data_ptr(), w["codes"].data_ptr(),
                                      w["scales"].data_ptr(), w["shared_w"].data_ptr(), T, y.data_ptr(), None,
                                      torch.cuda.current_stream().cuda_stream)
    assert st == m.EWORKSPACE
    assert m._lib.moe_w4_forward_static(x.data_ptr(), None, None, None, None, 0, y.data_ptr(), None, None) == m.OK
    torch.cuda.synchronize()
    assert bool((y == 7).all())
