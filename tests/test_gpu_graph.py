"""A captured HIP graph of the layer replays to the bits of the eager call.

The forward enqueues only kernels (no memset or copy), so it can be captured
on a stream and replayed.  Each replay is checked against the eager result,
with eager work and synchronisation between replays.
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


@pytest.mark.parametrize("T", [5, 40, 200])
def test_graph_replay_matches_eager(m, T):
    w = m.generated_layer(0, 0)
    x = P.to_dev_u16(synth.gen_x(500 + T, T))
    ws = m.workspace(T)
    y_eager = torch.empty((T, 2048), dtype=torch.int16, device="cuda")
    m.moe_w4_forward(x, w["router_w"], w["codes"], w["scales"], w["shared_w"], y_eager, ws)
    torch.cuda.synchronize()
    y = torch.zeros_like(y_eager)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        m.moe_w4_forward(x, w["router_w"], w["codes"], w["scales"], w["shared_w"], y, ws)
    for rep in range(4):
        y.zero_()
        ws.fill_(0xA5)                      # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager), f"replay {rep} differs"


@pytest.mark.parametrize("T", [1, 9])
def test_stack_graph_replay_matches_eager(m, T):
    """moe_w4_stack_forward (3 layers) captured once and replayed: every replay
    reproduces the eager residual bit for bit."""
    layers = [m.generated_layer(4, l) for l in range(3)]
    x0 = torch.empty((T, 2048), dtype=torch.int16, device="cuda")
    m.moe_w4_generate_x(4, 0, x0)
    resid0 = x0.view(torch.bfloat16).float().contiguous()
    ws = m.stack_workspace(T)
    arr = m.stack_layers(layers)
    resid = resid0.clone()
    m.moe_w4_stack_forward(resid, arr, ws)
    torch.cuda.synchronize()
    eager = resid.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        m.moe_w4_stack_forward(resid, arr, ws)
    for rep in range(4):
        resid.copy_(resid0)
        ws.fill_(0x5A)                      # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(resid, eager), f"replay {rep} differs"
