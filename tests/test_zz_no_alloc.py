"""The whole layer on the library's static per-GPU workspace (moe_layer_forward_static) against the
same call with a caller workspace (moe_layer_forward): same kernels, so bitwise the same outputs and
routing, on two calls in a row (the second smaller), and the device error word reported through
the caller's int32 and cleared."""

import ctypes

import numpy as np
import pytest
import torch

from layer_fixtures import MODEL, Layer


@pytest.fixture(scope="module")
def N():
    from mixture_experts_route_amd import native

    return native


def test_static_refuses_oversized_calls_on_host(N):
    """Beyond the static array (a 4096-token prefill's workspace) the call is MOE_EWORKSPACE and
    enqueues nothing (the pointers here are never dereferenced)."""
    d = N.dims(2048, 768, 512, 10, 1)
    assert N.moe_workspace_bytes(d, 4096) > N.MOE_STATIC_SCRATCH_BYTES
    fake = 1 << 20
    w = N.moe_layer_weights(fake, 1, None, fake, 2_654_208, 512, 1 << 24)
    f = N.raw("moe_layer_forward_static")
    assert f(ctypes.byref(d), ctypes.byref(w), None, None, fake, 1, 4096, fake, None, None, fake, None) == \
        N.MOE_EWORKSPACE
    assert f(ctypes.byref(d), ctypes.byref(w), None, None, fake, 1, 1, fake, None, None, None, None) == N.MOE_EINVAL


@pytest.mark.gpu
def test_static_workspace_matches_caller_workspace(N):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dev = torch.device("cuda:0")
    layer = Layer(MODEL, dev, seed=0, layer=3)
    d = layer.dims()
    wts = layer.native_weights()
    err = torch.full((1,), -1, dtype=torch.int32, device=dev)
    for call, T in enumerate((8, 3)):
        x, _ = layer.x(T, 500 + call, dev)
        ws = torch.zeros(N.moe_workspace_bytes(d, T) // 4 + 64, dtype=torch.int32, device=dev)
        N.moe_workspace_init(ws)
        ya = torch.full((T, layer.H), float("nan"), dtype=torch.float32, device=dev)
        yb = torch.full_like(ya, float("nan"))
        ia = torch.full((T, layer.k), -1, dtype=torch.int32, device=dev)
        ib = torch.full_like(ia, -1)
        wa = torch.zeros((T, layer.k), dtype=torch.float32, device=dev)
        wb = torch.zeros_like(wa)
        N.moe_layer_forward(d, wts, None, x, T, ya, ws, topk_ids=ia, topk_w=wa)
        err.fill_(-1)
        N.moe_layer_forward_static(d, wts, None, x, T, yb, err, topk_ids=ib, topk_w=wb)
        torch.cuda.synchronize()
        assert N.moe_check_device_error(ws) == 0
        assert int(err.item()) == 0, (call, T)
        assert torch.equal(ia, ib) and torch.equal(wa, wb), (call, T)
        assert torch.equal(ya, yb), (call, T, (ya - yb).abs().max().item())
    # a device error reaches the caller's word, and is cleared for the next call
    T = 1
    x, _ = layer.x(T, 600, dev)
    table = torch.full((layer.E,), -1, dtype=torch.int32, device=dev)
    y = torch.zeros((T, layer.H), dtype=torch.float32, device=dev)
    N.moe_layer_forward_static(d, wts, table, x, T, y, err)
    torch.cuda.synchronize()
    assert int(err.item()) & N.DERR_NOT_RESIDENT
    N.moe_layer_forward_static(d, wts, None, x, T, y, err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
