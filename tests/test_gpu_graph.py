"""The whole decode step as one HIP graph (Betelgeuse article, section "mechanism", scheduling
row: a decode step is a single graph replay): 48 layers of 8 tokens captured once, replayed with
eager work and new inputs in between; every replay bitwise equal to the eager step on the same
inputs, and sampled layers against the oracle."""

import numpy as np
import pytest
import torch

from layer_fixtures import MODEL, Layer, near_tie_tokens
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu

Y_TOL = 2e-3
CFG = 13


@pytest.fixture(scope="module")
def N():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mixture_experts_route_amd import native

    return native


def test_48_layer_decode_step_as_one_graph(N):
    from mixture_experts_route_amd import synth as S

    dev = torch.device("cuda:0")
    n_layers, T = 48, 8
    H, E, k = MODEL["H"], MODEL["E"], MODEL["k"]
    # one arena of 512 routed + 1 shared experts under every layer; each layer its own router and
    # Zipf(1.1) bias, so each layer routes differently
    base = Layer(dict(MODEL, cfg=CFG), dev, seed=0, layer=0)
    d = base.dims()
    r_codes = [S.bf16_normal_np(S.stream_key(0, CFG, "router", l, 0), (E, H), 0.02) for l in range(n_layers)]
    routers = [torch.from_numpy(c.view(np.int16)).to(dev) for c in r_codes]
    bias_np = [S.zipf_bias(S.rank_permutation(0, CFG, l, 0, E), S.ZIPF_C) for l in range(n_layers)]
    biases = [torch.from_numpy(b).to(dev) for b in bias_np]
    wts = [N.layer_weights(routers[l], base.arena, base.stride, base.n_slots, base.shared, biases[l])
           for l in range(n_layers)]
    xb = [torch.zeros((T, H), dtype=torch.int16, device=dev) for _ in range(n_layers)]
    yb = [torch.zeros((T, H), dtype=torch.float32, device=dev) for _ in range(n_layers)]
    ib = [torch.zeros((T, k), dtype=torch.int32, device=dev) for _ in range(n_layers)]
    ws = torch.zeros(N.moe_workspace_bytes(d, T) // 4 + 64, dtype=torch.int32, device=dev)
    N.moe_workspace_init(ws)

    def x_codes(layer, step):
        return S.bf16_normal_np(S.stream_key(0, CFG, "x", layer, step), (T, H), 1.0)

    def fill(step):
        for l in range(n_layers):
            xb[l].copy_(torch.from_numpy(x_codes(l, step).view(np.int16)))

    def run_step(stream):
        for l in range(n_layers):
            N.moe_layer_forward(d, wts[l], None, xb[l], T, yb[l], ws, topk_ids=ib[l], stream=stream)

    eager = {}
    for step in (0, 1):
        fill(step)
        run_step(torch.cuda.current_stream())
        torch.cuda.synchronize()
        assert N.moe_check_device_error(ws) == 0
        eager[step] = ([y.clone() for y in yb], [i.clone() for i in ib])
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    fill(0)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=side):
        run_step(torch.cuda.current_stream())
    torch.cuda.synchronize()
    x_other = torch.from_numpy(x_codes(5, 77).view(np.int16)).to(dev)
    y_other = torch.zeros((T, H), dtype=torch.float32, device=dev)
    for rep, step in enumerate((0, 1, 1, 0)):
        # eager work between replays: new inputs, and a layer call of its own on the same workspace
        fill(step)
        for y in yb:
            y.fill_(float("nan"))
        N.moe_layer_forward(d, wts[5], None, x_other, T, y_other, ws)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert N.moe_check_device_error(ws) == 0
        ys, ids = eager[step]
        for l in range(n_layers):
            assert torch.equal(ib[l], ids[l]), (rep, l)
            assert torch.equal(yb[l], ys[l]), (rep, l)
    # the replayed step against the oracle on sampled layers
    for l in (0, 23, 47):
        x64 = S.bf16_to_f32(x_codes(l, 0)).astype(np.float64)
        ref = O.moe_layer(x64, S.bf16_to_f32(r_codes[l]).astype(np.float64), bias_np[l], k, base.blob_np,
                          base.shared_np(), H, MODEL["F"])
        ok = ~near_tie_tokens(ref["logits64"], k)
        ys, ids = eager[0]
        assert np.array_equal(ids[l].cpu().numpy()[ok], ref["ids"][ok]), l
        err = O.per_token_rel_err(ys[l].cpu().numpy(), ref["y"])
        assert np.all(err[ok] <= Y_TOL), (l, err)
