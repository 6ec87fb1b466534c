"""GPU parity of the codebook and affine weight formats (halogen README, "Bring your own GGUF":
the IQ4_NL family as a small set of values times a block scale, the K-quants as exact affine
planes) against the oracle: dequantized weights bit-exact (in fp32), layer outputs within the
per-token 2e-3 bound through the decode kernels (1 to 16 tokens) and the prefill kernels, and a
token's decode output bitwise the same alone and in a batch."""

import numpy as np
import pytest
import torch

from layer_fixtures import MODEL, TINY, Layer, near_tie_tokens
from mixture_experts_route_amd import synth as S
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu

Y_TOL = 2e-3
FORMATS = [S.FMT_CB4, S.FMT_AFFINE4]


@pytest.fixture(scope="module")
def N():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mixture_experts_route_amd import native

    return native


@pytest.fixture(scope="module")
def dev():
    return torch.device("cuda:0")


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("shape", [(256, 128), (2048, 768)])
def test_debug_dequant_formats_bit_exact(N, dev, fmt, shape):
    """Every weight of the three matrices equals the oracle's exact value rounded to fp32 (the
    codebook format's products are exact in fp32; the affine u * s - m is rounded once)."""
    H, F = shape
    cb = S.synthetic_codebook()
    d = N.dims(H, F, 8, 2, 1, format=fmt, codebook=cb)
    blob_np = S.expert_blob_np(S.stream_key(7, 0, "blob", 0, fmt), H, F, fmt=fmt)
    assert len(blob_np) == N.moe_expert_blob_bytes(d)
    blob = torch.from_numpy(blob_np).to(dev)
    for m, ref in enumerate(O.expert_weights(blob_np, H, F, fmt, cb)):
        out = torch.full(ref.shape, float("nan"), dtype=torch.float32, device=dev)
        N.moe_debug_dequant(d, blob, m, out)
        got = out.cpu().numpy()
        want = ref.astype(np.float32)
        assert np.array_equal(got, want), f"matrix {m}: {np.sum(got != want)} mismatches"


def _check(N, dev, layer, T, step, via_layer=True):
    d = layer.dims()
    x, x64 = layer.x(T, step, dev)
    ws = torch.zeros(N.moe_workspace_bytes(d, T) // 4 + 64, dtype=torch.int32, device=dev)
    N.moe_workspace_init(ws)
    y = torch.full((T, layer.H), float("nan"), dtype=torch.float32, device=dev)
    ids = torch.zeros((T, layer.k), dtype=torch.int32, device=dev)
    w = torch.zeros((T, layer.k), dtype=torch.float32, device=dev)
    if via_layer:
        N.moe_layer_forward(d, layer.native_weights(), None, x, T, y, ws, topk_ids=ids, topk_w=w)
    else:
        N.moe_route(d, x, T, layer.router, layer.bias, ids, w, None, ws)
        if T <= N.MOE_DECODE_MAX_TOKENS:
            N.moe_expert_ffn_decode(d, layer.native_weights(), None, x, T, ids, w, y, ws)
        y2 = torch.full_like(y, float("nan"))
        N.moe_expert_ffn_prefill(d, layer.native_weights(), None, x, T, ids, w, y2, ws)
    torch.cuda.synchronize()
    assert N.moe_check_device_error(ws) == 0
    ref = layer.oracle(x64)
    ok = ~near_tie_tokens(ref["logits64"], layer.k)
    assert np.array_equal(ids.cpu().numpy()[ok], ref["ids"][ok])
    outs = [y] if via_layer else ([y, y2] if T <= N.MOE_DECODE_MAX_TOKENS else [y2])
    for o in outs:
        err = O.per_token_rel_err(o.cpu().numpy(), ref["y"])
        assert np.all(err[ok] <= Y_TOL), (T, err.max())
    return y


@pytest.mark.parametrize("fmt", FORMATS)
def test_tiny_layer_formats(N, dev, fmt):
    """The tiny shape: fp32 tokens through the decode kernels, bf16 tokens through both paths."""
    layer = Layer(dict(TINY, fmt=fmt), dev, seed=0)
    _check(N, dev, layer, 4, step=1)
    layer_b = Layer(dict(TINY, fmt=fmt, x_f32=False, r_f32=False, cfg=11), dev, seed=0)
    _check(N, dev, layer_b, 12, step=2, via_layer=False)
    _check(N, dev, layer_b, 40, step=3)


@pytest.fixture(scope="module", params=FORMATS)
def model_layer(request, N, dev):
    layer = Layer(dict(MODEL, fmt=request.param), dev, seed=0, layer=1)
    yield layer
    del layer
    torch.cuda.empty_cache()


@pytest.mark.parametrize("T", [1, 8, 16, 40])
def test_model_shape_formats(N, dev, model_layer, T):
    _check(N, dev, model_layer, T, step=60 + T)


def test_model_shape_formats_entry_points(N, dev, model_layer):
    _check(N, dev, model_layer, 9, step=7, via_layer=False)


def test_formats_decode_batch_invariant(N, dev, model_layer):
    layer = model_layer
    d = layer.dims()
    T = 16
    x, _ = layer.x(T, 5, dev)
    ws = torch.zeros(N.moe_workspace_bytes(d, T) // 4 + 64, dtype=torch.int32, device=dev)
    N.moe_workspace_init(ws)
    y = torch.zeros((T, layer.H), dtype=torch.float32, device=dev)
    N.moe_layer_forward(d, layer.native_weights(), None, x, T, y, ws)
    for t in (0, 9):
        y1 = torch.zeros((1, layer.H), dtype=torch.float32, device=dev)
        N.moe_layer_forward(d, layer.native_weights(), None, x[t:t + 1].contiguous(), 1, y1, ws)
        assert torch.equal(y1[0], y[t]), t
    torch.cuda.synchronize()
    assert N.moe_check_device_error(ws) == 0


@pytest.mark.parametrize("plan", [(128, 0, 0, 32), (64, 1, 1, 32), (128, 2, 2, 32)])
def test_model_shape_formats_prefill_plans(N, dev, model_layer, plan):
    """Each grouped-GEMM kernel a plan can name, forced, on the codebook and affine formats: the
    pipelined kernels dequantize both formats (the affine format's 128-row plan falls back to the
    general kernel, which the plan query reports)."""
    N.moe_debug_force_prefill_plan(N.moe_prefill_plan(*plan))
    try:
        got = N.moe_prefill_plan_get(model_layer.dims(), 300)
        want_gu = plan[1]
        if model_layer.fmt == S.FMT_AFFINE4 and plan[1] == N.MOE_GEMM_PIPE128:
            want_gu = N.MOE_GEMM_GENERAL
        assert got.gate_up_kernel == want_gu
        _check(N, dev, model_layer, 300, step=300 + plan[1])
    finally:
        N.moe_debug_force_prefill_plan(None)
