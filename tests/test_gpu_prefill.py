"""GPU parity of the prefill path (router GEMM, grouping, grouped-GEMM FFNs, combine) against the
CPU oracle, through the C interface.

Bars: grouping (counts, offsets, permutation) bit-exact; top-k ids bit-exact outside oracle
near-ties (k-th / (k+1)-th logit gap < 1e-4, counted); layer outputs within a per-token
normwise relative error of 2e-3.  The prefill GEMMs run fp16 MFMA on fp16-rounded weights
(q * scale) and an fp16 SwiGLU intermediate, so outputs are not bit-equal to the decode path.
"""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from layer_fixtures import MODEL, TINY, Layer, near_tie_tokens  # noqa: E402
from mixture_experts_route_amd import synth as S  # noqa: E402
from oracle import moe_oracle as O  # noqa: E402

Y_TOL = 2e-3
TINY_BF16 = dict(TINY, x_f32=False, r_f32=False, cfg=11)


@pytest.fixture(scope="module")
def N():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mixture_experts_route_amd import native

    return native


@pytest.fixture(scope="module")
def dev():
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def model_layer(N, dev):
    return Layer(MODEL, dev, seed=0)


def _ws(N, d, T, dev):
    ws = torch.zeros(N.moe_workspace_bytes(d, T) // 4 + 64, dtype=torch.int32, device=dev)
    N.moe_workspace_init(ws)
    return ws


@pytest.mark.parametrize("T,E,k", [(1, 8, 2), (9, 512, 10), (300, 512, 10), (4096, 512, 10), (37, 64, 16)])
def test_group_tokens_bit_exact(N, dev, T, E, k):
    rng = np.random.default_rng(T * 7 + E)
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    d = N.dims(2048, 768, E, k, 1)
    ws = _ws(N, d, T, dev)
    counts = torch.full((E,), -1, dtype=torch.int32, device=dev)
    offsets = torch.full((E + 1,), -1, dtype=torch.int32, device=dev)
    perm = torch.full((T * k,), -1, dtype=torch.int32, device=dev)
    N.moe_group_tokens(d, torch.from_numpy(ids).to(dev), T, counts, offsets, perm, ws)
    torch.cuda.synchronize()
    assert N.moe_check_device_error(ws) == 0
    c_ref, o_ref, p_ref = O.group_pairs(ids.ravel(), E)
    assert np.array_equal(counts.cpu().numpy(), c_ref)
    assert np.array_equal(offsets.cpu().numpy(), o_ref)
    assert np.array_equal(perm.cpu().numpy(), p_ref)


def test_group_tokens_skewed(N, dev):
    """Every token picks the same experts: one 600-row group per chosen expert."""
    T, E, k = 600, 512, 10
    ids = np.tile(np.array([5, 9, 100, 3, 7, 200, 511, 0, 42, 77], np.int32), (T, 1))
    d = N.dims(2048, 768, E, k, 1)
    ws = _ws(N, d, T, dev)
    counts = torch.zeros((E,), dtype=torch.int32, device=dev)
    offsets = torch.zeros((E + 1,), dtype=torch.int32, device=dev)
    perm = torch.zeros((T * k,), dtype=torch.int32, device=dev)
    N.moe_group_tokens(d, torch.from_numpy(ids).to(dev), T, counts, offsets, perm, ws)
    torch.cuda.synchronize()
    c_ref, o_ref, p_ref = O.group_pairs(ids.ravel(), E)
    assert np.array_equal(perm.cpu().numpy(), p_ref) and np.array_equal(counts.cpu().numpy(), c_ref)


def _prefill_check(N, dev, layer, T, step, sample=None, via_layer=True, table=None):
    # the whole-layer call decodes batches up to the decode limit: smaller ones reach the prefill
    # kernels through their own entry point
    via_layer = via_layer and T > N.MOE_DECODE_MAX_TOKENS
    d = layer.dims()
    x, x64 = layer.x(T, step, dev)
    ws = _ws(N, d, T, dev)
    y = torch.full((T, layer.H), float("nan"), dtype=torch.float32, device=dev)
    ids = torch.zeros((T, layer.k), dtype=torch.int32, device=dev)
    w = torch.zeros((T, layer.k), dtype=torch.float32, device=dev)
    wts = layer.native_weights()
    if via_layer:
        N.moe_layer_forward(d, wts, table, x, T, y, ws, topk_ids=ids, topk_w=w)
    else:
        logits = torch.zeros((T, layer.E), dtype=torch.float32, device=dev)
        N.moe_route(d, x, T, layer.router, layer.bias, ids, w, logits, ws)
        N.moe_expert_ffn_prefill(d, wts, table, x, T, ids, w, y, ws)
    torch.cuda.synchronize()
    assert N.moe_check_device_error(ws) == 0
    rows = np.arange(T) if sample is None else np.asarray(sample)
    ref = layer.oracle(x64[rows])
    ok = ~near_tie_tokens(ref["logits64"], layer.k)
    ids_np = ids.cpu().numpy()[rows]
    assert np.array_equal(ids_np[ok], ref["ids"][ok])
    err = O.per_token_rel_err(y.cpu().numpy()[rows], ref["y"])
    assert np.all(err[ok] <= Y_TOL), (err.max(), np.argmax(err))
    return y, err


@pytest.mark.parametrize("T", [9, 17, 40, 200])
def test_prefill_tiny(N, dev, T):
    layer = Layer(TINY_BF16, dev, seed=0)
    _, err = _prefill_check(N, dev, layer, T, step=T)
    assert err.max() < 1e-3


@pytest.mark.parametrize("T", [9, 17, 300])
def test_prefill_model_shape(N, dev, model_layer, T):
    _prefill_check(N, dev, model_layer, T, step=100 + T)


def test_prefill_ffn_entry_point(N, dev, model_layer):
    _prefill_check(N, dev, model_layer, 130, step=7, via_layer=False)


def test_prefill_4k_sampled(N, dev, model_layer):
    """The benchmark's shape (4096 tokens) on sampled tokens, including both ends."""
    rng = np.random.default_rng(0)
    sample = np.unique(np.concatenate([[0, 1, 4095], rng.choice(4096, 13, replace=False)]))
    _prefill_check(N, dev, model_layer, 4096, step=4096, sample=sample)


def test_prefill_32k_sampled_zipf(N, dev):
    """The long prefill shape (32,768 tokens) with Zipf(1.1)-skewed routing (hot experts with
    thousands of rows), on sampled tokens including both ends."""
    layer = Layer(MODEL, dev, seed=4, bias_c=S.ZIPF_C)
    T = 32768
    rng = np.random.default_rng(1)
    sample = np.unique(np.concatenate([[0, 1, T - 1], rng.choice(T, 13, replace=False)]))
    _prefill_check(N, dev, layer, T, step=T, sample=sample)


def test_prefill_skewed_zipf_routing(N, dev):
    """Zipf(1.1)-skewed routing (uneven groups, several 128-row items per hot expert)."""
    layer = Layer(MODEL, dev, seed=3, bias_c=S.ZIPF_C)
    _prefill_check(N, dev, layer, 700, step=1)


def test_prefill_slot_table_bitwise(N, dev):
    rng = np.random.default_rng(9)
    E = MODEL["E"]
    n_slots = E + 16
    perm = rng.permutation(n_slots)[:E]
    pooled = Layer(MODEL, dev, seed=0, n_slots=n_slots, slot_of=perm)
    direct = Layer(MODEL, dev, seed=0)
    d = direct.dims()
    T = 257
    x, _ = direct.x(T, 3, dev)
    ws = _ws(N, d, T, dev)
    ya = torch.zeros((T, direct.H), dtype=torch.float32, device=dev)
    yb = torch.zeros_like(ya)
    N.moe_layer_forward(d, direct.native_weights(), None, x, T, ya, ws)
    N.moe_layer_forward(d, pooled.native_weights(), pooled.table_tensor(dev), x, T, yb, ws)
    torch.cuda.synchronize()
    assert N.moe_check_device_error(ws) == 0
    assert torch.equal(ya, yb)


def test_prefill_deterministic_and_batch_invariant_rows(N, dev, model_layer):
    layer = model_layer
    d = layer.dims()
    T = 520
    x, _ = layer.x(T, 77, dev)
    ws = _ws(N, d, T, dev)
    y1 = torch.zeros((T, layer.H), dtype=torch.float32, device=dev)
    y2 = torch.zeros_like(y1)
    N.moe_layer_forward(d, layer.native_weights(), None, x, T, y1, ws)
    N.moe_layer_forward(d, layer.native_weights(), None, x, T, y2, ws)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


def test_prefill_route_model_shape(N, dev, model_layer):
    """The prefill router GEMM and top-k at the model shape (the pipelined router kernel: 32-row
    token works below ~3K tokens, 64-row works above, ragged last works at 300 and 5,000 tokens)
    against the oracle: logits within fp32 accumulation of the fp64 ones, ids exact away from near
    ties, weights within 1e-5; and a token's logits bitwise the same whatever batch it is routed in
    (each logit takes the same MFMA steps in every work shape)."""
    layer = model_layer
    d = layer.dims()
    T = 5000
    x, x64 = layer.x(T, 31, dev)
    got = {}
    for n in (T, 300, 40):
        ws = _ws(N, d, n, dev)
        ids = torch.full((n, layer.k), -7, dtype=torch.int32, device=dev)
        w = torch.zeros((n, layer.k), dtype=torch.float32, device=dev)
        logits = torch.zeros((n, layer.E), dtype=torch.float32, device=dev)
        N.moe_route(d, x[:n], n, layer.router, layer.bias, ids, w, logits, ws)
        torch.cuda.synchronize()
        assert N.moe_check_device_error(ws) == 0
        got[n] = (logits.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy())
    lg = got[T][0]
    assert np.array_equal(got[300][0], lg[:300]) and np.array_equal(got[40][0], lg[:40])
    rows = np.r_[0:40, 260:340, 4900:5000]  # the small batches, a work boundary, the ragged tail
    l64, _, ids_ref, w_ref = O.route(x64[rows], layer.router_np.astype(np.float64), layer.bias_np, layer.k)
    assert np.max(np.abs(lg[rows].astype(np.float64) - l64)) <= 1e-5 * max(1.0, np.max(np.abs(l64)))
    ok = ~near_tie_tokens(l64, layer.k)
    assert np.array_equal(got[T][1][rows][ok], ids_ref[ok])
    assert np.max(np.abs(got[T][2][rows][ok] - w_ref[ok])) <= 1e-5


def test_prefill_not_resident_is_an_error(N, dev, model_layer):
    layer = model_layer
    d = layer.dims()
    T = 64
    x, _ = layer.x(T, 5, dev)
    ws = _ws(N, d, T, dev)
    ids = torch.from_numpy(np.tile(np.arange(10, dtype=np.int32), (T, 1))).to(dev)
    w = torch.full((T, 10), 0.1, dtype=torch.float32, device=dev)
    table = torch.arange(layer.E, dtype=torch.int32, device=dev)
    table[4] = -1
    y = torch.zeros((T, layer.H), dtype=torch.float32, device=dev)
    N.moe_expert_ffn_prefill(d, layer.native_weights(), table, x, T, ids, w, y, ws)
    assert N.moe_check_device_error(ws) & N.DERR_NOT_RESIDENT


def _dup_ids(T, k, E, seed):
    """Distinct ids per token, except token T // 2 whose choice 3 repeats its choice 1."""
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    ids[T // 2, 3] = ids[T // 2, 1]
    return ids


@pytest.mark.parametrize("T", [1, 3, 8, 40])
def test_duplicate_ids_are_reported(N, dev, model_layer, T):
    """A token whose top-k list names one expert twice is an error (MOE_DERR_DUP_ID), never a silent
    result, through the grouping, the decode FFNs (up to 8 tokens) and the prefill FFNs; the
    workspace stays usable for the next call."""
    layer = model_layer
    d = layer.dims()
    E, k = layer.E, layer.k
    ids_np = _dup_ids(T, k, E, seed=T)
    ids = torch.from_numpy(ids_np).to(dev)
    w = torch.full((T, k), 1.0 / k, dtype=torch.float32, device=dev)
    x, _ = layer.x(T, 3, dev)
    ws = _ws(N, d, T, dev)
    counts = torch.zeros((E,), dtype=torch.int32, device=dev)
    offsets = torch.zeros((E + 1,), dtype=torch.int32, device=dev)
    perm = torch.zeros((T * k,), dtype=torch.int32, device=dev)
    N.moe_group_tokens(d, ids, T, counts, offsets, perm, ws)
    torch.cuda.synchronize()
    assert N.moe_check_device_error(ws) & N.DERR_DUP_ID
    y = torch.zeros((T, layer.H), dtype=torch.float32, device=dev)
    if T <= N.MOE_DECODE_MAX_TOKENS:
        N.moe_expert_ffn_decode(d, layer.native_weights(), None, x, T, ids, w, y, ws)
        torch.cuda.synchronize()
        assert N.moe_check_device_error(ws) & N.DERR_DUP_ID
    N.moe_expert_ffn_prefill(d, layer.native_weights(), None, x, T, ids, w, y, ws)
    torch.cuda.synchronize()
    assert N.moe_check_device_error(ws) & N.DERR_DUP_ID
    # the same workspace then serves a valid call with no error
    _prefill_check(N, dev, layer, 40, step=41)


def test_prefill_fp16_range_is_reported(N, dev, model_layer):
    """The prefill path holds activations, the SwiGLU intermediate and the weighted expert rows in
    fp16: a token whose values leave the fp16 range sets MOE_DERR_RANGE instead of turning into
    infinities.  Large activations (x 100) overflow the SwiGLU output; a bf16 activation beyond
    65504 overflows the conversion itself."""
    layer = model_layer
    d = layer.dims()
    T = 24
    x, _ = layer.x(T, 9, dev)
    ws = _ws(N, d, T, dev)
    y = torch.zeros((T, layer.H), dtype=torch.float32, device=dev)
    big = (x.view(torch.bfloat16).float() * 100.0).to(torch.bfloat16).view(torch.int16)
    N.moe_layer_forward(d, layer.native_weights(), None, big, T, y, ws)
    torch.cuda.synchronize()
    assert N.moe_check_device_error(ws) & N.DERR_RANGE
    huge = x.clone()
    huge[5, 17] = 0x4780  # bf16 65536.0
    N.moe_layer_forward(d, layer.native_weights(), None, huge, T, y, ws)
    torch.cuda.synchronize()
    assert N.moe_check_device_error(ws) & N.DERR_RANGE
    # the unscaled batch passes (and the flag is not left set)
    _prefill_check(N, dev, layer, T, step=9)


@pytest.mark.parametrize("plan", [(128, 0, 0, 32), (64, 1, 1, 32), (64, 0, 2, 64), (128, 2, 2, 64), (64, 2, 1, 32)])
@pytest.mark.parametrize("T", [300, 4096])
def test_prefill_plans_parity(N, dev, model_layer, plan, T):
    """Every grouped-GEMM kernel and item size a plan can choose (forced), against the oracle: in full
    at 300 tokens, on sampled rows at 4096."""
    N.moe_debug_force_prefill_plan(N.moe_prefill_plan(*plan))
    try:
        got = N.moe_prefill_plan_get(model_layer.dims(), T)
        assert (got.item_rows, got.gate_up_kernel, got.down_kernel, got.router_rows) == plan
        sample = None if T <= 300 else np.r_[0:3, 2047:2050, T - 3:T]
        _prefill_check(N, dev, model_layer, T, step=T + plan[1] * 10 + plan[2], sample=sample)
    finally:
        N.moe_debug_force_prefill_plan(None)


def test_prefill_deep_plan_zipf_routing(N, dev):
    """The 64-row deep-prefetch kernels under Zipf(1.1)-skewed routing (long and short groups)."""
    layer = Layer(dict(MODEL, cfg=4), dev, seed=0, layer=2, bias_c=S.ZIPF_C)
    N.moe_debug_force_prefill_plan(N.moe_prefill_plan(64, 1, 1, 32))
    try:
        _prefill_check(N, dev, layer, 700, step=1)
    finally:
        N.moe_debug_force_prefill_plan(None)
