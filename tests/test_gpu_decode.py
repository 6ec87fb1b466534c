"""GPU parity of the decode path (router, top-k, residency check, 4-bit GEMV FFNs, combine)
against the CPU oracle, through the C interface.

Bars: dequantized weights, top-k ids, slots and miss lists bit-exact (tokens whose oracle
k-th / (k+1)-th logit gap is below 1e-4 are excluded from id and output parity, and
counted); router weights within 1e-5; layer outputs within a per-token normwise relative
error of 2e-3 (max_o |y - y_ref| / max_o |y_ref|).
"""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from layer_fixtures import MODEL, TINY, Layer, near_tie_tokens  # noqa: E402
from oracle import moe_oracle as O  # noqa: E402

Y_TOL = 2e-3
W_TOL = 1e-5


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
    nbytes = N.moe_workspace_bytes(d, T)
    assert nbytes > 0
    ws = torch.zeros(nbytes // 4 + 64, dtype=torch.int32, device=dev)
    N.moe_workspace_init(ws)
    return ws


def _check_no_device_error(N, ws):
    assert N.moe_check_device_error(ws) == 0


@pytest.mark.parametrize("shape", [(256, 128), (2048, 768), (4096, 4096 // 4)])
def test_debug_dequant_bit_exact(N, dev, shape):
    from mixture_experts_route_amd import synth as S

    H, F = shape
    d = N.dims(H, F, 8, 2, 1)
    blob_np = S.expert_blob_np(S.stream_key(7, 0, "blob", 0, 0), H, F)
    blob = torch.from_numpy(blob_np).to(dev)
    Wg, Wu, Wd = O.expert_weights(blob_np, H, F)
    for m, ref in enumerate((Wg, Wu, Wd)):
        out = torch.full(ref.shape, float("nan"), dtype=torch.float32, device=dev)
        N.moe_debug_dequant(d, blob, m, out)
        got = out.cpu().numpy().astype(np.float64)
        assert np.array_equal(got, ref), f"matrix {m}: {np.sum(got != ref)} mismatches"


def _route_check(N, dev, layer, T, step):
    d = layer.dims()
    x, x64 = layer.x(T, step, dev)
    ws = _ws(N, d, T, dev)
    ids = torch.full((T, layer.k), -7, dtype=torch.int32, device=dev)
    w = torch.zeros((T, layer.k), dtype=torch.float32, device=dev)
    logits = torch.zeros((T, layer.E), dtype=torch.float32, device=dev)
    N.moe_route(d, x, T, layer.router, layer.bias, ids, w, logits, ws)
    torch.cuda.synchronize()
    _check_no_device_error(N, ws)
    l64, l32, ids_ref, w_ref = O.route(x64, layer.router_np.astype(np.float64), layer.bias_np, layer.k)
    lg = logits.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(lg - l64)) <= 1e-5 * max(1.0, np.max(np.abs(l64)))
    tie = near_tie_tokens(l64, layer.k)
    ok = ~tie
    assert np.array_equal(ids.cpu().numpy()[ok], ids_ref[ok])
    assert np.max(np.abs(w.cpu().numpy()[ok] - w_ref[ok])) <= W_TOL
    assert np.allclose(w.cpu().numpy().sum(axis=1), 1.0, atol=layer.k * 2.0**-23)
    return int(tie.sum())


def test_route_tiny(N, dev):
    layer = Layer(TINY, dev, seed=0)
    for step in range(4):
        _route_check(N, dev, layer, 4, step)


@pytest.mark.parametrize("T", [1, 3, 8, 16])
def test_route_model_shape(N, dev, model_layer, T):
    ties = sum(_route_check(N, dev, model_layer, T, step) for step in range(3))
    assert ties <= T  # near ties are rare at this logit spread


def _tied_router(dev, H, E):
    """bf16 router whose rows come in equal pairs (2i, 2i + 1), plus a run of 8 equal rows: the
    GPU's logits for equal rows are bitwise equal, so the selection meets exact ties."""
    from mixture_experts_route_amd import synth as S

    codes = S.bf16_normal_np(S.stream_key(3, 2, "router", 0, 0), (E, H), 0.02)
    codes[1::2] = codes[0::2]
    codes[40:48] = codes[40]
    return torch.from_numpy(codes.view(np.int16)).to(dev)


@pytest.mark.parametrize("E,k", [(512, 10), (1024, 10), (1024, 16)])
@pytest.mark.parametrize("T", [1, 5, 8, 16, 300])
def test_topk_exact_ties_lower_id_first(N, dev, T, E, k):
    """Selection on the GPU's own fp32 logits equals the oracle's ranking (logit desc, id asc)
    exactly when many logits are equal (decode route for T <= 8, prefill top-k above), at the
    model's 512 experts (8 logits per lane) and at the largest expert count and k (16 per lane)."""
    from mixture_experts_route_amd import synth as S

    H, F = 2048, 768
    d = N.dims(H, F, E, k, 1)
    router = _tied_router(dev, H, E)
    x = torch.from_numpy(S.bf16_normal_np(S.stream_key(3, 2, "x", 0, T), (T, H), 1.0).view(np.int16)).to(dev)
    ws = _ws(N, d, T, dev)
    ids = torch.full((T, k), -7, dtype=torch.int32, device=dev)
    w = torch.zeros((T, k), dtype=torch.float32, device=dev)
    logits = torch.zeros((T, E), dtype=torch.float32, device=dev)
    N.moe_route(d, x, T, router, None, ids, w, logits, ws)
    torch.cuda.synchronize()
    _check_no_device_error(N, ws)
    lg = logits.cpu().numpy()
    assert np.array_equal(lg[:, 1::2], lg[:, 0::2]), "equal router rows must give equal logits"
    got = ids.cpu().numpy()
    ref = O.select_topk(lg, k)
    assert np.array_equal(got, ref)
    assert np.max(np.abs(w.cpu().numpy() - O.route_weights(lg, ref))) <= 1e-6
    # the selections really contain tied pairs, ranked lower id first
    tied = sum(int(np.isin(row ^ 1, row).sum()) for row in got)
    assert tied >= T


@pytest.mark.parametrize("T", [1, 8, 16])
def test_layer_forward_exact_ties(N, dev, model_layer, T):
    """The decode plan path (router launch with selection and plan) ranks exact ties as moe_route."""
    layer = model_layer
    d = layer.dims()
    router = _tied_router(dev, layer.H, layer.E)
    x, _ = layer.x(T, 5, dev)
    from mixture_experts_route_amd import native as NN

    wts = NN.layer_weights(router, layer.arena, layer.stride, layer.n_slots, layer.shared, None)
    ws = _ws(N, d, T, dev)
    y = torch.zeros((T, layer.H), dtype=torch.float32, device=dev)
    ids = torch.zeros((T, layer.k), dtype=torch.int32, device=dev)
    w = torch.zeros((T, layer.k), dtype=torch.float32, device=dev)
    N.moe_layer_forward(d, wts, None, x, T, y, ws, topk_ids=ids, topk_w=w)
    ids2 = torch.zeros_like(ids)
    w2 = torch.zeros_like(w)
    logits = torch.zeros((T, layer.E), dtype=torch.float32, device=dev)
    N.moe_route(d, x, T, router, None, ids2, w2, logits, _ws(N, d, T, dev))
    torch.cuda.synchronize()
    _check_no_device_error(N, ws)
    assert np.array_equal(ids.cpu().numpy(), O.select_topk(logits.cpu().numpy(), layer.k))
    assert torch.equal(ids, ids2) and torch.equal(w, w2)


def _layer_check(N, dev, layer, T, step, table=None, via_layer=True):
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
        N.moe_expert_ffn_decode(d, wts, table, x, T, ids, w, y, ws)
    torch.cuda.synchronize()
    _check_no_device_error(N, ws)
    ref = layer.oracle(x64)
    ok = ~near_tie_tokens(ref["logits64"], layer.k)
    assert np.array_equal(ids.cpu().numpy()[ok], ref["ids"][ok])
    err = O.per_token_rel_err(y.cpu().numpy(), ref["y"])
    assert np.all(err[ok] <= Y_TOL), err
    return y, err


def test_layer_tiny_decode(N, dev):
    layer = Layer(TINY, dev, seed=0)
    for step in range(3):
        y, err = _layer_check(N, dev, layer, 4, step)
        assert err.max() < 1e-5  # fp32 activations ride as bf16 hi+lo; everything else fp32


@pytest.mark.parametrize("T", [1, 2, 5, 8, 9, 12, 16])
def test_layer_model_shape_decode(N, dev, model_layer, T):
    _layer_check(N, dev, model_layer, T, step=11 + T)


@pytest.fixture(scope="module")
def wide_layer(N, dev):
    """The largest supported routing: 1,024 experts, top-16 (+ shared), model widths."""
    return Layer(dict(MODEL, E=1024, k=16), dev, seed=0)


@pytest.mark.parametrize("T", [1, 3, 8, 16, 40])
def test_layer_wide_routing_1024_experts_top16(N, dev, wide_layer, T):
    """E = 1024, k = 16 through the whole layer: 16 logits per lane in the selection, up to 129
    decode tasks (the one-token down kernel's 17-task variant at T = 1), and the prefill path at
    T = 40; ids and outputs against the oracle."""
    _layer_check(N, dev, wide_layer, T, step=100 + T)


@pytest.mark.parametrize("H,F,E,k", [(1024, 512, 64, 6), (4096, 1536, 64, 8)])
@pytest.mark.parametrize("T", [1, 8, 16, 40])
def test_layer_other_widths(N, dev, H, F, E, k, T):
    """Hidden and FFN widths other than the model's (the decode kernels' other chunk counts, the
    generic prefill GEMM at T = 40), against the oracle."""
    layer = Layer(dict(MODEL, H=H, F=F, E=E, k=k), dev, seed=0, layer=H // 256)
    _layer_check(N, dev, layer, T, step=200 + T)
    del layer
    torch.cuda.empty_cache()


def test_layer_batched_decode_zipf_layers(N, dev):
    """The 48-layer batched decode's shape: 8 tokens per step through layers with their own
    Zipf(1.1) router bias (popular experts shared by several tokens of a step), one step in each
    of two layers."""
    from mixture_experts_route_amd import synth as S

    spec = dict(MODEL, cfg=3)
    for layer_id in (0, 47):
        layer = Layer(spec, dev, seed=0, layer=layer_id, bias_c=S.ZIPF_C)
        x, x64 = layer.x(8, 0, dev)
        ref = layer.oracle(x64)
        # the step really shares experts between tokens (tasks of several tokens)
        assert len(np.unique(ref["ids"])) < 8 * layer.k
        _layer_check(N, dev, layer, 8, 0)
        del layer
        torch.cuda.empty_cache()


@pytest.mark.parametrize("T", [3, 16])
def test_ffn_decode_entry_point(N, dev, model_layer, T):
    _layer_check(N, dev, model_layer, T, step=2 + T, via_layer=False)


def test_layer_batched_decode_16_tokens_zipf(N, dev):
    """A 16-token verify batch through a Zipf(1.1)-biased layer: popular experts are chosen by
    tokens on both sides of the 8-token boundary (tasks whose token slots fill both 16-row A
    blocks of the down kernels)."""
    from mixture_experts_route_amd import synth as S

    layer = Layer(dict(MODEL, cfg=3), dev, seed=0, layer=5, bias_c=S.ZIPF_C)
    x, x64 = layer.x(16, 3, dev)
    ids = layer.oracle(x64)["ids"]
    both = [e for e in np.unique(ids) if (ids[:8] == e).any() and (ids[8:] == e).any()]
    assert both, "no expert shared across the two halves"
    _layer_check(N, dev, layer, 16, 3)
    del layer
    torch.cuda.empty_cache()


def test_decode_bitwise_deterministic_and_batch_invariant(N, dev, model_layer):
    """A token's decode output is bitwise the same alone, in a batch of 8 and in a verify batch of
    16 at any position (halogen README, "Quality: what is measured, and what is not": a request
    batched with others emits the same bytes as alone; speculative verify = serial)."""
    layer = model_layer
    d = layer.dims()
    T = 16
    x, _ = layer.x(T, 99, dev)
    ws = _ws(N, d, T, dev)
    wts = layer.native_weights()
    ys = []
    for _ in range(2):
        y = torch.zeros((T, layer.H), dtype=torch.float32, device=dev)
        N.moe_layer_forward(d, wts, None, x, T, y, ws)
        ys.append(y.clone())
    assert torch.equal(ys[0], ys[1])
    # the first 8 tokens as a batch of 8, and every 4th token alone; the batch of 16 reversed
    y8 = torch.zeros((8, layer.H), dtype=torch.float32, device=dev)
    N.moe_layer_forward(d, wts, None, x[:8].contiguous(), 8, y8, ws)
    assert torch.equal(y8, ys[0][:8]), "tokens 0..7 differ in a batch of 8 vs 16"
    for t in (0, 5, 8, 15):
        y1 = torch.zeros((1, layer.H), dtype=torch.float32, device=dev)
        N.moe_layer_forward(d, wts, None, x[t:t + 1].contiguous(), 1, y1, ws)
        assert torch.equal(y1[0], ys[0][t]), f"token {t} differs alone vs in a batch of {T}"
    yr = torch.zeros((T, layer.H), dtype=torch.float32, device=dev)
    N.moe_layer_forward(d, wts, None, x.flip(0).contiguous(), T, yr, ws)
    assert torch.equal(yr.flip(0), ys[0]), "a token's output depends on its position in the batch"
    # 9..15 tokens (the other kernel variants' batch sizes) agree too
    for T2 in (3, 11):
        y2 = torch.zeros((T2, layer.H), dtype=torch.float32, device=dev)
        N.moe_layer_forward(d, wts, None, x[:T2].contiguous(), T2, y2, ws)
        assert torch.equal(y2, ys[0][:T2]), f"batch of {T2}"
    _check_no_device_error(N, ws)


def test_slot_table_equals_all_resident_bitwise(N, dev):
    """All experts resident at permuted slots of a larger arena == identity placement."""
    rng = np.random.default_rng(4)
    E = MODEL["E"]
    n_slots = E + 40
    perm = rng.permutation(n_slots)[:E]
    pooled = Layer(MODEL, dev, seed=0, n_slots=n_slots, slot_of=perm)
    direct = Layer(MODEL, dev, seed=0)
    d = direct.dims()
    T = 4
    x, _ = direct.x(T, 5, dev)
    ws = _ws(N, d, T, dev)
    ya = torch.zeros((T, direct.H), dtype=torch.float32, device=dev)
    yb = torch.zeros_like(ya)
    N.moe_layer_forward(d, direct.native_weights(), None, x, T, ya, ws)
    N.moe_layer_forward(d, pooled.native_weights(), pooled.table_tensor(dev), x, T, yb, ws)
    torch.cuda.synchronize()
    _check_no_device_error(N, ws)
    assert torch.equal(ya, yb)


def test_slot_lookup_bit_exact(N, dev):
    rng = np.random.default_rng(8)
    E, k = 512, 10
    d = N.dims(2048, 768, E, k, 1)
    # one launch up to 1,024 pairs (T = 1, 8, 102), two above (T = 103, 300)
    for T in (1, 8, 102, 103, 300):
        n_slots = 240
        table = np.full(E, -1, dtype=np.int32)
        res = rng.choice(E, n_slots, replace=False)
        table[res] = rng.permutation(n_slots)
        ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
        ws = _ws(N, d, T, dev)
        slots = torch.full((T, k), -9, dtype=torch.int32, device=dev)
        miss = torch.full((E,), -9, dtype=torch.int32, device=dev)
        cnt = torch.full((1,), -9, dtype=torch.int32, device=dev)
        N.moe_slot_lookup(d, torch.from_numpy(table).to(dev), n_slots, torch.from_numpy(ids).to(dev), T, slots, miss,
                          cnt, ws)
        torch.cuda.synchronize()
        _check_no_device_error(N, ws)
        s_ref, m_ref = O.slot_lookup(table, ids)
        assert np.array_equal(slots.cpu().numpy(), s_ref)
        n = int(cnt.item())
        assert n == len(m_ref)
        assert np.array_equal(miss.cpu().numpy()[:n], m_ref)


@pytest.mark.parametrize("T", [1, 300])
def test_slot_lookup_reports_bad_ids_and_slots(N, dev, T):
    """An id outside [0, E) and a table entry >= n_slots set their error bits (both launch shapes);
    the pair's slot reads -1 and the other pairs are still looked up."""
    E, k = 512, 10
    d = N.dims(2048, 768, E, k, 1)
    n_slots = 100
    table = np.arange(E, dtype=np.int32) % 128  # entries 100..127 are >= n_slots
    table[::3] = -1
    rng = np.random.default_rng(11)
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    ids[0, 0] = E + 5
    ws = _ws(N, d, T, dev)
    slots = torch.full((T, k), -9, dtype=torch.int32, device=dev)
    miss = torch.full((E,), -9, dtype=torch.int32, device=dev)
    cnt = torch.full((1,), -9, dtype=torch.int32, device=dev)
    N.moe_slot_lookup(d, torch.from_numpy(table).to(dev), n_slots, torch.from_numpy(ids).to(dev), T, slots, miss, cnt,
                      ws)
    bits = N.moe_check_device_error(ws)
    assert bits & N.DERR_EXPERT_ID
    assert bits & N.DERR_SLOT
    got = slots.cpu().numpy()
    assert got[0, 0] == -1
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            if 0 <= e < E:
                s_ref = int(table[e])
                assert got[t, j] == (s_ref if 0 <= s_ref < n_slots else -1), (t, j)


def test_device_errors_are_reported(N, dev, model_layer):
    layer = model_layer
    d = layer.dims()
    T = 2
    x, _ = layer.x(T, 0, dev)
    ws = _ws(N, d, T, dev)
    ids = torch.tensor([[0, 1, 2, 3, 4, 5, 6, 7, 8, 9], [1, 2, 3, 4, 5, 6, 7, 8, 9, 600]], dtype=torch.int32,
                       device=dev)
    w = torch.full((T, layer.k), 0.1, dtype=torch.float32, device=dev)
    y = torch.zeros((T, layer.H), dtype=torch.float32, device=dev)
    N.moe_expert_ffn_decode(d, layer.native_weights(), None, x, T, ids, w, y, ws)
    assert N.moe_check_device_error(ws) & N.DERR_EXPERT_ID
    assert N.moe_check_device_error(ws) == 0  # cleared
    # an expert the table marks absent is an error, never a silent zero contribution
    table = torch.arange(layer.E, dtype=torch.int32, device=dev)
    table[3] = -1
    ids[1, 9] = 11
    N.moe_expert_ffn_decode(d, layer.native_weights(), table, x, T, ids, w, y, ws)
    assert N.moe_check_device_error(ws) & N.DERR_NOT_RESIDENT


@pytest.mark.parametrize("T", [1, 8])
def test_layer_without_shared_expert(N, dev, T):
    """n_shared = 0 through the whole layer (one token: the gate/up launch selects; eight: the
    router launch plans): k tasks only, against the oracle."""
    layer = Layer(dict(MODEL, n_shared=0), dev, seed=0, layer=7)
    _layer_check(N, dev, layer, T, step=300 + T)


def test_layer_forward_not_resident_is_reported(N, dev, model_layer):
    """A selected expert the slot table marks absent (no doorbell attached) is an error of the call,
    in the one-token path where the gate/up launch selects and in the router-planned path."""
    layer = model_layer
    d = layer.dims()
    for T in (1, 8):
        x, _ = layer.x(T, 400 + T, dev)
        ws = _ws(N, d, T, dev)
        y = torch.zeros((T, layer.H), dtype=torch.float32, device=dev)
        ids = torch.zeros((T, layer.k), dtype=torch.int32, device=dev)
        N.moe_layer_forward(d, layer.native_weights(), None, x, T, y, ws, topk_ids=ids)
        torch.cuda.synchronize()
        _check_no_device_error(N, ws)
        table = torch.arange(layer.E, dtype=torch.int32, device=dev)
        table[int(ids[0, 0].item())] = -1  # token 0's first choice is now absent
        N.moe_layer_forward(d, layer.native_weights(), table, x, T, y, ws)
        assert N.moe_check_device_error(ws) & N.DERR_NOT_RESIDENT, T
        assert N.moe_check_device_error(ws) == 0
