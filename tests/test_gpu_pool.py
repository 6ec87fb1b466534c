"""GPU tests of the host slot-pool service (decode path): misses, fills and the slot table step
by step against the oracle's pool policy fed with the GPU's own selections, layer outputs
against the oracle layer, and the failure path (host-forced, no kernel waits)."""

import os
import sys

import numpy as np
import pytest
import torch

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
from layer_fixtures import MODEL, near_tie_tokens, slot_stride  # noqa: E402
from oracle import moe_oracle as O  # noqa: E402

pytestmark = pytest.mark.gpu

Y_TOL = 2e-3


@pytest.fixture(scope="module")
def N():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mixture_experts_route_amd import native

    return native


@pytest.fixture(scope="module")
def dev():
    return torch.device("cuda:0")


class PoolLayer:
    """One model-shaped layer whose routed experts live partly in `n_slots` HBM slots and partly in
    pinned host memory, with the router bias of a popularity ranking per topic."""

    def __init__(self, N, dev, layer_id, n_slots, topics=2, n_spares=1, initial=None):
        from mixture_experts_route_amd import synth as S

        self.S, self.N = S, N
        self.H, self.F, self.E, self.k = MODEL["H"], MODEL["F"], MODEL["E"], MODEL["k"]
        self.cfg, self.layer = 5, layer_id
        self.stride = slot_stride(self.H, self.F)
        self.blob = S.blob_bytes(self.H, self.F)
        E = self.E
        keys = [S.stream_key(0, self.cfg, "blob", layer_id, e) for e in range(E)]
        allb = torch.empty((E, self.stride), dtype=torch.uint8, device=dev)
        S.expert_blobs_torch_batch(keys, self.H, self.F, allb)
        self.ranks = [S.rank_permutation(0, self.cfg, layer_id, t, E) for t in range(topics)]
        self.bias_np = [S.zipf_bias(r, S.ZIPF_C) for r in self.ranks]
        self.bias = [torch.from_numpy(b).to(dev) for b in self.bias_np]
        # initial residency: the hottest experts of topic 0, hottest first (or the given list)
        self.initial = [int(e) for e in np.argsort(self.ranks[0], kind="stable")[:n_slots]] if initial is None \
            else [int(e) for e in initial]
        self.n_slots = n_slots
        self.arena = allb[torch.as_tensor(self.initial, device=dev, dtype=torch.long)].contiguous()
        resident = set(self.initial)
        self.away = [e for e in range(E) if e not in resident]
        self.homes = torch.empty((len(self.away) + n_spares, self.stride), dtype=torch.uint8, pin_memory=True)
        if self.away:
            self.homes[:len(self.away)].copy_(allb[torch.as_tensor(self.away, device=dev, dtype=torch.long)].cpu())
        del allb
        torch.cuda.empty_cache()
        self.home_addr = [0] * E
        for i, e in enumerate(self.away):
            self.home_addr[e] = self.homes[i].data_ptr()
        self.n_spares = n_spares
        self.spares = self.homes[len(self.away)]
        self.shared = torch.empty((self.stride,), dtype=torch.uint8, device=dev)
        S.expert_blobs_torch([S.stream_key(0, self.cfg, "shared", layer_id, 0)], self.H, self.F, self.shared.view(1, -1))
        rkey = S.stream_key(0, self.cfg, "router", layer_id, 0)
        codes = S.bf16_normal_np(rkey, (E, self.H), MODEL["r_sigma"])
        self.router_np = S.bf16_to_f32(codes).astype(np.float64)
        self.router = torch.from_numpy(codes.view(np.int16)).to(dev)
        self.table = torch.full((E,), -1, dtype=torch.int32, device=dev)
        self.ready = torch.zeros((64,), dtype=torch.int32, device=dev)
        self.hb_ids = N.HostBuffer(4 * E)
        self.hb_counts = N.HostBuffer(64)
        self.hb_step = N.HostBuffer(4 * N.MOE_DECODE_MAX_TOKENS * self.k)
        self.pool = N.moe_pool_create(self.dims(), self.arena, self.stride, n_slots, self.table, self.initial,
                                      self.home_addr, self.spares, n_spares, self.hb_ids.ptr, self.hb_counts.ptr,
                                      self.hb_step.ptr, self.ready)

    def dims(self):
        return self.N.dims(self.H, self.F, self.E, self.k, 1)

    def weights(self, topic):
        return self.N.layer_weights(self.router, self.arena, self.stride, self.n_slots, self.shared, self.bias[topic])

    def x(self, step):
        key = self.S.stream_key(0, self.cfg, "x", self.layer, step)
        codes = self.S.bf16_normal_np(key, (1, self.H), 1.0)
        return torch.from_numpy(codes.view(np.int16)), self.S.bf16_to_f32(codes).astype(np.float64)

    def blob_np(self, e):
        return self.S.expert_blob_np(self.S.stream_key(0, self.cfg, "blob", self.layer, e), self.H, self.F)

    def shared_np(self):
        return self.S.expert_blob_np(self.S.stream_key(0, self.cfg, "shared", self.layer, 0), self.H, self.F)

    def close(self):
        self.N.moe_pool_destroy(self.pool)
        for b in (self.hb_ids, self.hb_counts, self.hb_step):
            b.free()


def _ws(N, d, dev):
    ws = torch.zeros(N.moe_workspace_bytes(d, 1) // 4 + 64, dtype=torch.int32, device=dev)
    N.moe_workspace_init(ws)
    return ws


@pytest.mark.parametrize("n_spares,two_streams", [(1, False), (1, True), (4, True)])
def test_pool_decode_steps_match_oracle_policy_and_outputs(N, dev, pool_streams, n_spares, two_streams):
    """One copy stream and one spare buffer, or separate device->host and host->device streams
    with one spare (every copy out waits, by event, for the copy in that last read its buffer) or
    four (the copies of the two directions overlap): same fills, tables and outputs, and afterwards
    every evicted expert's bytes sit in the host buffer the swap rule gives it."""
    L = PoolLayer(N, dev, layer_id=20, n_slots=60, n_spares=n_spares)
    d = L.dims()
    ws = _ws(N, d, dev)
    compute, copy, h2d = pool_streams
    h2d = h2d if two_streams else None
    # the exclusive swap replayed on the host: a victim's bytes go to the oldest spare buffer,
    # the missed expert's buffer becomes the newest spare
    home = list(L.home_addr)
    spares = [L.spares.data_ptr() + i * L.stride for i in range(n_spares)]
    ref_pool = O.SlotPoolLRU(L.E, L.initial)
    ids = torch.zeros((1, L.k), dtype=torch.int32, device=dev)
    y = torch.zeros((1, L.H), dtype=torch.float32, device=dev)
    total_fills = 0
    for step in range(12):
        topic = step // 6  # the popularity ranking changes halfway: misses come in bursts
        x_cpu, x64 = L.x(step)
        x = x_cpu.to(dev)
        torch.cuda.synchronize()
        bell = N.moe_pool_arm(L.pool)
        with torch.cuda.stream(compute):
            N.moe_layer_forward(d, L.weights(topic), L.table, x, 1, y, ws, topk_ids=ids, bell=bell, stream=compute)
        fills = N.moe_pool_serve(L.pool, ws, copy, L.E, h2d_stream=h2d)
        compute.synchronize()
        copy.synchronize()
        if h2d is not None:
            h2d.synchronize()
        for e, _, old in fills:
            buf = spares.pop(0)
            spares.append(home[e])
            home[old], home[e] = buf, 0
        assert N.moe_check_device_error(ws) == 0
        got_ids = ids.cpu().numpy()
        misses, ref_fills = ref_pool.step(got_ids)
        assert [tuple(f) for f in fills] == [tuple(f) for f in ref_fills], (step, fills, ref_fills)
        assert np.array_equal(L.table.cpu().numpy(), ref_pool.table)
        assert np.array_equal(N.moe_pool_get_table(L.pool, L.E), ref_pool.table)
        total_fills += len(fills)
        ref = O.moe_layer(x64, L.router_np, L.bias_np[topic], L.k, L.blob_np, L.shared_np(), L.H, L.F)
        ok = ~near_tie_tokens(ref["logits64"], L.k)
        assert np.array_equal(got_ids[ok], ref["ids"][ok])
        if ok.all():
            err = O.per_token_rel_err(y.cpu().numpy(), ref["y"])
            assert err.max() <= Y_TOL, (step, err)
    st = N.moe_pool_get_stats(L.pool)
    assert st.calls == 12 and st.selections == 12 * L.k and st.misses == total_fills > 0
    assert st.bytes_h2d == st.bytes_d2h == total_fills * L.blob
    # the slots hold their experts' bytes after the fills (an evicted expert that comes back is
    # reloaded from the host buffer its bytes were swapped into, so the outputs above cover that)
    table = ref_pool.table
    arena = L.arena.cpu().numpy()
    filled = [int(e) for e in np.nonzero(table >= 0)[0] if int(e) not in set(L.initial)]
    for e in filled[:4] + [int(e) for e in np.nonzero(table >= 0)[0][:2]]:
        assert np.array_equal(arena[table[e], :L.blob], L.blob_np(e)), e
    # the evicted experts' bytes were copied out into the buffers the swap rule names
    base = L.homes.data_ptr()
    homes = L.homes.numpy()
    evicted = [int(e) for e in L.initial if table[e] < 0]
    assert evicted
    for e in evicted[:6]:
        assert home[e], e
        assert np.array_equal(homes[(home[e] - base) // L.stride, :L.blob], L.blob_np(e)), e
    L.close()


def test_pool_all_resident_never_misses(N, dev, pool_streams):
    """Every expert in a slot: the check kernel releases the stream itself on every call."""
    L = PoolLayer(N, dev, layer_id=3, n_slots=512)
    d = L.dims()
    ws = _ws(N, d, dev)
    compute, copy, _ = pool_streams
    y = torch.zeros((1, L.H), dtype=torch.float32, device=dev)
    for step in range(3):
        x = L.x(step)[0].to(dev)
        torch.cuda.synchronize()
        bell = N.moe_pool_arm(L.pool)
        with torch.cuda.stream(compute):
            N.moe_layer_forward(d, L.weights(0), L.table, x, 1, y, ws, bell=bell, stream=compute)
        assert N.moe_pool_serve(L.pool, ws, copy, L.E) == []
        compute.synchronize()
    assert N.moe_check_device_error(ws) == 0
    assert int(L.ready[0].item()) == 3  # written by the check kernel, epoch 3
    L.close()


def test_pool_serve_without_doorbell_times_out_and_flags(N, dev, pool_streams):
    """Host-forced failure: the call is armed but the layer is launched without the doorbell, so
    nothing rings; serve gives up after its timeout, releases the ready word and flags the
    workspace.  No kernel waits on anything here."""
    L = PoolLayer(N, dev, layer_id=40, n_slots=60)
    d = L.dims()
    ws = _ws(N, d, dev)
    copy = pool_streams[1]
    N.moe_pool_arm(L.pool)
    with pytest.raises(N.MoeError) as ei:
        N.moe_pool_serve(L.pool, ws, copy, L.E, timeout_us=200_000)
    assert ei.value.code == N.MOE_EFILL
    copy.synchronize()
    bits = ctypes_bits(N, ws)
    assert bits & N.DERR_FILL
    assert int(L.ready[0].item()) == 1
    L.close()


def ctypes_bits(N, ws):
    import ctypes

    b = ctypes.c_int32()
    N.raw("moe_check_device_error")(ws.data_ptr(), None, ctypes.byref(b))
    return b.value


def _pool_step(N, L, d, ws, compute, copy, step, topic, ref_pool, dev, ids, y, check=True):
    """One served decode call of the pool layer, checked against the oracle's policy and layer;
    returns the number of fills."""
    x_cpu, x64 = L.x(step)
    x = x_cpu.to(dev)
    torch.cuda.synchronize()
    bell = N.moe_pool_arm(L.pool)
    with torch.cuda.stream(compute):
        N.moe_layer_forward(d, L.weights(topic), L.table, x, 1, y, ws, topk_ids=ids, bell=bell, stream=compute)
    fills = N.moe_pool_serve(L.pool, ws, copy, L.E)
    compute.synchronize()
    copy.synchronize()
    assert N.moe_check_device_error(ws) == 0
    got_ids = ids.cpu().numpy()
    _, ref_fills = ref_pool.step(got_ids)
    assert [tuple(f) for f in fills] == [tuple(f) for f in ref_fills], (step, fills, ref_fills)
    assert np.array_equal(L.table.cpu().numpy(), ref_pool.table)
    if check:
        ref = O.moe_layer(x64, L.router_np, L.bias_np[topic], L.k, L.blob_np, L.shared_np(), L.H, L.F)
        ok = ~near_tie_tokens(ref["logits64"], L.k)
        assert np.array_equal(got_ids[ok], ref["ids"][ok])
        if ok.all():
            assert O.per_token_rel_err(y.cpu().numpy(), ref["y"]).max() <= Y_TOL, step
    return len(fills), got_ids.copy()


def test_pool_profile_seeds_the_initial_residency(N, dev, pool_streams):
    """The pool counts every selection it serves; moe_profile_seed turns those counts into the
    initial residency of a new pool (hottest first), which then serves the same steps with no more
    misses than the rank-seeded pool did, under the same LRU policy (checked step by step)."""
    n_slots, steps = 60, 10
    L = PoolLayer(N, dev, layer_id=22, n_slots=n_slots)
    d = L.dims()
    ws = _ws(N, d, dev)
    compute, copy, _ = pool_streams
    ids = torch.zeros((1, L.k), dtype=torch.int32, device=dev)
    y = torch.zeros((1, L.H), dtype=torch.float32, device=dev)
    ref_pool = O.SlotPoolLRU(L.E, L.initial)
    misses1, seen = 0, []
    for s in range(steps):
        n, got = _pool_step(N, L, d, ws, compute, copy, s, s * 2 // steps, ref_pool, dev, ids, y, check=s < 2)
        misses1 += n
        seen.append(got.ravel())
    profile = N.moe_pool_get_profile(L.pool, L.E)
    assert np.array_equal(profile, np.bincount(np.concatenate(seen), minlength=L.E))
    seed = N.moe_profile_seed(profile, n_slots)
    assert np.array_equal(seed, O.profile_seed(profile, n_slots))
    L.close()
    del L
    torch.cuda.empty_cache()
    L2 = PoolLayer(N, dev, layer_id=22, n_slots=n_slots, initial=seed)
    ref2 = O.SlotPoolLRU(L2.E, [int(e) for e in seed])
    misses2 = 0
    for s in range(steps):
        n, _ = _pool_step(N, L2, d, ws, compute, copy, s, s * 2 // steps, ref2, dev, ids, y, check=s < 2)
        misses2 += n
    assert misses2 <= misses1, (misses1, misses2)
    L2.close()


def test_pool_lends_slots_to_a_prefill_workspace(N, dev, pool_streams):
    """The pool's last 16 slots are lent as the workspace of a 256-token prefill of another layer
    (Basalt README, "Prompt chunks": chunk buffers carved from the expert cache's last slots, the
    experts copied back afterwards); the experts wait in host buffers, come back bit-exact, and the
    pool's policy and outputs continue as if nothing had been lent."""
    from layer_fixtures import Layer

    n_slots, n = 60, 16
    L = PoolLayer(N, dev, layer_id=24, n_slots=n_slots)
    B = Layer(MODEL, dev, seed=0, layer=7)
    d = L.dims()
    ws = _ws(N, d, dev)
    compute, copy, _ = pool_streams
    ids = torch.zeros((1, L.k), dtype=torch.int32, device=dev)
    y = torch.zeros((1, L.H), dtype=torch.float32, device=dev)
    ref_pool = O.SlotPoolLRU(L.E, L.initial)
    for s in range(3):
        _pool_step(N, L, d, ws, compute, copy, s, 0, ref_pool, dev, ids, y)
    table = L.table.cpu().numpy()
    lent_experts = [int(np.nonzero(table == slot)[0][0]) for slot in range(n_slots - n, n_slots)]
    bufs = torch.empty((n, L.stride), dtype=torch.uint8, pin_memory=True)
    region = N.moe_pool_lend(L.pool, n, bufs.data_ptr(), stream=compute)
    assert region == L.arena[n_slots - n].data_ptr()
    with pytest.raises(N.MoeError):
        N.moe_pool_arm(L.pool)  # no call while slots are lent
    compute.synchronize()
    t_lent = L.table.cpu().numpy()
    assert all(t_lent[e] == -1 for e in lent_experts)
    for i, e in enumerate(lent_experts[:4]):
        assert np.array_equal(bufs[i, :L.blob].numpy(), L.blob_np(e)), e
    # the region as another layer's prefill workspace
    T = 256
    dB = B.dims()
    assert N.moe_workspace_bytes(dB, T) <= n * L.stride
    wsB = L.arena[n_slots - n:].reshape(-1)
    xB, xB64 = B.x(T, 3, dev)
    yB = torch.zeros((T, B.H), dtype=torch.float32, device=dev)
    with torch.cuda.stream(compute):
        N.moe_workspace_init(wsB, stream=compute)
        N.moe_layer_forward(dB, B.native_weights(), None, xB, T, yB, wsB, stream=compute)
    compute.synchronize()
    assert N.moe_check_device_error(wsB, compute) == 0
    rows = np.array([0, 17, 128, 255])
    ref = B.oracle(xB64[rows])
    ok = ~near_tie_tokens(ref["logits64"], B.k)
    assert np.all(O.per_token_rel_err(yB.cpu().numpy()[rows], ref["y"])[ok] <= Y_TOL)
    N.moe_pool_unlend(L.pool, compute)
    compute.synchronize()
    assert np.array_equal(L.table.cpu().numpy(), ref_pool.table)
    arena = L.arena.cpu().numpy()
    for slot in (n_slots - n, n_slots - 1):
        assert np.array_equal(arena[slot, :L.blob], L.blob_np(lent_experts[slot - (n_slots - n)])), slot
    for s in range(3, 9):
        _pool_step(N, L, d, ws, compute, copy, s, s // 6, ref_pool, dev, ids, y)
    L.close()


def test_pool_copy_failure_is_an_error_not_a_result(N, dev, pool_streams):
    """A failed fill copy (injected on the host: the enqueue reports failure) is never a computed
    layer: serve returns MOE_EFILL and releases the waiting stream with MOE_DERR_FILL set, the
    layer's FFNs report the expert that never arrived (MOE_DERR_NOT_RESIDENT), nothing is placed,
    and the pool serves the next calls as if the failed one had not happened."""
    L = PoolLayer(N, dev, layer_id=30, n_slots=60)
    d = L.dims()
    ws = _ws(N, d, dev)
    compute, copy, _ = pool_streams
    ids = torch.zeros((1, L.k), dtype=torch.int32, device=dev)
    y = torch.zeros((1, L.H), dtype=torch.float32, device=dev)
    ref_pool = O.SlotPoolLRU(L.E, L.initial)
    for s in range(2):
        _pool_step(N, L, d, ws, compute, copy, s, 0, ref_pool, dev, ids, y, check=False)
    failed = False
    for s in range(2, 12):  # topic 1: the first call with a miss fails
        table_before = L.table.cpu().numpy().copy()
        N.moe_pool_debug_fail_copies(L.pool, 0)
        x = L.x(s)[0].to(dev)
        torch.cuda.synchronize()
        bell = N.moe_pool_arm(L.pool)
        with torch.cuda.stream(compute):
            N.moe_layer_forward(d, L.weights(1), L.table, x, 1, y, ws, topk_ids=ids, bell=bell, stream=compute)
        try:
            N.moe_pool_serve(L.pool, ws, copy, L.E)
        except N.MoeError as e:
            assert e.code == N.MOE_EFILL
            failed = True
        compute.synchronize()
        copy.synchronize()
        N.moe_pool_debug_fail_copies(L.pool, -1)
        if failed:
            bits = N.moe_check_device_error(ws)
            assert bits & N.DERR_FILL and bits & N.DERR_NOT_RESIDENT, bits
            assert np.array_equal(L.table.cpu().numpy(), table_before)
            assert np.array_equal(N.moe_pool_get_table(L.pool, L.E), table_before)
            break
        assert N.moe_check_device_error(ws) == 0
        ref_pool.step(ids.cpu().numpy())
    assert failed
    for s2 in range(s + 1, s + 4):
        _pool_step(N, L, d, ws, compute, copy, s2, 1, ref_pool, dev, ids, y)
    L.close()
