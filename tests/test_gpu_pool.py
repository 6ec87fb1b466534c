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

    def __init__(self, N, dev, layer_id, n_slots, topics=2, n_spares=1):
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
        # initial residency: the hottest experts of topic 0, hottest first
        self.initial = [int(e) for e in np.argsort(self.ranks[0], kind="stable")[:n_slots]]
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
def test_pool_decode_steps_match_oracle_policy_and_outputs(N, dev, n_spares, two_streams):
    """One copy stream and one spare buffer, or separate device->host and host->device streams
    with one spare (every copy out waits, by event, for the copy in that last read its buffer) or
    four (the copies of the two directions overlap): same fills, tables and outputs, and afterwards
    every evicted expert's bytes sit in the host buffer the swap rule gives it."""
    L = PoolLayer(N, dev, layer_id=20, n_slots=60, n_spares=n_spares)
    d = L.dims()
    ws = _ws(N, d, dev)
    compute, copy = N.new_stream(), N.new_stream()
    h2d = N.new_stream() if two_streams else None
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
    N.free_stream(compute)
    N.free_stream(copy)
    if h2d is not None:
        N.free_stream(h2d)
    L.close()


def test_pool_all_resident_never_misses(N, dev):
    """Every expert in a slot: the check kernel releases the stream itself on every call."""
    L = PoolLayer(N, dev, layer_id=3, n_slots=512)
    d = L.dims()
    ws = _ws(N, d, dev)
    compute, copy = N.new_stream(), N.new_stream()
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
    N.free_stream(compute)
    N.free_stream(copy)
    L.close()


def test_pool_serve_without_doorbell_times_out_and_flags(N, dev):
    """Host-forced failure: the call is armed but the layer is launched without the doorbell, so
    nothing rings; serve gives up after its timeout, releases the ready word and flags the
    workspace.  No kernel waits on anything here."""
    L = PoolLayer(N, dev, layer_id=40, n_slots=60)
    d = L.dims()
    ws = _ws(N, d, dev)
    copy = N.new_stream()
    N.moe_pool_arm(L.pool)
    with pytest.raises(N.MoeError) as ei:
        N.moe_pool_serve(L.pool, ws, copy, L.E, timeout_us=200_000)
    assert ei.value.code == N.MOE_EFILL
    copy.synchronize()
    bits = ctypes_bits(N, ws)
    assert bits & N.DERR_FILL
    assert int(L.ready[0].item()) == 1
    N.free_stream(copy)
    L.close()


def ctypes_bits(N, ws):
    import ctypes

    b = ctypes.c_int32()
    N.raw("moe_check_device_error")(ws.data_ptr(), None, ctypes.byref(b))
    return b.value
