"""The C interface on the CPU: the library loads, exports every declared symbol, and
rejects invalid arguments on the host before any HIP call (no GPU needed)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_route.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"MOE_API\s+[\w\s\*]+?\b(moe_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def N():
    from mixture_experts_route_amd import native

    return native


def test_header_declares_the_layer_entry_points():
    names = _declared()
    for n in ("moe_route", "moe_slot_lookup", "moe_expert_ffn_decode", "moe_expert_ffn_prefill",
              "moe_layer_forward", "moe_group_tokens"):
        assert n in names


def test_library_exports_every_declared_symbol(N):
    lib = ctypes.CDLL(N.LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name
    assert sorted(N.EXPORTS) == _declared()


def test_blob_and_workspace_sizes(N):
    d = N.dims(2048, 768, 512, 10, 1)
    assert N.moe_expert_blob_bytes(d) == 2_654_208
    assert N.moe_expert_blob_bytes(N.dims(256, 128, 8, 2, 1)) == 55_296
    assert N.moe_workspace_bytes(d, 1) > 0
    assert N.moe_workspace_bytes(d, 8) >= N.moe_workspace_bytes(d, 1)
    assert N.moe_workspace_bytes(d, 0) == 0


@pytest.mark.parametrize("bad,code", [
    (dict(block=16), -2),             # unsupported block size, refused by name
    (dict(hidden=100), -1),           # not a multiple of 32
    (dict(ffn=32 * 5), -1),           # whole blocks, but not whole groups of four blocks
    (dict(top_k=0), -1),
    (dict(top_k=600), -1),            # k > E
    (dict(n_shared=2), -1),
    (dict(n_experts=2048), -2),       # beyond the selection kernel's 1024
    (dict(top_k=17, n_experts=64), -2),
    (dict(hidden=4096 + 128), -2),    # beyond the 4096-wide rows the kernels are built for
])
def test_invalid_dims_rejected_on_host(N, bad, code):
    args = dict(hidden=2048, ffn=768, n_experts=512, top_k=10, n_shared=1, block=32)
    args.update(bad)
    d = N.dims(**args)
    assert N.moe_expert_blob_bytes(d) == 0
    f = N.raw("moe_route")
    rc = f(ctypes.byref(d), 1 << 20, 1, 1, 1 << 20, 1, None, 1 << 20, 1 << 20, None, 1 << 20, 1 << 30, None)
    assert rc == code


def test_invalid_arguments_rejected_on_host(N):
    d = N.dims(2048, 768, 512, 10, 1)
    route = N.raw("moe_route")
    # NULL x
    assert route(ctypes.byref(d), None, 1, 1, 1 << 20, 1, None, 1 << 20, 1 << 20, None, 1 << 20, 1 << 30, None) == -1
    # bad dtype
    assert route(ctypes.byref(d), 1 << 20, 7, 1, 1 << 20, 1, None, 1 << 20, 1 << 20, None, 1 << 20, 1 << 30, None) == -2
    # workspace missing / misaligned / too small
    assert route(ctypes.byref(d), 1 << 20, 1, 1, 1 << 20, 1, None, 1 << 20, 1 << 20, None, None, 1 << 30, None) == -3
    assert route(ctypes.byref(d), 1 << 20, 1, 1, 1 << 20, 1, None, 1 << 20, 1 << 20, None, (1 << 20) + 8, 1 << 30,
                 None) == -3
    assert route(ctypes.byref(d), 1 << 20, 1, 1, 1 << 20, 1, None, 1 << 20, 1 << 20, None, 1 << 20, 64, None) == -3
    # decode refuses more than MOE_DECODE_MAX_TOKENS bf16 tokens, and more than
    # MOE_DECODE_MAX_TOKENS_NARROW fp32 tokens or bf16 tokens with F > 2048
    dec = N.raw("moe_expert_ffn_decode")
    w = N.moe_layer_weights(1 << 20, 1, None, 1 << 20, 2_654_208, 512, 1 << 24)
    assert dec(ctypes.byref(d), ctypes.byref(w), None, 1 << 20, 1, 17, 1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 30,
               None) == -1
    assert dec(ctypes.byref(d), ctypes.byref(w), None, 1 << 20, 0, 9, 1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 30,
               None) == -1
    d_wide = N.dims(2048, 2304, 512, 10, 1)
    w_wide = N.moe_layer_weights(1 << 20, 1, None, 1 << 20, N.moe_expert_blob_bytes(d_wide) + 4096 -
                                 N.moe_expert_blob_bytes(d_wide) % 4096, 512, 1 << 24)
    assert dec(ctypes.byref(d_wide), ctypes.byref(w_wide), None, 1 << 20, 1, 9, 1 << 20, 1 << 20, 1 << 20, 1 << 20,
               1 << 30, None) == -1
    # slot stride must hold a blob and be 4 KiB aligned
    w_bad = N.moe_layer_weights(1 << 20, 1, None, 1 << 20, 2_654_208 + 512, 512, 1 << 24)
    assert dec(ctypes.byref(d), ctypes.byref(w_bad), None, 1 << 20, 1, 1, 1 << 20, 1 << 20, 1 << 20, 1 << 20,
               1 << 30, None) == -1
    # without a table the arena must hold every expert
    w_few = N.moe_layer_weights(1 << 20, 1, None, 1 << 20, 2_654_208, 100, 1 << 24)
    assert dec(ctypes.byref(d), ctypes.byref(w_few), None, 1 << 20, 1, 1, 1 << 20, 1 << 20, 1 << 20, 1 << 20,
               1 << 30, None) == -1
    # prefill takes bf16 activations only
    pre = N.raw("moe_expert_ffn_prefill")
    assert pre(ctypes.byref(d), ctypes.byref(w), None, 1 << 20, 0, 64, 1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 30,
               None) == -2
    # and n_tokens * H below 2^31 (32-bit activation offsets)
    assert pre(ctypes.byref(d), ctypes.byref(w), None, 1 << 20, 1, 1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20,
               1 << 62, None) == -2


def test_misaligned_activations_rejected_on_host(N):
    """x, y and the router matrix must be 16-byte aligned (the kernels move them with 16-byte vector
    accesses): an offset of one bf16 element is refused with MOE_EINVAL on the host, before any
    pointer is used."""
    d = N.dims(2048, 768, 512, 10, 1)
    fake, odd = 1 << 20, (1 << 20) + 2
    w = N.moe_layer_weights(fake, 1, None, fake, 2_654_208, 512, 1 << 24)
    w_odd_router = N.moe_layer_weights(odd, 1, None, fake, 2_654_208, 512, 1 << 24)
    route = N.raw("moe_route")
    assert route(ctypes.byref(d), odd, 1, 1, fake, 1, None, fake, fake, None, fake, 1 << 30, None) == N.MOE_EINVAL
    assert route(ctypes.byref(d), fake, 1, 1, odd, 1, None, fake, fake, None, fake, 1 << 30, None) == N.MOE_EINVAL
    dec = N.raw("moe_expert_ffn_decode")
    pre = N.raw("moe_expert_ffn_prefill")
    lay = N.raw("moe_layer_forward")
    for x, y in ((odd, fake), (fake, odd)):
        assert dec(ctypes.byref(d), ctypes.byref(w), None, x, 1, 1, fake, fake, y, fake, 1 << 30, None) == N.MOE_EINVAL
        assert pre(ctypes.byref(d), ctypes.byref(w), None, x, 1, 64, fake, fake, y, fake, 1 << 30, None) == N.MOE_EINVAL
        assert lay(ctypes.byref(d), ctypes.byref(w), None, None, x, 1, 1, y, None, None, fake, 1 << 30,
                   None) == N.MOE_EINVAL
    assert lay(ctypes.byref(d), ctypes.byref(w_odd_router), None, None, fake, 1, 1, fake, None, None, fake, 1 << 30,
               None) == N.MOE_EINVAL


@pytest.mark.parametrize("n_tokens", [0, -1])
def test_empty_batch_rejected_on_host(N, n_tokens):
    """An empty (or negative) token count is refused with MOE_EINVAL by every entry point that takes
    one, before any pointer is used (the pointers here are never dereferenced)."""
    d = N.dims(2048, 768, 512, 10, 1)
    fake = 1 << 20
    w = N.moe_layer_weights(fake, 1, None, fake, 2_654_208, 512, 1 << 24)
    wp = ctypes.byref(w)
    calls = {
        "moe_route": (ctypes.byref(d), fake, 1, n_tokens, fake, 1, None, fake, fake, None, fake, 1 << 30, None),
        "moe_slot_lookup": (ctypes.byref(d), fake, 512, fake, n_tokens, fake, fake, fake, None, fake, 1 << 30, None),
        "moe_group_tokens": (ctypes.byref(d), fake, n_tokens, fake, fake, fake, fake, 1 << 30, None),
        "moe_expert_ffn_decode": (ctypes.byref(d), wp, None, fake, 1, n_tokens, fake, fake, fake, fake, 1 << 30, None),
        "moe_expert_ffn_prefill": (ctypes.byref(d), wp, None, fake, 1, n_tokens, fake, fake, fake, fake, 1 << 30,
                                   None),
        "moe_layer_forward": (ctypes.byref(d), wp, None, None, fake, 1, n_tokens, fake, None, None, fake, 1 << 30,
                              None),
    }
    for name, args in calls.items():
        assert N.raw(name)(*args) == N.MOE_EINVAL, name


def test_strerror(N):
    for c in range(-6, 1):
        assert isinstance(N.strerror(c), str) and N.strerror(c)
    assert N.strerror(42) == "unknown status code"


def test_pool_create_rejects_inconsistent_residency(N):
    """The host pool service refuses, before touching any memory, a slot list with a repeated or
    out-of-range expert and an expert with no host home or with two homes (exclusive tiers)."""
    d = N.dims(2048, 768, 512, 10, 1)
    stride = 648 * 4096
    fake = 1 << 30  # never dereferenced: every case fails validation first

    def create(initial, homes):
        init = (ctypes.c_int32 * len(initial))(*initial)
        hh = (ctypes.c_void_p * 512)(*[h if h else None for h in homes])
        out = ctypes.c_void_p()
        return N.raw("moe_pool_create")(ctypes.byref(d), fake, stride, len(initial), fake, init, hh, fake, n_spares,
                                        fake, fake, fake, fake, ctypes.byref(out))

    n_spares = 2

    homes = [0 if e < 4 else fake + 4096 * e for e in range(512)]
    assert create([0, 1, 2, 2], homes) == -1            # expert 2 in two slots
    assert create([0, 1, 2, 600], homes) == -1          # id out of range
    assert create([0, 1, 2, 3], [0] * 512) == -1        # experts 4.. have no home
    both = list(homes)
    both[0] = fake
    assert create([0, 1, 2, 3], both) == -1             # expert 0 in a slot and on the host
    for n_spares in (0, 65):                            # spare count outside 1..MOE_POOL_MAX_SPARES
        assert create([0, 1, 2, 3], homes) == -1
    assert N.raw("moe_pool_arm")(None, None) == -1
    assert N.raw("moe_pool_serve")(None, None, None, None, None, None, 0) == -1


def test_header_blob_layout_packs_what_the_oracle_reads():
    """One expert blob packed by following the header's text alone (written here from the sentences
    it states, not from the oracle), then read by the oracle: every code and scale lands where the
    header says.  The header must still state the rule this packer follows."""
    import numpy as np

    from oracle import moe_oracle as O

    text = " ".join(" ".join(re.sub(r"^\s*\*", "", ln) for ln in open(HEADER).read().splitlines()).split())
    for phrase in ("the 64-byte record at byte 64 * (c * R + r) of the section",
                   "Word 4g + i (g, i = 0..3) holds slice g of block i",
                   "input 128c + 32i + 8g + 2j in bits 4j..4j+3",
                   "input 128c + 32i + 8g + 2j + 1 in bits 16+4j..16+4j+3",
                   "at byte 8 * (c * R + r) of the scale section",
                   "[gate codes F*H/2][up codes F*H/2][down codes H*F/2]",
                   "[gate scales F*H/16][up scales F*H/16][down scales H*F/16]"):
        assert phrase in text, phrase

    H, F = 256, 128
    rng = np.random.default_rng(11)
    u = {m: rng.integers(0, 16, size=(R, K)) for m, (R, K) in {"gate": (F, H), "up": (F, H), "down": (H, F)}.items()}
    sc = {m: rng.integers(0x0400, 0x3C00, size=(R, K // 32)).astype(np.uint16) for m, (R, K) in
          {"gate": (F, H), "up": (F, H), "down": (H, F)}.items()}

    def pack_codes(codes):
        R, K = codes.shape
        out = bytearray(R * K // 2)
        for c in range(K // 128):
            for r in range(R):
                rec = 64 * (c * R + r)
                for g in range(4):
                    for i in range(4):
                        word = 0
                        for j in range(4):
                            word |= int(codes[r, 128 * c + 32 * i + 8 * g + 2 * j]) << (4 * j)
                            word |= int(codes[r, 128 * c + 32 * i + 8 * g + 2 * j + 1]) << (16 + 4 * j)
                        out[rec + 4 * (4 * g + i): rec + 4 * (4 * g + i) + 4] = word.to_bytes(4, "little")
        return bytes(out)

    def pack_scales(s):
        R, nb = s.shape
        out = bytearray(R * nb * 2)
        for c in range(nb // 4):
            for r in range(R):
                for i in range(4):
                    out[8 * (c * R + r) + 2 * i: 8 * (c * R + r) + 2 * i + 2] = int(s[r, 4 * c + i]).to_bytes(2, "little")
        return bytes(out)

    blob = b"".join([pack_codes(u["gate"]), pack_codes(u["up"]), pack_codes(u["down"]),
                     pack_scales(sc["gate"]), pack_scales(sc["up"]), pack_scales(sc["down"])])
    assert len(blob) == O.blob_layout(H, F)["total"][1]
    Wg, Wu, Wd = O.expert_weights(np.frombuffer(blob, np.uint8), H, F)
    for m, W in (("gate", Wg), ("up", Wu), ("down", Wd)):
        s = sc[m].view(np.float16).astype(np.float64)
        want = (u[m] - 8).astype(np.float64) * np.repeat(s, 32, axis=1)
        assert np.array_equal(W, want), m


def test_doorbell_only_with_decode_sized_calls(N):
    """A doorbell publishes the step's selections for the pool's recency policy: the calls refuse it
    (MOE_EUNSUPPORTED, nothing enqueued) above MOE_DECODE_MAX_TOKENS tokens."""
    d = N.dims(2048, 768, 512, 10, 1)
    fake = 1 << 20
    bell = N.moe_doorbell(fake, fake, fake, 1, fake)
    w = N.moe_layer_weights(fake, 1, None, fake, 2_654_208, 512, 1 << 24)
    T = N.MOE_DECODE_MAX_TOKENS + 1
    assert N.raw("moe_slot_lookup")(ctypes.byref(d), fake, 512, fake, T, fake, fake, fake, ctypes.byref(bell), fake,
                                    1 << 30, None) == N.MOE_EUNSUPPORTED
    assert N.raw("moe_layer_forward")(ctypes.byref(d), ctypes.byref(w), fake, ctypes.byref(bell), fake, 1, T, fake,
                                      None, None, fake, 1 << 30, None) == N.MOE_EUNSUPPORTED


def test_profile_seed_matches_the_oracle(N):
    """moe_profile_seed (host code of the library) against the oracle's rule, ties included; bad
    sizes refused."""
    import numpy as np

    from oracle import moe_oracle as O

    rng = np.random.default_rng(3)
    for E, n in ((512, 60), (512, 240), (64, 64), (8, 1)):
        counts = rng.integers(0, 6, size=E).astype(np.int64)  # many equal counts
        assert np.array_equal(N.moe_profile_seed(counts, n), O.profile_seed(counts, n))
    f = N.raw("moe_profile_seed")
    c = (ctypes.c_int64 * 4)(1, 2, 3, 4)
    out = (ctypes.c_int32 * 8)()
    assert f(c, 4, 5, out) == N.MOE_EINVAL and f(c, 4, 0, out) == N.MOE_EINVAL and f(None, 4, 2, out) == N.MOE_EINVAL


def test_format_sizes_and_refusal(N):
    """Blob sizes per weight format (the affine format adds three fp16 min planes); an unknown
    format is refused by name (MOE_EUNSUPPORTED) before anything else."""
    assert N.moe_expert_blob_bytes(N.dims(2048, 768, 512, 10, 1, format=N.MOE_FMT_CB4)) == 2_654_208
    assert N.moe_expert_blob_bytes(N.dims(2048, 768, 512, 10, 1, format=N.MOE_FMT_AFFINE4)) == 2_654_208 + 3 * 98_304
    d = N.dims(2048, 768, 512, 10, 1, format=3)
    assert N.moe_expert_blob_bytes(d) == 0
    f = N.raw("moe_route")
    assert f(ctypes.byref(d), 1 << 20, 1, 1, 1 << 20, 1, None, 1 << 20, 1 << 20, None, 1 << 20, 1 << 30, None) == \
        N.MOE_EUNSUPPORTED


def test_prefill_plan_get_and_force(N):
    """The plan of a prefill call: the table (or default) plan, pipelined kernels only where they are
    built (the model's widths; the affine format not on the 128-row kernel); a forced plan overrides
    it until cleared; invalid plans are refused."""
    d = N.dims(2048, 768, 512, 10, 1)
    p = N.moe_prefill_plan_get(d, 4096)
    assert p.item_rows in (64, 128) and p.router_rows in (32, 64)
    wide = N.moe_prefill_plan_get(N.dims(4096, 1536, 64, 8, 1), 4096)
    assert wide.gate_up_kernel == N.MOE_GEMM_GENERAL and wide.down_kernel == N.MOE_GEMM_GENERAL
    # (256 experts: no table row, so the default plan, the 128-row pipelined kernel) the codebook
    # format runs it; the affine format's min records do not fit it, and the general kernel runs
    cb = N.moe_prefill_plan_get(N.dims(2048, 768, 256, 10, 1, format=N.MOE_FMT_CB4), 4096)
    assert cb.gate_up_kernel == N.MOE_GEMM_PIPE128 and cb.down_kernel == N.MOE_GEMM_PIPE128
    af = N.moe_prefill_plan_get(N.dims(2048, 768, 256, 10, 1, format=N.MOE_FMT_AFFINE4), 4096)
    assert af.gate_up_kernel == N.MOE_GEMM_GENERAL and af.down_kernel == N.MOE_GEMM_GENERAL
    # a measured row of the table for the affine format names a kernel it runs
    af_t = N.moe_prefill_plan_get(N.dims(2048, 768, 512, 10, 1, format=N.MOE_FMT_AFFINE4), 4096)
    assert af_t.gate_up_kernel != N.MOE_GEMM_PIPE128 and af_t.down_kernel != N.MOE_GEMM_PIPE128
    N.moe_debug_force_prefill_plan(N.moe_prefill_plan(64, 1, 2, 64))
    try:
        f = N.moe_prefill_plan_get(d, 100)
        assert (f.item_rows, f.gate_up_kernel, f.down_kernel, f.router_rows) == (64, 1, 2, 64)
    finally:
        N.moe_debug_force_prefill_plan(None)
    assert N.moe_prefill_plan_get(d, 4096).item_rows == p.item_rows
    for bad in ((96, 0, 0, 32), (128, 1, 0, 32), (64, 3, 0, 32), (64, 0, 0, 48)):
        with pytest.raises(N.MoeError):
            N.moe_debug_force_prefill_plan(N.moe_prefill_plan(*bad))


def _tuned_rows():
    path = os.path.join(ROOT, "mixture_experts_route_amd", "csrc", "tuned_plans.inc")
    pat = re.compile(r"^\{(\d+), (\d+), (\d+), (\d+), (\d+), (\d+), (\d+), \{(\d+), (\d+), (\d+), (\d+)\}\},")
    return [tuple(int(v) for v in m.groups()) for m in map(pat.match, open(path)) if m]


def test_tuned_plan_table_rows_are_what_the_library_returns(N):
    """Every row of the measured plan table (a range of token counts for one layer shape and weight
    format) is the plan the library picks at the range's first, middle and last token count; the rows
    of one shape and format cover 17 tokens upwards without gap or overlap; below the table, and for a
    shape with no row, the default plan applies (its router GEMM switches to 64-row works at 3,072
    tokens with the pipelined router kernel)."""
    rows = _tuned_rows()
    assert len(rows) >= 9
    groups = {}
    for r in rows:
        groups.setdefault(r[:5], []).append(r)
    for key, rs in groups.items():
        rs.sort(key=lambda r: r[5])
        assert rs[0][5] == 17 and rs[-1][6] == 2147483647, key
        for a, b in zip(rs, rs[1:]):
            assert b[5] == a[6] + 1, (key, a, b)
    for H, F, E, k, fmt, lo, hi, item_rows, gu, dn, rr in rows:
        d = N.dims(H, F, E, k, 1, format=fmt)
        for T in sorted({lo, (lo + min(hi, 1 << 19)) // 2, min(hi, 1 << 19)}):
            p = N.moe_prefill_plan_get(d, T)
            assert (p.item_rows, p.gate_up_kernel, p.down_kernel, p.router_rows) == (item_rows, gu, dn, rr), (fmt, T)
    below = N.moe_prefill_plan_get(N.dims(2048, 768, 512, 10, 1), 16)
    assert (below.item_rows, below.gate_up_kernel, below.down_kernel, below.router_rows) == (
        128, N.MOE_GEMM_PIPE128, N.MOE_GEMM_PIPE128, 32)
    d256 = N.dims(2048, 768, 256, 10, 1)
    assert N.moe_prefill_plan_get(d256, 3071).router_rows == 32
    assert N.moe_prefill_plan_get(d256, 3072).router_rows == 64
