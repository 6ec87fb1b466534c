"""Pins of the CPU oracle to facts fixed outside itself (CPU only).

Each test checks the oracle against hand-encoded bytes, closed forms, brute force
on tiny inputs, identities of the mathematics, or an independent library routine,
so that a dropped term, a wrong sign, index or nibble position, or a transposed
operand in the oracle fails at least one of them.
"""

import itertools
import math
import os
from collections import OrderedDict
from fractions import Fraction

import numpy as np
import pytest

from oracle import moe_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield [p.strip() for p in line.split(";")]


# ----------------------------------------------------------------------------- dequant

def _codes_field(field):
    parts = field.split()
    if parts[0] != "fill":
        return [int(c) for c in parts]
    u = [int(parts[1])] * 128
    for p in parts[2:]:
        e, v = p.split("=")
        u[int(e)] = int(v)
    return u


def test_dequant_hand_encoded_groups():
    n = 0
    for name, bhex, shex, svals, codes in _rows("dequant_groups.txt"):
        code_bytes = np.array([int(b, 16) for b in bhex.split()], dtype=np.uint8)
        scale_bits = [int(h, 16) for h in shex.split()]
        scales = [Fraction(v) for v in svals.split()]
        u = _codes_field(codes)
        assert len(code_bytes) == 64 and len(u) == 128 and len(scale_bits) == 4 == len(scales)
        # fp16 decoding of the scales is exact, subnormals and sign included
        assert list(O.fp16_codes_to_f64(np.array(scale_bits, np.uint16))) == [float(v) for v in scales], name
        scale_bytes = np.array(scale_bits, dtype=np.uint16).view(np.uint8)
        assert list(O.decode_codes(code_bytes, 1, 128)[0]) == u, name
        w = O.dequant(code_bytes, scale_bytes, 1, 128)[0]
        want = [float((ui - 8) * scales[e // 32]) for e, ui in enumerate(u)]
        assert list(w) == want, name
        n += 1
    assert n >= 14


def test_dequant_rows_and_groups_are_independent():
    # two rows of two groups, stored group-major: record (group c, row r) at 64 (2 c + r).
    # Each block takes its own scale; groups and rows do not mix.  No two records agree, so a
    # row-major reading fails.
    ramp = [0x20, 0x64, 0x31, 0x75] * 4 + [0xA8, 0xEC, 0xB9, 0xFD] * 4
    ramp = ramp * 2  # slices 0..3 of the four blocks (see dequant_groups.txt)
    zero = [0x88] * 64
    probe = list(zero)
    probe[20] = 0x8A  # element 40 of the group = 10 (dequant_groups.txt, only_el40)
    # records: (c0, r0) ramp, (c0, r1) zero, (c1, r0) probe, (c1, r1) ramp
    code_bytes = np.array(ramp + zero + probe + ramp, dtype=np.uint8)
    # scale records (c, r) of four fp16 each, in the same order
    scales = np.array([0x3C00, 0x4000, 0x3800, 0x4400] + [0x3C00] * 4 + [0x4400] * 4 + [0x4000] * 4,
                      dtype=np.uint16)  # (1, 2, 0.5, 4), 1..., 4..., 2...
    w = O.dequant(code_bytes, scales.view(np.uint8), 2, 256)
    q = np.array([(e % 16) - 8 for e in range(128)], dtype=np.float64)
    s0 = np.repeat([1.0, 2.0, 0.5, 4.0], 32)
    assert np.array_equal(w[0, :128], q * s0)
    want01 = np.zeros(128)
    want01[40] = (10 - 8) * 4.0
    assert np.array_equal(w[0, 128:], want01)
    assert np.array_equal(w[1, :128], np.zeros(128))
    assert np.array_equal(w[1, 128:], q * 2.0)


def test_dequant_group_major_three_rows():
    # three rows of one group each: records are consecutive rows, scales likewise
    zero = [0x88] * 64
    probe = list(zero)
    probe[20] = 0x8A  # element 40 of the group = 10 (dequant_groups.txt, only_el40)
    code_bytes = np.array(zero + probe + zero, dtype=np.uint8)
    scales = np.array([0x3C00] * 4 + [0x3C00, 0x4400, 0x3C00, 0x3C00] + [0x3C00] * 4, dtype=np.uint16)
    w = O.dequant(code_bytes, scales.view(np.uint8), 3, 128)
    want = np.zeros((3, 128))
    want[1, 40] = (10 - 8) * 4.0  # block 1 of row 1 has scale 4
    assert np.array_equal(w, want)


def test_blob_layout_sizes():
    # model shape: 3 matrices x (786,432 code bytes + 98,304 scale bytes) = 2,654,208 = 648 x 4 KiB
    lay = O.blob_layout(2048, 768)
    assert lay["total"][1] == 2_654_208 == 648 * 4096
    assert lay["gate_scales"][0] == 3 * 786_432
    assert O.blob_layout(256, 128)["total"][1] == 55_296


# ----------------------------------------------------------------------------- router

def test_router_one_hot_and_zero():
    rng = np.random.default_rng(3)
    E, H = 16, 64
    Wr = rng.standard_normal((E, H)).astype(np.float32).astype(np.float64)
    bias = rng.standard_normal(E).astype(np.float32)
    for h in (0, 17, 63):
        x = np.zeros((1, H))
        x[0, h] = 1.0
        assert np.array_equal(O.router_logits(x, Wr)[0], Wr[:, h])
    assert np.array_equal(O.router_logits(np.zeros((2, H)), Wr, bias), np.tile(bias.astype(np.float64), (2, 1)))


def test_select_closed_form_k10_of_512():
    rows = list(_rows("topk_closed_form.txt"))
    k = int([r for r in rows if r[0] == "k"][0][1])
    E = int([r for r in rows if r[0] == "E"][0][1])
    logits = -np.arange(E, dtype=np.float32)[None, :]
    ids = O.select_topk(logits, k)
    assert list(ids[0]) == list(range(k))
    w = O.route_weights(logits, ids)[0]
    for _, j, val in [r for r in rows if r[0] == "w"]:
        assert w[int(j)] == pytest.approx(float(val), rel=1e-14)
    assert abs(w.sum() - 1.0) < 1e-15


def test_select_all_equal_takes_lowest_ids():
    logits = np.zeros((3, 512), dtype=np.float32)
    ids = O.select_topk(logits, 10)
    assert (ids == np.arange(10)).all()
    w = O.route_weights(logits, ids)
    assert np.allclose(w, 0.1, rtol=0, atol=1e-16)


def _brute_topk(l, k):
    """The unique k-subset S with l_i > l_j, or l_i == l_j and i < j, for i in S, j not in S."""
    E = len(l)
    found = []
    for S in itertools.combinations(range(E), k):
        rest = [j for j in range(E) if j not in S]
        if all(l[i] > l[j] or (l[i] == l[j] and i < j) for i in S for j in rest):
            found.append(S)
    assert len(found) == 1
    return sorted(found[0], key=lambda i: (-l[i], i))


def test_select_matches_brute_force_with_ties():
    rng = np.random.default_rng(5)
    for trial in range(60):
        E = int(rng.integers(3, 9))
        k = int(rng.integers(1, E + 1))
        l = rng.integers(-3, 4, size=E).astype(np.float32)  # many ties
        ids = O.select_topk(l[None, :], k)[0]
        assert list(ids) == _brute_topk(list(l), k), (l, k)


def test_weights_equal_full_softmax_renormalised():
    rng = np.random.default_rng(7)
    l = (rng.standard_normal((8, 64)) * 2).astype(np.float32)
    ids = O.select_topk(l, 6)
    w = O.route_weights(l, ids)
    full = np.exp(l.astype(np.float64) - l.max(axis=1, keepdims=True))
    full /= full.sum(axis=1, keepdims=True)
    sel = np.take_along_axis(full, ids.astype(np.int64), axis=1)
    assert np.allclose(w, sel / sel.sum(axis=1, keepdims=True), rtol=1e-13, atol=0)
    # selected logits dominate the rest
    for t in range(8):
        rest = np.setdiff1d(np.arange(64), ids[t])
        assert l[t, ids[t]].min() >= l[t, rest].max()
        assert np.all(np.diff(w[t]) <= 0)


# ----------------------------------------------------------------------------- FFN

def _hand_blob():
    H, F = 128, 128
    lay = O.blob_layout(H, F)
    blob = np.zeros(lay["total"][1], dtype=np.uint8)
    for name in ("gate_codes", "up_codes", "down_codes"):
        off, sz = lay[name]
        blob[off:off + sz] = 0x88
    for name in ("gate_scales", "up_scales", "down_scales"):
        off, sz = lay[name]
        blob[off:off + sz].view(np.uint16)[:] = 0x3C00
    row_bytes = {"gate": H // 2, "up": H // 2, "down": F // 2}
    row_blocks = {"gate": H // 32, "up": H // 32, "down": F // 32}
    # element -> (byte within the row, nibble shift), hand-derived for the elements used
    pos = {0: (0, 0), 1: (2, 0), 5: (3, 0)}
    expect = {}
    for r in _rows("hand_expert.txt"):
        if r[0] == "expect":
            expect[int(r[1])] = float(r[2])
            continue
        mat, row, el, u, sbits = r[0], int(r[1]), int(r[2]), int(r[3]), int(r[4], 16)
        coff = lay[mat + "_codes"][0] + row * row_bytes[mat]
        b, sh = pos[el]
        blob[coff + b] = (blob[coff + b] & (0xF0 if sh == 0 else 0x0F)) | (u << sh)
        soff = lay[mat + "_scales"][0] + row * row_blocks[mat] * 2
        blob[soff:soff + 2].view(np.uint16)[0] = sbits
    return blob, H, F, expect


def test_ffn_hand_built_expert_closed_form():
    blob, H, F, expect = _hand_blob()
    Wg, Wu, Wd = O.expert_weights(blob, H, F)
    x = np.zeros((1, H))
    x[0, 0] = 2.0
    y = O.swiglu_ffn(Wg, Wu, Wd, x)[0]
    want = np.zeros(H)
    for o, v in expect.items():
        want[o] = v
    assert np.allclose(y, want, rtol=1e-15, atol=0), (np.nonzero(y), y[list(expect)])
    # the same expert through the whole layer (k = 1, no shared expert): weight exactly 1
    Wr = np.zeros((4, H))
    Wr[2, 0] = 1.0
    out = O.moe_layer(x, Wr, None, 1, lambda e: blob, None, H, F)
    assert list(out["ids"][0]) == [2] and out["w"][0, 0] == 1.0
    assert np.allclose(out["y"][0], want, rtol=1e-15, atol=0)


def test_silu_spot_values():
    assert O.silu(np.array([1.0]))[0] == pytest.approx(0.7310585786300049, rel=1e-15)
    assert O.silu(np.array([0.0]))[0] == 0.0
    assert O.silu(np.array([-40.0]))[0] == pytest.approx(-40.0 * math.exp(-40.0), rel=1e-12)


def _tiny_layer(seed, T=4, E=8, H=256, F=128, k=2, shared=True):
    rng = np.random.default_rng(seed)
    blobs = [rng.integers(0, 256, size=O.blob_layout(H, F)["total"][1], dtype=np.uint8) for _ in range(E + 1)]
    for b in blobs:  # sane scales: fp16 |N(0, 0.02)|
        lay = O.blob_layout(H, F)
        off = lay["gate_scales"][0]
        n = (len(b) - off) // 2
        b[off:] = np.abs(rng.standard_normal(n) * 0.02).astype(np.float16).view(np.uint8)
    Wr = (rng.standard_normal((E, H)) * 0.1).astype(np.float32).astype(np.float64)
    x = rng.standard_normal((T, H)).astype(np.float32).astype(np.float64)
    return x, Wr, blobs, (blobs[E] if shared else None)


def test_layer_matches_fp64_dense_brute_force():
    """Every expert computed densely, weighted by a dense gate vector zero off the top-k."""
    H, F, E, k = 256, 128, 8, 2
    x, Wr, blobs, sh = _tiny_layer(11)
    out = O.moe_layer(x, Wr, None, k, lambda e: blobs[e], sh, H, F)
    T = x.shape[0]
    y = np.zeros((T, H))
    l = x @ Wr.T
    for t in range(T):
        # brute-force selection on fp32 logits, weights by the plain softmax formula
        l32 = l[t].astype(np.float32)
        S = _brute_topk(list(l32), k)
        dense = np.zeros(E)
        z = sum(math.exp(float(l32[i]) - float(l32[S[0]])) for i in S)
        for i in S:
            dense[i] = math.exp(float(l32[i]) - float(l32[S[0]])) / z
        for e in range(E + 1):
            Wg, Wu, Wd = O.expert_weights(blobs[e], H, F)
            ge = sum(Wg[:, c] * x[t, c] for c in range(H))  # column-sum formulation
            ue = sum(Wu[:, c] * x[t, c] for c in range(H))
            he = ge / (1 + np.exp(-ge)) * ue
            ye = sum(Wd[:, r] * he[r] for r in range(F))
            y[t] += (dense[e] if e < E else 1.0) * ye
    assert np.allclose(out["y"], y, rtol=1e-10, atol=1e-10)


def test_layer_zero_input_gives_zero():
    x, Wr, blobs, sh = _tiny_layer(13)
    out = O.moe_layer(np.zeros_like(x), Wr, None, 2, lambda e: blobs[e], sh, 256, 128)
    assert np.array_equal(out["y"], np.zeros_like(out["y"]))


def test_layer_top1_without_shared_is_one_expert():
    H, F = 256, 128
    x, Wr, blobs, _ = _tiny_layer(17, shared=False)
    out = O.moe_layer(x, Wr, None, 1, lambda e: blobs[e], None, H, F)
    assert np.all(out["w"] == 1.0)
    for t in range(x.shape[0]):
        e = int(np.argmax((x[t] @ Wr.T).astype(np.float32)))
        Wg, Wu, Wd = O.expert_weights(blobs[e], H, F)
        # equal up to the BLAS's own rounding order (one row vs a batch of rows)
        assert np.allclose(out["y"][t], O.swiglu_ffn(Wg, Wu, Wd, x[t:t + 1])[0], rtol=1e-13, atol=1e-13)


def test_all_resident_equals_slot_pool_bitwise():
    H, F, E = 256, 128, 8
    x, Wr, blobs, sh = _tiny_layer(19)
    direct = O.moe_layer(x, Wr, None, 2, lambda e: blobs[e], sh, H, F)
    # the same experts scattered over a larger arena through a slot table
    rng = np.random.default_rng(1)
    n_slots = 13
    slots = rng.permutation(n_slots)[:E]
    arena = [None] * n_slots
    for e in range(E):
        arena[slots[e]] = blobs[e].copy()
    table = np.full(E, -1)
    table[np.arange(E)] = slots
    pooled = O.moe_layer(x, Wr, None, 2, lambda e: arena[table[e]], sh, H, F)
    assert np.array_equal(direct["y"], pooled["y"])


# ----------------------------------------------------------------------------- residency

def test_slot_lookup_identity_and_set_difference():
    ids = np.array([[3, 1, 7], [7, 0, 2]])
    slots, miss = O.slot_lookup(np.arange(8), ids)
    assert np.array_equal(slots, ids) and miss.size == 0
    rng = np.random.default_rng(2)
    for _ in range(50):
        E = 64
        table = np.where(rng.random(E) < 0.6, rng.permutation(E), -1)
        ids = np.stack([rng.choice(E, 10, replace=False) for _ in range(int(rng.integers(1, 9)))])
        slots, miss = O.slot_lookup(table, ids)
        assert np.array_equal(slots, table[ids])
        assert list(miss) == sorted(set(ids.ravel().tolist()) - set(np.nonzero(table >= 0)[0].tolist()))


def _lru_recency_list(n_experts, initial, steps):
    """LRU as a recency-ordered list of slots (an independent formulation)."""
    S = len(initial)
    where = {e: s for s, e in enumerate(initial)}
    holder = list(initial)
    order = OrderedDict((s, None) for s in reversed(range(S)))  # least recent first
    log = []
    for ids in steps:
        selected = set(int(e) for e in np.ravel(ids))
        misses = sorted(e for e in selected if e not in where)
        fills = []
        for e in misses:
            victim = next(s for s in order if holder[s] not in selected)
            old = holder[victim]
            del where[old]
            where[e] = victim
            holder[victim] = e
            fills.append((e, victim, old))
        for e in np.ravel(ids):
            s = where[int(e)]
            order.move_to_end(s)
        log.append((misses, fills))
    return log


def test_slot_pool_lru_matches_recency_list():
    rng = np.random.default_rng(23)
    for trial in range(30):
        E = int(rng.integers(12, 40))
        S = int(rng.integers(4, 10))
        k = int(rng.integers(1, min(S, 4) + 1))
        T = int(rng.integers(1, 3))
        if T * k > S:
            T = 1
        initial = list(rng.permutation(E)[:S])
        steps = [np.stack([rng.choice(E, k, replace=False) for _ in range(T)]) for _ in range(40)]
        pool = O.SlotPoolLRU(E, initial)
        got = [pool.step(s) for s in steps]
        want = _lru_recency_list(E, initial, steps)
        assert got == want
        # exclusive tiers: every expert is in exactly one place
        resident = set(np.nonzero(pool.table >= 0)[0].tolist())
        assert len(resident) == S and sorted(pool.table[list(resident)]) == list(range(S))


# ----------------------------------------------------------------------------- grouping

def test_group_pairs_matches_stable_argsort():
    rng = np.random.default_rng(29)
    for n, E in ((1, 1), (40, 8), (4096, 513), (3000, 5)):
        ids = rng.integers(0, E, size=n)
        counts, offsets, perm = O.group_pairs(ids, E)
        assert np.array_equal(perm, np.argsort(ids, kind="stable"))
        assert np.array_equal(counts, np.bincount(ids, minlength=E))
        assert offsets[0] == 0 and offsets[-1] == n
    counts, offsets, perm = O.group_pairs(np.zeros(0, dtype=np.int64), 4)
    assert counts.sum() == 0 and perm.size == 0 and list(offsets) == [0] * 5


# ----------------------------------------------------------------------------- comparison helpers

def _frac_or_pow(s):
    """'1/128', '2^-133', '127*2^-133', '-0' -> exact value (Fraction, or the float -0.0)."""
    s = s.strip()
    if s == "-0":
        return -0.0
    sign = -1 if s.startswith("-") else 1
    s = s.lstrip("-")
    if "^" in s:
        mant, _, rest = s.rpartition("*") if "*" in s else ("1", None, s)
        base, exp = rest.split("^")
        return sign * Fraction(int(mant)) * Fraction(int(base)) ** int(exp)
    return sign * Fraction(s)


def test_bf16_codes_hand_decoded():
    rows = list(_rows("bf16_codes.txt"))
    codes = np.array([int(r[0], 16) for r in rows], dtype=np.uint16)
    got = O.bf16_codes_to_f64(codes)
    for (code, val, _), g in zip(rows, got):
        want = _frac_or_pow(val)
        assert g == float(want), (code, g, want)
        assert math.copysign(1.0, g) == math.copysign(1.0, float(want)), code
    # the same codes given as signed 16-bit patterns decode the same
    assert np.array_equal(O.bf16_codes_to_f64(codes.view(np.int16)), got)
    # a plausible mistake (a shift by 15 instead of 16) fails the fixture
    wrong = (codes.astype(np.uint32) << np.uint32(15)).view(np.float32).astype(np.float64)
    assert not np.array_equal(wrong, got)


def test_topk_gap_hand_worked():
    rows = list(_rows("topk_gap.txt"))
    assert len(rows) >= 8
    for lg, k, want in rows:
        l = np.array([[float(v) for v in lg.split()]])
        got = O.topk_gap(l, int(k))[0]
        assert got == float(want), (lg, k, got)
    # the off-by-one variants differ from the fixture on at least one row each
    def shifted(l, k, d):
        s = -np.sort(-l, axis=1)
        i = k - 1 + d
        if i + 1 >= s.shape[1] or i < 0:
            return np.full(s.shape[0], np.inf)
        return s[:, i] - s[:, i + 1]
    for d in (-1, 1):
        assert any(shifted(np.array([[float(v) for v in lg.split()]]), int(k), d)[0] != float(w)
                   for lg, k, w in rows)


def test_parity_metric_hand_worked():
    rows = list(_rows("parity_metric.txt"))
    ref = np.array([[float(v) for v in r[0].split()] for r in rows])
    y = np.array([[float(v) for v in r[1].split()] for r in rows])
    want = np.array([float(r[2]) for r in rows])
    got = O.per_token_rel_err(y, ref)
    assert np.allclose(got, want, rtol=1e-15, atol=0), (got, want)
    # a mean in place of a max, or a missing absolute value, changes at least one row
    mean_for_max = np.abs(y - ref).mean(axis=1) / np.maximum(np.abs(ref).mean(axis=1), 1e-300)
    no_abs_ref = np.abs(y - ref).max(axis=1) / np.where(ref.max(axis=1) > 0, ref.max(axis=1), 1.0)
    assert not np.allclose(mean_for_max, want)
    assert not np.allclose(no_abs_ref, want)


def test_profile_seed_hand_worked():
    rows = list(_rows("profile_seed.txt"))
    assert len(rows) >= 5
    for counts, n, want in rows:
        c = [int(v) for v in counts.split()]
        got = O.profile_seed(c, int(n))
        assert list(got) == [int(v) for v in want.split()], (counts, n, list(got))


def test_profile_seed_brute_force():
    """The seeded list is the unique order in which every expert beats every later one by count,
    or by id on equal counts, and the n listed experts beat every unlisted one."""
    rng = np.random.default_rng(21)
    for _ in range(40):
        E = int(rng.integers(1, 12))
        n = int(rng.integers(1, E + 1))
        c = rng.integers(0, 4, size=E)
        got = [int(e) for e in O.profile_seed(c, n)]
        assert len(set(got)) == n
        beats = lambda a, b: c[a] > c[b] or (c[a] == c[b] and a < b)  # noqa: E731
        assert all(beats(got[i], got[i + 1]) for i in range(n - 1))
        assert all(beats(a, b) for a in got for b in range(E) if b not in got)


def test_codebook_and_affine_formats_hand_encoded():
    """The codebook and affine formats on a hand-encoded group: every listed element's weight is
    the hand-worked value (a wrong table index, a missing or doubled min, a sign error or a wrong
    block fails)."""
    fx = list(_rows("format_groups.txt"))
    cb = [int(v) for v in [r for r in fx if r[0] == "codebook"][0][1].split()]
    sbits = [int(h, 16) for h in [r for r in fx if r[0] == "scales"][0][1].split()]
    mbits = [int(h, 16) for h in [r for r in fx if r[0] == "mins"][0][1].split()]
    ramp = [r for r in _rows("dequant_groups.txt") if r[0] == "ramp_one"][0]
    code_bytes = np.array([int(b, 16) for b in ramp[1].split()], dtype=np.uint8)
    sb = np.array(sbits, dtype=np.uint16).view(np.uint8)
    mb = np.array(mbits, dtype=np.uint16).view(np.uint8)
    w_cb = O.dequant(code_bytes, sb, 1, 128, O.FMT_CB4, codebook=cb)[0]
    w_af = O.dequant(code_bytes, sb, 1, 128, O.FMT_AFFINE4, min_bytes=mb)[0]
    n = 0
    for fmt, e, val in [r for r in fx if r[0] in ("cb", "aff")]:
        got = (w_cb if fmt == "cb" else w_af)[int(e)]
        assert got == float(Fraction(val)), (fmt, e, got, val)
        n += 1
    assert n >= 20
    # the default format on the same bytes is unchanged
    assert O.dequant(code_bytes, sb, 1, 128)[0][15] == 7.0


def test_affine_blob_layout_appends_min_planes():
    q = O.blob_layout(2048, 768)
    a = O.blob_layout(2048, 768, O.FMT_AFFINE4)
    for name in ("gate_codes", "up_codes", "down_codes", "gate_scales", "up_scales", "down_scales"):
        assert q[name] == a[name]
    assert a["gate_mins"][0] == q["total"][1] and a["total"][1] == 2_654_208 + 3 * 98_304
    assert O.blob_layout(2048, 768, O.FMT_CB4) == q


@pytest.mark.parametrize("fmt", [1, 2])
def test_layer_formats_match_fp64_dense_brute_force(fmt):
    """The tiny layer in the codebook and affine formats: the oracle's layer equals a dense fp64
    mixture computed from the dequantized matrices of every expert."""
    rng = np.random.default_rng(40 + fmt)
    T, E, H, F, k = 4, 8, 256, 128, 2
    cb = np.sort(rng.choice(np.arange(-127, 128), 16, replace=False))
    nbytes = O.blob_layout(H, F, fmt)["total"][1]
    lay = O.blob_layout(H, F, fmt)

    def blob():
        b = rng.integers(0, 256, size=nbytes, dtype=np.uint8)
        for sec in ("gate_scales", "up_scales", "down_scales", "gate_mins", "up_mins", "down_mins"):
            if sec in lay:
                off, sz = lay[sec]
                v = (np.abs(rng.standard_normal(sz // 2)) * (0.02 if "scales" in sec else 0.1)).astype(np.float16)
                b[off:off + sz] = v.view(np.uint8)
        return b

    blobs = [blob() for _ in range(E)]
    shared = blob()
    x = rng.standard_normal((T, H))
    Wr = rng.standard_normal((E, H)) * 0.1
    out = O.moe_layer(x, Wr, None, k, lambda e: blobs[e], shared, H, F, fmt, cb)
    l = (x @ Wr.T).astype(np.float32).astype(np.float64)  # selection and weights on fp32 logits (R8)
    y = np.zeros((T, H))
    for t in range(T):
        sel = np.argsort(-l[t], kind="stable")[:k]
        w = np.exp(l[t, sel] - l[t, sel].max())
        w /= w.sum()
        for j, e in enumerate(sel):
            Wg, Wu, Wd = O.expert_weights(blobs[e], H, F, fmt, cb)
            g, u = Wg @ x[t], Wu @ x[t]
            y[t] += w[j] * (Wd @ (g / (1 + np.exp(-g)) * u))
        Wg, Wu, Wd = O.expert_weights(shared, H, F, fmt, cb)
        g, u = Wg @ x[t], Wu @ x[t]
        y[t] += Wd @ (g / (1 + np.exp(-g)) * u)
    assert np.allclose(out["y"], y, rtol=1e-12, atol=1e-12)
