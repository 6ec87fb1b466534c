"""CPU oracle of the routed mixture-of-experts layer.

TEST INFRASTRUCTURE ONLY.  The tests, the smoke check and the benchmark's CPU
baseline are the only code that may import or call anything here.  The layer's
product path (the HIP library and its Python binding) never does, and shares no
code with this module.

Plain numpy in float64, each step written as its definition, in the order the
definition gives, with a library matmul or sort as a step where noted and no
blocking, fusion or reordering beyond that.  Inputs arrive as the storage bytes
the layer reads (bf16 / fp32 activations and router, expert blobs), so every
value enters float64 exactly.

The pages this follows:

* [BG] Betelgeuse news article (fanjiajia.top, "Betelgeuse: RTX 3060 12GB + 16GB
  ... 22 tok/s"), section "mechanism: VRAM expert-slot pool, in-stream doorbell
  and victim cache": the model has 48 layers of 512 routed experts and each token
  takes 10 routed experts plus 1 shared one; the router and the shared expert
  stay resident; the other experts live in a per-layer pool of slots (240 / 92 /
  60 per layer for early / middle / late layers); a GPU-side check decides hits
  and rings the host only on a miss; the VRAM and RAM tiers never hold the same
  expert.  Section "what bit-exact means": the top-10 selection is never
  altered.
* [HG] halogen-flash-server README, section "Bring your own GGUF": expert
  weights are a small set of values times one scale per block (the Q4_0
  family), moved losslessly into the kernels' own layout.
* [BA] Basalt README, section "The .basalt model file": quantized bytes are
  used as stored, never requantized.

The pages give no formulas for the router, the expert FFN or the byte layout.
The readings taken here:

* R1 router weights are a softmax over the k selected logits, which is full
  softmax renormalised over the selection (weights sum to 1 over the chosen
  experts);
* R2 the shared expert has weight 1, no gate, the same width and format;
* R3 4-bit code u in 0..15 stands for q = u - 8; blocks of 32 run along the
  reduction dimension; one fp16 scale per block; the code words of each run of
  four blocks are interleaved and the runs stored group-major as in
  :func:`decode_codes` (rows hold a multiple of 128 elements);
* R4 a per-expert bias, when given, is added to the logits before both the
  selection and the weights;
* R5 equal logits: the lower expert id wins;
* R6 the expert FFN is SwiGLU: h = silu(Wg x) * (Wu x), y_e = Wd h;
* R7 combine: y = sum_j w_j y_{e_j} (j = 0..k-1 in selection order) + y_shared;
  no residual and no norm inside the layer;
* R8 the selection is decided on fp32 logits (the precision the GPU path
  decides in); the oracle computes the logits in float64 and rounds them to fp32
  before ranking;
* R9 miss list: unique expert ids, ascending;
* R10 slot pool policy: per-layer LRU with an exclusive swap (see
  :class:`SlotPoolLRU`).
* R15 codebook format ([HG] "Bring your own GGUF": the IQ4_NL / IQ4_XS family
  is a small set of values times a per-block scale): a 4-bit code u selects
  value u of the layer's codebook of 16 signed 8-bit integers, and the weight is
  codebook[u] * scale; codes and scales sit where the default format has them.
* R16 affine format ([HG] same section: Q4_K / Q5_K / Q5_1 read as exact affine
  planes): weight = u * scale - min with u in 0..15 and one fp16 scale and one
  fp16 min per block of 32; the min plane follows the scale planes in the blob,
  in the scales' record layout.
"""

from __future__ import annotations

import numpy as np

BLOCK = 32

# weight formats: (u - 8) * scale; codebook[u] * scale; u * scale - min
FMT_Q4_0, FMT_CB4, FMT_AFFINE4 = 0, 1, 2


# ----------------------------------------------------------------------------
# storage formats
# ----------------------------------------------------------------------------

def bf16_codes_to_f64(codes) -> np.ndarray:
    """bf16 codes (uint16 / int16 bit patterns) -> float64, exactly."""
    c = np.asarray(codes).astype(np.uint16).astype(np.uint32)
    return (c << np.uint32(16)).view(np.float32).astype(np.float64)


def fp16_codes_to_f64(codes) -> np.ndarray:
    """fp16 codes -> float64, exactly (subnormals included)."""
    return np.asarray(codes).astype(np.uint16).view(np.float16).astype(np.float64)


def blob_layout(H: int, F: int, fmt: int = FMT_Q4_0) -> dict:
    """Byte offsets of the sections of one expert blob.

    Order: gate codes (F rows of H), up codes (F rows of H), down codes (H rows
    of F), each F*H/2 bytes, then the fp16 scales of gate, up and down, F*H/32 * 2
    bytes each, and with the affine format (R16) the fp16 mins of gate, up and
    down, laid out like the scales; codes, scales and mins group-major
    (:func:`decode_codes`, :func:`decode_scales`).  (Layout is ours: [HG] "Bring
    your own GGUF" repacks a file's values into the kernels' layout.)
    """
    sizes = [
        ("gate_codes", F * H // 2), ("up_codes", F * H // 2), ("down_codes", H * F // 2),
        ("gate_scales", F * (H // BLOCK) * 2), ("up_scales", F * (H // BLOCK) * 2),
        ("down_scales", H * (F // BLOCK) * 2),
    ]
    if fmt == FMT_AFFINE4:
        sizes += [("gate_mins", F * (H // BLOCK) * 2), ("up_mins", F * (H // BLOCK) * 2),
                  ("down_mins", H * (F // BLOCK) * 2)]
    out, off = {}, 0
    for name, sz in sizes:
        out[name] = (off, sz)
        off += sz
    out["total"] = (0, off)
    return out


GROUP = 128  # elements per word group: four blocks of 32


def decode_codes(code_bytes: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """4-bit codes of a [rows][cols] matrix, as integers 0..15 (cols a multiple of 128).

    The codes are stored group-major: the cols/128 groups of 128 elements (four
    blocks of 32) of every row form 64-byte records, record (c, r) = group c of
    row r at byte 64 (c * rows + r).  A record is 16 little-endian 32-bit words;
    word 4g + i holds the eight elements 128c + 32i + 8g .. 128c + 32i + 8g + 7
    (slice g of block i of the group): its element 2j in bits 4j..4j+3 and its
    element 2j+1 in bits 16+4j..16+4j+3, for j = 0..3.
    """
    assert cols % GROUP == 0
    b = np.asarray(code_bytes, dtype=np.uint8).reshape(cols // GROUP, rows, 4, 4, 4).astype(np.uint32)
    # b[c, r, g, i, byte]: byte `byte` of word 4g + i of record (c, r)
    word = b[..., 0] | (b[..., 1] << 8) | (b[..., 2] << 16) | (b[..., 3] << 24)
    u = np.empty((rows, cols // GROUP, 4, 4, 8), dtype=np.int64)  # [r, c, i (block), g (slice), m]
    for i in range(4):
        for g in range(4):
            w = word[:, :, g, i].T  # [r, c]
            for j in range(4):
                u[:, :, i, g, 2 * j] = (w >> (4 * j)) & 0xF
                u[:, :, i, g, 2 * j + 1] = (w >> (16 + 4 * j)) & 0xF
    return u.reshape(rows, cols)


def decode_scales(scale_bytes, rows: int, cols: int) -> np.ndarray:
    """fp16 block scales of a [rows][cols] matrix -> float64 [rows][cols/32].

    Stored group-major like the codes: record (c, r) = the four scales of group c
    of row r (blocks 4c .. 4c+3) at byte 8 (c * rows + r).
    """
    s = fp16_codes_to_f64(np.asarray(scale_bytes, dtype=np.uint8).view(np.uint16))
    s = s.reshape(cols // GROUP, rows, 4)  # [c, r, i]
    return s.transpose(1, 0, 2).reshape(rows, cols // BLOCK)


def dequant(code_bytes, scale_bytes, rows: int, cols: int, fmt: int = FMT_Q4_0, codebook=None,
            min_bytes=None) -> np.ndarray:
    """The weights w[r][c] of a [rows][cols] matrix, with s = scale[r][c // 32]:

    * FMT_Q4_0 (R3): (u - 8) * s ([HG]: small set x block scale);
    * FMT_CB4 (R15): codebook[u] * s;
    * FMT_AFFINE4 (R16): u * s - min[r][c // 32].
    """
    u = decode_codes(code_bytes, rows, cols)
    s = np.repeat(decode_scales(scale_bytes, rows, cols), BLOCK, axis=1)
    if fmt == FMT_Q4_0:
        return (u - 8).astype(np.float64) * s
    if fmt == FMT_CB4:
        cb = np.asarray(codebook, dtype=np.int64)
        assert cb.shape == (16,)
        return cb[u].astype(np.float64) * s
    if fmt == FMT_AFFINE4:
        m = np.repeat(decode_scales(min_bytes, rows, cols), BLOCK, axis=1)
        return u.astype(np.float64) * s - m
    raise ValueError(fmt)


def expert_weights(blob: np.ndarray, H: int, F: int, fmt: int = FMT_Q4_0, codebook=None):
    """Dequantized (Wg [F][H], Wu [F][H], Wd [H][F]) of one expert blob."""
    lay = blob_layout(H, F, fmt)
    blob = np.asarray(blob, dtype=np.uint8)

    def sec(name):
        off, sz = lay[name]
        return blob[off:off + sz]

    def mins(name):
        return sec(name) if fmt == FMT_AFFINE4 else None

    Wg = dequant(sec("gate_codes"), sec("gate_scales"), F, H, fmt, codebook, mins("gate_mins"))
    Wu = dequant(sec("up_codes"), sec("up_scales"), F, H, fmt, codebook, mins("up_mins"))
    Wd = dequant(sec("down_codes"), sec("down_scales"), H, F, fmt, codebook, mins("down_mins"))
    return Wg, Wu, Wd


# ----------------------------------------------------------------------------
# router ([BG] 10 routed of 512 + 1 shared; readings R1, R4, R5, R8)
# ----------------------------------------------------------------------------

def router_logits(x: np.ndarray, Wr: np.ndarray, bias=None) -> np.ndarray:
    """l[t][e] = sum_h x[t][h] * Wr[e][h] (+ bias[e]); float64 (matmul as a step)."""
    l = np.asarray(x, np.float64) @ np.asarray(Wr, np.float64).T
    if bias is not None:
        l = l + np.asarray(bias, np.float64)[None, :]
    return l


def select_topk(logits32: np.ndarray, k: int) -> np.ndarray:
    """Ids of the k largest logits per token, ranked by (logit desc, id asc)."""
    logits32 = np.asarray(logits32)
    T, E = logits32.shape
    ids = np.empty((T, k), dtype=np.int32)
    idx = np.arange(E)
    for t in range(T):
        order = np.lexsort((idx, -logits32[t].astype(np.float64)))  # sort as a step
        ids[t] = order[:k]
    return ids


def route_weights(logits32: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """w_j = exp(l_j - m) / sum_i exp(l_i - m) over the selected logits (R1)."""
    sel = np.take_along_axis(np.asarray(logits32, np.float64), ids.astype(np.int64), axis=1)
    m = sel[:, :1]
    e = np.exp(sel - m)
    return e / e.sum(axis=1, keepdims=True)


def topk_gap(logits: np.ndarray, k: int) -> np.ndarray:
    """l_(k) - l_(k+1) per token (sorted descending); inf when k == E."""
    s = -np.sort(-np.asarray(logits, np.float64), axis=1)
    if k >= s.shape[1]:
        return np.full(s.shape[0], np.inf)
    return s[:, k - 1] - s[:, k]


def route(x, Wr, bias, k: int):
    """Router + selection + weights.  Returns (logits64, logits32, ids, w)."""
    l64 = router_logits(x, Wr, bias)
    l32 = l64.astype(np.float32)
    ids = select_topk(l32, k)
    w = route_weights(l32, ids)
    return l64, l32, ids, w


# ----------------------------------------------------------------------------
# expert FFN and combine (readings R2, R6, R7)
# ----------------------------------------------------------------------------

def silu(g: np.ndarray) -> np.ndarray:
    return g / (1.0 + np.exp(-g))


def swiglu_ffn(Wg, Wu, Wd, x: np.ndarray) -> np.ndarray:
    """y = Wd (silu(Wg x) * (Wu x)) for each row of x [n][H] (matmul as a step)."""
    g = x @ Wg.T
    u = x @ Wu.T
    h = silu(g) * u
    return h @ Wd.T


def combine(w: np.ndarray, y_routed: np.ndarray, y_shared) -> np.ndarray:
    """y[t] = sum_{j=0}^{k-1} w[t][j] * y_routed[t][j] + y_shared[t], in that order."""
    T, k, H = y_routed.shape
    y = np.zeros((T, H), dtype=np.float64)
    for j in range(k):
        y = y + w[:, j:j + 1] * y_routed[:, j, :]
    if y_shared is not None:
        y = y + y_shared
    return y


def moe_layer(x, Wr, bias, k: int, expert_blob, shared_blob, H: int, F: int, fmt: int = FMT_Q4_0,
              codebook=None):
    """The whole routed MoE layer on activations x [T][H] (exact values).

    ``expert_blob(e)`` returns routed expert e's blob; ``shared_blob`` is the
    shared expert's blob or None; ``fmt`` / ``codebook`` the weight format.
    Returns a dict with y [T][H] (float64) and the routing (logits64, logits32,
    ids, w).
    """
    x = np.asarray(x, np.float64)
    T = x.shape[0]
    l64, l32, ids, w = route(x, Wr, bias, k)
    y_routed = np.zeros((T, k, H), dtype=np.float64)
    for e in np.unique(ids):
        Wg, Wu, Wd = expert_weights(expert_blob(int(e)), H, F, fmt, codebook)
        rows = np.nonzero(ids == e)
        y_routed[rows[0], rows[1], :] = swiglu_ffn(Wg, Wu, Wd, x[rows[0]])
    y_shared = None
    if shared_blob is not None:
        Wg, Wu, Wd = expert_weights(shared_blob, H, F, fmt, codebook)
        y_shared = swiglu_ffn(Wg, Wu, Wd, x)
    y = combine(w, y_routed, y_shared)
    return {"y": y, "logits64": l64, "logits32": l32, "ids": ids, "w": w}


# ----------------------------------------------------------------------------
# residency check ([BG] slot pool, in-stream hit check; reading R9)
# ----------------------------------------------------------------------------

def slot_lookup(table: np.ndarray, ids: np.ndarray):
    """slots[t][j] = table[ids[t][j]] (-1 = not resident); ascending unique miss list."""
    table = np.asarray(table)
    slots = table[np.asarray(ids, np.int64)].astype(np.int32)
    missing = sorted({int(e) for e, s in zip(np.ravel(ids), np.ravel(slots)) if s < 0})
    return slots, np.array(missing, dtype=np.int32)


# ----------------------------------------------------------------------------
# grouping of (token, choice) pairs by expert (stable counting sort)
# ----------------------------------------------------------------------------

def group_pairs(ids_flat, n_buckets: int):
    """Stable counting sort of pair indices p by bucket ids_flat[p].

    Returns counts [n_buckets], offsets [n_buckets + 1] (exclusive prefix sums)
    and perm, the pair indices in (bucket, p) order.
    """
    ids_flat = [int(v) for v in np.ravel(ids_flat)]
    counts = [0] * n_buckets
    for e in ids_flat:
        counts[e] += 1
    offsets = [0] * (n_buckets + 1)
    for e in range(n_buckets):
        offsets[e + 1] = offsets[e] + counts[e]
    cursor = offsets[:-1].copy()
    perm = [0] * len(ids_flat)
    for p, e in enumerate(ids_flat):
        perm[cursor[e]] = p
        cursor[e] += 1
    return (np.array(counts, np.int32), np.array(offsets, np.int32), np.array(perm, np.int32))


# ----------------------------------------------------------------------------
# slot pool policy (reading R10)
# ----------------------------------------------------------------------------

class SlotPoolLRU:
    """One layer's slot pool: which expert sits in which HBM slot.

    [BG]: a fixed number of slots per layer; a miss is filled from host memory;
    VRAM and host copies are exclusive, so the evicted expert moves to the host.
    Policy (the pages name only a "victim cache"): least recently used.

    State: ``table[e]`` = slot of expert e or -1; ``holder[s]`` = expert in slot s;
    ``last_use[s]``.  Initially slot s holds ``initial[s]`` with last use
    ``-(s + 1)`` when ``initial`` is ordered hottest first, so colder initial
    experts are evicted first.

    One step (:meth:`step`): look up every selected id; the misses (unique,
    ascending) are placed one by one, each into the slot that is not holding an
    expert selected in this step and has the smallest (last_use, slot); its
    expert is evicted to the host.  Then every selection, in (token, choice)
    order, stamps its slot with an increasing clock.
    """

    def __init__(self, n_experts: int, initial):
        self.n_experts = n_experts
        initial = [int(e) for e in initial]
        self.n_slots = len(initial)
        self.table = np.full(n_experts, -1, dtype=np.int32)
        self.holder = np.array(initial, dtype=np.int64)
        self.last_use = np.array([-(s + 1) for s in range(self.n_slots)], dtype=np.int64)
        for s, e in enumerate(initial):
            self.table[e] = s
        self.clock = 0

    def step(self, ids):
        """Apply one step's selections; returns (misses, [(expert, slot, evicted)])."""
        ids = np.asarray(ids, np.int64)
        selected = {int(e) for e in ids.ravel()}
        misses = sorted(e for e in selected if self.table[e] < 0)
        fills = []
        for e in misses:
            best = None
            for s in range(self.n_slots):
                if int(self.holder[s]) in selected:
                    continue
                key = (int(self.last_use[s]), s)
                if best is None or key < best:
                    best = key
            if best is None:
                raise RuntimeError("slot pool smaller than one step's distinct experts")
            s = best[1]
            old = int(self.holder[s])
            self.table[old] = -1
            self.table[e] = s
            self.holder[s] = e
            fills.append((e, s, old))
        for e in ids.ravel():
            self.clock += 1
            self.last_use[self.table[int(e)]] = self.clock
        return misses, fills


def profile_seed(counts, n_slots: int) -> np.ndarray:
    """Initial residency from a hot-expert profile ([BG] "limits and licence": the profile only
    seeds the cache with hot experts): the n_slots experts with the most selections, hottest
    first; equal counts keep the lower id first (a stable sort as a step)."""
    counts = np.asarray(counts, dtype=np.int64)
    order = np.argsort(-counts, kind="stable")
    return order[:n_slots].astype(np.int32)


def per_token_rel_err(y_gpu: np.ndarray, y_ref: np.ndarray) -> np.ndarray:
    """max_o |y - y_ref| / max_o |y_ref| per token (normwise, the parity metric, reading R11).

    A token whose reference row is all zero is measured by its absolute error max_o |y - y_ref|.
    """
    y_gpu = np.asarray(y_gpu, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    num = np.max(np.abs(y_gpu - y_ref), axis=1)
    den = np.max(np.abs(y_ref), axis=1)
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), num)
