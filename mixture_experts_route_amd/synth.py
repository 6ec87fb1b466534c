"""Seeded synthetic inputs for the routed MoE layer.

This module only draws numbers and stores them in the storage formats the layer
reads; it holds none of the layer's arithmetic.  The CPU oracle's tests, the GPU
parity tests and the benchmark all take their inputs from here, so both sides
see the same bytes.

Generator.  Every stream is keyed by ``(seed, cfg, kind, layer, index)``.  Word
``i`` of a stream is the SplitMix64 output function (Steele, Lea and Flood,
"Fast splittable pseudorandom number generators", OOPSLA 2014) applied to
``key + (i + 1) * 0x9E3779B97F4A7C15`` (mod 2**64).  It is integer-only, so the
numpy and torch implementations below give identical bits on CPU and GPU.

Distributions.  A value that is stored as a 16-bit float (bf16 activations and
router rows, fp16 block scales) is drawn directly as a 16-bit code by an
inverse-CDF lookup: the uniform 32-bit word ``u`` selects code ``c`` when
``t[c-1] <= u < t[c]``, where ``t`` holds ``floor(2**32 * CDF)`` at the midpoints
between neighbouring representable values.  That is exactly "draw from the
normal law and round to nearest" up to a 2**-32 quantisation of probability.
fp32 values (the tiny configuration's activations and router) are drawn on the
CPU only, by numpy's PCG64 seeded from the same key.

Storage formats (the ones the layer's C interface reads):

* bf16: uint16 codes, little-endian.
* expert blob: six sections, in order the gate, up and down codes (F*H/2 bytes
  each) and then their fp16 block scales (F*H/16 bytes each), in the group-major
  record layout the library's header states (64 code bytes and 8 scale bytes per
  row and group of 128 inputs).  This module only fills the sections with random
  bytes: codes are uniform random bytes, so every 4-bit code is uniform over
  0..15 wherever it sits; scales are fp16(|N(0, 0.02)|), one per 2-byte slot.
"""

from __future__ import annotations

import math
from functools import lru_cache

import numpy as np

GOLDEN = 0x9E3779B97F4A7C15
MASK64 = (1 << 64) - 1

KINDS = {
    "blob": 1,        # routed expert blob (index = expert id)
    "shared": 2,      # shared expert blob
    "router": 3,      # router matrix
    "x": 4,           # activations (index = step)
    "rank": 5,        # popularity rank permutation (index = topic)
    "table": 6,       # slot-table permutation
    "misc": 7,
}

BLOCK = 32

# weight formats of the library (identifiers only; the values they stand for are the library's
# and the oracle's business): 0 = 4-bit codes with a block scale, 1 = codes into a 16-entry
# codebook with a block scale, 2 = codes with a block scale and a block min
FMT_Q4_0, FMT_CB4, FMT_AFFINE4 = 0, 1, 2
# scale and min laws per format, so that the weights of every format have magnitudes like the
# first one's (its codes stand for -8..7; a codebook entry is up to 127; affine codes are 0..15
# less a min): the layer's outputs then stay in the same range
SCALE_SIGMA = {FMT_Q4_0: 0.02, FMT_CB4: 0.00125, FMT_AFFINE4: 0.02}
MIN_SIGMA = 0.15


def synthetic_codebook():
    """16 signed 8-bit values, ascending and unevenly spaced: 127 * z_i / z_15 rounded, with z_i
    the normal quantile at (i + 0.5) / 16 (a small set of values, denser near zero)."""
    from statistics import NormalDist

    z = [NormalDist().inv_cdf((i + 0.5) / 16) for i in range(16)]
    return [int(round(127 * v / z[15])) for v in z]


# ----------------------------------------------------------------------------
# keys and the SplitMix64 stream
# ----------------------------------------------------------------------------

def _mix64(z: int) -> int:
    z &= MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return z ^ (z >> 31)


def stream_key(seed: int, cfg: int, kind: str, layer: int = 0, index: int = 0) -> int:
    """64-bit key of one stream; each component is folded in with SplitMix64."""
    k = 0
    for part in (seed, cfg, KINDS[kind], layer, index):
        k = _mix64((k ^ (int(part) & MASK64)) + GOLDEN)
    return k


def words_np(key: int, start: int, n: int) -> np.ndarray:
    """Words ``start .. start+n-1`` of stream ``key`` as uint64."""
    with np.errstate(over="ignore"):
        i = np.arange(start + 1, start + n + 1, dtype=np.uint64)
        z = np.uint64(key) + i * np.uint64(GOLDEN)
        z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
        return z ^ (z >> np.uint64(31))


def _signed64(v: int) -> int:
    v &= MASK64
    return v - (1 << 64) if v >= (1 << 63) else v


def _lsr_t(z, s: int):
    """Logical right shift of an int64 torch tensor."""
    return (z >> s) & ((1 << (64 - s)) - 1)


def words_torch(key: int, start: int, n: int, device):
    """Same words as :func:`words_np`, as an int64 torch tensor (two's complement)."""
    import torch

    i = torch.arange(start + 1, start + n + 1, dtype=torch.int64, device=device)
    z = i * _signed64(GOLDEN) + _signed64(key)
    z = (z ^ _lsr_t(z, 30)) * _signed64(0xBF58476D1CE4E5B9)
    z = (z ^ _lsr_t(z, 27)) * _signed64(0x94D049BB133111EB)
    return z ^ _lsr_t(z, 31)


# ----------------------------------------------------------------------------
# inverse-CDF tables over 16-bit float codes
# ----------------------------------------------------------------------------

def _fp16_value(codes: np.ndarray) -> np.ndarray:
    return codes.astype(np.uint16).view(np.float16).astype(np.float64)


def _bf16_value(codes: np.ndarray) -> np.ndarray:
    return (codes.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


@lru_cache(maxsize=None)
def _halfnormal_fp16_table(sigma: float):
    """Thresholds for fp16(|N(0, sigma)|) over the finite positive fp16 codes."""
    codes = np.arange(0, 0x7C00, dtype=np.uint16)
    v = _fp16_value(codes)
    mid = 0.5 * (v[:-1] + v[1:])
    cdf = np.array([math.erf(m / (sigma * math.sqrt(2.0))) for m in mid])
    t = np.floor(cdf * 2.0**32).astype(np.int64)
    return t, codes


@lru_cache(maxsize=None)
def _normal_bf16_table(sigma: float):
    """Thresholds for bf16(N(0, sigma)) over the finite bf16 codes sorted by value."""
    pos = np.arange(0x0001, 0x7F80, dtype=np.uint16)           # +min subnormal .. +max finite
    neg = (pos[::-1] | np.uint16(0x8000)).astype(np.uint16)   # -max .. -min subnormal
    codes = np.concatenate([neg, np.array([0], np.uint16), pos])
    v = _bf16_value(codes)
    mid = 0.5 * (v[:-1] + v[1:])
    cdf = np.array([0.5 * (1.0 + math.erf(m / (sigma * math.sqrt(2.0)))) for m in mid])
    t = np.floor(cdf * 2.0**32).astype(np.int64)
    return t, codes


def _u32_np(key: int, start_word: int, n: int) -> np.ndarray:
    """n uniform 32-bit draws: low then high half of each word."""
    w = words_np(key, start_word, (n + 1) // 2)
    lo = (w & np.uint64(0xFFFFFFFF)).astype(np.int64)
    hi = (w >> np.uint64(32)).astype(np.int64)
    return np.stack([lo, hi], axis=1).reshape(-1)[:n]


def _u32_torch(key: int, start_word: int, n: int, device):
    import torch

    w = words_torch(key, start_word, (n + 1) // 2, device)
    lo = w & 0xFFFFFFFF
    hi = _lsr_t(w, 32)
    return torch.stack([lo, hi], dim=1).reshape(-1)[:n]


def _lookup_np(table, u):
    t, codes = table
    return codes[np.searchsorted(t, u, side="right")]


def _lookup_torch(table, u):
    import torch

    t, codes = table
    tt = torch.from_numpy(t).to(u.device)
    cc = torch.from_numpy(codes.astype(np.int32)).to(u.device)
    return cc[torch.searchsorted(tt, u, right=True)]


# ----------------------------------------------------------------------------
# public generators
# ----------------------------------------------------------------------------

def bf16_normal_np(key: int, shape, sigma: float) -> np.ndarray:
    """bf16(N(0, sigma)) as uint16 codes."""
    n = int(np.prod(shape))
    return _lookup_np(_normal_bf16_table(float(sigma)), _u32_np(key, 0, n)).reshape(shape)


def bf16_normal_torch(key: int, shape, sigma: float, device):
    """Same codes as :func:`bf16_normal_np`, as an int16 torch tensor (bit pattern)."""
    import torch

    n = int(np.prod(shape))
    c = _lookup_torch(_normal_bf16_table(float(sigma)), _u32_torch(key, 0, n, device))
    c = torch.where(c >= 0x8000, c - 0x10000, c)
    return c.to(torch.int16).reshape(shape)


def f32_normal_np(key: int, shape, sigma: float) -> np.ndarray:
    """fp32 N(0, sigma) drawn with numpy PCG64 seeded from ``key`` (CPU only)."""
    g = np.random.Generator(np.random.PCG64(key))
    return (g.standard_normal(size=shape) * sigma).astype(np.float32)


def bf16_to_f32(codes: np.ndarray) -> np.ndarray:
    """Widen bf16 codes to fp32 (exact)."""
    return (np.asarray(codes).astype(np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def blob_sections(H: int, F: int):
    """(name, byte offset, byte size) of the six sections of one expert blob."""
    nib_gu = F * H // 2
    nib_d = H * F // 2
    sc_gu = F * (H // BLOCK) * 2
    sc_d = H * (F // BLOCK) * 2
    sizes = [("gate_codes", nib_gu), ("up_codes", nib_gu), ("down_codes", nib_d),
             ("gate_scales", sc_gu), ("up_scales", sc_gu), ("down_scales", sc_d)]
    out, off = [], 0
    for name, sz in sizes:
        out.append((name, off, sz))
        off += sz
    return out


def blob_bytes(H: int, F: int, fmt: int = FMT_Q4_0) -> int:
    name, off, sz = blob_sections(H, F)[-1]
    return off + sz + (3 * F * H // BLOCK * 2 if fmt == FMT_AFFINE4 else 0)


def _blob_counts(H: int, F: int):
    n_code_bytes = 3 * F * H // 2
    n_scales = 3 * F * H // BLOCK
    assert n_code_bytes % 8 == 0 and n_scales % 2 == 0
    return n_code_bytes, n_scales


def expert_blob_np(key: int, H: int, F: int, scale_sigma: float | None = None, fmt: int = FMT_Q4_0) -> np.ndarray:
    """One expert blob (uint8) from stream ``key``: codes, scales and (affine format) mins."""
    nb, ns = _blob_counts(H, F)
    sigma = SCALE_SIGMA[fmt] if scale_sigma is None else scale_sigma
    w = words_np(key, 0, nb // 8)
    codes = w.view(np.uint8)  # little-endian bytes of each word
    u = _u32_np(key, nb // 8, ns)
    scales = _lookup_np(_halfnormal_fp16_table(float(sigma)), u).astype(np.uint16)
    parts = [codes, scales.view(np.uint8)]
    if fmt == FMT_AFFINE4:
        um = _u32_np(key, nb // 8 + (ns + 1) // 2, ns)
        parts.append(_lookup_np(_halfnormal_fp16_table(MIN_SIGMA), um).astype(np.uint16).view(np.uint8))
    return np.concatenate(parts)


def expert_blobs_torch(keys, H: int, F: int, out, scale_sigma: float | None = None, fmt: int = FMT_Q4_0):
    """Write blob ``keys[i]`` into row ``i`` of the uint8 device tensor ``out``.

    ``out`` is ``[len(keys)][stride]`` with ``stride >= blob_bytes(H, F, fmt)``; bytes
    past the blob are left as they are.  Bit-identical to :func:`expert_blob_np`.
    """
    import torch

    nb, ns = _blob_counts(H, F)
    sigma = SCALE_SIGMA[fmt] if scale_sigma is None else scale_sigma
    dev = out.device

    def fp16_draws(key, start, sig):
        c = _lookup_torch(_halfnormal_fp16_table(float(sig)), _u32_torch(key, start, ns, dev))
        return torch.where(c >= 0x8000, c - 0x10000, c).to(torch.int16).view(torch.uint8)

    for i, key in enumerate(keys):
        w = words_torch(key, 0, nb // 8, dev)
        out[i, :nb].copy_(w.view(torch.uint8))
        out[i, nb:nb + 2 * ns].copy_(fp16_draws(key, nb // 8, sigma))
        if fmt == FMT_AFFINE4:
            out[i, nb + 2 * ns:nb + 4 * ns].copy_(fp16_draws(key, nb // 8 + (ns + 1) // 2, MIN_SIGMA))
    return out


def expert_blobs_torch_batch(keys, H: int, F: int, out, scale_sigma: float = 0.02, batch: int = 64):
    """:func:`expert_blobs_torch` for many keys at once (``batch`` blobs per pass); same bytes."""
    import torch

    nb, ns = _blob_counts(H, F)
    dev = out.device
    tt = torch.from_numpy(_halfnormal_fp16_table(float(scale_sigma))[0]).to(dev)
    cc = torch.from_numpy(_halfnormal_fp16_table(float(scale_sigma))[1].astype(np.int32)).to(dev)
    n_code_words = nb // 8
    n_scale_words = (ns + 1) // 2
    n_words = n_code_words + n_scale_words
    idx = torch.arange(1, n_words + 1, dtype=torch.int64, device=dev) * _signed64(GOLDEN)
    for b0 in range(0, len(keys), batch):
        kk = torch.tensor([_signed64(k) for k in keys[b0:b0 + batch]], dtype=torch.int64, device=dev)
        z = idx.unsqueeze(0) + kk.unsqueeze(1)
        z = (z ^ _lsr_t(z, 30)) * _signed64(0xBF58476D1CE4E5B9)
        z = (z ^ _lsr_t(z, 27)) * _signed64(0x94D049BB133111EB)
        z = z ^ _lsr_t(z, 31)
        rows = out[b0:b0 + len(kk)]
        rows[:, :nb].copy_(z[:, :n_code_words].contiguous().view(torch.uint8))
        w = z[:, n_code_words:]
        u = torch.stack([w & 0xFFFFFFFF, _lsr_t(w, 32)], dim=2).reshape(len(kk), -1)[:, :ns]
        sc = cc[torch.searchsorted(tt, u.contiguous(), right=True)]
        sc = torch.where(sc >= 0x8000, sc - 0x10000, sc).to(torch.int16)
        rows[:, nb:nb + 2 * ns].copy_(sc.view(torch.uint8).reshape(len(kk), 2 * ns))
        del z, w, u, sc
    return out


def rank_permutation(seed: int, cfg: int, layer: int, topic: int, E: int) -> np.ndarray:
    """Popularity rank (1 = hottest) of each expert for one (layer, topic)."""
    g = np.random.Generator(np.random.PCG64(stream_key(seed, cfg, "rank", layer, topic)))
    return (g.permutation(E) + 1).astype(np.int64)


def zipf_bias(rank: np.ndarray, c: float) -> np.ndarray:
    """Per-expert router bias ``-c * ln(rank)`` (fp32) that skews selection counts."""
    return (-c * np.log(rank.astype(np.float64))).astype(np.float32)


# Calibrated so that, for hidden 2048 with x ~ N(0,1) and a bf16 N(0,0.02) router
# (logit std ~0.9), the log-log slope of selection count against popularity rank
# over ranks 5..200 is about -1.1 at top-10 of 512 (a Zipf(1.1) popularity).
ZIPF_C = 0.46
