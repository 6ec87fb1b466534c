"""The seeded input generators (CPU only): reproducible, numpy == torch, right laws."""

import math

import numpy as np
import pytest
import torch

from mixture_experts_route_amd import synth as S
from oracle import moe_oracle as O


def test_splitmix64_reference_values():
    # SplitMix64 (Steele, Lea, Flood 2014) seeded with 0: the first outputs of the
    # published generator are 0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F.
    w = S.words_np(0, 0, 3)
    assert [int(v) for v in w] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_numpy_and_torch_words_agree():
    for key in (0, 1, S.stream_key(0, 2, "blob", 3, 511), (1 << 64) - 1):
        a = S.words_np(key, 17, 4099)
        b = S.words_torch(key, 17, 4099, "cpu").numpy().view(np.uint64)
        assert np.array_equal(a, b)


def test_blob_numpy_equals_torch_and_is_seeded():
    H, F = 256, 128
    k1 = S.stream_key(0, 1, "blob", 0, 3)
    a = S.expert_blob_np(k1, H, F)
    out = torch.zeros((2, S.blob_bytes(H, F) + 64), dtype=torch.uint8)
    S.expert_blobs_torch([k1, S.stream_key(0, 1, "blob", 0, 4)], H, F, out)
    assert np.array_equal(out[0, :a.size].numpy(), a)
    assert not np.array_equal(out[1, :a.size].numpy(), a)
    assert np.array_equal(S.expert_blob_np(k1, H, F), a)
    assert a.size == S.blob_bytes(H, F) == O.blob_layout(H, F)["total"][1]


def test_bf16_normal_numpy_equals_torch_and_law():
    key = S.stream_key(0, 2, "x", 0, 0)
    a = S.bf16_normal_np(key, (64, 2048), 1.0)
    b = S.bf16_normal_torch(key, (64, 2048), 1.0, "cpu").numpy()
    assert np.array_equal(a.view(np.int16), b)
    v = S.bf16_to_f32(a).astype(np.float64)
    assert abs(v.mean()) < 0.01 and abs(v.std() - 1.0) < 0.01
    # the codes are exactly bf16: widening then narrowing is the identity
    assert np.array_equal((v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16), a.astype(np.uint16))


def test_scale_law_is_halfnormal_fp16():
    blob = S.expert_blob_np(S.stream_key(0, 2, "blob", 0, 0), 2048, 768)
    off = O.blob_layout(2048, 768)["gate_scales"][0]
    s = blob[off:].view(np.float16).astype(np.float64)
    assert np.all(s >= 0)
    assert s.mean() == pytest.approx(0.02 * math.sqrt(2 / math.pi), rel=0.01)
    # fraction below the smallest normal fp16 (6.1e-5): erf(6.1035e-5 / (0.02 sqrt 2)) = 0.00243
    assert (s < 2.0**-14).mean() == pytest.approx(math.erf(2.0**-14 / (0.02 * math.sqrt(2))), rel=0.15)


def test_code_nibbles_uniform():
    blob = S.expert_blob_np(S.stream_key(0, 2, "blob", 0, 1), 2048, 768)
    codes = blob[:3 * 768 * 1024]
    for nib in (codes & 15, codes >> 4):
        h = np.bincount(nib, minlength=16) / nib.size
        assert np.all(np.abs(h - 1 / 16) < 0.002)


def test_zipf_bias_gives_zipf_11_popularity():
    """Selection counts vs popularity rank follow a power law of slope about -1.1 (ranks 5..200)."""
    E, H, T, k = 512, 2048, 4096, 10
    Wr = O.bf16_codes_to_f64(S.bf16_normal_np(S.stream_key(0, 4, "router"), (E, H), 0.02))
    x = O.bf16_codes_to_f64(S.bf16_normal_np(S.stream_key(0, 4, "x"), (T, H), 1.0))
    rank = S.rank_permutation(0, 4, 0, 0, E)
    l32 = (x @ Wr.T + S.zipf_bias(rank, S.ZIPF_C)).astype(np.float32)
    ids = np.argsort(-l32, axis=1, kind="stable")[:, :k]
    cnt = np.bincount(ids.ravel(), minlength=E)[np.argsort(rank)]
    r = np.arange(5, 201)
    slope = np.polyfit(np.log(r), np.log(np.maximum(cnt[r - 1], 1)), 1)[0]
    assert -1.2 < slope < -1.0


def test_batched_torch_blobs_equal_single():
    import torch

    H, F = 256, 128
    keys = [S.stream_key(0, 3, "blob", 5, e) for e in range(5)]
    stride = (S.blob_bytes(H, F) + 4095) // 4096 * 4096
    a = torch.zeros((5, stride), dtype=torch.uint8)
    b = torch.zeros((5, stride), dtype=torch.uint8)
    S.expert_blobs_torch(keys, H, F, a)
    S.expert_blobs_torch_batch(keys, H, F, b, batch=2)
    assert torch.equal(a, b)
    assert np.array_equal(b[3, :S.blob_bytes(H, F)].numpy(), S.expert_blob_np(keys[3], H, F))


def test_format_blobs_numpy_equals_torch():
    """The codebook and affine formats' blobs: the numpy and torch generators give the same bytes;
    the affine blob's min planes follow the scales and draw the min law."""
    import numpy as np
    import torch

    for fmt in (S.FMT_CB4, S.FMT_AFFINE4):
        keys = [S.stream_key(0, 1, "blob", 0, e) for e in range(3)]
        n = S.blob_bytes(256, 128, fmt)
        out = torch.zeros((3, n + 64), dtype=torch.uint8)
        S.expert_blobs_torch(keys, 256, 128, out, fmt=fmt)
        for i, k in enumerate(keys):
            assert np.array_equal(out[i, :n].numpy(), S.expert_blob_np(k, 256, 128, fmt=fmt))
        assert (out[:, n:] == 0).all()
    b = S.expert_blob_np(S.stream_key(0, 1, "blob", 0, 9), 2048, 768, fmt=S.FMT_AFFINE4)
    assert len(b) == 2_654_208 + 3 * 98_304
    mins = b[2_654_208:].view(np.float16).astype(np.float64)
    assert (mins >= 0).all() and abs(mins.mean() / (S.MIN_SIGMA * np.sqrt(2 / np.pi)) - 1) < 0.02
    cb = S.synthetic_codebook()
    assert len(cb) == 16 and cb == sorted(cb) and len(set(cb)) == 16 and max(map(abs, cb)) == 127
