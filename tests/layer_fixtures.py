"""Synthetic layers for the tests: device tensors from the seeded generator, and the
same bytes regenerated on the CPU for the oracle."""

from __future__ import annotations

import numpy as np

from mixture_experts_route_amd import synth as S
from oracle import moe_oracle as O

# The shapes of the pages' model (Betelgeuse article, "mechanism": 512 routed experts per
# layer, top-10 + 1 shared) with hidden 2048 / expert FFN 768, and the tiny parity shape.
TINY = dict(H=256, F=128, E=8, k=2, n_shared=1, cfg=1, x_sigma=1.0, r_sigma=0.1, x_f32=True, r_f32=True)
MODEL = dict(H=2048, F=768, E=512, k=10, n_shared=1, cfg=2, x_sigma=1.0, r_sigma=0.02, x_f32=False, r_f32=False)


def slot_stride(H, F, fmt=0):
    b = S.blob_bytes(H, F, fmt)
    return (b + 4095) // 4096 * 4096


class Layer:
    """One layer: arena of E routed blobs (slot e = expert e unless permuted), shared blob,
    router (+ optional Zipf bias).  Device tensors are built on `device` with the torch
    generator; oracle-side bytes are regenerated with numpy from the same keys."""

    def __init__(self, spec: dict, device, seed: int = 0, layer: int = 0, bias_c: float | None = None,
                 n_slots: int | None = None, slot_of=None):
        import torch

        self.spec = dict(spec)
        H, F, E = spec["H"], spec["F"], spec["E"]
        self.H, self.F, self.E, self.k, self.n_shared = H, F, E, spec["k"], spec["n_shared"]
        self.seed, self.cfg, self.layer = seed, spec["cfg"], layer
        self.fmt = spec.get("fmt", S.FMT_Q4_0)
        self.codebook = S.synthetic_codebook() if self.fmt == S.FMT_CB4 else None
        self.stride = slot_stride(H, F, self.fmt)
        self.n_slots = n_slots if n_slots is not None else E
        # slot_of[e] = slot of expert e (-1 = not resident); default identity
        self.slot_of = np.arange(E) if slot_of is None else np.asarray(slot_of)
        self.arena = torch.zeros((self.n_slots, self.stride), dtype=torch.uint8, device=device)
        experts = [e for e in range(E) if self.slot_of[e] >= 0]
        keys = [self.key(e) for e in experts]
        tmp = torch.empty((len(keys), self.stride), dtype=torch.uint8, device=device)
        S.expert_blobs_torch(keys, H, F, tmp, fmt=self.fmt)
        idx = torch.as_tensor([int(self.slot_of[e]) for e in experts], device=device, dtype=torch.long)
        self.arena[idx] = tmp
        del tmp
        self.shared = None
        if self.n_shared:
            self.shared = torch.zeros((self.stride,), dtype=torch.uint8, device=device)
            S.expert_blobs_torch([S.stream_key(seed, self.cfg, "shared", layer, 0)], H, F, self.shared.view(1, -1),
                                 fmt=self.fmt)
        rkey = S.stream_key(seed, self.cfg, "router", layer, 0)
        if spec["r_f32"]:
            self.router_np = S.f32_normal_np(rkey, (E, H), spec["r_sigma"])
            self.router = torch.from_numpy(self.router_np).to(device)
        else:
            self.router_codes = S.bf16_normal_np(rkey, (E, H), spec["r_sigma"])
            self.router_np = S.bf16_to_f32(self.router_codes)
            self.router = torch.from_numpy(self.router_codes.view(np.int16)).to(device)
        self.bias_np = None
        self.bias = None
        if bias_c is not None:
            rank = S.rank_permutation(seed, self.cfg, layer, 0, E)
            self.bias_np = S.zipf_bias(rank, bias_c)
            self.bias = torch.from_numpy(self.bias_np).to(device)

    def key(self, e):
        return S.stream_key(self.seed, self.cfg, "blob", self.layer, e)

    def blob_np(self, e):
        return S.expert_blob_np(self.key(e), self.H, self.F, fmt=self.fmt)

    def shared_np(self):
        if not self.n_shared:
            return None
        return S.expert_blob_np(S.stream_key(self.seed, self.cfg, "shared", self.layer, 0), self.H, self.F,
                                fmt=self.fmt)

    def table_tensor(self, device):
        import torch

        return torch.from_numpy(self.slot_of.astype(np.int32)).to(device)

    def x(self, T: int, step: int = 0, device=None):
        """Activations for one step: (device tensor, exact float64 copy)."""
        import torch

        key = S.stream_key(self.seed, self.cfg, "x", self.layer, step)
        if self.spec["x_f32"]:
            xn = S.f32_normal_np(key, (T, self.H), self.spec["x_sigma"])
            return torch.from_numpy(xn).to(device), xn.astype(np.float64)
        codes = S.bf16_normal_np(key, (T, self.H), self.spec["x_sigma"])
        return torch.from_numpy(codes.view(np.int16)).to(device), S.bf16_to_f32(codes).astype(np.float64)

    def oracle(self, x64):
        return O.moe_layer(x64, self.router_np.astype(np.float64), self.bias_np, self.k, self.blob_np,
                           self.shared_np(), self.H, self.F, self.fmt, self.codebook)

    def native_weights(self):
        from mixture_experts_route_amd import native as N

        return N.layer_weights(self.router, self.arena, self.stride, self.n_slots, self.shared, self.bias)

    def dims(self):
        from mixture_experts_route_amd import native as N

        return N.dims(self.H, self.F, self.E, self.k, self.n_shared, format=self.fmt, codebook=self.codebook)


def near_tie_tokens(logits64: np.ndarray, k: int, gap: float = 1e-4) -> np.ndarray:
    """Tokens whose k-th and (k+1)-th logits are closer than `gap` (excluded from id parity)."""
    return O.topk_gap(logits64, k) < gap
