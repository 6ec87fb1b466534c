"""Measures the prefill plans of the grouped GEMM on the GPU and writes the plan table.

    python -m mixture_experts_route_amd.tune --out PATH [--tokens 32,128,...] [--reps 10] [--formats 0,1,2]

For the model-shaped layer (512 routed experts top-10 + 1 shared, hidden 2048, expert FFN 768,
each weight format asked for) with Zipf(1.1)-skewed routing, it times every candidate plan of each token
count through moe_layer_forward (HIP events around the whole call; the median of --reps calls after
warm-up calls), the router rows separately from the rest, and writes the fastest plan per token
count as rows of csrc/tuned_plans.inc, each row covering the token counts up to the geometric mean
of its count and the next one.  The measured times go into the file as comments.  The library reads
the table when it is built; copy the file into csrc/ and rebuild.
"""

from __future__ import annotations

import argparse
import itertools
import math
import statistics
import sys
import time

H, F, E, K_TOP = 2048, 768, 512, 10


def candidates(only: str = ""):
    """(item_rows, gate_up kernel, down kernel) triples the library accepts (or those of `only`,
    a comma-separated list of rows:gate_up:down)."""
    if only:
        return [tuple(int(v) for v in c.split(":")) for c in only.split(",")]
    out = []
    for rows, gu, dn in itertools.product((128, 64), (0, 1, 2), (0, 1, 2)):
        if rows == 128 and (gu == 1 or dn == 1):
            continue
        out.append((rows, gu, dn))
    return out


def main():
    import numpy as np
    import torch

    from mixture_experts_route_amd import native as N
    from mixture_experts_route_amd import synth as S

    ap = argparse.ArgumentParser()
    ap.add_argument("--out", required=True)
    ap.add_argument("--tokens", default="17,64,256,1024,2048,4096,8192,16384,32768")
    ap.add_argument("--reps", type=int, default=10)
    ap.add_argument("--only", default="", help="candidate plans rows:gate_up:down,... (default: all)")
    ap.add_argument("--formats", default="0", help="weight formats to tune, comma-separated (0 default, "
                                                    "1 codebook, 2 affine)")
    args = ap.parse_args()
    dev = torch.device("cuda:0")
    cfg = 4
    tokens = [int(t) for t in args.tokens.split(",")]
    t_max = max(tokens)
    router = S.bf16_normal_torch(S.stream_key(0, cfg, "router", 0, 0), (E, H), 0.02, dev)
    bias = torch.from_numpy(S.zipf_bias(S.rank_permutation(0, cfg, 0, 0, E), S.ZIPF_C)).to(dev)
    x_all = S.bf16_normal_torch(S.stream_key(0, cfg, "x", 0, 2_000_000), (t_max, H), 1.0, dev)
    y = torch.empty((t_max, H), dtype=torch.float32, device=dev)

    rows = []
    for fmt in [int(f) for f in args.formats.split(",")]:
        stride = (S.blob_bytes(H, F, fmt) + 4095) // 4096 * 4096
        arena = torch.empty((E, stride), dtype=torch.uint8, device=dev)
        for e0 in range(0, E, 64):
            S.expert_blobs_torch([S.stream_key(0, cfg, "blob", 0, e) for e in range(e0, e0 + 64)], H, F,
                                 arena[e0:e0 + 64], fmt=fmt)
        shared = torch.empty((1, stride), dtype=torch.uint8, device=dev)
        S.expert_blobs_torch([S.stream_key(0, cfg, "shared", 0, 0)], H, F, shared, fmt=fmt)
        d = N.dims(H, F, E, K_TOP, 1, format=fmt, codebook=S.synthetic_codebook() if fmt == S.FMT_CB4 else None)
        w = N.layer_weights(router, arena, stride, E, shared[0], bias)
        ws = torch.zeros(N.moe_workspace_bytes(d, t_max) // 4 + 64, dtype=torch.int32, device=dev)
        N.moe_workspace_init(ws)

        def time_plan(T, plan):
            N.moe_debug_force_prefill_plan(plan)
            x = x_all[:T]
            for _ in range(3):
                N.moe_layer_forward(d, w, None, x, T, y[:T], ws)
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(args.reps)]
            torch.cuda.synchronize()
            for a, b in ev:
                a.record()
                N.moe_layer_forward(d, w, None, x, T, y[:T], ws)
                b.record()
            torch.cuda.synchronize()
            assert N.moe_check_device_error(ws) == 0
            return statistics.median(a.elapsed_time(b) * 1e3 for a, b in ev)  # us

        # candidates the format runs as named (the affine format has no 128-row pipelined kernel)
        cands = [c for c in candidates(args.only) if not (fmt == S.FMT_AFFINE4 and 0 in c[1:])]
        for T in tokens:
            t0 = time.perf_counter()
            default_router = 64 if T > 16384 else 32
            res = {}
            for rows_, gu, dn in cands:
                res[(rows_, gu, dn)] = time_plan(T, N.moe_prefill_plan(rows_, gu, dn, default_router))
            best = min(res, key=res.get)
            r_res = {r: time_plan(T, N.moe_prefill_plan(*best, r)) for r in (32, 64)}
            best_r = min(r_res, key=r_res.get)
            rows.append((fmt, T, best, best_r, res, r_res))
            print(f"tune: format {fmt} T={T}: best {best} router {best_r}: {res[best]:.1f} us "
                  f"({time.perf_counter() - t0:.1f} s)", file=sys.stderr, flush=True)
        N.moe_debug_force_prefill_plan(None)
        del arena, shared, ws
        torch.cuda.empty_cache()

    lines = ["// Prefill plans measured on one MI355X (gfx950).  Written by mixture_experts_route_amd/tune.py,",
             "// which times every candidate plan of each shape, weight format and token count through",
             "// moe_layer_forward and keeps the fastest; a row covers the token counts from t_lo to t_hi.  Rows:",
             "//   {H, F, E, k, format, t_lo, t_hi, {item_rows, gate_up kernel, down kernel, router rows}}",
             "// (kernels: 0 pipelined, 128-row items, weights 1 chunk ahead; 1 pipelined, 64-row items, weights",
             "// 3 chunks ahead; 2 general).  Shapes, formats or token counts with no row take the default plan.",
             f"// Command: python -m mixture_experts_route_amd.tune --out PATH --tokens {args.tokens} "
             f"--reps {args.reps} --formats {args.formats}" + (f" --only {args.only}" if args.only else ""),
             "// Layer: hidden 2048, expert FFN 768, 512 experts top-10 + 1 shared, Zipf(1.1) routing; median",
             "// microseconds per moe_layer_forward call, candidate (item_rows, gate_up, down)."]
    for i, (fmt, T, best, best_r, res, r_res) in enumerate(rows):
        same = [r for r in rows if r[0] == fmt]
        j = same.index(rows[i])
        lo = 17 if j == 0 else int(math.floor(math.sqrt(same[j - 1][1] * T))) + 1
        hi = 2**31 - 1 if j == len(same) - 1 else int(math.floor(math.sqrt(T * same[j + 1][1])))
        meas = ", ".join(f"{c}: {v:.0f}" for c, v in sorted(res.items(), key=lambda kv: kv[1]))
        lines.append(f"// format {fmt}, T = {T}: {meas}; router rows 32: {r_res[32]:.0f}, 64: {r_res[64]:.0f}")
        lines.append(f"{{{H}, {F}, {E}, {K_TOP}, {fmt}, {lo}, {hi}, {{{best[0]}, {best[1]}, {best[2]}, {best_r}}}}},")
    with open(args.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"tune: wrote {args.out}", file=sys.stderr, flush=True)


if __name__ == "__main__":
    main()
