#!/usr/bin/env python3
"""Benchmark of the routed MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--prefill 4096,32768]

A step is one pass of the whole layer (router -> top-k -> residency check -> expert FFNs ->
combine) through ``moe_layer_forward`` over one batch of seeded synthetic input that is
already resident in HBM.  The default workload is single-token decode through one
model-shaped layer (512 routed experts top-10 + 1 shared, hidden 2048, expert FFN 768,
4-bit block-32 weights with fp16 scales), with a fresh bf16 token each step.

One JSON line is printed, with the live roofline of the dominant kernel (timed per launch
with HIP events recorded around that kernel alone) and the CPU oracle timed on a bounded
sample on this host.
"""

from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s at decode (HBM GB/s %) and 4K prefill (MFMA %), 1 GPU"
HBM_PEAK_GBS = 8000.0
FP16_MFMA_PEAK_TFLOPS = 2500.0

H, F, E, K_TOP = 2048, 768, 512, 10
X_STREAM = 1_000_000  # stream index of the benchmark's activations
POOL_SPARES = 4  # spare pinned host buffers per slot-pool layer (victims' copies out run ahead)


def _hip():
    import torch  # noqa: F401  (loads the HIP runtime the library binds to)

    lib = ctypes.CDLL("libamdhip64.so.7")
    lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
    lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return lib


class KernelTimer:
    """One (start, stop) hipEvent pair per timed step around the named kernel."""

    def __init__(self, n: int):
        self.hip = _hip()
        self.pairs = []
        for _ in range(n):
            a, b = ctypes.c_void_p(), ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(a)) == 0 and self.hip.hipEventCreate(ctypes.byref(b)) == 0
            self.pairs.append((a, b))

    def durations_ms(self):
        out = []
        for a, b in self.pairs:
            ms = ctypes.c_float()
            assert self.hip.hipEventSynchronize(b) == 0
            assert self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
            out.append(ms.value)
        return out

    def close(self):
        for a, b in self.pairs:
            self.hip.hipEventDestroy(a)
            self.hip.hipEventDestroy(b)


def hold_queue(ms: float):
    """Enqueues about `ms` of GPU work (a clock spin) on the current stream, so that the launches
    the host issues next queue up behind it and then run back to back, as in a graph replay,
    instead of each starting on an idle GPU (which lengthens the first kernel of every step)."""
    import torch

    sleep = getattr(torch.cuda, "_sleep", None)
    if sleep is None:
        return
    cyc = getattr(hold_queue, "cycles_per_ms", None)
    if cyc is None:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        sleep(1_000_000)
        b.record()
        b.synchronize()
        cyc = hold_queue.cycles_per_ms = 1_000_000 / max(a.elapsed_time(b), 1e-3)
    sleep(int(cyc * ms))


def host_cpu():
    """(CPU model name, logical CPUs) of this host."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return model, os.cpu_count()


def cpu_baseline_record(units: float, dt1: float, dtn: float, n: int, unit: str, sample: str, scale: float = 1.0):
    """The cpu_baseline object: `units` of work (tokens) in the timed sample, `scale` the factor from
    the sample to the reported unit (e.g. 4 of 48 layers -> 1/12)."""
    model, ncpu = host_cpu()
    return {"value": units * scale / dtn, "unit": unit, "cores": n, "kind": "oracle", "sample": sample,
            "value_1_thread": units * scale / dt1, "seconds_1_thread": dt1, "seconds_all_threads": dtn,
            "host_cpus": ncpu, "cpu_model": model,
            "oracle": "float64 numpy (library matmul steps threaded by its BLAS; the rest single-threaded)"}


def build_model_layer(device, seed=0, cfg=2, layer=0, bias_c=None, table_perm=True):
    """Arena of the 512 routed experts, the shared expert, bf16 router: all in HBM."""
    import numpy as np
    import torch

    from mixture_experts_route_amd import synth as S

    stride = (S.blob_bytes(H, F) + 4095) // 4096 * 4096
    arena = torch.empty((E, stride), dtype=torch.uint8, device=device)
    keys = [S.stream_key(seed, cfg, "blob", layer, e) for e in range(E)]
    rng = np.random.default_rng(seed + 1000 * layer)
    slot_of = rng.permutation(E) if table_perm else np.arange(E)
    tmp = torch.empty((64, stride), dtype=torch.uint8, device=device)
    for i in range(0, E, 64):
        S.expert_blobs_torch(keys[i:i + 64], H, F, tmp)
        idx = torch.as_tensor(slot_of[i:i + 64], device=device, dtype=torch.long)
        arena[idx] = tmp[:len(keys[i:i + 64])]
    shared = torch.empty((stride,), dtype=torch.uint8, device=device)
    S.expert_blobs_torch([S.stream_key(seed, cfg, "shared", layer, 0)], H, F, shared.view(1, -1))
    router = S.bf16_normal_torch(S.stream_key(seed, cfg, "router", layer, 0), (E, H), 0.02, device)
    bias = None
    if bias_c is not None:
        bias = torch.from_numpy(S.zipf_bias(S.rank_permutation(seed, cfg, layer, 0, E), bias_c)).to(device)
    table = torch.from_numpy(slot_of.astype(np.int32)).to(device)
    return dict(arena=arena, shared=shared, router=router, bias=bias, table=table, stride=stride, keys=keys,
                slot_of=slot_of, seed=seed, cfg=cfg, layer=layer)


# ---------------------------------------------------------------------------------------------
# CPU baseline: the oracle (as it stands) on the host, on 1 thread and on all cores
# ---------------------------------------------------------------------------------------------
def _oracle_job(kind: str, share):
    """Builds (untimed) the oracle's inputs for one share of a bounded sample and returns the timed
    part as a closure.  Shares: single-token decode steps, layers of one 8-token decode step, or
    tokens of a prefill batch; the same streams as the GPU run."""
    import numpy as np

    from mixture_experts_route_amd import synth as S
    from oracle import moe_oracle as O

    if kind == "decode1":
        seed, cfg, layer = 0, 2, 0
        steps = list(share)
        Wr = S.bf16_to_f32(S.bf16_normal_np(S.stream_key(seed, cfg, "router", layer, 0), (E, H), 0.02))
        Wr = Wr.astype(np.float64)
        shared = S.expert_blob_np(S.stream_key(seed, cfg, "shared", layer, 0), H, F)
        xall = S.bf16_to_f32(S.bf16_normal_np(S.stream_key(seed, cfg, "x", layer, X_STREAM), (max(steps) + 1, H), 1.0))
        xs = [xall[s:s + 1].astype(np.float64) for s in steps]
        need = set()
        for x in xs:
            need.update(int(e) for e in O.route(x, Wr, None, K_TOP)[2].ravel())
        blobs = {e: S.expert_blob_np(S.stream_key(seed, cfg, "blob", layer, e), H, F) for e in need}

        def run():
            for x in xs:
                O.moe_layer(x, Wr, None, K_TOP, lambda e: blobs[e], shared, H, F)
        return run
    if kind == "decode48":
        step, layers, T, seed, cfg = share[0], share[1], 8, 0, 3
        work = []
        for layer in layers:
            Wr = S.bf16_to_f32(S.bf16_normal_np(S.stream_key(seed, cfg, "router", layer, 0), (E, H), 0.02))
            Wr = Wr.astype(np.float64)
            bias = S.zipf_bias(S.rank_permutation(seed, cfg, layer, 0, E), S.ZIPF_C)
            xall = S.bf16_normal_np(S.stream_key(seed, cfg, "x", layer, X_STREAM), ((step + 1) * T, H), 1.0)
            x = S.bf16_to_f32(xall[step * T:(step + 1) * T]).astype(np.float64)
            ids = O.route(x, Wr, bias, K_TOP)[2]
            blobs = {int(e): S.expert_blob_np(S.stream_key(seed, cfg, "blob", layer, int(e)), H, F)
                     for e in np.unique(ids)}
            shared = S.expert_blob_np(S.stream_key(seed, cfg, "shared", layer, 0), H, F)
            work.append((x, Wr, bias, blobs, shared))

        def run():
            for x, Wr, bias, blobs, shared in work:
                O.moe_layer(x, Wr, bias, K_TOP, lambda e, b=blobs: b[e], shared, H, F)
        return run
    if kind == "prefill":
        T, lo, hi = share
        seed, cfg, layer = 0, 4, 0
        Wr = S.bf16_to_f32(S.bf16_normal_np(S.stream_key(seed, cfg, "router", layer, 0), (E, H), 0.02))
        Wr = Wr.astype(np.float64)
        bias = S.zipf_bias(S.rank_permutation(seed, cfg, layer, 0, E), S.ZIPF_C)
        shared = S.expert_blob_np(S.stream_key(seed, cfg, "shared", layer, 0), H, F)
        x = S.bf16_to_f32(S.bf16_normal_np(S.stream_key(seed, cfg, "x", layer, X_STREAM), (hi, H), 1.0))[lo:hi]
        x = x.astype(np.float64)
        ids = O.route(x, Wr, bias, K_TOP)[2]
        blobs = {int(e): S.expert_blob_np(S.stream_key(seed, cfg, "blob", layer, int(e)), H, F) for e in np.unique(ids)}

        def run():
            O.moe_layer(x, Wr, bias, K_TOP, lambda e: blobs[e], shared, H, F)
        return run
    raise ValueError(kind)


def _oracle_worker(kind, share, barrier, out):
    """One process of the all-cores run: inputs built before the barrier, one numerical thread."""
    from threadpoolctl import threadpool_limits

    run = _oracle_job(kind, share)
    with threadpool_limits(1):
        barrier.wait()
        t0 = time.monotonic()
        run()
        out.put((t0, time.monotonic()))


def time_oracle(kind: str, whole, shares):
    """Seconds for the sample `whole` on 1 thread in this process, and for the same sample split in
    `shares` over as many worker processes (spawned: fresh interpreters that never touch the GPU),
    wall time from the common start to the last finish.  Returns (t_1, t_all, processes)."""
    import multiprocessing as mp

    from threadpoolctl import threadpool_limits

    run = _oracle_job(kind, whole)
    with threadpool_limits(1):
        t0 = time.monotonic()
        run()
        dt1 = time.monotonic() - t0
    ctx = mp.get_context("spawn")
    barrier, out = ctx.Barrier(len(shares)), ctx.Queue()
    procs = [ctx.Process(target=_oracle_worker, args=(kind, sh, barrier, out)) for sh in shares]
    for p in procs:
        p.start()
    spans = [out.get(timeout=600) for _ in procs]
    for p in procs:
        p.join()
    return dt1, max(b for _, b in spans) - min(a for a, _ in spans), len(procs)


def _split(items, n):
    n = max(1, min(n, len(items)))
    return [items[i::n] for i in range(n)]


def cpu_baselines(workers: int, decode_steps: int = 24, prefill_tokens: int = 48, decode48_layers: int = 4):
    """The oracle timed on bounded samples of the benchmark's workloads (data generation excluded),
    on 1 thread and on `workers` processes; one record per workload."""
    out = {}
    steps = list(range(50, 50 + decode_steps))  # the bench's first timed steps (after 50 warmup)
    dt1, dtn, n = time_oracle("decode1", steps, [sorted(sh) for sh in _split(steps, workers)])
    out["decode1"] = cpu_baseline_record(
        decode_steps, dt1, dtn, n, "tokens/s",
        f"{decode_steps} single-token steps of the same layer and token stream: {dt1:.1f} s on 1 thread, "
        f"{dtn:.1f} s on {n} processes (steps split between them)")
    layers = list(range(max(decode48_layers, workers)))
    dt1, dtn, n = time_oracle("decode48", (4, layers[:decode48_layers]),
                              [(4, sorted(sh)) for sh in _split(layers, workers)])
    # 1 thread: `decode48_layers` layers; all cores: len(layers) layers; both scaled to 48 layers
    rec = cpu_baseline_record(8, dtn, dtn, n, "tokens/s",
                              f"one 8-token step through {len(layers)} of the 48 layers on {n} processes (a layer "
                              f"each) in {dtn:.1f} s, and through {decode48_layers} layers on 1 thread in {dt1:.1f} s; "
                              f"both scaled to 48 layers", scale=len(layers) / 48)
    rec["value_1_thread"] = 8 * decode48_layers / 48 / dt1
    rec["seconds_1_thread"] = dt1
    out["decode48"] = rec
    toks = list(range(prefill_tokens))
    chunks = [(4096, c[0], c[-1] + 1) for c in
              [toks[i:i + max(1, prefill_tokens // workers)] for i in range(0, prefill_tokens, max(1, prefill_tokens // workers))]]
    dt1, dtn, n = time_oracle("prefill", (4096, 0, prefill_tokens), chunks)
    out["prefill"] = cpu_baseline_record(
        prefill_tokens, dt1, dtn, n, "tokens/s",
        f"first {prefill_tokens} tokens of the 4096-token batch: {dt1:.1f} s on 1 thread in one oracle call, "
        f"{dtn:.1f} s on {n} processes (consecutive token runs)")
    return out


def measured_traffic(path="profiles/decode1_gate_up_traffic.txt"):
    """HBM bytes per launch of a gate/up kernel (decode or prefill) from a committed rocprofv3 counter
    summary (FETCH_SIZE and WRITE_SIZE passes, scaled by a plain copy; the mean over the launches),
    or None once the kernel's sources differ from the ones the counters were taken on."""
    import hashlib

    root = os.path.dirname(os.path.abspath(__file__))
    try:
        fields = {}
        for line in open(os.path.join(root, path)):
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
        h = hashlib.sha256()
        for f in fields["source_files"].split():
            h.update(open(os.path.join(root, f), "rb").read())
        if h.hexdigest() != fields["source_sha256"]:
            return None
        return float(fields["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def bench_decode1(args):
    import numpy as np
    import torch

    from mixture_experts_route_amd import native as N
    from mixture_experts_route_amd import synth as S

    dev = torch.device("cuda:0")
    L = build_model_layer(dev)
    d = N.dims(H, F, E, K_TOP, 1)
    w = N.layer_weights(L["router"], L["arena"], L["stride"], E, L["shared"], L["bias"])
    n_steps = args.warmup + args.steps
    # fresh bf16 token per step, all resident before timing
    xs = S.bf16_normal_torch(S.stream_key(0, 2, "x", 0, X_STREAM), (n_steps, H), 1.0, dev)
    y = torch.empty((1, H), dtype=torch.float32, device=dev)
    ws = torch.zeros(N.moe_workspace_bytes(d, 1) // 4 + 64, dtype=torch.int32, device=dev)
    N.moe_workspace_init(ws)
    ids = torch.empty((1, K_TOP), dtype=torch.int32, device=dev)
    tw = torch.empty((1, K_TOP), dtype=torch.float32, device=dev)
    st = torch.cuda.Stream()

    def steps_on(stream, first, count):
        for i in range(count):
            s = first + i
            N.moe_layer_forward(d, w, L["table"], xs[s:s + 1], 1, y, ws, topk_ids=ids, topk_w=tw, stream=stream)

    torch.cuda.synchronize()
    if args.eager:
        with torch.cuda.stream(st):
            steps_on(st, 0, args.warmup)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        with torch.cuda.stream(st):
            steps_on(st, args.warmup, args.steps)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    else:
        # a decode step is a handful of short kernels: the steps are captured in HIP graphs (one for
        # the warmup steps, one for the timed steps, each step with its own token) and replayed, so the
        # host's launch rate does not set the pace
        gw, gt = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        with torch.cuda.graph(gw, stream=st):
            steps_on(torch.cuda.current_stream(), 0, args.warmup)
        with torch.cuda.graph(gt, stream=st):
            steps_on(torch.cuda.current_stream(), args.warmup, args.steps)
        torch.cuda.synchronize()
        gw.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        gt.replay()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    assert N.moe_check_device_error(ws) == 0
    elapsed = t1 - t0
    ms_per_step = elapsed * 1e3 / args.steps

    # per-kernel durations of the gate/up and down launches: HIP events around the kernel itself, on
    # the stream it runs on, over second (eager) passes of the same steps queued behind a hold (so
    # that they run back to back)
    n_k = min(args.steps, 200)

    def kernel_ms(which):
        timer = KernelTimer(n_k)
        torch.cuda.synchronize()
        with torch.cuda.stream(st):
            hold_queue(40.0)
            for i in range(n_k):
                s = args.warmup + i
                N.moe_debug_kernel_events(which, timer.pairs[i][0], timer.pairs[i][1])
                N.moe_layer_forward(d, w, L["table"], xs[s:s + 1], 1, y, ws, topk_ids=ids, topk_w=tw, stream=st)
        torch.cuda.synchronize()
        N.moe_debug_kernel_events(0, None, None)
        assert N.moe_check_device_error(ws) == 0
        out = timer.durations_ms()
        timer.close()
        return out

    k_ms = kernel_ms(N.TIME_DECODE_GATE_UP)
    dn_ms = kernel_ms(N.TIME_DECODE_DOWN)
    # algorithmic bytes of one gate/up launch: 11 experts (10 routed, distinct, + shared), each
    # reading its gate and up codes and scales once, plus x in and h out (bf16 hi + lo)
    per_expert = 2 * (F * H // 2 + F * (H // 32) * 2)
    # (+ the router's logits and the slot table, which every workgroup reads for its selection)
    gu_bytes = 11 * per_expert + H * 2 + 11 * F * 4 + E * 4 * 2
    gu_avg_s = float(np.mean(k_ms)) * 1e-3
    achieved = gu_bytes / gu_avg_s / 1e9
    # down (one token: the weighted combine is inside the launch): the 11 experts' down codes and
    # scales, h in, y out
    dn_bytes = 11 * (H * F // 2 + H * (F // 32) * 2) + 11 * F * 4 + H * 4
    dn_avg_s = float(np.mean(dn_ms)) * 1e-3
    result = {
        "metric": METRIC,
        "value": args.steps / elapsed,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 x int4 -> f32",
        "data": "synthetic",
        "config": {
            "workload": "single-token decode through one layer: 512 routed experts top-10 + 1 shared, hidden 2048, "
                        "expert FFN 768, SwiGLU, 4-bit block-32 weights with fp16 scales, bf16 activations N(0,1), "
                        "bf16 router N(0,0.02), all experts resident behind a permuted slot table; fresh token per step",
            "tokens_per_step": 1,
            "layer_bytes_per_step": 11 * 2_654_208 + E * H * 2 + H * 2 + H * 4,
        },
        "roofline": {
            "kernel": "k_decode_gate_up (4-bit GEMV gate+up, SwiGLU fused; each workgroup first selects the token's top-k from the logits)",
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": measured_traffic(),
            "bytes_per_launch": gu_bytes,
            "avg_launch_us": gu_avg_s * 1e6,
        },
        "decode_down": {"bytes_per_launch": dn_bytes, "avg_launch_us": dn_avg_s * 1e6,
                        "achieved_gbs": dn_bytes / dn_avg_s / 1e9, "frac": dn_bytes / dn_avg_s / 1e9 / HBM_PEAK_GBS},
        # expert-FFN HBM fraction: both FFN kernels' algorithmic bytes over their summed time
        "decode_ffn_hbm_frac": (gu_bytes + dn_bytes) / (gu_avg_s + dn_avg_s) / 1e9 / HBM_PEAK_GBS,
        "timed_region": "eager launches" if args.eager else "HIP graph replay of the timed steps",
    }
    if args.cpu:
        result["cpu_baseline"] = args.cpu["decode1"]
    return result


def bench_prefill(T: int, steps: int, warmup: int, cpu_baseline: dict | None):
    """T-token prefill through one model-shaped layer with Zipf(1.1)-skewed routing."""
    import numpy as np
    import torch

    from mixture_experts_route_amd import native as N
    from mixture_experts_route_amd import synth as S

    dev = torch.device("cuda:0")
    L = build_model_layer(dev, cfg=4, bias_c=S.ZIPF_C)
    d = N.dims(H, F, E, K_TOP, 1)
    w = N.layer_weights(L["router"], L["arena"], L["stride"], E, L["shared"], L["bias"])
    n_batches = 2
    xs = [S.bf16_normal_torch(S.stream_key(0, 4, "x", 0, X_STREAM + b), (T, H), 1.0, dev) for b in range(n_batches)]
    y = torch.empty((T, H), dtype=torch.float32, device=dev)
    ws = torch.zeros(N.moe_workspace_bytes(d, T) // 4 + 64, dtype=torch.int32, device=dev)
    N.moe_workspace_init(ws)
    ids = torch.empty((T, K_TOP), dtype=torch.int32, device=dev)
    for s in range(warmup):
        N.moe_layer_forward(d, w, L["table"], xs[s % n_batches], T, y, ws, topk_ids=ids)
    torch.cuda.synchronize()
    assert N.moe_check_device_error(ws) == 0
    timer = KernelTimer(steps)
    st = torch.cuda.current_stream()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        which = N.TIME_PREFILL_GATE_UP if i % 2 == 0 else N.TIME_PREFILL_DOWN
        N.moe_debug_kernel_events(which, timer.pairs[i][0], timer.pairs[i][1])
        N.moe_layer_forward(d, w, L["table"], xs[i % n_batches], T, y, ws, topk_ids=ids, stream=st)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    N.moe_debug_kernel_events(0, None, None)
    assert N.moe_check_device_error(ws) == 0
    k_ms = timer.durations_ms()
    timer.close()
    gu_s = float(np.mean(k_ms[0::2])) * 1e-3
    dn_s = float(np.mean(k_ms[1::2])) * 1e-3 if steps > 1 else float("nan")
    rows = T * (K_TOP + 1)
    gu_flop = rows * 2.0 * (2 * F) * H
    dn_flop = rows * 2.0 * H * F
    cnt = np.bincount(ids.cpu().numpy().ravel(), minlength=E)
    elapsed = t1 - t0
    out = {
        "workload": f"{T}-token prefill through one layer: 512 routed experts top-10 + 1 shared, hidden 2048, "
                    f"expert FFN 768, 4-bit block-32 weights dequantized to fp16 in registers, fp16 MFMA with fp32 "
                    f"accumulation, bf16 activations N(0,1), Zipf(1.1)-skewed routing",
        "tokens_per_s": T * steps / elapsed,
        "ms_per_step": elapsed * 1e3 / steps,
        "groups": {"max": int(cnt.max()), "median": float(np.median(cnt)), "under_16": int((cnt < 16).sum())},
        "expert_gflop_per_step": (gu_flop + dn_flop) / 1e9,
        "roofline": {
            "kernel": "k_expert_gemm<gate/up> (grouped GEMM, SwiGLU epilogue)",
            "bound": "mfma",
            "achieved": gu_flop / gu_s / 1e12,
            "peak": FP16_MFMA_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": gu_flop / gu_s / 1e12 / FP16_MFMA_PEAK_TFLOPS,
            "traffic": measured_traffic("profiles/prefill4k_gate_up_traffic.txt") if T == 4096 else None,
            "flop_per_launch": gu_flop,
            "avg_launch_us": gu_s * 1e6,
        },
        "down_gemm": {"achieved_tflops": dn_flop / dn_s / 1e12, "avg_launch_us": dn_s * 1e6,
                      "frac": dn_flop / dn_s / 1e12 / FP16_MFMA_PEAK_TFLOPS},
        "both_gemms_mfma_frac": (gu_flop + dn_flop) / (gu_s + dn_s) / 1e12 / FP16_MFMA_PEAK_TFLOPS,
    }
    if cpu_baseline:
        out["cpu_baseline"] = cpu_baseline
    return out


def bench_decode48(steps: int, warmup: int, graph: bool, time_steps: int = 4, cpu_baseline: dict | None = None):
    """Batched decode through all 48 layers: 8 tokens per step, every layer's 512 + 1 experts resident
    in HBM (one 65 GB arena), per-layer Zipf(1.1) router bias, fresh seeded tokens per (step, layer)."""
    import numpy as np
    import torch

    from mixture_experts_route_amd import native as N
    from mixture_experts_route_amd import synth as S

    dev = torch.device("cuda:0")
    n_layers, T, cfg = 48, 8, 3
    stride = (S.blob_bytes(H, F) + 4095) // 4096 * 4096
    per_layer = E + 1  # routed experts in slots 0..E-1, the shared expert after them
    arena = torch.empty((n_layers * per_layer, stride), dtype=torch.uint8, device=dev)
    for layer in range(n_layers):
        keys = [S.stream_key(0, cfg, "blob", layer, e) for e in range(E)] + [S.stream_key(0, cfg, "shared", layer, 0)]
        S.expert_blobs_torch_batch(keys, H, F, arena[layer * per_layer:(layer + 1) * per_layer])
        if layer % 12 == 11:
            torch.cuda.synchronize()
            print(f"bench: 48-layer arena, {layer + 1} layers generated", file=sys.stderr, flush=True)
    routers = [S.bf16_normal_torch(S.stream_key(0, cfg, "router", layer, 0), (E, H), 0.02, dev)
               for layer in range(n_layers)]
    biases = [torch.from_numpy(S.zipf_bias(S.rank_permutation(0, cfg, layer, 0, E), S.ZIPF_C)).to(dev)
              for layer in range(n_layers)]
    n_steps = warmup + steps
    xs = [S.bf16_normal_torch(S.stream_key(0, cfg, "x", layer, X_STREAM), (n_steps * T, H), 1.0, dev)
          for layer in range(n_layers)]
    d = N.dims(H, F, E, K_TOP, 1)
    ws_t = [N.layer_weights(routers[l], arena[l * per_layer:], stride, E, arena[l * per_layer + E], biases[l])
            for l in range(n_layers)]
    y = torch.empty((T, H), dtype=torch.float32, device=dev)
    ws = torch.zeros(N.moe_workspace_bytes(d, T) // 4 + 64, dtype=torch.int32, device=dev)
    N.moe_workspace_init(ws)
    st = torch.cuda.Stream()

    def run_steps(stream, first, count, ids_out=None):
        for i in range(count):
            s = first + i
            for layer in range(n_layers):
                ids = ids_out[i][layer] if ids_out is not None else None
                N.moe_layer_forward(d, ws_t[layer], None, xs[layer][s * T:(s + 1) * T], T, y, ws, topk_ids=ids,
                                    stream=stream)

    torch.cuda.synchronize()
    if graph:
        chunk = 16
        graphs = []
        for first in range(warmup, warmup + steps, chunk):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=st):
                run_steps(torch.cuda.current_stream(), first, min(chunk, warmup + steps - first))
            graphs.append(g)
        with torch.cuda.stream(st):
            run_steps(st, 0, warmup)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for g in graphs:
            g.replay()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    else:
        with torch.cuda.stream(st):
            run_steps(st, 0, warmup)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        with torch.cuda.stream(st):
            run_steps(st, warmup, steps)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    assert N.moe_check_device_error(ws) == 0
    elapsed = t1 - t0

    # per-kernel durations (HIP events around each gate/up and down launch of `time_steps` eager steps)
    # and the algorithmic bytes of each launch from its own routing (distinct experts U + shared)
    ids_out = [[torch.empty((T, K_TOP), dtype=torch.int32, device=dev) for _ in range(n_layers)]
               for _ in range(time_steps)]
    res_k = {}
    for which in (N.TIME_DECODE_GATE_UP, N.TIME_DECODE_DOWN):
        timer = KernelTimer(time_steps * n_layers)
        torch.cuda.synchronize()
        with torch.cuda.stream(st):
            hold_queue(40.0)
            for i in range(time_steps):
                for layer in range(n_layers):
                    pr = timer.pairs[i * n_layers + layer]
                    N.moe_debug_kernel_events(which, pr[0], pr[1])
                    s = warmup + i
                    N.moe_layer_forward(d, ws_t[layer], None, xs[layer][s * T:(s + 1) * T], T, y, ws,
                                        topk_ids=ids_out[i][layer], stream=st)
        torch.cuda.synchronize()
        N.moe_debug_kernel_events(0, None, None)
        res_k[which] = timer.durations_ms()
        timer.close()
    assert N.moe_check_device_error(ws) == 0
    u = np.array([len(np.unique(ids_out[i][l].cpu().numpy())) for i in range(time_steps) for l in range(n_layers)])
    gu_exp = 2 * (F * H // 2 + F * (H // 32) * 2)
    dn_exp = H * F // 2 + H * (F // 32) * 2
    pairs = T * (K_TOP + 1)
    gu_bytes = (u + 1) * gu_exp + T * H * 2 + pairs * F * 4
    dn_bytes = (u + 1) * dn_exp + pairs * F * 4 + pairs * H * 4
    gu_s = np.array(res_k[N.TIME_DECODE_GATE_UP]) * 1e-3
    dn_s = np.array(res_k[N.TIME_DECODE_DOWN]) * 1e-3
    gu_gbs = gu_bytes.sum() / gu_s.sum() / 1e9
    dn_gbs = dn_bytes.sum() / dn_s.sum() / 1e9
    ffn_gbs = (gu_bytes.sum() + dn_bytes.sum()) / (gu_s.sum() + dn_s.sum()) / 1e9
    step_bytes = float(np.mean(u + 1)) * 2_654_208 * n_layers + n_layers * (E * H * 2)
    out = {
        "workload": "batched decode through 48 layers: 8 tokens per step, 48 x (512 routed + 1 shared) experts "
                    "resident in HBM (65.4 GB of 4-bit weights), per-layer Zipf(1.1) router bias, top-10 + shared, "
                    "hidden 2048, expert FFN 768, fresh bf16 tokens per (step, layer)",
        "tokens_per_s": T * steps / elapsed,
        "ms_per_step": elapsed * 1e3 / steps,
        "steps": steps,
        "timed_region": "HIP graph replay of the timed steps" if graph else "eager launches",
        "distinct_experts_per_layer": float(np.mean(u)),
        "approx_weight_bytes_per_step": step_bytes,
        "roofline": {
            "kernel": "k_decode_gate_up (matrix-core 4-bit GEMV gate+up, SwiGLU fused), 8 tokens",
            "bound": "hbm",
            "achieved": gu_gbs,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": gu_gbs / HBM_PEAK_GBS,
            "traffic": measured_traffic("profiles/decode48_gate_up_traffic.txt"),
            "bytes_per_launch": float(gu_bytes.mean()),
            "avg_launch_us": float(gu_s.mean() * 1e6),
        },
        "decode_down": {"achieved_gbs": dn_gbs, "frac": dn_gbs / HBM_PEAK_GBS, "bytes_per_launch": float(dn_bytes.mean()),
                        "avg_launch_us": float(dn_s.mean() * 1e6)},
        "decode_ffn_hbm_frac": ffn_gbs / HBM_PEAK_GBS,
    }
    if cpu_baseline:
        out["cpu_baseline"] = cpu_baseline
    return out


def pool_slots(layer: int) -> int:
    """HBM slots of a layer in the slot-pool workload: 240 / 92 / 60 for early / middle / late
    layers (10 x 240 + 10 x 92 + 28 x 60 = 5,000)."""
    return 240 if layer < 10 else 92 if layer < 20 else 60


def bench_pool(steps: int, streams, topic_every: int = 128, n_layers: int = 48):
    """Single-token decode through 48 layers whose experts live in 5,000 HBM slots and pinned host
    memory (exclusive tiers); per-layer Zipf(1.1) bias redrawn every `topic_every` steps; misses
    filled from the host by the pool service on a copy stream."""
    import numpy as np
    import torch

    from mixture_experts_route_amd import native as N
    from mixture_experts_route_amd import synth as S

    dev = torch.device("cuda:0")
    cfg, T = 5, 1
    stride = (S.blob_bytes(H, F) + 4095) // 4096 * 4096
    blob = S.blob_bytes(H, F)
    d = N.dims(H, F, E, K_TOP, 1)
    n_topics = (steps + 2 + topic_every - 1) // topic_every + 1
    layers = []
    tmp = torch.empty((E, stride), dtype=torch.uint8, device=dev)
    for layer in range(n_layers):
        keys = [S.stream_key(0, cfg, "blob", layer, e) for e in range(E)]
        S.expert_blobs_torch_batch(keys, H, F, tmp)
        ranks = [S.rank_permutation(0, cfg, layer, t, E) for t in range(n_topics)]
        n_slots = pool_slots(layer)
        initial = [int(e) for e in np.argsort(ranks[0], kind="stable")[:n_slots]]
        arena = tmp[torch.as_tensor(initial, device=dev, dtype=torch.long)].contiguous()
        away = [e for e in range(E) if e not in set(initial)]
        homes = N.HostBuffer((len(away) + POOL_SPARES) * stride, flags=0)
        hv = torch.from_numpy(homes.view(np.uint8)).view(len(away) + POOL_SPARES, stride)
        hv[:len(away)].copy_(tmp[torch.as_tensor(away, device=dev, dtype=torch.long)])
        home_addr = [0] * E
        for i, e in enumerate(away):
            home_addr[e] = homes.ptr + i * stride
        shared = torch.empty((stride,), dtype=torch.uint8, device=dev)
        S.expert_blobs_torch([S.stream_key(0, cfg, "shared", layer, 0)], H, F, shared.view(1, -1))
        router = S.bf16_normal_torch(S.stream_key(0, cfg, "router", layer, 0), (E, H), 0.02, dev)
        biases = [torch.from_numpy(S.zipf_bias(r, S.ZIPF_C)).to(dev) for r in ranks]
        table = torch.full((E,), -1, dtype=torch.int32, device=dev)
        ready = torch.zeros((64,), dtype=torch.int32, device=dev)
        hb = [N.HostBuffer(4 * E), N.HostBuffer(64), N.HostBuffer(4 * N.MOE_DECODE_MAX_TOKENS * K_TOP)]
        pool = N.moe_pool_create(d, arena, stride, n_slots, table, initial, home_addr, homes.ptr + len(away) * stride,
                                 POOL_SPARES, hb[0].ptr, hb[1].ptr, hb[2].ptr, ready)
        layers.append(dict(arena=arena, homes=homes, shared=shared, router=router, biases=biases, table=table,
                           ready=ready, hb=hb, pool=pool, n_slots=n_slots))
    del tmp
    torch.cuda.empty_cache()
    xs = [S.bf16_normal_torch(S.stream_key(0, cfg, "x", layer, X_STREAM), (steps + 2, H), 1.0, dev)
          for layer in range(n_layers)]
    y = torch.empty((T, H), dtype=torch.float32, device=dev)
    ws = torch.zeros(N.moe_workspace_bytes(d, T) // 4 + 64, dtype=torch.int32, device=dev)
    N.moe_workspace_init(ws)
    compute, d2h, h2d = streams

    def step(s):
        topic = s // topic_every
        for layer, L in enumerate(layers):
            bell = N.moe_pool_arm(L["pool"])
            w = N.layer_weights(L["router"], L["arena"], stride, L["n_slots"], L["shared"], L["biases"][topic])
            N.moe_layer_forward(d, w, L["table"], xs[layer][s:s + 1], T, y, ws, bell=bell, stream=compute)
        for i, L in enumerate(layers):
            try:
                N.moe_pool_serve(L["pool"], ws, d2h, h2d_stream=h2d)
            except N.MoeError:
                # a stream that waits on the pool cannot drain once its fill failed: report and leave
                # without the runtime's teardown (which would wait for that stream)
                print(f"bench: slot-pool step {s} layer {i}: serve failed; control words "
                      f"{ws[:8].cpu().tolist()}", file=sys.stderr, flush=True)
                os._exit(3)

    torch.cuda.synchronize()
    for s in range(2):
        step(s)
    compute.synchronize()
    st0 = [N.moe_pool_get_stats(L["pool"]) for L in layers]
    t0 = time.perf_counter()
    for s in range(2, steps + 2):
        step(s)
    compute.synchronize()
    d2h.synchronize()
    h2d.synchronize()
    t1 = time.perf_counter()
    assert N.moe_check_device_error(ws) == 0
    st1 = [N.moe_pool_get_stats(L["pool"]) for L in layers]
    # run 2: the same steps again (same tokens and topics) on the pool as run 1 left it
    r0 = time.perf_counter()
    for s in range(2, steps + 2):
        step(s)
    compute.synchronize()
    d2h.synchronize()
    h2d.synchronize()
    r1 = time.perf_counter()
    assert N.moe_check_device_error(ws) == 0
    st2 = [N.moe_pool_get_stats(L["pool"]) for L in layers]
    # the standalone residency check of one token's selections (two launches: slots and miss flags,
    # then the ascending miss list), back to back on the compute stream
    L0 = layers[0]
    chk_ids = torch.as_tensor([[int(v) for v in range(0, 10 * 37, 37)]], dtype=torch.int32, device=dev)
    chk_slots = torch.empty((1, K_TOP), dtype=torch.int32, device=dev)
    chk_miss = torch.empty((E,), dtype=torch.int32, device=dev)
    chk_count = torch.empty((1,), dtype=torch.int32, device=dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    with torch.cuda.stream(compute):
        for rep in range(2):
            if rep:
                ev[0].record()
            for _ in range(200):
                N.moe_slot_lookup(d, L0["table"], L0["n_slots"], chk_ids, T, chk_slots, chk_miss, chk_count, ws,
                                  stream=compute)
        ev[1].record()
    ev[1].synchronize()
    check_us = ev[0].elapsed_time(ev[1]) * 1e3 / 200
    sel2 = sum(b.selections - a.selections for a, b in zip(st1, st2))
    mis2 = sum(b.misses - a.misses for a, b in zip(st1, st2))
    sel = sum(b.selections - a.selections for a, b in zip(st0, st1))
    mis = sum(b.misses - a.misses for a, b in zip(st0, st1))
    b_h2d = sum(b.bytes_h2d - a.bytes_h2d for a, b in zip(st0, st1))
    b_d2h = sum(b.bytes_d2h - a.bytes_d2h for a, b in zip(st0, st1))
    # pinned host <-> HBM copy rate for one expert blob, same process (the fills' bound)
    hb = N.HostBuffer(blob * 8, flags=0)
    dbuf = torch.empty((blob * 8,), dtype=torch.uint8, device=dev)
    hip = N._hiprt()
    hip.hipMemcpyAsync.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
    rates = {}
    for kind, name in ((1, "h2d"), (2, "d2h")):
        torch.cuda.synchronize()
        c0 = time.perf_counter()
        for rep in range(8):
            dst = dbuf.data_ptr() + rep * blob if kind == 1 else hb.ptr + rep * blob
            src = hb.ptr + rep * blob if kind == 1 else dbuf.data_ptr() + rep * blob
            hip.hipMemcpyAsync(dst, src, blob, kind, d2h.cuda_stream)
        d2h.synchronize()
        rates[name] = 8 * blob / (time.perf_counter() - c0) / 1e9
    hb.free()
    for L in layers:
        N.moe_pool_destroy(L["pool"])
    elapsed = t1 - t0
    return {
        "workload": "single-token decode through 48 layers with 5,000 HBM expert slots (240 / 92 / 60 per early / "
                    "middle / late layer) and the other 19,576 experts in pinned host memory (exclusive tiers); "
                    f"per-layer Zipf(1.1) router bias with a topic shift every {topic_every} steps; misses filled "
                    "by the host pool service (victims out on one copy stream, misses in on another, "
                    f"{POOL_SPARES} spare host buffers) while the compute stream waits in-stream",
        "tokens_per_s": steps / elapsed,
        "ms_per_token": elapsed * 1e3 / steps,
        "steps": steps,
        "hit_rate": 1.0 - mis / max(1, sel),
        "misses_per_token": mis / steps,
        "pcie_mib_per_token": (b_h2d + b_d2h) / steps / 2**20,
        "pcie_rate_gbs_per_blob_copy": rates,
        "fill_time_serial_ms_per_token": (b_h2d / rates["h2d"] + b_d2h / rates["d2h"]) / 1e6 / steps,
        "fill_time_overlapped_ms_per_token": max(b_h2d / rates["h2d"], b_d2h / rates["d2h"]) / 1e6 / steps,
        "check_us_standalone": check_us,
        "run2": {"what": "the same steps again on the pool as run 1 left it",
                 "tokens_per_s": steps / (r1 - r0), "hit_rate": 1.0 - mis2 / max(1, sel2),
                 "misses_per_token": mis2 / steps},
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="decode1", choices=["decode1"])
    ap.add_argument("--cpu-sample", type=int, default=24)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true", help="launch decode steps one by one instead of replaying graphs")
    ap.add_argument("--prefill", default="4096,32768", help="comma-separated prefill token counts to add ('' = none)")
    ap.add_argument("--prefill-steps", type=int, default=20)
    ap.add_argument("--decode48-steps", type=int, default=256, help="steps of the 48-layer batched decode (0 = skip)")
    ap.add_argument("--pool-steps", type=int, default=512, help="steps of the slot-pool decode workload (0 = skip)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run plain 256 MiB device copies (scale for the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the layer's data-parallel scale-out has no exchange on the path, "
              "so only --gpus 1 is run here", file=sys.stderr)
        sys.exit(2)
    def progress(msg):
        print(f"bench: {msg}", file=sys.stderr, flush=True)

    # the CPU baseline first, before this process touches the GPU (its workers are spawned
    # interpreters that never do)
    args.cpu = {}
    if not args.no_cpu_baseline:
        progress("CPU baseline (oracle)")
        args.cpu = cpu_baselines(min(16, os.cpu_count() or 1), decode_steps=args.cpu_sample)

    # The slot pool's compute and two copy streams are created first, while no other stream exists:
    # the runtime spreads streams over a few hardware queues, and the compute stream's in-stream
    # wait must not sit in front of the copies on a shared queue.
    pool_streams = None
    if args.pool_steps > 0:
        from mixture_experts_route_amd import native as N

        pool_streams = (N.new_stream(), N.new_stream(), N.new_stream())
    progress("single-token decode")
    res = bench_decode1(args)
    if args.copy_calibration:
        import torch

        a = torch.empty(256 << 20, dtype=torch.uint8, device="cuda:0").fill_(1)
        b = torch.empty_like(a)
        for _ in range(4):
            b.copy_(a)
        torch.cuda.synchronize()
        res["copy_calibration_bytes"] = 256 << 20
    if args.decode48_steps > 0:
        progress("48-layer batched decode")
        res["decode_8tok_48layers"] = bench_decode48(args.decode48_steps, 4, not args.eager,
                                                     cpu_baseline=args.cpu.get("decode48"))
        import torch

        torch.cuda.empty_cache()
    if args.pool_steps > 0:
        progress("slot-pool decode")
        res["decode_slot_pool_48layers"] = bench_pool(args.pool_steps, pool_streams)
    for T in [int(v) for v in args.prefill.split(",") if v.strip()]:
        steps = args.prefill_steps if T <= 8192 else max(4, args.prefill_steps // 4)
        progress(f"{T}-token prefill")
        base = args.cpu.get("prefill")
        if base and T != 4096:
            # the oracle's time is linear in the tokens (each token's experts, one after another): a
            # batch of T tokens runs at the sampled rate and takes T / 4096 times as long as 4096
            base = dict(base, sample=f"extrapolated from the 4096-token batch's sample ({base['sample']}): the "
                                     f"oracle's time is linear in the tokens, so {T} tokens take {T / 4096:g}x the "
                                     f"time of 4096")
        res[f"prefill_{T}"] = bench_prefill(T, steps, max(2, steps // 5), base)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
