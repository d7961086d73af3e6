"""Benchmark of one routed-expert MoE layer on one MI355X.

Workload: the Qwen3-30B-A3B-shaped MoE layer at decode (hidden 2048, 128
routed experts, top-8 softmax renormalised, SwiGLU intermediate 768, Q4_K
expert weights, no shared expert), batch of T tokens (default 2).  A step is
one pass of the whole layer: route -> batches -> expert FFN (activation
records, gate/up + SwiGLU GEMV, down GEMV) -> combine.

Inputs are seeded and synthetic and already resident in HBM when timing
starts.  The slot pool is replicated (16 copies by default) and step i uses
copy i mod 16 with input batch i mod 16, so a weight byte is read again only
after ~15 other steps' weights have streamed through; the 256 MB Infinity
Cache cannot serve it and the GEMV reads HBM.

Printed: one JSON line with the throughput of the timed region (K steps of
hipGraph replays, one graph per step, bracketed by synchronisation), the
roofline of the dominant kernel (the gate/up GEMV: algorithmic bytes =
selected experts' gate and up weights, over its duration in an eager pass of
the same K steps, from HIP events attached to its dispatches on the launch
stream), and the CPU oracle timed on a bounded
sample of the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
METRIC = "MoE-layer tokens/s + achieved HBM GB/s (decode) / MFMA util (prefill), 1 GPU"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_ffn_gateup_q4k_qwen3_decode.txt")
# sources the decode gate/up kernel is compiled from (the traffic figures are
# valid only for exactly these)
KERNEL_SOURCES = [os.path.join(ROOT, "quantized_routed_expert_moe_amd", "csrc", f)
                  for f in ("ffn_decode.hip", "device_common.h", "qmoe_internal.h")]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--tokens", type=int, default=2, choices=[1, 2])
    ap.add_argument("--copies", type=int, default=16, help="slot-pool replicas rotated over the steps")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="bounded CPU-oracle sample (wall seconds)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--prefill-steps", type=int, default=30,
                    help="timed steps of the T=4096 prefill layer reported beside the decode line (0 = skip)")
    ap.add_argument("--dsv3-steps", type=int, default=400,
                    help="timed steps of the DeepSeek-V3-shaped decode layer at T=2 and T=4 (0 = skip)")
    ap.add_argument("--residency-steps", type=int, default=96,
                    help="decode steps per arm of the adaptive residency run on the stack (0: skip it)")
    ap.add_argument("--stack-replays", type=int, default=10,
                    help="timed replays of the 58-layer partial-residency stack (0 = skip)")
    ap.add_argument("--profile-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration under rocprofv3)")
    return ap.parse_args()


def source_hash(paths: list) -> str:
    h = hashlib.sha256()
    for p in paths:
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def read_traffic() -> dict | None:
    """HBM bytes per launch of the gate/up kernel from committed rocprofv3
    --pmc summaries, valid only for the kernel source they were taken on."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if "=" in line and not line.startswith("#"):
            key, val = line.split("=", 1)
            kv[key.strip()] = val.strip()
    if kv.get("kernel_source_sha256_16") != source_hash(KERNEL_SOURCES):
        return None
    try:
        return dict(bytes_per_launch=float(kv["hbm_bytes_per_launch"]), note=kv.get("note", ""))
    except KeyError:
        return None


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: every box here has one MI355X and the layer's kernels run on one device; "
              f"--gpus {args.gpus} is not supported.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import fixtures as F
    import quantized_routed_expert_moe_amd as Q
    from fixtures import workloads as W
    from quantized_routed_expert_moe_amd.layer import LayerSpec, MoELayer

    Q.lib()  # fail loudly if the HIP library is missing
    assert torch.cuda.is_available()
    wl = W.QWEN3_DECODE_T2 if args.tokens == 2 else W.QWEN3_DECODE_T1
    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    F.set_num_threads(threads)

    # ---- inputs: weights, packed pool copies, input batches
    t0 = time.time()
    blobs = W.expert_blobs(wl)
    nb = Q.moe_expert_blob_bytes(wl.fmt, wl.H, wl.I)
    stride = (nb + 255) // 256 * 256
    host = np.zeros((wl.E, stride), dtype=np.uint8)
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(lambda e: Q.moe_pack_expert(wl.fmt, blobs[e], wl.H, wl.I, out=host[e, :nb]), range(wl.E)))
    pool0 = torch.from_numpy(host).cuda()
    pools = [pool0] + [pool0.clone() for _ in range(args.copies - 1)]
    del host
    nbatch = args.copies
    xs = [torch.from_numpy(W.x_of(wl, seed=100 + i)).cuda() for i in range(nbatch)]
    ls = [torch.from_numpy(W.logits_of(wl, seed=100 + i)).cuda() for i in range(nbatch)]
    soe = torch.arange(wl.E, dtype=torch.int32, device="cuda")
    spec = LayerSpec(wl.fmt, wl.H, wl.I, wl.E, wl.k, wl.score, wl.renormalize, wl.scale)
    layer = MoELayer(spec, wl.T, wl.E, pool0, stride, soe, path=Q.MOE_PATH_DECODE)
    torch.cuda.synchronize()
    setup_s = time.time() - t0

    # unique experts per input batch (algorithmic bytes of each step)
    uniq = []
    for i in range(nbatch):
        layer.forward(xs[i], ls[i], slot_pool=pools[i])
        uniq.append(int(torch.unique(layer.ids).numel()))
    torch.cuda.synchronize()
    gateup_bytes_per_expert = 2 * wl.I * wl.H // 256 * 144
    down_bytes_per_expert = wl.H * wl.I // 256 * 144

    def step(i):
        layer.forward(xs[i % nbatch], ls[i % nbatch], slot_pool=pools[i % args.copies])

    # ---- warmup (eager)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # ---- eager pass with the stage timers (HIP events attached to the stages' own
    # dispatches on the launch stream: kernel begin to kernel end)
    stages = {"route_batches": 8, "ffn_gateup": 3, "ffn_down": 4, "combine": 5}
    for s in stages.values():
        Q.moe_timer_begin(s, args.steps)
    torch.cuda.synchronize()
    te0 = time.time()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    eager_s = time.time() - te0
    kern = {}
    for name, s in stages.items():
        ms, n = Q.moe_timer_end(s)
        kern[name] = dict(avg_us=1e3 * ms / max(n, 1), launches=n)
    gu_bytes = sum(uniq[i % nbatch] * gateup_bytes_per_expert for i in range(args.steps))
    dn_bytes = sum(uniq[i % nbatch] * down_bytes_per_expert for i in range(args.steps))
    gu_time_s = kern["ffn_gateup"]["avg_us"] * 1e-6 * args.steps
    dn_time_s = kern["ffn_down"]["avg_us"] * 1e-6 * args.steps
    gu_gbs = gu_bytes / gu_time_s / 1e9
    dn_gbs = dn_bytes / dn_time_s / 1e9

    # ---- timed region: K steps as hipGraph replays (one captured graph per step slot)
    graphs = []
    for i in range(nbatch):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(i)
        graphs.append(g)
    for i in range(min(args.warmup, 64)):
        graphs[i % nbatch].replay()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.time()
    start.record()
    for i in range(args.steps):
        graphs[i % nbatch].replay()
    stop.record()
    torch.cuda.synchronize()
    wall_s = time.time() - wall0
    ms = start.elapsed_time(stop)
    ms_per_step = ms / args.steps
    tokens_per_s = wl.T * args.steps / (ms / 1e3)
    layer_bytes = (gu_bytes + dn_bytes) / args.steps
    layer_gbs = layer_bytes / (ms_per_step * 1e-3) / 1e9

    # ---- CPU oracle on a bounded sample of the same workload
    cpu = None
    if not args.no_cpu:
        import oracle as O
        O.set_threads(threads)
        n_done, c0 = 0, time.time()
        while time.time() - c0 < args.cpu_seconds:
            i = n_done % nbatch
            lg = ls[i].cpu().numpy()
            x = xs[i].cpu().numpy().astype(np.float64)
            O.moe_layer(wl.fmt, blobs, wl.H, wl.I, x, lg, wl.k, wl.score, wl.renormalize, wl.scale)
            n_done += 1
        cpu_s = time.time() - c0
        cpu = {"value": round(wl.T * n_done / cpu_s, 3), "unit": "tokens/s", "cores": O.threads(), "kind": "oracle",
               "sample": f"{n_done} steps of the same layer (T={wl.T}, fp64 oracle), {cpu_s:.1f} s wall"}
        # the same oracle on one thread, for a third of the time
        O.set_threads(1)
        n1, c1 = 0, time.time()
        while time.time() - c1 < args.cpu_seconds / 3:
            i = n1 % nbatch
            O.moe_layer(wl.fmt, blobs, wl.H, wl.I, xs[i].cpu().numpy().astype(np.float64), ls[i].cpu().numpy(), wl.k,
                        wl.score, wl.renormalize, wl.scale)
            n1 += 1
        cpu["value_1_thread"] = round(wl.T * n1 / (time.time() - c1), 3)
        O.set_threads(threads)

    if args.profile_copy:
        a = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()

    prefill = None
    if args.prefill_steps > 0:
        prefill = bench_prefill(args, blobs, pool0, stride)
    del pools, pool0
    torch.cuda.empty_cache()
    dsv3 = bench_dsv3(args, threads) if args.dsv3_steps > 0 else None
    formats = bench_formats(args, threads) if args.dsv3_steps > 0 else None
    stack = bench_stack(args, threads) if args.stack_replays > 0 else None

    traffic = read_traffic()
    out = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "arithmetic": "q4_k weights dequantized to fp16, fp16 x fp16 dot products, fp32 accumulate",
        "data": "synthetic (seeded N(0,0.02) weights quantized to Q4_K, N(0,1) activations and gate logits)",
        "config": {"workload": wl.name, "T": wl.T, "H": wl.H, "E": wl.E, "top_k": wl.k, "I": wl.I,
                   "routing": "softmax, renormalised over top-k", "weights": "Q4_K", "resident": "all 128",
                   "pool_copies": args.copies, "timed": "hipGraph replay, one graph per step"},
        "roofline": {"bound": "hbm", "kernel": "ffn_gateup (Q4_K gate/up GEMV + SwiGLU)",
                     "achieved": round(gu_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gu_gbs / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else traffic["bytes_per_launch"],
                     "algorithmic_bytes_per_launch": round(gu_bytes / args.steps),
                     "avg_launch_us": round(kern["ffn_gateup"]["avg_us"], 3)},
        "cpu_baseline": cpu,
        "prefill": prefill,
        "dsv3_decode": dsv3,
        "formats_decode": formats,
        "stack": stack,
        "kernels_us": {k2: round(v["avg_us"], 3) for k2, v in kern.items()},
        "down_gemv_GBs": round(dn_gbs, 1),
        "layer_effective_GBs": round(layer_gbs, 1),
        "unique_experts_per_step": round(float(np.mean([uniq[i % nbatch] for i in range(args.steps)])), 3),
        "eager_ms_per_step": round(1e3 * eager_s / args.steps, 5),
        "wall_s_timed": round(wall_s, 3),
        "setup_s": round(setup_s, 1),
    }
    print(json.dumps(out), flush=True)


def bench_prefill(args, blobs, pool, stride, fmt=None, ceiling=True) -> dict:
    """The same Qwen3-30B-A3B-shaped layer at prefill: 4096 bf16 tokens with
    Zipf(1.0)-skewed routing, through the grouped bf16 MFMA GEMM path (Q4_K
    experts, or fmt's)."""
    import dataclasses
    import numpy as np
    import torch

    import fixtures as F
    import quantized_routed_expert_moe_amd as Q
    from fixtures import workloads as W
    from quantized_routed_expert_moe_amd.layer import LayerSpec, MoELayer

    wl = W.QWEN3_PREFILL if fmt is None else dataclasses.replace(W.QWEN3_PREFILL, fmt=fmt)
    x = torch.from_numpy(W.x_of(wl).view(np.int16)).cuda().view(torch.bfloat16)
    lg = torch.from_numpy(W.logits_of(wl)).cuda()
    soe = torch.arange(wl.E, dtype=torch.int32, device="cuda")
    spec = LayerSpec(wl.fmt, wl.H, wl.I, wl.E, wl.k, wl.score, wl.renormalize, wl.scale)
    layer = MoELayer(spec, wl.T, wl.E, pool, stride, soe, path=Q.MOE_PATH_PREFILL, y_dtype=torch.bfloat16,
                     pair_dtype=torch.bfloat16)
    for _ in range(3):
        layer.forward(x, lg)
    torch.cuda.synchronize()
    M = int(layer.slot_offsets[-1].item())  # resident pairs = GEMM rows over all experts
    counts = np.diff(layer.slot_offsets.cpu().numpy())
    stages = {"route": 0, "batches": 1, "tiles": 2, "gemm_gateup": 6, "gemm_down": 7, "combine": 5}
    for st in stages.values():
        Q.moe_timer_begin(st, args.prefill_steps)
    for _ in range(args.prefill_steps):
        layer.forward(x, lg)
    torch.cuda.synchronize()
    kern = {}
    for name, st in stages.items():
        ms, n = Q.moe_timer_end(st)
        kern[name] = 1e3 * ms / max(n, 1)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.forward(x, lg)
    g.replay()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.prefill_steps):
        g.replay()
    stop.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(stop) / args.prefill_steps
    gu_flop = 2.0 * M * (2 * wl.I) * wl.H
    dn_flop = 2.0 * M * wl.H * wl.I
    gu_tf = gu_flop / (kern["gemm_gateup"] * 1e-6) / 1e12
    dn_tf = dn_flop / (kern["gemm_down"] * 1e-6) / 1e12
    return {
        "workload": wl.name, "T": wl.T, "steps": args.prefill_steps, "ms_per_step": round(ms_step, 4),
        "tokens_per_s": round(wl.T / (ms_step * 1e-3), 1),
        "expert_rows": {"total": M, "max": int(counts.max()), "median": float(np.median(counts)),
                        "min": int(counts.min())},
        "roofline": {"bound": "mfma", "kernel": "prefill gate/up grouped GEMM (%s->bf16 fragments, bf16 MFMA)" %
                     ("Q4_K" if fmt is None else {F.MXFP4: "MXFP4", F.Q5K: "Q5_K", F.Q6K: "Q6_K", F.Q4K: "Q4_K",
                                              F.Q3K_Q4K: "Q3_K gate/up"}[fmt]),
                     "achieved": round(gu_tf, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(gu_tf / MFMA_BF16_PEAK_TFLOPS, 4),
                     "algorithmic_flop_per_launch": gu_flop, "avg_launch_us": round(kern["gemm_gateup"], 2)},
        "down_gemm_TFLOPs": round(dn_tf, 1),
        "expert_gemms_TFLOPs": round((gu_flop + dn_flop) / ((kern["gemm_gateup"] + kern["gemm_down"]) * 1e-6) / 1e12,
                                     1),
        "expert_gemms_frac": round((gu_flop + dn_flop) / ((kern["gemm_gateup"] + kern["gemm_down"]) * 1e-6) / 1e12 /
                                   MFMA_BF16_PEAK_TFLOPS, 4),
        "kernels_us": {k2: round(v, 2) for k2, v in kern.items()},
        "library_gemm_ceiling": library_gemm_ceiling(M, wl.H, wl.I) if ceiling else None,
    }


def library_gemm_ceiling(M: int, H: int, I: int, reps: int = 20) -> dict:
    """What the platform's tuned dense bf16 GEMM (torch.matmul, i.e.
    hipBLASLt) reaches on plain dense operands of the prefill's total shapes
    (all M rows in one GEMM, weights already bf16, no grouping or
    dequantization), and on a large square GEMM: the practical MFMA ceiling
    the grouped kernels are read against.  Run only; nothing of it is used."""
    import torch

    out = {}
    for name, (m, k, n) in {"gateup_shape": (M, H, 2 * I), "down_shape": (M, I, H),
                            "square_8192": (8192, 8192, 8192)}.items():
        a = torch.randn(m, k, device="cuda", dtype=torch.bfloat16)
        b = torch.randn(k, n, device="cuda", dtype=torch.bfloat16).contiguous()
        for _ in range(3):
            torch.matmul(a, b)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            torch.matmul(a, b)
        e1.record()
        torch.cuda.synchronize()
        us = 1e3 * e0.elapsed_time(e1) / reps
        out[name] = {"m_k_n": [m, k, n], "us": round(us, 2), "TFLOPs": round(2.0 * m * k * n / (us * 1e-6) / 1e12, 1)}
        del a, b
    torch.cuda.empty_cache()
    return out


def bench_dsv3(args, threads: int) -> dict:
    """The DeepSeek-V3-shaped decode layer (256 Q4_K routed experts, top-8
    sigmoid x2.5, one Q8_0 shared expert) at T = 2 and T = 4, graph-replayed
    like the headline layer; all 256 experts resident (6.3 GB pool, so a step's
    ~16 experts x 24.8 MB never sit in the 256 MB Infinity Cache)."""
    import numpy as np
    import torch

    import fixtures as F
    import quantized_routed_expert_moe_amd as Q
    from concurrent.futures import ThreadPoolExecutor
    from fixtures import workloads as W
    from quantized_routed_expert_moe_amd.layer import LayerSpec, MoELayer

    res = {}
    wl0 = W.DSV3_DECODE_T2
    blobs = W.expert_blobs(wl0)
    nb = Q.moe_expert_blob_bytes(wl0.fmt, wl0.H, wl0.I)
    stride = (nb + 255) // 256 * 256
    host = np.zeros((wl0.E, stride), dtype=np.uint8)
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(lambda e: Q.moe_pack_expert(wl0.fmt, blobs[e], wl0.H, wl0.I, out=host[e, :nb]), range(wl0.E)))
    pool = torch.from_numpy(host).cuda()
    del host, blobs
    sh = W.shared_blob(wl0)
    nbs = Q.moe_expert_blob_bytes(F.Q8_0, wl0.H, wl0.I_shared)
    sh_host = np.zeros((1, (nbs + 255) // 256 * 256), dtype=np.uint8)
    Q.moe_pack_expert(F.Q8_0, sh, wl0.H, wl0.I_shared, out=sh_host[0, :nbs])
    shared = torch.from_numpy(sh_host).cuda()
    soe = torch.arange(wl0.E, dtype=torch.int32, device="cuda")
    expert_bytes = 3 * wl0.H * wl0.I // 256 * 144
    gateup_bytes = 2 * wl0.H * wl0.I // 256 * 144
    shared_bytes = 3 * wl0.H * wl0.I_shared // 32 * 34
    for wl in (W.DSV3_DECODE_T2, W.DSV3_DECODE_T4):
        spec = LayerSpec(wl.fmt, wl.H, wl.I, wl.E, wl.k, wl.score, wl.renormalize, wl.scale, wl.I_shared)
        layer = MoELayer(spec, wl.T, wl.E, pool, stride, soe, shared, Q.MOE_PATH_DECODE)
        nbatch = 8
        xs = [torch.from_numpy(W.x_of(wl, seed=200 + i)).cuda() for i in range(nbatch)]
        ls = [torch.from_numpy(W.logits_of(wl, seed=200 + i)).cuda() for i in range(nbatch)]
        uniq = []
        for i in range(nbatch):
            layer.forward(xs[i], ls[i])
            uniq.append(int(torch.unique(layer.ids).numel()))
        torch.cuda.synchronize()
        steps = args.dsv3_steps
        Q.moe_timer_begin(3, steps)
        for i in range(steps):
            layer.forward(xs[i % nbatch], ls[i % nbatch])
        torch.cuda.synchronize()
        gu_ms, gu_n = Q.moe_timer_end(3)
        # gate/up launches alternate routed and shared; the routed ones are every other one
        graphs = []
        for i in range(nbatch):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                layer.forward(xs[i], ls[i])
            graphs.append(g)
        for i in range(16):
            graphs[i % nbatch].replay()
        torch.cuda.synchronize()
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for i in range(steps):
            graphs[i % nbatch].replay()
        stop.record()
        torch.cuda.synchronize()
        ms_step = start.elapsed_time(stop) / steps
        mean_uniq = float(np.mean([uniq[i % nbatch] for i in range(steps)]))
        layer_bytes = mean_uniq * expert_bytes + shared_bytes
        layer_gbs = layer_bytes / (ms_step * 1e-3) / 1e9
        res[f"T{wl.T}"] = {
            "workload": wl.name, "tokens_per_s": round(wl.T / (ms_step * 1e-3), 1), "ms_per_step": round(ms_step, 4),
            "unique_experts_per_step": round(mean_uniq, 2),
            "layer_bytes_per_step": round(layer_bytes), "layer_GBs": round(layer_gbs, 1),
            "layer_frac_of_hbm": round(layer_gbs / HBM_PEAK_GBS, 4),
            "gateup_launch_us_routed_and_shared_avg": round(1e3 * gu_ms / max(gu_n, 1), 2),
        }
        del graphs, layer
        torch.cuda.empty_cache()
    res["bytes"] = {"routed_q4k_expert": expert_bytes, "routed_gateup": gateup_bytes, "shared_q8_0": shared_bytes}
    res["note"] = ("layer_GBs = (unique routed experts x 24.77 MB + 46.79 MB shared) per step / graph-replayed step "
                   "time, i.e. the whole layer (five routed and two shared-expert kernels) against the HBM peak")
    del pool, shared
    torch.cuda.empty_cache()
    return res


def bench_formats(args, threads: int) -> dict:
    """The decode layers with the other card expert types: MXFP4 (17 bytes per
    32 weights) Qwen3-shaped at T = 2 (8 pool copies rotated, 2.6 GB, so a
    step's experts come from HBM), its gate/up GEMV against the HBM peak, and
    DeepSeek-V3-shaped at T = 2 with the Q8_0 shared expert (one 6 GB pool);
    the DeepSeek-V3-shaped layer with the mixed experts of the engine's V4.1
    files (Q3_K gate/up, Q4_K down).  Graph-replayed like the other decode
    layers."""
    import numpy as np
    import torch

    import fixtures as F
    import quantized_routed_expert_moe_amd as Q
    from concurrent.futures import ThreadPoolExecutor
    from fixtures import workloads as W
    from quantized_routed_expert_moe_amd.layer import LayerSpec, MoELayer

    res = {}
    def gateup_bytes(wl) -> int:  # stored bytes of one expert's gate and up matrices
        w = 2 * wl.H * wl.I
        return {F.MXFP4: w // 32 * 17, F.Q3K_Q4K: w // 256 * 110, F.Q4K: w // 256 * 144, F.Q5K: w // 256 * 176,
                F.Q6K: w // 256 * 210}[wl.fmt]

    for key, wl, copies in (("mxfp4_qwen3_T2", W.QWEN3_MXFP4_DECODE_T2, 8), ("mxfp4_dsv3_T2", W.DSV3_MXFP4_DECODE_T2, 1),
                            ("q3k_q4k_dsv3_T2", W.DSV3_Q3K_DECODE_T2, 1), ("q3k_q4k_qwen3_T2", W.QWEN3_Q3K_DECODE_T2, 8),
                            ("q5k_qwen3_T2", W.QWEN3_Q5K_DECODE_T2, 8),
                            ("q5k_dsv3_T2", W.DSV3_Q5K_DECODE_T2, 1), ("q6k_qwen3_T2", W.QWEN3_Q6K_DECODE_T2, 8),
                            ("q6k_dsv3_T2", W.DSV3_Q6K_DECODE_T2, 1)):
        blobs = W.expert_blobs(wl)
        nb = Q.moe_expert_blob_bytes(wl.fmt, wl.H, wl.I)
        npk = Q.moe_packed_blob_bytes(wl.fmt, wl.H, wl.I)
        stride = (npk + 255) // 256 * 256
        host = np.zeros((wl.E, stride), dtype=np.uint8)
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(lambda e: Q.moe_pack_expert(wl.fmt, blobs[e], wl.H, wl.I, out=host[e, :npk]), range(wl.E)))
        del blobs
        pools = [torch.from_numpy(host).cuda() for _ in range(copies)]
        del host
        shared, shared_bytes = None, 0
        if wl.I_shared:
            nbs = Q.moe_expert_blob_bytes(F.Q8_0, wl.H, wl.I_shared)
            sh_host = np.zeros((1, (nbs + 255) // 256 * 256), dtype=np.uint8)
            Q.moe_pack_expert(F.Q8_0, W.shared_blob(wl), wl.H, wl.I_shared, out=sh_host[0, :nbs])
            shared = torch.from_numpy(sh_host).cuda()
            shared_bytes = nbs
        soe = torch.arange(wl.E, dtype=torch.int32, device="cuda")
        spec = LayerSpec(wl.fmt, wl.H, wl.I, wl.E, wl.k, wl.score, wl.renormalize, wl.scale, wl.I_shared)
        layer = MoELayer(spec, wl.T, wl.E, pools[0], stride, soe, shared, Q.MOE_PATH_DECODE)
        nbatch = 16
        xs = [torch.from_numpy(W.x_of(wl, seed=300 + i)).cuda() for i in range(nbatch)]
        ls = [torch.from_numpy(W.logits_of(wl, seed=300 + i)).cuda() for i in range(nbatch)]
        uniq = []
        for i in range(nbatch):
            layer.forward(xs[i], ls[i], slot_pool=pools[i % copies])
            uniq.append(int(torch.unique(layer.ids).numel()))
        torch.cuda.synchronize()
        steps = args.dsv3_steps
        Q.moe_timer_begin(3, steps * (2 if wl.I_shared else 1))
        for i in range(steps):
            layer.forward(xs[i % nbatch], ls[i % nbatch], slot_pool=pools[i % nbatch % copies])
        torch.cuda.synchronize()
        gu_ms, gu_n = Q.moe_timer_end(3)
        graphs = []
        for i in range(nbatch):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                layer.forward(xs[i], ls[i], slot_pool=pools[i % copies])
            graphs.append(g)
        for i in range(2 * nbatch):
            graphs[i % nbatch].replay()
        torch.cuda.synchronize()
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for i in range(steps):
            graphs[i % nbatch].replay()
        stop.record()
        torch.cuda.synchronize()
        ms_step = start.elapsed_time(stop) / steps
        mean_uniq = float(np.mean([uniq[i % nbatch] for i in range(steps)]))
        layer_bytes = mean_uniq * nb + shared_bytes
        r = {"workload": wl.name, "tokens_per_s": round(wl.T / (ms_step * 1e-3), 1), "ms_per_step": round(ms_step, 4),
             "unique_experts_per_step": round(mean_uniq, 2), "expert_bytes": nb, "packed_bytes": npk,
             "layer_bytes_per_step": round(layer_bytes),
             "layer_GBs": round(layer_bytes / (ms_step * 1e-3) / 1e9, 1),
             "layer_frac_of_hbm": round(layer_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
             "pool_copies": copies}
        if key in ("mxfp4_qwen3_T2", "q3k_q4k_qwen3_T2", "q5k_qwen3_T2", "q6k_qwen3_T2") and args.prefill_steps > 0:
            pre = bench_prefill(args, None, pools[0], stride, fmt=wl.fmt, ceiling=False)
            r["prefill_T4096"] = {kk: pre[kk] for kk in ("ms_per_step", "tokens_per_s", "roofline", "down_gemm_TFLOPs",
                                                         "expert_gemms_frac", "kernels_us")}
        if not wl.I_shared:  # stage 3 then times only the routed gate/up GEMV
            gu_us = 1e3 * gu_ms / max(gu_n, 1)
            gbytes = mean_uniq * gateup_bytes(wl)
            r["gateup"] = {"avg_launch_us": round(gu_us, 3), "algorithmic_bytes_per_launch": round(gbytes),
                           "GBs": round(gbytes / (gu_us * 1e-6) / 1e9, 1),
                           "frac_of_hbm": round(gbytes / (gu_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        res[key] = r
        del graphs, layer, pools, shared
        torch.cuda.empty_cache()
    res["note"] = ("MXFP4 codes converted to fp16 by the hardware FP4 conversion, Q3_K, Q5_K and Q6_K quants by and-or "
                   "operations into fp16 magic numbers; fp16 x fp16 dot products, fp32 accumulate; expert_bytes and "
                   "layer bytes count the stored (canonical) bytes")
    return res


def bench_stack(args, threads: int) -> dict:
    """The 58-layer DeepSeek-V3-shaped stack under partial residency (96 of 256
    experts per layer + 8 staging slots, one hipGraph), decode T = 2: replay
    time and bytes, swap-round copy rate alone and while replays run, graph
    node count."""
    import numpy as np
    import torch

    import fixtures as F
    import quantized_routed_expert_moe_amd as Q
    from concurrent.futures import ThreadPoolExecutor
    from fixtures import workloads as W
    from quantized_routed_expert_moe_amd.layer import LayerSpec
    from quantized_routed_expert_moe_amd.stack import ResidentStack

    wl = W.DSV3_STACK
    n_blobs, n_shared = 256, 8
    t0 = time.time()
    blobs = W.expert_blobs(wl)  # blob b = expert b of layer 0; expert e of layer l uses blob (e + 37 l) mod 256
    nb = Q.moe_expert_blob_bytes(wl.fmt, wl.H, wl.I)
    stride = (nb + 255) // 256 * 256
    host_blobs = torch.zeros((n_blobs, stride), dtype=torch.uint8).pin_memory()
    hb = host_blobs.numpy()
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(lambda b: Q.moe_pack_expert(wl.fmt, blobs[b], wl.H, wl.I, out=hb[b, :nb]), range(n_blobs)))
    # `blobs` (canonical) stays: the host leg reads the experts the card does not hold from them
    dev_blobs = host_blobs.cuda()
    nbs = Q.moe_expert_blob_bytes(F.Q8_0, wl.H, wl.I_shared)
    sh_host = torch.zeros((n_shared, (nbs + 255) // 256 * 256), dtype=torch.uint8).pin_memory()
    for i in range(n_shared):
        sh = F.expert_blob(F.Q8_0, wl.seed, 100 + i, F.TAG_SHARED_EXPERT, wl.H, wl.I_shared)
        Q.moe_pack_expert(F.Q8_0, sh, wl.H, wl.I_shared, out=sh_host.numpy()[i, :nbs])
    ranked = [W.frequency_resident_set(wl, l) for l in range(wl.layers)]
    spec = LayerSpec(wl.fmt, wl.H, wl.I, wl.E, wl.k, wl.score, wl.renormalize, wl.scale, wl.I_shared)
    st = ResidentStack(spec, wl.layers, wl.T, wl.resident, wl.staging, ranked,
                       lambda l, e: (e + 37 * l) % n_blobs, host_blobs, dev_blobs, lambda l: l % n_shared, sh_host)
    if args.residency_steps <= 0:
        del dev_blobs
        torch.cuda.empty_cache()
    xs = [W.x_of(wl, l) for l in range(wl.layers)]
    st.set_inputs([torch.from_numpy(a) for a in xs], [torch.from_numpy(W.logits_of(wl, l)) for l in range(wl.layers)])
    setup_s = time.time() - t0
    st.capture()
    nodes = st.graph_node_count()
    for _ in range(3):
        st.replay()
    torch.cuda.synchronize()

    def replay_bytes() -> tuple[float, float]:
        expert_bytes = 3 * wl.H * wl.I // 256 * 144
        shared_bytes = 3 * wl.H * wl.I_shared // 32 * 34
        total, served = 0.0, 0.0
        for l, lay in enumerate(st.layers):
            ids = lay.ids.cpu().numpy().ravel()
            soe = st.maps[l]
            resident = {int(e) for e in ids if soe[e] >= 0}
            total += len(resident) * expert_bytes + shared_bytes
            served += float(np.mean(soe[ids] >= 0))
        return total, served / wl.layers

    # replays alone
    R = args.stack_replays
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(R):
        st.replay()
    stop.record()
    torch.cuda.synchronize()
    replay_ms = start.elapsed_time(stop) / R
    nbytes, share = replay_bytes()
    swap_bytes = 8 * wl.layers * (3 * wl.H * wl.I // 256 * 144)

    # one swap round with nothing else on the GPU
    st.swap_begin(8)
    st.swap_copies_done.synchronize()
    swap_alone_ms = st.swap_start.elapsed_time(st.swap_copies_done)
    st.swap_commit(block=True)
    st.replay()
    torch.cuda.synchronize()

    # one swap round while replays run back to back on the compute stream
    st.swap_begin(8)
    w0 = time.time()
    n_during = 0
    while not st.swap_copies_done.query() and n_during < 1000:
        st.replay()
        st.replay_done.synchronize()
        n_during += 1
    during_s = time.time() - w0
    st.swap_copies_done.synchronize()
    swap_during_ms = st.swap_start.elapsed_time(st.swap_copies_done)
    st.swap_commit(block=True)
    st.replay()
    torch.cuda.synchronize()
    replay_ms_during = 1e3 * during_s / max(n_during, 1)

    # the host leg: one replay's pairs that the card does not hold, on the
    # host cores, from the canonical blobs in host memory
    st.replay()
    torch.cuda.synchronize()
    lists = [st.host_lists(l) for l in range(wl.layers)]
    expert_bytes = 3 * wl.H * wl.I // 256 * 144
    h0 = time.time()
    host_pairs = host_experts = 0
    for l, hl in enumerate(lists):
        if len(hl["token"]) == 0:
            continue
        experts = [None] * wl.E
        for e in set(hl["expert"].tolist()):
            experts[e] = blobs[(e + 37 * l) % n_blobs]
        host_experts += sum(b is not None for b in experts)
        host_pairs += len(hl["token"])
        Q.moe_host_leg(wl.fmt, experts, wl.H, wl.I, xs[l], hl["token"], hl["expert"], hl["weight"], threads=threads)
    host_ms = 1e3 * (time.time() - h0)
    host_leg = {"pairs_per_replay": host_pairs, "host_experts_per_replay": host_experts,
                "ms_per_replay": round(host_ms, 2), "threads": threads,
                "weight_GBs": round(host_experts * expert_bytes / (host_ms * 1e-3) / 1e9, 1),
                "stack_tokens_per_s_card_then_host": round(wl.T / ((replay_ms + host_ms) * 1e-3), 1),
                "note": "the host leg reads each listed expert's canonical Q4_K blocks once per replay (grouped by "
                        "expert); weight_GBs = those bytes over its wall time"}
    residency = None
    if args.residency_steps > 0:
        residency = bench_residency(st, wl, blobs, xs, dev_blobs, args.residency_steps, threads,
                                    lambda l, e: (e + 37 * l) % n_blobs)
        del dev_blobs
        torch.cuda.empty_cache()
    out = {
        "workload": wl.name, "layers": wl.layers, "resident": wl.resident, "staging": wl.staging,
        "graph_nodes": nodes, "replays": R, "replay_ms": round(replay_ms, 3),
        "layer_us": round(1e3 * replay_ms / wl.layers, 2),
        "tokens_per_s_per_layer": round(wl.T / (replay_ms * 1e-3 / wl.layers), 1),
        "stack_tokens_per_s": round(wl.T / (replay_ms * 1e-3), 1),
        "bytes_per_replay": round(nbytes), "replay_GBs": round(nbytes / (replay_ms * 1e-3) / 1e9, 1),
        "replay_frac_of_hbm": round(nbytes / (replay_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "card_served_share": round(share, 4),
        "swap_round_bytes": swap_bytes,
        "swap_alone_ms": round(swap_alone_ms, 1), "swap_alone_GBs": round(swap_bytes / (swap_alone_ms * 1e-3) / 1e9, 1),
        "swap_during_replays_ms": round(swap_during_ms, 1),
        "swap_during_replays_GBs": round(swap_bytes / (swap_during_ms * 1e-3) / 1e9, 1),
        "replays_during_swap": n_during, "replay_ms_during_swap": round(replay_ms_during, 3),
        "copy_stream": {"candidates_tried": st.side_probes, "overlaps_replays": st.side_overlaps},
        "pcie_gen5_x16_GBs": 64.0,
        "host_leg": host_leg,
        "adaptive_residency": residency,
        "setup_s": round(setup_s, 1),
    }
    del st
    torch.cuda.empty_cache()
    return out


def bench_residency(st, wl, blobs, xs, dev_blobs, steps: int, threads: int, blob_of) -> dict:
    """The adaptive residency policy on the stack, measured the way the pages
    measure it: decode steps from a start where each layer holds its lowest
    expert ids, with the policy off, with the swap rule, and with the swap
    rule after a prompt call has streamed its most-used experts onto the card.
    Each step: one graph replay (card), then the host leg for every pair the
    card does not hold (host cores), then the policy (counters -> scores ->
    an 8-swap plan per layer), whose copies run on a side stream beside the
    next steps and are committed between steps once they have landed."""
    import numpy as np
    import torch

    import fixtures as F
    import quantized_routed_expert_moe_amd as Q
    from quantized_routed_expert_moe_amd.stack import AdaptiveResidency

    L, E, T, k = wl.layers, wl.E, wl.T, wl.k
    lowest = [np.arange(E) for _ in range(L)]
    prompt_rows = 512
    margin, decay = 1 << Q.RESIDENCY_FRAC_BITS, 4
    step_logits = [np.stack([F.logits_zipf(wl.seed + 1000 + i, l, T, E, wl.zipf_s, perm_seed=wl.seed)
                             for l in range(L)]) for i in range(steps)]

    def host_leg() -> tuple[int, float]:
        pairs = 0
        h0 = time.time()
        for l in range(L):
            hl = st.host_lists(l)
            if len(hl["token"]) == 0:
                continue
            experts = [None] * E
            for e in set(hl["expert"].tolist()):
                experts[e] = blobs[blob_of(l, e)]
            pairs += len(hl["token"])
            Q.moe_host_leg(wl.fmt, experts, wl.H, wl.I, xs[l], hl["token"], hl["expert"], hl["weight"],
                           threads=threads)
        return pairs, time.time() - h0

    def arm(policy: bool, prompt: bool) -> dict:
        st.reset(lowest, dev_blobs)
        pol = AdaptiveResidency(st, decay_shift=decay, margin=margin) if policy else None
        res = {}
        if prompt:
            plg = [F.logits_zipf(wl.seed + 500, l, prompt_rows, E, wl.zipf_s, perm_seed=wl.seed) for l in range(L)]
            plans = pol.prompt_plans(st.prompt_counts(plg))
            n = sum(len(p[0]) for p in plans)
            secs = st.stream_in(plans)
            nb = n * Q.moe_expert_blob_bytes(wl.fmt, wl.H, wl.I)
            res.update(prompt_rows=prompt_rows, streamed_experts=n, stream_s=round(secs, 3),
                       stream_GBs=round(nb / max(secs, 1e-9) / 1e9, 1))
        share, card_s, host_s = [], 0.0, 0.0
        swaps = rounds = 0
        for i in range(steps):
            if st.swap_in_flight:
                st.swap_commit(block=False)
            st.set_logits(step_logits[i])
            c0 = time.time()
            st.replay()
            st.replay_done.synchronize()
            card_s += time.time() - c0
            pairs, hs = host_leg()
            host_s += hs
            share.append(1.0 - pairs / (L * T * k))
            if pol is not None:
                pol.observe()
                if not st.swap_in_flight:
                    plans = pol.plans(wl.staging)
                    n = sum(len(p[0]) for p in plans)
                    if n:
                        st.swap_begin(plans=plans)
                        swaps += n
                        rounds += 1
        if st.swap_in_flight:
            st.swap_commit(block=True)
        torch.cuda.synchronize()
        q = max(1, min(16, steps // 4))
        res.update(card_served_first=round(float(np.mean(share[:q])), 4),
                   card_served_last=round(float(np.mean(share[-q:])), 4),
                   card_served_all=round(float(np.mean(share)), 4),
                   replay_ms=round(1e3 * card_s / steps, 3), host_leg_ms=round(1e3 * host_s / steps, 2),
                   tokens_per_s=round(T * steps / (card_s + host_s), 2), swap_rounds=rounds, experts_swapped=swaps)
        return res

    out = {"steps": steps, "window": f"first/last {max(1, min(16, steps // 4))} steps",
           "start": "each layer's lowest 96 expert ids on the card",
           "policy": {"decay_shift": decay, "margin": margin, "swaps_per_layer_per_round": wl.staging,
                      "prompt_plan": "prompt counts, as many swaps as raise the card's count, margin 0"},
           "routing": "the stack workload's Zipf(1.1) ranking per layer; fresh Gumbel noise every step",
           "off": arm(False, False), "swap_rule": arm(True, False), "swap_rule_and_prompt_streaming": arm(True, True)}
    out["note"] = ("tokens_per_s = T x steps / (card replay + host leg), run one after the other; swap copies "
                   "overlap both")
    return out


if __name__ == "__main__":
    main()
