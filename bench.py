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
selected experts' gate and up weights, over its HIP-event-timed duration in
an eager pass of the same K steps), and the CPU oracle timed on a bounded
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

    # ---- eager pass with HIP-event stage timers (kernel durations on the launch stream)
    stages = {"route": 0, "batches": 1, "ffn_gateup": 3, "ffn_down": 4, "combine": 5}
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

    if args.profile_copy:
        a = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()

    prefill = None
    if args.prefill_steps > 0:
        prefill = bench_prefill(args, blobs, pool0, stride)

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
        "dtype": "q4_k weights dequantized to fp16, fp16 x fp16 dot products, fp32 accumulate",
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
        "kernels_us": {k2: round(v["avg_us"], 3) for k2, v in kern.items()},
        "down_gemv_GBs": round(dn_gbs, 1),
        "layer_effective_GBs": round(layer_gbs, 1),
        "unique_experts_per_step": round(float(np.mean([uniq[i % nbatch] for i in range(args.steps)])), 3),
        "eager_ms_per_step": round(1e3 * eager_s / args.steps, 5),
        "wall_s_timed": round(wall_s, 3),
        "setup_s": round(setup_s, 1),
    }
    print(json.dumps(out), flush=True)


def bench_prefill(args, blobs, pool, stride) -> dict:
    """The same Qwen3-30B-A3B-shaped layer at prefill: 4096 bf16 tokens with
    Zipf(1.0)-skewed routing, through the grouped bf16 MFMA GEMM path."""
    import numpy as np
    import torch

    import quantized_routed_expert_moe_amd as Q
    from fixtures import workloads as W
    from quantized_routed_expert_moe_amd.layer import LayerSpec, MoELayer

    wl = W.QWEN3_PREFILL
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
        "roofline": {"bound": "mfma", "kernel": "prefill gate/up grouped GEMM (Q4_K->bf16 tiles, bf16 MFMA)",
                     "achieved": round(gu_tf, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(gu_tf / MFMA_BF16_PEAK_TFLOPS, 4),
                     "algorithmic_flop_per_launch": gu_flop, "avg_launch_us": round(kern["gemm_gateup"], 2)},
        "down_gemm_TFLOPs": round(dn_tf, 1),
        "expert_gemms_TFLOPs": round((gu_flop + dn_flop) / ((kern["gemm_gateup"] + kern["gemm_down"]) * 1e-6) / 1e12,
                                     1),
        "kernels_us": {k2: round(v, 2) for k2, v in kern.items()},
    }


if __name__ == "__main__":
    main()
