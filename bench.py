"""Benchmark of the routed-expert MoE layer on one MI355X.

Headline: the 58-layer DeepSeek-V3-shaped stack under partial residency
(hidden 7168, 256 routed Q4_K experts of intermediate 2048 with 96 of them
resident per layer plus 8 staging slots, top-8 sigmoid x2.5, one Q8_0
shared expert of intermediate 2048), decode T = 2, all 58 layers replayed
as one hipGraph.  A step is one replay: every layer's routing, batching,
routed and shared expert FFN and combine.  `value` = T x 58 / replay time
(MoE-layer tokens per second).

Beside it, in the same JSON line, flat sub-objects:
  c4_decode_T2 / c4_decode_T4  the DeepSeek-V3-shaped layer, all 256 experts
                               resident, with its shared expert;
  c3_prefill                   the Qwen3-30B-A3B-shaped layer at T = 4096
                               (Zipf(1.0) loads) through the MFMA path;
  c2_decode_T2                 the Qwen3-30B-A3B-shaped layer at T = 2.
Each carries the roofline of its dominant kernel: algorithmic bytes (or
flops) per launch over that kernel's average duration, measured with HIP
events attached to the kernel's own dispatches (the library's stage timers)
during an eager pass of the same steps.

Inputs are seeded and synthetic and resident in HBM before timing starts.
The Infinity Cache (256 MB) cannot serve weights: the stack streams 58
distinct layers (about 19 GB) per replay, the C4 layer rotates 8 input
batches over a 6.3 GB pool and 8 copies of its shared expert, C2 rotates 16
copies of its 340 MB pool.

cpu_baseline: the fp64 oracle on layers of the stack (the card part each
computes: resident pairs plus the shared expert), on the host threads the
run may use, for a bounded wall time.
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
MFMA_INT8_PEAK_TOPS = 5000.0
METRIC = "MoE-layer tokens/s + achieved HBM GB/s (decode) / MFMA util (prefill), 1 GPU"
DSV3_GATEUP_BYTES = 2 * 7168 * 2048 // 256 * 144    # one routed Q4_K expert's gate and up matrices
DSV3_DOWN_BYTES = 7168 * 2048 // 256 * 144
DSV3_SHARED_BYTES = 3 * 7168 * 2048 // 32 * 34       # the Q8_0 shared expert
DSV3_SHARED_GATEUP_BYTES = 2 * 7168 * 2048 // 32 * 34
DSV3_SHARED_DOWN_BYTES = 7168 * 2048 // 32 * 34
# rocprofv3 --pmc summaries of the decode gate/up kernel (HBM bytes per launch),
# valid only while the kernel's sources hash to the value recorded in them
TRAFFIC = {
    "stack": os.path.join(ROOT, "profiles", "traffic_ffn_gateup_q4k_dsv3_stack_decode.txt"),
    "qwen3": os.path.join(ROOT, "profiles", "traffic_ffn_gateup_q4k_qwen3_decode.txt"),
}
KERNEL_SOURCES = [os.path.join(ROOT, "quantized_routed_expert_moe_amd", "csrc", f)
                  for f in ("ffn_decode.hip", "gemv_core.h", "device_common.h", "qmoe_internal.h")]
LEGS = ("stack", "dsv3", "prefill", "qwen3", "hbm", "mfma")
STAGE_GATEUP, STAGE_DOWN, STAGE_COMBINE, STAGE_ROUTE_BATCHES = 3, 4, 5, 8
STAGE_ROUTE, STAGE_BATCHES, STAGE_TILES, STAGE_PF_GATEUP, STAGE_PF_DOWN = 0, 1, 2, 6, 7


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100, help="timed replays of the 58-layer stack")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--legs", default=",".join(LEGS), help="comma-separated subset of " + ",".join(LEGS))
    ap.add_argument("--dsv3-steps", type=int, default=200, help="timed steps of each C4 layer")
    ap.add_argument("--prefill-steps", type=int, default=30, help="timed steps of the C3 prefill layer")
    ap.add_argument("--qwen3-steps", type=int, default=1000, help="timed steps of the C2 decode layer")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="bounded CPU-oracle sample (wall seconds)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--extra", action="store_true",
                    help="also the other card expert types, the host leg, swaps and adaptive residency (printed "
                         "as a second JSON line on stderr)")
    ap.add_argument("--profile-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration under rocprofv3)")
    return ap.parse_args()


def source_hash(paths: list) -> str:
    h = hashlib.sha256()
    for p in paths:
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def read_traffic(key: str) -> float | None:
    """HBM bytes per launch of a leg's gate/up kernel from a committed
    rocprofv3 --pmc summary, if it was taken on the current kernel source."""
    path = TRAFFIC[key]
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != source_hash(KERNEL_SOURCES):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def host_threads() -> dict:
    """Threads the CPU legs use: the run's CPU share (OMP_NUM_THREADS when
    set, as on a machine that caps a job's threads), else the affinity
    mask's size."""
    aff = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS", "")
    n = min(aff, int(env)) if env.isdigit() and int(env) > 0 else aff
    return {"threads": n, "affinity_cpus": aff, "os_cpu_count": os.cpu_count(), "omp_num_threads_env": env or None}


def timed_replays(fn, steps: int) -> float:
    """Milliseconds per call of fn over `steps` calls, between synchronisations."""
    import torch
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(steps):
        fn(i)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def pack_pool(fmt, blobs, H, I, threads, n=None):
    import numpy as np
    import quantized_routed_expert_moe_amd as Q
    from concurrent.futures import ThreadPoolExecutor
    n = blobs.shape[0] if n is None else n
    nb = Q.moe_packed_blob_bytes(fmt, H, I)
    stride = (nb + 255) // 256 * 256
    host = np.zeros((n, stride), dtype=np.uint8)
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(lambda e: Q.moe_pack_expert(fmt, blobs[e], H, I, out=host[e, :nb]), range(n)))
    return host, stride


# ---------------------------------------------------------------- C5: stack

def leg_stack(args, thr: dict, extra: dict | None) -> dict:
    import numpy as np
    import torch

    import fixtures as F
    import quantized_routed_expert_moe_amd as Q
    from fixtures import workloads as W
    from quantized_routed_expert_moe_amd.layer import LayerSpec
    from quantized_routed_expert_moe_amd.stack import ResidentStack

    threads = thr["threads"]
    wl = W.DSV3_STACK
    L = wl.layers
    n_blobs, n_shared = 256, 8
    blob_of = lambda l, e: (e + 37 * l) % n_blobs  # noqa: E731
    t0 = time.time()
    blobs = W.expert_blobs(wl)  # blob b = expert b of layer 0; expert e of layer l uses blob (e + 37 l) mod 256
    hb, stride = pack_pool(wl.fmt, blobs, wl.H, wl.I, threads)
    host_blobs = torch.zeros((n_blobs, stride), dtype=torch.uint8).pin_memory()
    host_blobs.numpy()[:] = hb
    del hb
    dev_blobs = host_blobs.cuda()
    nbs = Q.moe_expert_blob_bytes(F.Q8_0, wl.H, wl.I_shared)
    sh_canon = [F.expert_blob(F.Q8_0, wl.seed, 100 + i, F.TAG_SHARED_EXPERT, wl.H, wl.I_shared) for i in range(n_shared)]
    sh_host = torch.zeros((n_shared, (nbs + 255) // 256 * 256), dtype=torch.uint8).pin_memory()
    for i in range(n_shared):
        Q.moe_pack_expert(F.Q8_0, sh_canon[i], wl.H, wl.I_shared, out=sh_host.numpy()[i, :nbs])
    ranked = [W.frequency_resident_set(wl, l) for l in range(L)]
    spec = LayerSpec(wl.fmt, wl.H, wl.I, wl.E, wl.k, wl.score, wl.renormalize, wl.scale, wl.I_shared)
    st = ResidentStack(spec, L, wl.T, wl.resident, wl.staging, ranked, blob_of, host_blobs, dev_blobs,
                       lambda l: l % n_shared, sh_host)
    if extra is None:
        del dev_blobs
        dev_blobs = None
        torch.cuda.empty_cache()
    xs = [W.x_of(wl, l) for l in range(L)]
    lgs = [W.logits_of(wl, l) for l in range(L)]
    st.set_inputs([torch.from_numpy(a) for a in xs], [torch.from_numpy(a) for a in lgs])
    setup_s = time.time() - t0
    st.capture()
    nodes = st.graph_node_count()

    # bytes each layer streams: its resident selected experts and its shared expert
    st.replay()
    torch.cuda.synchronize()
    uniq = []
    served = []
    for l, lay in enumerate(st.layers):
        ids = lay.ids.cpu().numpy().ravel()
        soe = st.maps[l]
        uniq.append(len({int(e) for e in ids if 0 <= soe[e] < st.S}))
        served.append(float(np.mean((soe[ids] >= 0) & (soe[ids] < st.S))))
    bytes_per_replay = sum(u * (DSV3_GATEUP_BYTES + DSV3_DOWN_BYTES) + DSV3_SHARED_BYTES for u in uniq)

    # ---- warmup, then the timed region: K replays
    for _ in range(args.warmup):
        st.replay()
    replay_ms = timed_replays(lambda i: st.replay(), args.steps)

    # ---- eager pass with the stage timers: per-launch kernel times.  Each
    # layer is four launches: L0 routing + batching beside the shared gate/up
    # (stage 8), L1 routed gate/up + SwiGLU beside the shared down (stage 3),
    # L2 routed down (stage 4), L3 combine (stage 5).
    ne = max(1, min(args.steps, 20))
    st.run_eager()
    torch.cuda.synchronize()
    stages = (STAGE_GATEUP, STAGE_DOWN, STAGE_ROUTE_BATCHES, STAGE_COMBINE)
    for s in stages:
        Q.moe_timer_begin(s, L * ne)
    for _ in range(ne):
        st.run_eager()
    torch.cuda.synchronize()
    each = {s: Q.moe_timer_read(s, L * ne) for s in stages}
    for s in stages:
        Q.moe_timer_end(s)
    assert all(len(each[s]) == L * ne for s in stages), {s: len(each[s]) for s in stages}
    # algorithmic bytes per launch, averaged over the layers
    gu_bytes = sum(uniq) * DSV3_GATEUP_BYTES / L + DSV3_SHARED_DOWN_BYTES
    gu_us = 1e3 * float(np.mean(each[STAGE_GATEUP]))
    dn_bytes = sum(uniq) * DSV3_DOWN_BYTES / L
    dn_us = 1e3 * float(np.mean(each[STAGE_DOWN]))
    l0_us = 1e3 * float(np.mean(each[STAGE_ROUTE_BATCHES]))
    traffic = read_traffic("stack")

    # ---- the oracle on the same layers (card part: resident pairs + shared expert)
    cpu = None
    if not args.no_cpu:
        import oracle as O
        O.set_threads(threads)
        n, c0 = 0, time.time()
        while time.time() - c0 < args.cpu_seconds:
            l = n % L
            ids_needed = set(np.argsort(-lgs[l], axis=1, kind="stable")[:, :wl.k].ravel().tolist())
            experts = [blobs[blob_of(l, e)] if e in ids_needed else None for e in range(wl.E)]
            O.moe_layer(wl.fmt, experts, wl.H, wl.I, xs[l].astype(np.float64), lgs[l], wl.k, wl.score,
                        wl.renormalize, wl.scale, slot_of_expert=st.maps[l], shared_blob=sh_canon[l % n_shared],
                        shared_fmt=F.Q8_0, I_shared=wl.I_shared, S=st.S)
            n += 1
        cpu_s = time.time() - c0
        cpu = {"value": round(wl.T * n / cpu_s, 3), "unit": "tokens/s", "cores": O.threads(), "kind": "oracle",
               "sample": f"{n} layers of the stack (layer l = step mod 58, T={wl.T}, its resident pairs and shared "
                         f"expert), fp64 oracle, {cpu_s:.1f} s wall",
               "affinity_cpus": thr["affinity_cpus"], "os_cpu_count": thr["os_cpu_count"],
               "omp_num_threads_env": thr["omp_num_threads_env"]}

    out = {
        "value": wl.T * L / (replay_ms * 1e-3),
        "ms_per_step": replay_ms,
        "roofline": {"bound": "hbm", "kernel": "layer_l1_ht_kernel: routed Q4_K gate/up GEMV + SwiGLU over half tiles "
                               "with the shared expert's Q8_0 down GEMV in the same launch, in the stack",
                     "achieved": round(gu_bytes / (gu_us * 1e-6) / 1e9, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gu_bytes / (gu_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": round(gu_bytes), "avg_launch_us": round(gu_us, 3),
                     "launches_timed": int(len(each[STAGE_GATEUP]))},
        "cpu_baseline": cpu,
        "stack": {"layers": L, "resident": wl.resident, "staging": wl.staging, "graph_nodes": nodes,
                  "replay_ms": round(replay_ms, 4), "layer_us": round(1e3 * replay_ms / L, 2),
                  "stack_tokens_per_s": round(wl.T / (replay_ms * 1e-3), 2),
                  "bytes_per_replay": int(bytes_per_replay),
                  "replay_GBs": round(bytes_per_replay / (replay_ms * 1e-3) / 1e9, 1),
                  "replay_frac_of_hbm": round(bytes_per_replay / (replay_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                  "unique_resident_experts_per_layer": round(float(np.mean(uniq)), 3),
                  "card_served_share": round(float(np.mean(served)), 4),
                  "l0_route_and_shared_gateup_us": round(l0_us, 2),
                  "l0_GBs": round(DSV3_SHARED_GATEUP_BYTES / (l0_us * 1e-6) / 1e9, 1),
                  "l1_gateup_and_shared_down_us": round(gu_us, 2),
                  "l1_GBs": round(gu_bytes / (gu_us * 1e-6) / 1e9, 1),
                  "l2_down_us": round(dn_us, 2), "l2_GBs": round(dn_bytes / (dn_us * 1e-6) / 1e9, 1),
                  "l3_combine_us": round(1e3 * float(np.mean(each[STAGE_COMBINE])), 2),
                  "eager_steps_timed": ne, "setup_s": round(setup_s, 1)},
    }
    if extra is not None:
        extra["stack_swaps_and_host_leg"] = stack_swaps_and_host_leg(st, wl, blobs, xs, threads, blob_of)
        extra["adaptive_residency"] = bench_residency(st, wl, blobs, xs, dev_blobs, 96, threads, blob_of)
    del st, dev_blobs
    torch.cuda.empty_cache()
    return out


def stack_swaps_and_host_leg(st, wl, blobs, xs, threads, blob_of) -> dict:
    """One 8-expert-per-layer swap round alone and while replays run; one
    replay's host lists through the host leg."""
    import torch
    import quantized_routed_expert_moe_amd as Q
    swap_bytes = 8 * wl.layers * (DSV3_GATEUP_BYTES + DSV3_DOWN_BYTES)
    st.swap_begin(8)
    st.swap_copies_done.synchronize()
    swap_alone_ms = st.swap_start.elapsed_time(st.swap_copies_done)
    st.swap_commit(block=True)
    st.replay()
    torch.cuda.synchronize()
    st.swap_begin(8)
    w0, n_during = time.time(), 0
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
    lists = [st.host_lists(l) for l in range(wl.layers)]
    h0 = time.time()
    pairs = experts_n = 0
    for l, hl in enumerate(lists):
        if len(hl["token"]) == 0:
            continue
        experts = [None] * wl.E
        for e in set(hl["expert"].tolist()):
            experts[e] = blobs[blob_of(l, e)]
        experts_n += sum(b is not None for b in experts)
        pairs += len(hl["token"])
        Q.moe_host_leg(wl.fmt, experts, wl.H, wl.I, xs[l], hl["token"], hl["expert"], hl["weight"], threads=threads)
    host_ms = 1e3 * (time.time() - h0)
    return {"swap_round_bytes": swap_bytes, "swap_alone_ms": round(swap_alone_ms, 1),
            "swap_alone_GBs": round(swap_bytes / (swap_alone_ms * 1e-3) / 1e9, 1),
            "swap_during_replays_GBs": round(swap_bytes / (swap_during_ms * 1e-3) / 1e9, 1),
            "replays_during_swap": n_during, "replay_ms_during_swap": round(1e3 * during_s / max(n_during, 1), 3),
            "copy_stream": {"candidates_tried": st.side_probes, "overlaps_replays": st.side_overlaps},
            "host_leg": {"pairs_per_replay": pairs, "host_experts_per_replay": experts_n,
                         "ms_per_replay": round(host_ms, 2), "threads": threads,
                         "weight_GBs": round(experts_n * (DSV3_GATEUP_BYTES + DSV3_DOWN_BYTES) / (host_ms * 1e-3) / 1e9,
                                             1)}}


# ------------------------------------------------------------ C4: one layer

def leg_dsv3(args, thr: dict) -> dict:
    """The DeepSeek-V3-shaped decode layer (256 Q4_K routed experts, all
    resident, top-8 sigmoid x2.5, one Q8_0 shared expert) at T = 2 and T = 4,
    graph-replayed; 8 input batches and 8 copies of the shared expert rotate,
    so no weight byte is re-read within 7 other steps' 3 GB."""
    import numpy as np
    import torch

    import fixtures as F
    import quantized_routed_expert_moe_amd as Q
    from fixtures import workloads as W
    from quantized_routed_expert_moe_amd.layer import LayerSpec, MoELayer

    threads = thr["threads"]
    wl0 = W.DSV3_DECODE_T2
    host, stride = pack_pool(wl0.fmt, W.expert_blobs(wl0), wl0.H, wl0.I, threads)
    pool = torch.from_numpy(host).cuda()
    del host
    nbs = Q.moe_expert_blob_bytes(F.Q8_0, wl0.H, wl0.I_shared)
    sh = np.zeros((1, (nbs + 255) // 256 * 256), dtype=np.uint8)
    Q.moe_pack_expert(F.Q8_0, W.shared_blob(wl0), wl0.H, wl0.I_shared, out=sh[0, :nbs])
    nb = 8
    shared = [torch.from_numpy(sh).cuda() for _ in range(nb)]
    soe = torch.arange(wl0.E, dtype=torch.int32, device="cuda")
    res = {}
    for wl in (W.DSV3_DECODE_T2, W.DSV3_DECODE_T4):
        spec = LayerSpec(wl.fmt, wl.H, wl.I, wl.E, wl.k, wl.score, wl.renormalize, wl.scale, wl.I_shared)
        layer = MoELayer(spec, wl.T, wl.E, pool, stride, soe, shared[0], Q.MOE_PATH_DECODE)
        xs = [torch.from_numpy(W.x_of(wl, seed=200 + i)).cuda() for i in range(nb)]
        ls = [torch.from_numpy(W.logits_of(wl, seed=200 + i)).cuda() for i in range(nb)]
        uniq = []
        for i in range(nb):
            layer.forward(xs[i], ls[i], shared_pool=shared[i])
            uniq.append(int(torch.unique(layer.ids).numel()))
        torch.cuda.synchronize()
        steps = args.dsv3_steps
        step = lambda i: layer.forward(xs[i % nb], ls[i % nb], shared_pool=shared[i % nb])  # noqa: E731
        stages = (STAGE_ROUTE_BATCHES, STAGE_GATEUP, STAGE_DOWN, STAGE_COMBINE)
        for s in stages:
            Q.moe_timer_begin(s, steps)
        for i in range(steps):
            step(i)
        torch.cuda.synchronize()
        t_us = {s: 1e3 * float(np.mean(Q.moe_timer_read(s, steps))) for s in stages}
        for s in stages:
            Q.moe_timer_end(s)
        graphs = []
        for i in range(nb):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(i)
            graphs.append(g)
        for i in range(2 * nb):
            graphs[i % nb].replay()
        ms = timed_replays(lambda i: graphs[i % nb].replay(), steps)
        mean_uniq = float(np.mean([uniq[i % nb] for i in range(steps)]))
        layer_bytes = mean_uniq * (DSV3_GATEUP_BYTES + DSV3_DOWN_BYTES) + DSV3_SHARED_BYTES
        gu_us = t_us[STAGE_GATEUP]
        gu_bytes = mean_uniq * DSV3_GATEUP_BYTES + DSV3_SHARED_DOWN_BYTES
        dn_us = t_us[STAGE_DOWN]
        res[f"T{wl.T}"] = {
            "workload": wl.name, "tokens_per_s": round(wl.T / (ms * 1e-3), 1), "ms_per_step": round(ms, 5),
            "unique_experts_per_step": round(mean_uniq, 2), "layer_bytes_per_step": round(layer_bytes),
            "layer_GBs": round(layer_bytes / (ms * 1e-3) / 1e9, 1),
            "layer_frac_of_hbm": round(layer_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "roofline_kernel": "layer_l1_ht_kernel: routed Q4_K gate/up GEMV + SwiGLU over half tiles with the "
                               "shared Q8_0 down GEMV",
            "roofline_bound": "hbm",
            "roofline_achieved_GBs": round(gu_bytes / (gu_us * 1e-6) / 1e9, 1), "roofline_peak_GBs": HBM_PEAK_GBS,
            "roofline_frac": round(gu_bytes / (gu_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "roofline_algorithmic_bytes_per_launch": round(gu_bytes), "roofline_avg_launch_us": round(gu_us, 3),
            "l0_route_and_shared_gateup_us": round(t_us[STAGE_ROUTE_BATCHES], 3),
            "l2_down_us": round(dn_us, 3),
            "l2_down_GBs": round(mean_uniq * DSV3_DOWN_BYTES / (dn_us * 1e-6) / 1e9, 1),
            "l3_combine_us": round(t_us[STAGE_COMBINE], 3),
            "steps": steps, "shared_copies": nb,
        }
        del graphs, layer
        torch.cuda.empty_cache()
    del pool, shared
    torch.cuda.empty_cache()
    return res


# ----------------------------------------------------------- C3: prefill

def bench_prefill(args, pool, stride, fmt=None, ceiling=True) -> dict:
    """The Qwen3-30B-A3B-shaped layer at prefill: 4096 bf16 tokens with
    Zipf(1.0)-skewed routing, through the grouped bf16 MFMA GEMM path (Q4_K
    experts, or fmt's)."""
    import dataclasses
    import numpy as np
    import torch

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
    steps = args.prefill_steps
    stages = {"route": STAGE_ROUTE, "batches": STAGE_BATCHES, "tiles": STAGE_TILES, "gemm_gateup": STAGE_PF_GATEUP,
              "gemm_down": STAGE_PF_DOWN, "combine": STAGE_COMBINE}
    for st in stages.values():
        Q.moe_timer_begin(st, steps)
    for _ in range(steps):
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
    ms_step = timed_replays(lambda i: g.replay(), steps)
    gu_flop = 2.0 * M * (2 * wl.I) * wl.H
    dn_flop = 2.0 * M * wl.H * wl.I
    gu_tf = gu_flop / (kern["gemm_gateup"] * 1e-6) / 1e12
    dn_tf = dn_flop / (kern["gemm_down"] * 1e-6) / 1e12
    both_tf = (gu_flop + dn_flop) / ((kern["gemm_gateup"] + kern["gemm_down"]) * 1e-6) / 1e12
    out = {
        "workload": wl.name, "T": wl.T, "steps": steps, "ms_per_step": round(ms_step, 4),
        "tokens_per_s": round(wl.T / (ms_step * 1e-3), 1), "expert_rows_total": M,
        "expert_rows_max": int(counts.max()), "expert_rows_min": int(counts.min()),
        "roofline_kernel": "prefill gate/up grouped GEMM (weights -> bf16 fragments, bf16 MFMA)",
        "roofline_bound": "mfma", "roofline_achieved_TFLOPs": round(gu_tf, 1),
        "roofline_peak_TFLOPs": MFMA_BF16_PEAK_TFLOPS, "roofline_frac": round(gu_tf / MFMA_BF16_PEAK_TFLOPS, 4),
        "roofline_algorithmic_flop_per_launch": gu_flop, "roofline_avg_launch_us": round(kern["gemm_gateup"], 2),
        "down_gemm_us": round(kern["gemm_down"], 2), "down_gemm_TFLOPs": round(dn_tf, 1),
        "down_gemm_frac": round(dn_tf / MFMA_BF16_PEAK_TFLOPS, 4),
        "expert_gemms_TFLOPs": round(both_tf, 1), "expert_gemms_frac": round(both_tf / MFMA_BF16_PEAK_TFLOPS, 4),
        "route_us": round(kern["route"], 2), "batches_us": round(kern["batches"], 2),
        "tiles_us": round(kern["tiles"], 2), "combine_us": round(kern["combine"], 2),
    }
    if ceiling:
        out.update(library_gemm_ceiling(M, wl.H, wl.I))
    if fmt is None:
        out["int8_path"] = bench_prefill_i8(args, pool, stride, wl, x, lg, soe, spec, gu_flop, dn_flop)
    return out


def bench_prefill_i8(args, pool, stride, wl, x, lg, soe, spec, gu_flop: float, dn_flop: float) -> dict:
    """The same layer through MOE_PATH_PREFILL_I8 (int8 activations in two
    planes on the i8 MFMA, per-sub-block fp32 rescaling): its GEMMs' times
    (stage timers) against the int8 peak, and a step's time."""
    import torch

    import quantized_routed_expert_moe_amd as Q
    from quantized_routed_expert_moe_amd.layer import MoELayer

    layer = MoELayer(spec, wl.T, wl.E, pool, stride, soe, path=Q.MOE_PATH_PREFILL_I8, y_dtype=torch.bfloat16,
                     pair_dtype=torch.bfloat16)
    for _ in range(3):
        layer.forward(x, lg)
    torch.cuda.synchronize()
    steps = args.prefill_steps
    for st in (STAGE_PF_GATEUP, STAGE_PF_DOWN):
        Q.moe_timer_begin(st, steps)
    for _ in range(steps):
        layer.forward(x, lg)
    torch.cuda.synchronize()
    ms_gu, n_gu = Q.moe_timer_end(STAGE_PF_GATEUP)
    ms_dn, n_dn = Q.moe_timer_end(STAGE_PF_DOWN)
    gu_us, dn_us = 1e3 * ms_gu / max(n_gu, 1), 1e3 * ms_dn / max(n_dn, 1)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.forward(x, lg)
    g.replay()
    ms_step = timed_replays(lambda i: g.replay(), steps)
    # two int8 planes: the contraction's MACs run twice on the i8 MFMA
    gu_tops = 2 * gu_flop / (gu_us * 1e-6) / 1e12
    dn_tops = 2 * dn_flop / (dn_us * 1e-6) / 1e12
    return {"ms_per_step": round(ms_step, 4), "tokens_per_s": round(wl.T / (ms_step * 1e-3), 1),
            "gemm_gateup_us": round(gu_us, 2), "gemm_down_us": round(dn_us, 2),
            "gateup_TFLOPs_of_the_contraction": round(gu_flop / (gu_us * 1e-6) / 1e12, 1),
            "gateup_int8_TOPs": round(gu_tops, 1), "gateup_frac_of_int8_peak": round(gu_tops / MFMA_INT8_PEAK_TOPS, 4),
            "down_int8_TOPs": round(dn_tops, 1), "down_frac_of_int8_peak": round(dn_tops / MFMA_INT8_PEAK_TOPS, 4),
            "note": "int8 ops = 2 planes x the contraction's 2 M N K; the bf16 path (the object above) is AUTO's choice"}


def library_gemm_ceiling(M: int, H: int, I: int, reps: int = 20) -> dict:
    """What the platform's tuned dense bf16 GEMM (torch.matmul, i.e.
    hipBLASLt) reaches on plain dense operands of the prefill's total shapes
    (all M rows in one GEMM, weights already bf16, no grouping or
    dequantization): the practical MFMA ceiling the grouped kernels are read
    against.  Run only; nothing of it is used."""
    import torch
    out = {}
    for name, (m, k, n) in {"gateup": (M, H, 2 * I), "down": (M, I, H)}.items():
        a = torch.randn(m, k, device="cuda", dtype=torch.bfloat16)
        b = torch.randn(k, n, device="cuda", dtype=torch.bfloat16).contiguous()
        for _ in range(3):
            torch.matmul(a, b)
        us = 1e3 * timed_replays(lambda i: torch.matmul(a, b), reps)
        out[f"hipblaslt_dense_{name}_TFLOPs"] = round(2.0 * m * k * n / (us * 1e-6) / 1e12, 1)
        del a, b
    torch.cuda.empty_cache()
    return out


def leg_prefill(args, thr: dict) -> dict:
    import torch
    from fixtures import workloads as W
    wl = W.QWEN3_PREFILL
    host, stride = pack_pool(wl.fmt, W.expert_blobs(wl), wl.H, wl.I, thr["threads"])
    pool = torch.from_numpy(host).cuda()
    del host
    out = bench_prefill(args, pool, stride)
    del pool
    torch.cuda.empty_cache()
    return out


# ------------------------------------------------------------ C2: Qwen3 T=2

def leg_qwen3(args, thr: dict) -> dict:
    """The Qwen3-30B-A3B-shaped decode layer at T = 2; 16 copies of the slot
    pool rotate with 16 input batches."""
    import numpy as np
    import torch

    import quantized_routed_expert_moe_amd as Q
    from fixtures import workloads as W
    from quantized_routed_expert_moe_amd.layer import LayerSpec, MoELayer

    wl = W.QWEN3_DECODE_T2
    copies = 16
    host, stride = pack_pool(wl.fmt, W.expert_blobs(wl), wl.H, wl.I, thr["threads"])
    pool0 = torch.from_numpy(host).cuda()
    del host
    pools = [pool0] + [pool0.clone() for _ in range(copies - 1)]
    xs = [torch.from_numpy(W.x_of(wl, seed=100 + i)).cuda() for i in range(copies)]
    ls = [torch.from_numpy(W.logits_of(wl, seed=100 + i)).cuda() for i in range(copies)]
    soe = torch.arange(wl.E, dtype=torch.int32, device="cuda")
    spec = LayerSpec(wl.fmt, wl.H, wl.I, wl.E, wl.k, wl.score, wl.renormalize, wl.scale)
    layer = MoELayer(spec, wl.T, wl.E, pool0, stride, soe, path=Q.MOE_PATH_DECODE)
    uniq = []
    for i in range(copies):
        layer.forward(xs[i], ls[i], slot_pool=pools[i])
        uniq.append(int(torch.unique(layer.ids).numel()))
    torch.cuda.synchronize()
    gu_per = 2 * wl.I * wl.H // 256 * 144
    step = lambda i: layer.forward(xs[i % copies], ls[i % copies], slot_pool=pools[i % copies])  # noqa: E731
    steps = args.qwen3_steps
    for i in range(50):
        step(i)
    Q.moe_timer_begin(STAGE_GATEUP, steps)
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    gu = Q.moe_timer_read(STAGE_GATEUP, steps)
    Q.moe_timer_end(STAGE_GATEUP)
    graphs = []
    for i in range(copies):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(i)
        graphs.append(g)
    for i in range(2 * copies):
        graphs[i % copies].replay()
    ms = timed_replays(lambda i: graphs[i % copies].replay(), steps)
    gu_bytes = float(np.mean([uniq[i % copies] for i in range(steps)])) * gu_per
    gu_us = 1e3 * float(np.mean(gu))
    traffic = read_traffic("qwen3")
    out = {"workload": wl.name, "tokens_per_s": round(wl.T / (ms * 1e-3), 1), "ms_per_step": round(ms, 5),
           "roofline_kernel": "Q4_K gate/up GEMV + SwiGLU", "roofline_bound": "hbm",
           "roofline_achieved_GBs": round(gu_bytes / (gu_us * 1e-6) / 1e9, 1), "roofline_peak_GBs": HBM_PEAK_GBS,
           "roofline_frac": round(gu_bytes / (gu_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
           "roofline_algorithmic_bytes_per_launch": round(gu_bytes), "roofline_avg_launch_us": round(gu_us, 3),
           "roofline_traffic": traffic, "pool_copies": copies, "steps": steps}
    del graphs, layer, pools, pool0
    torch.cuda.empty_cache()
    return out


# ------------------------------------------- other card types (--extra only)

def bench_formats(args, thr: dict) -> dict:
    """The decode layers with the other card expert types (MXFP4, Q3_K/Q4_K,
    Q5_K, Q6_K) at the Qwen3 shape (8 pool copies rotated) and the
    DeepSeek-V3 shape with the Q8_0 shared expert, graph-replayed, and the
    Qwen3-shaped prefill of each."""
    import numpy as np
    import torch

    import fixtures as F
    import quantized_routed_expert_moe_amd as Q
    from fixtures import workloads as W
    from quantized_routed_expert_moe_amd.layer import LayerSpec, MoELayer

    threads = thr["threads"]
    res = {}
    for key, wl, copies in (("mxfp4_qwen3_T2", W.QWEN3_MXFP4_DECODE_T2, 8), ("mxfp4_dsv3_T2", W.DSV3_MXFP4_DECODE_T2, 1),
                            ("q3k_q4k_dsv3_T2", W.DSV3_Q3K_DECODE_T2, 1), ("q3k_q4k_qwen3_T2", W.QWEN3_Q3K_DECODE_T2, 8),
                            ("q5k_qwen3_T2", W.QWEN3_Q5K_DECODE_T2, 8), ("q5k_dsv3_T2", W.DSV3_Q5K_DECODE_T2, 1),
                            ("q6k_qwen3_T2", W.QWEN3_Q6K_DECODE_T2, 8), ("q6k_dsv3_T2", W.DSV3_Q6K_DECODE_T2, 1)):
        nb = Q.moe_expert_blob_bytes(wl.fmt, wl.H, wl.I)
        host, stride = pack_pool(wl.fmt, W.expert_blobs(wl), wl.H, wl.I, threads)
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
        graphs = []
        for i in range(nbatch):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                layer.forward(xs[i], ls[i], slot_pool=pools[i % copies])
            graphs.append(g)
        for i in range(2 * nbatch):
            graphs[i % nbatch].replay()
        steps = args.dsv3_steps
        ms = timed_replays(lambda i: graphs[i % nbatch].replay(), steps)
        mean_uniq = float(np.mean([uniq[i % nbatch] for i in range(steps)]))
        layer_bytes = mean_uniq * nb + shared_bytes
        r = {"tokens_per_s": round(wl.T / (ms * 1e-3), 1), "ms_per_step": round(ms, 5),
             "layer_GBs": round(layer_bytes / (ms * 1e-3) / 1e9, 1),
             "layer_frac_of_hbm": round(layer_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        if "qwen3" in key and args.prefill_steps > 0:
            pre = bench_prefill(args, pools[0], stride, fmt=wl.fmt, ceiling=False)
            r["prefill_T4096"] = {kk: pre[kk] for kk in ("ms_per_step", "tokens_per_s", "roofline_frac",
                                                         "down_gemm_TFLOPs", "expert_gemms_frac")}
        res[key] = r
        del graphs, layer, pools, shared
        torch.cuda.empty_cache()
    return res


def bench_residency(st, wl, blobs, xs, dev_blobs, steps: int, threads: int, blob_of) -> dict:
    """The adaptive residency policy on the stack: decode steps from a start
    where each layer holds its lowest expert ids, with the policy off, with
    the swap rule, and with the swap rule after a prompt call has streamed
    its most-used experts onto the card.  Each step: one graph replay
    (card), then the host leg for every pair the card does not hold, then the
    policy (counters -> scores -> an 8-swap plan per layer), whose copies run
    on a side stream beside the next steps and are committed between steps
    once they have landed."""
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
                   replay_ms=round(1e3 * card_s / steps, 3), host_leg_ms=round(1e3 * host_s / steps, 2),
                   tokens_per_s=round(T * steps / (card_s + host_s), 2), swap_rounds=rounds, experts_swapped=swaps)
        return res

    return {"steps": steps, "start": "each layer's lowest 96 expert ids on the card",
            "policy": {"decay_shift": decay, "margin": margin, "swaps_per_layer_per_round": wl.staging},
            "off": arm(False, False), "swap_rule": arm(True, False), "swap_rule_and_prompt_streaming": arm(True, True)}


def leg_hbm(args) -> dict:
    """The practical HBM read rate: the library's streaming-read probe over a
    4 GiB buffer (each wave a contiguous span, 16-byte loads, 1..16 per lane
    in flight), 5 timed passes per (waves, depth) after 2 untimed ones; the
    best rate is the ceiling a read-bound kernel can reach on this card."""
    import torch

    import quantized_routed_expert_moe_amd as Q
    buf = torch.zeros(4 << 30, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(16384 * 64, dtype=torch.int32, device="cuda")
    grid = {}
    for waves in (1024, 2048, 4096, 8192, 16384):
        for depth in (1, 2, 4, 8, 16):
            for _ in range(2):
                Q.moe_hbm_read_probe(buf, waves, depth, sink)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            n = sum(Q.moe_hbm_read_probe(buf, waves, depth, sink) for _ in range(5))
            e1.record()
            torch.cuda.synchronize()
            grid[f"waves{waves}_depth{depth}"] = round(n / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
    best = max(grid, key=grid.get)
    del buf, sink
    torch.cuda.empty_cache()
    return {"kernel": "hbm_read_kernel: one 16-byte load per lane per step, depth steps in flight, contiguous span "
                      "per wave, 4 GiB buffer", "best_GBs": grid[best], "best_config": best,
            "best_frac_of_peak": round(grid[best] / HBM_PEAK_GBS, 4), "GBs": grid}


def leg_mfma(args) -> dict:
    """The prefill contraction's two designs side by side, operands in
    registers: the library's inner-loop probe (variant 0: Q4_K nibbles
    dequantized to bf16 + v_mfma_f32_32x32x16_bf16, the prefill GEMM's
    design; variant 1: int8 activations + v_mfma_i32_32x32x32_i8 with the
    per-sub-block fp32 rescaling and min term Q4_K needs; variant 2: variant
    1 with the two activation planes the int8 prefill path runs), 5 timed launches
    of 4096 sub-blocks per wave after 2 untimed ones.  The rate is the flops
    of the contraction the loop stands for per second: the ceiling a GEMM
    built on that design reaches with its memory traffic fully hidden."""
    import torch

    import quantized_routed_expert_moe_amd as Q
    out = torch.zeros(Q.PREFILL_PROBE_OUT_FLOATS, dtype=torch.float32, device="cuda")
    res = {}
    for variant, name in ((0, "bf16_dequant_mfma"), (1, "int8_mfma_rescale"), (2, "int8_two_plane_rescale")):
        for _ in range(2):
            Q.moe_prefill_inner_probe(variant, 4096, out)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        flops = sum(Q.moe_prefill_inner_probe(variant, 4096, out) for _ in range(5))
        e1.record()
        torch.cuda.synchronize()
        tf = flops / (e0.elapsed_time(e1) * 1e-3) / 1e12
        res[name] = {"TFLOPs": round(tf, 1), "frac_of_bf16_peak": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                     "frac_of_int8_peak": round(tf / MFMA_INT8_PEAK_TOPS, 4)}
    res["int8_over_bf16"] = round(res["int8_mfma_rescale"]["TFLOPs"] / res["bf16_dequant_mfma"]["TFLOPs"], 3)
    res["int8_two_plane_over_bf16"] = round(res["int8_two_plane_rescale"]["TFLOPs"]
                                            / res["bf16_dequant_mfma"]["TFLOPs"], 3)
    del out
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: every box here has one MI355X and the layer's kernels run on one device; "
              f"--gpus {args.gpus} is not supported.", file=sys.stderr)
        sys.exit(2)
    legs = [l for l in args.legs.split(",") if l]
    bad = [l for l in legs if l not in LEGS]
    if bad:
        print(f"unknown legs {bad}; choose from {LEGS}", file=sys.stderr)
        sys.exit(2)

    import torch

    import fixtures as F
    import quantized_routed_expert_moe_amd as Q

    Q.lib()  # fail loudly if the HIP library is missing
    assert torch.cuda.is_available()
    thr = host_threads()
    F.set_num_threads(thr["threads"])
    t_start = time.time()
    extra = {} if args.extra else None

    def progress(msg: str) -> None:
        print(f"[bench {time.time() - t_start:6.1f} s] {msg}", file=sys.stderr, flush=True)

    res = {}
    if "stack" in legs:
        progress("58-layer stack")
        res["stack"] = leg_stack(args, thr, extra)
    if "dsv3" in legs:
        progress("DeepSeek-V3-shaped layer, T=2 and T=4")
        res["dsv3"] = leg_dsv3(args, thr)
    if "prefill" in legs:
        progress("Qwen3-shaped prefill, T=4096")
        res["prefill"] = leg_prefill(args, thr)
    if "qwen3" in legs:
        progress("Qwen3-shaped decode, T=2")
        res["qwen3"] = leg_qwen3(args, thr)
    if "hbm" in legs:
        progress("streaming-read probe")
        res["hbm"] = leg_hbm(args)
    if "mfma" in legs:
        progress("prefill inner-loop probe (bf16 vs int8 designs)")
        res["mfma"] = leg_mfma(args)
    if extra is not None:
        progress("other card expert types")
        extra["formats"] = bench_formats(args, thr)
        print(json.dumps({"bench_extra": extra}), file=sys.stderr, flush=True)
    if args.profile_copy:
        a = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()

    head = res.get("stack")
    out = {
        "metric": METRIC,
        "value": round(head["value"], 1) if head else None,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 5) if head else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "arithmetic": "q4_k/q8_0 weights dequantized to fp16, fp16 x fp16 dot products, fp32 accumulate",
        "data": "synthetic (seeded N(0,0.02) weights quantized to Q4_K / Q8_0, N(0,1) activations, Zipf(1.1) routing)",
        "config": {"workload": "58-layer DeepSeek-V3-shaped MoE stack, 96 of 256 routed experts resident per layer, "
                               "decode T=2, one hipGraph replay per step",
                   "layers": 58, "T": 2, "H": 7168, "E": 256, "top_k": 8, "I": 2048, "I_shared": 2048,
                   "routing": "sigmoid, renormalised over top-8, x2.5", "weights": "routed Q4_K, shared Q8_0",
                   "value": "T x 58 / replay time (MoE-layer tokens/s)"},
        "roofline": dict(head["roofline"], frac_of_measured_read_rate=round(
            head["roofline"]["achieved"] / res["hbm"]["best_GBs"], 4) if "hbm" in res else None) if head else None,
        "cpu_baseline": head["cpu_baseline"] if head else None,
        "stack": head["stack"] if head else None,
        "c4_decode_T2": res["dsv3"]["T2"] if "dsv3" in res else None,
        "c4_decode_T4": res["dsv3"]["T4"] if "dsv3" in res else None,
        "c3_prefill": res.get("prefill"),
        "c2_decode_T2": res.get("qwen3"),
        "hbm_read_probe": res.get("hbm"),
        "prefill_inner_loop_probe": res.get("mfma"),
        "host_threads": thr,
        "wall_s": round(time.time() - t_start, 1),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
