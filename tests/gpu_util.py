"""Helpers of the GPU parity tests: build a layer on the device from a
workload's seeded inputs, run it through the C ABI, and run the oracle on
the same bytes."""
from __future__ import annotations

import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import fixtures as F
import oracle as O
import quantized_routed_expert_moe_amd as Q
from fixtures import workloads as W
from quantized_routed_expert_moe_amd.layer import LayerSpec, MoELayer

THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def pack_pool(fmt: int, blobs: np.ndarray, H: int, I: int, slots: list, n_slots: int) -> tuple[torch.Tensor, int]:
    """Device slot pool [n_slots, stride]: slot s holds the packed blob blobs[slots[s]] (None = empty)."""
    nb = Q.moe_packed_blob_bytes(fmt, H, I)
    stride = (nb + 255) // 256 * 256
    host = np.zeros((n_slots, stride), dtype=np.uint8)

    def one(s):
        if slots[s] is not None:
            Q.moe_pack_expert(fmt, blobs[slots[s]], H, I, out=host[s, :nb])

    with ThreadPoolExecutor(THREADS) as ex:
        list(ex.map(one, range(n_slots)))
    dev = torch.from_numpy(host).cuda()
    del host
    return dev, stride


def spec_of(w: W.Workload) -> LayerSpec:
    return LayerSpec(w.fmt, w.H, w.I, w.E, w.k, w.score, w.renormalize, w.scale, w.I_shared)


def device_layer(w: W.Workload, blobs: np.ndarray, soe: np.ndarray, S: int, shared: np.ndarray | None,
                 T: int, path: int = Q.MOE_PATH_AUTO, pair_dtype=torch.float32, y_dtype=torch.float32,
                 pool=None, host_list_pinned: bool = False) -> MoELayer:
    """blobs: canonical blobs indexed by expert id (all E)."""
    if pool is None:
        slots = [None] * S
        for e in range(w.E):
            if 0 <= soe[e] < S:
                slots[int(soe[e])] = e
        pool, stride = pack_pool(w.fmt, blobs, w.H, w.I, slots, S)
    else:
        pool, stride = pool
    shared_pool = None
    if shared is not None:
        shared_pool, _ = pack_pool(F.Q8_0, shared[None, :], w.H, w.I_shared, [0], 1)
    return MoELayer(spec_of(w), T, S, pool, stride, torch.from_numpy(soe).cuda(), shared_pool, path,
                    y_dtype=y_dtype, pair_dtype=pair_dtype, host_list_pinned=host_list_pinned)


def to_dev_x(x: np.ndarray) -> torch.Tensor:
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(x).cuda()


def run_device(layer: MoELayer, x: np.ndarray, logits: np.ndarray) -> dict:
    xd, ld = to_dev_x(x), torch.from_numpy(logits).cuda()
    y = layer.forward(xd, ld)
    torch.cuda.synchronize()
    out = dict(ids=layer.ids.cpu().numpy(), w=layer.w.cpu().numpy(), y=y.float().cpu().numpy(),
               slot_offsets=layer.slot_offsets.cpu().numpy(), num_active=int(layer.num_active.item()),
               host_count=int(layer.host_count.item()))
    out["active_slots"] = layer.active_slots.cpu().numpy()[:out["num_active"]]
    out["perm_pair"] = layer.perm_pair.cpu().numpy()[:int(out["slot_offsets"][-1])]
    hc = out["host_count"]
    out["host_token"] = layer.host_token.cpu().numpy()[:hc]
    out["host_expert"] = layer.host_expert.cpu().numpy()[:hc]
    out["host_weight"] = layer.host_weight.cpu().numpy()[:hc]
    out["y_pairs"] = layer.y_pairs.float().cpu().numpy()
    return out


def run_oracle(w: W.Workload, blobs: np.ndarray, x: np.ndarray, logits: np.ndarray, soe: np.ndarray,
               shared: np.ndarray | None, want_pairs: bool = False, S: int | None = None) -> dict:
    """The oracle's layer; a pair is on the card iff its slot is in [0, S) (S defaults to E)."""
    O.set_threads(THREADS)
    ids_needed = set(np.argsort(-logits, axis=1, kind="stable")[:, :w.k].ravel().tolist())
    expert_list = [blobs[e] if e in ids_needed else None for e in range(w.E)]
    return O.moe_layer(w.fmt, expert_list, w.H, w.I, W.x_f64(w, x), logits, w.k, w.score, w.renormalize, w.scale,
                       soe, shared, F.Q8_0, w.I_shared, want_pairs, S=S)


def rel_max_err(got: np.ndarray, want: np.ndarray) -> float:
    return float(np.abs(got - want).max() / max(np.abs(want).max(), 1e-300))
