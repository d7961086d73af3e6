"""One MoE layer as library calls, with its buffers.

Orchestration only: device buffers come from torch, every step is a call
into libqmoe.  On the decode path (path = MOE_PATH_DECODE) the layer is one
call, moe_layer_decode: routing, batching, the routed and the shared expert
FFN and the combine as four launches on one stream.  Otherwise (prefill, or
fused=False) it is the sequence of separate calls: routing and batching
(moe_route_and_batch, one launch at decode sizes), the expert FFN, the
combine, with the optional shared expert served by moe_expert_ffn_q8_0 with
a one-slot identity batch on a side stream forked from the layer's stream by
an event and joined before the combine.  Nothing synchronises with the host,
so `forward` can be captured into a HIP graph.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from . import (MOE_FMT_Q8_0, MOE_PATH_AUTO, MOE_PATH_DECODE, MOE_PATH_PREFILL, moe_batches_workspace_size, moe_combine,
               moe_expert_ffn, moe_expert_ffn_q8_0, moe_ffn_workspace_size, moe_layer_decode,
               moe_layer_decode_workspace_size, moe_pack_expert, moe_packed_blob_bytes, moe_route_and_batch)


def upload_packed_experts(fmt: int, canonical_blobs: np.ndarray, H: int, I: int, stride: int | None = None,
                          device="cuda") -> tuple[torch.Tensor, int]:
    """Pack canonical blobs [n, bytes] on the host and upload them as a slot pool [n, stride] (uint8)."""
    n_bytes = moe_packed_blob_bytes(fmt, H, I)
    stride = stride or (n_bytes + 255) // 256 * 256
    n = canonical_blobs.shape[0]
    host = np.zeros((n, stride), dtype=np.uint8)
    for s in range(n):
        moe_pack_expert(fmt, canonical_blobs[s], H, I, out=host[s, :n_bytes])
    return torch.from_numpy(host).to(device), stride


@dataclass
class LayerSpec:
    fmt: int
    H: int
    I: int
    E: int
    k: int
    score: int = 0
    renormalize: bool = True
    scale: float = 1.0
    I_shared: int = 0  # 0 = no shared expert


class MoELayer:
    def __init__(self, spec: LayerSpec, T_max: int, S: int, slot_pool: torch.Tensor, stride: int,
                 slot_of_expert: torch.Tensor, shared_pool: torch.Tensor | None = None,
                 path: int = MOE_PATH_AUTO, y_dtype=torch.float32, pair_dtype=torch.float32, device="cuda",
                 host_list_pinned: bool = False, route_counts: torch.Tensor | None = None, fused: bool | None = None):
        """route_counts: optional device int32 [E] routing counters; every
        forward adds each routed pair to its expert's counter (the adaptive
        residency policy reads them).  fused: one moe_layer_decode call per
        forward (default on the decode path) or the separate calls."""
        self.spec, self.T_max, self.S, self.path = spec, T_max, S, path
        self.fused = (path == MOE_PATH_DECODE) if fused is None else bool(fused)
        if self.fused and (path != MOE_PATH_DECODE or y_dtype != torch.float32 or pair_dtype != torch.float32):
            raise ValueError("the fused layer is the decode path: fp32 y and y_pairs")
        self.slot_pool, self.stride, self.slot_of_expert = slot_pool, stride, slot_of_expert
        self.route_counts = route_counts
        self.shared_pool = shared_pool
        k, H, E = spec.k, spec.H, spec.E
        P = T_max * k
        i32 = dict(dtype=torch.int32, device=device)
        self.ids = torch.zeros((T_max, k), **i32)
        self.w = torch.zeros((T_max, k), dtype=torch.float32, device=device)
        self.slot_offsets = torch.zeros(S + 1, **i32)
        self.active_slots = torch.zeros(max(1, min(S, P)), **i32)
        self.num_active = torch.zeros(1, **i32)
        self.perm_pair = torch.zeros(max(1, P), **i32)
        # The host list (token, expert, weight per non-resident pair, then the
        # count) lives in one int32 buffer; the four arrays are views into it.
        # With host_list_pinned the buffer is pinned host memory that the
        # batching kernel writes directly (no copy): read it only once the
        # stream has passed forward().
        Pl = max(1, P)
        if host_list_pinned:
            self.host_list = torch.zeros(3 * Pl + 1, dtype=torch.int32, pin_memory=True)
        else:
            self.host_list = torch.zeros(3 * Pl + 1, **i32)
        self.host_token = self.host_list[0:Pl]
        self.host_expert = self.host_list[Pl:2 * Pl]
        self.host_weight = self.host_list[2 * Pl:3 * Pl].view(torch.float32)
        self.host_count = self.host_list[3 * Pl:]
        self.y_pairs = torch.zeros((max(1, P), H), dtype=pair_dtype, device=device)
        self.y = torch.zeros((T_max, H), dtype=y_dtype, device=device)
        if spec.I_shared:
            assert shared_pool is not None
        if self.fused:
            self.ws = torch.zeros(max(1, moe_layer_decode_workspace_size(spec.fmt, T_max, k, E, S, H, spec.I,
                                                                         spec.I_shared)), dtype=torch.uint8,
                                  device=device)
            return
        bws = moe_batches_workspace_size(T_max, k, E, S)
        self.batch_ws = torch.zeros(max(1, bws), dtype=torch.uint8, device=device) if bws else None
        self.ws = torch.zeros(max(1, moe_ffn_workspace_size(spec.fmt, T_max, k, H, spec.I, path)), dtype=torch.uint8,
                              device=device)
        if spec.I_shared:
            assert shared_pool is not None
            self.sh_offsets = torch.tensor([0, T_max], **i32)
            self.sh_active = torch.zeros(1, **i32)
            self.sh_num = torch.ones(1, **i32)
            self.sh_perm = torch.arange(T_max, **i32)
            self.sh_ws = torch.zeros(max(1, moe_ffn_workspace_size(MOE_FMT_Q8_0, T_max, 1, H, spec.I_shared,
                                                                   MOE_PATH_DECODE)), dtype=torch.uint8, device=device)
            self.y_shared = torch.zeros((T_max, H), dtype=torch.float32, device=device)
            self.sh_stride = shared_pool.shape[-1]
            # The shared expert needs no routing: it runs on a side stream
            # (default priority) forked from the layer's stream, so its weight
            # stream overlaps routing, batching and the routed FFN; combine
            # joins it.  Fork and join are events, so the pattern is captured
            # into graphs as two dependency edges.
            self.sh_stream = torch.cuda.Stream(device=device)
            self.sh_fork = torch.cuda.Event()
            self.sh_join = torch.cuda.Event()

    def forward(self, x: torch.Tensor, logits: torch.Tensor, stream=None, slot_pool: torch.Tensor | None = None,
                shared_pool: torch.Tensor | None = None):
        """slot_pool / shared_pool: another pool of the same layout for this
        call (e.g. one of several copies a benchmark rotates through)."""
        spec, T = self.spec, x.shape[0]
        assert T == self.T_max, "buffers are sized for T_max rows"
        pool = self.slot_pool if slot_pool is None else slot_pool
        sh_pool = self.shared_pool if shared_pool is None else shared_pool
        if self.fused:
            moe_layer_decode(spec.fmt, logits, x, spec.k, spec.score, spec.renormalize, spec.scale,
                             self.slot_of_expert, self.S, pool, self.stride, spec.I,
                             sh_pool if spec.I_shared else None, spec.I_shared, self.ids, self.w, self.slot_offsets,
                             self.active_slots, self.num_active, self.perm_pair, self.host_token, self.host_expert,
                             self.host_weight, self.host_count, self.y_pairs, self.y, self.ws, stream,
                             route_counts=self.route_counts)
            return self.y
        main = torch.cuda.current_stream() if stream is None else stream
        if spec.I_shared:
            self.sh_fork.record(main)
            self.sh_stream.wait_event(self.sh_fork)
            moe_expert_ffn_q8_0(sh_pool, self.sh_stride, 1, spec.H, spec.I_shared, x, 1, self.sh_offsets,
                                self.sh_active, self.sh_num, self.sh_perm, self.y_shared, MOE_PATH_DECODE, self.sh_ws,
                                self.sh_stream)
            self.sh_join.record(self.sh_stream)
        moe_route_and_batch(logits, spec.k, spec.score, spec.renormalize, spec.scale, self.ids, self.w, spec.E,
                            self.slot_of_expert, self.S, self.slot_offsets, self.active_slots, self.num_active,
                            self.perm_pair, self.host_token, self.host_expert, self.host_weight, self.host_count,
                            self.batch_ws, stream, route_counts=self.route_counts)
        moe_expert_ffn(spec.fmt)(pool, self.stride, self.S, spec.H, spec.I, x, spec.k, self.slot_offsets, self.active_slots,
            self.num_active, self.perm_pair, self.y_pairs, self.path, self.ws, stream)
        y_shared = None
        if spec.I_shared:
            main.wait_event(self.sh_join)
            y_shared = self.y_shared
        moe_combine(self.y_pairs, self.ids, self.w, self.slot_of_expert, self.S, y_shared, self.y, stream)
        return self.y
