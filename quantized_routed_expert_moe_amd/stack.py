"""A stack of MoE layers under partial residency, replayed as one HIP graph,
with expert swaps between replays.

Each layer keeps some of its routed experts in HBM slots and routes the rest
to a host list (bloomery README of 2026-09-24, opening list: each routed
layer keeps some of its experts on the GPU, the rest run on the host tier
inside the same captured step; bloomery V4.1 README, "Adaptive residency":
experts are swapped between the card and the host between steps).

Orchestration only; every computation is a libqmoe call:
  * per layer: an HBM slot pool of S = resident + staging slots, a slot map
    (expert -> slot, -1 = host), a shared expert, the layer's buffers;
  * capture(): all layers back to back on one stream into one graph; each
    layer's batching kernel writes its host list straight into pinned host
    memory, so the graph holds no copies;
  * swap_begin() / swap_commit(): for every layer, copy the packed blobs of
    `n` incoming experts from pinned host memory into free slots with
    hipMemcpyAsync on a side stream, overlapping any number of replays (free
    slots are not in the current maps); once the copies have landed, upload
    the new slot maps after the replay in flight; the next replay waits for
    that.  swap() does both for one round.

Which experts a round swaps is either given (`plans`, one (incoming,
outgoing) pair of lists per layer) or, without plans, the rotation rule that
measures swap throughput: the incoming experts are the next `n` non-resident
ones in the layer's frequency ranking after a cursor that starts at the first
non-resident rank and wraps, the outgoing ones the `n` lowest-ranked resident
experts.  Incoming experts take the free slots (at first the staging slots,
then the slots the previous round freed).

Adaptive residency (bloomery V4.1 README, "Adaptive residency": the engine
counts its own routing and swaps experts between card and host between
steps; a prompt call streams its hottest host experts onto the card): every
layer's routing launch also adds its pairs to that layer's row of
`counts` (device, [layers, E]); AdaptiveResidency reads them between steps
and plans the rounds with the host library's policy, and stream_in() seats a
prompt's most-used experts before decode starts.
"""
from __future__ import annotations

import numpy as np
import torch

from . import (MOE_FMT_Q4K, MOE_PATH_DECODE, RESIDENCY_FRAC_BITS, moe_count_routes, moe_residency_plan,
               moe_residency_update_scores, moe_route_topk, moe_validate_slot_map)
from .layer import LayerSpec, MoELayer


class ResidentStack:
    def __init__(self, spec: LayerSpec, n_layers: int, T: int, n_resident: int, n_staging: int,
                 ranked: list, blob_of, host_blobs: torch.Tensor, dev_blobs: torch.Tensor | None,
                 shared_of, shared_host: torch.Tensor):
        """ranked[l]: experts of layer l by descending routing frequency (rank r
        resident in slot r at start).  blob_of(l, e): row of host_blobs (packed,
        pinned, [n_blobs, stride]) holding expert e of layer l.  dev_blobs: the
        same rows on the device (used to fill the pools quickly; may be None).
        shared_of(l): row of shared_host (packed Q8_0 blobs) for layer l."""
        assert spec.fmt == MOE_FMT_Q4K
        self.spec, self.L, self.T = spec, n_layers, T
        self.nres, self.nstage = n_resident, n_staging
        self.S = n_resident + n_staging
        self.ranked = [np.asarray(r, dtype=np.int64) for r in ranked]
        self.blob_of, self.host_blobs = blob_of, host_blobs
        self.stride = host_blobs.shape[1]
        E = spec.E
        dev = "cuda"
        self.maps = []            # host slot maps (np.int32 [E]) of the next replay
        self.free = []            # free slots per layer
        self.cursor = []          # swap cursor into ranked[l]
        self.pools, self.dev_maps, self.layers = [], [], []
        self.x = []
        # routing counters (uint32 bits in int32) and the step's gate logits, one row per layer
        self.counts = torch.zeros((n_layers, E), dtype=torch.int32, device=dev)
        self.logits_all = torch.zeros((n_layers, T, E), dtype=torch.float32, device=dev)
        self.logits = [self.logits_all[l] for l in range(n_layers)]
        src = dev_blobs if dev_blobs is not None else host_blobs
        for l in range(n_layers):
            soe = np.full(E, -1, dtype=np.int32)
            soe[self.ranked[l][:n_resident]] = np.arange(n_resident, dtype=np.int32)
            self.maps.append(soe)
            self.free.append(list(range(n_resident, self.S)))
            self.cursor.append(n_resident)
            pool = torch.empty((self.S, self.stride), dtype=torch.uint8, device=dev)
            self.pools.append(pool)
            self.dev_maps.append(torch.from_numpy(soe.copy()).to(dev))
        # fill resident slots, grouped by source blob so each source stays hot in cache
        jobs = []
        for l in range(n_layers):
            for s in range(n_resident):
                jobs.append((self.blob_of(l, int(self.ranked[l][s])), l, s))
        jobs.sort()
        for b, l, s in jobs:
            self.pools[l][s].copy_(src[b], non_blocking=True)
        self.shared_pools = []
        for l in range(n_layers):
            sp = torch.empty((1, shared_host.shape[1]), dtype=torch.uint8, device=dev)
            sp[0].copy_(shared_host[shared_of(l)], non_blocking=True)
            self.shared_pools.append(sp)
        torch.cuda.synchronize()
        for l in range(n_layers):
            self.layers.append(MoELayer(spec, T, self.S, self.pools[l], self.stride, self.dev_maps[l],
                                        self.shared_pools[l], MOE_PATH_DECODE, host_list_pinned=True,
                                        route_counts=self.counts[l]))
            self.x.append(torch.zeros((T, spec.H), dtype=torch.float32, device=dev))
        self.pin_maps = [torch.zeros(E, dtype=torch.int32).pin_memory() for _ in range(n_layers)]
        self.graph = None
        self.side = torch.cuda.Stream()  # swap copies; capture() may replace it (_pick_copy_stream)
        self.side_probes, self.side_overlaps = 0, None
        self.replay_done = torch.cuda.Event(enable_timing=True)
        self.replay_start = torch.cuda.Event(enable_timing=True)
        self.swap_start = torch.cuda.Event(enable_timing=True)
        self.swap_copies_done = torch.cuda.Event(enable_timing=True)
        self.maps_done = torch.cuda.Event(enable_timing=True)
        self.pending_maps = False
        self.swap_in_flight = False
        self.swap_plans = None

    # ------------------------------------------------------------ step
    def set_inputs(self, xs, logits) -> None:
        for l in range(self.L):
            self.x[l].copy_(xs[l])
            self.logits[l].copy_(logits[l])

    def set_logits(self, logits: np.ndarray) -> None:
        """The next step's gate logits, float32 [layers, T, E], in one copy
        (ordered before the next replay on the current stream)."""
        self.logits_all.copy_(torch.from_numpy(np.ascontiguousarray(logits, dtype=np.float32)))

    def read_counts(self) -> np.ndarray:
        """The routing counters, uint32 [layers, E], once the current stream
        has passed every replay so far."""
        return self.counts.cpu().numpy().view(np.uint32)

    def prompt_counts(self, logits) -> np.ndarray:
        """A prompt's routing counts per layer, uint32 [layers, E]: each
        layer's prompt logits (float32 [P, E]) routed on the device and
        counted there (moe_route_topk, moe_count_routes)."""
        spec = self.spec
        counts = torch.zeros((self.L, spec.E), dtype=torch.int32, device="cuda")
        for l in range(self.L):
            lg = torch.from_numpy(np.ascontiguousarray(logits[l], dtype=np.float32)).cuda()
            P = lg.shape[0]
            ids = torch.empty((P, spec.k), dtype=torch.int32, device="cuda")
            w = torch.empty((P, spec.k), dtype=torch.float32, device="cuda")
            moe_route_topk(lg, spec.k, spec.score, spec.renormalize, spec.scale, ids, w)
            moe_count_routes(ids, spec.E, counts[l])
        return counts.cpu().numpy().view(np.uint32)

    def _step_body(self) -> None:
        for l in range(self.L):
            self.layers[l].forward(self.x[l], self.logits[l])

    def run_eager(self) -> None:
        self._wait_maps()
        self._step_body()
        self.replay_done.record()

    def capture(self) -> torch.cuda.CUDAGraph:
        self._step_body()  # warm-up outside capture
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph(keep_graph=True)
        with torch.cuda.graph(g):
            self._step_body()
        g.instantiate()
        self.graph = g
        self._pick_copy_stream()
        return g

    def _pick_copy_stream(self, tries: int = 8, n_copies: int = 40) -> None:
        """Choose the swap-copy stream that the replays do not queue behind.
        Streams share the process's few hardware queues, and a replay's
        kernels, forked branches included, queued on the copy stream's queue
        would wait for a whole round of copies.  Which queue a stream sits on
        is not visible, so candidates from torch's stream pool are tried with
        the captured graph itself: about 1 GB of expert blobs is copied into
        one free slot on the candidate while the graph replays on the current
        stream, and the candidate is kept if the replay ends while the copies
        still run.  Free slots hold nothing a replay reads, and the replay only
        repeats the step of the current inputs."""
        if self.swap_in_flight or not self.free[0]:
            return
        cand = self.side
        slot = self.pools[0][self.free[0][0]]
        srcs = [self.host_blobs[b % self.host_blobs.shape[0]] for b in range(n_copies)]
        copied = torch.cuda.Event()
        for n in range(1, tries + 1):
            torch.cuda.synchronize()
            with torch.cuda.stream(cand):
                for src in srcs:
                    slot.copy_(src, non_blocking=True)
                copied.record(cand)
            self.replay()
            self.replay_done.synchronize()
            overlapped = not copied.query()
            copied.synchronize()
            self.side_probes, self.side_overlaps = n, overlapped
            if overlapped:
                self.side = cand
                return
            cand = torch.cuda.Stream()

    def graph_node_count(self) -> int:
        import ctypes
        hip = ctypes.CDLL("libamdhip64.so")
        n = ctypes.c_size_t(0)
        rc = hip.hipGraphGetNodes(ctypes.c_void_p(self.graph.raw_cuda_graph()), None, ctypes.byref(n))
        if rc != 0:
            raise RuntimeError(f"hipGraphGetNodes failed ({rc})")
        return int(n.value)

    def _wait_maps(self) -> None:
        if self.pending_maps:
            torch.cuda.current_stream().wait_event(self.maps_done)
            self.pending_maps = False

    def replay(self) -> None:
        self._wait_maps()
        self.replay_start.record()
        self.graph.replay()
        self.replay_done.record()

    def outputs(self) -> list:
        return [lay.y for lay in self.layers]

    def host_lists(self, l: int) -> dict:
        """Layer l's host list from the last completed replay (the caller
        synchronises first)."""
        h = self.layers[l].host_list.numpy()
        P = (h.size - 1) // 3
        c = int(h[3 * P])
        return dict(token=h[:c].copy(), expert=h[P:P + c].copy(), weight=h[2 * P:2 * P + c].view(np.float32).copy())

    # ------------------------------------------------------------ swaps
    def plan_swap(self, l: int, n: int) -> tuple[list, list]:
        """(incoming experts, outgoing experts) of layer l for the next round."""
        soe, ranked, E = self.maps[l], self.ranked[l], self.spec.E
        incoming, c = [], self.cursor[l]
        for _ in range(E):
            e = int(ranked[c % E])
            c += 1
            if soe[e] < 0:
                incoming.append(e)
                if len(incoming) == n:
                    break
        self.cursor[l] = c % E
        rank_of = np.empty(E, dtype=np.int64)
        rank_of[ranked] = np.arange(E)
        resident = [int(e) for e in np.nonzero(soe >= 0)[0]]
        resident.sort(key=lambda e: -rank_of[e])
        outgoing = resident[:n]
        return incoming, outgoing

    def swap_begin(self, n: int = 8, plans: list | None = None) -> dict:
        """Start one swap round on every layer: take its plan (plans[l] =
        (incoming, outgoing), at most as many as the layer's free slots) or
        make one with the rotation rule, and enqueue the copies of the
        incoming experts into free slots on the side stream.  Returns at
        once; replays may go on with the current maps meanwhile (free slots are
        not referenced by them).  The side stream runs the rounds in order, so
        these copies also follow the previous round's map upload, i.e. the
        last replay that could still use a slot freed by that round."""
        assert not self.swap_in_flight, "commit the previous swap round first"
        given = plans
        plans = []
        self.swap_start.record(self.side)
        with torch.cuda.stream(self.side):
            for l in range(self.L):
                inc, out = self.plan_swap(l, n) if given is None else (list(given[l][0]), list(given[l][1]))
                if len(inc) != len(out) or len(self.free[l]) < len(inc):
                    raise ValueError(f"layer {l}: {len(inc)} incoming, {len(out)} outgoing, "
                                     f"{len(self.free[l])} free slots")
                if any(self.maps[l][e] >= 0 for e in inc) or any(self.maps[l][e] < 0 for e in out):
                    raise ValueError(f"layer {l}: plan swaps in a resident expert or out a host one")
                slots = [self.free[l].pop(0) for _ in inc]
                for e, s in zip(inc, slots):
                    self.pools[l][s].copy_(self.host_blobs[self.blob_of(l, e)], non_blocking=True)
                plans.append((inc, out, slots))
            self.swap_copies_done.record(self.side)
        self.swap_plans = plans
        self.swap_in_flight = True
        return dict(incoming=[p[0] for p in plans], outgoing=[p[1] for p in plans])

    def swap_commit(self, block: bool = False) -> bool:
        """If the copies of the round in flight have landed (or, with block,
        once they have), switch to the new slot maps: the side stream waits for
        the replay in flight, uploads the maps, and the next replay waits for
        the upload.  Returns whether the round was committed."""
        if not self.swap_in_flight:
            return False
        # Once this round's copies are done, so is everything earlier on the
        # side stream, including the previous upload from the pinned maps.
        if block:
            self.swap_copies_done.synchronize()
        elif not self.swap_copies_done.query():
            return False
        with torch.cuda.stream(self.side):
            self.side.wait_event(self.replay_done)  # the running replay still reads the old maps
            for l, (inc, out, slots) in enumerate(self.swap_plans):
                soe = self.maps[l]
                for e, s in zip(inc, slots):
                    soe[e] = s
                for e in out:
                    self.free[l].append(int(soe[e]))
                    soe[e] = -1
                moe_validate_slot_map(soe, self.S)
                self.pin_maps[l].copy_(torch.from_numpy(soe))
                self.dev_maps[l].copy_(self.pin_maps[l], non_blocking=True)
            self.maps_done.record(self.side)
        self.pending_maps = True
        self.swap_in_flight = False
        self.swap_plans = None
        return True

    def swap(self, n: int = 8) -> dict:
        """One swap round on every layer: copies on the side stream overlap the
        replay in flight; the new slot maps are uploaded after it finishes."""
        plan = self.swap_begin(n)
        self.swap_commit(block=True)
        return plan

    def stream_in(self, plans: list) -> float:
        """Apply plans[l] = (incoming, outgoing) in place, now: each incoming
        expert's blob is copied from pinned host memory into its outgoing
        partner's slot.  For the prompt call's streaming, before decode
        starts: waits for all work on the device first (no replay may still
        read the slots).  Returns the seconds the copies took."""
        import time
        assert not self.swap_in_flight, "commit the swap round in flight first"
        torch.cuda.synchronize()
        t0 = time.time()
        for l in range(self.L):
            inc, out = plans[l]
            soe = self.maps[l]
            if len(inc) != len(out) or any(soe[e] >= 0 for e in inc) or any(soe[e] < 0 for e in out):
                raise ValueError(f"layer {l}: bad plan")
            for e_in, e_out in zip(inc, out):
                slot = int(soe[e_out])
                self.pools[l][slot].copy_(self.host_blobs[self.blob_of(l, int(e_in))], non_blocking=True)
                soe[e_in], soe[e_out] = slot, -1
            moe_validate_slot_map(soe, self.S)
            self.dev_maps[l].copy_(torch.from_numpy(soe.copy()))
        torch.cuda.synchronize()
        return time.time() - t0

    def reset(self, ranked: list, src: torch.Tensor | None = None) -> None:
        """Start over with ranked[l][:n_resident] in slots 0.. of layer l (the
        rest on the host, the staging slots free), blobs copied from src
        (device rows as host_blobs; default host_blobs).  No swap round may be
        in flight."""
        assert not self.swap_in_flight, "commit the swap round in flight first"
        torch.cuda.synchronize()
        src = self.host_blobs if src is None else src
        E = self.spec.E
        self.ranked = [np.asarray(r, dtype=np.int64) for r in ranked]
        for l in range(self.L):
            soe = np.full(E, -1, dtype=np.int32)
            soe[self.ranked[l][:self.nres]] = np.arange(self.nres, dtype=np.int32)
            self.maps[l][:] = soe
            self.free[l] = list(range(self.nres, self.S))
            self.cursor[l] = self.nres
            for s in range(self.nres):
                self.pools[l][s].copy_(src[self.blob_of(l, int(self.ranked[l][s]))], non_blocking=True)
            self.dev_maps[l].copy_(torch.from_numpy(soe))
        self.pending_maps = False
        torch.cuda.synchronize()

    def current_maps(self) -> list:
        return [m.copy() for m in self.maps]


class AdaptiveResidency:
    """The adaptive residency policy driving a ResidentStack.  Between decode
    steps, observe() reads the stack's routing counters and updates each
    layer's running score with the pairs routed since the last read
    (moe_residency_update_scores); plans() gives each layer's swap plan
    (moe_residency_plan) for the next swap round.  prompt_plans() turns a
    prompt's routing counts into the scores and the plans of the prompt
    call's streaming (as many swaps as raise the card's count, margin 0)."""

    def __init__(self, stack: ResidentStack, decay_shift: int = 4, margin: int = 1 << RESIDENCY_FRAC_BITS):
        self.st, self.decay_shift, self.margin = stack, decay_shift, margin
        self.score = np.zeros((stack.L, stack.spec.E), dtype=np.uint64)
        self.prev = stack.read_counts().copy()

    def observe(self) -> np.ndarray:
        """Windows (uint32 [layers, E]): pairs routed since the last read; the
        scores are updated with them."""
        now = self.st.read_counts().copy()
        win = now - self.prev  # uint32: modulo 2^32, as the counters wrap
        self.prev = now
        for l in range(self.st.L):
            moe_residency_update_scores(self.score[l], win[l], self.decay_shift)
        return win

    def plans(self, max_swaps: int) -> list:
        return [moe_residency_plan(self.score[l], self.st.maps[l], max_swaps, self.margin) for l in range(self.st.L)]

    def prompt_plans(self, prompt_counts: np.ndarray) -> list:
        self.score = np.ascontiguousarray(prompt_counts, dtype=np.uint64) << np.uint64(RESIDENCY_FRAC_BITS)
        return [moe_residency_plan(self.score[l], self.st.maps[l], self.st.nres, 0) for l in range(self.st.L)]
