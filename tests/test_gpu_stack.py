"""The 58-layer DeepSeek-V3-shaped stack under partial residency (96 of 256
experts per layer in HBM slots, 8 staging slots), replayed as one HIP graph,
with 8-expert swaps per layer between replays.

Every layer's expert ids and host list match the oracle bit for bit; the
outputs of sampled layers are within the decode tolerance of the oracle run
with that replay's slot map; a graph replay equals eager execution bit for
bit; the graph's node count is pinned.  Under the adaptive residency policy
the routing counters, scores, prompt streaming and swap plans equal the
oracle's exactly.
"""
import numpy as np
import pytest
import torch

import fixtures as F
import oracle as O
import quantized_routed_expert_moe_amd as Q
from fixtures import workloads as W
from oracle import residency as OR
from quantized_routed_expert_moe_amd.stack import AdaptiveResidency, ResidentStack
from tests.gpu_util import THREADS, pack_pool, rel_max_err, say, spec_of

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

WL = W.DSV3_STACK
N_BLOBS, N_SHARED = 256, 8
SAMPLE_LAYERS = (0, 29, 57)
NODES_PER_LAYER = 4  # the fused decode layer: route + batches + shared gate/up, routed gate/up + shared down, down, combine


def blob_of(l, e):
    return (e + 37 * l) % N_BLOBS


def shared_of(l):
    return l % N_SHARED


@pytest.fixture(scope="module")
def stack():
    import time
    F.set_num_threads(THREADS)
    t0 = time.time()
    say("generating 256 Q4_K experts and 8 Q8_0 shared experts")
    blobs = W.expert_blobs(WL)  # blob b = expert b of layer 0
    shared = np.stack([F.expert_blob(F.Q8_0, WL.seed, 100 + i, F.TAG_SHARED_EXPERT, WL.H, WL.I_shared)
                       for i in range(N_SHARED)])
    dev_blobs, stride = pack_pool(WL.fmt, blobs, WL.H, WL.I, list(range(N_BLOBS)), N_BLOBS)
    host_blobs = torch.empty(dev_blobs.shape, dtype=torch.uint8).pin_memory()
    host_blobs.copy_(dev_blobs)
    sh_dev, _ = pack_pool(F.Q8_0, shared, WL.H, WL.I_shared, list(range(N_SHARED)), N_SHARED)
    sh_host = sh_dev.cpu().pin_memory()
    ranked = [W.frequency_resident_set(WL, l) for l in range(WL.layers)]
    say(f"  inputs ready in {time.time() - t0:.1f} s; filling {WL.layers} x {WL.resident} slots")
    torch.cuda.synchronize()
    t1 = time.time()
    st = ResidentStack(spec_of(WL), WL.layers, WL.T, WL.resident, WL.staging, ranked, blob_of, host_blobs, dev_blobs,
                       shared_of, sh_host)
    torch.cuda.synchronize()
    say(f"  pools filled in {time.time() - t1:.1f} s; device memory allocated "
        f"{torch.cuda.memory_allocated() / 2**30:.1f} GiB")
    rng = np.random.default_rng(0)
    for _ in range(24):  # every resident slot holds its expert's packed blob
        l, s = int(rng.integers(WL.layers)), int(rng.integers(WL.resident))
        e = int(ranked[l][s])
        assert torch.equal(st.pools[l][s], dev_blobs[blob_of(l, e)]), (l, s)
    del dev_blobs
    torch.cuda.empty_cache()
    say(f"  stack ready in {time.time() - t0:.1f} s")
    xs = [W.x_of(WL, l) for l in range(WL.layers)]
    lgs = [W.logits_of(WL, l) for l in range(WL.layers)]
    st.set_inputs([torch.from_numpy(a) for a in xs], [torch.from_numpy(a) for a in lgs])
    return dict(st=st, blobs=blobs, shared=shared, xs=xs, lgs=lgs)


def _check_replay(ctx, check_layers, lgs=None):
    st = ctx["st"]
    lgs = ctx["lgs"] if lgs is None else lgs
    maps = st.current_maps()
    for l in range(WL.layers):
        ids, w = O.route(lgs[l], WL.k, WL.score, WL.renormalize, WL.scale)
        got_ids = st.layers[l].ids.cpu().numpy()
        assert np.array_equal(got_ids, ids), l
        ob = O.batches(ids, w, WL.E, maps[l], st.S)
        hl = st.host_lists(l)
        assert np.array_equal(hl["token"], ob["host_token"]) and np.array_equal(hl["expert"], ob["host_expert"]), l
        assert np.abs(hl["weight"] - ob["host_weight"]).max(initial=0.0) <= 1e-6 * WL.scale, l
    for l in check_layers:
        needed = set(lgs[l].argsort(axis=1)[:, ::-1][:, :WL.k].ravel().tolist())
        experts = [ctx["blobs"][blob_of(l, e)] if e in needed else None for e in range(WL.E)]
        O.set_threads(THREADS)
        want = O.moe_layer(WL.fmt, experts, WL.H, WL.I, ctx["xs"][l].astype(np.float64), lgs[l], WL.k,
                           WL.score, WL.renormalize, WL.scale, maps[l], ctx["shared"][shared_of(l)], F.Q8_0,
                           WL.I_shared, S=st.S)
        err = rel_max_err(st.layers[l].y.cpu().numpy(), want["y"])
        say(f"  layer {l}: max|y-y*|/max|y*| = {err:.2e}")
        assert err <= 2e-3


def test_stack_graph_replay(stack):
    st = stack["st"]
    say("capture 58 layers")
    st.capture()
    n = st.graph_node_count()
    say(f"  graph nodes: {n}")
    assert n == WL.layers * NODES_PER_LAYER
    st.replay()
    torch.cuda.synchronize()
    _check_replay(stack, SAMPLE_LAYERS)
    y_graph = [y.clone() for y in st.outputs()]
    st.run_eager()
    torch.cuda.synchronize()
    for l, y in enumerate(st.outputs()):
        assert torch.equal(y, y_graph[l]), l
    share = np.mean([float(st.layers[l].slot_offsets[-1].item()) / (WL.T * WL.k) for l in range(WL.layers)])
    say(f"  card-served share of routed pairs: {share:.3f}")


def test_stack_replays_run_during_a_swap_round(stack):
    """The swap copies go on a stream whose work the replays do not queue
    behind: a replay issued after a round's copies ends while they still
    stream (11.5 GB at PCIe rates against a few ms per replay)."""
    st = stack["st"]
    if st.graph is None:
        st.capture()
    say(f"copy stream: {st.side_probes} candidate(s) tried against a replay, overlaps = {st.side_overlaps}")
    assert st.side_overlaps
    st.swap_begin(8)
    st.replay()
    st.replay_done.synchronize()
    still_copying = not st.swap_copies_done.query()
    st.swap_commit(block=True)
    st.replay()
    torch.cuda.synchronize()
    assert still_copying
    _check_replay(stack, (7,))


def test_stack_swap_rounds(stack):
    st = stack["st"]
    if st.graph is None:
        st.capture()
    before = st.current_maps()
    for rnd in range(2):
        say(f"swap round {rnd}")
        st.replay()
        plan = st.swap(8)
        st.replay()
        torch.cuda.synchronize()
        maps = st.current_maps()
        for l in range(WL.layers):
            assert len(plan["incoming"][l]) == 8 and len(plan["outgoing"][l]) == 8
            Q.moe_validate_slot_map(maps[l], st.S)
            assert int((maps[l] >= 0).sum()) == WL.resident
            for e in plan["incoming"][l]:
                assert maps[l][e] >= 0
            for e in plan["outgoing"][l]:
                assert maps[l][e] < 0
        _check_replay(stack, (3, 40))
    changed = sum(int((b >= 0).sum() != 0 and not np.array_equal(b >= 0, a >= 0))
                  for a, b in zip(before, st.current_maps()))
    assert changed == WL.layers


def test_stack_adaptive_residency(stack):
    """Routing drifts to another expert ranking: a prompt's counts stream its
    most-used experts onto the card, then three decode steps run under the
    policy (counters -> scores -> an 8-swap plan per layer per step)."""
    st = stack["st"]
    if st.graph is None:
        st.capture()
    margin, decay = 1 << OR.FRAC_BITS, 4
    pol = AdaptiveResidency(st, decay_shift=decay, margin=margin)
    drift = WL.seed + 5  # another expert ranking than the one the card was filled by
    say("prompt: 64 rows per layer, routed and counted on the device")
    plg = np.stack([F.logits_zipf(drift, l, 64, WL.E, WL.zipf_s, perm_seed=drift) for l in range(WL.layers)])
    pc = st.prompt_counts(plg)
    for l in range(WL.layers):
        oids, _ = O.route(plg[l], WL.k, WL.score, WL.renormalize, WL.scale)
        assert pc[l].tolist() == OR.route_counts(oids, WL.E), l
    before = st.current_maps()
    plans = pol.prompt_plans(pc)
    for l in range(WL.layers):
        (inc, out), _ = OR.prompt_plan(pc[l].tolist(), before[l].tolist())
        assert (list(plans[l][0]), list(plans[l][1])) == (inc, out), l
    n = sum(len(p[0]) for p in plans)
    secs = st.stream_in(plans)
    say(f"  streamed {n} experts in {secs:.2f} s")
    maps = st.current_maps()
    for l in range(WL.layers):
        Q.moe_validate_slot_map(maps[l], st.S)
        for e_in, e_out in zip(*plans[l]):
            assert maps[l][e_in] == before[l][e_out] and maps[l][e_out] == -1
        card = maps[l] >= 0
        assert int(card.sum()) == WL.resident
        assert pc[l][card].min() >= pc[l][~card].max(), l  # the prompt's most-used experts are on the card
    score = [[int(c) << OR.FRAC_BITS for c in pc[l]] for l in range(WL.layers)]
    for step in range(3):
        say(f"decode step {step}")
        lg = np.stack([F.logits_zipf(drift + 100 + step, l, WL.T, WL.E, WL.zipf_s, perm_seed=drift)
                       for l in range(WL.layers)])
        st.set_logits(lg)
        st.replay()
        torch.cuda.synchronize()
        _check_replay(stack, (11,) if step == 2 else (), lgs=lg)
        win = pol.observe()
        maps = st.current_maps()
        for l in range(WL.layers):
            oids, _ = O.route(lg[l], WL.k, WL.score, WL.renormalize, WL.scale)
            assert win[l].tolist() == OR.route_counts(oids, WL.E), l
            score[l] = OR.update_scores(score[l], win[l].tolist(), decay)
            assert pol.score[l].tolist() == score[l], l
        plans = pol.plans(WL.staging)
        for l in range(WL.layers):
            want = OR.plan(score[l], maps[l].tolist(), WL.staging, margin)
            assert (list(plans[l][0]), list(plans[l][1])) == want, l
        say(f"  swaps planned: {sum(len(p[0]) for p in plans)}")
        st.swap_begin(plans=plans)
        st.swap_commit(block=True)
        after = st.current_maps()
        for l in range(WL.layers):
            assert all(after[l][e] >= 0 for e in plans[l][0]) and all(after[l][e] < 0 for e in plans[l][1])
            assert int((after[l] >= 0).sum()) == WL.resident
    st.replay()
    torch.cuda.synchronize()
    _check_replay(stack, (40,), lgs=lg)
