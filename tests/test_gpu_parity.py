"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Integer outputs (expert ids, slot offsets, active slots, the permutation,
the host list) must match bit for bit.  Routing weights: |w - w*| <= 1e-6 *
max(1, scale).  Decode outputs: max |y - y*| <= 2e-3 * max |y*| over the
whole [T, H] output (fp16 activations, fp32 accumulation).
"""
import dataclasses

import numpy as np
import pytest
import torch

import fixtures as F
import oracle as O
from oracle import residency as OR
import quantized_routed_expert_moe_amd as Q
from fixtures import workloads as W
from tests.gpu_util import THREADS, device_layer, pack_pool, rel_max_err, run_device, run_oracle, say

pytestmark = pytest.mark.gpu

DECODE_TOL = 2e-3


def _w_tol(w):
    return 1e-6 * max(1.0, w.scale)


# ------------------------------------------------------------------ route

def _route_device(logits, k, score, renorm, scale):
    T, E = logits.shape
    ld = torch.from_numpy(np.ascontiguousarray(logits)).cuda()
    ids = torch.full((max(T, 1), k), -7, dtype=torch.int32, device="cuda")[:T]
    w = torch.zeros((max(T, 1), k), dtype=torch.float32, device="cuda")[:T]
    Q.moe_route_topk(ld, k, score, renorm, scale, ids, w)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy()


@pytest.mark.parametrize("wl", [W.TINY, W.QWEN3_DECODE_T2, W.QWEN3_PREFILL, W.DSV3_DECODE_T4, W.DSV3_STACK],
                         ids=lambda w: w.name.split(",")[0][:24])
def test_route_matches_oracle(wl):
    say(f"route {wl.name}")
    lg = W.logits_of(wl)
    ids, w = _route_device(lg, wl.k, wl.score, wl.renormalize, wl.scale)
    oids, ow = O.route(lg, wl.k, wl.score, wl.renormalize, wl.scale)
    assert np.array_equal(ids, oids)
    assert np.abs(w - ow).max() <= _w_tol(wl)


@pytest.mark.parametrize("T,E,k,score,renorm,scale", [
    (33, 1000, 64, 0, True, 1.0),
    (5, 1024, 8, 1, True, 2.5),
    (7, 64, 64, 0, True, 1.0),
    (9, 130, 3, 0, False, 1.0),
    (9, 130, 3, 1, False, 0.5),
    (1, 1, 1, 0, True, 1.0),
    (3, 256, 64, 0, True, 1.0),    # two-level rank: every key a candidate
    (4, 200, 33, 1, True, 2.5),    # two-level rank, ragged last group
    (2, 1024, 64, 1, True, 2.5),   # both maxima: MOE_MAX_EXPERTS and MOE_MAX_TOPK
])
def test_route_shapes(T, E, k, score, renorm, scale):
    say(f"route T={T} E={E} k={k} score={score} renorm={renorm}")
    lg = F.logits_normal(3, 0, T, E)
    ids, w = _route_device(lg, k, score, renorm, scale)
    oids, ow = O.route(lg, k, score, renorm, scale)
    assert np.array_equal(ids, oids)
    assert np.abs(w - ow).max() <= 1e-6 * max(1.0, scale)


def test_route_ties_take_lower_id():
    say("route ties")
    lg = np.zeros((4, 200), dtype=np.float32)
    lg[0] = 1.0                      # all equal
    lg[1, ::7] = 2.0                 # equal maxima spread over lanes
    lg[2, [3, 67, 131, 195]] = 5.0   # equal maxima in the same lane slot of different registers
    lg[3] = np.arange(200) % 5       # many tie groups
    for score in (0, 1):
        ids, w = _route_device(lg, 16, score, True, 1.0)
        oids, ow = O.route(lg, 16, score, True, 1.0)
        assert np.array_equal(ids, oids)
        assert np.abs(w - ow).max() <= 1e-6


def test_route_empty():
    say("route T=0")
    ids, w = _route_device(np.zeros((0, 64), dtype=np.float32), 4, 0, True, 1.0)
    assert ids.shape == (0, 4)


# ---------------------------------------------------------------- batches

def _batches_device(ids, w, E, soe, S):
    T, k = ids.shape
    P = T * k
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    i32 = dict(dtype=torch.int32, device="cuda")
    out = dict(slot_offsets=torch.full((S + 1,), -5, **i32), active_slots=torch.full((max(1, min(S, P)),), -5, **i32),
               num_active=torch.full((1,), -5, **i32), perm_pair=torch.full((max(1, P),), -5, **i32),
               host_token=torch.full((max(1, P),), -5, **i32), host_expert=torch.full((max(1, P),), -5, **i32),
               host_weight=torch.full((max(1, P),), -5.0, dtype=torch.float32, device="cuda"),
               host_count=torch.full((1,), -5, **i32))
    wsb = Q.moe_batches_workspace_size(T, k, E, S)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda") if wsb else None
    Q.moe_build_expert_batches(dev(ids.astype(np.int32)), dev(w.astype(np.float32)), E, dev(soe), S,
                               out["slot_offsets"], out["active_slots"], out["num_active"], out["perm_pair"],
                               out["host_token"], out["host_expert"], out["host_weight"], out["host_count"], ws)
    torch.cuda.synchronize()
    o = {key: v.cpu().numpy() for key, v in out.items()}
    na, nres, hc = int(o["num_active"][0]), int(o["slot_offsets"][S]), int(o["host_count"][0])
    o["active_slots"] = o["active_slots"][:na]
    o["perm_pair"] = o["perm_pair"][:nres]
    for key in ("host_token", "host_expert", "host_weight"):
        o[key] = o[key][:hc]
    return o


def _slot_maps(E, rng):
    perm = rng.permutation(E).astype(np.int32)
    half = np.full(E, -1, dtype=np.int32)
    chosen = rng.permutation(E)[:E // 2]
    half[chosen] = rng.permutation(E // 2)
    return {"identity": (np.arange(E, dtype=np.int32), E), "shuffled": (perm, E), "half": (half, E // 2 + 3),
            "none": (np.full(E, -1, dtype=np.int32), 0)}


@pytest.mark.parametrize("wl", [W.TINY, W.QWEN3_DECODE_T1, W.QWEN3_PREFILL, W.DSV3_DECODE_T4],
                         ids=lambda w: w.name.split(",")[0][:24])
@pytest.mark.parametrize("smap", ["identity", "shuffled", "half", "none"])
def test_batches_match_oracle(wl, smap):
    say(f"batches {wl.name} map={smap}")
    lg = W.logits_of(wl)
    ids, w = O.route(lg, wl.k, wl.score, wl.renormalize, wl.scale)
    soe, S = _slot_maps(wl.E, np.random.default_rng(wl.E + len(smap)))[smap]
    got = _batches_device(ids, w, wl.E, soe, S)
    want = O.batches(ids, w, wl.E, soe, S)
    for key in ("slot_offsets", "active_slots", "perm_pair", "host_token", "host_expert"):
        assert np.array_equal(got[key], want[key]), key
    assert int(got["num_active"][0]) == int(want["num_active"][0])
    assert int(got["host_count"][0]) == int(want["host_count"][0])
    assert np.array_equal(got["host_weight"], w.astype(np.float32).ravel()[
        [t * wl.k + j for t in range(wl.T) for j in range(wl.k)
         if not (0 <= soe[ids[t, j]] < S)]])


# ------------------------------------------------------- route and batch

def _route_batch_device(logits, k, score, renorm, scale, soe, S, route_counts=None):
    T, E = logits.shape
    P = T * k
    i32 = dict(dtype=torch.int32, device="cuda")
    ids = torch.full((max(T, 1), k), -7, **i32)[:T]
    w = torch.zeros((max(T, 1), k), dtype=torch.float32, device="cuda")[:T]
    out = dict(slot_offsets=torch.full((S + 1,), -5, **i32), active_slots=torch.full((max(1, min(S, P)),), -5, **i32),
               num_active=torch.full((1,), -5, **i32), perm_pair=torch.full((max(1, P),), -5, **i32),
               host_token=torch.full((max(1, P),), -5, **i32), host_expert=torch.full((max(1, P),), -5, **i32),
               host_weight=torch.full((max(1, P),), -5.0, dtype=torch.float32, device="cuda"),
               host_count=torch.full((1,), -5, **i32))
    wsb = Q.moe_batches_workspace_size(T, k, E, S)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda") if wsb else None
    Q.moe_route_and_batch(torch.from_numpy(np.ascontiguousarray(logits)).cuda(), k, score, renorm, scale, ids, w, E,
                          torch.from_numpy(soe).cuda(), S, out["slot_offsets"], out["active_slots"],
                          out["num_active"], out["perm_pair"], out["host_token"], out["host_expert"],
                          out["host_weight"], out["host_count"], ws, route_counts=route_counts)
    torch.cuda.synchronize()
    o = {key: v.cpu().numpy() for key, v in out.items()}
    na, nres, hc = int(o["num_active"][0]), int(o["slot_offsets"][S]), int(o["host_count"][0])
    o["active_slots"] = o["active_slots"][:na]
    o["perm_pair"] = o["perm_pair"][:nres]
    for key in ("host_token", "host_expert", "host_weight"):
        o[key] = o[key][:hc]
    o["ids"], o["w"] = ids.cpu().numpy(), w.cpu().numpy()
    return o


@pytest.mark.parametrize("T,E,k,score,renorm,scale", [
    (1, 128, 8, 0, True, 1.0),     # fused: Qwen3 decode shape
    (2, 128, 8, 0, True, 1.0),
    (4, 256, 8, 1, True, 2.5),     # fused: DeepSeek-V3 decode shape
    (4, 8, 2, 0, True, 1.0),       # fused: tiny
    (4, 256, 16, 0, False, 1.0),   # fused: 64 pairs, full softmax denominator
    (3, 100, 5, 1, False, 0.5),    # fused: E not a power of two
    (5, 128, 8, 0, True, 1.0),     # two launches: T > 4
    (2, 64, 40, 0, True, 1.0),     # two launches: 80 pairs
    (3, 300, 8, 1, True, 2.5),     # two launches: E > 256
])
@pytest.mark.parametrize("smap", ["identity", "half", "none"])
def test_route_and_batch_matches_oracle_and_two_calls(T, E, k, score, renorm, scale, smap):
    say(f"route and batch T={T} E={E} k={k} score={score} renorm={renorm} map={smap}")
    lg = F.logits_normal(11, T, T, E)
    soe, S = _slot_maps(E, np.random.default_rng(E + T + len(smap)))[smap]
    got = _route_batch_device(lg, k, score, renorm, scale, soe, S)
    oids, ow = O.route(lg, k, score, renorm, scale)
    assert np.array_equal(got["ids"], oids)
    assert np.abs(got["w"] - ow).max() <= 1e-6 * max(1.0, scale)
    want = O.batches(oids, ow, E, soe, S)
    for key in ("slot_offsets", "active_slots", "perm_pair", "host_token", "host_expert"):
        assert np.array_equal(got[key], want[key]), key
    assert int(got["num_active"][0]) == int(want["num_active"][0])
    assert int(got["host_count"][0]) == int(want["host_count"][0])
    # the same bits as the two separate calls
    ids2, w2 = _route_device(lg, k, score, renorm, scale)
    assert np.array_equal(got["ids"], ids2) and np.array_equal(got["w"].view(np.uint32), w2.view(np.uint32))
    two = _batches_device(ids2, w2, E, soe, S)
    for key in ("slot_offsets", "active_slots", "perm_pair", "host_token", "host_expert", "host_weight"):
        assert np.array_equal(got[key], two[key]), key


@pytest.mark.parametrize("T,E,k,score", [
    (2, 128, 8, 0),    # fused launch
    (4, 256, 8, 1),    # fused launch, two-level rank
    (5, 128, 8, 0),    # two launches: T > 4
    (3, 300, 8, 1),    # two launches: E > 256
])
def test_route_and_batch_counts_routing(T, E, k, score):
    """The routing counters: two calls add twice the oracle's per-expert pair
    counts to whatever the counters held (uint32, wrapping)."""
    say(f"route and batch counters T={T} E={E} k={k}")
    lg = F.logits_normal(31, T, T, E)
    soe, S = _slot_maps(E, np.random.default_rng(E))["half"]
    start = np.random.default_rng(T).integers(0, 1 << 32, size=E, dtype=np.uint64).astype(np.uint32)
    start[:3] = 0xFFFFFFFF  # wraps if routed to
    counts = torch.from_numpy(start.view(np.int32).copy()).cuda()
    for _ in range(2):
        _route_batch_device(lg, k, score, True, 2.5 if score else 1.0, soe, S, route_counts=counts)
    oids, _ = O.route(lg, k, score, True, 2.5 if score else 1.0)
    want = (start.astype(np.uint64) + 2 * np.array(OR.route_counts(oids, E), dtype=np.uint64)) % (1 << 32)
    assert np.array_equal(counts.cpu().numpy().view(np.uint32), want.astype(np.uint32))


@pytest.mark.parametrize("T,E,k", [(4096, 128, 8), (700, 1000, 6), (1, 8, 2)])
def test_count_routes_matches_oracle(T, E, k):
    say(f"count routes T={T} E={E} k={k}")
    lg = F.logits_normal(41, T, T, E)
    oids, _ = O.route(lg, k, 0, True, 1.0)
    ids = oids.copy()
    ids[0, 0] = -1      # ids outside [0, E) are skipped
    ids[-1, -1] = E
    counts = torch.zeros(E, dtype=torch.int32, device="cuda")
    Q.moe_count_routes(torch.from_numpy(ids).cuda(), E, counts)
    torch.cuda.synchronize()
    assert counts.cpu().numpy().tolist() == OR.route_counts(ids, E)


def test_route_and_batch_ties():
    """The rank order (logit desc, id asc) with many equal logits, through the
    single-launch path (4 rows, 64 pairs)."""
    say("route and batch ties")
    lg = np.zeros((4, 200), dtype=np.float32)
    lg[0] = 1.0
    lg[1, ::7] = 2.0
    lg[2, [3, 67, 131, 195]] = 5.0
    lg[3] = np.arange(200) % 5
    soe, S = _slot_maps(200, np.random.default_rng(5))["half"]
    got = _route_batch_device(lg, 16, 0, True, 1.0, soe, S)
    oids, ow = O.route(lg, 16, 0, True, 1.0)
    assert np.array_equal(got["ids"], oids)
    want = O.batches(oids, ow, 200, soe, S)
    for key in ("slot_offsets", "active_slots", "perm_pair", "host_token", "host_expert"):
        assert np.array_equal(got[key], want[key]), key


@pytest.mark.parametrize("T", [8192, 9000])
def test_batches_block_counts_around_the_fused_scan_limit(T):
    """64 blocks of 1024 pairs (the scan folded into the scatter) and 71
    blocks (the separate scan launch)."""
    E, k = 128, 8
    say(f"batches T={T} k={k} ({T * k} pairs)")
    lg = F.logits_normal(21, 0, T, E)
    ids, w = O.route(lg, k, 0, True, 1.0)
    soe, S = _slot_maps(E, np.random.default_rng(T))["half"]
    got = _batches_device(ids, w, E, soe, S)
    want = O.batches(ids, w, E, soe, S)
    for key in ("slot_offsets", "active_slots", "perm_pair", "host_token", "host_expert"):
        assert np.array_equal(got[key], want[key]), key
    assert int(got["host_count"][0]) == int(want["host_count"][0])


def test_batches_stack_residency():
    wl = W.DSV3_STACK
    for layer in (0, 29, 57):
        say(f"batches stack layer {layer}")
        soe, S = W.slot_map(wl, layer)
        lg = W.logits_of(wl, layer)
        ids, w = O.route(lg, wl.k, wl.score, wl.renormalize, wl.scale)
        got = _batches_device(ids, w, wl.E, soe, S)
        want = O.batches(ids, w, wl.E, soe, S)
        for key in ("slot_offsets", "active_slots", "perm_pair", "host_token", "host_expert"):
            assert np.array_equal(got[key], want[key]), key


def test_batches_workspace_required_for_large_batches():
    assert Q.moe_batches_workspace_size(64, 8, 128, 128) == 0
    assert Q.moe_batches_workspace_size(4096, 8, 128, 128) > 0


def test_batches_empty():
    say("batches T=0")
    got = _batches_device(np.zeros((0, 4), np.int32), np.zeros((0, 4), np.float32), 16, np.arange(16, dtype=np.int32),
                          16)
    assert got["slot_offsets"].tolist() == [0] * 17 and int(got["num_active"][0]) == 0
    assert int(got["host_count"][0]) == 0


# ------------------------------------------------------------ decode layer

def _layer_case(wl, blobs=None, soe=None, S=None, T=None, path=Q.MOE_PATH_AUTO, x=None, logits=None,
                host_list_pinned=False):
    soe_, S_ = W.slot_map(wl)
    soe = soe_ if soe is None else soe
    S = S_ if S is None else S
    x = W.x_of(wl) if x is None else x
    logits = W.logits_of(wl) if logits is None else logits
    T = x.shape[0]
    if blobs is None:
        blobs = W.expert_blobs(wl)
    shared = W.shared_blob(wl)
    layer = device_layer(wl, blobs, soe, S, shared, T, path, host_list_pinned=host_list_pinned)
    got = run_device(layer, x, logits)
    want = run_oracle(wl, blobs, x, logits, soe, shared, want_pairs=True, S=S)
    return got, want, soe, S


def _check_layer(wl, got, want, soe, S, tol=DECODE_TOL):
    assert np.array_equal(got["ids"], want["ids"])
    assert np.abs(got["w"] - want["w"]).max() <= _w_tol(wl)
    ob = O.batches(want["ids"], want["w"], wl.E, soe, S)
    for key in ("slot_offsets", "active_slots", "perm_pair", "host_token", "host_expert"):
        assert np.array_equal(got[key], ob[key]), key
    assert np.abs(got["host_weight"] - ob["host_weight"]).max(initial=0.0) <= _w_tol(wl)
    err = rel_max_err(got["y"], want["y"])
    say(f"  max|y-y*|/max|y*| = {err:.3e}")
    assert err <= tol


MXFP4_SMALL = W.Workload("small MXFP4 layer (H256 E8 k2 I256 T4)", F.MXFP4, 256, 256, 8, 2, 4)
Q3K_SMALL = W.Workload("small Q3_K/Q4_K layer (H512 E8 k2 I256 T4)", F.Q3K_Q4K, 512, 256, 8, 2, 4)
Q5K_SMALL = W.Workload("small Q5_K layer (H512 E8 k2 I256 T4)", F.Q5K, 512, 256, 8, 2, 4)
Q5K_QWEN3_T2 = W.Workload("Qwen3-30B-A3B-shaped MoE layer, Q5_K experts, decode T=2", F.Q5K, 2048, 768, 128, 8, 2)
Q6K_SMALL = W.Workload("small Q6_K layer (H512 E8 k2 I256 T4)", F.Q6K, 512, 256, 8, 2, 4)
Q3K_QWEN3_T2 = W.Workload("Qwen3-30B-A3B-shaped MoE layer, Q3_K/Q4_K experts, decode T=2", F.Q3K_Q4K, 2048, 768, 128,
                          8, 2)


@pytest.mark.parametrize("wl", [W.TINY, W.QWEN3_DECODE_T1, W.QWEN3_DECODE_T2, MXFP4_SMALL, W.QWEN3_MXFP4_DECODE_T2,
                                Q3K_SMALL, Q3K_QWEN3_T2, Q5K_SMALL, Q5K_QWEN3_T2, Q6K_SMALL,
                                W.QWEN3_Q6K_DECODE_T2],
                         ids=lambda w: w.name.split(",")[0][:24] + f"-fmt{w.fmt}-T{w.T}")
def test_decode_layer_matches_oracle(wl):
    say(f"decode layer {wl.name}")
    got, want, soe, S = _layer_case(wl)
    _check_layer(wl, got, want, soe, S)
    # every resident pair's own output, too
    res = [p for p in range(wl.T * wl.k) if 0 <= soe[want["ids"].ravel()[p]] < S]
    assert rel_max_err(got["y_pairs"][res], want["y_pairs"][res]) <= DECODE_TOL


@pytest.fixture(scope="module")
def dsv3_blobs():
    say("generating 256 DeepSeek-V3-shaped Q4_K experts")
    F.set_num_threads(THREADS)
    return W.expert_blobs(W.DSV3_DECODE_T2)


@pytest.mark.parametrize("wl", [W.DSV3_DECODE_T2, W.DSV3_DECODE_T4], ids=["T2", "T4"])
def test_dsv3_decode_layer_matches_oracle(wl, dsv3_blobs):
    say(f"decode layer {wl.name}")
    got, want, soe, S = _layer_case(wl, blobs=dsv3_blobs)
    _check_layer(wl, got, want, soe, S)


def test_dsv3_partial_residency(dsv3_blobs):
    """Stack layer 0's 96-of-256 residency on the DeepSeek-V3-shaped layer:
    non-resident pairs add nothing on the card and form the host list."""
    wl = W.DSV3_STACK
    soe, S = W.slot_map(wl, 0)
    base = W.DSV3_DECODE_T2
    say("decode layer with 96 resident experts")
    logits = W.logits_of(wl, 0)
    got, want, soe, S = _layer_case(base, blobs=dsv3_blobs, soe=soe, S=S, logits=logits)
    _check_layer(base, got, want, soe, S)
    assert got["host_count"] > 0 and got["num_active"] > 0
    # the host leg on the card's host list completes the layer: card + host = every expert served
    x = W.x_of(base)
    y_host = Q.moe_host_leg(base.fmt, list(dsv3_blobs), base.H, base.I, x, got["host_token"], got["host_expert"],
                            got["host_weight"], threads=THREADS)
    full = run_oracle(base, dsv3_blobs, x, logits, np.arange(base.E, dtype=np.int32), W.shared_blob(base))
    err = rel_max_err(got["y"] + y_host, full["y"])
    say(f"  card + host leg vs all experts served: {err:.2e}")
    assert err <= DECODE_TOL


def test_dsv3_disjoint_halves_add_up(dsv3_blobs):
    """The single-GPU stand-in for an expert-parallel split: the DeepSeek-V3-
    shaped layer at T = 2 with the even experts resident (map A, shared
    expert included) and with the odd ones (map B, no shared expert) adds up
    to the layer with every expert resident, y(A) + y(B) = y(A u B), and each
    half matches the oracle at its own map.  One slot pool (slot = expert id)
    serves the three maps."""
    wl = W.DSV3_DECODE_T2
    wl_b = dataclasses.replace(wl, I_shared=0)
    x, logits = W.x_of(wl), W.logits_of(wl)
    pool = pack_pool(wl.fmt, dsv3_blobs, wl.H, wl.I, list(range(wl.E)), wl.E)
    ids = np.arange(wl.E, dtype=np.int32)
    soe_a = np.where(ids % 2 == 0, ids, -1).astype(np.int32)
    soe_b = np.where(ids % 2 == 1, ids, -1).astype(np.int32)
    shared = W.shared_blob(wl)
    out = {}
    for name, w_, soe, sh in (("all", wl, ids, shared), ("A", wl, soe_a, shared), ("B", wl_b, soe_b, None)):
        say(f"  map {name}")
        layer = device_layer(w_, dsv3_blobs, soe, wl.E, sh, wl.T, Q.MOE_PATH_DECODE, pool=pool)
        out[name] = run_device(layer, x, logits)
        del layer
    torch.cuda.empty_cache()
    sel = out["all"]["ids"].ravel()
    assert (sel % 2 == 0).any() and (sel % 2 == 1).any(), "both halves must hold selected experts"
    err = rel_max_err(out["A"]["y"] + out["B"]["y"], out["all"]["y"])
    say(f"  y(A) + y(B) vs y(A u B): {err:.2e}")
    assert err <= DECODE_TOL
    for name, w_, soe, sh in (("A", wl, soe_a, shared), ("B", wl_b, soe_b, None)):
        want = run_oracle(w_, dsv3_blobs, x, logits, soe, sh, S=wl.E)
        _check_layer(w_, out[name], want, soe, wl.E)


def test_slot_values_beyond_s_go_to_the_host():
    """A slot-map value of S or more is not a slot: the pair goes to the host
    list and adds nothing on the card, in the batching and the combine alike
    (the oracle's rule 0 <= slot < S).  Qwen3-shaped layer at T = 2 with 64
    slots: experts 0..63 in slots 0..63, experts 64..127 mapped to their own
    id (>= S), so about half the routed pairs carry such values."""
    wl = W.QWEN3_DECODE_T2
    S = 64
    soe = np.arange(wl.E, dtype=np.int32)
    say(wl.name + ", 64 slots, slot values up to 127")
    blobs = W.expert_blobs(wl)
    pool = pack_pool(wl.fmt, blobs, wl.H, wl.I, list(range(S)), S)
    x, logits = W.x_of(wl), W.logits_of(wl)
    layer = device_layer(wl, blobs, soe, S, None, wl.T, Q.MOE_PATH_DECODE, pool=pool)
    got = run_device(layer, x, logits)
    want = run_oracle(wl, blobs, x, logits, soe, None, S=S)
    assert (got["ids"] >= S).any() and (got["ids"] < S).any()
    _check_layer(wl, got, want, soe, S)
    assert sorted(got["host_expert"].tolist()) == sorted(e for e in got["ids"].ravel().tolist() if e >= S)
    # the same layer with those experts marked -1 gives the same outputs, bit for bit
    soe_m = np.where(soe < S, soe, -1).astype(np.int32)
    layer_m = device_layer(wl, blobs, soe_m, S, None, wl.T, Q.MOE_PATH_DECODE, pool=pool)
    got_m = run_device(layer_m, x, logits)
    assert np.array_equal(got_m["y"], got["y"])


def test_dsv3_experts_many_tokens_per_slot(dsv3_blobs):
    """DeepSeek-V3-sized experts (H 7168, I 2048) with 24 tokens over 16
    experts on the decode path: the K split gives each wave several units
    (the prefetching loop, with odd and even unit counts) and slots hold
    several chunks of tokens (the loop's refill with the first unit)."""
    wl = W.Workload("DeepSeek-V3-sized Q4_K experts, 16 resident, 24 tokens", F.Q4K, 7168, 2048, 16, 2, 24)
    say(wl.name)
    got, want, soe, S = _layer_case(wl, blobs=dsv3_blobs[:16], path=Q.MOE_PATH_DECODE)
    _check_layer(wl, got, want, soe, S)
    assert int(np.diff(got["slot_offsets"]).max()) > 2


@pytest.mark.parametrize("fmt", [F.Q4K, F.Q8_0, F.MXFP4, F.Q3K_Q4K, F.Q5K, F.Q6K])
def test_decode_k_split_across_workgroups(fmt):
    """Two experts with a long K (H 7168): too few row tiles to fill the chip,
    so K is split across workgroups too (partial sums finished by the reduce
    kernel), with an uneven last part and a slot holding several chunks of
    tokens."""
    name = {F.Q4K: "Q4_K", F.Q8_0: "Q8_0", F.MXFP4: "MXFP4", F.Q3K_Q4K: "Q3_K/Q4_K", F.Q5K: "Q5_K",
            F.Q6K: "Q6_K"}[fmt]
    wl = W.Workload(f"{name} layer H 7168, 2 experts, k 1, T 5", fmt, 7168, 256, 2, 1, 5)
    say(wl.name)
    got, want, soe, S = _layer_case(wl, path=Q.MOE_PATH_DECODE)
    _check_layer(wl, got, want, soe, S)


def test_decode_many_tokens_per_slot():
    """48 tokens over 8 experts on the decode path: slots hold up to dozens of
    tokens (chunks of two plus a remainder)."""
    wl = W.Workload("small Q4_K layer, 48 tokens", F.Q4K, 512, 256, 8, 3, 48)
    say(wl.name)
    got, want, soe, S = _layer_case(wl, path=Q.MOE_PATH_DECODE)
    _check_layer(wl, got, want, soe, S)


def test_decode_q8_0_many_tokens():
    wl = W.Workload("small Q8_0 layer, 37 tokens, partial residency", F.Q8_0, 384, 256, 12, 4, 37)
    say(wl.name)
    soe = np.array([3, -1, 0, 5, -1, 1, 2, -1, 4, 6, -1, 7], dtype=np.int32)
    got, want, soe, S = _layer_case(wl, soe=soe, S=9)
    _check_layer(wl, got, want, soe, S)


def test_decode_mxfp4_many_tokens_partial_residency():
    """MXFP4 experts, 37 tokens over 12 experts, 8 of them resident: chunks of
    two tokens per slot plus remainders, and a host list."""
    wl = W.Workload("small MXFP4 layer, 37 tokens, partial residency", F.MXFP4, 512, 256, 12, 4, 37)
    say(wl.name)
    soe = np.array([3, -1, 0, 5, -1, 1, 2, -1, 4, 6, -1, 7], dtype=np.int32)
    got, want, soe, S = _layer_case(wl, soe=soe, S=9, path=Q.MOE_PATH_DECODE)
    _check_layer(wl, got, want, soe, S)
    assert got["host_count"] > 0


def test_dsv3_sized_mxfp4_experts_many_tokens():
    """DeepSeek-V3-sized MXFP4 experts (H 7168, I 2048), 16 of them, 24
    tokens: several K units per wave (the prefetching loop) and several
    chunks of tokens per slot."""
    wl = W.Workload("DeepSeek-V3-sized MXFP4 experts, 16 resident, 24 tokens", F.MXFP4, 7168, 2048, 16, 2, 24)
    say(wl.name)
    F.set_num_threads(THREADS)
    got, want, soe, S = _layer_case(wl, path=Q.MOE_PATH_DECODE)
    _check_layer(wl, got, want, soe, S)
    assert int(np.diff(got["slot_offsets"]).max()) > 2


def test_decode_q3k_many_tokens_partial_residency():
    """Q3_K gate/up + Q4_K down experts, 37 tokens over 12 experts, 8 of them
    resident: chunks of two tokens per slot plus remainders, and a host list
    that the host leg completes."""
    wl = W.Workload("small Q3_K/Q4_K layer, 37 tokens, partial residency", F.Q3K_Q4K, 512, 256, 12, 4, 37)
    say(wl.name)
    soe = np.array([3, -1, 0, 5, -1, 1, 2, -1, 4, 6, -1, 7], dtype=np.int32)
    blobs = W.expert_blobs(wl)
    got, want, soe, S = _layer_case(wl, blobs=blobs, soe=soe, S=9, path=Q.MOE_PATH_DECODE)
    _check_layer(wl, got, want, soe, S)
    assert got["host_count"] > 0
    x, logits = W.x_of(wl), W.logits_of(wl)
    y_host = Q.moe_host_leg(wl.fmt, list(blobs), wl.H, wl.I, x, got["host_token"], got["host_expert"],
                            got["host_weight"], threads=THREADS)
    full = run_oracle(wl, blobs, x, logits, np.arange(wl.E, dtype=np.int32), None)
    assert rel_max_err(got["y"] + y_host, full["y"]) <= DECODE_TOL


def test_dsv3_sized_q3k_experts_many_tokens():
    """DeepSeek-V3-sized experts of the engine's V4.1 files (Q3_K gate/up,
    Q4_K down; H 7168, I 2048), 16 of them, 24 tokens: several K units per
    wave in both GEMVs and several chunks of tokens per slot."""
    wl = W.Workload("DeepSeek-V3-sized Q3_K/Q4_K experts, 16 resident, 24 tokens", F.Q3K_Q4K, 7168, 2048, 16, 2, 24)
    say(wl.name)
    F.set_num_threads(THREADS)
    got, want, soe, S = _layer_case(wl, path=Q.MOE_PATH_DECODE)
    _check_layer(wl, got, want, soe, S)
    assert int(np.diff(got["slot_offsets"]).max()) > 2


@pytest.mark.parametrize("T", [8, 24], ids=["K-split", "pipelined"])
def test_dsv3_sized_q5k_experts(T):
    """DeepSeek-V3-sized Q5_K experts (H 7168, I 2048), 16 of them: at 16
    pairs the gate/up GEMV splits K across workgroups (its pipelined kernel
    would spill); at 48 pairs the partial sums would not fit and the
    pipelined kernel runs.  The down GEMV pipelines in both."""
    wl = W.Workload(f"DeepSeek-V3-sized Q5_K experts, 16 resident, {T} tokens", F.Q5K, 7168, 2048, 16, 2, T)
    say(wl.name)
    F.set_num_threads(THREADS)
    got, want, soe, S = _layer_case(wl, path=Q.MOE_PATH_DECODE)
    _check_layer(wl, got, want, soe, S)


def test_decode_q5k_many_tokens_partial_residency():
    wl = W.Workload("small Q5_K layer, 37 tokens, partial residency", F.Q5K, 512, 256, 12, 4, 37)
    say(wl.name)
    soe = np.array([3, -1, 0, 5, -1, 1, 2, -1, 4, 6, -1, 7], dtype=np.int32)
    got, want, soe, S = _layer_case(wl, soe=soe, S=9, path=Q.MOE_PATH_DECODE)
    _check_layer(wl, got, want, soe, S)
    assert got["host_count"] > 0


@pytest.mark.parametrize("T", [8, 24], ids=["K-split", "pipelined"])
def test_dsv3_sized_q6k_experts(T):
    """DeepSeek-V3-sized Q6_K experts (H 7168, I 2048), 16 of them: the
    gate/up GEMV splits K across workgroups at 16 pairs and runs its
    pipelined kernel at 48; the down GEMV (per-half constants in the h
    records) pipelines in both."""
    wl = W.Workload(f"DeepSeek-V3-sized Q6_K experts, 16 resident, {T} tokens", F.Q6K, 7168, 2048, 16, 2, T)
    say(wl.name)
    F.set_num_threads(THREADS)
    got, want, soe, S = _layer_case(wl, path=Q.MOE_PATH_DECODE)
    _check_layer(wl, got, want, soe, S)


def test_decode_q6k_many_tokens_partial_residency():
    """Q6_K, 37 tokens over 12 experts, 8 resident: chunks of two tokens per
    slot plus remainders; the host leg completes the layer."""
    wl = W.Workload("small Q6_K layer, 37 tokens, partial residency", F.Q6K, 512, 256, 12, 4, 37)
    say(wl.name)
    soe = np.array([3, -1, 0, 5, -1, 1, 2, -1, 4, 6, -1, 7], dtype=np.int32)
    blobs = W.expert_blobs(wl)
    got, want, soe, S = _layer_case(wl, blobs=blobs, soe=soe, S=9, path=Q.MOE_PATH_DECODE)
    _check_layer(wl, got, want, soe, S)
    assert got["host_count"] > 0
    x, logits = W.x_of(wl), W.logits_of(wl)
    y_host = Q.moe_host_leg(wl.fmt, list(blobs), wl.H, wl.I, x, got["host_token"], got["host_expert"],
                            got["host_weight"], threads=THREADS)
    full = run_oracle(wl, blobs, x, logits, np.arange(wl.E, dtype=np.int32), None)
    assert rel_max_err(got["y"] + y_host, full["y"]) <= DECODE_TOL


@pytest.mark.parametrize("fmt", [F.Q4K, F.Q6K])
def test_decode_layer_every_expert_per_token(fmt):
    """k = E = 64 (MOE_MAX_TOPK): every token goes to every expert, 3 tokens,
    so every slot holds three pairs (one chunk of two tokens and a remainder)
    and the combine sums 64 terms per token; 40 of the 64 experts resident."""
    wl = W.Workload("small layer, k = E = 64, T 3", fmt, 256 if fmt == F.Q4K else 512, 256, 64, 64, 3)
    say(wl.name)
    soe = np.full(64, -1, dtype=np.int32)
    soe[np.random.default_rng(2).permutation(64)[:40]] = np.arange(40, dtype=np.int32)
    got, want, soe, S = _layer_case(wl, soe=soe, S=40, path=Q.MOE_PATH_DECODE)
    _check_layer(wl, got, want, soe, S)
    assert got["host_count"] == 3 * 24


def test_host_list_written_into_pinned_memory():
    """The batching kernel stores the host list straight into pinned host
    memory (its device address); nothing is copied."""
    wl = W.Workload("small Q8_0 layer, 37 tokens, partial residency", F.Q8_0, 384, 256, 12, 4, 37)
    say(wl.name + ", host list in pinned memory")
    soe = np.array([3, -1, 0, 5, -1, 1, 2, -1, 4, 6, -1, 7], dtype=np.int32)
    got, want, soe, S = _layer_case(wl, soe=soe, S=9, host_list_pinned=True)
    _check_layer(wl, got, want, soe, S)
    assert got["host_count"] > 0


def test_decode_zero_input_gives_zero():
    wl = W.QWEN3_DECODE_T2
    say("decode x = 0")
    x = np.zeros((wl.T, wl.H), dtype=np.float32)
    got, want, soe, S = _layer_case(wl, x=x)
    assert np.all(got["y"] == 0.0)


# ---------------------------------------------------- determinism and graphs

def test_eager_runs_bitwise_equal_and_graph_replay_equals_eager():
    wl = W.QWEN3_DECODE_T2
    say("determinism and graph replay")
    blobs = W.expert_blobs(wl)
    soe, S = W.slot_map(wl)
    layer = device_layer(wl, blobs, soe, S, None, wl.T)
    xs = [torch.from_numpy(W.x_of(wl, seed=s)).cuda() for s in range(3)]
    ls = [torch.from_numpy(W.logits_of(wl, seed=s)).cuda() for s in range(3)]
    eager = []
    for i in range(3):
        eager.append(layer.forward(xs[i], ls[i]).clone())
    again = layer.forward(xs[0], ls[0]).clone()
    torch.cuda.synchronize()
    assert torch.equal(eager[0], again)
    # capture one forward on static inputs, replay with new contents
    x_static, l_static = xs[0].clone(), ls[0].clone()
    layer.forward(x_static, l_static)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        y_graph = layer.forward(x_static, l_static)
    for rep in range(3):
        for i in (2, 0, 1):
            x_static.copy_(xs[i])
            l_static.copy_(ls[i])
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(y_graph, eager[i]), (rep, i)
            torch.cuda.synchronize()
