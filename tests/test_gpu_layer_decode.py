"""The fused decode layer (moe_layer_decode: routing, batching, routed and
shared expert FFN and combine in four launches on one stream) against the
CPU oracle, and against the separate calls it replaces.

Integer outputs (ids, slot offsets, active slots, permutation, host list)
bit for bit; routing weights |w - w*| <= 1e-6 * max(1, scale); y and the
resident pairs' y_pairs within max |y - y*| <= 2e-3 * max |y*|.  Without a
shared expert the layer runs the separate calls' kernels, so the routed
pairs' y_pairs and y are bit for bit theirs.  With one, the layer's gate/up
launch (Q4_K: over half tiles, four waves splitting K) may split K at other
points than the separate call, so the fp32 sums round differently and an h
value can land on the neighbouring fp16: y_pairs and y agree with the
separate calls within SPLIT_TOL of their largest value."""
import dataclasses

import numpy as np
import pytest
import torch

import fixtures as F
import oracle as O
import quantized_routed_expert_moe_amd as Q
from fixtures import workloads as W
from tests.gpu_util import THREADS, device_layer, pack_pool, rel_max_err, run_device, run_oracle, say

pytestmark = pytest.mark.gpu

DECODE_TOL = 2e-3
# fused vs separate calls with a shared expert: a few h values one fp16 step
# apart (relative 2^-11) through one down row each, far below DECODE_TOL
SPLIT_TOL = 1e-4


def _w_tol(wl):
    return 1e-6 * max(1.0, wl.scale)


def _case(wl, soe=None, S=None, blobs=None, pool=None, logits=None):
    soe_, S_ = W.slot_map(wl)
    soe = soe_ if soe is None else soe
    S = S_ if S is None else S
    blobs = W.expert_blobs(wl) if blobs is None else blobs
    shared = W.shared_blob(wl)
    x = W.x_of(wl)
    logits = W.logits_of(wl) if logits is None else logits
    if pool is None:
        slots = [None] * S
        for e in range(wl.E):
            if 0 <= soe[e] < S:
                slots[int(soe[e])] = e
        pool = pack_pool(wl.fmt, blobs, wl.H, wl.I, slots, S)
    fused = device_layer(wl, blobs, soe, S, shared, wl.T, Q.MOE_PATH_DECODE, pool=pool)
    assert fused.fused
    got = run_device(fused, x, logits)
    sep = device_layer(wl, blobs, soe, S, shared, wl.T, Q.MOE_PATH_AUTO, pool=pool)
    assert not sep.fused
    two = run_device(sep, x, logits)
    want = run_oracle(wl, blobs, x, logits, soe, shared, want_pairs=True, S=S)
    return got, two, want, soe, S


def _check(wl, got, two, want, soe, S):
    assert np.array_equal(got["ids"], want["ids"])
    assert np.abs(got["w"] - want["w"]).max() <= _w_tol(wl)
    assert np.array_equal(got["w"], two["w"])
    ob = O.batches(want["ids"], want["w"], wl.E, soe, S)
    for key in ("slot_offsets", "active_slots", "perm_pair", "host_token", "host_expert"):
        assert np.array_equal(got[key], ob[key]), key
    assert np.abs(got["host_weight"] - ob["host_weight"]).max(initial=0.0) <= _w_tol(wl)
    res = [p for p in range(wl.T * wl.k) if 0 <= soe[want["ids"].ravel()[p]] < S]
    if wl.I_shared == 0:
        assert np.array_equal(got["y_pairs"][res], two["y_pairs"][res]), "routed y_pairs differ from the separate call"
    elif res:
        split = rel_max_err(got["y_pairs"][res], two["y_pairs"][res])
        say(f"  routed y_pairs vs the separate call: {split:.1e}")
        assert split <= SPLIT_TOL
    if res:
        assert rel_max_err(got["y_pairs"][res], want["y_pairs"][res]) <= DECODE_TOL
    err = rel_max_err(got["y"], want["y"])
    say(f"  max|y-y*|/max|y*| = {err:.3e}; vs separate calls {rel_max_err(got['y'], two['y']):.1e}")
    assert err <= DECODE_TOL
    assert rel_max_err(got["y"], two["y"]) <= SPLIT_TOL
    if wl.I_shared == 0:
        assert np.array_equal(got["y"], two["y"]), "combine differs from the separate combine"


SMALL_SHARED = [
    W.Workload("small Q4_K + shared (H512 E8 k2 I256 Ish256 T4)", F.Q4K, 512, 256, 8, 2, 4, I_shared=256),
    W.Workload("small Q4_K + shared, T=3", F.Q4K, 512, 256, 8, 2, 3, I_shared=384, seed=2),
    W.Workload("small Q4_K + shared, T=1", F.Q4K, 512, 256, 8, 2, 1, I_shared=128, seed=3),
    W.Workload("small MXFP4 + shared", F.MXFP4, 512, 256, 8, 2, 4, I_shared=256, seed=4),
    W.Workload("small Q3_K/Q4_K + shared", F.Q3K_Q4K, 512, 256, 8, 2, 4, I_shared=256, seed=5),
    W.Workload("small Q5_K + shared", F.Q5K, 512, 256, 8, 2, 4, I_shared=256, seed=6),
    W.Workload("small Q6_K + shared", F.Q6K, 512, 256, 8, 2, 4, I_shared=256, seed=7),
    W.Workload("small Q8_0 + shared", F.Q8_0, 256, 128, 8, 2, 4, I_shared=128, seed=8),
    W.Workload("sigmoid x2.5 + shared, E=256", F.Q4K, 512, 256, 256, 8, 2, score=1, scale=2.5, I_shared=256, seed=9),
    W.Workload("T=8: routing in its own launches (beyond the one-workgroup step)", F.Q4K, 512, 256, 16, 4, 8,
               I_shared=256, seed=10),
    W.Workload("E=300: routing in its own launches", F.Q4K, 256, 256, 300, 4, 2, I_shared=128, seed=11),
    W.Workload("k=16, T=4: 64 pairs, the one-workgroup routing's limit", F.Q4K, 512, 256, 64, 16, 4, I_shared=256,
               seed=13),
    W.Workload("k=32, T=2: 64 pairs over two rows", F.Q4K, 512, 256, 64, 32, 2, I_shared=256, seed=14),
]


@pytest.mark.parametrize("wl", SMALL_SHARED, ids=lambda w: w.name.split("(")[0].strip().replace(" ", "_")[:40])
def test_fused_decode_layer_small(wl):
    say(wl.name)
    _check(wl, *_case(wl))


@pytest.mark.parametrize("wl", [W.QWEN3_DECODE_T2,
                                W.Workload("small Q4_K, no shared, k=16 T=4", F.Q4K, 512, 256, 32, 16, 4, seed=15),
                                W.Workload("small Q4_K, no shared, k=32 T=2", F.Q4K, 512, 256, 64, 32, 2, seed=16)],
                         ids=["qwen3_T2", "k16_T4", "k32_T2"])
def test_fused_decode_layer_without_shared_expert(wl):
    say(wl.name)
    _check(wl, *_case(wl))


@pytest.fixture(scope="module")
def dsv3():
    say("generating 256 DeepSeek-V3-shaped Q4_K experts")
    F.set_num_threads(THREADS)
    wl = W.DSV3_DECODE_T2
    blobs = W.expert_blobs(wl)
    return blobs, pack_pool(wl.fmt, blobs, wl.H, wl.I, list(range(wl.E)), wl.E)


@pytest.mark.parametrize("wl", [W.DSV3_DECODE_T2, W.DSV3_DECODE_T4], ids=["T2", "T4"])
def test_fused_dsv3_layer(wl, dsv3):
    say(wl.name)
    blobs, pool = dsv3
    _check(wl, *_case(wl, blobs=blobs, pool=pool))


def test_fused_dsv3_partial_residency(dsv3):
    """Stack layer 0's 96-of-256 residency (+8 empty staging slots): the host
    list and the card part of the layer, shared expert included."""
    blobs, _ = dsv3
    wl = W.DSV3_DECODE_T2
    soe, S = W.slot_map(W.DSV3_STACK, 0)
    say("fused DeepSeek-V3-shaped layer, 96 resident")
    got, two, want, soe, S = _case(wl, soe=soe, S=S, blobs=blobs, logits=W.logits_of(W.DSV3_STACK, 0))
    _check(wl, got, two, want, soe, S)
    assert got["host_count"] > 0


@pytest.mark.parametrize("fmt", [F.Q5K, F.Q6K])
def test_fused_dsv3_sized_k_split_gateup(fmt):
    """DeepSeek-V3-sized Q5_K / Q6_K experts: their gate/up GEMV splits K over
    workgroups (its prefetch ring would spill), so a reduce launch follows
    the fused gate/up + shared down launch."""
    wl = W.Workload(f"DeepSeek-V3-sized fmt{fmt} experts, 16 resident, T=2, shared", fmt, 7168, 2048, 16, 4, 2,
                    score=1, scale=2.5, I_shared=2048, seed=12)
    say(wl.name)
    F.set_num_threads(THREADS)
    _check(wl, *_case(wl))


def test_fused_layer_graph_replay_equals_eager():
    wl = SMALL_SHARED[0]
    soe, S = W.slot_map(wl)
    blobs = W.expert_blobs(wl)
    layer = device_layer(wl, blobs, soe, S, W.shared_blob(wl), wl.T, Q.MOE_PATH_DECODE)
    x, lg = torch.from_numpy(W.x_of(wl)).cuda(), torch.from_numpy(W.logits_of(wl)).cuda()
    y0 = layer.forward(x, lg).clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.forward(x, lg)
    for _ in range(3):
        layer.y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(layer.y, y0)
        layer.forward(x, lg)  # eager work between replays
        torch.cuda.synchronize()


def test_fused_layer_refusals():
    """Checked before any launch: a shared pool without a width, a width
    without a pool, a Q8_0 width that is not a multiple of 128."""
    wl = SMALL_SHARED[0]
    soe, S = W.slot_map(wl)
    layer = device_layer(wl, W.expert_blobs(wl), soe, S, W.shared_blob(wl), wl.T, Q.MOE_PATH_DECODE)
    x, lg = torch.from_numpy(W.x_of(wl)).cuda(), torch.from_numpy(W.logits_of(wl)).cuda()
    args = (wl.fmt, lg, x, wl.k, wl.score, wl.renormalize, wl.scale, layer.slot_of_expert, S, layer.slot_pool,
            layer.stride, wl.I)
    outs = (layer.ids, layer.w, layer.slot_offsets, layer.active_slots, layer.num_active, layer.perm_pair,
            layer.host_token, layer.host_expert, layer.host_weight, layer.host_count, layer.y_pairs, layer.y, layer.ws)
    with pytest.raises(Q.QmoeError, match="shared_pool and I_shared"):
        Q.moe_layer_decode(*args, layer.shared_pool, 0, *outs)
    with pytest.raises(Q.QmoeError, match="multiples of 128"):
        Q.moe_layer_decode(*args, layer.shared_pool, 200, *outs)
    small = layer.ws[:16]
    with pytest.raises(Q.QmoeError, match="workspace"):
        Q.moe_layer_decode(*args, layer.shared_pool, wl.I_shared, *outs[:-1], small)
