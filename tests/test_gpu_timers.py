"""Stage timers on the GPU (moe_timer_begin / moe_timer_end): one event pair
per launch of a stage, attached to the stage's own kernel dispatches.  Every
launch is counted, each time is positive and no longer than the wall time of
the launches, and a stage of two kernels (a K split across workgroups:
partial sums, then the reduce) is timed over both."""
import time

import numpy as np
import pytest
import torch

import fixtures as F
import quantized_routed_expert_moe_amd as Q
from fixtures import workloads as W
from tests.gpu_util import device_layer, say, to_dev_x

pytestmark = pytest.mark.gpu

N = 20
STAGE_ROUTE_BATCHES, STAGE_GATEUP, STAGE_DOWN, STAGE_COMBINE = 8, 3, 4, 5
STAGE_TILES, STAGE_PREFILL_GATEUP, STAGE_PREFILL_DOWN = 2, 6, 7


def _timed(layer, x, lg, stages):
    xd, ld = to_dev_x(x), torch.from_numpy(lg).cuda()
    layer.forward(xd, ld)
    torch.cuda.synchronize()
    for s in stages:
        Q.moe_timer_begin(s, N)
    t0 = time.perf_counter()
    for _ in range(N):
        layer.forward(xd, ld)
    torch.cuda.synchronize()
    wall_ms = 1e3 * (time.perf_counter() - t0)
    out = {s: Q.moe_timer_end(s) for s in stages}
    return out, wall_ms


def _check(out, wall_ms, stages):
    total = 0.0
    for s in stages:
        ms, n = out[s]
        say(f"  stage {s}: {n} launches, {1e3 * ms / max(n, 1):.2f} us each")
        assert n == N, (s, n)
        assert 0.0 < ms, s
        total += ms
    assert total <= wall_ms, (total, wall_ms)


def test_decode_stage_timers():
    wl = W.Workload("small Q4_K layer (H512 E8 k2 I256 T4)", F.Q4K, 512, 256, 8, 2, 4)
    say(wl.name)
    soe, S = W.slot_map(wl)
    layer = device_layer(wl, W.expert_blobs(wl), soe, S, None, wl.T, Q.MOE_PATH_DECODE)
    stages = (STAGE_ROUTE_BATCHES, STAGE_GATEUP, STAGE_DOWN, STAGE_COMBINE)
    out, wall = _timed(layer, W.x_of(wl), W.logits_of(wl), stages)
    _check(out, wall, stages)


def test_k_split_stage_is_timed_over_both_kernels():
    """H 7168 over two experts: the gate/up GEMV splits K across workgroups and
    a reduce launch finishes it; the stage's time spans both kernels, so it
    exceeds the time of the same GEMV's down stage, which is one kernel over
    a 256-wide K."""
    wl = W.Workload("Q4_K layer H 7168, 2 experts, k 1, T 5", F.Q4K, 7168, 256, 2, 1, 5)
    say(wl.name)
    soe, S = W.slot_map(wl)
    layer = device_layer(wl, W.expert_blobs(wl), soe, S, None, wl.T, Q.MOE_PATH_DECODE)
    stages = (STAGE_GATEUP, STAGE_DOWN)
    out, wall = _timed(layer, W.x_of(wl), W.logits_of(wl), stages)
    _check(out, wall, stages)
    assert out[STAGE_GATEUP][0] > out[STAGE_DOWN][0]


def test_prefill_stage_timers():
    wl = W.Workload("prefill T128 E8 k2", F.Q4K, 512, 256, 8, 2, 128, x_bf16=True, seed=5)
    say(wl.name)
    soe, S = W.slot_map(wl)
    layer = device_layer(wl, W.expert_blobs(wl), soe, S, None, wl.T, Q.MOE_PATH_PREFILL,
                         pair_dtype=torch.bfloat16, y_dtype=torch.bfloat16)
    stages = (STAGE_TILES, STAGE_PREFILL_GATEUP, STAGE_PREFILL_DOWN)
    out, wall = _timed(layer, W.x_of(wl), W.logits_of(wl), stages)
    _check(out, wall, stages)


def test_timer_counts_nothing_without_launches():
    """T = 0: no kernel runs, so nothing is timed."""
    wl = W.Workload("small Q4_K layer, no tokens", F.Q4K, 512, 256, 8, 2, 0)
    soe, S = W.slot_map(wl)
    layer = device_layer(wl, W.expert_blobs(wl), soe, S, None, 0, Q.MOE_PATH_DECODE)
    x = np.zeros((0, wl.H), dtype=np.float32)
    lg = np.zeros((0, wl.E), dtype=np.float32)
    out, _ = _timed(layer, x, lg, (STAGE_GATEUP,))
    assert out[STAGE_GATEUP] == (0.0, 0)


def test_timer_read_gives_each_launch():
    """moe_timer_read: one positive time per launch, in launch order, whose
    sum is the total moe_timer_end returns; reading leaves the timer armed."""
    wl = W.Workload("small Q4_K layer (H512 E8 k2 I256 T4)", F.Q4K, 512, 256, 8, 2, 4)
    soe, S = W.slot_map(wl)
    layer = device_layer(wl, W.expert_blobs(wl), soe, S, None, wl.T, Q.MOE_PATH_DECODE)
    xd, ld = to_dev_x(W.x_of(wl)), torch.from_numpy(W.logits_of(wl)).cuda()
    layer.forward(xd, ld)
    torch.cuda.synchronize()
    Q.moe_timer_begin(STAGE_GATEUP, 2 * N)
    for _ in range(N):
        layer.forward(xd, ld)
    each = Q.moe_timer_read(STAGE_GATEUP, 2 * N)
    assert each.shape == (N,) and (each > 0).all()
    layer.forward(xd, ld)  # still armed: one more launch is timed
    again = Q.moe_timer_read(STAGE_GATEUP, 2 * N)
    ms, n = Q.moe_timer_end(STAGE_GATEUP)
    assert n == N + 1 and again.shape == (N + 1,)
    assert np.array_equal(again[:N], each)
    assert abs(float(again.astype(np.float64).sum()) - ms) <= 1e-5 * ms
