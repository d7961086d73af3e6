"""Parity of the int8-activation prefill path (MOE_PATH_PREFILL_I8: Q4_K
experts, two int8 planes per activation row on the i8 MFMA, per-sub-block
fp32 rescaling) with the CPU oracle, to the prefill bound: per token row t,
max_i |y_ti - y*_ti| <= 1e-2 * max_i |y*_ti|; ids, batches and host list
bit-exact.  The cases are the bf16 path's: the 4096-token Qwen3-shaped layer
on a sample of rows covering every expert, small layers with several and
ragged M tiles and both y_pairs types, partial residency, tile boundaries,
1024 slots."""
import numpy as np
import pytest
import torch

import fixtures as F
import quantized_routed_expert_moe_amd as Q
from fixtures import workloads as W
from tests.gpu_util import THREADS, say
from tests.test_gpu_prefill import PREFILL_TOL, _covering_sample, _prefill_case

pytestmark = pytest.mark.gpu

I8 = Q.MOE_PATH_PREFILL_I8


def test_prefill_i8_qwen3_full_size():
    wl = W.QWEN3_PREFILL
    say(wl.name + ", int8 activations")
    F.set_num_threads(THREADS)
    assert _prefill_case(wl, sample=_covering_sample(wl, 320), path=I8) <= PREFILL_TOL


@pytest.mark.parametrize("T,E,k,pd,yd", [
    (300, 16, 4, torch.bfloat16, torch.bfloat16),
    (129, 8, 2, torch.float32, torch.float32),
    (64, 32, 8, torch.float32, torch.bfloat16),
])
def test_prefill_i8_small_layers(T, E, k, pd, yd):
    wl = W.Workload(f"prefill int8 T{T} E{E} k{k}", F.Q4K, 512, 256, E, k, T, x_bf16=True, zipf_s=1.0, seed=3)
    say(wl.name)
    assert _prefill_case(wl, pair_dtype=pd, y_dtype=yd, path=I8) <= PREFILL_TOL


def test_prefill_i8_partial_residency():
    wl = W.Workload("prefill int8 T200 E24 k3, 15 resident of 24", F.Q4K, 768, 512, 24, 3, 200, x_bf16=True,
                    zipf_s=1.2, seed=5)
    say(wl.name)
    rng = np.random.default_rng(1)
    soe = np.full(24, -1, dtype=np.int32)
    soe[rng.permutation(24)[:15]] = rng.permutation(17)[:15]
    assert _prefill_case(wl, soe=soe, S=17, path=I8) <= PREFILL_TOL


def test_prefill_i8_tile_boundaries():
    """One expert receives exactly 128, another 129, another 1 pair (a wave
    whose row half of the tile is empty, and a single-row tile)."""
    wl = W.Workload("prefill int8 tile boundaries", F.Q4K, 256, 256, 4, 1, 258, x_bf16=True, seed=7)
    say(wl.name)
    logits = np.full((258, 4), -5.0, dtype=np.float32)
    logits[:128, 0] = 5.0
    logits[128:257, 1] = 5.0
    logits[257, 2] = 5.0
    x = W.x_of(wl)
    from tests.gpu_util import device_layer, run_device, run_oracle
    soe, S = W.slot_map(wl)
    blobs = W.expert_blobs(wl)
    layer = device_layer(wl, blobs, soe, S, None, wl.T, I8, pair_dtype=torch.float32, y_dtype=torch.float32)
    got = run_device(layer, x, logits)
    want = run_oracle(wl, blobs, x, logits, soe, None)
    err = float(np.max(np.abs(got["y"] - want["y"]).max(axis=1) / np.abs(want["y"]).max(axis=1)))
    say(f"  max per-row error {err:.3e}")
    assert err <= PREFILL_TOL


def test_prefill_i8_at_the_slot_limit():
    """E = S = 1024 (MOE_MAX_EXPERTS): 640 tokens x k 8 over every expert,
    most slots a handful of rows in one ragged tile, a few several tiles."""
    wl = W.Workload("prefill int8 T640 E1024 k8, all resident", F.Q4K, 256, 256, 1024, 8, 640, x_bf16=True,
                    zipf_s=1.0, seed=9)
    say(wl.name)
    F.set_num_threads(THREADS)
    assert _prefill_case(wl, pair_dtype=torch.float32, y_dtype=torch.float32, path=I8) <= PREFILL_TOL


def test_prefill_i8_refuses_other_formats():
    assert Q.moe_ffn_workspace_size(F.MXFP4, 64, 2, 512, 256, I8) == 0
    assert Q.moe_ffn_workspace_size(F.Q4K, 64, 2, 512, 256, I8) > Q.moe_ffn_workspace_size(F.Q4K, 64, 2, 512, 256,
                                                                                            Q.MOE_PATH_PREFILL)
