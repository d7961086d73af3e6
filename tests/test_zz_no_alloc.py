"""The allocation-free expert FFN (moe_expert_ffn_q4k_noalloc) against
moe_expert_ffn_q4k with a caller-owned workspace: the same kernels, so the
outputs must agree bit for bit.  Two calls in a row on one GPU share the
library's scratch, the second with a smaller input than the first."""
import numpy as np
import pytest
import torch

import fixtures as F
import quantized_routed_expert_moe_amd as Q
from fixtures import workloads as W
from tests.gpu_util import device_layer, say, to_dev_x

pytestmark = pytest.mark.gpu


def _both(wl, path, pair_dtype):
    """y_pairs of one layer's expert FFN through both entry points, on the batches the layer's own forward built."""
    soe, S = W.slot_map(wl)
    layer = device_layer(wl, W.expert_blobs(wl), soe, S, None, wl.T, path, pair_dtype=pair_dtype,
                         y_dtype=pair_dtype)
    x = to_dev_x(W.x_of(wl))
    layer.forward(x, torch.from_numpy(W.logits_of(wl)).cuda())
    want = layer.y_pairs.clone()
    got = torch.full_like(layer.y_pairs, float("nan"))
    Q.moe_expert_ffn_q4k_noalloc(layer.slot_pool, layer.stride, layer.S, wl.H, wl.I, x, wl.k, layer.slot_offsets,
                                 layer.active_slots, layer.num_active, layer.perm_pair, got, path)
    torch.cuda.synchronize()
    n_res = int(layer.slot_offsets[-1].item())
    rows = layer.perm_pair[:n_res].long()
    return got[rows].float().cpu().numpy(), want[rows].float().cpu().numpy(), n_res


def test_noalloc_matches_workspace_entry_point_twice():
    big = W.Workload("prefill T300 E16 k4 Q4_K", F.Q4K, 512, 256, 16, 4, 300, x_bf16=True, zipf_s=1.0, seed=3)
    small = W.Workload("decode T2 E8 k2 Q4_K", F.Q4K, 512, 256, 8, 2, 2, seed=4)
    for wl, path, pd in ((big, Q.MOE_PATH_PREFILL, torch.bfloat16), (small, Q.MOE_PATH_DECODE, torch.float32)):
        say(f"noalloc vs workspace: {wl.name}")
        got, want, n_res = _both(wl, path, pd)
        assert n_res == wl.T * wl.k
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), wl.name


def test_noalloc_int8_path_matches_workspace_entry_point_twice():
    """The same on the int8-activation prefill path, whose workspace adds the
    activation planes and their sums to the bf16 path's."""
    big = W.Workload("prefill int8 T300 E16 k4 Q4_K", F.Q4K, 512, 256, 16, 4, 300, x_bf16=True, zipf_s=1.0, seed=3)
    small = W.Workload("prefill int8 T129 E8 k2 Q4_K", F.Q4K, 512, 256, 8, 2, 129, x_bf16=True, zipf_s=1.0, seed=3)
    for wl, pd in ((big, torch.bfloat16), (small, torch.float32)):
        say(f"noalloc vs workspace: {wl.name}")
        got, want, n_res = _both(wl, Q.MOE_PATH_PREFILL_I8, pd)
        assert n_res == wl.T * wl.k
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), wl.name
