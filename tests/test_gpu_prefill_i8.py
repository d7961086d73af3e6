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
import oracle as O
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


def _two_planes(v: np.ndarray) -> np.ndarray:
    """A row as the int8 path represents it, in fp64: s (q1 + q2 / 254) with
    s = max|v| / 127, each code decided in fp32 (v * (1 / s) rounded to
    nearest even, the remainder times 254 likewise), clamped to [-127, 127]."""
    v32 = v.astype(np.float32)
    mx = np.float32(np.max(np.abs(v32)))
    s = mx / np.float32(127.0) if mx > 0 else np.float32(1.0)
    y = v32 * (np.float32(1.0) / s)
    f1 = np.clip(np.rint(y), -127, 127).astype(np.float32)
    f2 = np.clip(np.rint((y - f1) * np.float32(254.0)), -127, 127)
    return float(s) * (f1.astype(np.float64) + f2.astype(np.float64) / 254.0)


def test_prefill_i8_equals_its_two_plane_model():
    """The int8 path is the exact layer with three roundings: x split into
    two int8 planes per row, h rounded to bf16, and h split into two planes;
    the Q4_K weights enter exactly (d sc and dmin m are exact in fp32).
    Emulating those on the oracle's fp64 dequantized weights reproduces the
    GPU's y_pairs up to fp32 accumulation noise.  Each sub-block's scale
    term d sc (T1 + T2 / 254) and min term dmin m X are formed apart in fp32
    and largely cancel, so g and u carry up to about 2^-14 of their own value
    in rounding error: an h that close to a bf16 rounding midpoint may round
    either way, which moves that element by one bf16 ulp plus the two planes'
    representation error (allowed for); a pair whose largest |h| is such an
    element (its scale may differ) is left out, and such pairs must be rare
    (measured: 3 of 128, the rest within 1.2e-7 of the model)."""
    from tests.gpu_util import device_layer, run_device
    wl = W.Workload("prefill int8 rounding model", F.Q4K, 512, 256, 4, 2, 64, x_bf16=True, seed=11)
    say(wl.name)
    x, logits = W.x_of(wl), W.logits_of(wl)
    blobs = W.expert_blobs(wl)
    soe, S = W.slot_map(wl)
    got = run_device(device_layer(wl, blobs, soe, S, None, wl.T, I8, pair_dtype=torch.float32), x, logits)
    H, I = wl.H, wl.I
    gb = F.matrix_bytes(F.Q4K, I, H)
    xf = W.x_f64(wl, x)
    worst, left_out = 0.0, 0
    for t in range(wl.T):
        xt = _two_planes(xf[t])
        for j in range(wl.k):
            b = blobs[int(got["ids"][t, j])]
            Wg = O.dequant(F.Q4K, b[:gb], I * H).reshape(I, H)
            Wu = O.dequant(F.Q4K, b[gb:2 * gb], I * H).reshape(I, H)
            Wd = O.dequant(F.Q4K, b[2 * gb:], H * I).reshape(H, I)
            g, u = Wg @ xt, Wu @ xt
            hx = g / (1 + np.exp(-g)) * u
            h = F.bf16_bits_to_f32(F.to_bf16_bits(hx.astype(np.float32))).astype(np.float64)
            ulp = np.ldexp(1.0, np.frexp(np.abs(h) + 1e-300)[1] - 8)
            mid = np.minimum(np.abs(np.abs(hx) - (np.abs(h) - ulp / 2)), np.abs(np.abs(hx) - (np.abs(h) + ulp / 2)))
            amb = mid <= np.abs(hx) * 2.0 ** -14
            if amb.any() and np.abs(h[amb]).max() >= np.abs(h).max() - ulp.max():
                left_out += 1
                continue
            y = Wd @ _two_planes(h)
            slack = np.abs(Wd[:, amb]) @ (ulp[amb] + np.abs(h).max() / 127 / 254)
            dev = np.abs(got["y_pairs"][t * wl.k + j] - y)
            worst = max(worst, float(np.max((dev - slack) / np.abs(y).max())))
    say(f"  max (|y_pair - model| - midpoint allowance) / max |model| = {worst:.3e}, pairs left out {left_out}")
    assert left_out <= 6
    assert worst <= 2e-5


def test_prefill_i8_refuses_other_formats():
    assert Q.moe_ffn_workspace_size(F.MXFP4, 64, 2, 512, 256, I8) == 0
    assert Q.moe_ffn_workspace_size(F.Q4K, 64, 2, 512, 256, I8) > Q.moe_ffn_workspace_size(F.Q4K, 64, 2, 512, 256,
                                                                                            Q.MOE_PATH_PREFILL)
