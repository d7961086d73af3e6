"""Parity of the prefill path (bf16 MFMA grouped GEMM over Q4_K, MXFP4, Q5_K,
Q6_K or Q3_K/Q4_K tiles) with the CPU oracle.

Ids, slot offsets, active slots, permutation and host list: bit-exact on
every row.  Outputs: per token row t, max_i |y_ti - y*_ti| <= 1e-2 *
max_i |y*_ti| (bf16 activations, weights rounded to bf16 tiles, h rounded
to bf16, fp32 accumulation).  At the full 4096-token size the oracle runs on
a seeded sample of rows (routing is per row, so a row's output depends only
on that row's x and logits).
"""
import dataclasses

import numpy as np
import pytest
import torch

import fixtures as F
import oracle as O
import quantized_routed_expert_moe_amd as Q
from fixtures import workloads as W
from tests.gpu_util import THREADS, device_layer, run_device, run_oracle, say

pytestmark = pytest.mark.gpu

PREFILL_TOL = 1e-2


def _row_err(got, want):
    return float(np.max(np.abs(got - want).max(axis=1) / np.maximum(np.abs(want).max(axis=1), 1e-30)))


def _check_ints(wl, got, ids, w, soe, S):
    ob = O.batches(ids, w, wl.E, soe, S)
    for key in ("slot_offsets", "active_slots", "perm_pair", "host_token", "host_expert"):
        assert np.array_equal(got[key], ob[key]), key


def _prefill_case(wl, soe=None, S=None, pair_dtype=torch.bfloat16, y_dtype=torch.bfloat16, sample=None, blobs=None,
                  path=Q.MOE_PATH_PREFILL):
    soe_, S_ = W.slot_map(wl)
    soe = soe_ if soe is None else soe
    S = S_ if S is None else S
    x, logits = W.x_of(wl), W.logits_of(wl)
    blobs = W.expert_blobs(wl) if blobs is None else blobs
    layer = device_layer(wl, blobs, soe, S, None, wl.T, path, pair_dtype=pair_dtype, y_dtype=y_dtype)
    got = run_device(layer, x, logits)
    ids, w = O.route(logits, wl.k, wl.score, wl.renormalize, wl.scale)
    assert np.array_equal(got["ids"], ids)
    assert np.abs(got["w"] - w).max() <= 1e-6
    _check_ints(wl, got, ids, w, soe, S)
    rows = np.arange(wl.T) if sample is None else sample
    want = run_oracle(wl, blobs, x[rows], logits[rows], soe, None)
    err = _row_err(got["y"][rows], want["y"])
    say(f"  rows checked {len(rows)}, max per-row error {err:.3e}")
    return err


@pytest.mark.parametrize("fmt", [F.Q4K, F.MXFP4, F.Q5K, F.Q6K, F.Q3K_Q4K], ids=["Q4_K", "MXFP4", "Q5_K", "Q6_K", "Q3_K-Q4_K"])
def test_prefill_qwen3_full_size(fmt):
    """4096 tokens, Zipf(1.0)-skewed loads over 128 experts, all resident."""
    names = {F.MXFP4: "MXFP4", F.Q5K: "Q5_K", F.Q6K: "Q6_K", F.Q3K_Q4K: "Q3_K gate/up + Q4_K down"}
    wl = W.QWEN3_PREFILL if fmt == F.Q4K else dataclasses.replace(W.QWEN3_PREFILL, fmt=fmt,
                                                                  name=W.QWEN3_PREFILL.name + f", {names[fmt]} experts")
    say(wl.name)
    F.set_num_threads(THREADS)
    sample = _covering_sample(wl, 320)
    assert _prefill_case(wl, sample=sample) <= PREFILL_TOL


def _covering_sample(wl, n_rows: int) -> np.ndarray:
    """Rows whose outputs the oracle checks at full size: for every expert the
    first and the last row routed to it (a slot's pairs are in row order, so
    these sit in its first and its last, ragged, M tile), then seeded random
    rows up to n_rows.  Every expert's weights are thus compared."""
    ids, _ = O.route(W.logits_of(wl), wl.k, wl.score, wl.renormalize, wl.scale)
    rows = set()
    for e in range(wl.E):
        r = np.nonzero((ids == e).any(axis=1))[0]
        if r.size:
            rows.update((int(r[0]), int(r[-1])))
    rng = np.random.default_rng(0)
    rest = rng.permutation(np.setdiff1d(np.arange(wl.T), sorted(rows)))
    sample = np.sort(np.concatenate([np.array(sorted(rows), dtype=np.int64), rest[:max(0, n_rows - len(rows))]]))
    covered = set(np.unique(ids[sample]).tolist())
    assert covered == set(np.unique(ids).tolist()) and len(covered) == wl.E, "sample misses an expert"
    return sample


@pytest.mark.parametrize("fmt", [F.Q4K, F.MXFP4, F.Q5K, F.Q6K, F.Q3K_Q4K], ids=["Q4_K", "MXFP4", "Q5_K", "Q6_K", "Q3_K-Q4_K"])
@pytest.mark.parametrize("T,E,k,pd,yd", [
    (300, 16, 4, torch.bfloat16, torch.bfloat16),
    (129, 8, 2, torch.float32, torch.float32),
    (64, 32, 8, torch.float32, torch.bfloat16),
])
def test_prefill_small_layers(T, E, k, pd, yd, fmt):
    """Several M tiles per slot, ragged last tiles, slots with a single row."""
    wl = W.Workload(f"prefill T{T} E{E} k{k} fmt{fmt}", fmt, 512, 256, E, k, T, x_bf16=True, zipf_s=1.0, seed=3)
    say(wl.name)
    assert _prefill_case(wl, pair_dtype=pd, y_dtype=yd) <= PREFILL_TOL


def test_prefill_at_the_slot_limit():
    """E = S = 1024 (MOE_MAX_EXPERTS, one tile-list thread per slot): 640
    tokens x k 8 spread over every expert, so most slots hold a handful of
    rows in one ragged tile and a few (Zipf head) several tiles."""
    wl = W.Workload("prefill T640 E1024 k8, all resident", F.Q4K, 256, 256, 1024, 8, 640, x_bf16=True,
                    zipf_s=1.0, seed=9)
    say(wl.name)
    F.set_num_threads(THREADS)
    # fp32 y_pairs and y: the case is about the tile list at 1024 slots; the
    # error left is the bf16 model's own (weights and h rounded once each),
    # about 5e-3 of a row's largest output at this short K
    assert _prefill_case(wl, pair_dtype=torch.float32, y_dtype=torch.float32) <= PREFILL_TOL


@pytest.mark.parametrize("fmt", [F.Q4K, F.MXFP4, F.Q5K, F.Q6K, F.Q3K_Q4K], ids=["Q4_K", "MXFP4", "Q5_K", "Q6_K", "Q3_K-Q4_K"])
def test_prefill_partial_residency(fmt):
    wl = W.Workload("prefill T200 E24 k3, 15 resident of 24", fmt, 768, 512, 24, 3, 200, x_bf16=True,
                    zipf_s=1.2, seed=5)
    say(wl.name)
    rng = np.random.default_rng(1)
    soe = np.full(24, -1, dtype=np.int32)
    soe[rng.permutation(24)[:15]] = rng.permutation(17)[:15]
    assert _prefill_case(wl, soe=soe, S=17) <= PREFILL_TOL


@pytest.mark.parametrize("fmt", [F.Q4K, F.MXFP4, F.Q5K, F.Q6K, F.Q3K_Q4K], ids=["Q4_K", "MXFP4", "Q5_K", "Q6_K", "Q3_K-Q4_K"])
def test_prefill_tile_boundaries(fmt):
    """One expert receives exactly 128, another 129, another 1 pair."""
    wl = W.Workload("prefill tile boundaries", fmt, 256, 256, 4, 1, 258, x_bf16=True, seed=7)
    say(wl.name)
    x = W.x_of(wl)
    logits = np.zeros((258, 4), dtype=np.float32)
    logits[:, 3] = -1.0
    logits[:128, 0] = 5.0
    logits[128:257, 1] = 5.0
    logits[257, 2] = 5.0
    blobs = W.expert_blobs(wl)
    soe, S = W.slot_map(wl)
    layer = device_layer(wl, blobs, soe, S, None, wl.T, Q.MOE_PATH_PREFILL, pair_dtype=torch.float32)
    got = run_device(layer, x, logits)
    assert got["slot_offsets"].tolist() == [0, 128, 257, 258, 258]
    want = run_oracle(wl, blobs, x, logits, soe, None)
    assert _row_err(got["y"], want["y"]) <= PREFILL_TOL


def test_prefill_matches_decode_path_closely():
    """The same layer through both paths: decode (fp16 activations) and
    prefill (bf16 tiles) agree within the prefill tolerance."""
    wl = W.Workload("prefill vs decode", F.Q4K, 512, 512, 8, 2, 40, x_bf16=True, seed=9)
    say(wl.name)
    x, logits = W.x_of(wl), W.logits_of(wl)
    blobs = W.expert_blobs(wl)
    soe, S = W.slot_map(wl)
    pre = run_device(device_layer(wl, blobs, soe, S, None, wl.T, Q.MOE_PATH_PREFILL, pair_dtype=torch.float32),
                     x, logits)
    dec = run_device(device_layer(wl, blobs, soe, S, None, wl.T, Q.MOE_PATH_DECODE), x, logits)
    assert _row_err(pre["y"], dec["y"]) <= PREFILL_TOL


def _bf16_round(a: np.ndarray) -> np.ndarray:
    return F.bf16_bits_to_f32(F.to_bf16_bits(a.astype(np.float32))).astype(np.float64)


@pytest.mark.parametrize("fmt", [F.Q4K, F.MXFP4, F.Q5K, F.Q6K, F.Q3K_Q4K], ids=["Q4_K", "MXFP4", "Q5_K", "Q6_K", "Q3_K-Q4_K"])
def test_prefill_equals_its_bf16_rounding_model(fmt):
    """The prefill arithmetic is the exact layer with three roundings: each
    dequantized weight to fp32 then bf16 (MXFP4 weights are bf16 values
    already), and h to bf16.  Emulating those roundings on the oracle's fp64
    dequantized weights must reproduce the GPU's y_pairs up to fp32
    accumulation noise, where an h that sits on a bf16 rounding midpoint may
    round either way."""
    wl = W.Workload("prefill rounding model", fmt, 512, 256, 4, 2, 64, x_bf16=True, seed=11)
    say(wl.name)
    x, logits = W.x_of(wl), W.logits_of(wl)
    blobs = W.expert_blobs(wl)
    soe, S = W.slot_map(wl)
    got = run_device(device_layer(wl, blobs, soe, S, None, wl.T, Q.MOE_PATH_PREFILL, pair_dtype=torch.float32),
                     x, logits)
    H, I = wl.H, wl.I
    fgu, fdn = (F.Q3K, F.Q4K) if fmt == F.Q3K_Q4K else (fmt, fmt)  # block types of gate/up and down
    gb = F.matrix_bytes(fgu, I, H)
    xf = W.x_f64(wl, x)
    worst = 0.0
    for t in range(wl.T):
        for j in range(wl.k):
            e = int(got["ids"][t, j])
            b = blobs[e]
            Wg = _bf16_round(O.dequant(fgu, b[:gb], I * H)).reshape(I, H)
            Wu = _bf16_round(O.dequant(fgu, b[gb:2 * gb], I * H)).reshape(I, H)
            Wd = _bf16_round(O.dequant(fdn, b[2 * gb:], H * I)).reshape(H, I)
            g, u = Wg @ xf[t], Wu @ xf[t]
            hx = g / (1 + np.exp(-g)) * u
            h = _bf16_round(hx)
            y = Wd @ h
            # The GPU's silu (hardware exp2 and reciprocal) is a few fp32 ulps
            # off the exact one, so an h within that of a bf16 rounding midpoint
            # may round the other way: allow one bf16 ulp for exactly those.
            ulp = np.ldexp(1.0, np.frexp(np.abs(h) + 1e-300)[1] - 8)
            mid = np.abs(np.abs(hx) - (np.abs(h) - ulp / 2))
            mid = np.minimum(mid, np.abs(np.abs(hx) - (np.abs(h) + ulp / 2)))
            amb = mid <= np.abs(hx) * 2.0 ** -18
            slack = np.abs(Wd[:, amb]) @ ulp[amb]
            dev = np.abs(got["y_pairs"][t * wl.k + j] - y)
            worst = max(worst, float(np.max((dev - slack) / np.abs(y).max())))
    say(f"  max (|y_pair - model| - rounding-flip allowance) / max |model| = {worst:.3e}")
    assert worst <= 2e-5


@pytest.mark.parametrize("path", [Q.MOE_PATH_PREFILL, Q.MOE_PATH_PREFILL_I8], ids=["bf16", "int8"])
def test_prefill_nothing_resident(path):
    """Every expert on the host (slot map all -1, four empty slots): no
    active slot and no tile, every pair on the host list, y zero."""
    wl = W.Workload("prefill T96 E8 k2, nothing resident", F.Q4K, 256, 256, 8, 2, 96, x_bf16=True, seed=11)
    say(f"{wl.name}, path {path}")
    assert _prefill_case(wl, soe=np.full(8, -1, dtype=np.int32), S=4, path=path) == 0.0


@pytest.mark.parametrize("path", [Q.MOE_PATH_DECODE, Q.MOE_PATH_PREFILL, Q.MOE_PATH_PREFILL_I8],
                         ids=["decode", "bf16", "int8"])
def test_expert_ffn_empty_step(path):
    """T = 0 through moe_expert_ffn_q4k: the call succeeds and leaves y_pairs
    as it was."""
    say(f"expert FFN T=0, path {path}")
    H, I, S, k = 256, 256, 2, 2
    dev = dict(device="cuda")
    stride = (Q.moe_packed_blob_bytes(F.Q4K, H, I) + 255) // 256 * 256
    pool = torch.zeros(S * stride, dtype=torch.uint8, **dev)
    x = torch.zeros((0, H), dtype=torch.float32 if path == Q.MOE_PATH_DECODE else torch.bfloat16, **dev)
    offsets = torch.zeros(S + 1, dtype=torch.int32, **dev)
    active = torch.zeros(S, dtype=torch.int32, **dev)
    num = torch.zeros(1, dtype=torch.int32, **dev)
    perm = torch.zeros(1, dtype=torch.int32, **dev)
    y_pairs = torch.full((1, H), float("nan"), dtype=torch.float32, **dev)
    ws = torch.zeros(max(1, Q.moe_ffn_workspace_size(F.Q4K, 0, k, H, I, path)), dtype=torch.uint8, **dev)
    Q.moe_expert_ffn_q4k(pool, stride, S, H, I, x, k, offsets, active, num, perm, y_pairs, path, ws=ws)
    torch.cuda.synchronize()
    assert torch.isnan(y_pairs).all()


@pytest.mark.parametrize("path", [Q.MOE_PATH_PREFILL, Q.MOE_PATH_PREFILL_I8], ids=["bf16", "int8"])
def test_prefill_graph_replay_equals_eager(path):
    """One prefill forward (routing, batching, tile list, GEMMs, combine)
    captured in a hipGraph on static inputs: every replay, with new input
    contents copied in eagerly and a synchronization between replays, equals
    the eager forward on the same inputs bit for bit."""
    from tests.gpu_util import to_dev_x
    wl = W.Workload("prefill T300 E16 k4 Q4_K", F.Q4K, 512, 256, 16, 4, 300, x_bf16=True, zipf_s=1.0, seed=3)
    say(f"prefill graph replay, path {path}")
    soe, S = W.slot_map(wl)
    layer = device_layer(wl, W.expert_blobs(wl), soe, S, None, wl.T, path)
    xs = [to_dev_x(W.x_of(wl, seed=s)) for s in range(3)]
    ls = [torch.from_numpy(W.logits_of(wl, seed=s)).cuda() for s in range(3)]
    eager = [layer.forward(xs[i], ls[i]).clone() for i in range(3)]
    torch.cuda.synchronize()
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


@pytest.mark.parametrize("path", [Q.MOE_PATH_PREFILL, Q.MOE_PATH_PREFILL_I8], ids=["bf16", "int8"])
def test_prefill_zero_and_outlier_rows(path):
    """Token rows of zeros give y exactly zero (on the int8 path the row
    scale of a zero row falls back to 1 with every code 0); a row with one
    element 1000 times the others' scale stays within the bound."""
    from tests.gpu_util import run_oracle
    wl = W.Workload("prefill zero and outlier rows", F.Q4K, 512, 256, 8, 2, 96, x_bf16=True, seed=13)
    say(f"{wl.name}, path {path}")
    x = W.x_of(wl).copy()
    zero = np.arange(wl.T) % 3 == 0
    x[zero] = 0
    x[1, 5] = F.to_bf16_bits(np.array([1000.0], dtype=np.float32))[0]
    logits = W.logits_of(wl)
    soe, S = W.slot_map(wl)
    blobs = W.expert_blobs(wl)
    got = run_device(device_layer(wl, blobs, soe, S, None, wl.T, path), x, logits)
    want = run_oracle(wl, blobs, x, logits, soe, None)
    assert np.all(got["y"][zero] == 0)
    assert np.all(want["y"][zero] == 0)
    assert _row_err(got["y"][~zero], want["y"][~zero]) <= PREFILL_TOL
