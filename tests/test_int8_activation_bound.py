"""Why the prompt path keeps bf16 activations: on the Qwen3-30B-A3B-shaped
layer, quantizing the activations to int8 (x before gate/up, h before down),
with exact rounding and exact fp64 weights, already moves a token row's
output by more than the prefill tolerance of 1e-2 * max |y*_t|, at every
usual scale granularity (one scale per row, per 256 and per 32 elements;
int8 tensor-core prompts are the pages' own prompt design: bloomery README
0.3.1, "Why it is fast").  The same rows through the bf16 path's rounding
model (weights rounded once to bf16, h rounded to bf16) stay well inside the
bound (about half of it).  No GPU: fp64 oracle dequantization of the stored blocks and numpy
products on a seeded sample."""
import numpy as np
import pytest
from scipy.special import expit

import fixtures as F
import oracle as O
from fixtures import workloads as W

PREFILL_TOL = 1e-2


def _q8(v: np.ndarray, block: int) -> np.ndarray:
    """Symmetric int8 with one scale per `block` consecutive values (absmax / 127), round to nearest."""
    vb = v.reshape(-1, block)
    s = np.abs(vb).max(axis=1, keepdims=True) / 127.0
    s[s == 0] = 1.0
    return (np.clip(np.rint(vb / s), -127, 127) * s).reshape(v.shape)


def _bf16(a: np.ndarray) -> np.ndarray:
    return F.bf16_bits_to_f32(F.to_bf16_bits(a.astype(np.float32))).astype(np.float64)


@pytest.fixture(scope="module")
def layer():
    wl = W.QWEN3_PREFILL
    H, I, n = wl.H, wl.I, wl.H * wl.I
    nb = n // 256 * 144
    mats = []
    for b in W.expert_blobs(wl, experts=range(8)):
        g = O.dequant(O.Q4K, b[:nb], n).reshape(I, H)
        u = O.dequant(O.Q4K, b[nb:2 * nb], n).reshape(I, H)
        d = O.dequant(O.Q4K, b[2 * nb:], n).reshape(H, I)
        mats.append((g, u, d))
    rng = np.random.default_rng(5)
    T, k = 12, 4
    x = _bf16(rng.normal(size=(T, H)))
    sel = np.stack([rng.choice(8, k, replace=False) for _ in range(T)])
    w = rng.dirichlet(np.ones(k), size=T)
    return mats, x, sel, w


def _row_errors(layer, fx, fh, fw=lambda a: a) -> np.ndarray:
    mats, x, sel, w = layer
    errs = []
    for t in range(x.shape[0]):
        y, ye = np.zeros(x.shape[1]), np.zeros(x.shape[1])
        for j, e in enumerate(sel[t]):
            g, u, d = mats[e]
            ge, ue = g @ x[t], u @ x[t]
            ye += w[t, j] * (d @ (ge * expit(ge) * ue))
            xq = fx(x[t])
            gq, uq = fw(g) @ xq, fw(u) @ xq
            y += w[t, j] * (fw(d) @ fh(gq * expit(gq) * uq))
        errs.append(np.abs(y - ye).max() / np.abs(ye).max())
    return np.array(errs)


@pytest.mark.parametrize("block", [2048, 256, 32])
def test_int8_activations_exceed_the_prefill_tolerance(layer, block):
    err = _row_errors(layer, lambda v: _q8(v, block), lambda v: _q8(v, min(block, v.size)))
    print(f"x and h int8, one scale per {block}: max per-row error {err.max():.3e}, median {np.median(err):.3e}")
    assert err.max() > PREFILL_TOL, err.max()


def test_int8_x_alone_exceeds_it(layer):
    """Only the gate/up GEMM's input quantized, one scale per 32 elements (the
    Q4_K sub-block, as an int8 MFMA per sub-block would take it), weights and
    h exact: still over the bound on some row."""
    err = _row_errors(layer, lambda v: _q8(v, 32), lambda v: v)
    print(f"x int8 per 32, weights and h exact: max per-row error {err.max():.3e}, median {np.median(err):.3e}")
    assert err.max() > PREFILL_TOL, err.max()


def test_bf16_rounding_model_stays_inside_it(layer):
    err = _row_errors(layer, lambda v: v, _bf16, _bf16)
    print(f"bf16 model: max per-row error {err.max():.3e}, median {np.median(err):.3e}")
    assert err.max() < PREFILL_TOL, err.max()
