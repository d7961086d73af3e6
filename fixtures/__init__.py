"""Seeded synthetic inputs for the routed-expert MoE layer (shared by both sides).

This package draws the random inputs and writes them in the stored block
formats.  It contains none of the layer's arithmetic (no dequantization,
routing, grouping, FFN or combine); see ``fixtures.c`` for the generators and
their published definitions.  Both the HIP path (tests, bench) and the CPU
oracle (tests) consume what it returns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fixtures.c")
_SO = os.path.join(_HERE, "libqmoe_fixtures.so")

Q8_0 = 0
Q4K = 1
MXFP4 = 2
Q3K_Q4K = 3  # mixed expert: Q3_K gate and up, Q4_K down
Q3K = 100  # block type of a Q3_K matrix (the mixed expert's gate and up)
Q5K = 4
Q6K = 5

# Counter-stream tags (the second Philox key word) of the non-weight inputs.
TAG_X = 0x58000000
TAG_SHARED_EXPERT = 0x10000  # expert id used for the always-on shared expert's weights

_lib = None


def build() -> str:
    """Compile the generator library with gcc (OpenMP; no fast-math and no FMA
    contraction, so vector and scalar loop iterations round identically)."""
    cmd = ["gcc", "-O3", "-std=c11", "-march=x86-64-v3", "-ffp-contract=off", "-fno-math-errno", "-fopenmp", "-fPIC",
           "-shared", _SRC, "-o", _SO + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_SO + ".tmp", _SO)
    return _SO


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        u32, i32, i64, f32, f64 = ctypes.c_uint32, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_double
        vp = ctypes.c_void_p
        L.fx_philox4x32_10.argtypes = [vp, vp, vp]
        L.fx_f32_to_f16.argtypes = [f32]
        L.fx_f32_to_f16.restype = ctypes.c_uint16
        L.fx_f16_to_f32.argtypes = [ctypes.c_uint16]
        L.fx_f16_to_f32.restype = f32
        L.fx_f32_to_bf16_array.argtypes = [vp, vp, i64]
        L.fx_encode_q8_0.argtypes = [vp, i64, vp]
        L.fx_encode_q4k.argtypes = [vp, i64, vp]
        L.fx_encode_mxfp4.argtypes = [vp, i64, vp]
        L.fx_encode_q3k.argtypes = [vp, i64, vp]
        L.fx_encode_q5k.argtypes = [vp, i64, vp]
        L.fx_encode_q6k.argtypes = [vp, i64, vp]
        L.fx_matrix_bytes.argtypes = [i32, i64, i64]
        L.fx_matrix_bytes.restype = i64
        L.fx_expert_bytes.argtypes = [i32, i64, i64]
        L.fx_expert_bytes.restype = i64
        L.fx_gen_expert.argtypes = [i32, u32, u32, u32, i64, i64, f32, vp]
        L.fx_gen_experts.argtypes = [i32, u32, u32, vp, i32, i64, i64, f32, vp]
        L.fx_gen_matrix_f32.argtypes = [u32, u32, u32, u32, i64, i64, f32, vp]
        L.fx_normal_rows.argtypes = [u32, u32, u32, i64, i64, f32, f32, vp]
        L.fx_logits_normal.argtypes = [u32, u32, i64, i32, vp]
        L.fx_permutation.argtypes = [u32, u32, i32, vp]
        L.fx_logits_zipf.argtypes = [u32, u32, u32, i64, i32, f64, vp]
        L.fx_num_threads.restype = i32
        L.fx_set_num_threads.argtypes = [i32]
        _lib = L
    return _lib


def _p(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def philox4x32_10(ctr, key) -> np.ndarray:
    c = np.ascontiguousarray(np.asarray(ctr, dtype=np.uint32))
    k = np.ascontiguousarray(np.asarray(key, dtype=np.uint32))
    out = np.zeros(4, dtype=np.uint32)
    lib().fx_philox4x32_10(_p(c), _p(k), _p(out))
    return out


def f32_to_f16_bits(v: float) -> int:
    return int(lib().fx_f32_to_f16(float(v)))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 array -> bfloat16 bit patterns (uint16), round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().fx_f32_to_bf16_array(_p(x), _p(out), x.size)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def encode(fmt: int, x: np.ndarray) -> np.ndarray:
    """Encode a float32 row-major matrix (last dim a multiple of the block size) into stored blocks."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    cols = x.shape[-1]
    rows = x.size // cols
    if cols % (256 if fmt in (Q4K, Q3K, Q5K, Q6K) else 32) != 0:
        raise ValueError(f"row length {cols} is not a whole number of blocks")
    out = np.empty(lib().fx_matrix_bytes(fmt, rows, cols), dtype=np.uint8)
    enc = {Q8_0: lib().fx_encode_q8_0, Q4K: lib().fx_encode_q4k, MXFP4: lib().fx_encode_mxfp4,
           Q3K: lib().fx_encode_q3k, Q5K: lib().fx_encode_q5k, Q6K: lib().fx_encode_q6k}[fmt]
    enc(_p(x), x.size, _p(out))
    return out


def matrix_bytes(fmt: int, rows: int, cols: int) -> int:
    return int(lib().fx_matrix_bytes(fmt, rows, cols))


def expert_bytes(fmt: int, H: int, I: int) -> int:
    return int(lib().fx_expert_bytes(fmt, H, I))


def expert_blob(fmt: int, seed: int, layer: int, expert: int, H: int, I: int, std: float = 0.02,
                out: np.ndarray | None = None) -> np.ndarray:
    """Canonical blob W_gate[I,H] | W_up[I,H] | W_down[H,I] of one seeded expert."""
    n = expert_bytes(fmt, H, I)
    if out is None:
        out = np.empty(n, dtype=np.uint8)
    assert out.nbytes == n and out.flags["C_CONTIGUOUS"]
    lib().fx_gen_expert(fmt, seed, layer, expert, H, I, std, _p(out))
    return out


def expert_blobs(fmt: int, seed: int, layer: int, experts, H: int, I: int, std: float = 0.02) -> np.ndarray:
    """[len(experts), blob_bytes] canonical blobs of the listed expert ids (same bytes as expert_blob)."""
    ids = np.ascontiguousarray(np.asarray(list(experts), dtype=np.int32))
    out = np.empty((ids.size, expert_bytes(fmt, H, I)), dtype=np.uint8)
    if ids.size:
        lib().fx_gen_experts(fmt, seed, layer, _p(ids), ids.size, H, I, std, _p(out))
    return out


def matrix_f32(seed: int, layer: int, expert: int, matrix: int, rows: int, cols: int, std: float = 0.02) -> np.ndarray:
    """The float weights an expert's matrix is encoded from (0 gate, 1 up, 2 down)."""
    out = np.empty((rows, cols), dtype=np.float32)
    lib().fx_gen_matrix_f32(seed, layer, expert, matrix, rows, cols, std, _p(out))
    return out


def normal_rows(seed: int, tag: int, layer: int, rows: int, cols: int, mean: float = 0.0, std: float = 1.0) -> np.ndarray:
    out = np.empty((rows, cols), dtype=np.float32)
    lib().fx_normal_rows(seed, tag, layer, rows, cols, mean, std, _p(out))
    return out


def activations(seed: int, layer: int, T: int, H: int) -> np.ndarray:
    """Token activations x ~ N(0,1), float32 [T, H]."""
    return normal_rows(seed, TAG_X, layer, T, H)


def logits_normal(seed: int, layer: int, T: int, E: int) -> np.ndarray:
    """Gate logits ~ N(0,1), float32 [T, E], no two equal values in a row."""
    out = np.empty((T, E), dtype=np.float32)
    lib().fx_logits_normal(seed, layer, T, E, _p(out))
    return out


def permutation(seed: int, layer: int, E: int) -> np.ndarray:
    out = np.empty(E, dtype=np.int32)
    lib().fx_permutation(seed, layer, E, _p(out))
    return out


def logits_zipf(seed: int, layer: int, T: int, E: int, s: float, perm_seed: int | None = None) -> np.ndarray:
    """Gumbel-perturbed Zipf(s) log-probabilities, float32 [T, E], no ties in a row.
    The expert ranking comes from perm_seed (default: seed), the noise from seed."""
    out = np.empty((T, E), dtype=np.float32)
    lib().fx_logits_zipf(seed, seed if perm_seed is None else perm_seed, layer, T, E, float(s), _p(out))
    return out


def num_threads() -> int:
    return int(lib().fx_num_threads())


def set_num_threads(n: int) -> None:
    lib().fx_set_num_threads(int(n))
