"""CPU oracle for one routed-expert MoE layer (fp64, plain C, OpenMP).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are its only users.  The HIP library never loads it, and it
shares no code with the HIP library (see ``oracle.h`` for the definition it
computes and the passages it follows).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_SO = os.path.join(_HERE, "liboracle.so")

Q8_0 = 0
Q4K = 1
MXFP4 = 2
Q3K_Q4K = 3  # mixed expert: Q3_K gate and up, Q4_K down
Q3K = 100  # block type of a Q3_K matrix (the mixed expert's gate and up)
Q5K = 4
Q6K = 5
SOFTMAX = 0
SIGMOID = 1

_lib = None


def build(src: str = _SRC, out: str = _SO) -> str:
    """Compile the oracle (or, for the pin tests' mutants, another version of
    its source) with gcc: -O2, OpenMP, strict IEEE (no fast-math)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-I" + _HERE, src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def _bind(path: str) -> ctypes.CDLL:
    L = ctypes.CDLL(path)
    i32, i64, f64, vp = ctypes.c_int, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
    L.oracle_dequant_q8_0.argtypes = [vp, i64, vp]
    L.oracle_dequant_q4k.argtypes = [vp, i64, vp]
    L.oracle_dequant_mxfp4.argtypes = [vp, i64, vp]
    L.oracle_dequant_q3k.argtypes = [vp, i64, vp]
    L.oracle_dequant_q5k.argtypes = [vp, i64, vp]
    L.oracle_dequant_q6k.argtypes = [vp, i64, vp]
    L.oracle_route.argtypes = [vp, i32, i32, i32, i32, i32, f64, vp, vp]
    L.oracle_route.restype = i32
    L.oracle_batches.argtypes = [vp, vp, i32, i32, i32, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp]
    L.oracle_batches.restype = i32
    L.oracle_expert_ffn.argtypes = [i32, vp, i32, i32, vp, vp]
    L.oracle_moe_layer.argtypes = [i32, vp, i32, i32, i32, i32, vp, vp, i32, i32, i32, f64, vp, i32, i32, vp,
                                   i32, vp, vp, vp, vp]
    L.oracle_moe_layer.restype = i32
    L.oracle_set_threads.argtypes = [i32]
    L.oracle_threads.restype = i32
    return L


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        _lib = _bind(_SO)
    return _lib


class use_library:
    """Context manager for the pin tests: the module's functions call the
    compiled oracle at `path` (a mutant of the source) instead of the
    oracle, until the block ends."""

    def __init__(self, path: str):
        self.path = path

    def __enter__(self):
        global _lib
        self.saved = lib()
        _lib = _bind(self.path)
        return _lib

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def _p(a) -> int:
    if a is None:
        return 0
    assert a.flags["C_CONTIGUOUS"], "arrays passed to the oracle must be contiguous"
    return a.ctypes.data


def set_threads(n: int) -> None:
    lib().oracle_set_threads(int(n))


def threads() -> int:
    return int(lib().oracle_threads())


def dequant(fmt: int, blocks: np.ndarray, n: int) -> np.ndarray:
    blocks = np.ascontiguousarray(blocks, dtype=np.uint8)
    bs, bb = {Q8_0: (32, 34), Q4K: (256, 144), MXFP4: (32, 17), Q3K: (256, 110), Q5K: (256, 176),
              Q6K: (256, 210)}[fmt]
    if n % bs or blocks.nbytes < n // bs * bb:
        raise ValueError("block count does not match n")
    out = np.empty(n, dtype=np.float64)
    fn = {Q8_0: lib().oracle_dequant_q8_0, Q4K: lib().oracle_dequant_q4k, MXFP4: lib().oracle_dequant_mxfp4,
          Q3K: lib().oracle_dequant_q3k, Q5K: lib().oracle_dequant_q5k, Q6K: lib().oracle_dequant_q6k}[fmt]
    fn(_p(blocks), n, _p(out))
    return out


def route(logits: np.ndarray, k: int, score: int = SOFTMAX, renormalize: bool = True, scale: float = 1.0):
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    rc = lib().oracle_route(_p(logits), T, E, k, score, int(bool(renormalize)), float(scale), _p(ids), _p(w))
    if rc != 0:
        raise ValueError("oracle_route: bad sizes")
    return ids, w


def batches(ids: np.ndarray, w: np.ndarray | None, E: int, slot_of_expert: np.ndarray, S: int) -> dict:
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, k = ids.shape
    P = T * k
    soe = np.ascontiguousarray(slot_of_expert, dtype=np.int32)
    wd = None if w is None else np.ascontiguousarray(w, dtype=np.float64)
    out = dict(
        slot_offsets=np.empty(S + 1, dtype=np.int32),
        active_slots=np.full(max(1, min(S, P)), -1, dtype=np.int32),
        num_active=np.zeros(1, dtype=np.int32),
        perm_pair=np.full(max(1, P), -1, dtype=np.int32),
        host_token=np.full(max(1, P), -1, dtype=np.int32),
        host_expert=np.full(max(1, P), -1, dtype=np.int32),
        host_weight=np.zeros(max(1, P), dtype=np.float64),
        host_count=np.zeros(1, dtype=np.int32),
    )
    rc = lib().oracle_batches(_p(ids), _p(wd), T, k, E, _p(soe), S, _p(out["slot_offsets"]), _p(out["active_slots"]),
                              _p(out["num_active"]), _p(out["perm_pair"]), _p(out["host_token"]),
                              _p(out["host_expert"]), _p(out["host_weight"]), _p(out["host_count"]))
    if rc != 0:
        raise ValueError("oracle_batches: bad sizes")
    na, n_res, hc = int(out["num_active"][0]), int(out["slot_offsets"][S]), int(out["host_count"][0])
    out["active_slots"] = out["active_slots"][:na]
    out["perm_pair"] = out["perm_pair"][:n_res]
    for key in ("host_token", "host_expert", "host_weight"):
        out[key] = out[key][:hc]
    return out


def expert_ffn(fmt: int, blob: np.ndarray, H: int, I: int, x: np.ndarray) -> np.ndarray:
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    x = np.ascontiguousarray(x, dtype=np.float64)
    assert x.shape == (H,)
    y = np.empty(H, dtype=np.float64)
    lib().oracle_expert_ffn(fmt, _p(blob), H, I, _p(x), _p(y))
    return y


def moe_layer(fmt: int, expert_blobs, H: int, I: int, x: np.ndarray, logits: np.ndarray, k: int,
              score: int = SOFTMAX, renormalize: bool = True, scale: float = 1.0,
              slot_of_expert: np.ndarray | None = None, shared_blob: np.ndarray | None = None,
              shared_fmt: int = Q8_0, I_shared: int = 0, want_pairs: bool = False, S: int | None = None) -> dict:
    """The whole layer in fp64.  expert_blobs: sequence of E canonical blobs
    (None for an expert that is never selected) or a 2-D uint8 array [E, bytes].
    A pair is on the card iff its expert's slot is in [0, S) (S defaults to E)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    assert x.shape == (T, H)
    keep = []
    ptrs = (ctypes.c_void_p * E)()
    for e in range(E):
        b = expert_blobs[e]
        if b is None:
            ptrs[e] = None
        else:
            b = np.ascontiguousarray(b, dtype=np.uint8)
            keep.append(b)
            ptrs[e] = b.ctypes.data
    soe = np.arange(E, dtype=np.int32) if slot_of_expert is None else np.ascontiguousarray(slot_of_expert, np.int32)
    sb = None if shared_blob is None else np.ascontiguousarray(shared_blob, dtype=np.uint8)
    y = np.empty((T, H), dtype=np.float64)
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    yp = np.empty((T * k, H), dtype=np.float64) if want_pairs else None
    S = E if S is None else int(S)
    rc = lib().oracle_moe_layer(fmt, ctypes.cast(ptrs, ctypes.c_void_p), E, H, I, T, _p(x), _p(logits), k, score,
                                int(bool(renormalize)), float(scale), _p(soe), S, shared_fmt, _p(sb), int(I_shared),
                                _p(y), _p(ids), _p(w), _p(yp))
    if rc != 0:
        raise ValueError(f"oracle_moe_layer failed ({rc})")
    return dict(y=y, ids=ids, w=w, y_pairs=yp)
