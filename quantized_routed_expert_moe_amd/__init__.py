"""Python binding of libqmoe (include/qmoe.h): one routed-expert MoE layer on MI355X.

Argument marshalling only: every function here has the name of a C entry
point, checks that the tensors it is given are contiguous device tensors of
the right dtype, and passes their addresses, the sizes and the current HIP
stream to the library.  All compute runs in the library's HIP kernels.  If
the library is not built the first call raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqmoe.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "qmoe.h")

MOE_OK, MOE_ERR_INVALID_ARGUMENT, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE_TOO_SMALL, MOE_ERR_HIP = range(5)
MOE_SCORE_SOFTMAX, MOE_SCORE_SIGMOID = 0, 1
MOE_F32, MOE_BF16 = 0, 1
MOE_PATH_AUTO, MOE_PATH_DECODE, MOE_PATH_PREFILL, MOE_PATH_PREFILL_I8 = 0, 1, 2, 3
MOE_FMT_Q8_0, MOE_FMT_Q4K, MOE_FMT_MXFP4, MOE_FMT_Q3K_Q4K, MOE_FMT_Q5K, MOE_FMT_Q6K = 0, 1, 2, 3, 4, 5
# (MOE_FMT_Q3K_Q4K: Q3_K gate and up, Q4_K down)
STAGES = ("route", "batches", "prefill_tiles", "ffn_gateup", "ffn_down", "combine", "prefill_gateup", "prefill_down",
          "route_batches")


class QmoeError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        super().__init__(f"{_status_name(status)}: {message}")


_lib = None


def lib() -> ctypes.CDLL:
    """Load libqmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
        L = ctypes.CDLL(LIB_PATH)
        i32, f32, vp, sz = ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
        L.moe_status_name.argtypes = [i32]
        L.moe_status_name.restype = ctypes.c_char_p
        L.moe_last_error.restype = ctypes.c_char_p
        L.moe_route_topk.argtypes = [vp, i32, i32, i32, i32, i32, f32, vp, vp, vp]
        L.moe_batches_workspace_size.argtypes = [i32, i32, i32, i32]
        L.moe_batches_workspace_size.restype = sz
        L.moe_build_expert_batches.argtypes = [vp, vp, i32, i32, i32, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                               vp]
        L.moe_route_and_batch.argtypes = [vp, i32, i32, i32, i32, i32, f32, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp,
                                          vp, vp, vp, vp, sz, vp]
        L.moe_count_routes.argtypes = [vp, i32, i32, i32, vp, vp]
        L.moe_expert_blob_bytes.argtypes = [i32, i32, i32]
        L.moe_expert_blob_bytes.restype = sz
        L.moe_packed_blob_bytes.argtypes = [i32, i32, i32]
        L.moe_packed_blob_bytes.restype = sz
        L.moe_pack_expert.argtypes = [i32, vp, vp, i32, i32]
        L.moe_unpack_expert.argtypes = [i32, vp, vp, i32, i32]
        L.moe_pack_q4k.argtypes = [vp, vp, i32, i32, i32]
        L.moe_pack_q8_0.argtypes = [vp, vp, i32, i32, i32]
        L.moe_validate_slot_map.argtypes = [vp, i32, i32]
        L.moe_ffn_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32]
        L.moe_ffn_workspace_size.restype = sz
        ffn = [vp, sz, i32, i32, i32, vp, i32, i32, i32, vp, vp, vp, vp, vp, i32, i32, vp, sz, vp]
        L.moe_expert_ffn_q4k.argtypes = ffn
        L.moe_expert_ffn_q8_0.argtypes = ffn
        L.moe_expert_ffn_mxfp4.argtypes = ffn
        L.moe_expert_ffn_q3k_q4k.argtypes = ffn
        L.moe_expert_ffn_q5k.argtypes = ffn
        L.moe_expert_ffn_q6k.argtypes = ffn
        L.moe_expert_ffn_q4k_noalloc.argtypes = ffn[:16] + [vp]
        L.moe_combine.argtypes = [vp, i32, vp, vp, vp, i32, i32, vp, i32, i32, i32, vp, i32, vp]
        L.moe_layer_decode_workspace_size.argtypes = [i32] * 8
        L.moe_layer_decode_workspace_size.restype = sz
        L.moe_layer_decode.argtypes = [i32, vp, vp, i32, i32, i32, i32, i32, i32, f32, vp, i32, vp, sz, i32, i32, vp,
                                       i32] + \
            [vp] * 13 + [vp, sz, vp]
        L.moe_timer_begin.argtypes = [i32, i32]
        L.moe_timer_end.argtypes = [i32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int)]
        L.moe_timer_read.argtypes = [i32, vp, i32, ctypes.POINTER(ctypes.c_int)]
        L.moe_hbm_read_probe.argtypes = [vp, sz, i32, i32, vp, ctypes.POINTER(ctypes.c_size_t), vp]
        L.moe_prefill_inner_probe.argtypes = [i32, i32, vp, sz, vp]
        for name in ("moe_route_topk", "moe_build_expert_batches", "moe_route_and_batch", "moe_count_routes",
                     "moe_pack_expert", "moe_unpack_expert", "moe_pack_q4k", "moe_pack_q8_0",
                     "moe_validate_slot_map", "moe_expert_ffn_q4k", "moe_expert_ffn_q8_0", "moe_expert_ffn_mxfp4",
                     "moe_expert_ffn_q3k_q4k", "moe_expert_ffn_q5k", "moe_expert_ffn_q6k", "moe_expert_ffn_q4k_noalloc",
                     "moe_combine", "moe_layer_decode",
                     "moe_timer_begin", "moe_timer_end", "moe_timer_read", "moe_hbm_read_probe",
                     "moe_prefill_inner_probe"):
            getattr(L, name).restype = i32
        _lib = L
    return _lib


def header_functions(header: str | None = None) -> list[str]:
    """Names of the functions a header declares (default include/qmoe.h)."""
    text = open(header or HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def _status_name(st: int) -> str:
    return lib().moe_status_name(st).decode()


def _check(st: int) -> None:
    if st != MOE_OK:
        raise QmoeError(st, lib().moe_last_error().decode())


# ------------------------------------------------------------ marshalling

def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(t, dtypes=None, name="tensor") -> int:
    if t is None:
        return 0
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    return t.data_ptr()


_MAPPED = {}  # pinned host allocation base -> its device address


def _dev_or_mapped(t, dtypes=None, name="tensor") -> int:
    """Device address of a device tensor, or of a pinned host tensor (the
    device-side address of its pinned allocation from hipHostGetDevicePointer;
    an allocation the device cannot address raises here, before any launch)."""
    import torch
    if isinstance(t, torch.Tensor) and not t.is_cuda and t.is_pinned():
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if dtypes is not None and t.dtype not in dtypes:
            raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
        base = t.untyped_storage().data_ptr()
        if base not in _MAPPED:
            hip = ctypes.CDLL("libamdhip64.so")
            dptr = ctypes.c_void_p()
            rc = hip.hipHostGetDevicePointer(ctypes.byref(dptr), ctypes.c_void_p(base), 0)
            if rc != 0 or not dptr.value:
                raise QmoeError(MOE_ERR_HIP, f"{name}: pinned host memory has no device address (hip error {rc})")
            _MAPPED[base] = dptr.value
        return _MAPPED[base] + (t.data_ptr() - base)
    return _dev(t, dtypes, name)


def _stream(stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _i32():
    import torch
    return (torch.int32,)


def _f32():
    import torch
    return (torch.float32,)


def _fb():
    import torch
    return (torch.float32, torch.bfloat16)


def _u32():
    """Counters: uint32 in the ABI; an int32 tensor holds the same bits."""
    import torch
    return tuple(t for t in (torch.int32, getattr(torch, "uint32", None)) if t is not None)


# ------------------------------------------------------------------ calls

def moe_route_topk(logits, k: int, score: int, renormalize: bool, scale: float, topk_ids, topk_w, stream=None):
    T, E = logits.shape
    _check(lib().moe_route_topk(_dev(logits, _f32(), "logits"), T, E, k, score, int(bool(renormalize)), float(scale),
                                _dev(topk_ids, _i32(), "topk_ids"), _dev(topk_w, _f32(), "topk_w"),
                                _stream(stream)))


def moe_batches_workspace_size(T: int, k: int, E: int, S: int) -> int:
    return int(lib().moe_batches_workspace_size(T, k, E, S))


def moe_build_expert_batches(topk_ids, topk_w, E: int, slot_of_expert, S: int, slot_offsets, active_slots, num_active,
                             perm_pair, host_token, host_expert, host_weight, host_count, ws=None, stream=None):
    T, k = topk_ids.shape
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().moe_build_expert_batches(
        _dev(topk_ids, _i32(), "topk_ids"), _dev(topk_w, _f32(), "topk_w"), T, k, E,
        _dev(slot_of_expert, _i32(), "slot_of_expert"), S, _dev(slot_offsets, _i32(), "slot_offsets"),
        _dev(active_slots, _i32(), "active_slots"), _dev(num_active, _i32(), "num_active"),
        _dev(perm_pair, _i32(), "perm_pair"), _dev_or_mapped(host_token, _i32(), "host_token"),
        _dev_or_mapped(host_expert, _i32(), "host_expert"), _dev_or_mapped(host_weight, _f32(), "host_weight"),
        _dev_or_mapped(host_count, _i32(), "host_count"), _dev(ws, None, "ws"), ws_bytes, _stream(stream)))


def moe_route_and_batch(logits, k: int, score: int, renormalize: bool, scale: float, topk_ids, topk_w, E: int,
                        slot_of_expert, S: int, slot_offsets, active_slots, num_active, perm_pair, host_token,
                        host_expert, host_weight, host_count, ws=None, stream=None, route_counts=None):
    """route_counts: optional device int32/uint32 [E] routing counters (each
    pair adds one to its expert)."""
    T, E_ = logits.shape
    if E_ != E:
        raise ValueError(f"logits have {E_} experts, E = {E}")
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().moe_route_and_batch(
        _dev(logits, _f32(), "logits"), T, E, k, score, int(bool(renormalize)), float(scale),
        _dev(topk_ids, _i32(), "topk_ids"), _dev(topk_w, _f32(), "topk_w"),
        _dev(slot_of_expert, _i32(), "slot_of_expert"), S, _dev(slot_offsets, _i32(), "slot_offsets"),
        _dev(active_slots, _i32(), "active_slots"), _dev(num_active, _i32(), "num_active"),
        _dev(perm_pair, _i32(), "perm_pair"), _dev_or_mapped(host_token, _i32(), "host_token"),
        _dev_or_mapped(host_expert, _i32(), "host_expert"), _dev_or_mapped(host_weight, _f32(), "host_weight"),
        _dev_or_mapped(host_count, _i32(), "host_count"), _dev(route_counts, _u32(), "route_counts"),
        _dev(ws, None, "ws"), ws_bytes, _stream(stream)))


def moe_count_routes(topk_ids, E: int, counts, stream=None):
    """counts[e] += pairs of topk_ids [T, k] routed to e (device, int32/uint32 [E])."""
    T, k = topk_ids.shape
    if counts is None:
        raise ValueError("counts must be a device tensor")
    _check(lib().moe_count_routes(_dev(topk_ids, _i32(), "topk_ids"), T, k, E, _dev(counts, _u32(), "counts"),
                                  _stream(stream)))


def moe_expert_blob_bytes(fmt: int, H: int, I: int) -> int:
    return int(lib().moe_expert_blob_bytes(fmt, H, I))


def moe_packed_blob_bytes(fmt: int, H: int, I: int) -> int:
    """Bytes of a packed blob (a slot's minimum size)."""
    return int(lib().moe_packed_blob_bytes(fmt, H, I))


def moe_pack_expert(fmt: int, canonical: np.ndarray, H: int, I: int, out: np.ndarray | None = None) -> np.ndarray:
    n = moe_expert_blob_bytes(fmt, H, I)
    canonical = np.ascontiguousarray(canonical, dtype=np.uint8)
    if canonical.nbytes != n:
        raise ValueError(f"canonical blob has {canonical.nbytes} bytes, expected {n}")
    npk = moe_packed_blob_bytes(fmt, H, I)
    if out is None:
        out = np.empty(npk, dtype=np.uint8)
    if out.nbytes != npk or not out.flags.c_contiguous:
        raise ValueError(f"out must be a contiguous {npk}-byte array")
    _check(lib().moe_pack_expert(fmt, canonical.ctypes.data, out.ctypes.data, H, I))
    return out


def moe_unpack_expert(fmt: int, packed: np.ndarray, H: int, I: int) -> np.ndarray:
    n, npk = moe_expert_blob_bytes(fmt, H, I), moe_packed_blob_bytes(fmt, H, I)
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    if packed.nbytes != npk:
        raise ValueError(f"packed blob has {packed.nbytes} bytes, expected {npk}")
    out = np.empty(n, dtype=np.uint8)
    _check(lib().moe_unpack_expert(fmt, packed.ctypes.data, out.ctypes.data, H, I))
    return out


def _pack_matrix(fn, block_w: int, block_b: int, canonical: np.ndarray, rows: int, cols: int,
                 gate_up_interleave: bool) -> np.ndarray:
    n = rows * cols * (2 if gate_up_interleave else 1) // block_w * block_b
    canonical = np.ascontiguousarray(canonical, dtype=np.uint8)
    if canonical.nbytes != n:
        raise ValueError(f"canonical matrix data has {canonical.nbytes} bytes, expected {n}")
    out = np.empty(n, dtype=np.uint8)
    _check(fn(canonical.ctypes.data, out.ctypes.data, rows, cols, int(bool(gate_up_interleave))))
    return out


def moe_pack_q4k(canonical: np.ndarray, rows: int, cols: int, gate_up_interleave: bool) -> np.ndarray:
    """Device layout of one Q4_K matrix [rows, cols] (or of W_gate | W_up with gate_up_interleave)."""
    return _pack_matrix(lib().moe_pack_q4k, 256, 144, canonical, rows, cols, gate_up_interleave)


def moe_pack_q8_0(canonical: np.ndarray, rows: int, cols: int, gate_up_interleave: bool) -> np.ndarray:
    """Device layout of one Q8_0 matrix [rows, cols] (or of W_gate | W_up with gate_up_interleave)."""
    return _pack_matrix(lib().moe_pack_q8_0, 32, 34, canonical, rows, cols, gate_up_interleave)


def moe_validate_slot_map(slot_of_expert: np.ndarray, S: int) -> None:
    soe = np.ascontiguousarray(slot_of_expert, dtype=np.int32)
    _check(lib().moe_validate_slot_map(soe.ctypes.data, soe.size, S))


def moe_ffn_workspace_size(fmt: int, T: int, k: int, H: int, I: int, path: int) -> int:
    return int(lib().moe_ffn_workspace_size(fmt, T, k, H, I, path))


def _ffn(fn, slot_pool, slot_stride: int, S: int, H: int, I: int, x, k: int, slot_offsets, active_slots, num_active,
         perm_pair, y_pairs, path: int, ws, stream):
    T = x.shape[0]
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    pool_ptr = slot_pool if isinstance(slot_pool, int) else _dev(slot_pool, None, "slot_pool")
    _check(fn(pool_ptr, slot_stride, S, H, I, _dev(x, _fb(), "x"), _dtype_code(x), T, k,
              _dev(slot_offsets, _i32(), "slot_offsets"), _dev(active_slots, _i32(), "active_slots"),
              _dev(num_active, _i32(), "num_active"), _dev(perm_pair, _i32(), "perm_pair"),
              _dev(y_pairs, _fb(), "y_pairs"), _dtype_code(y_pairs), path, _dev(ws, None, "ws"), ws_bytes,
              _stream(stream)))


def moe_expert_ffn_q4k(slot_pool, slot_stride, S, H, I, x, k, slot_offsets, active_slots, num_active, perm_pair,
                       y_pairs, path=MOE_PATH_AUTO, ws=None, stream=None):
    _ffn(lib().moe_expert_ffn_q4k, slot_pool, slot_stride, S, H, I, x, k, slot_offsets, active_slots, num_active,
         perm_pair, y_pairs, path, ws, stream)


def moe_expert_ffn_q4k_noalloc(slot_pool, slot_stride, S, H, I, x, k, slot_offsets, active_slots, num_active,
                               perm_pair, y_pairs, path=MOE_PATH_AUTO, stream=None):
    """moe_expert_ffn_q4k with the library's own scratch as its workspace (no allocation)."""
    T = x.shape[0]
    pool_ptr = slot_pool if isinstance(slot_pool, int) else _dev(slot_pool, None, "slot_pool")
    _check(lib().moe_expert_ffn_q4k_noalloc(
        pool_ptr, slot_stride, S, H, I, _dev(x, _fb(), "x"), _dtype_code(x), T, k,
        _dev(slot_offsets, _i32(), "slot_offsets"), _dev(active_slots, _i32(), "active_slots"),
        _dev(num_active, _i32(), "num_active"), _dev(perm_pair, _i32(), "perm_pair"), _dev(y_pairs, _fb(), "y_pairs"),
        _dtype_code(y_pairs), path, _stream(stream)))


MOE_NOALLOC_SCRATCH_BYTES = 64 << 20


def moe_expert_ffn_q8_0(slot_pool, slot_stride, S, H, I, x, k, slot_offsets, active_slots, num_active, perm_pair,
                        y_pairs, path=MOE_PATH_AUTO, ws=None, stream=None):
    _ffn(lib().moe_expert_ffn_q8_0, slot_pool, slot_stride, S, H, I, x, k, slot_offsets, active_slots, num_active,
         perm_pair, y_pairs, path, ws, stream)


def moe_expert_ffn_mxfp4(slot_pool, slot_stride, S, H, I, x, k, slot_offsets, active_slots, num_active, perm_pair,
                         y_pairs, path=MOE_PATH_AUTO, ws=None, stream=None):
    _ffn(lib().moe_expert_ffn_mxfp4, slot_pool, slot_stride, S, H, I, x, k, slot_offsets, active_slots, num_active,
         perm_pair, y_pairs, path, ws, stream)


def moe_expert_ffn_q3k_q4k(slot_pool, slot_stride, S, H, I, x, k, slot_offsets, active_slots, num_active, perm_pair,
                           y_pairs, path=MOE_PATH_AUTO, ws=None, stream=None):
    _ffn(lib().moe_expert_ffn_q3k_q4k, slot_pool, slot_stride, S, H, I, x, k, slot_offsets, active_slots, num_active,
         perm_pair, y_pairs, path, ws, stream)


def moe_expert_ffn_q5k(slot_pool, slot_stride, S, H, I, x, k, slot_offsets, active_slots, num_active, perm_pair,
                       y_pairs, path=MOE_PATH_AUTO, ws=None, stream=None):
    _ffn(lib().moe_expert_ffn_q5k, slot_pool, slot_stride, S, H, I, x, k, slot_offsets, active_slots, num_active,
         perm_pair, y_pairs, path, ws, stream)


def moe_expert_ffn_q6k(slot_pool, slot_stride, S, H, I, x, k, slot_offsets, active_slots, num_active, perm_pair,
                       y_pairs, path=MOE_PATH_AUTO, ws=None, stream=None):
    _ffn(lib().moe_expert_ffn_q6k, slot_pool, slot_stride, S, H, I, x, k, slot_offsets, active_slots, num_active,
         perm_pair, y_pairs, path, ws, stream)


def moe_expert_ffn(fmt: int):
    """The expert-FFN call of a block format."""
    return {MOE_FMT_Q8_0: moe_expert_ffn_q8_0, MOE_FMT_Q4K: moe_expert_ffn_q4k, MOE_FMT_MXFP4: moe_expert_ffn_mxfp4,
            MOE_FMT_Q3K_Q4K: moe_expert_ffn_q3k_q4k, MOE_FMT_Q5K: moe_expert_ffn_q5k,
            MOE_FMT_Q6K: moe_expert_ffn_q6k}[fmt]


def moe_combine(y_pairs, topk_ids, topk_w, slot_of_expert, S: int, y_shared, y, stream=None):
    T, k = topk_ids.shape
    H = y.shape[1]
    E = slot_of_expert.numel()
    _check(lib().moe_combine(_dev(y_pairs, _fb(), "y_pairs"), _dtype_code(y_pairs), _dev(topk_ids, _i32(), "topk_ids"),
                             _dev(topk_w, _f32(), "topk_w"), _dev(slot_of_expert, _i32(), "slot_of_expert"), E, S,
                             _dev(y_shared, _f32(), "y_shared"), T, k, H, _dev(y, _fb(), "y"), _dtype_code(y),
                             _stream(stream)))


def moe_layer_decode_workspace_size(fmt: int, T: int, k: int, E: int, S: int, H: int, I: int, I_shared: int) -> int:
    return int(lib().moe_layer_decode_workspace_size(fmt, T, k, E, S, H, I, I_shared))


def moe_layer_decode(fmt: int, logits, x, k: int, score: int, renormalize: bool, scale: float, slot_of_expert, S: int,
                     slot_pool, slot_stride: int, I: int, shared_pool, I_shared: int, topk_ids, topk_w, slot_offsets,
                     active_slots, num_active, perm_pair, host_token, host_expert, host_weight, host_count, y_pairs, y,
                     ws, stream=None, route_counts=None):
    """The whole decode layer (routing, batching, routed and shared expert FFN, combine) in one call."""
    T, E = logits.shape
    H = x.shape[1]
    pool_ptr = slot_pool if isinstance(slot_pool, int) else _dev(slot_pool, None, "slot_pool")
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().moe_layer_decode(
        fmt, _dev(logits, _f32(), "logits"), _dev(x, _fb(), "x"), _dtype_code(x), T, E, k, score, int(bool(renormalize)),
        float(scale), _dev(slot_of_expert, _i32(), "slot_of_expert"), S, pool_ptr, slot_stride, H, I,
        _dev(shared_pool, None, "shared_pool"), I_shared if shared_pool is not None else 0,
        _dev(topk_ids, _i32(), "topk_ids"), _dev(topk_w, _f32(), "topk_w"), _dev(slot_offsets, _i32(), "slot_offsets"),
        _dev(active_slots, _i32(), "active_slots"), _dev(num_active, _i32(), "num_active"),
        _dev(perm_pair, _i32(), "perm_pair"), _dev_or_mapped(host_token, _i32(), "host_token"),
        _dev_or_mapped(host_expert, _i32(), "host_expert"), _dev_or_mapped(host_weight, _f32(), "host_weight"),
        _dev_or_mapped(host_count, _i32(), "host_count"), _dev(route_counts, _u32(), "route_counts"),
        _dev(y_pairs, _f32(), "y_pairs"), _dev(y, _f32(), "y"), _dev(ws, None, "ws"), ws_bytes, _stream(stream)))


# ------------------------------------------------------------ host leg

HOST_LIB_PATH = os.path.join(_HERE, "libqmoe_host.so")
_host_lib = None


def host_lib() -> ctypes.CDLL:
    """libqmoe_host.so: the CPU expert FFN for the pairs the card does not
    hold, and the adaptive residency policy (include/qmoe_host.h)."""
    global _host_lib
    if _host_lib is None:
        if not os.path.exists(HOST_LIB_PATH):
            raise ImportError(f"{HOST_LIB_PATH} is not built; run __graft_entry__.build() first")
        L = ctypes.CDLL(HOST_LIB_PATH)
        vp = ctypes.c_void_p
        i32 = ctypes.c_int
        L.moe_host_leg.argtypes = [i32, vp, i32, i32, i32, vp, i32, vp, vp, vp, i32, vp, i32]
        L.moe_host_leg.restype = i32
        L.moe_host_last_error.restype = ctypes.c_char_p
        L.moe_residency_update_scores.argtypes = [vp, vp, i32, i32]
        L.moe_residency_update_scores.restype = i32
        L.moe_residency_plan.argtypes = [vp, i32, vp, i32, ctypes.c_uint64, vp, vp, vp]
        L.moe_residency_plan.restype = i32
        _host_lib = L
    return _host_lib


def moe_host_leg(fmt: int, expert_blobs, H: int, I: int, x: np.ndarray, host_token, host_expert, host_weight,
                 threads: int = 0, out: np.ndarray | None = None) -> np.ndarray:
    """y_host [T, H] fp32 of the listed (token, expert, weight) pairs.
    expert_blobs: E entries, each a canonical blob (uint8 array) or None."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    T = x.shape[0]
    tok = np.ascontiguousarray(host_token, dtype=np.int32)
    exp = np.ascontiguousarray(host_expert, dtype=np.int32)
    wt = np.ascontiguousarray(host_weight, dtype=np.float32)
    if not (tok.shape == exp.shape == wt.shape) or tok.ndim != 1:
        raise ValueError("host_token, host_expert and host_weight must be 1-D of equal length")
    E = len(expert_blobs)
    keep = []
    ptrs = (ctypes.c_void_p * max(E, 1))()
    for e, b in enumerate(expert_blobs):
        if b is not None:
            b = np.ascontiguousarray(b, dtype=np.uint8)
            keep.append(b)
            ptrs[e] = b.ctypes.data
    y = np.empty((T, H), dtype=np.float32) if out is None else out
    if y.shape != (T, H) or y.dtype != np.float32 or not y.flags.c_contiguous:
        raise ValueError("out must be a contiguous float32 [T, H] array")
    st = host_lib().moe_host_leg(fmt, ctypes.cast(ptrs, ctypes.c_void_p), E, H, I, x.ctypes.data, T,
                                 tok.ctypes.data, exp.ctypes.data, wt.ctypes.data, int(tok.size), y.ctypes.data,
                                 int(threads))
    if st != 0:
        raise QmoeError(st, host_lib().moe_host_last_error().decode())
    return y


RESIDENCY_FRAC_BITS = 16  # MOE_RESIDENCY_FRAC_BITS


def moe_residency_update_scores(score: np.ndarray, window, decay_shift: int) -> np.ndarray:
    """score (uint64 [E], updated in place) <- score - (score >> decay_shift)
    + (window << 16); window: uint32 [E] pairs routed since the last update."""
    if score.dtype != np.uint64 or score.ndim != 1 or not score.flags.c_contiguous:
        raise ValueError("score must be a contiguous uint64 [E] array")
    win = np.ascontiguousarray(window, dtype=np.uint32)
    if win.shape != score.shape:
        raise ValueError("window must have the shape of score")
    st = host_lib().moe_residency_update_scores(score.ctypes.data, win.ctypes.data, int(score.size), int(decay_shift))
    if st != 0:
        raise QmoeError(st, host_lib().moe_host_last_error().decode())
    return score


def moe_residency_plan(score, slot_of_expert, max_swaps: int, margin: int = 0) -> tuple[list, list]:
    """(incoming, outgoing) experts of one layer's swap plan."""
    sc = np.ascontiguousarray(score, dtype=np.uint64)
    soe = np.ascontiguousarray(slot_of_expert, dtype=np.int32)
    if sc.ndim != 1 or soe.shape != sc.shape:
        raise ValueError("score and slot_of_expert must be 1-D of equal length")
    m = max(int(max_swaps), 0)
    inc = np.zeros(max(m, 1), dtype=np.int32)
    out = np.zeros(max(m, 1), dtype=np.int32)
    n = ctypes.c_int(0)
    st = host_lib().moe_residency_plan(sc.ctypes.data, int(sc.size), soe.ctypes.data, int(max_swaps), int(margin),
                                       inc.ctypes.data, out.ctypes.data, ctypes.byref(n))
    if st != 0:
        raise QmoeError(st, host_lib().moe_host_last_error().decode())
    return inc[:n.value].tolist(), out[:n.value].tolist()


def moe_timer_begin(stage: int, capacity: int) -> None:
    _check(lib().moe_timer_begin(stage, capacity))


def moe_timer_read(stage: int, capacity: int) -> np.ndarray:
    """Kernel milliseconds of each launch timed so far (the timer stays armed)."""
    out = np.zeros(max(int(capacity), 1), dtype=np.float32)
    n = ctypes.c_int(0)
    _check(lib().moe_timer_read(stage, out.ctypes.data, int(capacity), ctypes.byref(n)))
    return out[:min(n.value, int(capacity))].copy()


def moe_hbm_read_probe(buf, waves: int, depth: int, sink, stream=None) -> int:
    """One pass of the streaming-read probe over the device tensor buf; returns the bytes read."""
    if sink.numel() * sink.element_size() < 256 * int(waves):
        raise ValueError(f"sink holds fewer than waves x 64 words ({waves} waves)")
    n = ctypes.c_size_t(0)
    _check(lib().moe_hbm_read_probe(_dev(buf, name="buf"), buf.numel() * buf.element_size(), int(waves), int(depth),
                                    _dev(sink, name="sink"), ctypes.byref(n),
                                    _stream(stream)))
    return n.value


PREFILL_PROBE_OUT_FLOATS = 131072  # MOE_PREFILL_PROBE_OUT_FLOATS


def moe_prefill_inner_probe(variant: int, sub_blocks: int, out, stream=None) -> float:
    """One launch of the prefill inner-loop probe (variant 0: bf16
    dequantization + bf16 MFMA; 1: int8 MFMA + fp32 rescaling per
    sub-block; 2: variant 1 with two int8 activation planes); returns the
    flops the launch stands for."""
    import torch
    ptr = _dev(out, (torch.float32,), name="out")
    _check(lib().moe_prefill_inner_probe(int(variant), int(sub_blocks), ptr, out.numel(), _stream(stream)))
    return 1024.0 * int(sub_blocks) * 2 * 256 * 64 * 32


def moe_timer_end(stage: int) -> tuple[float, int]:
    ms = ctypes.c_double(0.0)
    n = ctypes.c_int(0)
    _check(lib().moe_timer_end(stage, ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value
