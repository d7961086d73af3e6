"""The C-ABI library without a GPU: it loads, exports what the header
declares, packs blobs reversibly and refuses bad arguments by name before
touching the device."""
import ctypes

import numpy as np
import pytest

import fixtures as F
import quantized_routed_expert_moe_amd as Q


def test_library_exports_every_header_function():
    names = Q.header_functions()
    assert "moe_route_topk" in names and "moe_combine" in names and len(names) >= 15
    L = Q.lib()
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing


def test_host_library_exports_every_host_header_function():
    import os
    names = Q.header_functions(os.path.join(os.path.dirname(Q.HEADER_PATH), "qmoe_host.h"))
    assert {"moe_host_leg", "moe_residency_plan", "moe_residency_update_scores"} <= set(names)
    L = Q.host_lib()
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing


def test_status_names():
    assert Q._status_name(0) == "MOE_OK"
    assert Q._status_name(3) == "MOE_ERR_WORKSPACE_TOO_SMALL"
    assert Q._status_name(99) == "MOE_STATUS_UNKNOWN"


def _call(name, *args):
    st = getattr(Q.lib(), name)(*args)
    return st, Q.lib().moe_last_error().decode()


FAKE = 1 << 20  # aligned non-null address; never dereferenced on these paths


@pytest.mark.parametrize("T,E,k,score,want", [
    (-1, 8, 2, 0, Q.MOE_ERR_INVALID_ARGUMENT),
    (4, 0, 1, 0, Q.MOE_ERR_INVALID_ARGUMENT),
    (4, 2000, 2, 0, Q.MOE_ERR_INVALID_ARGUMENT),
    (4, 8, 9, 0, Q.MOE_ERR_INVALID_ARGUMENT),
    (4, 256, 65, 0, Q.MOE_ERR_INVALID_ARGUMENT),
    (4, 8, 0, 0, Q.MOE_ERR_INVALID_ARGUMENT),
    (4, 8, 2, 7, Q.MOE_ERR_INVALID_ARGUMENT),
    (1 << 22, 64, 8, 0, Q.MOE_ERR_INVALID_ARGUMENT),
])
def test_route_rejects(T, E, k, score, want):
    st, msg = _call("moe_route_topk", FAKE, T, E, k, score, 1, ctypes.c_float(1.0), FAKE, FAKE, None)
    assert st == want and msg


def test_route_rejects_null():
    st, msg = _call("moe_route_topk", None, 4, 8, 2, 0, 1, ctypes.c_float(1.0), FAKE, FAKE, None)
    assert st == Q.MOE_ERR_INVALID_ARGUMENT and "NULL" in msg


def _route_batch(T=4, E=8, k=2, score=0, scale=1.0, S=8, ws_bytes=0, logits=FAKE):
    return _call("moe_route_and_batch", logits, T, E, k, score, 1, ctypes.c_float(scale), FAKE, FAKE, FAKE, S, FAKE,
                 FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, ws_bytes, None)


@pytest.mark.parametrize("kw,want,needle", [
    (dict(k=9), Q.MOE_ERR_INVALID_ARGUMENT, ""),
    (dict(score=7), Q.MOE_ERR_INVALID_ARGUMENT, "score"),
    (dict(scale=float("nan")), Q.MOE_ERR_INVALID_ARGUMENT, "NaN"),
    (dict(S=9), Q.MOE_ERR_INVALID_ARGUMENT, "S = 9"),
    (dict(logits=None), Q.MOE_ERR_INVALID_ARGUMENT, "NULL"),
    (dict(T=4096, E=128, k=8, S=128), Q.MOE_ERR_WORKSPACE_TOO_SMALL, "workspace"),
])
def test_route_and_batch_rejects(kw, want, needle):
    st, msg = _route_batch(**kw)
    assert st == want and needle in msg, msg


@pytest.mark.parametrize("T,k,E,ids,counts,needle", [
    (4, 2, 0, FAKE, FAKE, "E = 0"),
    (4, 9, 8, FAKE, FAKE, "k = 9"),
    (4, 2, 8, FAKE, None, "NULL"),
    (4, 2, 8, None, FAKE, "NULL"),
])
def test_count_routes_rejects(T, k, E, ids, counts, needle):
    st, msg = _call("moe_count_routes", ids, T, k, E, counts, None)
    assert st == Q.MOE_ERR_INVALID_ARGUMENT and needle in msg, msg


def test_batches_rejects_bad_slot_count():
    st, msg = _call("moe_build_expert_batches", FAKE, FAKE, 4, 2, 8, FAKE, 9, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                    FAKE, None, 0, None)
    assert st == Q.MOE_ERR_INVALID_ARGUMENT and "S = 9" in msg


def _ffn(name, **kw):
    a = dict(pool=FAKE, stride=Q.moe_expert_blob_bytes(Q.MOE_FMT_Q4K, 2048, 768) // 16 * 16 + 256, S=128, H=2048,
             I=768, x=FAKE, x_dtype=Q.MOE_F32, T=2, k=8, offs=FAKE, act=FAKE, na=FAKE, perm=FAKE, yp=FAKE,
             y_dtype=Q.MOE_F32, path=Q.MOE_PATH_DECODE, ws=FAKE, ws_bytes=1 << 30)
    a.update(kw)
    return _call(name, a["pool"], a["stride"], a["S"], a["H"], a["I"], a["x"], a["x_dtype"], a["T"], a["k"],
                 a["offs"], a["act"], a["na"], a["perm"], a["yp"], a["y_dtype"], a["path"], a["ws"], a["ws_bytes"],
                 None)


@pytest.mark.parametrize("kw,want,needle", [
    (dict(H=2000), Q.MOE_ERR_UNSUPPORTED, "multiples of 256"),
    (dict(I=640), Q.MOE_ERR_UNSUPPORTED, "multiples of 256"),
    (dict(pool=None), Q.MOE_ERR_INVALID_ARGUMENT, "NULL"),
    (dict(pool=FAKE + 8), Q.MOE_ERR_INVALID_ARGUMENT, "aligned"),
    (dict(stride=1024), Q.MOE_ERR_INVALID_ARGUMENT, "smaller than the blob"),
    (dict(S=0), Q.MOE_ERR_INVALID_ARGUMENT, "S = 0"),
    (dict(k=65), Q.MOE_ERR_INVALID_ARGUMENT, "k = 65"),
    (dict(ws_bytes=100), Q.MOE_ERR_WORKSPACE_TOO_SMALL, "workspace"),
    (dict(y_dtype=Q.MOE_BF16), Q.MOE_ERR_UNSUPPORTED, "decode path"),
    (dict(path=7), Q.MOE_ERR_INVALID_ARGUMENT, "bad path"),
    (dict(x_dtype=5), Q.MOE_ERR_INVALID_ARGUMENT, "bad x_dtype"),
    (dict(x=None), Q.MOE_ERR_INVALID_ARGUMENT, "NULL"),
    (dict(perm=None), Q.MOE_ERR_INVALID_ARGUMENT, "NULL"),
    (dict(T=0, offs=None), Q.MOE_ERR_INVALID_ARGUMENT, "NULL"),
])
def test_ffn_q4k_rejects(kw, want, needle):
    st, msg = _ffn("moe_expert_ffn_q4k", **kw)
    assert st == want and needle in msg, msg


def test_ffn_with_no_tokens_takes_null_activations():
    """T = 0: nothing is launched, so x, perm_pair and y_pairs may be NULL
    (zero-size tensors have no storage); the call returns before any HIP call."""
    st, msg = _ffn("moe_expert_ffn_q4k", T=0, x=None, perm=None, yp=None)
    assert st == Q.MOE_OK, msg


def test_ffn_q8_0_rejects_prefill():
    st, msg = _ffn("moe_expert_ffn_q8_0", H=256, I=128, stride=Q.moe_expert_blob_bytes(Q.MOE_FMT_Q8_0, 256, 128) + 64,
                   path=Q.MOE_PATH_PREFILL, x_dtype=Q.MOE_BF16)
    assert st == Q.MOE_ERR_UNSUPPORTED and "serves Q8_0" in msg


def test_ffn_q4k_prefill_size_limits():
    """The prefill GEMMs address activation rows with 32-bit byte offsets:
    a token count whose h buffer (T*k*I*2 bytes) reaches 4 GiB is refused."""
    st, msg = _ffn("moe_expert_ffn_q4k", T=400000, k=8, H=2048, I=768, path=Q.MOE_PATH_PREFILL, x_dtype=Q.MOE_BF16,
                   y_dtype=Q.MOE_BF16, ws_bytes=1 << 40)
    assert st == Q.MOE_ERR_UNSUPPORTED and "prefill path limits" in msg, msg


def test_ffn_q8_0_rejects_shape():
    st, msg = _ffn("moe_expert_ffn_q8_0", H=256, I=96)
    assert st == Q.MOE_ERR_UNSUPPORTED and "multiples of 128" in msg


def test_combine_rejects():
    st, msg = _call("moe_combine", FAKE, 0, FAKE, FAKE, FAKE, 8, 8, None, 4, 2, 252, FAKE, 0, None)
    assert st == Q.MOE_ERR_UNSUPPORTED and "multiple of 8" in msg
    st, msg = _call("moe_combine", FAKE, 3, FAKE, FAKE, FAKE, 8, 8, None, 4, 2, 256, FAKE, 0, None)
    assert st == Q.MOE_ERR_INVALID_ARGUMENT
    # S must lie in 0..E: the residency rule (slot in [0, S)) needs it
    st, msg = _call("moe_combine", FAKE, 0, FAKE, FAKE, FAKE, 8, 9, None, 4, 2, 256, FAKE, 0, None)
    assert st == Q.MOE_ERR_INVALID_ARGUMENT and "S = 9" in msg


def test_workspace_sizes_are_monotone():
    a = Q.moe_ffn_workspace_size(Q.MOE_FMT_Q4K, 2, 8, 7168, 2048, Q.MOE_PATH_DECODE)
    b = Q.moe_ffn_workspace_size(Q.MOE_FMT_Q4K, 4, 8, 7168, 2048, Q.MOE_PATH_DECODE)
    assert 0 < a < b
    assert Q.moe_ffn_workspace_size(Q.MOE_FMT_Q4K, 2, 8, 7000, 2048, Q.MOE_PATH_DECODE) == 0


@pytest.mark.parametrize("fmt", [Q.MOE_FMT_Q4K, Q.MOE_FMT_MXFP4, Q.MOE_FMT_Q3K_Q4K, Q.MOE_FMT_Q5K, Q.MOE_FMT_Q6K])
def test_prefill_workspace_for_every_prefill_format(fmt):
    """Every format but Q8_0 has a prefill path: its prefill workspace is the
    Q4_K one (bf16 h rows and the tile list do not depend on the block type),
    and AUTO asks for the larger of the two paths'."""
    T, k, H, I = 4096, 8, 2048, 768
    pre = Q.moe_ffn_workspace_size(fmt, T, k, H, I, Q.MOE_PATH_PREFILL)
    dec = Q.moe_ffn_workspace_size(fmt, T, k, H, I, Q.MOE_PATH_DECODE)
    assert pre == Q.moe_ffn_workspace_size(Q.MOE_FMT_Q4K, T, k, H, I, Q.MOE_PATH_PREFILL) > 0
    assert Q.moe_ffn_workspace_size(fmt, T, k, H, I, Q.MOE_PATH_AUTO) == max(pre, dec)


def test_q8_0_has_no_prefill_workspace():
    T, k, H, I = 4096, 8, 2048, 768
    dec = Q.moe_ffn_workspace_size(Q.MOE_FMT_Q8_0, T, k, H, I, Q.MOE_PATH_DECODE)
    assert Q.moe_ffn_workspace_size(Q.MOE_FMT_Q8_0, T, k, H, I, Q.MOE_PATH_AUTO) == dec


@pytest.mark.parametrize("fmt,H,I", [(Q.MOE_FMT_Q4K, 512, 256), (Q.MOE_FMT_Q4K, 768, 512), (Q.MOE_FMT_Q8_0, 256, 128),
                                     (Q.MOE_FMT_Q8_0, 384, 256), (Q.MOE_FMT_MXFP4, 512, 256),
                                     (Q.MOE_FMT_MXFP4, 768, 512), (Q.MOE_FMT_Q3K_Q4K, 512, 256),
                                     (Q.MOE_FMT_Q3K_Q4K, 768, 512), (Q.MOE_FMT_Q5K, 512, 256),
                                     (Q.MOE_FMT_Q5K, 768, 512), (Q.MOE_FMT_Q6K, 512, 256),
                                     (Q.MOE_FMT_Q6K, 768, 512)])
def test_pack_round_trip(fmt, H, I):
    blob = F.expert_blob(fmt, 5, 0, 1, H, I)
    packed = Q.moe_pack_expert(fmt, blob, H, I)
    assert blob.nbytes == Q.moe_expert_blob_bytes(fmt, H, I) and packed.nbytes == Q.moe_packed_blob_bytes(fmt, H, I)
    assert packed.nbytes == blob.nbytes or fmt == Q.MOE_FMT_Q3K_Q4K
    assert packed.nbytes != blob.nbytes or not np.array_equal(packed, blob)
    assert np.array_equal(Q.moe_unpack_expert(fmt, packed, H, I), blob)


def test_pack_places_q4k_fields():
    """Row r, super-block sb of W_up: its 16 header bytes sit at tile (r//64, sb), offset 1024 + 16*(r%64);
    quant element 8d+n of sub-block j sits in nibble n of the dword of group d, groups stored 0, 2, 1, 3."""
    H, I = 512, 256
    blob = F.expert_blob(Q.MOE_FMT_Q4K, 2, 0, 0, H, I)
    packed = Q.moe_pack_expert(Q.MOE_FMT_Q4K, blob, H, I)
    rb = H // 256 * 144
    for r, sb in [(0, 0), (70, 1), (255, 1)]:
        canon = blob[I * rb + r * rb + sb * 144: I * rb + r * rb + (sb + 1) * 144]
        tile = ((r // 64) * (H // 256) + sb) * 18432
        assert np.array_equal(packed[tile + 1024 + 16 * (r % 64): tile + 1040 + 16 * (r % 64)], canon[:16])
        for j in (0, 3, 7):
            slot = packed[tile + 3072 + j * 2048 + 16 * (r % 64): tile + 3088 + j * 2048 + 16 * (r % 64)]
            words = slot.view(np.uint32)
            for e in (0, 9, 31):
                byte = canon[16 + (j // 2) * 32 + e]
                q = (byte >> 4) if j % 2 else (byte & 15)
                assert (int(words[[0, 2, 1, 3][e // 8]]) >> (4 * (e % 8))) & 15 == q


def test_pack_places_mxfp4_fields():
    """Row r of W_down, block b: its E8M0 byte sits at down tile (r//64, b//8), offset 8*(r%64) + b%8; code
    element 8d+p of the block in the low nibble of byte p of the dword of group d and 8d+p+4 in its high nibble,
    groups stored 0, 2, 1, 3, at offset 512 + 1024*(b%8) + 16*(r%64)."""
    H, I = 512, 512
    blob = F.expert_blob(Q.MOE_FMT_MXFP4, 3, 0, 0, H, I)
    packed = Q.moe_pack_expert(Q.MOE_FMT_MXFP4, blob, H, I)
    rbH, rbI = H // 32 * 17, I // 32 * 17
    down = 2 * I * rbH
    base = (I // 64) * (H // 256) * 17408
    for r, b in [(0, 0), (70, 9), (511, 15)]:
        canon = blob[down + r * rbI + b * 17: down + r * rbI + (b + 1) * 17]
        codes = [canon[1 + i] & 15 for i in range(16)] + [canon[1 + i] >> 4 for i in range(16)]
        tile = base + ((r // 64) * (I // 256) + b // 8) * 8704
        assert packed[tile + 8 * (r % 64) + b % 8] == canon[0]
        slot = packed[tile + 512 + 1024 * (b % 8) + 16 * (r % 64): tile + 528 + 1024 * (b % 8) + 16 * (r % 64)]
        words = slot.view(np.uint32)
        for e in range(32):
            d, n = e // 8, e % 8
            p, half = n % 4, n // 4
            assert (int(words[[0, 2, 1, 3][d]]) >> (8 * p + 4 * half)) & 15 == codes[e]


def test_pack_places_q3k_fields():
    """Mixed blob, row r of W_gate, super-block u: header (12 scale bytes, d) at gate/up tile (r//64, u), offset
    16*(r%64); element 32b + 8d + n's low bits in LA (d < 2) or LB at bit 4n + 2(d % 2), its high bit in HB at bit
    4n + (2 + d) % 4; the Q4_K down section follows the Q3_K tiles."""
    H, I = 512, 256
    blob = F.expert_blob(Q.MOE_FMT_Q3K_Q4K, 4, 0, 0, H, I)
    packed = Q.moe_pack_expert(Q.MOE_FMT_Q3K_Q4K, blob, H, I)
    rb = H // 256 * 110
    for r, u in [(0, 0), (70, 1), (255, 1)]:
        canon = blob[r * rb + u * 110: r * rb + (u + 1) * 110]
        tile = ((r // 64) * (H // 256) + u) * 14336
        hdr = packed[tile + 16 * (r % 64): tile + 16 * (r % 64) + 16]
        assert np.array_equal(hdr[:12], canon[96:108]) and np.array_equal(hdr[12:14], canon[108:110])
        for i in (0, 37, 129, 255):
            h, g, l = i // 128, (i % 128) // 32, i % 32
            low, high = (canon[32 + 32 * h + l] >> (2 * g)) & 3, (canon[l] >> (4 * h + g)) & 1
            b, d, n = i // 32, (i % 32) // 8, i % 8
            lw = packed[tile + 2048 + (b // 2) * 2048 + 16 * (r % 64): tile + 2064 + (b // 2) * 2048 + 16 * (r % 64)]
            word = int(lw.view(np.uint32)[2 * (b % 2) + (d // 2)])
            assert (word >> (4 * n + 2 * (d % 2))) & 3 == low
            hw = packed[tile + 10240 + (b // 4) * 2048 + 16 * (r % 64): tile + 10256 + (b // 4) * 2048 + 16 * (r % 64)]
            assert (int(hw.view(np.uint32)[b % 4]) >> (4 * n + (2 + d) % 4)) & 1 == high
    # the down section is the Q4_K blob's: same bytes as packing a Q4_K expert with this W_down
    q4 = np.concatenate([np.zeros(2 * I * (H // 256 * 144), np.uint8), blob[2 * I * rb:]])
    q4p = Q.moe_pack_expert(Q.MOE_FMT_Q4K, q4, H, I)
    base3, base4 = (I // 64) * (H // 256) * 14336, (I // 64) * (H // 256) * 18432
    assert np.array_equal(packed[base3:], q4p[base4:])


def test_pack_places_q5k_fields():
    """Row r of W_up, super-block u: header at gate/up tile (r//64, u), offset 1024 + 16*(r%64); element 8d+n of
    sub-block j's nibble in nibble n of group d's dword (groups stored 0, 2, 1, 3) and its high bit at bit 4n + d of
    the sub-block's HB word."""
    H, I = 512, 256
    blob = F.expert_blob(Q.MOE_FMT_Q5K, 6, 0, 0, H, I)
    packed = Q.moe_pack_expert(Q.MOE_FMT_Q5K, blob, H, I)
    rb = H // 256 * 176
    for r, u in [(0, 0), (70, 1), (255, 1)]:
        canon = blob[I * rb + r * rb + u * 176: I * rb + r * rb + (u + 1) * 176]
        tile = ((r // 64) * (H // 256) + u) * 22528
        assert np.array_equal(packed[tile + 1024 + 16 * (r % 64): tile + 1040 + 16 * (r % 64)], canon[:16])
        for j in (0, 3, 6):
            words = packed[tile + 2048 + j * 2048 + 1024 + 16 * (r % 64): tile + 2064 + j * 2048 + 1024 +
                           16 * (r % 64)].view(np.uint32)
            hw = packed[tile + 18432 + (j // 4) * 2048 + 1024 + 16 * (r % 64):
                        tile + 18448 + (j // 4) * 2048 + 1024 + 16 * (r % 64)].view(np.uint32)[j % 4]
            for e in (0, 9, 21, 31):
                byte = canon[48 + (j // 2) * 32 + e]
                low = (byte >> 4) if j % 2 else (byte & 15)
                high = (canon[16 + e] >> j) & 1
                assert (int(words[[0, 2, 1, 3][e // 8]]) >> (4 * (e % 8))) & 15 == low
                assert (int(hw) >> (4 * (e % 8) + e // 8)) & 1 == high


def test_pack_places_q6k_fields():
    """Row r of W_up (gate/up tiles, matrix 1) and row r of W_down (down tiles, one matrix), super-block u:
    the 16 scale bytes at m KB + 16 (r % 64) of the tile (matrix m of NMAT); element 8d+n of block j's low nibble in nibble n of
    group d's dword (groups stored 0, 2, 1, 3); its two high bits at bits 4n + 2 (d % 2) of word d // 2 of the
    block's (H0, H1) pair; fp16 d at 13 NMAT KB + 2 NMAT (r % 64) + 2m."""
    H, I = 512, 256
    blob = F.expert_blob(Q.MOE_FMT_Q6K, 7, 0, 0, H, I)
    packed = Q.moe_pack_expert(Q.MOE_FMT_Q6K, blob, H, I)
    rbH, rbI = H // 256 * 210, I // 256 * 210
    gate_up = (I // 64) * (H // 256) * 26880
    cases = [(1, 2, I * rbH + r * rbH, H // 256, 0, r) for r in (0, 70, 255)]            # W_up rows
    cases += [(0, 1, 2 * I * rbH + r * rbI, I // 256, gate_up, r) for r in (1, 200, 511)]  # W_down rows
    for m, nmat, row0, units, base, r in cases:
        for u in range(units):
            canon = blob[row0 + u * 210: row0 + (u + 1) * 210]
            tile = base + ((r // 64) * units + u) * nmat * 13440
            lr = r % 64
            assert np.array_equal(packed[tile + m * 1024 + 16 * lr: tile + m * 1024 + 16 * lr + 16], canon[192:208])
            dpos = tile + nmat * 13312 + 2 * nmat * lr + 2 * m
            assert np.array_equal(packed[dpos: dpos + 2], canon[208:210])
            for j in (0, 3, 5, 7):
                nib = tile + nmat * 1024 + j * nmat * 1024 + m * 1024 + 16 * lr
                words = packed[nib: nib + 16].view(np.uint32)
                hp = tile + nmat * 9216 + (j // 2) * nmat * 1024 + m * 1024 + 16 * lr
                hw = packed[hp: hp + 16].view(np.uint32)[2 * (j % 2): 2 * (j % 2) + 2]
                for e in (0, 6, 9, 15, 16, 21, 31):
                    i = 32 * j + e
                    h, g, l = i // 128, (i % 128) // 32, i % 32
                    byte = canon[64 * h + l + 32 * (g % 2)]
                    low = (byte & 15) if g < 2 else (byte >> 4)
                    high = (canon[128 + 32 * h + l] >> (2 * g)) & 3
                    dd, n = e // 8, e % 8
                    assert (int(words[[0, 2, 1, 3][dd]]) >> (4 * n)) & 15 == low
                    assert (int(hw[dd // 2]) >> (4 * n + 2 * (dd % 2))) & 3 == high


def test_validate_slot_map():
    Q.moe_validate_slot_map(np.array([0, -1, 2, 1], dtype=np.int32), 3)
    with pytest.raises(Q.QmoeError, match="slot 1 holds"):
        Q.moe_validate_slot_map(np.array([1, 1, -1], dtype=np.int32), 2)
    with pytest.raises(Q.QmoeError, match="outside"):
        Q.moe_validate_slot_map(np.array([0, 3], dtype=np.int32), 2)
    with pytest.raises(Q.QmoeError, match="outside"):
        Q.moe_validate_slot_map(np.array([0, -2], dtype=np.int32), 2)


def test_timer_misuse():
    st, msg = _call("moe_timer_end", 0, ctypes.byref(ctypes.c_double()), ctypes.byref(ctypes.c_int()))
    assert st == Q.MOE_ERR_INVALID_ARGUMENT and "not armed" in msg
    st, msg = _call("moe_timer_begin", 99, 4)
    assert st == Q.MOE_ERR_INVALID_ARGUMENT


def test_product_path_fails_loudly_without_the_library(monkeypatch):
    """No libqmoe.so, no computation: the first call raises (there is no CPU
    fallback anywhere in the package)."""
    monkeypatch.setattr(Q, "_lib", None)
    monkeypatch.setattr(Q, "LIB_PATH", "/nonexistent/libqmoe.so")
    with pytest.raises(ImportError, match="not built"):
        Q.lib()
    with pytest.raises(ImportError, match="not built"):
        Q.moe_expert_blob_bytes(Q.MOE_FMT_Q4K, 512, 256)


@pytest.mark.parametrize("fmt,H,I", [(Q.MOE_FMT_Q4K, 512, 256), (Q.MOE_FMT_Q4K, 768, 512), (Q.MOE_FMT_Q8_0, 256, 128),
                                     (Q.MOE_FMT_Q8_0, 384, 256)])
def test_per_matrix_pack_builds_the_expert_blob(fmt, H, I):
    """moe_pack_q4k / moe_pack_q8_0 of W_gate | W_up (interleaved) followed by W_down (not) give
    exactly the bytes moe_pack_expert writes for the whole expert, through the C ABI."""
    blob = F.expert_blob(fmt, 7, 0, 1, H, I)
    wb, bb = (256, 144) if fmt == Q.MOE_FMT_Q4K else (32, 34)
    gate_up = blob[:2 * I * H // wb * bb]
    down = blob[2 * I * H // wb * bb:]
    pack = Q.moe_pack_q4k if fmt == Q.MOE_FMT_Q4K else Q.moe_pack_q8_0
    got = np.concatenate([pack(gate_up, I, H, True), pack(down, H, I, False)])
    assert np.array_equal(got, Q.moe_pack_expert(fmt, blob, H, I))


def test_per_matrix_pack_rejects():
    buf = np.zeros(1 << 16, dtype=np.uint8)
    out = np.zeros(1 << 16, dtype=np.uint8)
    st, msg = _call("moe_pack_q4k", buf.ctypes.data, out.ctypes.data, 64, 200, 0)
    assert st == Q.MOE_ERR_UNSUPPORTED and "cols of 256" in msg
    st, msg = _call("moe_pack_q8_0", buf.ctypes.data, out.ctypes.data, 32, 128, 1)
    assert st == Q.MOE_ERR_UNSUPPORTED and "multiple of 64" in msg
    st, msg = _call("moe_pack_q4k", buf.ctypes.data, out.ctypes.data, 64, 256, 2)
    assert st == Q.MOE_ERR_INVALID_ARGUMENT and "gate_up_interleave" in msg
    st, msg = _call("moe_pack_q8_0", None, out.ctypes.data, 64, 128, 0)
    assert st == Q.MOE_ERR_INVALID_ARGUMENT
    st, msg = _call("moe_pack_q4k", buf.ctypes.data, buf.ctypes.data + 16, 64, 256, 0)
    assert st == Q.MOE_ERR_INVALID_ARGUMENT and "overlap" in msg


def test_noalloc_ffn_rejects_beyond_its_scratch_without_touching_the_device():
    """moe_expert_ffn_q4k_noalloc: the checks of moe_expert_ffn_q4k, then the
    workspace against the library's fixed scratch; a call that needs more is
    refused by name before any HIP call (so this runs without a GPU)."""
    stride = Q.moe_expert_blob_bytes(Q.MOE_FMT_Q4K, 2048, 768) // 16 * 16 + 256
    args = [FAKE, stride, 128, 2048, 768, FAKE, Q.MOE_BF16, 8192, 8, FAKE, FAKE, FAKE, FAKE, FAKE, Q.MOE_BF16,
            Q.MOE_PATH_PREFILL, None]
    need = Q.moe_ffn_workspace_size(Q.MOE_FMT_Q4K, 8192, 8, 2048, 768, Q.MOE_PATH_PREFILL)
    assert need > Q.MOE_NOALLOC_SCRATCH_BYTES
    st, msg = _call("moe_expert_ffn_q4k_noalloc", *args)
    assert st == Q.MOE_ERR_UNSUPPORTED and f"needs {need} bytes" in msg and str(Q.MOE_NOALLOC_SCRATCH_BYTES) in msg
    # the other checks come first, as in moe_expert_ffn_q4k
    args[3] = 2000
    st, msg = _call("moe_expert_ffn_q4k_noalloc", *args)
    assert st == Q.MOE_ERR_UNSUPPORTED and "multiples of 256" in msg
    # the 4096-token prefill layer's workspace fits
    assert Q.moe_ffn_workspace_size(Q.MOE_FMT_Q4K, 4096, 8, 2048, 768, Q.MOE_PATH_PREFILL) <= Q.MOE_NOALLOC_SCRATCH_BYTES
    # through the int8-activation path (two activation planes) it does not
    args[3], args[7], args[15] = 2048, 4096, Q.MOE_PATH_PREFILL_I8
    need = Q.moe_ffn_workspace_size(Q.MOE_FMT_Q4K, 4096, 8, 2048, 768, Q.MOE_PATH_PREFILL_I8)
    assert need > Q.MOE_NOALLOC_SCRATCH_BYTES
    st, msg = _call("moe_expert_ffn_q4k_noalloc", *args)
    assert st == Q.MOE_ERR_UNSUPPORTED and f"needs {need} bytes" in msg


def test_ffn_int8_path_refusals():
    """MOE_PATH_PREFILL_I8 serves Q4_K experts with bf16 activations, with the
    larger workspace the activation planes need."""
    mx_stride = Q.moe_expert_blob_bytes(Q.MOE_FMT_MXFP4, 2048, 768) // 16 * 16 + 256
    st, msg = _ffn("moe_expert_ffn_mxfp4", stride=mx_stride, path=Q.MOE_PATH_PREFILL_I8, x_dtype=Q.MOE_BF16,
                   y_dtype=Q.MOE_BF16)
    assert st == Q.MOE_ERR_UNSUPPORTED and "MOE_PATH_PREFILL_I8" in msg, msg
    st, msg = _ffn("moe_expert_ffn_q4k", path=Q.MOE_PATH_PREFILL_I8, x_dtype=Q.MOE_F32, y_dtype=Q.MOE_BF16)
    assert st == Q.MOE_ERR_UNSUPPORTED and "MOE_BF16 x" in msg, msg
    need = Q.moe_ffn_workspace_size(Q.MOE_FMT_Q4K, 2, 8, 2048, 768, Q.MOE_PATH_PREFILL_I8)
    assert need > Q.moe_ffn_workspace_size(Q.MOE_FMT_Q4K, 2, 8, 2048, 768, Q.MOE_PATH_PREFILL)
    st, msg = _ffn("moe_expert_ffn_q4k", path=Q.MOE_PATH_PREFILL_I8, x_dtype=Q.MOE_BF16, y_dtype=Q.MOE_BF16,
                   ws_bytes=need - 1)
    assert st == Q.MOE_ERR_WORKSPACE_TOO_SMALL, msg


@pytest.mark.parametrize("args,needle", [
    ((0, 8, None, 131072, None), "NULL"),
    ((3, 8, FAKE, 131072, None), "variant"),
    ((-1, 8, FAKE, 131072, None), "variant"),
    ((0, 0, FAKE, 131072, None), "sub_blocks"),
    ((1, (1 << 20) + 1, FAKE, 131072, None), "sub_blocks"),
    ((2, 8, FAKE, 131071, None), "fewer than"),
])
def test_prefill_probe_refusals(args, needle):
    st, msg = _call("moe_prefill_inner_probe", *args)
    assert st == Q.MOE_ERR_INVALID_ARGUMENT and needle in msg, msg


@pytest.mark.parametrize("args,needle", [
    ((None, 1 << 20, 64, 8, FAKE, FAKE, None), "NULL"),
    ((FAKE + 8, 1 << 20, 64, 8, FAKE, FAKE, None), "aligned"),
    ((FAKE, 1 << 20, 12, 8, FAKE, FAKE, None), "multiple of 8"),
    ((FAKE, 1 << 20, 64, 3, FAKE, FAKE, None), "depth"),
    ((FAKE, 64 * 1024 * 8 - 1, 64, 8, FAKE, FAKE, None), "less than"),
])
def test_read_probe_refusals(args, needle):
    n = ctypes.c_size_t(0)  # a host location for the byte count, never written on these paths
    st, msg = _call("moe_hbm_read_probe", *args[:5], ctypes.byref(n), args[6])
    assert st == Q.MOE_ERR_INVALID_ARGUMENT and needle in msg, msg
