// C ABI of the qmoe library: argument checks, named statuses, packing of
// expert blobs, stage timers and dispatch to the HIP launchers.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "qmoe.h"
#include "qmoe_internal.h"
#include "prefill_i8.h"

namespace {

thread_local std::string g_error;

moe_status fail(moe_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_error = buf;
    return st;
}

moe_status hip_fail(hipError_t e, const char* what) {
    return fail(MOE_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr long long kMaxPairs = 1ll << 24;

moe_status check_route_shape(int T, int E, int k) {
    if (T < 0) return fail(MOE_ERR_INVALID_ARGUMENT, "T = %d must be >= 0", T);
    if (E < 1 || E > MOE_MAX_EXPERTS) return fail(MOE_ERR_INVALID_ARGUMENT, "E = %d outside 1..%d", E, MOE_MAX_EXPERTS);
    if (k < 1 || k > E || k > MOE_MAX_TOPK)
        return fail(MOE_ERR_INVALID_ARGUMENT, "k = %d outside 1..min(E=%d, %d)", k, E, MOE_MAX_TOPK);
    if ((long long)T * k > kMaxPairs) return fail(MOE_ERR_INVALID_ARGUMENT, "T*k = %lld exceeds 2^24", (long long)T * k);
    return MOE_OK;
}

moe_status check_shape(int format, int H, int I) {
    if (format < MOE_FMT_Q8_0 || format > MOE_FMT_Q6K)
        return fail(MOE_ERR_INVALID_ARGUMENT,
                    "format = %d is not MOE_FMT_Q8_0, MOE_FMT_Q4K, MOE_FMT_MXFP4, MOE_FMT_Q3K_Q4K, MOE_FMT_Q5K or "
                    "MOE_FMT_Q6K", format);
    const int m = format == MOE_FMT_Q8_0 ? 128 : 256;
    static const char* const kNames[] = {"Q8_0", "Q4_K", "MXFP4", "Q3_K/Q4_K", "Q5_K", "Q6_K"};
    if (H <= 0 || I <= 0) return fail(MOE_ERR_INVALID_ARGUMENT, "H = %d, I = %d must be positive", H, I);
    if (H % m || I % m)
        return fail(MOE_ERR_UNSUPPORTED, "%s needs H and I multiples of %d (H = %d, I = %d)",
                    kNames[format], m, H, I);
    if ((long long)H * I > (1ll << 31))
        return fail(MOE_ERR_UNSUPPORTED, "H*I = %lld too large", (long long)H * I);
    return MOE_OK;
}

size_t blob_bytes(int format, int H, int I) {
    const size_t w = (size_t)H * I;  // weights per matrix
    switch (format) {
        case MOE_FMT_Q4K: return 3 * w / 256 * 144;
        case MOE_FMT_MXFP4: return 3 * w / 32 * 17;
        case MOE_FMT_Q3K_Q4K: return 2 * w / 256 * 110 + w / 256 * 144;
        case MOE_FMT_Q5K: return 3 * w / 256 * 176;
        case MOE_FMT_Q6K: return 3 * w / 256 * 210;
        default: return 3 * w / 32 * 34;
    }
}

// Bytes of a packed blob: the canonical count, except for the mixed expert,
// whose Q3_K rows take a 16-byte header per 256 inputs (14 bytes stored).
size_t packed_bytes(int format, int H, int I) {
    if (format == MOE_FMT_Q3K_Q4K) return qmoe::q3k_gateup_bytes(H, I) + (size_t)H * I / 256 * 144;
    return blob_bytes(format, H, I);
}

// Formats the prefill GEMM takes (Q8_0 runs the decode path at any T).
bool has_prefill(int format) { return format != MOE_FMT_Q8_0; }

int resolve_path(int format, int T, int x_dtype, int path) {
    if (path != MOE_PATH_AUTO) return path;
    return (has_prefill(format) && x_dtype == MOE_BF16 && T > 32) ? MOE_PATH_PREFILL : MOE_PATH_DECODE;
}

// ------------------------------------------------------------------ timers
struct StageTimer {
    std::atomic<int> armed{0};
    int capacity = 0;
    int used = 0;
    std::vector<hipEvent_t> start, stop;
};
StageTimer g_timer[qmoe::kStageCount];
static_assert(MOE_STAGE_COUNT == qmoe::kStageCount, "stage counts differ");
std::mutex g_timer_mu;

// ------------------------------------------------------------------ packing
// Q4_K: the 32 quants of sub-block j of a canonical super-block.
void q4k_subblock(const uint8_t* blk, int j, uint8_t* q) {
    const uint8_t* qs = blk + 16 + (j / 2) * 32;
    for (int l = 0; l < 32; ++l) q[l] = (j % 2 == 0) ? (qs[l] & 15) : (qs[l] >> 4);
}
void q4k_set_subblock(uint8_t* blk, int j, const uint8_t* q) {
    uint8_t* qs = blk + 16 + (j / 2) * 32;
    for (int l = 0; l < 32; ++l) {
        if (j % 2 == 0) qs[l] = (uint8_t)((qs[l] & 0xF0) | q[l]);
        else qs[l] = (uint8_t)((qs[l] & 0x0F) | (q[l] << 4));
    }
}
// 32 quants -> 16 packed bytes: element 8d+n in nibble n of the little-endian
// dword of group d, groups stored in the order 0, 2, 1, 3 (so the two groups
// one MFMA operand lane needs for a 32-wide sub-block are adjacent).
constexpr int kDwordSlot[4] = {0, 2, 1, 3};
void nibbles_pack(const uint8_t* q, uint8_t* dst) {
    for (int d = 0; d < 4; ++d) {
        uint32_t w = 0;
        for (int n = 0; n < 8; ++n) w |= (uint32_t)(q[8 * d + n] & 15) << (4 * n);
        memcpy(dst + 4 * kDwordSlot[d], &w, 4);
    }
}
void nibbles_unpack(const uint8_t* src, uint8_t* q) {
    for (int d = 0; d < 4; ++d) {
        uint32_t w;
        memcpy(&w, src + 4 * kDwordSlot[d], 4);
        for (int n = 0; n < 8; ++n) q[8 * d + n] = (uint8_t)((w >> (4 * n)) & 15);
    }
}

// The Q4_K gate/up section: canonical W_gate [I, H] at offset 0 and W_up
// right after it, packed tiles at offset 0 (PACK: canonical -> packed;
// otherwise packed -> canonical).
template <bool PACK>
void q4k_gateup_walk(const uint8_t* in, uint8_t* out, int H, int I) {
    const size_t rbH = (size_t)H / 256 * 144;
    const size_t gbytes = (size_t)I * rbH;
    const int SBH = H / 256;
    uint8_t q[32];
    for (int rg = 0; rg < I / 64; ++rg)
        for (int sb = 0; sb < SBH; ++sb) {
            const size_t tile = ((size_t)rg * SBH + sb) * qmoe::kQ4kGateUpTile;
            for (int r = 0; r < 64; ++r) {
                const size_t row = (size_t)rg * 64 + r;
                for (int mat = 0; mat < 2; ++mat) {
                    const size_t canon = mat * gbytes + row * rbH + (size_t)sb * 144;
                    const size_t hdr = tile + mat * 1024 + r * 16;
                    if (PACK) {
                        memcpy(out + hdr, in + canon, 16);
                        for (int j = 0; j < 8; ++j) {
                            q4k_subblock(in + canon, j, q);
                            nibbles_pack(q, out + tile + 2048 + j * 2048 + mat * 1024 + r * 16);
                        }
                    } else {
                        memcpy(out + canon, in + hdr, 16);
                        for (int j = 0; j < 8; ++j) {
                            nibbles_unpack(in + tile + 2048 + j * 2048 + mat * 1024 + r * 16, q);
                            q4k_set_subblock(out + canon, j, q);
                        }
                    }
                }
            }
        }
}

template <bool PACK>
void q4k_down_walk(const uint8_t* in, uint8_t* out, int H, int I, size_t canon_base, size_t base);

// Move every field of a blob between the canonical and the packed layout
// (PACK: canonical -> packed; otherwise packed -> canonical).
template <bool PACK>
void q4k_walk(const uint8_t* in, uint8_t* out, int H, int I) {
    q4k_gateup_walk<PACK>(in, out, H, I);
    q4k_down_walk<PACK>(in, out, H, I, 2 * (size_t)I * (H / 256 * 144), qmoe::q4k_gateup_bytes(H, I));
}

// The Q4_K down matrix: canonical rows at canon_base, packed tiles at base.
template <bool PACK>
void q4k_down_walk(const uint8_t* in, uint8_t* out, int H, int I, size_t canon_base, size_t base) {
    const size_t rbI = (size_t)I / 256 * 144;
    const int SBI = I / 256;
    uint8_t q[32];
    for (int rg = 0; rg < H / 64; ++rg)
        for (int sb = 0; sb < SBI; ++sb) {
            const size_t tile = base + ((size_t)rg * SBI + sb) * qmoe::kQ4kDownTile;
            for (int r = 0; r < 64; ++r) {
                const size_t row = (size_t)rg * 64 + r;
                const size_t canon = canon_base + row * rbI + (size_t)sb * 144;
                if (PACK) {
                    memcpy(out + tile + r * 16, in + canon, 16);
                    for (int j = 0; j < 8; ++j) {
                        q4k_subblock(in + canon, j, q);
                        nibbles_pack(q, out + tile + 1024 + j * 1024 + r * 16);
                    }
                } else {
                    memcpy(out + canon, in + tile + r * 16, 16);
                    for (int j = 0; j < 8; ++j) {
                        nibbles_unpack(in + tile + 1024 + j * 1024 + r * 16, q);
                        q4k_set_subblock(out + canon, j, q);
                    }
                }
            }
        }
}

// One Q8_0 34-byte block <-> (2-byte scale, two 16-byte halves), quants
// offset by 128.
void q8_block(const uint8_t* canon, uint8_t* scale, uint8_t* lo, uint8_t* hi, bool pack) {
    if (pack) {
        memcpy(scale, canon, 2);
        for (int e = 0; e < 16; ++e) lo[e] = canon[2 + e] ^ 0x80;
        for (int e = 0; e < 16; ++e) hi[e] = canon[18 + e] ^ 0x80;
    } else {
        uint8_t* dst = const_cast<uint8_t*>(canon);
        memcpy(dst, scale, 2);
        for (int e = 0; e < 16; ++e) dst[2 + e] = lo[e] ^ 0x80;
        for (int e = 0; e < 16; ++e) dst[18 + e] = hi[e] ^ 0x80;
    }
}

// The Q8_0 gate/up section: canonical W_gate [I, H] at offset 0 and W_up
// right after it, packed tiles at offset 0.
template <bool PACK>
void q8_gateup_walk(const uint8_t* in, uint8_t* out, int H, int I) {
    const size_t rbH = (size_t)H / 32 * 34;
    const size_t gbytes = (size_t)I * rbH;
    const int BH = H / 128;
    uint8_t* dev = PACK ? out : const_cast<uint8_t*>(in);
    const uint8_t* canon_base = PACK ? in : out;
    for (int rg = 0; rg < I / 64; ++rg)
        for (int bg = 0; bg < BH; ++bg) {
            uint8_t* tile = dev + ((size_t)rg * BH + bg) * qmoe::kQ8GateUpTile;
            for (int r = 0; r < 64; ++r) {
                const size_t row = (size_t)rg * 64 + r;
                for (int mat = 0; mat < 2; ++mat)
                    for (int jj = 0; jj < 4; ++jj) {
                        uint8_t* lo = tile + 1024 + mat * 2048 + jj * 4096 + r * 16;
                        q8_block(canon_base + mat * gbytes + row * rbH + (size_t)(bg * 4 + jj) * 34,
                                 tile + mat * 512 + r * 8 + jj * 2, lo, lo + 1024, PACK);
                    }
            }
        }
}

// The Q8_0 down matrix [H, I]: canonical rows at canon_base, packed tiles at base.
template <bool PACK>
void q8_down_walk(const uint8_t* in, uint8_t* out, int H, int I, size_t canon_base, size_t base) {
    const size_t rbI = (size_t)I / 32 * 34;
    const int BI = I / 128;
    uint8_t* dev = PACK ? out : const_cast<uint8_t*>(in);
    const uint8_t* canon = (PACK ? in : out) + canon_base;
    for (int rg = 0; rg < H / 64; ++rg)
        for (int bg = 0; bg < BI; ++bg) {
            uint8_t* tile = dev + base + ((size_t)rg * BI + bg) * qmoe::kQ8DownTile;
            for (int r = 0; r < 64; ++r) {
                const size_t row = (size_t)rg * 64 + r;
                for (int jj = 0; jj < 4; ++jj) {
                    uint8_t* lo = tile + 512 + jj * 2048 + r * 16;
                    q8_block(canon + row * rbI + (size_t)(bg * 4 + jj) * 34, tile + r * 8 + jj * 2, lo, lo + 1024,
                             PACK);
                }
            }
        }
}

template <bool PACK>
void q8_walk(const uint8_t* in, uint8_t* out, int H, int I) {
    q8_gateup_walk<PACK>(in, out, H, I);
    q8_down_walk<PACK>(in, out, H, I, 2 * (size_t)I * (H / 32 * 34), qmoe::q8_gateup_bytes(H, I));
}

// MXFP4: one 17-byte block (E8M0 scale, element i < 16 in the low nibble of
// byte 1 + i, 16 + i in its high nibble) <-> (scale byte, 16 packed code
// bytes: group d of elements 8d..8d+7 in dword slot 0, 2, 1, 3, byte p =
// element 8d+p low, 8d+p+4 high).
void mx4_block(const uint8_t* canon, uint8_t* scale, uint8_t* codes, bool pack) {
    uint8_t e[32];
    if (pack) {
        *scale = canon[0];
        for (int i = 0; i < 16; ++i) {
            e[i] = canon[1 + i] & 15;
            e[16 + i] = canon[1 + i] >> 4;
        }
        for (int d = 0; d < 4; ++d)
            for (int p = 0; p < 4; ++p)
                codes[4 * kDwordSlot[d] + p] = (uint8_t)(e[8 * d + p] | (e[8 * d + p + 4] << 4));
    } else {
        uint8_t* dst = const_cast<uint8_t*>(canon);
        dst[0] = *scale;
        for (int d = 0; d < 4; ++d)
            for (int p = 0; p < 4; ++p) {
                const uint8_t b = codes[4 * kDwordSlot[d] + p];
                e[8 * d + p] = b & 15;
                e[8 * d + p + 4] = b >> 4;
            }
        for (int i = 0; i < 16; ++i) dst[1 + i] = (uint8_t)(e[i] | (e[16 + i] << 4));
    }
}

template <bool PACK>
void mx4_walk(const uint8_t* in, uint8_t* out, int H, int I) {
    const size_t rbH = (size_t)H / 32 * 17, rbI = (size_t)I / 32 * 17;
    const size_t gbytes = (size_t)I * rbH;
    const int UH = H / 256, UI = I / 256;
    uint8_t* dev = PACK ? out : const_cast<uint8_t*>(in);
    const uint8_t* canon_base = PACK ? in : out;
    for (int rg = 0; rg < I / 64; ++rg)
        for (int u = 0; u < UH; ++u) {
            const size_t tile = ((size_t)rg * UH + u) * qmoe::kMx4GateUpTile;
            for (int r = 0; r < 64; ++r) {
                const size_t row = (size_t)rg * 64 + r;
                for (int mat = 0; mat < 2; ++mat)
                    for (int j = 0; j < 8; ++j)
                        mx4_block(canon_base + mat * gbytes + row * rbH + (size_t)(u * 8 + j) * 17,
                                  dev + tile + mat * 512 + r * 8 + j, dev + tile + 1024 + j * 2048 + mat * 1024 + r * 16,
                                  PACK);
            }
        }
    const size_t base = qmoe::mx4_gateup_bytes(H, I);
    for (int rg = 0; rg < H / 64; ++rg)
        for (int u = 0; u < UI; ++u) {
            const size_t tile = base + ((size_t)rg * UI + u) * qmoe::kMx4DownTile;
            for (int r = 0; r < 64; ++r) {
                const size_t row = (size_t)rg * 64 + r;
                for (int j = 0; j < 8; ++j)
                    mx4_block(canon_base + 2 * gbytes + row * rbI + (size_t)(u * 8 + j) * 17, dev + tile + r * 8 + j,
                              dev + tile + 512 + j * 1024 + r * 16, PACK);
            }
        }
}

// Q3_K: one canonical 110-byte super-block (high bits, low bits, scales, d)
// <-> its packed fields: 16-byte header (scales, d, 2 zero bytes), the (LA,
// LB) words of its 8 blocks and their HB words.
void q3k_block(const uint8_t* canon, uint8_t* hdr, uint32_t* la, uint32_t* lb, uint32_t* hb, bool pack) {
    if (pack) {
        memcpy(hdr, canon + 96, 12);
        memcpy(hdr + 12, canon + 108, 2);
        hdr[14] = hdr[15] = 0;
        for (int b = 0; b < 8; ++b) la[b] = lb[b] = hb[b] = 0;
        for (int i = 0; i < 256; ++i) {
            const int h = i / 128, g = (i % 128) / 32, l = i % 32;
            const uint32_t low = (canon[32 + 32 * h + l] >> (2 * g)) & 3, high = (canon[l] >> (4 * h + g)) & 1;
            const int b = i / 32, d = (i % 32) / 8, n = i % 8;
            (d < 2 ? la : lb)[b] |= low << (4 * n + 2 * (d & 1));
            hb[b] |= high << (4 * n + (2 + d) % 4);
        }
    } else {
        uint8_t* dst = const_cast<uint8_t*>(canon);
        memset(dst, 0, 110);
        memcpy(dst + 96, hdr, 12);
        memcpy(dst + 108, hdr + 12, 2);
        for (int i = 0; i < 256; ++i) {
            const int b = i / 32, d = (i % 32) / 8, n = i % 8;
            const uint32_t low = ((d < 2 ? la : lb)[b] >> (4 * n + 2 * (d & 1))) & 3;
            const uint32_t high = (hb[b] >> (4 * n + (2 + d) % 4)) & 1;
            const int h = i / 128, g = (i % 128) / 32, l = i % 32;
            dst[32 + 32 * h + l] |= (uint8_t)(low << (2 * g));
            dst[l] |= (uint8_t)(high << (4 * h + g));
        }
    }
}

// The mixed blob: Q3_K gate/up tiles (layout in qmoe_internal.h), then the
// Q4_K down section.
template <bool PACK>
void q3k_mix_walk(const uint8_t* in, uint8_t* out, int H, int I) {
    const size_t rbH = (size_t)H / 256 * 110;
    const size_t gbytes = (size_t)I * rbH;
    const int UH = H / 256;
    uint8_t* dev = PACK ? out : const_cast<uint8_t*>(in);
    const uint8_t* canon_base = PACK ? in : out;
    uint32_t la[8], lb[8], hb[8];
    for (int rg = 0; rg < I / 64; ++rg)
        for (int u = 0; u < UH; ++u) {
            uint8_t* tile = dev + ((size_t)rg * UH + u) * qmoe::kQ3kGateUpTile;
            for (int r = 0; r < 64; ++r) {
                const size_t row = (size_t)rg * 64 + r;
                for (int mat = 0; mat < 2; ++mat) {
                    const uint8_t* canon = canon_base + mat * gbytes + row * rbH + (size_t)u * 110;
                    uint8_t* hdr = tile + mat * 1024 + r * 16;
                    if (!PACK) {
                        for (int c = 0; c < 4; ++c) {
                            const uint8_t* p = tile + 2048 + c * 2048 + mat * 1024 + r * 16;
                            memcpy(&la[2 * c], p, 4);
                            memcpy(&lb[2 * c], p + 4, 4);
                            memcpy(&la[2 * c + 1], p + 8, 4);
                            memcpy(&lb[2 * c + 1], p + 12, 4);
                        }
                        for (int c = 0; c < 2; ++c) memcpy(&hb[4 * c], tile + 10240 + c * 2048 + mat * 1024 + r * 16, 16);
                    }
                    q3k_block(canon, hdr, la, lb, hb, PACK);
                    if (PACK) {
                        for (int c = 0; c < 4; ++c) {
                            uint8_t* p = tile + 2048 + c * 2048 + mat * 1024 + r * 16;
                            memcpy(p, &la[2 * c], 4);
                            memcpy(p + 4, &lb[2 * c], 4);
                            memcpy(p + 8, &la[2 * c + 1], 4);
                            memcpy(p + 12, &lb[2 * c + 1], 4);
                        }
                        for (int c = 0; c < 2; ++c) memcpy(tile + 10240 + c * 2048 + mat * 1024 + r * 16, &hb[4 * c], 16);
                    }
                }
            }
        }
    q4k_down_walk<PACK>(in, out, H, I, 2 * gbytes, qmoe::q3k_gateup_bytes(H, I));
}

// Q5_K: one canonical 176-byte super-block (d, dmin, 12 scale bytes, 32
// bytes of high bits, 128 bytes of nibbles) <-> header (the first 16 bytes),
// eight 16-byte nibble slots in the Q4_K packed order, eight HB words
// (element 8d + n's high bit at bit 4n + d).
void q5k_block(const uint8_t* canon, uint8_t* hdr, uint8_t* const* nib, uint32_t* hb, bool pack) {
    uint8_t q[32];
    if (pack) {
        memcpy(hdr, canon, 16);
        for (int j = 0; j < 8; ++j) {
            hb[j] = 0;
            for (int l = 0; l < 32; ++l) {
                const uint8_t byte = canon[48 + (j / 2) * 32 + l];
                q[l] = (j % 2) ? (byte >> 4) : (byte & 15);
                hb[j] |= (uint32_t)((canon[16 + l] >> j) & 1) << (4 * (l % 8) + l / 8);
            }
            nibbles_pack(q, nib[j]);
        }
    } else {
        uint8_t* dst = const_cast<uint8_t*>(canon);
        memset(dst, 0, 176);
        memcpy(dst, hdr, 16);
        for (int j = 0; j < 8; ++j) {
            nibbles_unpack(nib[j], q);
            for (int l = 0; l < 32; ++l) {
                dst[48 + (j / 2) * 32 + l] |= (uint8_t)(q[l] << (4 * (j % 2)));
                dst[16 + l] |= (uint8_t)(((hb[j] >> (4 * (l % 8) + l / 8)) & 1) << j);
            }
        }
    }
}

template <bool PACK>
void q5k_walk(const uint8_t* in, uint8_t* out, int H, int I) {
    const size_t rbH = (size_t)H / 256 * 176, rbI = (size_t)I / 256 * 176;
    const size_t gbytes = (size_t)I * rbH;
    uint8_t* dev = PACK ? out : const_cast<uint8_t*>(in);
    const uint8_t* canon_base = PACK ? in : out;
    uint32_t hb[8];
    uint8_t* nib[8];
    // one matrix section: tiles of `rows` x 256 inputs, NMAT matrices interleaved
    auto section = [&](size_t base, int nmat, int row_tiles, int units, size_t rb, size_t canon0, size_t cstride) {
        const size_t tbytes = (size_t)nmat * qmoe::kQ5kDownTile;
        for (int rg = 0; rg < row_tiles; ++rg)
            for (int u = 0; u < units; ++u) {
                uint8_t* tile = dev + base + ((size_t)rg * units + u) * tbytes;
                for (int r = 0; r < 64; ++r)
                    for (int m = 0; m < nmat; ++m) {
                        const uint8_t* canon = canon_base + canon0 + m * cstride + ((size_t)rg * 64 + r) * rb + (size_t)u * 176;
                        for (int j = 0; j < 8; ++j) nib[j] = tile + nmat * 1024 + j * nmat * 1024 + m * 1024 + r * 16;
                        uint8_t* hw = tile + nmat * 9216 + m * 1024 + r * 16;  // chunk 0; chunk 1 at + nmat KB
                        if (!PACK) {
                            memcpy(hb, hw, 16);
                            memcpy(hb + 4, hw + nmat * 1024, 16);
                        }
                        q5k_block(canon, tile + m * 1024 + r * 16, nib, hb, PACK);
                        if (PACK) {
                            memcpy(hw, hb, 16);
                            memcpy(hw + nmat * 1024, hb + 4, 16);
                        }
                    }
            }
    };
    section(0, 2, I / 64, H / 256, rbH, 0, gbytes);
    section(qmoe::q5k_gateup_bytes(H, I), 1, H / 64, I / 256, rbI, 2 * gbytes, 0);
}

// Q6_K: one canonical 210-byte super-block (low nibbles, high bit pairs, 16
// signed scales, fp16 d) <-> its packed fields: the 16 scale bytes, eight
// 16-byte nibble slots in the Q4_K packed order, per block the words (H0,
// H1) of two high bits per element, and d.
void q6k_block(const uint8_t* canon, uint8_t* sc, uint8_t* const* nib, uint32_t* hw, uint8_t* d, bool pack) {
    uint8_t q[32];
    if (pack) {
        memcpy(sc, canon + 192, 16);
        memcpy(d, canon + 208, 2);
        for (int j = 0; j < 8; ++j) {
            hw[2 * j] = hw[2 * j + 1] = 0;
            for (int e = 0; e < 32; ++e) {
                const int i = 32 * j + e, h = i / 128, g = (i % 128) / 32, l = i % 32;
                const uint8_t byte = canon[64 * h + l + 32 * (g % 2)];
                q[e] = g < 2 ? (byte & 15) : (byte >> 4);
                const uint32_t high = (canon[128 + 32 * h + l] >> (2 * g)) & 3;
                const int dd = e / 8, n = e % 8;
                hw[2 * j + dd / 2] |= high << (4 * n + 2 * (dd % 2));
            }
            nibbles_pack(q, nib[j]);
        }
    } else {
        uint8_t* dst = const_cast<uint8_t*>(canon);
        memset(dst, 0, 210);
        memcpy(dst + 192, sc, 16);
        memcpy(dst + 208, d, 2);
        for (int j = 0; j < 8; ++j) {
            nibbles_unpack(nib[j], q);
            for (int e = 0; e < 32; ++e) {
                const int i = 32 * j + e, h = i / 128, g = (i % 128) / 32, l = i % 32;
                const int dd = e / 8, n = e % 8;
                const uint32_t high = (hw[2 * j + dd / 2] >> (4 * n + 2 * (dd % 2))) & 3;
                dst[64 * h + l + 32 * (g % 2)] |= (uint8_t)(q[e] << (g < 2 ? 0 : 4));
                dst[128 + 32 * h + l] |= (uint8_t)(high << (2 * g));
            }
        }
    }
}

template <bool PACK>
void q6k_walk(const uint8_t* in, uint8_t* out, int H, int I) {
    const size_t rbH = (size_t)H / 256 * 210, rbI = (size_t)I / 256 * 210;
    const size_t gbytes = (size_t)I * rbH;
    uint8_t* dev = PACK ? out : const_cast<uint8_t*>(in);
    const uint8_t* canon_base = PACK ? in : out;
    uint32_t hw[16];
    uint8_t* nib[8];
    auto section = [&](size_t base, int nmat, int row_tiles, int units, size_t rb, size_t canon0, size_t cstride) {
        const size_t tbytes = (size_t)nmat * qmoe::kQ6kDownTile;
        for (int rg = 0; rg < row_tiles; ++rg)
            for (int u = 0; u < units; ++u) {
                uint8_t* tile = dev + base + ((size_t)rg * units + u) * tbytes;
                for (int r = 0; r < 64; ++r)
                    for (int m = 0; m < nmat; ++m) {
                        const uint8_t* canon = canon_base + canon0 + m * cstride + ((size_t)rg * 64 + r) * rb + (size_t)u * 210;
                        for (int j = 0; j < 8; ++j) nib[j] = tile + nmat * 1024 + j * nmat * 1024 + m * 1024 + r * 16;
                        uint8_t* hp = tile + nmat * 9216 + m * 1024 + r * 16;  // chunk c at + c nmat KB
                        uint8_t* dp = tile + nmat * 13312 + 2 * nmat * r + 2 * m;
                        if (!PACK)
                            for (int c = 0; c < 4; ++c) memcpy(hw + 4 * c, hp + c * nmat * 1024, 16);
                        q6k_block(canon, tile + m * 1024 + r * 16, nib, hw, dp, PACK);
                        if (PACK)
                            for (int c = 0; c < 4; ++c) memcpy(hp + c * nmat * 1024, hw + 4 * c, 16);
                    }
            }
    };
    section(0, 2, I / 64, H / 256, rbH, 0, gbytes);
    section(qmoe::q6k_gateup_bytes(H, I), 1, H / 64, I / 256, rbI, 2 * gbytes, 0);
}

// One matrix, or the gate/up pair, of a blob (the pieces moe_pack_expert
// puts together).
moe_status pack_matrix(int format, const void* canonical, void* packed, int rows, int cols, int gate_up_interleave) {
    const char* name = format == MOE_FMT_Q4K ? "moe_pack_q4k" : "moe_pack_q8_0";
    const int cb = format == MOE_FMT_Q4K ? 256 : 128;
    if (!canonical || !packed) return fail(MOE_ERR_INVALID_ARGUMENT, "%s: NULL pointer", name);
    if (gate_up_interleave != 0 && gate_up_interleave != 1)
        return fail(MOE_ERR_INVALID_ARGUMENT, "%s: gate_up_interleave = %d is not 0 or 1", name, gate_up_interleave);
    if (rows <= 0 || cols <= 0 || rows % 64 || cols % cb)
        return fail(MOE_ERR_UNSUPPORTED, "%s: rows must be a positive multiple of 64 and cols of %d (rows = %d, "
                                         "cols = %d)", name, cb, rows, cols);
    if ((long long)rows * cols > (1ll << 31))
        return fail(MOE_ERR_UNSUPPORTED, "%s: rows*cols = %lld too large", name, (long long)rows * cols);
    const size_t w = (size_t)rows * cols * (gate_up_interleave ? 2 : 1);
    const size_t n = format == MOE_FMT_Q4K ? w / 256 * 144 : w / 32 * 34;
    const uint8_t* in = static_cast<const uint8_t*>(canonical);
    uint8_t* out = static_cast<uint8_t*>(packed);
    if (in < out + n && out < in + n) return fail(MOE_ERR_INVALID_ARGUMENT, "%s: buffers overlap", name);
    memset(out, 0, n);
    if (format == MOE_FMT_Q4K) {
        if (gate_up_interleave) q4k_gateup_walk<true>(in, out, cols, rows);
        else q4k_down_walk<true>(in, out, rows, cols, 0, 0);
    } else {
        if (gate_up_interleave) q8_gateup_walk<true>(in, out, cols, rows);
        else q8_down_walk<true>(in, out, rows, cols, 0, 0);
    }
    return MOE_OK;
}

// Every check of an expert-FFN call but those of the workspace; on success
// *need is the workspace the call needs and *resolved its path.
moe_status ffn_check(int format, const void* slot_pool, size_t slot_stride, int S, int H, int I, const void* x,
                     int x_dtype, int T, int k, const int32_t* slot_offsets, const int32_t* active_slots,
                     const int32_t* num_active, const int32_t* perm_pair, void* y_pairs, int y_dtype, int path,
                     size_t* need, int* resolved) {
    moe_status st = check_shape(format, H, I);
    if (st != MOE_OK) return st;
    if (S < 1 || S > MOE_MAX_EXPERTS) return fail(MOE_ERR_INVALID_ARGUMENT, "S = %d outside 1..%d", S, MOE_MAX_EXPERTS);
    if (T < 0) return fail(MOE_ERR_INVALID_ARGUMENT, "T = %d must be >= 0", T);
    if (k < 1 || k > MOE_MAX_TOPK) return fail(MOE_ERR_INVALID_ARGUMENT, "k = %d outside 1..%d", k, MOE_MAX_TOPK);
    if ((long long)T * k > kMaxPairs) return fail(MOE_ERR_INVALID_ARGUMENT, "T*k exceeds 2^24");
    // (with T = 0 nothing is read or written: x, perm_pair and y_pairs may be NULL)
    if (!slot_pool || !slot_offsets || !active_slots || !num_active || (T > 0 && (!x || !perm_pair || !y_pairs)))
        return fail(MOE_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
    if (!aligned16(slot_pool) || (slot_stride & 15u))
        return fail(MOE_ERR_INVALID_ARGUMENT, "slot_pool and slot_stride must be 16-byte aligned");
    if (slot_stride < packed_bytes(format, H, I))
        return fail(MOE_ERR_INVALID_ARGUMENT, "slot_stride %zu is smaller than the blob (%zu bytes)", slot_stride,
                    packed_bytes(format, H, I));
    if (x_dtype != MOE_F32 && x_dtype != MOE_BF16) return fail(MOE_ERR_INVALID_ARGUMENT, "bad x_dtype %d", x_dtype);
    if (y_dtype != MOE_F32 && y_dtype != MOE_BF16) return fail(MOE_ERR_INVALID_ARGUMENT, "bad y_dtype %d", y_dtype);
    if (path < MOE_PATH_AUTO || path > MOE_PATH_PREFILL_I8) return fail(MOE_ERR_INVALID_ARGUMENT, "bad path %d", path);
    if (path == MOE_PATH_PREFILL_I8 && format != MOE_FMT_Q4K)
        return fail(MOE_ERR_UNSUPPORTED, "MOE_PATH_PREFILL_I8 is implemented for Q4_K experts");
    if (!aligned16(x) || !aligned16(y_pairs)) return fail(MOE_ERR_INVALID_ARGUMENT, "x and y_pairs must be 16-byte aligned");
    const int p = resolve_path(format, T, x_dtype, path);
    *resolved = p;
    if (p == MOE_PATH_DECODE) {
        if (y_dtype != MOE_F32) return fail(MOE_ERR_UNSUPPORTED, "the decode path writes MOE_F32 y_pairs");
        *need = qmoe::decode_workspace_bytes(T, k, H, I);
    } else {
        if (!has_prefill(format))
            return fail(MOE_ERR_UNSUPPORTED, "the prefill path is implemented for Q4_K, Q5_K, Q6_K, MXFP4 and "
                                             "Q3_K/Q4_K (MOE_PATH_DECODE serves Q8_0 at any T)");
        if (x_dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "the prefill path takes MOE_BF16 x");
        // The GEMMs address x and h rows with 32-bit byte offsets, and the
        // tile list counts tiles in 16 bits.
        const long long P = (long long)T * k;
        if ((long long)T * H * 2 > 0xFFFFFFFFLL || P * I * 2 > 0xFFFFFFFFLL || (P + 255) / 256 + 1024 > 0xFFFF)
            return fail(MOE_ERR_UNSUPPORTED, "prefill path limits: T*H*2 and T*k*I*2 below 4 GiB, T*k below %d",
                        (0xFFFF - 1024) * 256);
        *need = p == MOE_PATH_PREFILL_I8 ? qmoe::prefill_i8_workspace_bytes(T, k, H, I)
                                         : qmoe::prefill_workspace_bytes(T, k, H, I);
    }
    return MOE_OK;
}

moe_status ffn_common(int format, const void* slot_pool, size_t slot_stride, int S, int H, int I, const void* x,
                      int x_dtype, int T, int k, const int32_t* slot_offsets, const int32_t* active_slots,
                      const int32_t* num_active, const int32_t* perm_pair, void* y_pairs, int y_dtype, int path,
                      void* ws, size_t ws_bytes, void* stream) {
    size_t need = 0;
    int p = MOE_PATH_DECODE;
    moe_status st = ffn_check(format, slot_pool, slot_stride, S, H, I, x, x_dtype, T, k, slot_offsets, active_slots,
                              num_active, perm_pair, y_pairs, y_dtype, path, &need, &p);
    if (st != MOE_OK) return st;
    if (ws_bytes < need)
        return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes, %zu needed", ws_bytes, need);
    if (need > 0 && !ws) return fail(MOE_ERR_INVALID_ARGUMENT, "workspace pointer is NULL");
    if (need > 0 && !aligned16(ws)) return fail(MOE_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
    if (T == 0) return MOE_OK;

    qmoe::FfnArgs a{format, static_cast<const uint8_t*>(slot_pool), slot_stride, S, H, I, x, x_dtype, T, k,
                    slot_offsets, active_slots, num_active, perm_pair, y_pairs, y_dtype, ws};
    hipError_t e = p == MOE_PATH_DECODE       ? qmoe::launch_ffn_decode(a, (hipStream_t)stream)
                   : p == MOE_PATH_PREFILL_I8 ? qmoe::launch_ffn_prefill_i8(a, (hipStream_t)stream)
                                              : qmoe::launch_ffn_prefill(a, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "expert FFN launch");
    return MOE_OK;
}

// ------------------------------------------------- allocation-free FFN
// The workspace of moe_expert_ffn_q4k_noalloc: one file-scope device array
// per GPU (each device holds its own copy, at its own address, from the
// first such call on it until the process ends).  Host code must not pass
// `scratch` itself to a kernel (its host-side name is not a device address):
// its device address is looked up once per device with
// hipGetSymbolAddress and kept in g_scratch_ptr.
static_assert(MOE_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

moe_status scratch_address(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!p) return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) gave NULL");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}

}  // namespace

namespace qmoe {

StageEvents timer_events(int stage) {
    StageTimer& t = g_timer[stage];
    StageEvents ev;
    if (!t.armed.load(std::memory_order_relaxed)) return ev;
    std::lock_guard<std::mutex> lk(g_timer_mu);
    if (t.armed.load() && t.used < t.capacity) {
        ev.start = t.start[t.used];
        ev.stop = t.stop[t.used];
        ++t.used;
    }
    return ev;
}

}  // namespace qmoe

extern "C" {

const char* moe_status_name(int status) {
    switch (status) {
        case MOE_OK: return "MOE_OK";
        case MOE_ERR_INVALID_ARGUMENT: return "MOE_ERR_INVALID_ARGUMENT";
        case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
        case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL";
        case MOE_ERR_HIP: return "MOE_ERR_HIP";
        default: return "MOE_STATUS_UNKNOWN";
    }
}

const char* moe_last_error(void) { return g_error.c_str(); }

moe_status moe_route_topk(const float* logits, int T, int E, int k, int score, int renormalize, float scale,
                          int32_t* topk_ids, float* topk_w, void* stream) {
    moe_status st = check_route_shape(T, E, k);
    if (st != MOE_OK) return st;
    if (score != MOE_SCORE_SOFTMAX && score != MOE_SCORE_SIGMOID)
        return fail(MOE_ERR_INVALID_ARGUMENT, "score = %d is not softmax or sigmoid", score);
    if (T > 0 && (!logits || !topk_ids || !topk_w)) return fail(MOE_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
    if (!(scale == scale)) return fail(MOE_ERR_INVALID_ARGUMENT, "scale is NaN");
    hipError_t e = qmoe::launch_route_topk(logits, T, E, k, score, renormalize, scale, topk_ids, topk_w,
                                           (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "route launch");
    return MOE_OK;
}

size_t moe_batches_workspace_size(int T, int k, int E, int S) {
    if (T < 0 || k < 1 || E < 1 || S < 0 || S > E || E > MOE_MAX_EXPERTS) return 0;
    return qmoe::batches_workspace_bytes(T, k, S);
}

moe_status moe_build_expert_batches(const int32_t* topk_ids, const float* topk_w, int T, int k, int E,
                                    const int32_t* slot_of_expert, int S, int32_t* slot_offsets,
                                    int32_t* active_slots, int32_t* num_active, int32_t* perm_pair,
                                    int32_t* host_token, int32_t* host_expert, float* host_weight,
                                    int32_t* host_count, void* ws, size_t ws_bytes, void* stream) {
    moe_status st = check_route_shape(T, E, k);
    if (st != MOE_OK) return st;
    if (S < 0 || S > E) return fail(MOE_ERR_INVALID_ARGUMENT, "S = %d outside 0..E (%d)", S, E);
    if (!slot_of_expert || !slot_offsets || !num_active || !host_count)
        return fail(MOE_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
    if (T > 0 && (!topk_ids || !topk_w || !perm_pair || !host_token || !host_expert || !host_weight ||
                  (S > 0 && !active_slots)))
        return fail(MOE_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
    const size_t need = moe_batches_workspace_size(T, k, E, S);
    if (ws_bytes < need)
        return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "batches workspace %zu bytes, %zu needed", ws_bytes, need);
    if (need > 0 && !ws) return fail(MOE_ERR_INVALID_ARGUMENT, "batches workspace pointer is NULL");
    hipError_t e = qmoe::launch_batches(topk_ids, topk_w, T, k, E, slot_of_expert, S, slot_offsets, active_slots,
                                        num_active, perm_pair, host_token, host_expert, host_weight, host_count, ws,
                                        (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "batches launch");
    return MOE_OK;
}

moe_status moe_route_and_batch(const float* logits, int T, int E, int k, int score, int renormalize, float scale,
                               int32_t* topk_ids, float* topk_w, const int32_t* slot_of_expert, int S,
                               int32_t* slot_offsets, int32_t* active_slots, int32_t* num_active, int32_t* perm_pair,
                               int32_t* host_token, int32_t* host_expert, float* host_weight, int32_t* host_count,
                               uint32_t* route_counts, void* ws, size_t ws_bytes, void* stream) {
    moe_status st = check_route_shape(T, E, k);
    if (st != MOE_OK) return st;
    if (score != MOE_SCORE_SOFTMAX && score != MOE_SCORE_SIGMOID)
        return fail(MOE_ERR_INVALID_ARGUMENT, "score = %d is not softmax or sigmoid", score);
    if (!(scale == scale)) return fail(MOE_ERR_INVALID_ARGUMENT, "scale is NaN");
    if (S < 0 || S > E) return fail(MOE_ERR_INVALID_ARGUMENT, "S = %d outside 0..E (%d)", S, E);
    if (!slot_of_expert || !slot_offsets || !num_active || !host_count)
        return fail(MOE_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
    if (T > 0 && (!logits || !topk_ids || !topk_w || !perm_pair || !host_token || !host_expert || !host_weight ||
                  (S > 0 && !active_slots)))
        return fail(MOE_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
    const size_t need = moe_batches_workspace_size(T, k, E, S);
    if (ws_bytes < need)
        return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "batches workspace %zu bytes, %zu needed", ws_bytes, need);
    if (need > 0 && !ws) return fail(MOE_ERR_INVALID_ARGUMENT, "batches workspace pointer is NULL");
    hipError_t e = qmoe::launch_route_batches(logits, T, E, k, score, renormalize, scale, topk_ids, topk_w,
                                              slot_of_expert, S, slot_offsets, active_slots, num_active, perm_pair,
                                              host_token, host_expert, host_weight, host_count, route_counts, ws,
                                              (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "route and batch launch");
    return MOE_OK;
}

moe_status moe_count_routes(const int32_t* topk_ids, int T, int k, int E, uint32_t* counts, void* stream) {
    moe_status st = check_route_shape(T, E, k);
    if (st != MOE_OK) return st;
    if (!counts || (T > 0 && !topk_ids)) return fail(MOE_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
    hipError_t e = qmoe::launch_count_routes(topk_ids, T * k, E, counts, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "count launch");
    return MOE_OK;
}

size_t moe_expert_blob_bytes(int format, int H, int I) {
    if (check_shape(format, H, I) != MOE_OK) return 0;
    return blob_bytes(format, H, I);
}

size_t moe_packed_blob_bytes(int format, int H, int I) {
    if (check_shape(format, H, I) != MOE_OK) return 0;
    return packed_bytes(format, H, I);
}

moe_status moe_pack_expert(int format, const void* canonical, void* packed, int H, int I) {
    moe_status st = check_shape(format, H, I);
    if (st != MOE_OK) return st;
    if (!canonical || !packed) return fail(MOE_ERR_INVALID_ARGUMENT, "NULL blob pointer");
    const uint8_t* in = static_cast<const uint8_t*>(canonical);
    uint8_t* out = static_cast<uint8_t*>(packed);
    const size_t nc = blob_bytes(format, H, I), np = packed_bytes(format, H, I);
    if (in < out + np && out < in + nc) return fail(MOE_ERR_INVALID_ARGUMENT, "blobs overlap");
    memset(out, 0, np);
    if (format == MOE_FMT_Q4K) q4k_walk<true>(in, out, H, I);
    else if (format == MOE_FMT_MXFP4) mx4_walk<true>(in, out, H, I);
    else if (format == MOE_FMT_Q3K_Q4K) q3k_mix_walk<true>(in, out, H, I);
    else if (format == MOE_FMT_Q5K) q5k_walk<true>(in, out, H, I);
    else if (format == MOE_FMT_Q6K) q6k_walk<true>(in, out, H, I);
    else q8_walk<true>(in, out, H, I);
    return MOE_OK;
}

moe_status moe_unpack_expert(int format, const void* packed, void* canonical, int H, int I) {
    moe_status st = check_shape(format, H, I);
    if (st != MOE_OK) return st;
    if (!canonical || !packed) return fail(MOE_ERR_INVALID_ARGUMENT, "NULL blob pointer");
    const uint8_t* in = static_cast<const uint8_t*>(packed);
    uint8_t* out = static_cast<uint8_t*>(canonical);
    const size_t nc = blob_bytes(format, H, I), np = packed_bytes(format, H, I);
    if (in < out + nc && out < in + np) return fail(MOE_ERR_INVALID_ARGUMENT, "blobs overlap");
    memset(out, 0, nc);
    if (format == MOE_FMT_Q4K) q4k_walk<false>(in, out, H, I);
    else if (format == MOE_FMT_MXFP4) mx4_walk<false>(in, out, H, I);
    else if (format == MOE_FMT_Q3K_Q4K) q3k_mix_walk<false>(in, out, H, I);
    else if (format == MOE_FMT_Q5K) q5k_walk<false>(in, out, H, I);
    else if (format == MOE_FMT_Q6K) q6k_walk<false>(in, out, H, I);
    else q8_walk<false>(in, out, H, I);
    return MOE_OK;
}

moe_status moe_pack_q4k(const void* canonical, void* device_layout, int rows, int cols, int gate_up_interleave) {
    return pack_matrix(MOE_FMT_Q4K, canonical, device_layout, rows, cols, gate_up_interleave);
}

moe_status moe_pack_q8_0(const void* canonical, void* device_layout, int rows, int cols, int gate_up_interleave) {
    return pack_matrix(MOE_FMT_Q8_0, canonical, device_layout, rows, cols, gate_up_interleave);
}

moe_status moe_validate_slot_map(const int32_t* slot_of_expert, int E, int S) {
    if (!slot_of_expert) return fail(MOE_ERR_INVALID_ARGUMENT, "slot_of_expert is NULL");
    if (E < 1 || E > MOE_MAX_EXPERTS) return fail(MOE_ERR_INVALID_ARGUMENT, "E = %d outside 1..%d", E, MOE_MAX_EXPERTS);
    if (S < 0 || S > E) return fail(MOE_ERR_INVALID_ARGUMENT, "S = %d outside 0..E", S);
    std::vector<int> owner(S, -1);
    for (int e = 0; e < E; ++e) {
        const int s = slot_of_expert[e];
        if (s == -1) continue;
        if (s < 0 || s >= S) return fail(MOE_ERR_INVALID_ARGUMENT, "expert %d maps to slot %d outside [0, %d)", e, s, S);
        if (owner[s] >= 0) return fail(MOE_ERR_INVALID_ARGUMENT, "slot %d holds experts %d and %d", s, owner[s], e);
        owner[s] = e;
    }
    return MOE_OK;
}

size_t moe_ffn_workspace_size(int format, int T, int k, int H, int I, int path) {
    if (check_shape(format, H, I) != MOE_OK || T < 0 || k < 1 || k > MOE_MAX_TOPK) return 0;
    const size_t dec = qmoe::decode_workspace_bytes(T, k, H, I);
    static_assert(MOE_MAX_EXPERTS == qmoe::kMaxExpertsInternal, "expert limits differ");
    if (!has_prefill(format) || path == MOE_PATH_DECODE) return dec;
    const size_t pre = qmoe::prefill_workspace_bytes(T, k, H, I);
    if (path == MOE_PATH_PREFILL) return pre;
    if (path == MOE_PATH_PREFILL_I8) return format == MOE_FMT_Q4K ? qmoe::prefill_i8_workspace_bytes(T, k, H, I) : 0;
    return std::max(dec, pre);
}

moe_status moe_expert_ffn_q4k(const void* slot_pool, size_t slot_stride, int S, int H, int I, const void* x,
                              int x_dtype, int T, int k, const int32_t* slot_offsets, const int32_t* active_slots,
                              const int32_t* num_active, const int32_t* perm_pair, void* y_pairs, int y_dtype,
                              int path, void* ws, size_t ws_bytes, void* stream) {
    return ffn_common(MOE_FMT_Q4K, slot_pool, slot_stride, S, H, I, x, x_dtype, T, k, slot_offsets, active_slots,
                      num_active, perm_pair, y_pairs, y_dtype, path, ws, ws_bytes, stream);
}

moe_status moe_expert_ffn_q4k_noalloc(const void* slot_pool, size_t slot_stride, int S, int H, int I, const void* x,
                                      int x_dtype, int T, int k, const int32_t* slot_offsets,
                                      const int32_t* active_slots, const int32_t* num_active,
                                      const int32_t* perm_pair, void* y_pairs, int y_dtype, int path, void* stream) {
    size_t need = 0;
    int p = MOE_PATH_DECODE;
    moe_status st = ffn_check(MOE_FMT_Q4K, slot_pool, slot_stride, S, H, I, x, x_dtype, T, k, slot_offsets,
                              active_slots, num_active, perm_pair, y_pairs, y_dtype, path, &need, &p);
    if (st != MOE_OK) return st;
    if (need > (size_t)MOE_NOALLOC_SCRATCH_BYTES)
        return fail(MOE_ERR_UNSUPPORTED, "moe_expert_ffn_q4k_noalloc: this call needs %zu bytes of workspace, the "
                                         "library's scratch holds %zu (call moe_expert_ffn_q4k with a workspace)",
                    need, (size_t)MOE_NOALLOC_SCRATCH_BYTES);
    if (T == 0) return MOE_OK;
    void* ws = nullptr;
    st = scratch_address(&ws);
    if (st != MOE_OK) return st;
    return ffn_common(MOE_FMT_Q4K, slot_pool, slot_stride, S, H, I, x, x_dtype, T, k, slot_offsets, active_slots,
                      num_active, perm_pair, y_pairs, y_dtype, path, ws, MOE_NOALLOC_SCRATCH_BYTES, stream);
}

moe_status moe_expert_ffn_q8_0(const void* slot_pool, size_t slot_stride, int S, int H, int I, const void* x,
                               int x_dtype, int T, int k, const int32_t* slot_offsets, const int32_t* active_slots,
                               const int32_t* num_active, const int32_t* perm_pair, void* y_pairs, int y_dtype,
                               int path, void* ws, size_t ws_bytes, void* stream) {
    return ffn_common(MOE_FMT_Q8_0, slot_pool, slot_stride, S, H, I, x, x_dtype, T, k, slot_offsets, active_slots,
                      num_active, perm_pair, y_pairs, y_dtype, path, ws, ws_bytes, stream);
}

moe_status moe_expert_ffn_mxfp4(const void* slot_pool, size_t slot_stride, int S, int H, int I, const void* x,
                                int x_dtype, int T, int k, const int32_t* slot_offsets, const int32_t* active_slots,
                                const int32_t* num_active, const int32_t* perm_pair, void* y_pairs, int y_dtype,
                                int path, void* ws, size_t ws_bytes, void* stream) {
    return ffn_common(MOE_FMT_MXFP4, slot_pool, slot_stride, S, H, I, x, x_dtype, T, k, slot_offsets, active_slots,
                      num_active, perm_pair, y_pairs, y_dtype, path, ws, ws_bytes, stream);
}

moe_status moe_expert_ffn_q3k_q4k(const void* slot_pool, size_t slot_stride, int S, int H, int I, const void* x,
                                  int x_dtype, int T, int k, const int32_t* slot_offsets, const int32_t* active_slots,
                                  const int32_t* num_active, const int32_t* perm_pair, void* y_pairs, int y_dtype,
                                  int path, void* ws, size_t ws_bytes, void* stream) {
    return ffn_common(MOE_FMT_Q3K_Q4K, slot_pool, slot_stride, S, H, I, x, x_dtype, T, k, slot_offsets, active_slots,
                      num_active, perm_pair, y_pairs, y_dtype, path, ws, ws_bytes, stream);
}

moe_status moe_expert_ffn_q5k(const void* slot_pool, size_t slot_stride, int S, int H, int I, const void* x,
                              int x_dtype, int T, int k, const int32_t* slot_offsets, const int32_t* active_slots,
                              const int32_t* num_active, const int32_t* perm_pair, void* y_pairs, int y_dtype,
                              int path, void* ws, size_t ws_bytes, void* stream) {
    return ffn_common(MOE_FMT_Q5K, slot_pool, slot_stride, S, H, I, x, x_dtype, T, k, slot_offsets, active_slots,
                      num_active, perm_pair, y_pairs, y_dtype, path, ws, ws_bytes, stream);
}

moe_status moe_expert_ffn_q6k(const void* slot_pool, size_t slot_stride, int S, int H, int I, const void* x,
                              int x_dtype, int T, int k, const int32_t* slot_offsets, const int32_t* active_slots,
                              const int32_t* num_active, const int32_t* perm_pair, void* y_pairs, int y_dtype,
                              int path, void* ws, size_t ws_bytes, void* stream) {
    return ffn_common(MOE_FMT_Q6K, slot_pool, slot_stride, S, H, I, x, x_dtype, T, k, slot_offsets, active_slots,
                      num_active, perm_pair, y_pairs, y_dtype, path, ws, ws_bytes, stream);
}

size_t moe_layer_decode_workspace_size(int format, int T, int k, int E, int S, int H, int I, int I_shared) {
    if (check_shape(format, H, I) != MOE_OK || T < 0 || k < 1 || k > MOE_MAX_TOPK || E < 1 ||
        E > MOE_MAX_EXPERTS || S < 1 || S > E || I_shared < 0 || (I_shared > 0 && I_shared % 128))
        return 0;
    return qmoe::layer_decode_workspace_bytes(format, T, k, E, S, H, I, I_shared);
}

moe_status moe_layer_decode(int format, const float* logits, const void* x, int x_dtype, int T, int E, int k,
                            int score, int renormalize, float scale, const int32_t* slot_of_expert, int S, const void* slot_pool,
                            size_t slot_stride, int H, int I, const void* shared_pool, int I_shared,
                            int32_t* topk_ids, float* topk_w, int32_t* slot_offsets, int32_t* active_slots,
                            int32_t* num_active, int32_t* perm_pair, int32_t* host_token, int32_t* host_expert,
                            float* host_weight, int32_t* host_count, uint32_t* route_counts, float* y_pairs,
                            float* y, void* ws, size_t ws_bytes, void* stream) {
    moe_status st = check_route_shape(T, E, k);
    if (st != MOE_OK) return st;
    if (score != MOE_SCORE_SOFTMAX && score != MOE_SCORE_SIGMOID)
        return fail(MOE_ERR_INVALID_ARGUMENT, "score = %d is not softmax or sigmoid", score);
    if (!(scale == scale)) return fail(MOE_ERR_INVALID_ARGUMENT, "scale is NaN");
    if (S < 1 || S > E) return fail(MOE_ERR_INVALID_ARGUMENT, "S = %d outside 1..E (%d)", S, E);
    if (!slot_of_expert || !slot_offsets || !num_active || !host_count || !active_slots)
        return fail(MOE_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
    if (T > 0 && (!logits || !topk_ids || !topk_w || !host_token || !host_expert || !host_weight || !y))
        return fail(MOE_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
    size_t need_ffn = 0;
    int p = MOE_PATH_DECODE;
    st = ffn_check(format, slot_pool, slot_stride, S, H, I, x, x_dtype, T, k, slot_offsets, active_slots, num_active,
                   perm_pair, y_pairs, MOE_F32, MOE_PATH_DECODE, &need_ffn, &p);
    if (st != MOE_OK) return st;
    if (I_shared < 0 || (I_shared > 0) != (shared_pool != nullptr))
        return fail(MOE_ERR_INVALID_ARGUMENT, "shared_pool and I_shared > 0 go together (I_shared = %d)", I_shared);
    if (I_shared > 0) {
        st = check_shape(MOE_FMT_Q8_0, H, I_shared);
        if (st != MOE_OK) return st;
        if (!aligned16(shared_pool)) return fail(MOE_ERR_INVALID_ARGUMENT, "shared_pool must be 16-byte aligned");
    }
    if (T > 0 && !aligned16(y)) return fail(MOE_ERR_INVALID_ARGUMENT, "y must be 16-byte aligned");
    const size_t need = qmoe::layer_decode_workspace_bytes(format, T, k, E, S, H, I, I_shared);
    if (ws_bytes < need) return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes, %zu needed", ws_bytes, need);
    if (need > 0 && (!ws || !aligned16(ws)))
        return fail(MOE_ERR_INVALID_ARGUMENT, "workspace must be non-NULL and 16-byte aligned");
    if (T == 0) return MOE_OK;
    const qmoe::LayerDecodeArgs a{format, logits, x, x_dtype, T, E, k, score, renormalize, scale, slot_of_expert, S,
                                  slot_pool, slot_stride, H, I, shared_pool, I_shared, topk_ids, topk_w, slot_offsets,
                                  active_slots, num_active, perm_pair, host_token, host_expert, host_weight,
                                  host_count, route_counts, y_pairs, y, ws};
    hipError_t e = qmoe::launch_layer_decode(a, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "decode layer launch");
    return MOE_OK;
}

moe_status moe_combine(const void* y_pairs, int y_pairs_dtype, const int32_t* topk_ids, const float* topk_w,
                       const int32_t* slot_of_expert, int E, int S, const float* y_shared, int T, int k, int H,
                       void* y, int y_dtype, void* stream) {
    if (T < 0) return fail(MOE_ERR_INVALID_ARGUMENT, "T = %d must be >= 0", T);
    if (E < 1 || E > MOE_MAX_EXPERTS) return fail(MOE_ERR_INVALID_ARGUMENT, "E = %d outside 1..%d", E, MOE_MAX_EXPERTS);
    if (S < 0 || S > E) return fail(MOE_ERR_INVALID_ARGUMENT, "S = %d outside 0..E (%d)", S, E);
    if (k < 1 || k > MOE_MAX_TOPK) return fail(MOE_ERR_INVALID_ARGUMENT, "k = %d outside 1..%d", k, MOE_MAX_TOPK);
    if (H <= 0 || H % 8) return fail(MOE_ERR_UNSUPPORTED, "H = %d must be a positive multiple of 8", H);
    if ((long long)T * k > kMaxPairs) return fail(MOE_ERR_INVALID_ARGUMENT, "T*k exceeds 2^24");
    if (y_pairs_dtype != MOE_F32 && y_pairs_dtype != MOE_BF16) return fail(MOE_ERR_INVALID_ARGUMENT, "bad y_pairs dtype");
    if (y_dtype != MOE_F32 && y_dtype != MOE_BF16) return fail(MOE_ERR_INVALID_ARGUMENT, "bad y dtype");
    if (T > 0 && (!y_pairs || !topk_ids || !topk_w || !slot_of_expert || !y))
        return fail(MOE_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
    if (T > 0 && (!aligned16(y_pairs) || !aligned16(y) || (y_shared && !aligned16(y_shared))))
        return fail(MOE_ERR_INVALID_ARGUMENT, "y_pairs, y and y_shared must be 16-byte aligned");
    hipError_t e = qmoe::launch_combine(y_pairs, y_pairs_dtype, topk_ids, topk_w, slot_of_expert, E, S, y_shared, T,
                                        k, H, y, y_dtype, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "combine launch");
    return MOE_OK;
}

moe_status moe_timer_begin(int stage, int capacity) {
    if (stage < 0 || stage >= qmoe::kStageCount) return fail(MOE_ERR_INVALID_ARGUMENT, "bad stage %d", stage);
    if (capacity < 1 || capacity > (1 << 20)) return fail(MOE_ERR_INVALID_ARGUMENT, "bad capacity %d", capacity);
    std::lock_guard<std::mutex> lk(g_timer_mu);
    StageTimer& t = g_timer[stage];
    if (t.armed.load()) return fail(MOE_ERR_INVALID_ARGUMENT, "stage %d timer already armed", stage);
    t.start.assign(capacity, nullptr);
    t.stop.assign(capacity, nullptr);
    for (int i = 0; i < capacity; ++i) {
        hipError_t e1 = hipEventCreate(&t.start[i]);
        hipError_t e2 = hipEventCreate(&t.stop[i]);
        if (e1 != hipSuccess || e2 != hipSuccess) {
            for (int j = 0; j <= i; ++j) {
                if (t.start[j]) hipEventDestroy(t.start[j]);
                if (t.stop[j]) hipEventDestroy(t.stop[j]);
            }
            t.start.clear();
            t.stop.clear();
            return hip_fail(e1 != hipSuccess ? e1 : e2, "hipEventCreate");
        }
    }
    t.capacity = capacity;
    t.used = 0;
    t.armed.store(1);
    return MOE_OK;
}

moe_status moe_timer_read(int stage, float* ms_each, int capacity, int* launches) {
    if (stage < 0 || stage >= qmoe::kStageCount) return fail(MOE_ERR_INVALID_ARGUMENT, "bad stage %d", stage);
    if (!launches || (capacity > 0 && !ms_each) || capacity < 0)
        return fail(MOE_ERR_INVALID_ARGUMENT, "bad output buffer");
    std::lock_guard<std::mutex> lk(g_timer_mu);
    StageTimer& t = g_timer[stage];
    if (!t.armed.load()) return fail(MOE_ERR_INVALID_ARGUMENT, "stage %d timer not armed", stage);
    hipError_t err = hipSuccess;
    if (t.used > 0) err = hipEventSynchronize(t.stop[t.used - 1]);
    const int n = std::min(t.used, capacity);
    for (int i = 0; i < n && err == hipSuccess; ++i) err = hipEventElapsedTime(&ms_each[i], t.start[i], t.stop[i]);
    *launches = t.used;
    if (err != hipSuccess) return hip_fail(err, "stage timer");
    return MOE_OK;
}

moe_status moe_hbm_read_probe(const void* buf, size_t bytes, int waves, int depth, uint32_t* sink, size_t* read,
                              void* stream) {
    if (!buf || !sink || !read) return fail(MOE_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
    if (((uintptr_t)buf & 15) != 0) return fail(MOE_ERR_INVALID_ARGUMENT, "buf must be 16-byte aligned");
    if (waves < 8 || waves > 65536 || waves % 8 != 0)
        return fail(MOE_ERR_INVALID_ARGUMENT, "waves = %d is not a multiple of 8 in 8..65536", waves);
    if (depth != 1 && depth != 2 && depth != 4 && depth != 8 && depth != 16)
        return fail(MOE_ERR_INVALID_ARGUMENT, "depth = %d is not 1, 2, 4, 8 or 16", depth);
    if (bytes / 1024 / (size_t)waves < (size_t)depth)
        return fail(MOE_ERR_INVALID_ARGUMENT, "%zu bytes is less than 1024 x waves x depth", bytes);
    const hipError_t e = qmoe::launch_hbm_read(buf, bytes, waves, depth, sink, read, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "read probe launch");
    return MOE_OK;
}

moe_status moe_prefill_inner_probe(int variant, int sub_blocks, float* out, size_t out_floats, void* stream) {
    if (!out) return fail(MOE_ERR_INVALID_ARGUMENT, "out is NULL");
    if (variant < 0 || variant > 2) return fail(MOE_ERR_INVALID_ARGUMENT, "variant = %d is not 0, 1 or 2", variant);
    if (sub_blocks < 1 || sub_blocks > (1 << 20))
        return fail(MOE_ERR_INVALID_ARGUMENT, "sub_blocks = %d is not in 1..1048576", sub_blocks);
    if (out_floats < (size_t)MOE_PREFILL_PROBE_OUT_FLOATS)
        return fail(MOE_ERR_INVALID_ARGUMENT, "out holds %zu floats, fewer than %d", out_floats,
                    MOE_PREFILL_PROBE_OUT_FLOATS);
    static_assert(qmoe::kPrefillProbeWorkgroups * 256 == MOE_PREFILL_PROBE_OUT_FLOATS, "probe output size");
    const hipError_t e = qmoe::launch_prefill_probe(variant, sub_blocks, out, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "prefill probe launch");
    return MOE_OK;
}

moe_status moe_timer_end(int stage, double* total_ms, int* launches) {
    if (stage < 0 || stage >= qmoe::kStageCount) return fail(MOE_ERR_INVALID_ARGUMENT, "bad stage %d", stage);
    if (!total_ms || !launches) return fail(MOE_ERR_INVALID_ARGUMENT, "NULL output pointer");
    std::lock_guard<std::mutex> lk(g_timer_mu);
    StageTimer& t = g_timer[stage];
    if (!t.armed.load()) return fail(MOE_ERR_INVALID_ARGUMENT, "stage %d timer not armed", stage);
    t.armed.store(0);
    double sum = 0.0;
    hipError_t err = hipSuccess;
    if (t.used > 0) err = hipEventSynchronize(t.stop[t.used - 1]);
    for (int i = 0; i < t.used && err == hipSuccess; ++i) {
        float ms = 0.f;
        err = hipEventElapsedTime(&ms, t.start[i], t.stop[i]);
        sum += ms;
    }
    for (int i = 0; i < t.capacity; ++i) {
        hipEventDestroy(t.start[i]);
        hipEventDestroy(t.stop[i]);
    }
    *total_ms = sum;
    *launches = t.used;
    t.start.clear();
    t.stop.clear();
    t.capacity = t.used = 0;
    if (err != hipSuccess) return hip_fail(err, "stage timer");
    return MOE_OK;
}

}  // extern "C"
