// Host leg: the expert FFN of the pairs whose expert is not on the card, on
// the host CPU (bloomery README of 2026-09-24, opening list: the experts a
// routed layer does not keep on the GPU run on an AVX2 host tier inside the
// same step).  Interface and arithmetic: include/qmoe_host.h.
//
// Design: the pairs are grouped by expert, so each expert's blocks are read
// from host memory once for all of its tokens.  Within an expert, output
// rows are split over OpenMP threads (a static split: every output element
// is produced by one thread in a fixed order, whatever the thread count).  A
// thread dequantizes one weight row into fp32 (AVX2: nibbles or bytes
// widened to int32 and converted, then d sc_j q - dmin m_j, or d q, by fused
// multiply-add) and dots it with each of the expert's tokens (FMA into four
// 8-wide accumulators).  Gate and up give h = silu(g) u per token; the down
// rows then give y, added into y_host with the pair's weight.
#include <immintrin.h>
#include <omp.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "qmoe.h"
#include "qmoe_host.h"

namespace {

thread_local std::string g_error;

int fail(int status, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_error = buf;
    return status;
}

// IEEE binary16 -> binary32, exact for every input.
float half_bits_to_float(uint16_t h) {
    const uint32_t sign = (uint32_t)(h >> 15) << 31;
    const uint32_t e = (h >> 10) & 0x1F, m = h & 0x3FF;
    uint32_t bits;
    if (e == 0x1F) {
        bits = sign | 0x7F800000u | (m << 13);
    } else if (e != 0) {
        bits = sign | ((e + 112) << 23) | (m << 13);
    } else if (m == 0) {
        bits = sign;
    } else {  // subnormal: normalize
        int shift = 0;
        uint32_t mm = m;
        while (!(mm & 0x400)) {
            mm <<= 1;
            ++shift;
        }
        bits = sign | ((uint32_t)(113 - shift) << 23) | ((mm & 0x3FF) << 13);
    }
    float f;
    std::memcpy(&f, &bits, sizeof(f));
    return f;
}

uint16_t load_u16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }

constexpr int kQ4kBlock = 256, kQ4kBytes = 144;
constexpr int kQ8Block = 32, kQ8Bytes = 34;
constexpr int kMx4Block = 32, kMx4Bytes = 17;
constexpr int kQ3kBlock = 256, kQ3kBytes = 110;
constexpr int kQ5kBytes = 176;
constexpr int kQ6kBytes = 210;
constexpr int kRowQ3k = 100;  // block type of a Q3_K matrix (the mixed expert's gate and up)

size_t row_bytes(int type, int n) {
    if (type == MOE_FMT_Q4K) return (size_t)(n / kQ4kBlock) * kQ4kBytes;
    if (type == MOE_FMT_MXFP4) return (size_t)(n / kMx4Block) * kMx4Bytes;
    if (type == kRowQ3k) return (size_t)(n / kQ3kBlock) * kQ3kBytes;
    if (type == MOE_FMT_Q5K) return (size_t)(n / kQ4kBlock) * kQ5kBytes;
    if (type == MOE_FMT_Q6K) return (size_t)(n / kQ4kBlock) * kQ6kBytes;
    return (size_t)(n / kQ8Block) * kQ8Bytes;
}

__attribute__((target("avx2,fma")))
inline void widen_store(__m128i lo8, __m128i hi8, __m256 scale, __m256 offset, float* out) {
    // 16 unsigned bytes (lo8: bytes 0-7 in its low half, 8-15 in its high half;
    // likewise hi8 for bytes 16-31) -> 32 floats q * scale - offset
    const __m256 f0 = _mm256_cvtepi32_ps(_mm256_cvtepu8_epi32(lo8));
    const __m256 f1 = _mm256_cvtepi32_ps(_mm256_cvtepu8_epi32(_mm_srli_si128(lo8, 8)));
    const __m256 f2 = _mm256_cvtepi32_ps(_mm256_cvtepu8_epi32(hi8));
    const __m256 f3 = _mm256_cvtepi32_ps(_mm256_cvtepu8_epi32(_mm_srli_si128(hi8, 8)));
    _mm256_storeu_ps(out, _mm256_fmsub_ps(f0, scale, offset));
    _mm256_storeu_ps(out + 8, _mm256_fmsub_ps(f1, scale, offset));
    _mm256_storeu_ps(out + 16, _mm256_fmsub_ps(f2, scale, offset));
    _mm256_storeu_ps(out + 24, _mm256_fmsub_ps(f3, scale, offset));
}

// One Q4_K row of n weights (n / 256 super-blocks of 144 bytes: fp16 d and
// dmin, 12 bytes of 6-bit scales and mins, 128 bytes of nibbles; byte 32c + l
// holds element l of sub-block 2c in its low nibble and of sub-block 2c + 1
// in its high nibble) -> n floats d sc_j q - dmin m_j.
__attribute__((target("avx2,fma")))
void dequant_row_q4k(const uint8_t* row, int n, float* out) {
    const __m256i low4 = _mm256_set1_epi8(0x0F);
    for (int sb = 0; sb < n / kQ4kBlock; ++sb, row += kQ4kBytes, out += kQ4kBlock) {
        const float d = half_bits_to_float(load_u16(row)), dmin = half_bits_to_float(load_u16(row + 2));
        const uint8_t* s = row + 4;
        float dsc[8], dm[8];
        for (int j = 0; j < 8; ++j) {
            int sc, m;
            if (j < 4) {
                sc = s[j] & 63;
                m = s[j + 4] & 63;
            } else {
                sc = (s[j + 4] & 0x0F) | ((s[j - 4] >> 6) << 4);
                m = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
            }
            dsc[j] = d * (float)sc;
            dm[j] = dmin * (float)m;
        }
        const uint8_t* q = row + 16;
        for (int c = 0; c < 4; ++c) {
            const __m256i v = _mm256_loadu_si256(reinterpret_cast<const __m256i*>(q + 32 * c));
            const __m256i lo = _mm256_and_si256(v, low4);
            const __m256i hi = _mm256_and_si256(_mm256_srli_epi16(v, 4), low4);
            widen_store(_mm256_castsi256_si128(lo), _mm256_extracti128_si256(lo, 1), _mm256_set1_ps(dsc[2 * c]),
                        _mm256_set1_ps(dm[2 * c]), out + 64 * c);
            widen_store(_mm256_castsi256_si128(hi), _mm256_extracti128_si256(hi, 1), _mm256_set1_ps(dsc[2 * c + 1]),
                        _mm256_set1_ps(dm[2 * c + 1]), out + 64 * c + 32);
        }
    }
}

// One Q8_0 row of n weights (n / 32 blocks of 34 bytes: fp16 d, 32 int8)
// -> n floats d q.
__attribute__((target("avx2,fma")))
void dequant_row_q8_0(const uint8_t* row, int n, float* out) {
    for (int b = 0; b < n / kQ8Block; ++b, row += kQ8Bytes, out += kQ8Block) {
        const __m256 d = _mm256_set1_ps(half_bits_to_float(load_u16(row)));
        const __m128i q0 = _mm_loadu_si128(reinterpret_cast<const __m128i*>(row + 2));
        const __m128i q1 = _mm_loadu_si128(reinterpret_cast<const __m128i*>(row + 18));
        _mm256_storeu_ps(out, _mm256_mul_ps(_mm256_cvtepi32_ps(_mm256_cvtepi8_epi32(q0)), d));
        _mm256_storeu_ps(out + 8, _mm256_mul_ps(_mm256_cvtepi32_ps(_mm256_cvtepi8_epi32(_mm_srli_si128(q0, 8))), d));
        _mm256_storeu_ps(out + 16, _mm256_mul_ps(_mm256_cvtepi32_ps(_mm256_cvtepi8_epi32(q1)), d));
        _mm256_storeu_ps(out + 24, _mm256_mul_ps(_mm256_cvtepi32_ps(_mm256_cvtepi8_epi32(_mm_srli_si128(q1, 8))), d));
    }
}

// One MXFP4 row of n weights (n / 32 blocks of 17 bytes: an E8M0 scale byte
// X, then element i < 16 in the low nibble of byte 1 + i and 16 + i in its
// high nibble, FP4 E2M1 codes) -> n floats 2^(X - 127) fp4(q).  The code's
// magnitude (bits 0-2) selects one of the eight E2M1 values by a register
// permute, bit 3 becomes the float's sign; X builds the scale's bits
// directly (X = 0: the subnormal 2^-127, X = 255: NaN).
__attribute__((target("avx2,fma")))
void dequant_row_mxfp4(const uint8_t* row, int n, float* out) {
    const __m256 mag = _mm256_setr_ps(0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f);
    const __m256i seven = _mm256_set1_epi32(7), eight = _mm256_set1_epi32(8);
    const __m128i low4 = _mm_set1_epi8(0x0F);
    for (int b = 0; b < n / kMx4Block; ++b, row += kMx4Bytes, out += kMx4Block) {
        const uint32_t x = row[0];
        const uint32_t sbits = x == 0 ? 0x00400000u : (x == 255 ? 0x7FC00000u : x << 23);
        float sf;
        std::memcpy(&sf, &sbits, sizeof(sf));
        const __m256 scale = _mm256_set1_ps(sf);
        const __m128i v = _mm_loadu_si128(reinterpret_cast<const __m128i*>(row + 1));
        const __m128i lo = _mm_and_si128(v, low4);                        // elements 0-15
        const __m128i hi = _mm_and_si128(_mm_srli_epi16(v, 4), low4);     // elements 16-31
        const __m128i parts[4] = {lo, _mm_srli_si128(lo, 8), hi, _mm_srli_si128(hi, 8)};
        for (int k = 0; k < 4; ++k) {
            const __m256i c = _mm256_cvtepu8_epi32(parts[k]);
            const __m256 m = _mm256_permutevar8x32_ps(mag, _mm256_and_si256(c, seven));
            const __m256 sign = _mm256_castsi256_ps(_mm256_slli_epi32(_mm256_and_si256(c, eight), 28));
            _mm256_storeu_ps(out + 8 * k, _mm256_mul_ps(_mm256_xor_ps(m, sign), scale));
        }
    }
}

// One Q6_K row of n weights (n / 256 super-blocks of 210 bytes: 128 bytes of
// low nibbles, 64 bytes of high bit pairs, 16 signed scales, fp16 d; element
// 128h + 32g + l has its low four bits in byte 64h + l + 32 (g % 2), low
// nibble for g < 2, and its high two bits at bits 2g of byte 128 + 32h + l)
// -> n floats d sc_j (q - 32) = q (d sc_j) - 32 d sc_j, one fused
// multiply-subtract each (d sc_j is exact in fp32).
__attribute__((target("avx2,fma")))
void dequant_row_q6k(const uint8_t* row, int n, float* out) {
    const __m256i low4 = _mm256_set1_epi8(0x0F), three = _mm256_set1_epi8(3);
    for (int sb = 0; sb < n / kQ4kBlock; ++sb, row += kQ6kBytes, out += kQ4kBlock) {
        const float d = half_bits_to_float(load_u16(row + 208));
        const int8_t* sc = reinterpret_cast<const int8_t*>(row + 192);
        for (int h = 0; h < 2; ++h) {
            const __m256i hbytes = _mm256_loadu_si256(reinterpret_cast<const __m256i*>(row + 128 + 32 * h));
            for (int g = 0; g < 4; ++g) {
                const __m256i v = _mm256_loadu_si256(reinterpret_cast<const __m256i*>(row + 64 * h + 32 * (g % 2)));
                const __m256i nib = g < 2 ? _mm256_and_si256(v, low4) : _mm256_and_si256(_mm256_srli_epi16(v, 4), low4);
                const __m256i hb = _mm256_and_si256(_mm256_srli_epi16(hbytes, 2 * g), three);
                const __m256i qv = _mm256_or_si256(nib, _mm256_slli_epi16(hb, 4));
                const int j = 8 * h + 2 * g;  // sub-blocks j (elements 0-15) and j + 1 (16-31)
                const float s0 = d * (float)sc[j], s1 = d * (float)sc[j + 1];
                const __m128i lo8 = _mm256_castsi256_si128(qv), hi8 = _mm256_extracti128_si256(qv, 1);
                const __m256 a0 = _mm256_set1_ps(s0), a1 = _mm256_set1_ps(s1);
                const __m256 o0 = _mm256_set1_ps(32.0f * s0), o1 = _mm256_set1_ps(32.0f * s1);
                float* o = out + 128 * h + 32 * g;
                _mm256_storeu_ps(o, _mm256_fmsub_ps(_mm256_cvtepi32_ps(_mm256_cvtepu8_epi32(lo8)), a0, o0));
                _mm256_storeu_ps(o + 8, _mm256_fmsub_ps(_mm256_cvtepi32_ps(_mm256_cvtepu8_epi32(_mm_srli_si128(lo8, 8))), a0, o0));
                _mm256_storeu_ps(o + 16, _mm256_fmsub_ps(_mm256_cvtepi32_ps(_mm256_cvtepu8_epi32(hi8)), a1, o1));
                _mm256_storeu_ps(o + 24, _mm256_fmsub_ps(_mm256_cvtepi32_ps(_mm256_cvtepu8_epi32(_mm_srli_si128(hi8, 8))), a1, o1));
            }
        }
    }
}

// One Q5_K row of n weights (n / 256 super-blocks of 176 bytes: the Q4_K
// header, 32 bytes of high bits (bit j of byte l: element l of sub-block j),
// 128 bytes of nibbles in the Q4_K order) -> n floats d sc_j q - dmin m_j,
// q = nibble + 16 high bit.
__attribute__((target("avx2,fma")))
void dequant_row_q5k(const uint8_t* row, int n, float* out) {
    const __m256i low4 = _mm256_set1_epi8(0x0F), one = _mm256_set1_epi8(1);
    for (int sb = 0; sb < n / kQ4kBlock; ++sb, row += kQ5kBytes, out += kQ4kBlock) {
        const float d = half_bits_to_float(load_u16(row)), dmin = half_bits_to_float(load_u16(row + 2));
        const uint8_t* s = row + 4;
        float dsc[8], dm[8];
        for (int j = 0; j < 8; ++j) {
            int sc, m;
            if (j < 4) {
                sc = s[j] & 63;
                m = s[j + 4] & 63;
            } else {
                sc = (s[j + 4] & 0x0F) | ((s[j - 4] >> 6) << 4);
                m = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
            }
            dsc[j] = d * (float)sc;
            dm[j] = dmin * (float)m;
        }
        const __m256i hbits = _mm256_loadu_si256(reinterpret_cast<const __m256i*>(row + 16));
        const uint8_t* q = row + 48;
        for (int c = 0; c < 4; ++c) {
            const __m256i v = _mm256_loadu_si256(reinterpret_cast<const __m256i*>(q + 32 * c));
            for (int half = 0; half < 2; ++half) {
                const int j = 2 * c + half;
                const __m256i nib = half ? _mm256_and_si256(_mm256_srli_epi16(v, 4), low4) : _mm256_and_si256(v, low4);
                const __m256i hb = _mm256_and_si256(_mm256_srli_epi16(hbits, j), one);
                const __m256i qv = _mm256_or_si256(nib, _mm256_slli_epi16(hb, 4));
                widen_store(_mm256_castsi256_si128(qv), _mm256_extracti128_si256(qv, 1), _mm256_set1_ps(dsc[j]),
                            _mm256_set1_ps(dm[j]), out + 32 * j);
            }
        }
    }
}

// One Q3_K row of n weights (n / 256 super-blocks of 110 bytes: 32 bytes of
// high bits, 64 of 2-bit quants, 12 of 6-bit scales, fp16 d; element i =
// 128h + 32g + l has its low bits at bits 2g of quant byte 32h + l and its
// high bit at bit 4h + g of byte l; scale j of the 16-element sub-block i /
// 16: low nibble of byte j (j < 8) or the high nibble of byte j - 8, top two
// bits at bit 2 (j / 4) of byte 8 + j % 4) -> n floats d (sc_j - 32) (low + 4
// high - 4).  Per 32 elements (one g of one h), one 32-byte load of the
// quant bytes and of the high-bit bytes.
__attribute__((target("avx2,fma")))
void dequant_row_q3k(const uint8_t* row, int n, float* out) {
    const __m256i three = _mm256_set1_epi8(3), one = _mm256_set1_epi8(1);
    alignas(32) int8_t q[32];
    for (int sb = 0; sb < n / kQ3kBlock; ++sb, row += kQ3kBytes, out += kQ3kBlock) {
        const uint8_t* hm = row;
        const uint8_t* qs = row + 32;
        const uint8_t* s = row + 96;
        const float d = half_bits_to_float(load_u16(row + 108));
        float ds[16];
        for (int j = 0; j < 16; ++j) {
            const int lo = j < 8 ? (s[j] & 15) : (s[j - 8] >> 4);
            const int hi = (s[8 + j % 4] >> (2 * (j / 4))) & 3;
            ds[j] = d * (float)((lo | (hi << 4)) - 32);
        }
        const __m256i hbits = _mm256_loadu_si256(reinterpret_cast<const __m256i*>(hm));
        for (int h = 0; h < 2; ++h) {
            const __m256i qv = _mm256_loadu_si256(reinterpret_cast<const __m256i*>(qs + 32 * h));
            for (int g = 0; g < 4; ++g) {
                const __m256i low = _mm256_and_si256(_mm256_srli_epi16(qv, 2 * g), three);
                const __m256i high = _mm256_and_si256(_mm256_srli_epi16(hbits, 4 * h + g), one);
                // q = low + 4 high - 4, in -4..3
                const __m256i v = _mm256_sub_epi8(_mm256_add_epi8(low, _mm256_slli_epi16(high, 2)), _mm256_set1_epi8(4));
                _mm256_store_si256(reinterpret_cast<__m256i*>(q), v);
                float* o = out + 128 * h + 32 * g;
                for (int k = 0; k < 4; ++k) {
                    const __m256 f = _mm256_cvtepi32_ps(_mm256_cvtepi8_epi32(_mm_loadl_epi64(reinterpret_cast<const __m128i*>(q + 8 * k))));
                    _mm256_storeu_ps(o + 8 * k, _mm256_mul_ps(f, _mm256_set1_ps(ds[(128 * h + 32 * g + 8 * k) / 16])));
                }
            }
        }
    }
}

// sum_i a[i] b[i], n a multiple of 32: four 8-wide FMA accumulators, then a
// fixed reduction tree.
__attribute__((target("avx2,fma")))
float dot(const float* a, const float* b, int n) {
    __m256 s0 = _mm256_setzero_ps(), s1 = s0, s2 = s0, s3 = s0;
    for (int i = 0; i < n; i += 32) {
        s0 = _mm256_fmadd_ps(_mm256_loadu_ps(a + i), _mm256_loadu_ps(b + i), s0);
        s1 = _mm256_fmadd_ps(_mm256_loadu_ps(a + i + 8), _mm256_loadu_ps(b + i + 8), s1);
        s2 = _mm256_fmadd_ps(_mm256_loadu_ps(a + i + 16), _mm256_loadu_ps(b + i + 16), s2);
        s3 = _mm256_fmadd_ps(_mm256_loadu_ps(a + i + 24), _mm256_loadu_ps(b + i + 24), s3);
    }
    const __m256 s = _mm256_add_ps(_mm256_add_ps(s0, s1), _mm256_add_ps(s2, s3));
    const __m128 h = _mm_add_ps(_mm256_castps256_ps128(s), _mm256_extractf128_ps(s, 1));
    const __m128 h2 = _mm_add_ps(h, _mm_movehl_ps(h, h));
    return _mm_cvtss_f32(_mm_add_ss(h2, _mm_shuffle_ps(h2, h2, 1)));
}

bool cpu_supported() {
    __builtin_cpu_init();
    return __builtin_cpu_supports("avx2") && __builtin_cpu_supports("fma") && __builtin_cpu_supports("f16c");
}

__attribute__((target("avx2,fma")))
void run(int format, const uint8_t* const* expert_blob, int H, int I, const float* x, int T,
         const int32_t* host_token, const int32_t* host_expert, const float* host_weight, int count, float* y,
         int threads) {
    std::fill(y, y + (size_t)T * H, 0.0f);
    if (count == 0) return;
    std::vector<int> order(count);
    for (int p = 0; p < count; ++p) order[p] = p;
    std::stable_sort(order.begin(), order.end(),
                     [&](int a, int b) { return host_expert[a] < host_expert[b]; });
    const int nthreads = threads > 0 ? threads : omp_get_max_threads();
    // block types of the gate/up and down matrices (the mixed expert: Q3_K, then Q4_K)
    const int tgu = format == MOE_FMT_Q3K_Q4K ? kRowQ3k : format;
    const int tdn = format == MOE_FMT_Q3K_Q4K ? MOE_FMT_Q4K : format;
    const size_t rbH = row_bytes(tgu, H), rbI = row_bytes(tdn, I);
    auto pick = [](int type) {
        return type == MOE_FMT_Q4K ? dequant_row_q4k
             : type == MOE_FMT_MXFP4 ? dequant_row_mxfp4
             : type == kRowQ3k ? dequant_row_q3k
             : type == MOE_FMT_Q5K ? dequant_row_q5k
             : type == MOE_FMT_Q6K ? dequant_row_q6k
                               : dequant_row_q8_0;
    };
    auto dequant = pick(tgu);
    auto dequant_down = pick(tdn);
    std::vector<float> g, u;
    for (int g0 = 0; g0 < count;) {
        const int e = host_expert[order[g0]];
        int g1 = g0;
        while (g1 < count && host_expert[order[g1]] == e) ++g1;
        const int n = g1 - g0;
        const uint8_t* wg = expert_blob[e];
        const uint8_t* wu = wg + (size_t)I * rbH;
        const uint8_t* wd = wu + (size_t)I * rbH;
        g.assign((size_t)n * I, 0.0f);
        u.assign((size_t)n * I, 0.0f);
#pragma omp parallel num_threads(nthreads)
        {
            std::vector<float> wrow(std::max(H, I));
#pragma omp for schedule(static)
            for (int r = 0; r < I; ++r) {
                dequant(wg + (size_t)r * rbH, H, wrow.data());
                for (int t = 0; t < n; ++t) g[(size_t)t * I + r] = dot(wrow.data(), x + (size_t)host_token[order[g0 + t]] * H, H);
                dequant(wu + (size_t)r * rbH, H, wrow.data());
                for (int t = 0; t < n; ++t) u[(size_t)t * I + r] = dot(wrow.data(), x + (size_t)host_token[order[g0 + t]] * H, H);
            }
#pragma omp for schedule(static)
            for (size_t i = 0; i < (size_t)n * I; ++i) {
                const float z = g[i];
                g[i] = z / (1.0f + std::exp(-z)) * u[i];  // h
            }
#pragma omp for schedule(static)
            for (int c = 0; c < H; ++c) {
                dequant_down(wd + (size_t)c * rbI, I, wrow.data());
                for (int t = 0; t < n; ++t) {
                    const int p = order[g0 + t];
                    y[(size_t)host_token[p] * H + c] += host_weight[p] * dot(wrow.data(), g.data() + (size_t)t * I, I);
                }
            }
        }
        g0 = g1;
    }
}

}  // namespace

namespace qmoe_host {
// The library's one error text, also set by the residency policy.
__attribute__((visibility("hidden"))) int set_error(int status, const char* msg) {
    g_error = msg;
    return status;
}
}  // namespace qmoe_host

extern "C" {

const char* moe_host_last_error(void) { return g_error.c_str(); }

int moe_host_leg(int format, const uint8_t* const* expert_blob, int E, int H, int I, const float* x, int T,
                 const int32_t* host_token, const int32_t* host_expert, const float* host_weight, int count,
                 float* y_host, int threads) {
    if (format < MOE_FMT_Q8_0 || format > MOE_FMT_Q6K) return fail(MOE_ERR_UNSUPPORTED, "bad format %d", format);
    const int blk = (format == MOE_FMT_Q4K || format == MOE_FMT_Q3K_Q4K || format == MOE_FMT_Q5K ||
                     format == MOE_FMT_Q6K) ? kQ4kBlock
                    : format == MOE_FMT_MXFP4                           ? kMx4Block
                                                                        : kQ8Block;
    if (H <= 0 || I <= 0 || H % blk || I % blk)
        return fail(MOE_ERR_UNSUPPORTED, "H = %d and I = %d must be positive multiples of %d", H, I, blk);
    if (E < 1 || T < 0 || count < 0) return fail(MOE_ERR_INVALID_ARGUMENT, "E = %d, T = %d, count = %d", E, T, count);
    if (T > 0 && (!x || !y_host)) return fail(MOE_ERR_INVALID_ARGUMENT, "x and y_host must not be NULL");
    if (count > 0 && (!expert_blob || !host_token || !host_expert || !host_weight))
        return fail(MOE_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
    for (int p = 0; p < count; ++p) {
        const int t = host_token[p], e = host_expert[p];
        if (t < 0 || t >= T) return fail(MOE_ERR_INVALID_ARGUMENT, "pair %d: token %d outside [0, %d)", p, t, T);
        if (e < 0 || e >= E) return fail(MOE_ERR_INVALID_ARGUMENT, "pair %d: expert %d outside [0, %d)", p, e, E);
        if (!expert_blob[e]) return fail(MOE_ERR_INVALID_ARGUMENT, "pair %d: expert %d has no blob", p, e);
    }
    if (!cpu_supported()) return fail(MOE_ERR_UNSUPPORTED, "the host CPU lacks AVX2, FMA or F16C");
    if (T == 0) return MOE_OK;
    run(format, expert_blob, H, I, x, T, host_token, host_expert, host_weight, count, y_host, threads);
    return MOE_OK;
}

}  // extern "C"
