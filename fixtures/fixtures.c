/*
 * Seeded synthetic inputs for the routed-expert MoE layer.
 *
 * This module is shared by the HIP path and by the CPU oracle, and it holds
 * none of the layer's arithmetic: it draws random numbers and writes them in
 * the stored formats the layer reads.  Nothing here dequantizes, routes,
 * groups, multiplies or combines.
 *
 *   - Philox4x32-10, the counter-based generator of Salmon, Moraes, Dror and
 *     Shaw, "Parallel random numbers: as easy as 1, 2, 3" (SC'11): ten rounds
 *     of two 32x32->64 multiplies with a Weyl-sequence key schedule.  Each
 *     value is addressed by (seed, tag, counter), so the output does not depend
 *     on the thread count or on which process draws it.
 *   - Box-Muller (1958) for N(0,1) from two uniforms.
 *   - Gumbel(0,1) = -log(-log U); adding it to log-probabilities and taking
 *     the top k samples k categories without replacement (Gumbel-top-k, Kool,
 *     van Hoof and Welling, ICML 2019).  With Zipf rank probabilities this
 *     gives the skewed expert loads of the prefill and partial-residency
 *     workloads.
 *   - Encoders that turn float weights into the two stored block formats
 *     (weights arrive pre-quantized; the layer itself never quantizes):
 *       Q8_0: 34 bytes per 32 weights = fp16 d (little-endian) + 32 int8 q;
 *             w = d*q, d = absmax/127.
 *       Q4_K: 144 bytes per 256 weights = fp16 d, fp16 dmin, 12 bytes of
 *             packed 6-bit (scale, min) for eight 32-weight sub-blocks, then
 *             128 bytes of 4-bit quants; w = d*sc_j*q - dmin*m_j.
 *     The bloomery README (0.3.1) names these "k-quant" stored types in its
 *     Status table ("Quant types" row) and its "References and credits"
 *     section; the per-block formulas are the problem statement's.  The byte
 *     order inside a Q4_K block is the GGUF order as read here.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ Philox */

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

static inline void mulhilo(uint32_t a, uint32_t b, uint32_t* hi, uint32_t* lo) {
    uint64_t p = (uint64_t)a * (uint64_t)b;
    *hi = (uint32_t)(p >> 32);
    *lo = (uint32_t)p;
}

void fx_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
    uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int r = 0; r < 10; ++r) {
        uint32_t hi0, lo0, hi1, lo1;
        mulhilo(PHILOX_M0, c0, &hi0, &lo0);
        mulhilo(PHILOX_M1, c2, &hi1, &lo1);
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n1 = lo1;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        uint32_t n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
        k0 += PHILOX_W0;
        k1 += PHILOX_W1;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* Uniform in the open interval (0, 1): 24 random bits centred in their cell. */
static inline float u01(uint32_t r) { return ((float)(r >> 8) + 0.5f) * 0x1p-24f; }

/* Natural log on (0, 1]: x = m * 2^e with m in [sqrt(1/2), sqrt(2)), then
 * log m = 2 atanh(s), s = (m-1)/(m+1), |s| <= 0.172, by its odd series to s^11
 * (truncation < 1e-10).  Branch-free so the row loop vectorizes. */
static inline float bm_log(float x) {
    uint32_t bits;
    memcpy(&bits, &x, 4);
    int e = (int)((bits >> 23) & 0xFFu) - 127;
    uint32_t mb = (bits & 0x7FFFFFu) | 0x3F800000u;
    float m;
    memcpy(&m, &mb, 4);
    int big = m > 1.41421356f;
    m = m * (1.0f - 0.5f * (float)big);
    e = e + big;
    float s = (m - 1.0f) / (m + 1.0f);
    float s2 = s * s;
    float p = 1.0f / 11.0f;
    p = 1.0f / 9.0f + s2 * p;
    p = 1.0f / 7.0f + s2 * p;
    p = 1.0f / 5.0f + s2 * p;
    p = 1.0f / 3.0f + s2 * p;
    p = 1.0f + s2 * p;
    return 2.0f * s * p + (float)e * 0.693147180559945f;
}

/* sin and cos of 2*pi*u for u in (0, 1): reduce to b = 2*pi*(u - q/4) with
 * |b| <= pi/4 and quadrant q, then Taylor polynomials to b^11 / b^10. */
static inline void bm_sincos2pi(float u, float* sn, float* cs) {
    float q = (float)(int)(4.0f * u + 0.5f); /* floor, argument > 0: 0..4 */
    float r = u - 0.25f * q;           /* [-1/8, 1/8] */
    float b = 6.28318530717958647692f * r;
    float b2 = b * b;
    float sp = -1.0f / 39916800.0f;
    sp = 1.0f / 362880.0f + b2 * sp;
    sp = -1.0f / 5040.0f + b2 * sp;
    sp = 1.0f / 120.0f + b2 * sp;
    sp = -1.0f / 6.0f + b2 * sp;
    float sb = b + b * b2 * sp;
    float cp = -1.0f / 3628800.0f;
    cp = 1.0f / 40320.0f + b2 * cp;
    cp = -1.0f / 720.0f + b2 * cp;
    cp = 1.0f / 24.0f + b2 * cp;
    cp = -0.5f + b2 * cp;
    float cb = 1.0f + b2 * cp;
    int qi = ((int)q) & 3;
    /* quadrant qi: sin = (+sb, +cb, -sb, -cb), cos = (+cb, -sb, -cb, +sb) */
    float odd = (float)(qi & 1);
    float ssign = 1.0f - (float)(qi & 2);
    float csign = 1.0f - (float)((qi + 1) & 2);
    *sn = ssign * (odd * cb + (1.0f - odd) * sb);
    *cs = csign * (odd * sb + (1.0f - odd) * cb);
}

/* n normals of one "row" stream: Philox block c = counter (c, row, c2, c3)
 * gives four values, z = r*cos(t), r*sin(t) for the pairs (r0,r1), (r2,r3)
 * with r = sqrt(-2 log U), t = 2*pi*U' (Box-Muller). */
static void normal_row(uint32_t seed, uint32_t tag, uint32_t row, uint32_t c2, uint32_t c3,
                       float mean, float std, float* out, int64_t n) {
    enum { CH = 256 }; /* Philox blocks per batch */
    uint32_t key[2] = {seed, tag};
    uint32_t raw[CH * 4];
    float z[CH * 4];
    int64_t chunks = (n + 3) / 4;
    for (int64_t c0 = 0; c0 < chunks; c0 += CH) {
        int nb = (int)((chunks - c0) < CH ? (chunks - c0) : CH);
        for (int c = 0; c < nb; ++c) {
            uint32_t ctr[4] = {(uint32_t)(c0 + c), row, c2, c3};
            fx_philox4x32_10(ctr, key, raw + 4 * c);
        }
        for (int i = 0; i < 2 * nb; ++i) {
            float rad = sqrtf(-2.0f * bm_log(u01(raw[2 * i])));
            float sn, cs;
            bm_sincos2pi(u01(raw[2 * i + 1]), &sn, &cs);
            z[2 * i] = rad * cs;
            z[2 * i + 1] = rad * sn;
        }
        for (int i = 0; i < 4 * nb; ++i) {
            int64_t idx = c0 * 4 + i;
            if (idx < n) out[idx] = mean + std * z[i];
        }
    }
}

/* ------------------------------------------------------------ fp16 / bf16 */

/* float -> IEEE binary16 bits, round to nearest even (overflow -> inf). */
uint16_t fx_f32_to_f16(float f) {
    uint32_t x;
    memcpy(&x, &f, 4);
    uint32_t sign = (x >> 16) & 0x8000u;
    uint32_t ax = x & 0x7FFFFFFFu;
    if (ax >= 0x7F800000u) { /* inf or nan */
        return (uint16_t)(sign | 0x7C00u | (ax > 0x7F800000u ? 0x200u : 0u));
    }
    if (ax >= 0x477FF000u) return (uint16_t)(sign | 0x7C00u); /* rounds to >= 65520 */
    if (ax < 0x38800000u) {                                    /* below 2^-14: subnormal */
        if (ax < 0x33000000u) return (uint16_t)sign;           /* < 2^-25: rounds to 0 */
        uint32_t e = ax >> 23;
        uint32_t m = (ax & 0x7FFFFFu) | 0x800000u;
        uint32_t shift = 126u - e; /* 14..24 */
        uint32_t q = m >> shift;
        uint32_t rem = m & ((1u << shift) - 1u);
        uint32_t half = 1u << (shift - 1u);
        if (rem > half || (rem == half && (q & 1u))) ++q;
        return (uint16_t)(sign | q);
    }
    uint32_t e = (ax >> 23) - 127u + 15u;
    uint32_t m = ax & 0x7FFFFFu;
    uint32_t q = (e << 10) | (m >> 13);
    uint32_t rem = m & 0x1FFFu;
    if (rem > 0x1000u || (rem == 0x1000u && (q & 1u))) ++q;
    return (uint16_t)(sign | q);
}

float fx_f16_to_f32(uint16_t h) {
    uint32_t sign = ((uint32_t)h & 0x8000u) << 16;
    uint32_t e = (h >> 10) & 0x1Fu;
    uint32_t m = h & 0x3FFu;
    uint32_t x;
    if (e == 0) {
        if (m == 0) {
            x = sign;
        } else { /* subnormal: value m * 2^-24 */
            float v = (float)m * 0x1p-24f;
            memcpy(&x, &v, 4);
            x |= sign;
        }
    } else if (e == 31) {
        x = sign | 0x7F800000u | (m << 13);
    } else {
        x = sign | ((e - 15u + 127u) << 23) | (m << 13);
    }
    float f;
    memcpy(&f, &x, 4);
    return f;
}

/* float -> bfloat16 bits, round to nearest even (inputs are finite here). */
static inline uint16_t f32_to_bf16(float f) {
    uint32_t x;
    memcpy(&x, &f, 4);
    uint32_t lsb = (x >> 16) & 1u;
    x += 0x7FFFu + lsb;
    return (uint16_t)(x >> 16);
}

void fx_f32_to_bf16_array(const float* in, uint16_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16(in[i]);
}

/* ------------------------------------------------------------- encoders */

/* Round half away from zero for |v| < 2^31 (the encoders' arguments are
 * bounded by the clamp ranges plus rounding slack). */
static inline float round_half_away(float v) {
    float a = (float)(int)(fabsf(v) + 0.5f);
    return v >= 0.0f ? a : -a;
}

static inline void put_u16(uint8_t* p, uint16_t v) {
    p[0] = (uint8_t)(v & 0xFF);
    p[1] = (uint8_t)(v >> 8);
}

/* n floats (n % 32 == 0) -> n/32 Q8_0 blocks of 34 bytes. */
void fx_encode_q8_0(const float* x, int64_t n, uint8_t* out) {
    for (int64_t b = 0; b < n / 32; ++b) {
        const float* v = x + b * 32;
        uint8_t* o = out + b * 34;
        float amax = 0.0f;
        for (int i = 0; i < 32; ++i) {
            float a = fabsf(v[i]);
            if (a > amax) amax = a;
        }
        float d32 = amax / 127.0f;
        put_u16(o, fx_f32_to_f16(d32));
        for (int i = 0; i < 32; ++i) {
            float q = d32 > 0.0f ? round_half_away(v[i] / d32) : 0.0f;
            if (q > 127.0f) q = 127.0f;
            if (q < -127.0f) q = -127.0f;
            o[2 + i] = (uint8_t)(int8_t)q;
        }
    }
}

/* n floats (n % 256 == 0) -> n/256 Q4_K super-blocks of 144 bytes.
 * Per 32-weight sub-block j: lo = min(0, min x), hi = max x,
 * scale_j = (hi - lo)/15, min_j = -lo; d = fp16(max scale_j / 63),
 * dmin = fp16(max min_j / 63); sc_j, m_j are the 6-bit multiples of d and dmin;
 * q = round((x + dmin*m_j) / (d*sc_j)) clamped to [0, 15]. */
void fx_encode_q4k(const float* x, int64_t n, uint8_t* out) {
    for (int64_t b = 0; b < n / 256; ++b) {
        const float* v = x + b * 256;
        uint8_t* o = out + b * 144;
        float scale[8], mins[8];
        float maxscale = 0.0f, maxmin = 0.0f;
        for (int j = 0; j < 8; ++j) {
            float lo = 0.0f, hi = v[j * 32];
            for (int i = 0; i < 32; ++i) {
                float t = v[j * 32 + i];
                if (t < lo) lo = t;
                if (t > hi) hi = t;
            }
            scale[j] = (hi - lo) / 15.0f;
            mins[j] = -lo;
            if (scale[j] > maxscale) maxscale = scale[j];
            if (mins[j] > maxmin) maxmin = mins[j];
        }
        uint16_t dh = fx_f32_to_f16(maxscale / 63.0f);
        uint16_t mh = fx_f32_to_f16(maxmin / 63.0f);
        float df = fx_f16_to_f32(dh), mf = fx_f16_to_f32(mh);
        int sc[8], mm[8];
        for (int j = 0; j < 8; ++j) {
            float s = df > 0.0f ? round_half_away(scale[j] / df) : 0.0f;
            float m = mf > 0.0f ? round_half_away(mins[j] / mf) : 0.0f;
            sc[j] = s < 0.0f ? 0 : (s > 63.0f ? 63 : (int)s);
            mm[j] = m < 0.0f ? 0 : (m > 63.0f ? 63 : (int)m);
        }
        put_u16(o, dh);
        put_u16(o + 2, mh);
        uint8_t* s12 = o + 4;
        for (int j = 0; j < 4; ++j) {
            s12[j] = (uint8_t)((sc[j] & 63) | ((sc[j + 4] >> 4) << 6));
            s12[j + 4] = (uint8_t)((mm[j] & 63) | ((mm[j + 4] >> 4) << 6));
            s12[j + 8] = (uint8_t)((sc[j + 4] & 15) | ((mm[j + 4] & 15) << 4));
        }
        uint8_t* qs = o + 16;
        memset(qs, 0, 128);
        for (int j = 0; j < 8; ++j) {
            float step = df * (float)sc[j];
            float off = mf * (float)mm[j];
            for (int i = 0; i < 32; ++i) {
                float q = step > 0.0f ? round_half_away((v[j * 32 + i] + off) / step) : 0.0f;
                int qi = q < 0.0f ? 0 : (q > 15.0f ? 15 : (int)q);
                uint8_t* byte = qs + (j / 2) * 32 + i;
                if (j % 2 == 0) *byte |= (uint8_t)qi;
                else *byte |= (uint8_t)(qi << 4);
            }
        }
    }
}

/* n floats (n % 32 == 0) -> n/32 MXFP4 blocks of 17 bytes: an E8M0 scale
 * byte X, then element i < 16 in the low nibble of byte 1 + i and element
 * 16 + i in its high nibble, as FP4 (E2M1) codes.  The scale is the
 * smallest power of two s = 2^(X - 127) with 6 s >= max |x| (no element
 * saturates); each x / s goes to the nearest E2M1 magnitude (0, 0.5, 1,
 * 1.5, 2, 3, 4, 6), ties to the even code, with x's sign.  A zero block
 * stores X = 0 and zero codes. */
void fx_encode_mxfp4(const float* x, int64_t n, uint8_t* out) {
    static const float mag[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
    for (int64_t b = 0; b < n / 32; ++b) {
        const float* v = x + b * 32;
        uint8_t* o = out + b * 17;
        float amax = 0.0f;
        for (int i = 0; i < 32; ++i) {
            float a = fabsf(v[i]);
            if (a > amax) amax = a;
        }
        memset(o, 0, 17);
        if (amax == 0.0f) continue;
        int k;
        frexpf(amax / 6.0f, &k);  /* amax / 6 in [2^(k-1), 2^k) */
        while (k > -127 && 6.0f * ldexpf(1.0f, k - 1) >= amax) --k;
        while (6.0f * ldexpf(1.0f, k) < amax) ++k;
        if (k < -127) k = -127;
        if (k > 127) k = 127;
        o[0] = (uint8_t)(k + 127);
        const float s = ldexpf(1.0f, k);
        for (int i = 0; i < 32; ++i) {
            float a = fabsf(v[i]) / s;
            int best = 0;
            for (int c = 1; c < 8; ++c) {
                float dc = fabsf(a - mag[c]), db = fabsf(a - mag[best]);
                if (dc < db || (dc == db && (c & 1) == 0)) best = c;
            }
            int code = best | ((v[i] < 0.0f && best) ? 8 : 0);
            if (i < 16) o[1 + i] |= (uint8_t)code;
            else o[1 + i - 16] |= (uint8_t)(code << 4);
        }
    }
}

/* n floats (n % 256 == 0) -> n/256 Q3_K super-blocks of 110 bytes: 32
 * bytes of high bits, 64 bytes of 2-bit quants, 12 scale bytes, fp16 d.
 * Per 16-weight sub-block j: the element of largest magnitude m_j sets the
 * signed scale s_j = -m_j / 4 (it then encodes as -4); d = fp16(max |s_j| /
 * 31); sc_j = round(s_j / d) clamped to [-32, 31], stored + 32 in 6 bits;
 * q = round(x / (d sc_j)) clamped to [-4, 3], stored as q + 4 = low two bits
 * + 4 * high bit.  Element i: half h = i / 128, group g = (i % 128) / 32,
 * l = i % 32: low bits at bits 2g of qs[32h + l], high bit at bit 4h + g of
 * hmask[l].  Scale j: low nibble in byte j (j < 8) or the high nibble of
 * byte j - 8, top two bits at bit 2 (j / 4) of byte 8 + j % 4. */
void fx_encode_q3k(const float* x, int64_t n, uint8_t* out) {
    for (int64_t b = 0; b < n / 256; ++b) {
        const float* v = x + b * 256;
        uint8_t* o = out + b * 110;
        memset(o, 0, 110);
        float s[16], smax = 0.0f;
        for (int j = 0; j < 16; ++j) {
            float m = 0.0f;
            for (int i = 0; i < 16; ++i)
                if (fabsf(v[16 * j + i]) > fabsf(m)) m = v[16 * j + i];
            s[j] = -m / 4.0f;
            if (fabsf(s[j]) > smax) smax = fabsf(s[j]);
        }
        uint16_t dh = fx_f32_to_f16(smax / 31.0f);
        float df = fx_f16_to_f32(dh);
        uint8_t* hm = o;
        uint8_t* qs = o + 32;
        uint8_t* s12 = o + 96;
        for (int j = 0; j < 16; ++j) {
            float r = df > 0.0f ? round_half_away(s[j] / df) : 0.0f;
            int sc = r < -32.0f ? -32 : (r > 31.0f ? 31 : (int)r);
            int u = sc + 32;
            if (j < 8) s12[j] |= (uint8_t)(u & 15);
            else s12[j - 8] |= (uint8_t)((u & 15) << 4);
            s12[8 + j % 4] |= (uint8_t)((u >> 4) << (2 * (j / 4)));
            float step = df * (float)sc;
            for (int i = 0; i < 16; ++i) {
                int e = 16 * j + i;
                float q = step != 0.0f ? round_half_away(v[e] / step) : 0.0f;
                int qi = q < -4.0f ? -4 : (q > 3.0f ? 3 : (int)q);
                int w = qi + 4;
                int h = e / 128, g = (e % 128) / 32, l = e % 32;
                qs[32 * h + l] |= (uint8_t)((w & 3) << (2 * g));
                hm[l] |= (uint8_t)((w >> 2) << (4 * h + g));
            }
        }
        put_u16(o + 108, dh);
    }
}

/* n floats (n % 256 == 0) -> n/256 Q5_K super-blocks of 176 bytes: the
 * Q4_K scheme with 31 levels (scale_j = (hi - lo) / 31, q clamped to
 * [0, 31]); fp16 d, dmin, the 12 scale bytes as in Q4_K, then 32 bytes of
 * high bits (bit j of byte l: element l of sub-block j), then the low
 * nibbles in the Q4_K order. */
void fx_encode_q5k(const float* x, int64_t n, uint8_t* out) {
    for (int64_t b = 0; b < n / 256; ++b) {
        const float* v = x + b * 256;
        uint8_t* o = out + b * 176;
        memset(o, 0, 176);
        float scale[8], mins[8], maxscale = 0.0f, maxmin = 0.0f;
        for (int j = 0; j < 8; ++j) {
            float lo = 0.0f, hi = v[j * 32];
            for (int i = 0; i < 32; ++i) {
                float t = v[j * 32 + i];
                if (t < lo) lo = t;
                if (t > hi) hi = t;
            }
            scale[j] = (hi - lo) / 31.0f;
            mins[j] = -lo;
            if (scale[j] > maxscale) maxscale = scale[j];
            if (mins[j] > maxmin) maxmin = mins[j];
        }
        uint16_t dh = fx_f32_to_f16(maxscale / 63.0f), mh = fx_f32_to_f16(maxmin / 63.0f);
        float df = fx_f16_to_f32(dh), mf = fx_f16_to_f32(mh);
        int sc[8], mm[8];
        for (int j = 0; j < 8; ++j) {
            float s2 = df > 0.0f ? round_half_away(scale[j] / df) : 0.0f;
            float m2 = mf > 0.0f ? round_half_away(mins[j] / mf) : 0.0f;
            sc[j] = s2 < 0.0f ? 0 : (s2 > 63.0f ? 63 : (int)s2);
            mm[j] = m2 < 0.0f ? 0 : (m2 > 63.0f ? 63 : (int)m2);
        }
        put_u16(o, dh);
        put_u16(o + 2, mh);
        uint8_t* s12 = o + 4;
        for (int j = 0; j < 4; ++j) {
            s12[j] = (uint8_t)((sc[j] & 63) | ((sc[j + 4] >> 4) << 6));
            s12[j + 4] = (uint8_t)((mm[j] & 63) | ((mm[j + 4] >> 4) << 6));
            s12[j + 8] = (uint8_t)((sc[j + 4] & 15) | ((mm[j + 4] & 15) << 4));
        }
        uint8_t* qh = o + 16;
        uint8_t* qs = o + 48;
        for (int j = 0; j < 8; ++j) {
            float step = df * (float)sc[j], off = mf * (float)mm[j];
            for (int i = 0; i < 32; ++i) {
                float q = step > 0.0f ? round_half_away((v[j * 32 + i] + off) / step) : 0.0f;
                int qi = q < 0.0f ? 0 : (q > 31.0f ? 31 : (int)q);
                qs[(j / 2) * 32 + i] |= (uint8_t)((qi & 15) << (4 * (j % 2)));
                qh[i] |= (uint8_t)((qi >> 4) << j);
            }
        }
    }
}

/* n floats (n % 256 == 0) -> n/256 Q6_K super-blocks of 210 bytes.  Per
 * 16-weight sub-block j: the element of largest magnitude m_j sets the
 * signed scale s_j = -m_j / 32 (it encodes as q - 32 = -32); d = fp16(max
 * |s_j| / 127); sc_j = round(s_j / d) clamped to [-128, 127]; q - 32 =
 * round(x / (d sc_j)) clamped to [-32, 31].  Layout: low nibbles (element
 * 128h + 32g + l: byte 64h + l + 32 (g % 2), low nibble for g < 2), high bit
 * pairs (bits 2g of byte 128 + 32h + l), the 16 scales, fp16 d. */
void fx_encode_q6k(const float* x, int64_t n, uint8_t* out) {
    for (int64_t b = 0; b < n / 256; ++b) {
        const float* v = x + b * 256;
        uint8_t* o = out + b * 210;
        memset(o, 0, 210);
        float s[16], smax = 0.0f;
        for (int j = 0; j < 16; ++j) {
            float m = 0.0f;
            for (int i = 0; i < 16; ++i)
                if (fabsf(v[16 * j + i]) > fabsf(m)) m = v[16 * j + i];
            s[j] = -m / 32.0f;
            if (fabsf(s[j]) > smax) smax = fabsf(s[j]);
        }
        uint16_t dh = fx_f32_to_f16(smax / 127.0f);
        float df = fx_f16_to_f32(dh);
        for (int j = 0; j < 16; ++j) {
            float r = df > 0.0f ? round_half_away(s[j] / df) : 0.0f;
            int sc = r < -128.0f ? -128 : (r > 127.0f ? 127 : (int)r);
            o[192 + j] = (uint8_t)(int8_t)sc;
            float step = df * (float)sc;
            for (int i = 0; i < 16; ++i) {
                int e = 16 * j + i;
                float q = step != 0.0f ? round_half_away(v[e] / step) : 0.0f;
                int qi = (q < -32.0f ? -32 : (q > 31.0f ? 31 : (int)q)) + 32;
                int h = e / 128, g = (e % 128) / 32, l = e % 32;
                o[64 * h + l + 32 * (g % 2)] |= (uint8_t)((qi & 15) << (g < 2 ? 0 : 4));
                o[128 + 32 * h + l] |= (uint8_t)((qi >> 4) << (2 * g));
            }
        }
        put_u16(o + 208, dh);
    }
}

/* ------------------------------------------------------------- experts */

/* Block types; FX_Q3K_Q4K is the mixed expert (Q3_K gate and up, Q4_K down). */
enum { FX_Q8_0 = 0, FX_Q4K = 1, FX_MXFP4 = 2, FX_Q3K_Q4K = 3, FX_Q5K = 4, FX_Q6K = 5, FX_Q3K = 100 };

static int gate_up_fmt(int fmt) { return fmt == FX_Q3K_Q4K ? FX_Q3K : fmt; }
static int down_fmt(int fmt) { return fmt == FX_Q3K_Q4K ? FX_Q4K : fmt; }

static int64_t row_bytes(int fmt, int64_t cols) {
    switch (fmt) {
        case FX_Q8_0: return cols / 32 * 34;
        case FX_MXFP4: return cols / 32 * 17;
        case FX_Q3K: return cols / 256 * 110;
        case FX_Q5K: return cols / 256 * 176;
        case FX_Q6K: return cols / 256 * 210;
        default: return cols / 256 * 144;
    }
}

static void encode_row(int fmt, const float* x, int64_t n, uint8_t* out) {
    if (fmt == FX_Q8_0) fx_encode_q8_0(x, n, out);
    else if (fmt == FX_MXFP4) fx_encode_mxfp4(x, n, out);
    else if (fmt == FX_Q3K) fx_encode_q3k(x, n, out);
    else if (fmt == FX_Q5K) fx_encode_q5k(x, n, out);
    else if (fmt == FX_Q6K) fx_encode_q6k(x, n, out);
    else fx_encode_q4k(x, n, out);
}

int64_t fx_matrix_bytes(int fmt, int64_t rows, int64_t cols) { return rows * row_bytes(fmt, cols); }

/* Canonical expert blob = W_gate [I x H] | W_up [I x H] | W_down [H x I],
 * every matrix row-major with blocks along its input dimension. */
int64_t fx_expert_bytes(int fmt, int64_t H, int64_t I) {
    return 2 * fx_matrix_bytes(gate_up_fmt(fmt), I, H) + fx_matrix_bytes(down_fmt(fmt), H, I);
}

/* One seeded matrix: element (r, c) ~ N(0, std) from counter (chunk, r, expert, layer),
 * key (seed, 0x57000000 | matrix). */
static void gen_matrix(int fmt, uint32_t seed, uint32_t layer, uint32_t expert, uint32_t matrix,
                       int64_t rows, int64_t cols, float std, uint8_t* out) {
    int64_t rb = row_bytes(fmt, cols);
#pragma omp parallel
    {
        float* buf = (float*)malloc((size_t)cols * sizeof(float));
#pragma omp for schedule(static)
        for (int64_t r = 0; r < rows; ++r) {
            normal_row(seed, 0x57000000u | matrix, (uint32_t)r, expert, layer, 0.0f, std, buf, cols);
            encode_row(fmt, buf, cols, out + r * rb);
        }
        free(buf);
    }
}

void fx_gen_expert(int fmt, uint32_t seed, uint32_t layer, uint32_t expert, int64_t H, int64_t I, float std,
                   uint8_t* out) {
    int64_t gb = fx_matrix_bytes(gate_up_fmt(fmt), I, H);
    gen_matrix(gate_up_fmt(fmt), seed, layer, expert, 0, I, H, std, out);
    gen_matrix(gate_up_fmt(fmt), seed, layer, expert, 1, I, H, std, out + gb);
    gen_matrix(down_fmt(fmt), seed, layer, expert, 2, H, I, std, out + 2 * gb);
}

/* Several experts at once, one parallel loop over every row of every matrix:
 * out[i] = fx_gen_expert(fmt, seed, layer, experts[i], ...), blob i at
 * out + i * fx_expert_bytes(fmt, H, I). */
void fx_gen_experts(int fmt, uint32_t seed, uint32_t layer, const int32_t* experts, int n, int64_t H, int64_t I,
                    float std, uint8_t* out) {
    int64_t eb = fx_expert_bytes(fmt, H, I);
    int64_t gb = fx_matrix_bytes(gate_up_fmt(fmt), I, H);
    int64_t rbH = row_bytes(gate_up_fmt(fmt), H), rbI = row_bytes(down_fmt(fmt), I);
    int64_t rows_per_expert = 2 * I + H;
    int64_t total = (int64_t)n * rows_per_expert;
#pragma omp parallel
    {
        float* buf = (float*)malloc((size_t)(H > I ? H : I) * sizeof(float));
#pragma omp for schedule(dynamic, 64)
        for (int64_t g = 0; g < total; ++g) {
            int64_t i = g / rows_per_expert, r = g % rows_per_expert;
            uint32_t matrix = r < I ? 0u : (r < 2 * I ? 1u : 2u);
            int64_t row = matrix == 2 ? r - 2 * I : r - (int64_t)matrix * I;
            int64_t cols = matrix == 2 ? I : H;
            uint8_t* dst = out + i * eb + (matrix == 2 ? 2 * gb + row * rbI : matrix * gb + row * rbH);
            normal_row(seed, 0x57000000u | matrix, (uint32_t)row, (uint32_t)experts[i], layer, 0.0f, std, buf, cols);
            encode_row(matrix == 2 ? down_fmt(fmt) : gate_up_fmt(fmt), buf, cols, dst);
        }
        free(buf);
    }
}

/* Dense float copy of one generated matrix (before encoding), for tests of the encoders. */
void fx_gen_matrix_f32(uint32_t seed, uint32_t layer, uint32_t expert, uint32_t matrix, int64_t rows,
                       int64_t cols, float std, float* out) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        normal_row(seed, 0x57000000u | matrix, (uint32_t)r, expert, layer, 0.0f, std, out + r * cols, cols);
}

/* --------------------------------------------------------- activations */

/* rows x cols normals: counter (chunk, row, layer, 0), key (seed, tag). */
void fx_normal_rows(uint32_t seed, uint32_t tag, uint32_t layer, int64_t rows, int64_t cols, float mean, float std,
                    float* out) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        normal_row(seed, tag, (uint32_t)r, layer, 0, mean, std, out + r * cols, cols);
}

static int cmp_float(const void* a, const void* b) {
    float x = *(const float*)a, y = *(const float*)b;
    return (x > y) - (x < y);
}

static int row_has_tie(const float* v, int E, float* scratch) {
    memcpy(scratch, v, (size_t)E * sizeof(float));
    qsort(scratch, (size_t)E, sizeof(float), cmp_float);
    for (int i = 1; i < E; ++i)
        if (scratch[i] == scratch[i - 1]) return 1;
    return 0;
}

/* Gate logits N(0,1), [T x E].  A row with two equal values is drawn again
 * (attempt index in the last counter word), so ties never occur. */
void fx_logits_normal(uint32_t seed, uint32_t layer, int64_t T, int E, float* out) {
#pragma omp parallel
    {
        float* scratch = (float*)malloc((size_t)E * sizeof(float));
#pragma omp for schedule(static)
        for (int64_t t = 0; t < T; ++t) {
            float* row = out + t * E;
            for (uint32_t attempt = 0;; ++attempt) {
                normal_row(seed, 0x4C000000u, (uint32_t)t, layer, attempt, 0.0f, 1.0f, row, E);
                if (!row_has_tie(row, E, scratch)) break;
            }
        }
        free(scratch);
    }
}

/* A seeded permutation of 0..E-1 (Fisher-Yates, uniform index by rejection). */
void fx_permutation(uint32_t seed, uint32_t layer, int E, int32_t* perm) {
    for (int i = 0; i < E; ++i) perm[i] = i;
    uint32_t key[2] = {seed, 0x50000000u};
    for (int i = E - 1; i > 0; --i) {
        uint32_t bound = (uint32_t)(i + 1);
        uint32_t limit = (uint32_t)(0x100000000ull - (0x100000000ull % bound));
        uint32_t draw = 0;
        for (uint32_t attempt = 0;; ++attempt) {
            uint32_t ctr[4] = {(uint32_t)i, layer, attempt, 0};
            uint32_t r[4];
            fx_philox4x32_10(ctr, key, r);
            if (r[0] < limit || limit == 0) {
                draw = r[0] % bound;
                break;
            }
        }
        int32_t t = perm[i];
        perm[i] = perm[draw];
        perm[draw] = t;
    }
}

/* Zipf-skewed gate logits: l[t][e] = log p(rank_of[e]) + Gumbel(0,1), with
 * p(r) = r^-s / sum_r' r'^-s over ranks r = 1..E and rank_of[e] = perm[e] + 1
 * (perm drawn from perm_seed, the Gumbel noise from seed).  Taking the top k
 * of such a row samples k experts without replacement with probabilities p,
 * so expert loads follow the Zipf law.  Ties redrawn. */
void fx_logits_zipf(uint32_t seed, uint32_t perm_seed, uint32_t layer, int64_t T, int E, double s, float* out) {
    int32_t* perm = (int32_t*)malloc((size_t)E * sizeof(int32_t));
    double* logp = (double*)malloc((size_t)E * sizeof(double));
    fx_permutation(perm_seed, layer, E, perm);
    double z = 0.0;
    for (int r = 1; r <= E; ++r) z += pow((double)r, -s);
    for (int e = 0; e < E; ++e) logp[e] = -s * log((double)(perm[e] + 1)) - log(z);
#pragma omp parallel
    {
        float* scratch = (float*)malloc((size_t)E * sizeof(float));
#pragma omp for schedule(static)
        for (int64_t t = 0; t < T; ++t) {
            float* row = out + t * E;
            uint32_t key[2] = {seed, 0x47000000u};
            for (uint32_t attempt = 0;; ++attempt) {
                for (int c = 0; c < (E + 3) / 4; ++c) {
                    uint32_t ctr[4] = {(uint32_t)c, (uint32_t)t, layer, attempt};
                    uint32_t r[4];
                    fx_philox4x32_10(ctr, key, r);
                    for (int i = 0; i < 4; ++i) {
                        int e = c * 4 + i;
                        if (e < E) {
                            double u = ((double)(r[i] >> 8) + 0.5) * 0x1p-24;
                            double g = -log(-log(u));
                            row[e] = (float)(logp[e] + g);
                        }
                    }
                }
                if (!row_has_tie(row, E, scratch)) break;
            }
        }
        free(scratch);
    }
    free(perm);
    free(logp);
}

int fx_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void fx_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
