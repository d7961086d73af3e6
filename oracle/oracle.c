/*
 * CPU oracle for one routed-expert MoE layer: plain, slow, fp64.
 * TEST INFRASTRUCTURE ONLY (see oracle.h for who may use it and what it
 * computes).  Every loop follows the definition in the order it is stated;
 * nothing is blocked, fused or reordered.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

void oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int oracle_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* IEEE binary16, little-endian bytes -> exact double. */
static double half_le(const uint8_t* p) {
    unsigned h = (unsigned)p[0] | ((unsigned)p[1] << 8);
    int sign = (h >> 15) & 1;
    int exp = (h >> 10) & 31;
    int man = h & 1023;
    double v;
    if (exp == 0) v = ldexp((double)man, -24);                   /* subnormal or zero */
    else if (exp == 31) v = man ? NAN : INFINITY;                /* inf / nan */
    else v = ldexp((double)(1024 + man), exp - 25);              /* (1 + man/1024) * 2^(exp-15) */
    return sign ? -v : v;
}

/* ------------------------------------------------------------ dequant */

/* Q8_0 block (34 bytes): fp16 d, then 32 signed bytes q; w_i = d * q_i.
 * Parity pinned by hand-built golden blocks and the encoder round trip. */
void oracle_dequant_q8_0(const uint8_t* blocks, int64_t n, double* out) {
    for (int64_t b = 0; b < n / 32; ++b) {
        const uint8_t* blk = blocks + b * 34;
        double d = half_le(blk);
        for (int i = 0; i < 32; ++i) {
            int q = (int)(int8_t)blk[2 + i];
            out[b * 32 + i] = d * (double)q;
        }
    }
}

/* 6-bit scale and min of sub-block j (0..7) from the 12 packed bytes:
 * j < 4: sc = low 6 bits of byte j, m = low 6 bits of byte j+4;
 * j >= 4: sc = low nibble of byte j+4 | (top 2 bits of byte j-4) << 4,
 *         m  = high nibble of byte j+4 | (top 2 bits of byte j) << 4. */
static void q4k_scale_min(const uint8_t* s12, int j, int* sc, int* m) {
    if (j < 4) {
        *sc = s12[j] & 63;
        *m = s12[j + 4] & 63;
    } else {
        int hi_sc = s12[j - 4] >> 6;
        *sc = (s12[j + 4] & 15) | (hi_sc << 4);
        *m = (s12[j + 4] >> 4) | ((s12[j] >> 6) << 4);
    }
}

/* Q4_K super-block (144 bytes): fp16 d, fp16 dmin, 12 scale bytes, 128 quant
 * bytes.  Quant byte 32*c + l holds element l of sub-block 2c in its low
 * nibble and element l of sub-block 2c+1 in its high nibble.
 * w = d * sc_j * q - dmin * m_j.
 * Parity pinned by hand-built golden blocks (all 64x64 scale/min values at
 * every sub-block position) and the encoder round trip. */
void oracle_dequant_q4k(const uint8_t* blocks, int64_t n, double* out) {
    for (int64_t b = 0; b < n / 256; ++b) {
        const uint8_t* blk = blocks + b * 144;
        double d = half_le(blk);
        double dmin = half_le(blk + 2);
        const uint8_t* s12 = blk + 4;
        const uint8_t* qs = blk + 16;
        for (int j = 0; j < 8; ++j) {
            int sc, m;
            q4k_scale_min(s12, j, &sc, &m);
            int high = (j % 2 == 1);
            for (int l = 0; l < 32; ++l) {
                uint8_t byte = qs[(j / 2) * 32 + l];
                int q = high ? (byte >> 4) : (byte & 15);
                double w = d * (double)sc * (double)q;
                w -= dmin * (double)m;
                out[b * 256 + j * 32 + l] = w;
            }
        }
    }
}

/* One FP4 (E2M1) code, OCP Microscaling Formats (MX) v1.0, element type
 * FP4: bit 3 sign, bits 2-1 exponent (bias 1), bit 0 mantissa; exponent 0
 * is subnormal (0 or 0.5), otherwise (1 + m/2) 2^(e - 1). */
static double e2m1_value(int code) {
    int sign = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    double v = e == 0 ? 0.5 * (double)m : ldexp(1.0 + 0.5 * (double)m, e - 1);
    return sign ? -v : v;
}

/* MXFP4 block (17 bytes): one E8M0 scale byte X (2^(X - 127); X = 255 is
 * NaN), then 16 bytes of FP4 codes: element i < 16 in the low nibble of byte
 * 1 + i, element 16 + i in its high nibble.  w_i = 2^(X - 127) * fp4(q_i).
 * Parity pinned by hand-built golden blocks (every code, extreme scales)
 * and the encoder round trip. */
void oracle_dequant_mxfp4(const uint8_t* blocks, int64_t n, double* out) {
    for (int64_t b = 0; b < n / 32; ++b) {
        const uint8_t* blk = blocks + b * 17;
        int x = blk[0];
        double scale = x == 255 ? NAN : ldexp(1.0, x - 127);
        for (int i = 0; i < 32; ++i) {
            int code = i < 16 ? (blk[1 + i] & 15) : (blk[1 + i - 16] >> 4);
            out[b * 32 + i] = scale * e2m1_value(code);
        }
    }
}

/* 6-bit scale of sub-block j (0..15) from the 12 packed bytes: low four
 * bits from byte j (j < 8) or the high nibble of byte j - 8 (j >= 8); top two
 * bits from byte 8 + j % 4, at bit 2 * (j / 4). */
static int q3k_scale(const uint8_t* s12, int j) {
    int lo = j < 8 ? (s12[j] & 15) : (s12[j - 8] >> 4);
    int hi = (s12[8 + j % 4] >> (2 * (j / 4))) & 3;
    return lo | (hi << 4);
}

/* Q3_K super-block (110 bytes): 32 bytes of high bits (hmask), 64 bytes of
 * 2-bit quants (qs), 12 scale bytes, fp16 d.  Element i: half h = i / 128,
 * group g = (i % 128) / 32, l = i % 32; its low two bits are bits 2g..2g+1 of
 * qs[32h + l], its high bit is bit 4h + g of hmask[l]; q = low + 4 * high - 4
 * (in -4..3).  Sub-block j = i / 16 has the 6-bit scale sc_j.
 * w = d * (sc_j - 32) * q.
 * Parity pinned by hand-built golden blocks and the encoder round trip. */
void oracle_dequant_q3k(const uint8_t* blocks, int64_t n, double* out) {
    for (int64_t b = 0; b < n / 256; ++b) {
        const uint8_t* blk = blocks + b * 110;
        const uint8_t* hm = blk;
        const uint8_t* qs = blk + 32;
        const uint8_t* s12 = blk + 96;
        double d = half_le(blk + 108);
        for (int i = 0; i < 256; ++i) {
            int h = i / 128, g = (i % 128) / 32, l = i % 32;
            int low = (qs[32 * h + l] >> (2 * g)) & 3;
            int high = (hm[l] >> (4 * h + g)) & 1;
            int q = low + 4 * high - 4;
            int sc = q3k_scale(s12, i / 16) - 32;
            out[b * 256 + i] = d * (double)sc * (double)q;
        }
    }
}

/* Q5_K super-block (176 bytes): fp16 d, fp16 dmin, 12 scale bytes (the Q4_K
 * packing), 32 bytes of high bits (qh), 128 bytes of low nibbles (the Q4_K
 * order).  Element l of sub-block j: low four bits as in Q4_K, high bit =
 * bit j of qh[l]; q = low + 16 * high (0..31).  w = d * sc_j * q - dmin * m_j.
 * Parity pinned by hand-built golden blocks and the encoder round trip. */
void oracle_dequant_q5k(const uint8_t* blocks, int64_t n, double* out) {
    for (int64_t b = 0; b < n / 256; ++b) {
        const uint8_t* blk = blocks + b * 176;
        double d = half_le(blk);
        double dmin = half_le(blk + 2);
        const uint8_t* s12 = blk + 4;
        const uint8_t* qh = blk + 16;
        const uint8_t* qs = blk + 48;
        for (int j = 0; j < 8; ++j) {
            int sc, m;
            q4k_scale_min(s12, j, &sc, &m);
            for (int l = 0; l < 32; ++l) {
                uint8_t byte = qs[(j / 2) * 32 + l];
                int low = (j % 2) ? (byte >> 4) : (byte & 15);
                int high = (qh[l] >> j) & 1;
                int q = low + 16 * high;
                out[b * 256 + j * 32 + l] = d * (double)sc * (double)q - dmin * (double)m;
            }
        }
    }
}

/* Q6_K super-block (210 bytes): 128 bytes of low nibbles (ql), 64 bytes of
 * high bit pairs (qh), 16 signed 8-bit scales, fp16 d.  Element i: half
 * h = i / 128, quarter g = (i % 128) / 32, l = i % 32; low four bits from
 * ql[64h + l + 32 (g % 2)], its low nibble for g < 2 and high nibble
 * otherwise; high two bits = bits 2g..2g+1 of qh[32h + l]; q = low + 16 *
 * high (0..63).  Sub-block j = i / 16 has the signed scale sc_j.
 * w = d * sc_j * (q - 32).
 * Parity pinned by hand-built golden blocks and the encoder round trip. */
void oracle_dequant_q6k(const uint8_t* blocks, int64_t n, double* out) {
    for (int64_t b = 0; b < n / 256; ++b) {
        const uint8_t* blk = blocks + b * 210;
        const uint8_t* ql = blk;
        const uint8_t* qh = blk + 128;
        const int8_t* sc = (const int8_t*)(blk + 192);
        double d = half_le(blk + 208);
        for (int i = 0; i < 256; ++i) {
            int h = i / 128, g = (i % 128) / 32, l = i % 32;
            uint8_t byte = ql[64 * h + l + 32 * (g % 2)];
            int low = g < 2 ? (byte & 15) : (byte >> 4);
            int high = (qh[32 * h + l] >> (2 * g)) & 3;
            int q = low + 16 * high - 32;
            out[b * 256 + i] = d * (double)sc[i / 16] * (double)q;
        }
    }
}

static void dequant_row(int fmt, const uint8_t* row, int64_t n, double* out) {
    if (fmt == ORACLE_Q8_0) oracle_dequant_q8_0(row, n, out);
    else if (fmt == ORACLE_MXFP4) oracle_dequant_mxfp4(row, n, out);
    else if (fmt == ORACLE_Q3K) oracle_dequant_q3k(row, n, out);
    else if (fmt == ORACLE_Q5K) oracle_dequant_q5k(row, n, out);
    else if (fmt == ORACLE_Q6K) oracle_dequant_q6k(row, n, out);
    else oracle_dequant_q4k(row, n, out);
}

static int64_t row_bytes(int fmt, int64_t cols) {
    switch (fmt) {
        case ORACLE_Q8_0: return cols / 32 * 34;
        case ORACLE_MXFP4: return cols / 32 * 17;
        case ORACLE_Q3K: return cols / 256 * 110;
        case ORACLE_Q5K: return cols / 256 * 176;
        case ORACLE_Q6K: return cols / 256 * 210;
        default: return cols / 256 * 144;
    }
}

/* Block types of an expert's gate/up and down matrices: one type for both,
 * except the mixed expert (Q3_K gate and up, Q4_K down). */
static int gate_up_fmt(int fmt) { return fmt == ORACLE_Q3K_Q4K ? ORACLE_Q3K : fmt; }
static int down_fmt(int fmt) { return fmt == ORACLE_Q3K_Q4K ? ORACLE_Q4K : fmt; }

/* ------------------------------------------------------------- routing */

/* Does expert a come before expert b?  Larger logit first; equal logits:
 * lower id first.  Parity pinned against a library stable argsort. */
static int ranks_before(float la, int a, float lb, int b) {
    if (la != lb) return la > lb;
    return a < b;
}

int oracle_route(const float* logits, int T, int E, int k, int score, int renormalize, double scale,
                 int32_t* ids, double* w) {
    if (T < 0 || E <= 0 || k <= 0 || k > E) return -1;
    int* taken = (int*)calloc((size_t)E, sizeof(int));
    double* p = (double*)malloc((size_t)E * sizeof(double));
    for (int t = 0; t < T; ++t) {
        const float* l = logits + (int64_t)t * E;
        memset(taken, 0, (size_t)E * sizeof(int));
        /* selection: k passes, each picks the first remaining expert in rank order */
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || ranks_before(l[e], e, l[best], best)) best = e;
            }
            taken[best] = 1;
            ids[(int64_t)t * k + j] = best;
        }
        /* scores of all experts */
        if (score == ORACLE_SOFTMAX) {
            double mx = -INFINITY;
            for (int e = 0; e < E; ++e) mx = fmax(mx, (double)l[e]);
            double z = 0.0;
            for (int e = 0; e < E; ++e) z += exp((double)l[e] - mx);
            for (int e = 0; e < E; ++e) p[e] = exp((double)l[e] - mx) / z;
        } else {
            for (int e = 0; e < E; ++e) p[e] = 1.0 / (1.0 + exp(-(double)l[e]));
        }
        double sel = 0.0;
        for (int j = 0; j < k; ++j) sel += p[ids[(int64_t)t * k + j]];
        for (int j = 0; j < k; ++j) {
            double v = p[ids[(int64_t)t * k + j]];
            w[(int64_t)t * k + j] = renormalize ? scale * (v / sel) : scale * v;
        }
    }
    free(taken);
    free(p);
    return 0;
}

/* ------------------------------------------------------------- batches */

/* Parity pinned against a library stable sort and by the invariants
 * (bijection onto [0, offsets[S]), offsets[S] + host_count = T*k). */
int oracle_batches(const int32_t* ids, const double* w, int T, int k, int E, const int32_t* slot_of_expert, int S,
                   int32_t* slot_offsets, int32_t* active_slots, int32_t* num_active, int32_t* perm_pair,
                   int32_t* host_token, int32_t* host_expert, double* host_weight, int32_t* host_count) {
    if (T < 0 || k <= 0 || E <= 0 || S < 0) return -1;
    int64_t P = (int64_t)T * k;
    int32_t pos = 0;
    int32_t na = 0;
    for (int s = 0; s < S; ++s) {
        slot_offsets[s] = pos;
        int32_t first = pos;
        for (int64_t p = 0; p < P; ++p) {
            int id = ids[p];
            int slot = (id >= 0 && id < E) ? slot_of_expert[id] : -1;
            if (slot == s) perm_pair[pos++] = (int32_t)p;
        }
        if (pos > first) active_slots[na++] = s;
    }
    slot_offsets[S] = pos;
    *num_active = na;
    int32_t hc = 0;
    for (int64_t p = 0; p < P; ++p) {
        int id = ids[p];
        int slot = (id >= 0 && id < E) ? slot_of_expert[id] : -1;
        if (slot < 0 || slot >= S) {
            host_token[hc] = (int32_t)(p / k);
            host_expert[hc] = id;
            if (host_weight) host_weight[hc] = w ? w[p] : 0.0;
            ++hc;
        }
    }
    *host_count = hc;
    return 0;
}

/* ---------------------------------------------------------- expert FFN */

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* g = Wg x, u = Wu x (Wg, Wu: I rows of H), h = silu(g) * u, y = Wd h (Wd: H rows of I).
 * Parity pinned against dense matrix products on exactly representable weights. */
void oracle_expert_ffn(int fmt, const uint8_t* blob, int H, int I, const double* x, double* y) {
    const int fgu = gate_up_fmt(fmt), fdn = down_fmt(fmt);
    int64_t rb_h = row_bytes(fgu, H), rb_i = row_bytes(fdn, I);
    const uint8_t* wg = blob;
    const uint8_t* wu = blob + (int64_t)I * rb_h;
    const uint8_t* wd = blob + 2 * (int64_t)I * rb_h;
    double* h = (double*)malloc((size_t)I * sizeof(double));
#pragma omp parallel
    {
        double* row = (double*)malloc((size_t)(H > I ? H : I) * sizeof(double));
#pragma omp for schedule(static)
        for (int i = 0; i < I; ++i) {
            double g = 0.0, u = 0.0;
            dequant_row(fgu, wg + (int64_t)i * rb_h, H, row);
            for (int c = 0; c < H; ++c) g += row[c] * x[c];
            dequant_row(fgu, wu + (int64_t)i * rb_h, H, row);
            for (int c = 0; c < H; ++c) u += row[c] * x[c];
            h[i] = silu(g) * u;
        }
#pragma omp for schedule(static)
        for (int r = 0; r < H; ++r) {
            double acc = 0.0;
            dequant_row(fdn, wd + (int64_t)r * rb_i, I, row);
            for (int c = 0; c < I; ++c) acc += row[c] * h[c];
            y[r] = acc;
        }
        free(row);
    }
    free(h);
}

/* ------------------------------------------------------------- the layer */

int oracle_moe_layer(int fmt, const uint8_t* const* expert_blob, int E, int H, int I, int T, const double* x,
                     const float* logits, int k, int score, int renormalize, double scale,
                     const int32_t* slot_of_expert, int S, int shared_fmt, const uint8_t* shared_blob, int I_shared,
                     double* y, int32_t* ids, double* w, double* y_pairs) {
    if (S < 0 || S > E) return -1;
    if (oracle_route(logits, T, E, k, score, renormalize, scale, ids, w) != 0) return -1;
    double* yp = (double*)malloc((size_t)H * sizeof(double));
    for (int t = 0; t < T; ++t) {
        const double* xt = x + (int64_t)t * H;
        double* yt = y + (int64_t)t * H;
        for (int c = 0; c < H; ++c) yt[c] = 0.0;
        for (int j = 0; j < k; ++j) {
            int64_t p = (int64_t)t * k + j;
            int id = ids[p];
            int resident = slot_of_expert[id] >= 0 && slot_of_expert[id] < S;
            if (!resident) {
                if (y_pairs) memset(y_pairs + p * H, 0, (size_t)H * sizeof(double));
                continue;
            }
            if (!expert_blob[id]) {
                free(yp);
                return -2; /* a selected expert has no weights */
            }
            oracle_expert_ffn(fmt, expert_blob[id], H, I, xt, yp);
            if (y_pairs) memcpy(y_pairs + p * H, yp, (size_t)H * sizeof(double));
            for (int c = 0; c < H; ++c) yt[c] += w[p] * yp[c];
        }
        if (shared_blob) {
            oracle_expert_ffn(shared_fmt, shared_blob, H, I_shared, xt, yp);
            for (int c = 0; c < H; ++c) yt[c] += yp[c];
        }
    }
    free(yp);
    return 0;
}
