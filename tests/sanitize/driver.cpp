// Host-side code under AddressSanitizer and UndefinedBehaviorSanitizer: the
// packing, unpacking and argument checks of the C ABI (include/qmoe.h), the
// host leg and the residency policy (include/qmoe_host.h), the CPU oracle
// and the seeded input generator.  Every buffer is heap-allocated at its
// exact size, so an access one byte past it is reported.  No GPU work is
// enqueued: the device entry points are called only with arguments they
// refuse before launching anything.  Exit status 0 = every check held.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "../../include/qmoe.h"
#include "../../include/qmoe_host.h"
#include "../../oracle/oracle.h"

extern "C" {
int64_t fx_expert_bytes(int fmt, int64_t H, int64_t I);
void fx_gen_expert(int fmt, uint32_t seed, uint32_t layer, uint32_t expert, int64_t H, int64_t I, float std,
                   uint8_t* out);
void fx_normal_rows(uint32_t seed, uint32_t tag, uint32_t layer, int64_t rows, int64_t cols, float mean, float std,
                    float* out);
void fx_logits_normal(uint32_t seed, uint32_t layer, int64_t T, int E, float* out);
void fx_logits_zipf(uint32_t seed, uint32_t perm_seed, uint32_t layer, int64_t T, int E, double s, float* out);
}

static int g_failures = 0;
#define CHECK(cond)                                                             \
    do {                                                                        \
        if (!(cond)) {                                                          \
            std::fprintf(stderr, "CHECK failed at line %d: %s\n", __LINE__, #cond); \
            ++g_failures;                                                       \
        }                                                                       \
    } while (0)

static const void* const kFake = reinterpret_cast<const void*>(uintptr_t(1) << 20);  // never dereferenced

static void pack_round_trips() {
    const int shapes[][2] = {{512, 256}, {768, 512}};
    for (int fmt = MOE_FMT_Q8_0; fmt <= MOE_FMT_Q6K; ++fmt)
        for (const auto& hi : shapes) {
            const int H = hi[0], I = hi[1];
            const size_t nc = moe_expert_blob_bytes(fmt, H, I), np = moe_packed_blob_bytes(fmt, H, I);
            CHECK(nc > 0 && np >= nc);
            CHECK((int64_t)nc == fx_expert_bytes(fmt, H, I));
            std::vector<uint8_t> canon(nc), packed(np), back(nc);
            fx_gen_expert(fmt, 11, 0, (uint32_t)fmt, H, I, 0.02f, canon.data());
            CHECK(moe_pack_expert(fmt, canon.data(), packed.data(), H, I) == MOE_OK);
            CHECK(moe_unpack_expert(fmt, packed.data(), back.data(), H, I) == MOE_OK);
            CHECK(back == canon);
            if (fmt == MOE_FMT_Q4K || fmt == MOE_FMT_Q8_0) {
                // per-matrix packing builds the same blob
                const size_t gu = fmt == MOE_FMT_Q4K ? (size_t)2 * I * H / 256 * 144 : (size_t)2 * I * H / 32 * 34;
                std::vector<uint8_t> a(gu), b(nc - gu);
                auto pack = fmt == MOE_FMT_Q4K ? moe_pack_q4k : moe_pack_q8_0;
                CHECK(pack(canon.data(), a.data(), I, H, 1) == MOE_OK);
                CHECK(pack(canon.data() + gu, b.data(), H, I, 0) == MOE_OK);
                CHECK(std::memcmp(a.data(), packed.data(), gu) == 0);
                CHECK(std::memcmp(b.data(), packed.data() + gu, nc - gu) == 0);
                CHECK(pack(canon.data(), a.data(), I, H, 2) == MOE_ERR_INVALID_ARGUMENT);
                CHECK(pack(canon.data(), a.data(), I + 1, H, 1) == MOE_ERR_UNSUPPORTED);
            }
        }
    std::vector<uint8_t> small(64);
    CHECK(moe_pack_expert(MOE_FMT_Q4K, small.data(), small.data() + 1, 300, 256) == MOE_ERR_UNSUPPORTED);
    CHECK(moe_pack_expert(7, small.data(), small.data(), 256, 256) == MOE_ERR_INVALID_ARGUMENT);
    CHECK(moe_expert_blob_bytes(MOE_FMT_Q4K, 256, 100) == 0);
}

static void slot_maps() {
    std::vector<int32_t> m = {0, -1, 2, 1, -1};
    CHECK(moe_validate_slot_map(m.data(), 5, 3) == MOE_OK);
    m[4] = 2;  // slot 2 used twice
    CHECK(moe_validate_slot_map(m.data(), 5, 3) == MOE_ERR_INVALID_ARGUMENT);
    m[4] = 3;  // slot >= S
    CHECK(moe_validate_slot_map(m.data(), 5, 3) == MOE_ERR_INVALID_ARGUMENT);
    m[4] = -2;
    CHECK(moe_validate_slot_map(m.data(), 5, 3) == MOE_ERR_INVALID_ARGUMENT);
    CHECK(moe_validate_slot_map(m.data(), 5, 6) == MOE_ERR_INVALID_ARGUMENT);
    CHECK(moe_validate_slot_map(nullptr, 5, 3) == MOE_ERR_INVALID_ARGUMENT);
}

static void refusals() {
    const float* f = static_cast<const float*>(kFake);
    float* fo = const_cast<float*>(f);
    const int32_t* i = static_cast<const int32_t*>(kFake);
    int32_t* io = const_cast<int32_t*>(i);
    void* v = const_cast<void*>(kFake);
    CHECK(moe_route_topk(f, 4, 8, 9, 0, 1, 1.0f, io, fo, nullptr) == MOE_ERR_INVALID_ARGUMENT);
    CHECK(moe_route_topk(f, -1, 8, 2, 0, 1, 1.0f, io, fo, nullptr) == MOE_ERR_INVALID_ARGUMENT);
    CHECK(moe_route_topk(f, 4, 8, 2, 5, 1, 1.0f, io, fo, nullptr) == MOE_ERR_INVALID_ARGUMENT);
    CHECK(moe_route_topk(f, 4, 8, 2, 0, 1, NAN, io, fo, nullptr) == MOE_ERR_INVALID_ARGUMENT);
    CHECK(moe_build_expert_batches(i, f, 4, 2, 8, i, 9, io, io, io, io, io, io, fo, io, v, 1 << 20, nullptr) ==
          MOE_ERR_INVALID_ARGUMENT);
    CHECK(moe_build_expert_batches(i, f, 4, 2, 8, nullptr, 8, io, io, io, io, io, io, fo, io, v, 1 << 20, nullptr) ==
          MOE_ERR_INVALID_ARGUMENT);
    CHECK(moe_route_and_batch(f, 4, 8, 2, 0, 1, 1.0f, io, fo, i, 9, io, io, io, io, io, io, fo, io, nullptr, v,
                              1 << 20, nullptr) == MOE_ERR_INVALID_ARGUMENT);
    CHECK(moe_count_routes(i, 4, 2, 0, reinterpret_cast<uint32_t*>(v), nullptr) == MOE_ERR_INVALID_ARGUMENT);
    const size_t stride = moe_packed_blob_bytes(MOE_FMT_Q4K, 2048, 768);
    CHECK(moe_expert_ffn_q4k(kFake, stride, 128, 2000, 768, f, MOE_F32, 2, 8, i, i, i, i, v, MOE_F32,
                             MOE_PATH_DECODE, v, 1 << 30, nullptr) == MOE_ERR_UNSUPPORTED);
    CHECK(moe_expert_ffn_q4k(kFake, stride - 16, 128, 2048, 768, f, MOE_F32, 2, 8, i, i, i, i, v, MOE_F32,
                             MOE_PATH_DECODE, v, 1 << 30, nullptr) == MOE_ERR_INVALID_ARGUMENT);
    CHECK(moe_expert_ffn_q4k(kFake, stride, 128, 2048, 768, f, MOE_F32, 2, 8, i, i, i, i, v, MOE_F32,
                             MOE_PATH_DECODE, v, 16, nullptr) == MOE_ERR_WORKSPACE_TOO_SMALL);
    const size_t stride8 = moe_packed_blob_bytes(MOE_FMT_Q8_0, 2048, 768);
    CHECK(moe_expert_ffn_q8_0(kFake, stride8, 128, 2048, 768, f, MOE_BF16, 64, 8, i, i, i, i, v, MOE_BF16,
                              MOE_PATH_PREFILL, v, 1 << 30, nullptr) == MOE_ERR_UNSUPPORTED);
    CHECK(moe_expert_ffn_q4k_noalloc(kFake, stride, 128, 2048, 768, f, MOE_BF16, 8192, 8, i, i, i, i, v, MOE_BF16,
                                     MOE_PATH_PREFILL, nullptr) == MOE_ERR_UNSUPPORTED);
    // the int8-activation path: Q4_K only, bf16 activations, its larger workspace
    const size_t stride_mx = moe_packed_blob_bytes(MOE_FMT_MXFP4, 2048, 768);
    CHECK(moe_expert_ffn_mxfp4(kFake, stride_mx, 128, 2048, 768, f, MOE_BF16, 64, 8, i, i, i, i, v, MOE_BF16,
                               MOE_PATH_PREFILL_I8, v, 1 << 30, nullptr) == MOE_ERR_UNSUPPORTED);
    CHECK(moe_expert_ffn_q4k(kFake, stride, 128, 2048, 768, f, MOE_F32, 64, 8, i, i, i, i, v, MOE_BF16,
                             MOE_PATH_PREFILL_I8, v, 1 << 30, nullptr) == MOE_ERR_UNSUPPORTED);
    const size_t need_i8 = moe_ffn_workspace_size(MOE_FMT_Q4K, 64, 8, 2048, 768, MOE_PATH_PREFILL_I8);
    CHECK(need_i8 > moe_ffn_workspace_size(MOE_FMT_Q4K, 64, 8, 2048, 768, MOE_PATH_PREFILL));
    CHECK(moe_expert_ffn_q4k(kFake, stride, 128, 2048, 768, f, MOE_BF16, 64, 8, i, i, i, i, v, MOE_BF16,
                             MOE_PATH_PREFILL_I8, v, need_i8 - 1, nullptr) == MOE_ERR_WORKSPACE_TOO_SMALL);
    CHECK(moe_expert_ffn_q4k_noalloc(kFake, stride, 128, 2048, 768, f, MOE_BF16, 4096, 8, i, i, i, i, v, MOE_BF16,
                                     MOE_PATH_PREFILL_I8, nullptr) == MOE_ERR_UNSUPPORTED);
    // the measurement probes' argument checks
    CHECK(moe_prefill_inner_probe(3, 8, fo, MOE_PREFILL_PROBE_OUT_FLOATS, nullptr) == MOE_ERR_INVALID_ARGUMENT);
    CHECK(moe_prefill_inner_probe(0, 0, fo, MOE_PREFILL_PROBE_OUT_FLOATS, nullptr) == MOE_ERR_INVALID_ARGUMENT);
    CHECK(moe_prefill_inner_probe(2, 8, fo, MOE_PREFILL_PROBE_OUT_FLOATS - 1, nullptr) == MOE_ERR_INVALID_ARGUMENT);
    size_t nread = 0;
    uint32_t* sink = reinterpret_cast<uint32_t*>(v);
    CHECK(moe_hbm_read_probe(kFake, 1 << 20, 12, 8, sink, &nread, nullptr) == MOE_ERR_INVALID_ARGUMENT);
    CHECK(moe_hbm_read_probe(kFake, 1 << 20, 64, 3, sink, &nread, nullptr) == MOE_ERR_INVALID_ARGUMENT);
    CHECK(moe_hbm_read_probe(kFake, 1024, 64, 8, sink, &nread, nullptr) == MOE_ERR_INVALID_ARGUMENT);
    CHECK(moe_combine(v, MOE_F32, i, f, i, 8, 9, nullptr, 4, 2, 256, v, MOE_F32, nullptr) ==
          MOE_ERR_INVALID_ARGUMENT);
    CHECK(moe_combine(v, MOE_F32, i, f, i, 8, 8, nullptr, 4, 2, 252, v, MOE_F32, nullptr) == MOE_ERR_UNSUPPORTED);
    CHECK(moe_layer_decode(MOE_FMT_Q4K, f, f, MOE_F32, 2, 128, 8, 0, 1, 1.0f, i, 128, kFake, stride, 2048, 768,
                           kFake, 0, io, fo, io, io, io, io, io, io, fo, io, nullptr, fo, fo, v, 1 << 30,
                           nullptr) == MOE_ERR_INVALID_ARGUMENT);
    CHECK(moe_layer_decode(MOE_FMT_Q4K, f, f, MOE_F32, 2, 128, 8, 0, 1, 1.0f, i, 129, kFake, stride, 2048, 768,
                           nullptr, 0, io, fo, io, io, io, io, io, io, fo, io, nullptr, fo, fo, v, 1 << 30,
                           nullptr) == MOE_ERR_INVALID_ARGUMENT);
    CHECK(moe_timer_begin(99, 4) == MOE_ERR_INVALID_ARGUMENT);
    double ms = 0;
    int n = 0;
    CHECK(moe_timer_end(3, &ms, &n) == MOE_ERR_INVALID_ARGUMENT);
    CHECK(std::strlen(moe_last_error()) > 0);
    CHECK(std::strcmp(moe_status_name(99), "MOE_STATUS_UNKNOWN") == 0);
    // workspace queries at their edges
    CHECK(moe_ffn_workspace_size(MOE_FMT_Q4K, 0, 8, 2048, 768, MOE_PATH_DECODE) > 0);
    CHECK(moe_ffn_workspace_size(MOE_FMT_Q4K, 2, 65, 2048, 768, MOE_PATH_DECODE) == 0);
    CHECK(moe_batches_workspace_size(4096, 8, 128, 129) == 0);
    CHECK(moe_layer_decode_workspace_size(MOE_FMT_Q4K, 2, 8, 256, 104, 7168, 2048, 2048) > 0);
    CHECK(moe_layer_decode_workspace_size(MOE_FMT_Q4K, 2, 8, 256, 104, 7168, 2048, 200) == 0);
}

// The host leg on a small layer against the oracle's FFN of the same pairs.
static void host_leg() {
    const int E = 4, H = 256, I = 256, T = 3, fmts[] = {MOE_FMT_Q4K, MOE_FMT_Q8_0, MOE_FMT_Q6K, MOE_FMT_Q3K_Q4K};
    for (int fmt : fmts) {
        const size_t nb = moe_expert_blob_bytes(fmt, H, I);
        std::vector<std::vector<uint8_t>> blobs(E, std::vector<uint8_t>(nb));
        std::vector<const uint8_t*> ptr(E);
        for (int e = 0; e < E; ++e) {
            fx_gen_expert(fmt, 3, 0, (uint32_t)e, H, I, 0.02f, blobs[e].data());
            ptr[e] = blobs[e].data();
        }
        ptr[2] = nullptr;  // an expert no pair uses need not be given
        std::vector<float> x((size_t)T * H);
        fx_normal_rows(5, 1, 0, T, H, 0.0f, 1.0f, x.data());
        const std::vector<int32_t> tok = {0, 2, 1, 2, 0}, exp = {1, 3, 0, 1, 0};
        const std::vector<float> w = {0.5f, 0.25f, 1.0f, 0.75f, 0.125f};
        std::vector<float> y((size_t)T * H);
        CHECK(moe_host_leg(fmt, ptr.data(), E, H, I, x.data(), T, tok.data(), exp.data(), w.data(), (int)tok.size(),
                           y.data(), 2) == MOE_OK);
        const int oracle_fmt = fmt;
        std::vector<double> want((size_t)T * H, 0.0), xd(H), yd(H);
        for (size_t p = 0; p < tok.size(); ++p) {
            for (int c = 0; c < H; ++c) xd[c] = x[(size_t)tok[p] * H + c];
            oracle_expert_ffn(oracle_fmt, blobs[exp[p]].data(), H, I, xd.data(), yd.data());
            for (int c = 0; c < H; ++c) want[(size_t)tok[p] * H + c] += w[p] * yd[c];
        }
        double err = 0, mx = 0;
        for (size_t q = 0; q < want.size(); ++q) {
            err = std::fmax(err, std::fabs(y[q] - want[q]));
            mx = std::fmax(mx, std::fabs(want[q]));
        }
        CHECK(err <= 1e-4 * mx);
        // refusals: a pair with an expert given as NULL, a token out of range
        const std::vector<int32_t> bad_exp = {2};
        const std::vector<int32_t> bad_tok = {T};
        const std::vector<int32_t> one_tok = {0}, one_exp = {1};
        CHECK(moe_host_leg(fmt, ptr.data(), E, H, I, x.data(), T, one_tok.data(), bad_exp.data(), w.data(), 1,
                           y.data(), 1) != MOE_OK);
        CHECK(moe_host_leg(fmt, ptr.data(), E, H, I, x.data(), T, bad_tok.data(), one_exp.data(), w.data(), 1,
                           y.data(), 1) != MOE_OK);
    }
}

static void residency() {
    const int E = 64;
    std::vector<uint64_t> score(E, 0);
    std::vector<uint32_t> win(E);
    std::vector<int32_t> soe(E, -1), in(8), out(8);
    for (int e = 0; e < 32; ++e) soe[e] = e;
    for (int step = 0; step < 5; ++step) {
        for (int e = 0; e < E; ++e) win[e] = (uint32_t)((e * 7 + step * 3) % 11);
        CHECK(moe_residency_update_scores(score.data(), win.data(), E, 4) == MOE_OK);
    }
    int n = -1;
    CHECK(moe_residency_plan(score.data(), E, soe.data(), 8, 1u << 16, in.data(), out.data(), &n) == MOE_OK);
    CHECK(n >= 0 && n <= 8);
    for (int j = 0; j < n; ++j) CHECK(soe[in[j]] < 0 && soe[out[j]] >= 0);
    CHECK(moe_residency_plan(score.data(), E, soe.data(), 0, 0, nullptr, nullptr, &n) == MOE_OK && n == 0);
    CHECK(moe_residency_update_scores(score.data(), win.data(), E, 64) == MOE_ERR_INVALID_ARGUMENT);
}

// The oracle's routing, batching and whole layer on a small partial-residency case.
static void oracle_layer() {
    const int E = 8, H = 256, I = 256, T = 5, k = 3, S = 5;
    std::vector<float> lg((size_t)T * E);
    fx_logits_zipf(2, 2, 0, T, E, 1.0, lg.data());
    std::vector<int32_t> ids((size_t)T * k);
    std::vector<double> w((size_t)T * k);
    CHECK(oracle_route(lg.data(), T, E, k, ORACLE_SIGMOID, 1, 2.5, ids.data(), w.data()) == 0);
    const std::vector<int32_t> soe = {0, -1, 1, 2, -1, 3, 9, 4};  // expert 6 holds a slot >= S: on the host
    std::vector<int32_t> off(S + 1), act(std::min(S, T * k)), na(1), perm(T * k), ht(T * k), he(T * k), hc(1);
    std::vector<double> hw(T * k);
    CHECK(oracle_batches(ids.data(), w.data(), T, k, E, soe.data(), S, off.data(), act.data(), na.data(),
                         perm.data(), ht.data(), he.data(), hw.data(), hc.data()) == 0);
    CHECK(off[S] + hc[0] == T * k);
    const size_t nb = moe_expert_blob_bytes(MOE_FMT_Q4K, H, I);
    std::vector<std::vector<uint8_t>> blobs(E, std::vector<uint8_t>(nb));
    std::vector<const uint8_t*> ptr(E);
    for (int e = 0; e < E; ++e) {
        fx_gen_expert(MOE_FMT_Q4K, 4, 0, (uint32_t)e, H, I, 0.02f, blobs[e].data());
        ptr[e] = blobs[e].data();
    }
    const size_t ns = moe_expert_blob_bytes(MOE_FMT_Q8_0, H, 128);
    std::vector<uint8_t> shared(ns);
    fx_gen_expert(MOE_FMT_Q8_0, 4, 1, 0, H, 128, 0.02f, shared.data());
    std::vector<float> xf((size_t)T * H);
    fx_normal_rows(6, 1, 0, T, H, 0.0f, 1.0f, xf.data());
    std::vector<double> x(xf.begin(), xf.end()), y((size_t)T * H), yp((size_t)T * k * H), w2((size_t)T * k);
    std::vector<int32_t> ids2((size_t)T * k);
    CHECK(oracle_moe_layer(ORACLE_Q4K, ptr.data(), E, H, I, T, x.data(), lg.data(), k, ORACLE_SIGMOID, 1, 2.5,
                           soe.data(), S, ORACLE_Q8_0, shared.data(), 128, y.data(), ids2.data(), w2.data(),
                           yp.data()) == 0);
    CHECK(ids2 == ids);
}

int main() {
    pack_round_trips();
    slot_maps();
    refusals();
    host_leg();
    residency();
    oracle_layer();
    if (g_failures) std::fprintf(stderr, "%d checks failed\n", g_failures);
    else std::printf("sanitized host checks: all passed\n");
    return g_failures ? 1 : 0;
}
