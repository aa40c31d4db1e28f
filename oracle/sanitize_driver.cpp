// TEST INFRASTRUCTURE ONLY: drives every entry point of the CPU oracle on
// small seeded inputs (every weight width, groups, forced routing, taps,
// accumulate, ragged FP8 blocks, rejected arguments) so that a build with
// AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_oracle_sanitize.py)
// sees every access the oracle makes. Exits 0 when every call returned what
// it should.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

extern "C" {
int coli_ref_pack(const float*, int64_t, int64_t, int, uint8_t*, float*);
int coli_ref_pack_int4(const float*, int64_t, int64_t, uint8_t*, float*);
float coli_ref_e4m3_to_f32(uint8_t);
int coli_ref_fp8_to_f32(const uint8_t*, const float*, int64_t, int64_t, float*);
int coli_ref_pack_fp8_int4(const uint8_t*, const float*, int64_t, int64_t, uint8_t*, float*);
int coli_ref_unpack(const uint8_t*, int64_t, int64_t, int, int8_t*);
int coli_ref_unpack_int4(const uint8_t*, int64_t, int64_t, int8_t*);
int coli_ref_quant_q8(const float*, int64_t, int64_t, int8_t*, float*);
int coli_ref_block_dots_bits(const uint8_t*, int64_t, int64_t, int, const int8_t*, int64_t, int32_t*);
int coli_ref_block_dots(const uint8_t*, int64_t, int64_t, const int8_t*, int64_t, int32_t*);
int coli_ref_route(const float*, const float*, const float*, int64_t, int64_t, int64_t, int64_t,
                   int, double, int64_t, int64_t, int32_t*, float*, double*);
int coli_ref_gates(const float*, const float*, const float*, int64_t, int64_t, int64_t, int64_t,
                   int, double, const int32_t*, float*);
int coli_ref_rmsnorm(const float*, int64_t, int64_t, double, float*);
typedef struct {
    int64_t hidden, inter, n_experts, top_k, n_shared, norm_topk;
    double rho;
    const float* w_router;
    const float* bias;
    const uint8_t* const* gate_q;
    const uint8_t* const* up_q;
    const uint8_t* const* down_q;
    const float* const* gate_s;
    const float* const* up_s;
    const float* const* down_s;
    int64_t n_group, topk_group, weight_bits;
} Layer;
typedef struct {
    int32_t* idx; float* w; double* logits; int8_t* qx; float* dx; float* g; float* u;
    float* h; int8_t* qh; float* dh; float* ye;
} Taps;
int coli_ref_moe_forward(const Layer*, const float*, int64_t, const int32_t*, const float*,
                         float*, int, Taps*);
void coli_ref_set_threads(int);
}

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static float rnd(float sigma) {  // uniform in [-sigma, sigma): enough for memory checks
    g_state = g_state * 6364136223846793005ull + 1442695040888963407ull;
    return sigma * ((float)((g_state >> 40) & 0xFFFFFF) / 8388608.0f - 1.0f);
}
static std::vector<float> rvec(size_t n, float sigma) {
    std::vector<float> v(n);
    for (auto& x : v) x = rnd(sigma);
    return v;
}

static int failures = 0;
#define EXPECT(c)                                                        \
    do {                                                                 \
        if (!(c)) {                                                      \
            std::fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
            ++failures;                                                  \
        }                                                                \
    } while (0)

static void layer_case(int bits, int64_t H, int64_t I, int64_t E, int64_t K, int64_t S,
                       int64_t ng, int64_t tg, int64_t T) {
    const int64_t n = E + S;
    std::vector<std::vector<uint8_t>> gq(n), uq(n), dq(n);
    std::vector<std::vector<float>> gs(n), us(n), ds(n);
    std::vector<const uint8_t*> pg(n), pu(n), pd(n);
    std::vector<const float*> psg(n), psu(n), psd(n);
    for (int64_t e = 0; e < n; ++e) {
        auto wg = rvec(I * H, 0.02f), wu = rvec(I * H, 0.02f), wd = rvec(H * I, 0.02f);
        gq[e].resize(I * H * bits / 8); uq[e].resize(I * H * bits / 8); dq[e].resize(H * I * bits / 8);
        gs[e].resize(I); us[e].resize(I); ds[e].resize(H);
        EXPECT(coli_ref_pack(wg.data(), I, H, bits, gq[e].data(), gs[e].data()) == 0);
        EXPECT(coli_ref_pack(wu.data(), I, H, bits, uq[e].data(), us[e].data()) == 0);
        EXPECT(coli_ref_pack(wd.data(), H, I, bits, dq[e].data(), ds[e].data()) == 0);
        pg[e] = gq[e].data(); pu[e] = uq[e].data(); pd[e] = dq[e].data();
        psg[e] = gs[e].data(); psu[e] = us[e].data(); psd[e] = ds[e].data();
    }
    auto wr = rvec(E * H, 0.02f), b = rvec(E, 0.01f), x = rvec(T * H, 1.0f);
    Layer L{H, I, E, K, S, 1, 2.5, wr.data(), b.data(), pg.data(), pu.data(), pd.data(),
            psg.data(), psu.data(), psd.data(), ng, tg, bits};
    const int64_t KS = K + S;
    std::vector<int32_t> idx(T * K);
    std::vector<float> w(T * K), g(T * KS * I), u(T * KS * I), h(T * KS * I), dx(T * H / 32),
        dh(T * KS * I / 32), ye(T * KS * H), y(T * H, 0.5f);
    std::vector<double> lg(T * E);
    std::vector<int8_t> qx(T * H), qh(T * KS * I);
    Taps tp{idx.data(), w.data(), lg.data(), qx.data(), dx.data(), g.data(), u.data(),
            h.data(), qh.data(), dh.data(), ye.data()};
    EXPECT(coli_ref_moe_forward(&L, x.data(), T, nullptr, nullptr, y.data(), 1, &tp) == 0);
    std::vector<float> w2(T * K);
    EXPECT(coli_ref_gates(x.data(), wr.data(), b.data(), T, H, E, K, 1, 2.5, idx.data(),
                          w2.data()) == 0);
    EXPECT(std::memcmp(w2.data(), w.data(), w.size() * 4) == 0 || ng > 1);
    EXPECT(coli_ref_moe_forward(&L, x.data(), T, idx.data(), w.data(), y.data(), 0, nullptr) == 0);
    std::vector<int32_t> bad(idx);
    bad[0] = (int32_t)E;  // out of range: rejected
    EXPECT(coli_ref_moe_forward(&L, x.data(), T, bad.data(), w.data(), y.data(), 0, nullptr) != 0);
    std::vector<int32_t> ri(T * K);
    std::vector<float> rw(T * K);
    EXPECT(coli_ref_route(x.data(), wr.data(), b.data(), T, H, E, K, 1, 2.5, ng, tg, ri.data(),
                          rw.data(), lg.data()) == 0);
    std::vector<int32_t> dots(T * I * (H / 32));
    EXPECT(coli_ref_block_dots_bits(gq[0].data(), I, H, bits, qx.data(), T, dots.data()) == 0);
    std::vector<int8_t> codes(I * H);
    EXPECT(coli_ref_unpack(gq[0].data(), I, H, bits, codes.data()) == 0);
}

int main() {
    coli_ref_set_threads(2);
    // packs of every width, ragged rows, a zero row; quant; rmsnorm
    for (int bits : {2, 4, 8}) {
        auto wv = rvec(7 * 96, 1.0f);
        std::fill(wv.begin() + 96, wv.begin() + 192, 0.0f);
        std::vector<uint8_t> q(7 * 96 * bits / 8);
        std::vector<float> s(7);
        EXPECT(coli_ref_pack(wv.data(), 7, 96, bits, q.data(), s.data()) == 0);
        if (bits != 8)  // rows must fill whole bytes
            EXPECT(coli_ref_pack(wv.data(), 7, 97, bits, q.data(), s.data()) != 0);
        EXPECT(coli_ref_pack(wv.data(), -1, 96, bits, q.data(), s.data()) != 0);
        EXPECT(coli_ref_pack(wv.data(), 7, 96, 3, q.data(), s.data()) != 0);     // width
    }
    {
        auto wv = rvec(5 * 64, 1.0f);
        std::vector<uint8_t> q(5 * 32);
        std::vector<float> s(5);
        std::vector<int8_t> c(5 * 64);
        EXPECT(coli_ref_pack_int4(wv.data(), 5, 64, q.data(), s.data()) == 0);
        EXPECT(coli_ref_unpack_int4(q.data(), 5, 64, c.data()) == 0);
        std::vector<int8_t> qx(3 * 64);
        std::vector<float> dx(3 * 2);
        auto xv = rvec(3 * 64, 2.0f);
        EXPECT(coli_ref_quant_q8(xv.data(), 3, 64, qx.data(), dx.data()) == 0);
        std::vector<int32_t> dots(3 * 5 * 2);
        EXPECT(coli_ref_block_dots(q.data(), 5, 64, qx.data(), 3, dots.data()) == 0);
        std::vector<float> out(3 * 64);
        EXPECT(coli_ref_rmsnorm(xv.data(), 3, 64, 1e-5, out.data()) == 0);
    }
    // FP8 front-end on ragged 128 x 128 block grids, every code
    for (int c = 0; c < 256; ++c) {
        const float v = coli_ref_e4m3_to_f32((uint8_t)c);
        EXPECT(std::isfinite(v));
    }
    for (auto rc : {std::pair<int64_t, int64_t>{200, 352}, {3, 32}, {129, 160}}) {
        const int64_t rows = rc.first, cols = rc.second;
        std::vector<uint8_t> q8(rows * cols);
        for (auto& v : q8) v = (uint8_t)(rnd(1.0f) * 127.0f + 128.0f);
        const int64_t br = (rows + 127) / 128, bc = (cols + 127) / 128;
        auto bs = rvec(br * bc, 1.0f);
        for (auto& v : bs) v = std::fabs(v) + 0.01f;
        std::vector<float> wv(rows * cols);
        EXPECT(coli_ref_fp8_to_f32(q8.data(), bs.data(), rows, cols, wv.data()) == 0);
        std::vector<uint8_t> q(rows * cols / 2);
        std::vector<float> s(rows);
        EXPECT(coli_ref_pack_fp8_int4(q8.data(), bs.data(), rows, cols, q.data(), s.data()) == 0);
    }
    // layers: every width, shared / no shared expert, groups, several tokens
    layer_case(4, 64, 64, 8, 2, 1, 1, 1, 5);
    layer_case(8, 64, 64, 8, 3, 0, 1, 1, 3);
    layer_case(2, 96, 32, 6, 2, 1, 1, 1, 4);
    layer_case(4, 64, 32, 16, 4, 1, 4, 2, 6);
    std::printf("oracle sanitizer driver: %d failed checks\n", failures);
    return failures == 0 ? 0 : 1;
}
