// TEST INFRASTRUCTURE ONLY — plain, slow CPU oracle of one sigmoid-routed
// Mixture-of-Experts layer with symmetric int4 expert weights (one F32 scale
// per row) and Q8_0-style int8 activations. Only the tests, the smoke check
// and the bench's CPU-baseline leg load this library; the product path never
// does. It shares no code with the HIP library.
//
// Sources (the text of five web pages on the colibri engine for GLM-5.2):
//  [A] wmrh.cn, "GLM-5.2-colibri-int4架构解析MoE专家混合与INT4量化原理":
//      section "GLM-5.2的MoE实现" (256 routed experts, 1 shared, 8 per token,
//      hidden 6144, expert intermediate 2048); section "MoE的工作原理"
//      (per-token router scores, top-8, score-weighted sum of expert outputs);
//      section "量化流程" (FP8 -> F32 -> int4 by np.rint to agree with the
//      engine's lrintf, one F32 scale per weight row, two 4-bit values per U8);
//      section "路由策略定制" (knobs topk_method, routed_scaling_factor,
//      norm_topk_prob); section "量化保留模块" (some modules stay F32).
//  [C] "Colibri：在笔记本上跑744B参数的AI模型", feature list (关键特性):
//      DeepSeek-V3-style sigmoid router plus shared expert; integer dot
//      kernel over Q8_0-style int8 activations; quantisation kernels for
//      int8, int4 and int2 weights.
//  [E] hn mirror of the project summary, feature list: batched MoE — an
//      expert used by several positions of a batch is read once.
// Where the pages are silent the reading taken is stated at the function.
//
// Numerics: everything that can decide an integer (a quantised code, a
// top-k choice) is computed exactly as written below, in IEEE float/double
// with round-to-nearest-even, no FMA contraction (-ffp-contract=off), no
// fast-math. Block dot products are exact int32; the sums of scaled block
// dots are formed in double.
//
// Parity pins: see tests/test_oracle_*.py. Every function here is pinned by
// a closed form, a hand-worked case, an invariant, a textbook special case
// or brute force (no function is "parity unpinned").

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>
#ifdef _OPENMP
#include <omp.h>
#endif

extern "C" {

enum { REF_OK = 0, REF_EINVAL = -1 };

// ---------------------------------------------------------------------------
// Symmetric b-bit weight quantisation, b = 4 ([A] section 量化流程), and the
// sibling int8 and int2 formats the engine's kernels also handle ([C] feature
// list, 关键特性: quantisation kernels for int8, int4 and int2):
//   Q    = 2^(b-1) - 1                          (7 for int4, 127 int8, 1 int2)
//   s_r  = fp32( max_j |W_rj| / Q )             (IEEE single division)
//   q_rj = clamp( rint(W_rj / s_r), -Q, Q )     (round half to even, the
//          behaviour of both np.rint and lrintf in the default rounding mode)
//   s_r == 0  ->  q_rj = 0
//   codes are b-bit two's complement, packed little end first: element j of
//   a row sits in byte (j b) / 8 at bit (j b) % 8 (int4: the even element in
//   the low nibble; int2: element 4i + k at bits 2k of byte i).
// Readings: divide (not multiply by 1/s); symmetric range +-Q (int4's
// max|row|/7 carried over to the other widths, so int2 is ternary); a "row"
// is an output channel.
// ---------------------------------------------------------------------------
static bool ref_bits_ok(int bits) { return bits == 2 || bits == 4 || bits == 8; }

static int ref_code(float w, float s, int qmax) {
    float r = rintf(w / s);
    if (r > (float)qmax) r = (float)qmax;
    if (r < -(float)qmax) r = -(float)qmax;
    return (int)r;
}

int coli_ref_pack(const float* w, int64_t rows, int64_t cols, int bits, uint8_t* q,
                  float* scale) {
    if (!w || !q || !scale || rows < 0 || cols <= 0 || !ref_bits_ok(bits) ||
        (cols * bits) % 8 != 0)
        return REF_EINVAL;
    const int qmax = (1 << (bits - 1)) - 1;
    const int64_t row_bytes = cols * bits / 8;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const float* row = w + r * cols;
        float amax = 0.0f;
        for (int64_t j = 0; j < cols; ++j) {
            float a = std::fabs(row[j]);
            if (a > amax) amax = a;
        }
        float s = amax / (float)qmax;
        scale[r] = s;
        uint8_t* out = q + r * row_bytes;
        std::memset(out, 0, (size_t)row_bytes);
        for (int64_t j = 0; j < cols; ++j) {
            const int c = (s != 0.0f) ? ref_code(row[j], s, qmax) : 0;
            const int64_t bit = j * bits;
            out[bit / 8] |= (uint8_t)((c & ((1 << bits) - 1)) << (bit % 8));
        }
    }
    return REF_OK;
}

int coli_ref_pack_int4(const float* w, int64_t rows, int64_t cols, uint8_t* q, float* scale) {
    return coli_ref_pack(w, rows, cols, 4, q, scale);
}

// ---------------------------------------------------------------------------
// FP8 -> int4 converter front-end ([W] section 量化流程: source weights in
// FP8 e4m3 with 128 x 128 block scales, converted to F32, then packed to int4
// as above; the block size is the quantization_config shown in that section).
//   e4m3: 1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent 0 is
//   subnormal (m * 2^-9); S.1111.111 is NaN; there are no infinities.
//   w[r][c] = fp32( e4m3(q[r][c]) * bs[r / 128][c / 128] ), one rounding.
// Readings: the block scale multiplies (it is stored as the inverse of the
// quantiser's scale, as in the FP8 checkpoints of this model family); the NaN
// code converts to 0 (a checkpoint holds none, and a NaN must not poison the
// scale of its whole row).
// ---------------------------------------------------------------------------
float coli_ref_e4m3_to_f32(uint8_t b) {
    const int sign = b >> 7, e = (b >> 3) & 0xF, m = b & 7;
    if (e == 15 && m == 7) return 0.0f;  // NaN code
    double v = (e == 0) ? std::ldexp((double)m, -9) : std::ldexp(1.0 + m / 8.0, e - 7);
    return (float)(sign ? -v : v);
}

int coli_ref_fp8_to_f32(const uint8_t* q, const float* bs, int64_t rows, int64_t cols, float* w) {
    if (!q || !bs || !w || rows < 0 || cols <= 0) return REF_EINVAL;
    const int64_t nbc = (cols + 127) / 128;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            const float scale = bs[(r / 128) * nbc + c / 128];
            w[r * cols + c] = coli_ref_e4m3_to_f32(q[r * cols + c]) * scale;
        }
    return REF_OK;
}

int coli_ref_pack_fp8_int4(const uint8_t* q8, const float* bs, int64_t rows, int64_t cols,
                           uint8_t* q, float* scale) {
    if (!q8 || !bs || !q || !scale || rows < 0 || cols <= 0 || (cols % 2) != 0) return REF_EINVAL;
    std::vector<float> w((size_t)(rows * cols));
    int rc = coli_ref_fp8_to_f32(q8, bs, rows, cols, w.data());
    if (rc) return rc;
    return coli_ref_pack_int4(w.data(), rows, cols, q, scale);
}

// Signed value of element j of a packed b-bit row (b-bit two's complement:
// the most negative code, e.g. 0x8 for int4, decodes to -2^(b-1)).
static int ref_code_at(const uint8_t* row, int64_t j, int bits) {
    const int64_t bit = j * bits;
    const int v = (row[bit / 8] >> (bit % 8)) & ((1 << bits) - 1);
    return v >= (1 << (bits - 1)) ? v - (1 << bits) : v;
}

int coli_ref_unpack(const uint8_t* q, int64_t rows, int64_t cols, int bits, int8_t* codes) {
    if (!q || !codes || rows < 0 || cols <= 0 || !ref_bits_ok(bits) || (cols * bits) % 8 != 0)
        return REF_EINVAL;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t j = 0; j < cols; ++j)
            codes[r * cols + j] = (int8_t)ref_code_at(q + r * (cols * bits / 8), j, bits);
    return REF_OK;
}

int coli_ref_unpack_int4(const uint8_t* q, int64_t rows, int64_t cols, int8_t* codes) {
    return coli_ref_unpack(q, rows, cols, 4, codes);
}

// ---------------------------------------------------------------------------
// Q8_0 activation quantisation ([C] feature list: Q8_0-style int8 activations)
//   per block of 32 consecutive elements:
//   d = fp32( max|x| / 127 ),  q = clamp( rint(x / d), -127, 127 ),  d == 0 -> q = 0
// Readings: the block scale is kept as fp32 (the pages do not give its
// precision); x/d with round-half-even mirrors the weight recipe above.
// ---------------------------------------------------------------------------
static void ref_q8_block(const float* x, int8_t* q, float* d) {
    float amax = 0.0f;
    for (int i = 0; i < 32; ++i) {
        float a = std::fabs(x[i]);
        if (a > amax) amax = a;
    }
    float dd = amax / 127.0f;
    *d = dd;
    for (int i = 0; i < 32; ++i) {
        int v = 0;
        if (dd != 0.0f) {
            float r = rintf(x[i] / dd);
            if (r > 127.0f) r = 127.0f;
            if (r < -127.0f) r = -127.0f;
            v = (int)r;
        }
        q[i] = (int8_t)v;
    }
}

int coli_ref_quant_q8(const float* x, int64_t n_tok, int64_t dim, int8_t* q, float* d) {
    if (!x || !q || !d || n_tok < 0 || dim <= 0 || (dim % 32) != 0) return REF_EINVAL;
    const int64_t nb = dim / 32;
    for (int64_t t = 0; t < n_tok; ++t)
        for (int64_t b = 0; b < nb; ++b)
            ref_q8_block(x + t * dim + b * 32, q + t * dim + b * 32, d + t * nb + b);
    return REF_OK;
}

// ---------------------------------------------------------------------------
// Exact int32 dot of one 32-wide block: sum_i code(w_i) * q_i.
// ---------------------------------------------------------------------------
static int32_t ref_block_dot(const uint8_t* wrow, int64_t b, const int8_t* q, int bits) {
    int32_t acc = 0;
    for (int i = 0; i < 32; ++i) {
        int64_t j = b * 32 + i;
        acc += ref_code_at(wrow, j, bits) * (int32_t)q[j];
    }
    return acc;
}

// dots[t, r, b] for every token t, weight row r and block b (debug reference).
int coli_ref_block_dots_bits(const uint8_t* wq, int64_t rows, int64_t cols, int bits,
                             const int8_t* qx, int64_t n_tok, int32_t* dots) {
    if (!wq || !qx || !dots || rows < 0 || cols <= 0 || (cols % 32) != 0 || n_tok < 0 ||
        !ref_bits_ok(bits))
        return REF_EINVAL;
    const int64_t nb = cols / 32;
    for (int64_t t = 0; t < n_tok; ++t)
        for (int64_t r = 0; r < rows; ++r)
            for (int64_t b = 0; b < nb; ++b)
                dots[(t * rows + r) * nb + b] =
                    ref_block_dot(wq + r * (cols * bits / 8), b, qx + t * cols, bits);
    return REF_OK;
}

int coli_ref_block_dots(const uint8_t* wq, int64_t rows, int64_t cols, const int8_t* qx,
                        int64_t n_tok, int32_t* dots) {
    return coli_ref_block_dots_bits(wq, rows, cols, 4, qx, n_tok, dots);
}

// Row r of a packed weight matrix times a Q8_0 vector, in double:
//   D_r = sum_b d_b * I_b            (each product exact in double)
// followed by the row scale, rounded once to fp32:  fp32( s_r * D_r ).
static float ref_row_dot(const uint8_t* wrow, float s_r, const int8_t* q, const float* d,
                         int64_t nb, int bits) {
    double acc = 0.0;
    for (int64_t b = 0; b < nb; ++b) acc += (double)d[b] * (double)ref_block_dot(wrow, b, q, bits);
    return (float)((double)s_r * acc);
}

// ---------------------------------------------------------------------------
// Router ([A] MoE的工作原理, 路由策略定制; [C] sigmoid router)
//   l[t,e] = sum_h x[t,h] * Wr[e,h]          (double, ascending h)
//   s = 1 / (1 + exp(-l))                      (double)
//   c = s + bias[e]                            (selection score)
//   pick the K largest c, ties to the lower expert index, in descending order
//   w_k = s[e_k]; if normalising: w_k = w_k / sum_k w_k; w_k = w_k * rho; fp32
// Readings: the correction bias only steers selection (the gate value is
// the unbiased sigmoid, DeepSeek-V3 style).
// Group-limited selection (the topk_method knob of [A] 路由策略定制, read as
// DeepSeek-V3's: the pages name the knob, not its algorithm), when
// n_group > 1: the E experts form n_group consecutive groups of E / n_group;
// a group's score is the sum of its two largest c (its only c when a group
// holds one expert); the topk_group groups with the largest scores (ties to
// the lower group index) stay eligible and the K experts are chosen among
// their experts only. n_group = 1 is the plain selection above.
// ---------------------------------------------------------------------------
// Router scores of one token: l_e = x . W_r[e] (double sum over h), the
// sigmoid s_e = 1 / (1 + exp(-l_e)) and the selection score c_e = s_e + b_e.
static void ref_scores(const float* x, const float* wr, const float* bias, int64_t H,
                       int64_t E, double* s, double* c, double* logits_out) {
    for (int64_t e = 0; e < E; ++e) {
        double l = 0.0;
        for (int64_t h = 0; h < H; ++h) l += (double)x[h] * (double)wr[e * H + h];
        if (logits_out) logits_out[e] = l;
        s[e] = 1.0 / (1.0 + std::exp(-l));
        c[e] = s[e] + (double)bias[e];
    }
}

// Gate values of the chosen experts idx[0..K): the unbiased scores s, divided
// by their sum (k ascending) when normalising, times rho, rounded to fp32.
static void ref_gate_values(const double* s, const int32_t* idx, int64_t K, int norm,
                            double rho, float* w) {
    double sum = 0.0;
    for (int64_t k = 0; k < K; ++k) sum += s[idx[k]];
    for (int64_t k = 0; k < K; ++k) {
        double v = s[idx[k]];
        if (norm) v = v / sum;
        v = v * rho;
        w[k] = (float)v;
    }
}

static void ref_route_token(const float* x, const float* wr, const float* bias, int64_t H,
                            int64_t E, int64_t K, int norm, double rho, int64_t n_group,
                            int64_t topk_group, int32_t* idx, float* w, double* logits_out) {
    std::vector<double> s(E), c(E);
    ref_scores(x, wr, bias, H, E, s.data(), c.data(), logits_out);
    std::vector<char> eligible(E, 1);
    if (n_group > 1) {
        const int64_t gs = E / n_group;
        std::vector<double> gscore(n_group);
        for (int64_t g = 0; g < n_group; ++g) {
            // the largest and second largest c of the group
            int64_t first = g * gs;
            for (int64_t e = g * gs; e < (g + 1) * gs; ++e)
                if (c[e] > c[first]) first = e;
            double second = 0.0;
            bool have_second = false;
            for (int64_t e = g * gs; e < (g + 1) * gs; ++e) {
                if (e == first) continue;
                if (!have_second || c[e] > second) second = c[e];
                have_second = true;
            }
            gscore[g] = have_second ? c[first] + second : c[first];
        }
        std::vector<char> kept(n_group, 0);
        for (int64_t j = 0; j < topk_group; ++j) {
            int64_t best = -1;
            for (int64_t g = 0; g < n_group; ++g) {
                if (kept[g]) continue;
                if (best < 0 || gscore[g] > gscore[best]) best = g;  // ties: lower group
            }
            kept[best] = 1;
        }
        for (int64_t e = 0; e < E; ++e) eligible[e] = kept[e / gs];
    }
    std::vector<char> taken(E, 0);
    for (int64_t k = 0; k < K; ++k) {
        int64_t best = -1;
        for (int64_t e = 0; e < E; ++e) {
            if (taken[e] || !eligible[e]) continue;
            if (best < 0 || c[e] > c[best]) best = e;  // strict '>' keeps the lower index on ties
        }
        taken[best] = 1;
        idx[k] = (int32_t)best;
    }
    ref_gate_values(s.data(), idx, K, norm, rho, w);
}

// n_group >= 1 must divide n_experts; 1 <= topk_group <= n_group; the kept
// groups must hold at least top_k experts.
static bool ref_groups_ok(int64_t E, int64_t K, int64_t n_group, int64_t topk_group) {
    return n_group >= 1 && E % n_group == 0 && topk_group >= 1 && topk_group <= n_group &&
           (n_group == 1 || topk_group * (E / n_group) >= K);
}

int coli_ref_route(const float* x, const float* wr, const float* bias, int64_t n_tok,
                   int64_t hidden, int64_t n_experts, int64_t top_k, int norm, double rho,
                   int64_t n_group, int64_t topk_group, int32_t* idx, float* w, double* logits) {
    if (!x || !wr || !bias || !idx || !w || n_tok < 0 || hidden <= 0 || n_experts <= 0 ||
        top_k <= 0 || top_k > n_experts || !ref_groups_ok(n_experts, top_k, n_group, topk_group))
        return REF_EINVAL;
    for (int64_t t = 0; t < n_tok; ++t)
        ref_route_token(x + t * hidden, wr, bias, hidden, n_experts, top_k, norm, rho, n_group,
                        topk_group, idx + t * top_k, w + t * top_k,
                        logits ? logits + t * n_experts : nullptr);
    return REF_OK;
}

// Gate values the router gives a given choice of experts: for each token the
// scores of ref_scores and the gate values of ref_gate_values for the K
// experts idx[t][0..K) (distinct, in range), as coli_ref_route computes them
// for its own choice. Used where several choices are correct (scores within a
// tolerance of each other at the K-th place): the gate values of another
// correct choice.
int coli_ref_gates(const float* x, const float* wr, const float* bias, int64_t n_tok,
                   int64_t hidden, int64_t n_experts, int64_t top_k, int norm, double rho,
                   const int32_t* idx, float* w) {
    if (!x || !wr || !bias || !idx || !w || n_tok < 0 || hidden <= 0 || n_experts <= 0 ||
        top_k <= 0 || top_k > n_experts)
        return REF_EINVAL;
    std::vector<double> s(n_experts), c(n_experts);
    for (int64_t t = 0; t < n_tok; ++t) {
        const int32_t* it = idx + t * top_k;
        for (int64_t k = 0; k < top_k; ++k) {
            if (it[k] < 0 || it[k] >= n_experts) return REF_EINVAL;
            for (int64_t j = 0; j < k; ++j)
                if (it[j] == it[k]) return REF_EINVAL;
        }
        ref_scores(x + t * hidden, wr, bias, hidden, n_experts, s.data(), c.data(), nullptr);
        ref_gate_values(s.data(), it, top_k, norm, rho, w + t * top_k);
    }
    return REF_OK;
}

// ---------------------------------------------------------------------------
// RMSNorm with unit gain: out = fp32( x / sqrt( mean(x^2) + eps ) ), in double.
// (Only the layer-stack workload uses it: a pre-norm residual between layers.)
// ---------------------------------------------------------------------------
int coli_ref_rmsnorm(const float* x, int64_t n_tok, int64_t dim, double eps, float* out) {
    if (!x || !out || n_tok < 0 || dim <= 0) return REF_EINVAL;
    for (int64_t t = 0; t < n_tok; ++t) {
        double ss = 0.0;
        for (int64_t i = 0; i < dim; ++i) ss += (double)x[t * dim + i] * (double)x[t * dim + i];
        double rms = std::sqrt(ss / (double)dim + eps);
        for (int64_t i = 0; i < dim; ++i) out[t * dim + i] = (float)((double)x[t * dim + i] / rms);
    }
    return REF_OK;
}

// ---------------------------------------------------------------------------
// The layer.
// ---------------------------------------------------------------------------
typedef struct coli_ref_layer {
    int64_t hidden, inter, n_experts, top_k, n_shared, norm_topk;
    double rho;
    const float* w_router;        // [E, H]
    const float* bias;            // [E]
    const uint8_t* const* gate_q; // per expert (E + n_shared; shared last): [I, H b/8] or NULL
    const uint8_t* const* up_q;   // [I, H b/8]
    const uint8_t* const* down_q; // [H, I b/8]
    const float* const* gate_s;   // [I]
    const float* const* up_s;     // [I]
    const float* const* down_s;   // [H]
    int64_t n_group, topk_group;  // group-limited selection (1, 1: none)
    int64_t weight_bits;          // 2, 4 or 8 (0 reads as 4)
} coli_ref_layer;

// Optional intermediate outputs, indexed by token t and slot k (k < K: the
// k-th routed expert of t; k == K: the shared expert). NULL = not wanted.
typedef struct coli_ref_taps {
    int32_t* idx;   // [T, K]
    float* w;       // [T, K]
    double* logits; // [T, E]
    int8_t* qx;     // [T, H]
    float* dx;      // [T, H/32]
    float* g;       // [T, K+S, I]
    float* u;       // [T, K+S, I]
    float* h;       // [T, K+S, I]
    int8_t* qh;     // [T, K+S, I]
    float* dh;      // [T, K+S, I/32]
    float* ye;      // [T, K+S, H]
} coli_ref_taps;

// One SwiGLU expert on one Q8_0 token:
//   g_r = fp32(s_gate[r] * sum_b d_b I_b(gate row r)),  u_r likewise with up
//   h_r = fp32( silu(g_r) * u_r ),  silu(z) = z / (1 + exp(-z))  in double
//   (q_h, d_h) = Q8_0(h)
//   y_c = fp32( s_down[c] * sum_b d_h,b I_b(down row c) )
// Readings: the SwiGLU form and the requantisation of h before the down
// projection (the pages give only the intermediate size).
static void ref_expert(const coli_ref_layer* L, int64_t e, const int8_t* qx, const float* dx,
                       float* g, float* u, float* h, int8_t* qh, float* dh, float* ye) {
    const int64_t H = L->hidden, I = L->inter;
    const int bits = L->weight_bits ? (int)L->weight_bits : 4;
    const uint8_t* gq = L->gate_q[e];
    const uint8_t* uq = L->up_q[e];
    const uint8_t* dq = L->down_q[e];
    const float* gs = L->gate_s[e];
    const float* us = L->up_s[e];
    const float* ds = L->down_s[e];
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < I; ++r) {
        float gr = ref_row_dot(gq + r * (H * bits / 8), gs[r], qx, dx, H / 32, bits);
        float ur = ref_row_dot(uq + r * (H * bits / 8), us[r], qx, dx, H / 32, bits);
        double zg = (double)gr;
        double silu = zg / (1.0 + std::exp(-zg));
        g[r] = gr;
        u[r] = ur;
        h[r] = (float)(silu * (double)ur);
    }
    for (int64_t b = 0; b < I / 32; ++b) ref_q8_block(h + b * 32, qh + b * 32, dh + b);
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < H; ++c)
        ye[c] = ref_row_dot(dq + c * (I * bits / 8), ds[c], qh, dh, I / 32, bits);
}

// y[t] = fp32( sum_k w[t,k] * y_{e_k}[t] + y_shared[t] )   (double, k ascending, shared last)
// The shared expert enters with weight 1 (DeepSeek-V3 convention; the pages
// say only that its output is added). With `accumulate`, the fp32 result is
// added to the existing y (residual): y = y + fp32(...).
// forced_idx/forced_w (both or neither) replace the router's choice.
int coli_ref_moe_forward(const coli_ref_layer* L, const float* x, int64_t n_tok,
                         const int32_t* forced_idx, const float* forced_w, float* y,
                         int accumulate, coli_ref_taps* taps) {
    if (!L || !x || !y || n_tok < 0) return REF_EINVAL;
    const int64_t H = L->hidden, I = L->inter, E = L->n_experts, K = L->top_k,
                  S = L->n_shared;
    if (H <= 0 || I <= 0 || (H % 32) || (I % 32) || E <= 0 || K <= 0 || K > E || S < 0 ||
        S > 1 || !ref_groups_ok(E, K, L->n_group, L->topk_group) ||
        (L->weight_bits != 0 && !ref_bits_ok((int)L->weight_bits)))
        return REF_EINVAL;
    if ((forced_idx == nullptr) != (forced_w == nullptr)) return REF_EINVAL;
    const int64_t KS = K + S;
    std::vector<int32_t> idx(K);
    std::vector<float> w(K);
    std::vector<int8_t> qx(H), qh(I);
    std::vector<float> dx(H / 32), dh(I / 32), g(I), u(I), h(I), ye(H);
    std::vector<double> acc(H);
    for (int64_t t = 0; t < n_tok; ++t) {
        const float* xt = x + t * H;
        if (forced_idx) {
            for (int64_t k = 0; k < K; ++k) {
                idx[k] = forced_idx[t * K + k];
                w[k] = forced_w[t * K + k];
                if (idx[k] < 0 || idx[k] >= E) return REF_EINVAL;
            }
        } else {
            if (!L->w_router || !L->bias) return REF_EINVAL;
            ref_route_token(xt, L->w_router, L->bias, H, E, K, (int)L->norm_topk, L->rho,
                            L->n_group, L->topk_group, idx.data(), w.data(),
                            (taps && taps->logits) ? taps->logits + t * E : nullptr);
        }
        coli_ref_quant_q8(xt, 1, H, qx.data(), dx.data());
        std::fill(acc.begin(), acc.end(), 0.0);
        for (int64_t k = 0; k < KS; ++k) {
            const int64_t e = (k < K) ? idx[k] : E;  // shared expert stored at index E
            if (!L->gate_q[e] || !L->up_q[e] || !L->down_q[e] || !L->gate_s[e] ||
                !L->up_s[e] || !L->down_s[e])
                return REF_EINVAL;
            ref_expert(L, e, qx.data(), dx.data(), g.data(), u.data(), h.data(), qh.data(),
                       dh.data(), ye.data());
            const double wk = (k < K) ? (double)w[k] : 1.0;
            for (int64_t c = 0; c < H; ++c) acc[c] += wk * (double)ye[c];
            if (taps) {
                const int64_t slot = t * KS + k;
                if (taps->g) std::memcpy(taps->g + slot * I, g.data(), I * sizeof(float));
                if (taps->u) std::memcpy(taps->u + slot * I, u.data(), I * sizeof(float));
                if (taps->h) std::memcpy(taps->h + slot * I, h.data(), I * sizeof(float));
                if (taps->qh) std::memcpy(taps->qh + slot * I, qh.data(), I);
                if (taps->dh)
                    std::memcpy(taps->dh + slot * (I / 32), dh.data(), (I / 32) * sizeof(float));
                if (taps->ye) std::memcpy(taps->ye + slot * H, ye.data(), H * sizeof(float));
            }
        }
        for (int64_t c = 0; c < H; ++c) {
            float v = (float)acc[c];
            y[t * H + c] = accumulate ? y[t * H + c] + v : v;
        }
        if (taps) {
            if (taps->idx) std::memcpy(taps->idx + t * K, idx.data(), K * sizeof(int32_t));
            if (taps->w) std::memcpy(taps->w + t * K, w.data(), K * sizeof(float));
            if (taps->qx) std::memcpy(taps->qx + t * H, qx.data(), H);
            if (taps->dx) std::memcpy(taps->dx + t * (H / 32), dx.data(), (H / 32) * sizeof(float));
        }
    }
    return REF_OK;
}

int coli_ref_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void coli_ref_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

}  // extern "C"
