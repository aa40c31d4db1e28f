// Host side of the C ABI (include/coli_moe.h): argument checks, workspace
// layout, kernel selection and the launches of the routing and small kernels;
// the few-token, grouped MFMA and GEMV kernel families are launched from
// their own translation units (coli_launch.h). No allocation, no
// synchronisation.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>

#include "coli_moe.h"
#include "coli_launch.h"
#include "k_probe.h"
#include "k_route.h"
#include "k_small.h"

namespace {

constexpr int kMaxHidden = 8192;  // 4 blocks of 64 per lane in the GEMV kernels
constexpr int kMaxInter = 8192;
constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 16;
constexpr int kGemvChunk = 4;     // tokens per item on the GEMV path
constexpr int kMaxRouterSplit = 16;  // hidden-dimension slices of the router GEMM
constexpr int64_t kTapBudget = 1ll << 24;  // int32 entries of the block-dot tap

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Router GEMM partial sums: slices x tokens the split (router_ksplit) may use
// at T tokens. The split is at most kMaxRouterSplit and, once it exceeds one,
// at most 1024 / tiles with tiles >= (T / 64) ceil(E / 64), so slices x T <=
// 65536 / ceil(E / 64); with one slice it is T. The bound never decreases as
// T grows, and router_ksplit never exceeds it.
int64_t router_part_slots(int64_t T, int E) {
    const int64_t et = (E + kRouterTile - 1) / kRouterTile;
    return std::min<int64_t>((int64_t)kMaxRouterSplit * T,
                             std::max<int64_t>(T, 1024 * kRouterTile / et));
}

inline bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

int check_cfg(const coli_moe_cfg* c) {
    if (!c) return COLI_E_INVAL;
    if (c->hidden <= 0 || c->hidden % 32 || c->inter <= 0 || c->inter % 32) return COLI_E_INVAL;
    if (c->n_experts <= 0 || c->top_k <= 0 || c->top_k > c->n_experts) return COLI_E_INVAL;
    if (c->n_shared < 0 || c->n_shared > 1) return COLI_E_INVAL;
    if (!std::isfinite(c->routed_scale)) return COLI_E_INVAL;
    if (c->n_group < 0) return COLI_E_INVAL;
    if (c->weight_bits != 0 && c->weight_bits != 2 && c->weight_bits != 4 && c->weight_bits != 8)
        return COLI_E_INVAL;
    if (c->n_group > 1) {
        if (c->n_group > 64) return COLI_E_UNSUPPORTED;
        if (c->n_experts % c->n_group || c->topk_group < 1 || c->topk_group > c->n_group ||
            (int64_t)c->topk_group * (c->n_experts / c->n_group) < c->top_k)
            return COLI_E_INVAL;
    }
    if (c->hidden > kMaxHidden || c->inter > kMaxInter || c->n_experts > kMaxExperts ||
        c->top_k > kMaxTopK)
        return COLI_E_UNSUPPORTED;
    return COLI_OK;
}

GroupSel group_sel(const coli_moe_cfg& c) {
    GroupSel g{1, c.n_experts, 1};
    if (c.n_group > 1) g = GroupSel{c.n_group, c.n_experts / c.n_group, c.topk_group};
    return g;
}

struct Layout {
    coli_moe_ws_layout pub;
    size_t lists, items, n_items, uinfo, rpart, sig;
    size_t mx, ex, mh, eh;  // integer block scales of x and h (grouped MFMA path)
    int64_t max_items;
    int ch;
};

int64_t max_items_for(const coli_moe_cfg& c, int64_t T, int ch) {
    const int64_t TK = T * c.top_k;
    const int64_t routed = (TK < c.n_experts ? TK : c.n_experts) + TK / ch;
    const int64_t shared = c.n_shared ? (T + ch - 1) / ch : 0;
    return routed + shared;
}

void make_layout(const coli_moe_cfg& c, int64_t T, uint32_t flags, Layout* L) {
    const int64_t H = c.hidden, I = c.inter, E = c.n_experts, K = c.top_k, S = c.n_shared;
    const int64_t NE = E + S, KS = K + S, NS = T * KS;
    std::memset(L, 0, sizeof(*L));
    L->ch = kGemvChunk;
    L->max_items = max_items_for(c, T, L->ch);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = align256(off + bytes);
        return at;
    };
    coli_moe_ws_layout& P = L->pub;
    P.n_slots = NS;
    P.qx = take(T * H);
    P.dx = take(T * (H / 32) * 4);
    P.logits = take(T * E * 8);
    P.topk_idx = take(T * K * 4);
    P.topk_w = take(T * K * 4);
    P.counts = take(NE * 4);
    P.offs = take((NE + 1) * 4);
    L->lists = take(NE * T * 4);
    P.slot_of = take(T * KS * 4);
    P.slot_tok = take(NS * 4);
    L->items = take(3 * L->max_items * 4);
    L->n_items = take(4);
    L->uinfo = take(4 * (1 + 4 * dec::kMaxEntries + 64));
    L->rpart = take(T > 8 ? (size_t)router_part_slots(T, (int)E) * E * 8 : 0);
    // s and c of the few-token path; reserved for min(T, its token limit) at
    // every T so that the total never shrinks as T grows
    L->sig = take((size_t)2 * std::min<int64_t>(T, dec::kMaxTok) * E * 8);

    P.qh = take(NS * I);
    P.dh = take(NS * (I / 32) * 4);
    P.ye = take(NS * H * 4);
    L->mx = take(T * (H / 32) * 4);
    L->ex = take(T * 4);
    L->mh = take(NS * (I / 32) * 4);
    L->eh = take(NS * 4);
    if (flags & COLI_FWD_DEBUG_TAPS) {
        const int64_t per_row = NS * (H / 32);
        int64_t stride = 1;
        // sampled gate rows (every stride-th) keep the tap near the budget; one
        // row per slot at the least
        while (stride < I && per_row * ((I + stride - 1) / stride) > kTapBudget) stride *= 2;
        P.tap_stride = stride;
        P.tap_rows = (I + stride - 1) / stride;
        // once rows are sampled the tap takes the whole budget, so that the
        // total never shrinks as T grows (a caller sizes for its largest T)
        const size_t tap_bytes = (size_t)NS * P.tap_rows * (H / 32) * 4;
        P.tap = take(stride == 1 ? tap_bytes : std::max(tap_bytes, (size_t)kTapBudget * 4));
    }

    P.total = off;
}

// Router + top-k into ws (shared by coli_moe_route and coli_moe_forward).
// Slices of the hidden dimension for the many-token router GEMM: about 1024
// workgroups (four per CU), each slice a multiple of 32.
int router_ksplit(int H, int64_t T, int E) {
    const int64_t tiles = ((T + kRouterTile - 1) / kRouterTile) * ((E + kRouterTile - 1) / kRouterTile);
    int ks = (int)std::max<int64_t>(1, std::min<int64_t>(kMaxRouterSplit, 1024 / std::max<int64_t>(tiles, 1)));
    while (ks > 1 && (int64_t)ks * T > router_part_slots(T, E)) --ks;  // the workspace holds these
    while (ks > 1 && H % (kRouterK * ks) != 0) --ks;
    return ks;
}

void launch_route(const coli_moe_cfg& c, const float* x, const float* wr, const float* bias,
                  int64_t T, double* logits, double* rpart, int32_t* idx, float* wts,
                  hipStream_t s, Marks& mk) {
    const int H = c.hidden, E = c.n_experts, K = c.top_k;
    mk.mark("router_logits");
    if (T <= 8) {
        if (T <= 1)
            launch(mk, k_router_gemv<1>, E, 256, 0, s, x, wr, (int)T, H, E, logits);
        else if (T <= 4)
            launch(mk, k_router_gemv<4>, E, 256, 0, s, x, wr, (int)T, H, E, logits);
        else
            launch(mk, k_router_gemv<8>, E, 256, 0, s, x, wr, (int)T, H, E, logits);
    } else {
        const int ks = router_ksplit(H, T, E);
        dim3 g((unsigned)((T + kRouterTile - 1) / kRouterTile),
               (unsigned)((E + kRouterTile - 1) / kRouterTile), (unsigned)ks);
        launch(mk, k_router_gemm, g, 256, 0, s, x, wr, (int)T, H, E, ks, rpart);
        const int64_t n = T * E;
        mk.mark("router_reduce");
        launch(mk, k_router_reduce, (unsigned)((n + 255) / 256), 256, 0, s, rpart, ks, n, logits);
    }
    mk.mark("topk");
    const unsigned gb = (unsigned)((T + 3) / 4);
    const double rho = (double)c.routed_scale;
    const int norm = c.norm_topk ? 1 : 0;
    const GroupSel gsel = group_sel(c);
    // with groups, each wave stages its token's biased scores in LDS
    const size_t tk_lds = gsel.ng > 1 ? (size_t)4 * E * sizeof(double) : 0;
    if (E <= 256 && K <= 16)
        launch_topk_wave(logits, bias, T, E, K, norm, rho, gsel, idx, wts, s, mk);
    else if (E <= 64)
        launch(mk, k_topk<1>, gb, 256, tk_lds, s, logits, bias, (int)T, E, K, norm, rho, gsel, idx, wts);
    else if (E <= 128)
        launch(mk, k_topk<2>, gb, 256, tk_lds, s, logits, bias, (int)T, E, K, norm, rho, gsel, idx, wts);
    else if (E <= 256)
        launch(mk, k_topk<4>, gb, 256, tk_lds, s, logits, bias, (int)T, E, K, norm, rho, gsel, idx, wts);
    else if (E <= 512)
        launch(mk, k_topk<8>, gb, 256, tk_lds, s, logits, bias, (int)T, E, K, norm, rho, gsel, idx, wts);
    else
        launch(mk, k_topk<16>, gb, 256, tk_lds, s, logits, bias, (int)T, E, K, norm, rho, gsel, idx, wts);
}

int hip_status() {
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? COLI_OK : COLI_E_HIP;
}

int forward_impl(const coli_moe_weights* w, const float* x, int64_t T, float* y, void* ws,
                 size_t ws_bytes, uint32_t flags, hipStream_t s, Marks& mk) {
    if (!w || T < 0) return COLI_E_INVAL;
    int rc = check_cfg(&w->cfg);
    if (rc) return rc;
    if (w->cfg.reserved != 0) return COLI_E_INVAL;
    if (flags & ~(COLI_FWD_ACCUM | COLI_FWD_DEBUG_TAPS)) return COLI_E_INVAL;
    if (T == 0) return COLI_OK;  // no-op; x, y and ws may be NULL
    if (!x || !y || !ws) return COLI_E_INVAL;
    if (!w->w_router || !w->bias || !w->experts_q || !w->experts_scale) return COLI_E_INVAL;
    if (misaligned(x) || misaligned(y) || misaligned(ws) || misaligned(w->w_router) ||
        misaligned(w->bias) || misaligned(w->experts_q) || misaligned(w->experts_scale))
        return COLI_E_ALIGN;
    if (T > (int64_t)1 << 20) return COLI_E_UNSUPPORTED;
    const coli_moe_cfg& c = w->cfg;
    Layout L;
    make_layout(c, T, flags, &L);
    if (ws_bytes < L.pub.total) return COLI_E_WORKSPACE;

    const int H = c.hidden, I = c.inter, E = c.n_experts, K = c.top_k, S = c.n_shared;
    const int bits = weight_bits(c);
    const int64_t blob_q = 3ll * I * H * bits / 8, blob_s = 2ll * I + H;
    // few tokens: the fused kernels (every width); else the grouped MFMA
    // path when the row tiles divide the shapes, else the GEMV path, which
    // has int4 weights only
    const bool mfma = (H % pf::kRows) == 0 && (I % pf::kRows) == 0;
    if (bits != 4 && !mfma && !small_path_fits(c, T)) return COLI_E_UNSUPPORTED;
    char* base = static_cast<char*>(ws);
    int8_t* qx = reinterpret_cast<int8_t*>(base + L.pub.qx);
    float* dx = reinterpret_cast<float*>(base + L.pub.dx);
    double* logits = reinterpret_cast<double*>(base + L.pub.logits);
    int32_t* idx = reinterpret_cast<int32_t*>(base + L.pub.topk_idx);
    float* wts = reinterpret_cast<float*>(base + L.pub.topk_w);
    int32_t* counts = reinterpret_cast<int32_t*>(base + L.pub.counts);
    int32_t* offs = reinterpret_cast<int32_t*>(base + L.pub.offs);
    int32_t* lists = reinterpret_cast<int32_t*>(base + L.lists);
    int32_t* slot_of = reinterpret_cast<int32_t*>(base + L.pub.slot_of);
    int32_t* slot_tok = reinterpret_cast<int32_t*>(base + L.pub.slot_tok);
    int32_t* items = reinterpret_cast<int32_t*>(base + L.items);
    int32_t* n_items = reinterpret_cast<int32_t*>(base + L.n_items);
    int8_t* qh = reinterpret_cast<int8_t*>(base + L.pub.qh);
    float* dh = reinterpret_cast<float*>(base + L.pub.dh);
    float* ye = reinterpret_cast<float*>(base + L.pub.ye);
    int32_t* tap = (flags & COLI_FWD_DEBUG_TAPS) ? reinterpret_cast<int32_t*>(base + L.pub.tap)
                                                 : nullptr;
    ItemArgs it{items, items + L.max_items, items + 2 * L.max_items, n_items};

    if (small_path_fits(c, T)) {
        dec::DecArgs a{};
        a.x = x; a.wr = w->w_router; a.bias = w->bias; a.eq = w->experts_q; a.es = w->experts_scale;
        a.blob_q = blob_q; a.blob_s = blob_s;
        a.T = (int)T; a.H = H; a.I = I; a.E = E; a.K = K; a.S = S; a.norm = c.norm_topk ? 1 : 0;
        a.rho = (double)c.routed_scale;
        a.gsel = group_sel(c);
        a.logits = logits; a.qx = qx; a.dx = dx; a.idx = idx; a.wts = wts; a.counts = counts;
        a.offs = offs; a.slot_of = slot_of; a.slot_tok = slot_tok;
        a.uinfo = reinterpret_cast<int32_t*>(base + L.uinfo);
        a.sig = reinterpret_cast<double*>(base + L.sig);
        a.cval = a.sig + T * E;
        a.qh = qh; a.dh = dh; a.tap = tap;
        a.tap_rows = (int)L.pub.tap_rows;
        a.tap_stride = (int)(L.pub.tap_stride ? L.pub.tap_stride : 1);
        a.y = y; a.accum = (flags & COLI_FWD_ACCUM) ? 1 : 0;
        launch_small(a, bits, s, mk);
        return hip_status();
    }

    mk.mark("quant_x");
    const int64_t nblk = T * (H / 32);
    // activations in the element order of the weight width's operand
    const unsigned qg = (unsigned)((nblk * 4 + 255) / 256);
    if (bits == 4) launch(mk, k_quant_q8<1>, qg, 256, 0, s, x, nblk, qx, dx);
    else if (bits == 2) launch(mk, k_quant_q8<2>, qg, 256, 0, s, x, nblk, qx, dx);
    else launch(mk, k_quant_q8<0>, qg, 256, 0, s, x, nblk, qx, dx);

    launch_route(c, x, w->w_router, w->bias, T, logits,
                 reinterpret_cast<double*>(base + L.rpart), idx, wts, s, mk);

    // tokens per work item of the MFMA kernels: 64 once the routed experts
    // average 48 tokens or more (fewer weight re-reads, each staged block used
    // by up to four token groups), else 32 (more workgroups per CU)
    const int kt = (T * K >= 48 * (int64_t)E) ? 64 : 32;
    const int ch = mfma ? kt : L.ch;
    const int64_t n_it = max_items_for(c, T, ch);
    mk.mark("bucket_lists");
    launch(mk, k_bucket_lists, E + S, 256, 0, s, idx, (int)T, K, E, S, lists, counts);
    mk.mark("bucket_fill");
    launch(mk, k_bucket_fill, E + S, 256, 0, s, counts, lists, (int)T, K, E, S, ch, offs, slot_of,
           slot_tok, it.item_e, it.item_s0, it.item_n, n_items);

    if (mfma) {
        pf::PfArgs pa{};
        pa.eq = w->experts_q; pa.es = w->experts_scale; pa.blob_q = blob_q; pa.blob_s = blob_s;
        pa.H = H; pa.I = I; pa.qx = qx; pa.dx = dx;
        pa.item_e = it.item_e; pa.item_s0 = it.item_s0; pa.item_n = it.item_n;
        pa.n_items = it.n_items; pa.offs = offs; pa.slot_tok = slot_tok;
        pa.qh = qh; pa.dh = dh; pa.ye = ye; pa.tap = tap;
        pa.tap_rows = (int)L.pub.tap_rows;
        pa.tap_stride = (int)(L.pub.tap_stride ? L.pub.tap_stride : 1);
        // integer block scales (exact int64 sums in the K loop) from 16 tokens
        // on; below that their two launches cost more than they save, and
        // the kernels take the fp64 epilogue
        if (T >= 16) {
            pa.mx = reinterpret_cast<int32_t*>(base + L.mx);
            pa.ex = reinterpret_cast<int32_t*>(base + L.ex);
            pa.mh = reinterpret_cast<int32_t*>(base + L.mh);
            pa.eh = reinterpret_cast<int32_t*>(base + L.eh);
        }
        launch_pf_path(pa, bits, kt, T, L.pub.n_slots, n_it, s, mk);
    } else {
        launch_gemv_path(w, blob_q, blob_s, qx, dx, it, slot_tok, qh, dh, ye, tap,
                         (int)L.pub.tap_rows, (int)(L.pub.tap_stride ? L.pub.tap_stride : 1), T,
                         L.max_items, s, mk);
    }
    mk.mark("combine");
    launch_combine(ye, slot_of, wts, K, S, H, y, T, (flags & COLI_FWD_ACCUM) ? 1 : 0, s, mk);
    return hip_status();
}

}  // namespace

extern "C" {

COLI_API const char* coli_strerror(int code) {
    switch (code) {
        case COLI_OK: return "ok";
        case COLI_E_INVAL: return "invalid argument (null pointer, bad shape or flag)";
        case COLI_E_ALIGN: return "pointer not 16-byte aligned";
        case COLI_E_WORKSPACE: return "workspace too small";
        case COLI_E_HIP: return "HIP launch failed";
        case COLI_E_UNSUPPORTED: return "size beyond the compiled limits";
        default: return "unknown error";
    }
}

COLI_API int coli_pack_weights(const float* w, int64_t rows, int64_t cols, int bits, uint8_t* q,
                               float* scale, void* stream) {
    if (rows < 0 || cols <= 0 || cols % 32 || (bits != 2 && bits != 4 && bits != 8))
        return COLI_E_INVAL;
    if (rows == 0) return COLI_OK;
    if (!w || !q || !scale) return COLI_E_INVAL;
    if (misaligned(w) || misaligned(q) || misaligned(scale)) return COLI_E_ALIGN;
    if (rows > 0x7fffffffll) return COLI_E_UNSUPPORTED;
    const hipStream_t st = (hipStream_t)stream;
    if (bits == 4) k_pack_bits<4><<<(unsigned)rows, 256, 0, st>>>(w, cols, q, scale);
    else if (bits == 8) k_pack_bits<8><<<(unsigned)rows, 256, 0, st>>>(w, cols, q, scale);
    else k_pack_bits<2><<<(unsigned)rows, 256, 0, st>>>(w, cols, q, scale);
    return hip_status();
}

COLI_API int coli_pack_int4(const float* w, int64_t rows, int64_t cols, uint8_t* q, float* scale,
                            void* stream) {
    return coli_pack_weights(w, rows, cols, 4, q, scale, stream);
}

COLI_API int coli_pack_fp8_int4(const uint8_t* q8, const float* block_scale, int64_t rows,
                                int64_t cols, uint8_t* q, float* scale, void* stream) {
    if (rows < 0 || cols <= 0 || cols % 32) return COLI_E_INVAL;
    if (rows == 0) return COLI_OK;
    if (!q8 || !block_scale || !q || !scale) return COLI_E_INVAL;
    if (misaligned(q8) || misaligned(block_scale) || misaligned(q) || misaligned(scale))
        return COLI_E_ALIGN;
    if (rows > 0x7fffffffll) return COLI_E_UNSUPPORTED;
    const hipStream_t st = (hipStream_t)stream;
    if (cols % 1024 == 0 && cols <= 8192) {
        const int cpl = (int)(cols / 1024);
        const int64_t rpw = (8 % cpl == 0) ? 8 / cpl : 1;
        const int64_t waves = (rows + rpw - 1) / rpw;
        const unsigned grid = (unsigned)((waves + 3) / 4);
        switch (cpl) {
#define COLI_PACK_FP8(n) \
    case n: k_pack_fp8_int4_wave<n><<<grid, 256, 0, st>>>(q8, block_scale, rows, q, scale); break;
            COLI_PACK_FP8(1) COLI_PACK_FP8(2) COLI_PACK_FP8(3) COLI_PACK_FP8(4)
            COLI_PACK_FP8(5) COLI_PACK_FP8(6) COLI_PACK_FP8(7) COLI_PACK_FP8(8)
#undef COLI_PACK_FP8
        }
    } else {
        k_pack_fp8_int4<<<(unsigned)rows, 256, 0, st>>>(q8, block_scale, cols, q, scale);
    }
    return hip_status();
}

COLI_API int coli_quant_q8(const float* x, int64_t n_tok, int64_t dim, int8_t* q, float* d,
                           void* stream) {
    if (n_tok < 0 || dim <= 0 || dim % 32) return COLI_E_INVAL;
    if (n_tok == 0) return COLI_OK;
    if (!x || !q || !d) return COLI_E_INVAL;
    if (misaligned(x) || misaligned(q) || misaligned(d)) return COLI_E_ALIGN;
    const int64_t nblk = n_tok * (dim / 32);
    const int64_t nthr = nblk * 4;
    if ((nthr + 255) / 256 > 0x7fffffffll) return COLI_E_UNSUPPORTED;
    k_quant_q8<0><<<(unsigned)((nthr + 255) / 256), 256, 0, (hipStream_t)stream>>>(x, nblk, q,
                                                                                       d);
    return hip_status();
}

COLI_API size_t coli_moe_workspace_bytes(const coli_moe_cfg* cfg, int64_t max_tok,
                                         uint32_t flags) {
    if (check_cfg(cfg) != COLI_OK || max_tok < 0) return 0;
    Layout L;
    make_layout(*cfg, max_tok, flags, &L);
    return L.pub.total;
}

COLI_API int coli_moe_workspace_layout(const coli_moe_cfg* cfg, int64_t n_tok, uint32_t flags,
                                       coli_moe_ws_layout* out) {
    const int rc = check_cfg(cfg);
    if (rc) return rc;
    if (!out || n_tok < 0) return COLI_E_INVAL;
    Layout L;
    make_layout(*cfg, n_tok, flags, &L);
    *out = L.pub;
    return COLI_OK;
}

COLI_API int coli_moe_route(const float* x, const float* w_router, const float* bias,
                            int64_t n_tok, const coli_moe_cfg* cfg, int32_t* topk_idx,
                            float* topk_w, void* ws, size_t ws_bytes, void* stream) {
    int rc = check_cfg(cfg);
    if (rc) return rc;
    if (n_tok < 0) return COLI_E_INVAL;
    if (n_tok == 0) return COLI_OK;
    if (!x || !w_router || !bias || !topk_idx || !topk_w || !ws) return COLI_E_INVAL;
    if (misaligned(x) || misaligned(w_router) || misaligned(bias) || misaligned(topk_idx) ||
        misaligned(topk_w) || misaligned(ws))
        return COLI_E_ALIGN;
    if (n_tok > (int64_t)1 << 20) return COLI_E_UNSUPPORTED;
    Layout L;
    make_layout(*cfg, n_tok, 0, &L);
    if (ws_bytes < L.pub.total) return COLI_E_WORKSPACE;
    Marks mk{(hipStream_t)stream};
    launch_route(*cfg, x, w_router, bias, n_tok,
                 reinterpret_cast<double*>(static_cast<char*>(ws) + L.pub.logits),
                 reinterpret_cast<double*>(static_cast<char*>(ws) + L.rpart), topk_idx, topk_w,
                 (hipStream_t)stream, mk);
    return hip_status();
}

COLI_API int coli_moe_forward(const coli_moe_weights* w, const float* x, int64_t n_tok, float* y,
                              void* ws, size_t ws_bytes, uint32_t flags, void* stream) {
    Marks mk{(hipStream_t)stream};
    return forward_impl(w, x, n_tok, y, ws, ws_bytes, flags, (hipStream_t)stream, mk);
}

}  // extern "C"

namespace {

// Workspace of coli_moe_forward_static: one array per GPU the library runs
// on, alive until the process ends. In host code `scratch` is only a
// stand-in for the symbol; its device address comes from
// hipGetSymbolAddress, once per device, and only that address is used.
constexpr size_t kStaticScratchBytes = COLI_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch array (nullptr on failure).
void* static_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p) return p;
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr) return nullptr;
    g_scratch_ptr[dev].store(q, std::memory_order_release);  // same value from any racing thread
    return q;
}

}  // namespace

extern "C" {

COLI_API int coli_moe_forward_static(const coli_moe_weights* w, const float* x, int64_t n_tok,
                                     float* y, uint32_t flags, void* stream) {
    Marks mk{(hipStream_t)stream};
    if (!w || n_tok < 0) return COLI_E_INVAL;
    const int rc = check_cfg(&w->cfg);
    if (rc) return rc;
    if (n_tok == 0)  // no-op after the argument checks; touches no scratch
        return forward_impl(w, x, 0, y, nullptr, 0, flags, (hipStream_t)stream, mk);
    if (n_tok > (int64_t)1 << 20) return COLI_E_UNSUPPORTED;
    Layout L;
    make_layout(w->cfg, n_tok, flags, &L);
    if (L.pub.total > kStaticScratchBytes) return COLI_E_WORKSPACE;
    void* ws = static_scratch();
    if (!ws) return COLI_E_HIP;
    return forward_impl(w, x, n_tok, y, ws, kStaticScratchBytes, flags, (hipStream_t)stream, mk);
}

COLI_API int coli_moe_forward_profiled(const coli_moe_weights* w, const float* x, int64_t n_tok,
                                       float* y, void* ws, size_t ws_bytes, uint32_t flags,
                                       void* stream, void* const* events, int n_events,
                                       int* n_used, const char** names) {
    Marks mk{(hipStream_t)stream, events, names, n_events < 0 ? 0 : n_events, 0};
    const int rc = forward_impl(w, x, n_tok, y, ws, ws_bytes, flags, (hipStream_t)stream, mk);
    if (n_used) *n_used = mk.used;
    return rc;
}

COLI_API int coli_mfma_probe(int kind, int64_t n_workgroups, int iters, int64_t* cycles,
                             void* stream) {
    if (kind < 0 || kind > 7 || n_workgroups <= 0 || n_workgroups > (1 << 20) || iters <= 0 ||
        !cycles)
        return COLI_E_INVAL;
    if (reinterpret_cast<uintptr_t>(cycles) & 7u) return COLI_E_ALIGN;
    const hipStream_t st = (hipStream_t)stream;
    const unsigned g = (unsigned)n_workgroups;
    long long* c = reinterpret_cast<long long*>(cycles);
    switch (kind) {
#define COLI_PROBE(k) \
    case k: probe::k_mfma_probe<k><<<g, 256, 0, st>>>(iters, 1, c); break;
        COLI_PROBE(0) COLI_PROBE(1) COLI_PROBE(2) COLI_PROBE(3)
        COLI_PROBE(4) COLI_PROBE(5) COLI_PROBE(6) COLI_PROBE(7)
#undef COLI_PROBE
    }
    return hip_status();
}

COLI_API int coli_rmsnorm(const float* x, int64_t n_tok, int64_t dim, float eps, float* out,
                          void* stream) {
    if (n_tok < 0 || dim <= 0 || !(eps >= 0.0f)) return COLI_E_INVAL;
    if (n_tok == 0) return COLI_OK;
    if (!x || !out) return COLI_E_INVAL;
    if (misaligned(x) || misaligned(out)) return COLI_E_ALIGN;
    if (n_tok > 0x7fffffffll) return COLI_E_UNSUPPORTED;
    const int vec = dim % 4 == 0 && dim <= 8192;  // rows then 16-byte aligned too
    k_rmsnorm<<<(unsigned)n_tok, 256, 0, (hipStream_t)stream>>>(x, dim, (double)eps, out, vec);
    return hip_status();
}

COLI_API int coli_stream_read(const void* src, int64_t bytes, uint32_t* sink, void* stream) {
    if (bytes < 0 || (bytes & 15) != 0) return COLI_E_INVAL;
    if (bytes == 0) return COLI_OK;
    if (!src || !sink) return COLI_E_INVAL;
    if (misaligned(src) || (reinterpret_cast<uintptr_t>(sink) & 3) != 0) return COLI_E_ALIGN;
    const int64_t n16 = bytes >> 4;
    const int64_t want = (n16 + 255) / 256;
    const unsigned grid = (unsigned)(want < 256 ? want : 256);  // one workgroup per CU
    k_stream_read<<<grid, 256, 0, (hipStream_t)stream>>>(reinterpret_cast<const v4u_s*>(src), n16,
                                                         sink);
    return hip_status();
}

}  // extern "C"
