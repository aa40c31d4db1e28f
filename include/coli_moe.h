/*
 * coli_moe.h — C ABI of the MI355X (gfx950) library for one sigmoid-routed
 * Mixture-of-Experts layer with symmetric int4 expert weights and Q8_0 int8
 * activations.
 *
 * The operation comes from the pages on the colibri engine for GLM-5.2:
 *  - wmrh.cn, "GLM-5.2-colibri-int4架构解析MoE专家混合与INT4量化原理",
 *    section "GLM-5.2的MoE实现": 256 routed experts, 1 shared expert, 8
 *    experts per token, hidden size 6144, expert intermediate size 2048;
 *    section "MoE的工作原理": every token gets router scores, the 8
 *    highest-scoring experts run and their outputs are summed weighted by
 *    score; section "量化流程": weights go FP8 -> F32 -> int4 with np.rint
 *    (chosen to agree with the engine's lrintf), one F32 scale per weight
 *    row, 4-bit values packed into U8; section "路由策略定制": the knobs
 *    topk_method, routed_scaling_factor and norm_topk_prob.
 *  - "Colibri：在笔记本上跑744B参数的AI模型", feature list (关键特性): a
 *    DeepSeek-V3-style sigmoid router with a shared expert; an integer dot
 *    kernel over Q8_0-style int8 activations.
 *  - hn mirror (hn.213312.xyz) of the project summary, feature list: in a
 *    batch an expert needed by several positions is read once and shared.
 *
 * Conventions for every call
 *  - Pointers are DEVICE pointers owned by the caller, row-major and
 *    contiguous, 16-byte aligned (else COLI_E_ALIGN). The library never
 *    allocates, frees or keeps them.
 *  - `stream` is a hipStream_t passed as void*; NULL is the null stream.
 *    Every call only enqueues work on that stream: it neither allocates nor
 *    synchronises, and results are ready when the stream reaches them.
 *  - Calls return COLI_OK (0) or a negative code; arguments are checked on
 *    the host before anything is launched, so a rejected call has no effect.
 *    A call with zero rows/tokens is a no-op and may pass NULL data pointers
 *    (shape and config arguments are still checked).
 *    COLI_E_HIP reports a launch failure from the HIP runtime.
 *  - The library keeps no state between calls; concurrent calls are safe
 *    when they use different workspaces (calls sharing one workspace must be
 *    ordered, e.g. on one stream).
 */
#ifndef COLI_MOE_H
#define COLI_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define COLI_API __attribute__((visibility("default")))

#define COLI_OK 0
#define COLI_E_INVAL (-1)       /* null pointer, bad size, dim % 32 != 0, K > E, K > 16 ... */
#define COLI_E_ALIGN (-2)       /* a pointer is not 16-byte aligned */
#define COLI_E_WORKSPACE (-3)   /* ws_bytes smaller than coli_moe_workspace_bytes() */
#define COLI_E_HIP (-4)         /* the HIP runtime rejected a launch */
#define COLI_E_UNSUPPORTED (-5) /* a size beyond the compiled limits */

/* coli_moe_forward flags */
#define COLI_FWD_ACCUM 1u      /* y += layer(x) (residual add in fp32) instead of y = layer(x) */
#define COLI_FWD_DEBUG_TAPS 2u /* also store per-block int32 dots of the gate rows in ws */

/* Layer shape and routing knobs (the knob names follow the model's
 * config.json fields named on the wmrh.cn page, section 路由策略定制). */
typedef struct coli_moe_cfg {
    int32_t hidden;       /* H, multiple of 32, <= 8192 */
    int32_t inter;        /* I, expert intermediate size, multiple of 32, <= 8192 */
    int32_t n_experts;    /* E routed experts, 1..1024 */
    int32_t top_k;        /* K experts per token, 1..min(E, 16) */
    int32_t n_shared;     /* 0 or 1 shared expert (stored after the routed ones) */
    int32_t norm_topk;    /* norm_topk_prob: 1 = divide the K gate values by their sum */
    float routed_scale;   /* routed_scaling_factor rho, applied after normalisation */
    int32_t n_group;      /* group-limited selection (topk_method): 0 or 1 = none; else
                             2..64 groups of n_experts / n_group consecutive experts */
    int32_t topk_group;   /* groups kept when n_group > 1: 1..n_group, and the kept
                             groups must hold at least top_k experts */
    int32_t weight_bits;  /* expert weight codes: 4 (0 reads as 4), 8 or 2; beyond the
                             few-token path (up to 4 tokens, int2: 2, with H <= 6144,
                             I <= 2048 and I a multiple of 64) int8 and int2 need hidden
                             and inter multiples of 64, else COLI_E_UNSUPPORTED */
    int32_t reserved;     /* must be 0 */
} coli_moe_cfg;

/* Weights of one layer (all device memory, owned by the caller).
 *  w_router      [E, H] fp32 router weight (kept in F32, not quantised)
 *  bias          [E] fp32 correction bias: added to the sigmoid score for
 *                expert selection only; the gate value is the unbiased score
 *  experts_q     E + n_shared contiguous expert blobs of 3*I*H*b/8 bytes (b =
 *                weight_bits), blob e = [gate I x H b/8 | up I x H b/8 |
 *                down H x I b/8], rows = output channels, in the
 *                coli_pack_weights format of width b (int4: byte j of a row =
 *                code(2j) | code(2j+1) << 4 with 4-bit two's complement codes
 *                in -7..7, the coli_pack_int4 format);
 *                the shared expert is blob E. One blob is the unit the engine
 *                reads with a single pread (devtrends.cc page, section
 *                引擎是如何工作的).
 *  experts_scale E + n_shared blobs of 2*I + H fp32 row scales:
 *                [gate I | up I | down H].
 */
typedef struct coli_moe_weights {
    coli_moe_cfg cfg;
    const float* w_router;
    const float* bias;
    const uint8_t* experts_q;
    const float* experts_scale;
} coli_moe_weights;

/* Where the intermediates of one forward live inside the workspace (byte
 * offsets from ws). Slot s indexes the (token, expert) assignments in
 * expert-bucketed order; tokens of one expert occupy consecutive slots in
 * ascending token order, experts in ascending id order, the shared expert last.
 *   qx     [T, H] int8 Q8_0 codes of x, each group of 8 stored as
 *          (e0,e2,e4,e6,e1,e3,e5,e7)
 *   dx     [T, H/32] fp32 block scales of x
 *   logits [T, E] fp64 router logits
 *   topk_idx [T, K] int32, topk_w [T, K] fp32
 *   counts [E + S] int32 tokens per expert, offs [E + S + 1] int32 first slot
 *   slot_of [T, K + S] int32 slot of (t, k) (k == K: shared expert)
 *   slot_tok [T*(K+S)] int32 token of each slot
 *   qh     [T*(K+S), I] int8 Q8_0 codes of the SwiGLU output h (same 8-group order)
 *   dh     [T*(K+S), I/32] fp32
 *   ye     [T*(K+S), H] fp32 expert outputs (only written when T is above the
 *          decode path's token limit)
 *   tap    [T*(K+S), tap_rows, H/32] int32 gate-row block dots of rows
 *          r = i * tap_stride (COLI_FWD_DEBUG_TAPS only)
 */
typedef struct coli_moe_ws_layout {
    size_t total;
    size_t qx, dx, logits, topk_idx, topk_w, counts, offs, slot_of, slot_tok, qh, dh, ye, tap;
    int64_t n_slots, tap_rows, tap_stride;
    size_t reserved[4];
} coli_moe_ws_layout;

/* Message for a return code (static string, never NULL). */
COLI_API const char* coli_strerror(int code);

/* Pack an fp32 matrix [rows, cols] into symmetric b-bit codes, b = 4 as
 * coli_pack_int4 below, or its int8 / int2 siblings (Colibri page, feature
 * list 关键特性: quantisation kernels for int8, int4 and int2): per row
 * s = fp32(max|w|/Q), Q = 2^(b-1) - 1 (127, 7, 1); code = clamp(rint(w/s),
 * -Q, Q) with round-half-to-even and IEEE division; s == 0 gives code 0;
 * codes are b-bit two's complement packed little end first (element j of a
 * row in byte j b / 8 at bit (j b) % 8).
 *   w [rows, cols] fp32 (in), q [rows, cols b/8] u8 (out), scale [rows] fp32
 *   (out). cols must be a positive multiple of 32, rows >= 0 (0: no-op), b
 *   in {2, 4, 8} (else COLI_E_INVAL). Bit-exact with the plain definition. */
COLI_API int coli_pack_weights(const float* w, int64_t rows, int64_t cols, int bits, uint8_t* q,
                               float* scale, void* stream);

/* Pack an fp32 matrix [rows, cols] into symmetric int4 (wmrh.cn page,
 * section 量化流程): per row s = fp32(max|w|/7); code = clamp(rint(w/s), -7, 7)
 * with round-half-to-even and IEEE division; s == 0 gives code 0; byte j of
 * a row = code(2j) & 0xF | (code(2j+1) & 0xF) << 4.
 *   w [rows, cols] fp32 (in), q [rows, cols/2] u8 (out), scale [rows] fp32 (out).
 * cols must be a positive multiple of 32, rows >= 0 (0: no-op).
 * Result is bit-exact with the plain definition above. */
COLI_API int coli_pack_int4(const float* w, int64_t rows, int64_t cols, uint8_t* q,
                            float* scale, void* stream);

/* FP8 front-end of coli_pack_int4 (wmrh.cn page, section 量化流程: the
 * source weights are FP8 e4m3 with one scale per 128 x 128 block — the
 * weight_block_size of the quantization_config shown there — converted to F32
 * and then packed to int4):
 *   w[r][c] = fp32(e4m3(q8[r][c]) * block_scale[r/128][c/128]), one rounding;
 *   e4m3 = 1 sign, 4 exponent bits (bias 7), 3 mantissa bits, exponent 0
 *   subnormal (m * 2^-9), no infinities; the NaN code S.1111.111 converts
 *   to 0; then the rows are packed exactly as by coli_pack_int4.
 *   q8 [rows, cols] u8 codes, block_scale [ceil(rows/128), ceil(cols/128)]
 *   fp32 (in); q [rows, cols/2] u8, scale [rows] fp32 (out). cols must be a
 *   positive multiple of 32, rows >= 0 (0: no-op). Bit-exact with the plain
 *   definition. */
COLI_API int coli_pack_fp8_int4(const uint8_t* q8, const float* block_scale, int64_t rows,
                                int64_t cols, uint8_t* q, float* scale, void* stream);

/* Q8_0 quantisation of activations ("Colibri：在笔记本上跑744B参数的AI模型",
 * 关键特性: Q8_0-style int8 activations): per block of 32 consecutive
 * elements d = fp32(max|x|/127), q = clamp(rint(x/d), -127, 127), d == 0
 * gives q = 0.
 *   x [n_tok, dim] fp32 (in), q [n_tok, dim] int8 (out, plain element order),
 *   d [n_tok, dim/32] fp32 (out). dim must be a positive multiple of 32. */
COLI_API int coli_quant_q8(const float* x, int64_t n_tok, int64_t dim, int8_t* q, float* d,
                           void* stream);

/* Bytes of workspace that coli_moe_route / coli_moe_forward need for up to
 * max_tok tokens with the given flags; 0 if cfg is invalid. */
COLI_API size_t coli_moe_workspace_bytes(const coli_moe_cfg* cfg, int64_t max_tok,
                                         uint32_t flags);

/* Offsets of the intermediates inside a workspace for n_tok tokens. */
COLI_API int coli_moe_workspace_layout(const coli_moe_cfg* cfg, int64_t n_tok, uint32_t flags,
                                       coli_moe_ws_layout* out);

/* Sigmoid router with correction bias and top-k (wmrh.cn page, sections
 * MoE的工作原理 and 路由策略定制; Colibri page, 关键特性):
 *   l = x . w_router^T (accumulated in fp64), s = 1/(1+exp(-l)), c = s + bias;
 *   the K largest c in descending order, ties to the lower expert index;
 *   with cfg->n_group > 1 (the topk_method knob, read as DeepSeek-V3's
 *   group-limited selection) only the experts of the cfg->topk_group groups
 *   with the largest group scores compete, a group's score being the sum of
 *   its two largest c (ties to the lower group index);
 *   w_k = s[e_k], divided by sum_k s[e_k] when cfg->norm_topk, times
 *   cfg->routed_scale, rounded to fp32.
 *   x [n_tok, H] fp32, w_router [E, H], bias [E] (in); topk_idx [n_tok, K]
 *   int32 and topk_w [n_tok, K] fp32 (out); ws: workspace of at least
 *   coli_moe_workspace_bytes(cfg, n_tok, 0) bytes, overwritten. The
 *   selection needs every expert's logit of a token at once, so the logits
 *   l [n_tok, E] (fp64) pass through ws between the GEMV/GEMM and the top-k
 *   launch; above 8 tokens the router GEMM also cuts H into up to 16 slices
 *   whose fp64 partial sums [slices, n_tok, E] live in ws until a second
 *   launch adds them in slice order (a fixed order, so results do not depend
 *   on scheduling). Nothing in ws is a result.
 * Errors: COLI_E_INVAL (null pointer, bad cfg, n_tok < 0), COLI_E_ALIGN,
 *   COLI_E_WORKSPACE (ws_bytes too small), COLI_E_UNSUPPORTED (n_tok > 2^20),
 *   COLI_E_HIP (a launch failed); nothing is launched on the other errors.
 *   n_tok == 0 is a no-op. */
COLI_API int coli_moe_route(const float* x, const float* w_router, const float* bias,
                            int64_t n_tok, const coli_moe_cfg* cfg, int32_t* topk_idx,
                            float* topk_w, void* ws, size_t ws_bytes, void* stream);

/* The whole layer on n_tok tokens (pages as above):
 *   route (as coli_moe_route); q_x, d_x = Q8_0(x);
 *   for every selected expert e of token t and for the shared expert:
 *     g_r = fp32(s_gate[r] * sum_b d_x,b * I_b) with I_b the exact int32 dot
 *           of block b of gate row r with q_x (sum in fp64), u_r likewise,
 *     h_r = fp32(silu(g_r) * u_r), silu(z) = z/(1+exp(-z)) in fp64,
 *     q_h, d_h = Q8_0(h),
 *     y_e,c = fp32(s_down[c] * sum_b d_h,b * I_b(down row c));
 *   y_t = fp32(sum_k w_k * y_e_k + y_shared) in fp64 (shared weight 1).
 * Tokens that share an expert read its weights once (bucketing).
 *   w: layer weights; x [n_tok, H] fp32 (the normalised layer input);
 *   y [n_tok, H] fp32 (out; with COLI_FWD_ACCUM y = y + fp32(layer)).
 *   ws/ws_bytes: workspace (see coli_moe_workspace_bytes), overwritten.
 * n_tok == 0 is a no-op. */
COLI_API int coli_moe_forward(const coli_moe_weights* w, const float* x, int64_t n_tok,
                              float* y, void* ws, size_t ws_bytes, uint32_t flags,
                              void* stream);

/* As coli_moe_forward, and additionally times each kernel launch of the
 * forward: launch j is enqueued with hipExtLaunchKernel and its own start and
 * stop events, events[2j] and events[2j + 1] (hipEvent_t passed as void*,
 * created with timing), which the packet processor stamps at the kernel's
 * begin and end, so that hipEventElapsedTime gives the kernel's duration
 * without the gaps between launches. names[j] (the caller's array of at least
 * n_events / 2 entries, or null) receives a static name of launch j. Returns
 * the number of launches in *n_used; launches past n_events / 2 run untimed.
 * Results are identical to coli_moe_forward. */
COLI_API int coli_moe_forward_profiled(const coli_moe_weights* w, const float* x,
                                       int64_t n_tok, float* y, void* ws, size_t ws_bytes,
                                       uint32_t flags, void* stream, void* const* events,
                                       int n_events, int* n_used, const char** names);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * coli_moe_forward without a workspace argument. Its intermediates live in a
 * fixed scratch array of COLI_STATIC_SCRATCH_BYTES that the library holds on
 * every GPU it runs on until the process ends; the call itself allocates
 * nothing. Results are identical to coli_moe_forward (same kernels).
 *   w, x, n_tok, y, flags, stream: as coli_moe_forward.
 * Errors: as coli_moe_forward, and COLI_E_WORKSPACE when the intermediates of
 * n_tok tokens with these flags need more than the scratch array holds (for
 * the GLM-5.2 layer shape about 120 tokens without COLI_FWD_DEBUG_TAPS;
 * coli_moe_workspace_bytes gives the need); COLI_E_HIP when the array's
 * address cannot be obtained.
 * All calls on one GPU share its array, and each call overwrites it: calls
 * that overlap in time on one GPU (different streams, different threads
 * without ordering) race and give wrong results; order them, e.g. on one
 * stream. */
#define COLI_STATIC_SCRATCH_BYTES ((size_t)32 << 20)
COLI_API int coli_moe_forward_static(const coli_moe_weights* w, const float* x, int64_t n_tok,
                                     float* y, uint32_t flags, void* stream);

/* RMSNorm with unit gain (the pre-norm between stacked layers):
 *   out = fp32(x / sqrt(mean(x^2) + eps)), computed in fp64.
 *   x [n_tok, dim] fp32 (in), out [n_tok, dim] fp32 (out, may alias x). */
COLI_API int coli_rmsnorm(const float* x, int64_t n_tok, int64_t dim, float eps, float* out,
                          void* stream);

/* Measurement helper, not a step of the layer: reads `bytes` of device memory
 * at src once with streaming (nontemporal) 16-byte loads, the pattern of the
 * layer's weight streams, so that timing it gives the HBM read ceiling the
 * expert-weight rates are quoted against beside the published peak. It has
 * no counterpart in the pages (their engine reads experts from disk).
 *   src   device pointer, 16-byte aligned; bytes a multiple of 16 (0: no-op)
 *   sink  device uint32 (4-byte aligned): an XOR checksum of the data is
 *         folded into it atomically (its old value is kept in the XOR); it
 *         exists so that no load is dead code
 * Errors: COLI_E_INVAL (bytes < 0 or not a multiple of 16, null pointers),
 * COLI_E_ALIGN. Enqueues one kernel on `stream`. */
COLI_API int coli_stream_read(const void* src, int64_t bytes, uint32_t* sink, void* stream);

/* Measurement helper, not a step of the layer: issue rates of the int8 MFMA
 * forms and of the exact per-block epilogue the grouped kernels apply to
 * every MFMA result (one scaled add per row, token and 32-block, fixed by the
 * Q8_0 format). Enqueues n_workgroups workgroups of 4 waves; every wave runs
 * `iters` iterations of one instruction mix and stores the shader-clock
 * cycles its loop took. kind: 0 = 8 v_mfma_i32_16x16x32_i8, 1 = 8
 * v_mfma_i32_16x16x64_i8, 2 = 4 v_mfma_i32_32x32x32_i8, 3 = 16
 * v_mad_i64_i32, 4 = 16 (v_cvt_f64_i32 + v_fma_f64), 5 = 2 32x32x32 each
 * followed by the int64 epilogue of its 16 results, 6 = the same with the
 * fp64 epilogue, 7 = 4 16x16x32 with the int64 epilogue of their 4 results.
 *   cycles: device int64 [4 n_workgroups + 1] (out; entry 4 w + v = wave v of
 *   workgroup w; the last entry is scratch). Errors: COLI_E_INVAL (kind
 *   outside 0..7, n_workgroups outside 1..2^20, iters <= 0, null pointer),
 *   COLI_E_ALIGN (cycles not 8-byte aligned). */
COLI_API int coli_mfma_probe(int kind, int64_t n_workgroups, int iters, int64_t* cycles,
                             void* stream);

#ifdef __cplusplus
}
#endif

#endif /* COLI_MOE_H */
