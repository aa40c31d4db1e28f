// Grouped int8 MFMA kernels for many tokens on the full-rate K=32 form
// (v_mfma_i32_32x32x32_i8: its K extent is exactly one Q8_0 block, and on
// gfx950 it issues at the full int8 rate, twice the 16x16x32 form).
//
// Work item = (expert, first slot, n <= 32 or 64 of its tokens), as for the
// 16x16 kernels (k_prefill.h). A gate/up workgroup takes one item and 128
// h-rows; wave w owns rows 32w .. 32w + 31 as two 32-row MFMA tiles, its gate
// rows and the matching up rows, so SwiGLU needs no exchange. (The library
// runs it for 64-token items; the down projection stays on the 16x16 kernel,
// which was faster at this K extent.)
// Per 32-wide block b and 32-token group, each wave issues one
//   D = v_mfma_i32_32x32x32_i8(A = 32 weight rows, B = 32 tokens)
// per tile; D holds 32 x 32 exact block dots (times the weight width's code
// multiplier), and the epilogue adds m[token, b] * D into int64 accumulators
// (exact; the integer block scales of k_scale_int) or d[token, b] * D into
// fp64 ones (rows without integer scales). Every lane's 16 results share one
// token (its column), so the epilogue takes one scale per lane and block.
//
// Operand layout (checked on the device): lane l holds row (A) / column (B)
// l % 32 and 16 k values of the block, the half g = l / 32 (A and B take the
// same half, so the product is the block dot); result register i of lane l
// is row 8 (i / 4) + 4 (l / 32) + i % 4, column l % 32. Activations are
// stored per block in the weight width's element order (k_prefill.h), so the
// B operand is the 16 bytes 16 g .. 16 g + 15 of the token's block and the A
// operand their weights: int4 two packed dwords expanded with the x16 nibble
// trick, int8 16 plain bytes, int2 one dword expanded x64.
//
// Staging as in k_prefill.h: direct-to-LDS loads into a three-slot ring of
// stages of CH blocks (CH = 16 / BITS, so a row's stage is 64 bytes at every
// width), per-row XOR swizzle of the 16-byte pieces, explicit vmcnt waits and
// one barrier per stage.
#pragma once

#include "k_prefill.h"

namespace pf {

constexpr int kRows32 = 128;    // gate/up: h rows per workgroup (32 per wave)

typedef int v16i __attribute__((ext_vector_type(16)));

template <int BITS, int KT>
struct Geo32 {
    static constexpr int CH = 16 / BITS;                 // 32-blocks per stage
    static constexpr int RB = 64;                        // bytes of a row per stage
    static constexpr int NPC = 4;                        // 16-byte pieces per row
    static constexpr int KS = 4;                         // rows per 256-byte bank period
    static constexpr int RW = 64;                        // staged weight rows per wave
    static constexpr int WBYTES = RW * RB;               // 4 KB per wave
    static constexpr int WINSTR = WBYTES / 1024;         // weight loads per wave and stage
    static constexpr int RPI = 1024 / RB;                // rows per load instruction (16)
    static constexpr int ARB = CH * 32;                  // activation bytes per token
    static constexpr int ANPC = ARB / 16;
    static constexpr int AKS = ARB >= 256 ? 1 : 256 / ARB;
    static constexpr int ARPI = 1024 / ARB;              // token rows per load instruction
    static constexpr int AINSTR = KT * ARB / 1024;       // activation loads per stage
    static constexpr int AIW = (AINSTR + 3) / 4;         // ... per wave (the first waves)
    static constexpr int TPI = 64 / CH;                  // tokens per scale load instruction
    static constexpr int SINSTR = KT / TPI;              // scale loads per stage
    static constexpr int SIW = (SINSTR + 3) / 4;         // ... per wave (the first waves)
    static constexpr int A_OFF = 4 * WBYTES;
    static constexpr int D_OFF = A_OFF + KT * ARB;
    static constexpr int SLOT = (D_OFF + KT * CH * 4 + 255) & ~255;
    static constexpr int NG = KT / 32;                   // 32-token groups of an item
    static constexpr int Scale = BITS == 4 ? 16 : BITS == 2 ? 64 : 1;  // code multiplier
    static constexpr double InvScale = 1.0 / Scale;                    // exact
    static constexpr int Layout = BITS == 4 ? 1 : BITS == 2 ? 2 : 0;   // activation order
    static_assert(KT == 32 || KT == 64, "item size");
    static_assert(AINSTR % AIW == 0 && SINSTR % SIW == 0, "load split over waves");
    // 32 rows / tokens are whole swizzle-key periods: tile 1 and token group 1
    // sit at immediate offsets with the same keys
    static_assert(32 % (NPC * KS) == 0 && 32 % (ANPC * AKS) == 0, "swizzle keys");
};

// A operand (16 k values of one row) from the staged block at p: int4 two
// packed dwords, int8 16 bytes, int2 one dword.
template <int BITS>
__device__ __forceinline__ v4i a_op32(const uint8_t* p) {
    if constexpr (BITS == 4) {
        typedef unsigned v2u __attribute__((ext_vector_type(2)));
        const v2u x = *reinterpret_cast<const v2u*>(p);
        return v4i{nib_lo16(x.x), nib_hi16(x.x), nib_lo16(x.y), nib_hi16(x.y)};
    } else if constexpr (BITS == 8) {
        return *reinterpret_cast<const v4i*>(p);
    } else {
        constexpr uint32_t M = 0xC0C0C0C0u;
        const uint32_t x = lds_u32(p);
        return v4i{(int)((x << 6) & M), (int)((x << 4) & M), (int)((x << 2) & M), (int)(x & M)};
    }
}

// Per-lane load plan of one wave for a stage (see k_prefill.h Plan): WINSTR
// weight loads (rows 16 i + lane / 4 of the wave's 64; rows 0..31 tile 0,
// 32..63 tile 1), AIW activation loads and SIW scale loads for the waves that
// have them. With 4-block stages and a block count that is a multiple of 4,
// wave 0 loads the stage's scales with one 16-byte load per token instead
// (lane j: token j's four scales, at the same LDS bytes).
template <int BITS, int KT>
struct Plan32 {
    typedef Geo32<BITS, KT> G;
    const uint8_t* wrow[G::WINSTR];
    int wpo[G::WINSTR];
    int rowb;
    const int8_t* arow[G::AIW];
    int apo[G::AIW];
    int arowb;
    const uint8_t* srow[G::SIW];
    int sbk[G::SIW];
    int NB;
    int wave;
    bool act, scl;   // this wave loads activation rows / block scales
    bool sx4;        // ... scales with one 16-byte load per token

    __device__ __forceinline__ void init(const uint8_t* const (&tile)[2], const int (&nrow)[2],
                                         int64_t rowb_, const int8_t* act_, int64_t arowb_,
                                         const int32_t* rows_of, int n, const void* scales,
                                         int NB_) {
        const int lane = threadIdx.x & 63;
        wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        rowb = (int)rowb_;
        arowb = (int)arowb_;
        NB = NB_;
#pragma unroll
        for (int i = 0; i < G::WINSTR; ++i) {
            const int r = i * G::RPI + lane / G::NPC;  // staged row 0..63
            const int t = r >> 5, rr = min(r & 31, nrow[t] - 1);
            const int piece = (lane % G::NPC) ^ wkey(r, G::KS, G::NPC);
            wrow[i] = tile[t] + (int64_t)rr * rowb_;
            wpo[i] = piece * 16;
        }
        act = wave * G::AIW < G::AINSTR;
#pragma unroll
        for (int i = 0; i < G::AIW; ++i) {
            const int j = (wave * G::AIW + i) * G::ARPI + lane / G::ANPC;  // token row
            const int piece = (lane % G::ANPC) ^ wkey(j, G::AKS, G::ANPC);
            arow[i] = act_ + (int64_t)rows_of[min(j, n - 1)] * arowb_;
            apo[i] = piece * 16;
        }
        sx4 = G::CH == 4 && NB_ % 4 == 0;
        if (sx4) {
            static_assert(G::CH != 4 || (G::SIW == 1 && KT <= 64), "one 16-byte scale load");
            scl = wave == 0;
            sbk[0] = 0;
            srow[0] = static_cast<const uint8_t*>(scales) +
                      (int64_t)rows_of[min(lane, n - 1)] * NB_ * 4;
            return;
        }
        scl = wave * G::SIW < G::SINSTR;
#pragma unroll
        for (int i = 0; i < G::SIW; ++i) {
            const int js = min((wave * G::SIW + i) * G::TPI, KT - G::TPI) + lane / G::CH;
            sbk[i] = lane % G::CH;
            srow[i] = static_cast<const uint8_t*>(scales) + (int64_t)rows_of[min(js, n - 1)] * NB_ * 4;
        }
    }
    // Issues the stage's loads into the slot at LDS address `slot`; pieces
    // past a row's end are clamped to its last piece, their blocks read scale 0.
    __device__ __forceinline__ void issue(int c, uint32_t slot) const {
        const uint32_t wdst = slot + wave * G::WBYTES;
#pragma unroll
        for (int i = 0; i < G::WINSTR; ++i)
            dma_b128(wrow[i] + min(c * G::RB + wpo[i], rowb - 16), wdst + i * 1024);
        if (act) {
            const uint32_t adst = slot + G::A_OFF + wave * G::AIW * 1024;
#pragma unroll
            for (int i = 0; i < G::AIW; ++i)
                dma_b128(arow[i] + min(c * G::ARB + apo[i], arowb - 16), adst + i * 1024);
        }
        if (scl && sx4) {
            if ((int)(threadIdx.x & 63) < KT) dma_b128(srow[0] + 16 * c, slot + G::D_OFF);
        } else if (scl) {
#pragma unroll
            for (int i = 0; i < G::SIW; ++i) {
                const int b = c * G::CH + sbk[i];
                dma_b32(b < NB ? static_cast<const void*>(srow[i] + 4 * b) : &kZeroScale,
                        slot + G::D_OFF + (wave * G::SIW + i) * 256);
            }
        }
    }
};

// Waits until this wave's loads of the stage about to be used are in: those
// of the next stage (LD of them, fewer for waves without activation or scale
// loads) may still be in flight, unless this is the last stage (all).
template <int BITS, int KT, bool TAP>
__device__ __forceinline__ void wait_stage32(const Plan32<BITS, KT>& pl, bool last) {
    typedef Geo32<BITS, KT> G;
    if (last || TAP) {
        wait_vm<0, false>();
        return;
    }
    constexpr int W = G::WINSTR, A = G::AIW, S = G::SIW;
    if (pl.act && pl.scl) wait_vm<W + A + S, false>();
    else if (pl.act) wait_vm<W + A, false>();
    else if (pl.scl) wait_vm<W + S, false>();
    else wait_vm<W, false>();
}

// K loop: acc[t][g][i] = sum over blocks of d[token] * D(tile t, group g)[i]
// (see k_prefill.h mm_loop; INT: exact int64 sums over integer scales,
// scaled by 2^etok[g] and rounded once at the end). TAP records the block dots
// of tile 0 for sampled rows (row tap_r0 + 8 (i / 4) + 4 g + i % 4).
template <int BITS, int KT, int NG, bool TAP, bool INT>
__device__ __forceinline__ void mm_loop32(const Plan32<BITS, KT>& pl, uint8_t* smem,
                                          double (&acc)[2][KT / 32][16],
                                          const int (&etok)[KT / 32], int nst, const PfArgs& a,
                                          int tap_r0, int s0, int n) {
    typedef Geo32<BITS, KT> G;
    const int lane = threadIdx.x & 63;
    const int lr = lane & 31, q = lane >> 5;
    long acci[2][NG][16];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
#pragma unroll
            for (int g = 0; g < KT / 32; ++g) acc[t][g][i] = 0.0;
#pragma unroll
            for (int g = 0; g < NG; ++g) acci[t][g][i] = 0;
        }
    // slot-relative lane bases of the operand reads; the piece index of a
    // block is XORed into the piece bits (the other terms have them clear)
    const int r0k = wkey(lr, G::KS, G::NPC), a0k = wkey(lr, G::AKS, G::ANPC);
    const int wbase = pl.wave * G::WBYTES + lr * G::RB;
    const int abase = G::A_OFF + lr * G::ARB;
    const int dbase = G::D_OFF + lr * G::CH * 4;
    int wo[G::CH], ao[G::CH], dof[G::CH];
#pragma unroll
    for (int bi = 0; bi < G::CH; ++bi) {
        // weights: int4 a block is one piece, lanes of half q read its bytes
        // 8q..8q+7; int8 a block is two pieces, half q reads piece 2 bi + q;
        // int2 a block is half a piece, half q reads its dword q
        int piece, byte;
        if (BITS == 4) { piece = bi; byte = 8 * q; }
        else if (BITS == 8) { piece = 2 * bi + q; byte = 0; }
        else { piece = bi >> 1; byte = 8 * (bi & 1) + 4 * q; }
        wo[bi] = wbase + ((piece ^ r0k) << 4) + byte;
        ao[bi] = abase + (((2 * bi + q) ^ a0k) << 4);
        dof[bi] = dbase + 4 * bi;
    }
    const v16i zero = {};
    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void*)smem;

    pl.issue(0, lds0);
    if (nst > 1) pl.issue(1, lds0 + G::SLOT);
#pragma unroll 1
    for (int cb = 0; cb < nst; cb += kSlots) {
#pragma unroll
        for (int sl = 0; sl < kSlots; ++sl) {
            const int c = cb + sl;
            if (c >= nst) break;
            const uint8_t* cur = smem + sl * G::SLOT;
            wait_stage32<BITS, KT, TAP>(pl, c + 1 >= nst);
            stage_barrier();  // every wave's loads of stage c are in; slot c - 1 is free
            if (c + 2 < nst) pl.issue(c + 2, lds0 + ((sl + 2) % kSlots) * G::SLOT);
#pragma unroll
            for (int bi = 0; bi < G::CH; ++bi) {
                const v4i a0 = a_op32<BITS>(cur + wo[bi]);
                const v4i a1 = a_op32<BITS>(cur + wo[bi] + 32 * G::RB);
#pragma unroll
                for (int g = 0; g < NG; ++g) {
                    const v4i bv = *reinterpret_cast<const v4i*>(cur + ao[bi] + g * 32 * G::ARB);
                    const uint8_t* dp = cur + dof[bi] + g * 32 * G::CH * 4;
                    const v16i c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, bv, zero, 0, 0, 0);
                    const v16i c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, bv, zero, 0, 0, 0);
                    if constexpr (INT) {
                        const long dm = *reinterpret_cast<const int*>(dp);
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            acci[0][g][i] += dm * (long)c0[i];
                            acci[1][g][i] += dm * (long)c1[i];
                            asm volatile("" : "+v"(acci[0][g][i]), "+v"(acci[1][g][i]));
                        }
                    } else {
                        const double dd = (double)*reinterpret_cast<const float*>(dp);
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            acc[0][g][i] += dd * (double)c0[i];
                            acc[1][g][i] += dd * (double)c1[i];
                            asm volatile("" : "+v"(acc[0][g][i]), "+v"(acc[1][g][i]));
                        }
                    }
                    if (TAP) {
                        const int b = c * G::CH + bi, j = 32 * g + lr, BH = pl.NB;
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            const int r = tap_r0 + 8 * (i >> 2) + 4 * q + (i & 3);
                            if (j < n && b < BH && (r % a.tap_stride) == 0)
                                a.tap[((int64_t)(s0 + j) * a.tap_rows + r / a.tap_stride) * BH +
                                      b] = c0[i] / G::Scale;
                        }
                    }
                }
            }
        }
    }
    if constexpr (INT) {
        // one rounding of the exact sum, then an exact power-of-two scale
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int g = 0; g < NG; ++g)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[t][g][i] = ldexp((double)acci[t][g][i], etok[g]);
    }
}

// Gate/up + SwiGLU + Q8_0(h) for one item and 128 intermediate rows.
template <int BITS, int KT, bool TAP>
__global__ __launch_bounds__(256) void k_pf32_gateup(PfArgs a) {
    typedef Geo32<BITS, KT> G;
    constexpr int NGM = KT / 32;
    __shared__ __align__(1024) uint8_t smem[kSlots * G::SLOT];
    static_assert(kSlots * G::SLOT >= KT * (kRows32 + 1) * 4, "h reuses the ring");
    const int nrt = a.I / kRows32;
    int it, rt;
    if (!work_of<KT>(a, nrt, it, rt)) return;
    const int e = a.item_e[it], s0 = a.item_s0[it], n = a.item_n[it];
    const int H = a.H, I = a.I, BH = H >> 5;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lr = lane & 31, q = lane >> 5;
    const int64_t rowb = (int64_t)H * BITS / 8;
    const uint8_t* gate = a.eq + (int64_t)e * a.blob_q;
    const uint8_t* up = gate + (int64_t)I * rowb;
    const int r0 = rt * kRows32 + wave * 32;
    const int nst = (BH + G::CH - 1) / G::CH;

    const uint8_t* const tiles[2] = {gate + (int64_t)r0 * rowb, up + (int64_t)r0 * rowb};
    const int nrow[2] = {32, 32};
    const int32_t* rows_of = a.slot_tok + s0;  // token of each of the item's slots
    // integer scales unless the call has none (few tokens) or a token of the
    // item has none
    bool wide = a.ex == nullptr;
    int etok[NGM] = {};
    if (!wide) {
        const int tv = rows_of[min((int)threadIdx.x, n - 1)];
        wide = __syncthreads_or((int)threadIdx.x < n && a.ex[tv] == kWideRow);
#pragma unroll
        for (int g = 0; g < NGM; ++g) etok[g] = a.ex[rows_of[min(32 * g + lr, n - 1)]];
    }
    double acc[2][NGM][16];
    auto run = [&](auto ng, auto in) {
        constexpr int NG = decltype(ng)::value;
        constexpr bool INT = decltype(in)::value;
        Plan32<BITS, KT> pl;
        pl.init(tiles, nrow, rowb, a.qx, H, rows_of, n,
                INT ? static_cast<const void*>(a.mx) : static_cast<const void*>(a.dx), BH);
        mm_loop32<BITS, KT, NG, TAP, INT>(pl, smem, acc, etok, nst, a, r0, s0, n);
    };
    typedef std::integral_constant<int, 1> G1;
    typedef std::integral_constant<int, 2> G2;
    typedef std::integral_constant<bool, true> Int;
    typedef std::integral_constant<bool, false> F64;
    if (!wide) {
        if (KT == 32 || n <= 32) run(G1{}, Int{});
        else if constexpr (KT == 64) run(G2{}, Int{});
    } else {
        if (KT == 32 || n <= 32) run(G1{}, F64{});
        else if constexpr (KT == 64) run(G2{}, F64{});
    }
    __syncthreads();  // the ring is reused for h below
    float (*hbuf)[kRows32 + 1] = reinterpret_cast<float (*)[kRows32 + 1]>(smem);

    // SwiGLU (lane: token 32 g + lr, rows 8 (i / 4) + 4 q + i % 4 of the wave's 32)
    const float* gs = a.es + (int64_t)e * a.blob_s;
    const float* us = gs + I;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int rl = 8 * (i >> 2) + 4 * q + (i & 3);
        const float gsr = gs[r0 + rl], usr = us[r0 + rl];
#pragma unroll
        for (int g = 0; g < NGM; ++g) {
            if (32 * g >= n) continue;
            // the sums carry the multiplier of the weight codes: scale it away (exact)
            const float gv = (float)((double)gsr * (acc[0][g][i] * G::InvScale));
            const float uv = (float)((double)usr * (acc[1][g][i] * G::InvScale));
            hbuf[32 * g + lr][wave * 32 + rl] = swiglu_f32(gv, uv);
        }
    }
    __syncthreads();
    // Q8_0 over each 32 consecutive h rows of a token: 4 blocks per token
    for (int v = threadIdx.x; v < 4 * n; v += 256) {
        const int j = v >> 2, kb = v & 3;
        const float* hv = &hbuf[j][32 * kb];
        float amax = 0.0f;
#pragma unroll
        for (int k = 0; k < 32; ++k) amax = fmaxf(amax, fabsf(hv[k]));
        const float d = amax / 127.0f;
        uint32_t w[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            w[i] = pack4_i8(q8_code(hv[act_elem<G::Layout>(4 * i)], d),
                            q8_code(hv[act_elem<G::Layout>(4 * i + 1)], d),
                            q8_code(hv[act_elem<G::Layout>(4 * i + 2)], d),
                            q8_code(hv[act_elem<G::Layout>(4 * i + 3)], d));
        typedef unsigned v4u __attribute__((ext_vector_type(4)));
        v4u* o = reinterpret_cast<v4u*>(a.qh + (int64_t)(s0 + j) * I + rt * kRows32 + 32 * kb);
        o[0] = v4u{w[0], w[1], w[2], w[3]};
        o[1] = v4u{w[4], w[5], w[6], w[7]};
        a.dh[(int64_t)(s0 + j) * (I >> 5) + rt * 4 + kb] = d;
    }
}

}  // namespace pf
