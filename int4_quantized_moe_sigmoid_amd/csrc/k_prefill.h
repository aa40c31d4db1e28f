// Grouped int8 MFMA kernels for many tokens (prefill, stacked layers).
//
// Work item = (expert, first slot, n <= 32 or 64 of its tokens). A workgroup takes
// one item and a tile of output rows; each wave owns two 16-row tiles (gate/up:
// 16 gate rows and the matching 16 up rows, so SwiGLU needs no exchange; down:
// 32 consecutive output rows). Per 32-wide block b every wave issues
//   D = v_mfma_i32_16x16x32_i8(A = 16 weight rows, B = 16 tokens)
// whose K extent is exactly one Q8_0 block, so D holds 16 x 16 exact block
// dots (x16, see below); the fp64 epilogue adds d_b * D into per-lane fp64
// accumulators, which is the numerics of the plain definition (exact block
// dots, fp64 sum of scaled dots) regardless of tiling.
//
// MFMA operand layout (16x16x32 int8, checked on the device): lane l holds
// row (A) / column (B) l % 16 and k = 8 (l / 16) + i, i = 0..7; result
// register i of lane l is row 4 (l / 16) + i, column l % 16. A dword of
// packed int4 codes (8 consecutive elements) becomes an A operand with the
// x16 nibble trick: (x << 4) & 0xF0F0F0F0 holds 16 * the even elements and
// x & 0xF0F0F0F0 16 * the odd ones, i.e. the element order (e0 e2 e4 e6 e1
// e3 e5 e7) in which activations are stored, so B is 8 plain bytes of the
// activation row.
//
// The int8 and int2 weight formats use the same kernels: an int8 row is its
// own A operand (8 plain bytes, activations in natural order); for int2 a
// dword holds 16 codes and (x << s) & 0xC0C0C0C0, s = 6, 4, 2, 0, holds 64 *
// the elements 4j + (6 - s) / 2 of bytes j, i.e. the 16-element order (e0 e4
// e8 e12 e1 e5 e9 e13 e2 e6 e10 e14 e3 e7 e11 e15) of the activations. The
// x16 / x64 leave the fp64 epilogue as an exact power-of-two scale.
//
// Staging: the K range is cut into stages of CH blocks. Weight rows, the
// item's activation rows and their block scales reach LDS with direct-to-LDS
// loads (global_load_lds_dwordx4 / _dword: lane l of a wave writes 16 / 4
// bytes at a wave-uniform LDS base + 16 l / 4 l), so no registers hold data
// in flight. A ring of three LDS slots keeps two stages loading while the
// third is computed, with one workgroup barrier per stage; each wave waits
// only for its own loads of the stage it is about to use (vmcnt), and the
// barrier makes every wave's loads visible. Inside a slot the 16-byte pieces
// of a row are stored at position piece ^ key(row) (an XOR swizzle chosen per
// row so that the MFMA operand reads of 16 rows / 16 tokens hit distinct LDS
// banks); the loads scatter global pieces accordingly.
#pragma once

#include <type_traits>

#include "coli_common.h"
#include "coli_args.h"

namespace pf {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kSlots = 3;     // LDS ring: one stage computed, two loading

// Work of a gate/up workgroup: item `it` and row tile `rt` (nrt tiles per
// item). Workgroups go to the 8 XCDs in turn (block b to XCD b % 8, each XCD
// taking its blocks in order), and each XCD has its own L2. The work list --
// experts in ascending order, each one's items interleaved per row tile
// ((i0, r0), (i1, r0), .., (i0, r1), ..) -- is cut into 8 equal runs, run x
// going to XCD x, so the items of one expert ask for each weight tile at
// about the same time on one XCD and one fill of its L2 serves them (the
// expert's weights are fetched about once however many items it has). The
// grid is a multiple of 8 of at least items x nrt blocks; false: no work for
// this block.
template <int KT>
__device__ __forceinline__ bool work_of(const PfArgs& a, int nrt, int& it, int& rt) {
    const int N = *a.n_items * nrt;
    const int L = (N + 7) >> 3;
    const int l = blockIdx.x >> 3;
    const int p = (blockIdx.x & 7) * L + l;
    if (l >= L || p >= N) return false;
    // expert e owns positions nrt io .. nrt (io + m) - 1 of the list (io its
    // first item, m its item count), so p / nrt is one of its items
    const int i0 = p / nrt;
    const int e = a.item_e[i0];
    const int io = i0 - (a.item_s0[i0] - a.offs[e]) / KT;
    const int m = (a.offs[e + 1] - a.offs[e] + KT - 1) / KT;
    const int q = p - nrt * io;
    rt = q / m;
    it = io + (q - rt * m);
    return true;
}

// Stage geometry of one weight width (2, 4 or 8 bits) and item size KT (32
// or 64 tokens, in groups of 16; the host takes 64 when the routed experts
// average 48 tokens or more). Kernels are instantiated for both sizes, since
// the 64-token form needs more registers and LDS per workgroup.
template <int BITS, int KT>
struct Geo {
    static constexpr int CH = 4;                         // 32-blocks per stage
    static constexpr int WB = 4 * BITS;                  // bytes of a row's block
    static constexpr int RB = CH * WB;                   // bytes of a row per stage
    static constexpr int NPC = RB / 16;                  // 16-byte pieces per row
    static constexpr int KS = RB >= 256 ? 1 : 256 / RB;  // rows per 256-byte bank period
    static constexpr int RPI = 1024 / RB;                // rows per load instruction
    static constexpr int WBYTES = 32 * RB;               // staged weight bytes per wave
    static constexpr int WINSTR = WBYTES / 1024;         // weight loads per wave and stage
    static constexpr int ARB = CH * 32;                  // activation bytes per token
    static constexpr int ANPC = ARB / 16;
    static constexpr int AKS = ARB >= 256 ? 1 : 256 / ARB;
    static constexpr int ARPI = 1024 / ARB;              // token rows per load instruction
    static constexpr int A_OFF = 4 * WBYTES;
    static constexpr int kTok = KT;
    static constexpr int kMaxG = KT / 16;
    static constexpr int D_OFF = A_OFF + KT * ARB;
    static constexpr int SLOT = (D_OFF + KT * CH * 4 + 255) & ~255;
    static constexpr int Scale = BITS == 4 ? 16 : BITS == 2 ? 64 : 1;  // code multiplier
    static constexpr double InvScale = 1.0 / Scale;                    // exact
    static constexpr int Layout = BITS == 4 ? 1 : BITS == 2 ? 2 : 0;   // activation order
    // activation loads per wave and stage for NG 16-token groups (they cover
    // 4 * AIW * ARPI >= 16 NG token rows)
    static constexpr int aiw(int NG) { return (NG * ARB + 255) / 256; }
    static_assert(RB >= 32 && RB <= 256 && ARB <= 256, "stage geometry");
    // 16 rows / tokens span whole swizzle-key periods
    static_assert(16 % (NPC * KS) == 0 && 16 % (ANPC * AKS) == 0, "swizzle keys");
};

__device__ __forceinline__ int wkey(int r, int ks, int npc) { return (r / ks) % npc; }


// Exponent marking a row whose block scales span more than 2^7 (no 31-bit
// integer form): its items take the fp64 epilogue.
constexpr int kWideRow = -0x40000000;

// Integer form of block scales, one wave per row of NB scales (>= 0): with
// d = M 2^e (M the 24-bit significand) and e0 the least e over the row's
// nonzero scales, mi = M << (e - e0), so sum_b d_b I_b = 2^e0 sum_b mi_b I_b
// exactly, and that integer sum fits in int64 (|mi| < 2^31, |I_b| < 2^19, at
// most 2^19 blocks). exps[row] = e0, or kWideRow when some e - e0 exceeds 7 or
// a scale is not finite.
__global__ __launch_bounds__(256) void k_scale_int(const float* __restrict__ d, int64_t rows,
                                                   int NB, int32_t* __restrict__ mi,
                                                   int32_t* __restrict__ exps) {
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const int lane = threadIdx.x & 63;
    const float* dr = d + row * NB;
    int emin = 0x7fffffff, emax = -0x7fffffff;
    bool bad = false;
    for (int b = lane; b < NB; b += 64) {
        const uint32_t u = __float_as_uint(dr[b]);
        const int E = (int)(u >> 23);  // d >= 0: no sign bit
        if (E >= 255) bad = true;
        if ((u & 0x7fffffffu) == 0) continue;
        const int e = E == 0 ? -149 : E - 150;
        emin = min(emin, e);
        emax = max(emax, e);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        emin = min(emin, __shfl_xor(emin, o, 64));
        emax = max(emax, __shfl_xor(emax, o, 64));
    }
    bad = __any(bad);
    const bool empty = emin == 0x7fffffff;
    const bool wide = bad || (!empty && emax - emin > 7);
    const int e0 = empty ? 0 : emin;
    int32_t* mr = mi + row * NB;
    for (int b = lane; b < NB; b += 64) {
        const uint32_t u = __float_as_uint(dr[b]);
        const int E = (int)(u >> 23);
        int32_t m = 0;
        if (!wide && (u & 0x7fffffffu) != 0) {
            const uint32_t M = E == 0 ? (u & 0x7fffffu) : ((u & 0x7fffffu) | 0x800000u);
            const int e = E == 0 ? -149 : E - 150;
            m = (int32_t)(M << (e - e0));
        }
        mr[b] = m;
    }
    if (lane == 0) exps[row] = wide ? kWideRow : e0;
}

__device__ __forceinline__ uint32_t lds_u32(const uint8_t* p) {
    return *reinterpret_cast<const uint32_t*>(p);
}

// s_waitcnt on the vector memory counter only (lgkmcnt(0) with it when LGKM).
template <int N, bool LGKM>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | ((LGKM ? 0 : 15) << 8));
}

// Workgroup barrier without a memory fence (LDS visibility is ordered by the
// explicit waits around it); the empty asm keeps the compiler from moving
// memory operations across it.
__device__ __forceinline__ void stage_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// A operand of a staged block for lane group q; p points at the byte this
// lane reads (swizzled position already applied).
template <int BITS>
__device__ __forceinline__ long a_op(const uint8_t* p, int q) {
    if (BITS == 4) {
        const uint32_t w = lds_u32(p);
        return (long)(uint32_t)nib_lo16(w) | ((long)(uint32_t)nib_hi16(w) << 32);
    }
    if (BITS == 8) return *reinterpret_cast<const long*>(p);
    const uint32_t x = lds_u32(p);
    const int s1 = (q & 1) ? 2 : 6;
    const uint32_t lo = (x << s1) & 0xC0C0C0C0u, hi = (x << (s1 - 2)) & 0xC0C0C0C0u;
    return (long)lo | ((long)hi << 32);
}

// 0 (as 0.0f and as integer) in global memory: the source of the block
// scales past a row's end
__device__ const float kZeroScale = 0.0f;

// Direct-to-LDS loads (lane l writes at LDS address lds + size * l). Issued
// in asm so that the compiler neither waits on them before unrelated LDS
// reads nor counts them; every wait for them is explicit (wait_vm).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma_b128(const void* g, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(g), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory", "m0");
}
__device__ __forceinline__ void dma_b32(const void* g, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
                 :: "v"(g), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory", "m0");
}
#pragma clang diagnostic pop

// Position key of the block scales of token j in a stage row (CH floats):
// tokens j and j + 8 differ, so the reads of 16 tokens hit 16 banks.
template <int CH>
__device__ __forceinline__ int skey(int j) { return CH == 8 ? (j >> 3) & 1 : 0; }

// Per-lane load plan of one wave for a stage: WINSTR weight loads (staged
// rows 16t + i of tile t), AIW activation loads and one load of block scales.
template <int BITS, int KT, int NG>
struct Plan {
    typedef Geo<BITS, KT> G;
    static constexpr int AIW = G::aiw(NG);
    static constexpr int TPI = 64 / G::CH;         // tokens per scale load
    static constexpr int LD = G::WINSTR + AIW + 1;  // loads per wave and stage (with scales)
    // The block scales of a stage: when a row's block count is a multiple of
    // CH, wave 0 loads them all with one 16-byte load per token (lane j: the
    // CH scales of token j, lanes past the item size idle); else the waves'
    // 4-byte loads cover the item's tokens (with 32-token items waves 0 and
    // 1 load them all and waves 2 and 3 none). Waves without a scale load
    // wait on one load fewer per stage.
    static_assert(4 * TPI >= G::kTok && G::kTok % TPI == 0, "scale loads");
    static_assert(G::CH * 4 == 16 && G::kTok <= 64, "one 16-byte scale load per token");
    static_assert(4 * AIW * G::ARPI >= 16 * NG && 4 * AIW * G::ARPI <= G::kTok, "activation loads");
    const uint8_t* wrow[G::WINSTR];  // this lane's weight row
    int wpo[G::WINSTR];              // byte offset of its piece in the stage
    int rowb;
    const int8_t* arow[AIW];         // this lane's activation row
    int apo[AIW];
    int arowb;                       // activation row bytes (H or I)
    const uint8_t* srow;             // scale row of this lane's token (4-byte values)
    int sbk;                         // block of the stage this lane's scale is
    int NB;                          // blocks per row
    int wave;
    bool scl;                        // this wave loads block scales
    bool sx4;                        // ... with one 16-byte load per token

    // tile[t]: row 0 of tile t (16 rows, `rowb` bytes apart, rows from
    // nrow[t] on clamped to its last); rows_of[j]: activation row of token j
    // (j < n; tokens past n repeat token n - 1).
    __device__ __forceinline__ void init(const uint8_t* const (&tile)[2], const int (&nrow)[2],
                                         int64_t rowb_, const int8_t* act, int64_t arowb_,
                                         const int32_t* rows_of, int n, const void* scales,
                                         int NB_) {
        const int lane = threadIdx.x & 63;
        wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        rowb = (int)rowb_;
        arowb = (int)arowb_;
        NB = NB_;
#pragma unroll
        for (int i = 0; i < G::WINSTR; ++i) {
            const int r = i * G::RPI + lane / G::NPC;  // staged row 0..31
            const int t = r >> 4, rr = min(r & 15, nrow[t] - 1);
            const int piece = (lane % G::NPC) ^ wkey(r, G::KS, G::NPC);
            wrow[i] = tile[t] + (int64_t)rr * rowb_;
            wpo[i] = piece * 16;
        }
#pragma unroll
        for (int i = 0; i < AIW; ++i) {
            const int j = (wave * AIW + i) * G::ARPI + lane / G::ANPC;  // token row
            const int piece = (lane % G::ANPC) ^ wkey(j, G::AKS, G::ANPC);
            arow[i] = act + (int64_t)rows_of[min(j, n - 1)] * arowb_;
            apo[i] = piece * 16;
        }
        sx4 = NB_ % G::CH == 0;
        if (sx4) {
            scl = wave == 0;
            sbk = 0;
            srow = static_cast<const uint8_t*>(scales) +
                   (int64_t)rows_of[min(lane, n - 1)] * NB_ * 4;
        } else {
            scl = wave * TPI < G::kTok;
            const int js = min(wave * TPI, G::kTok - TPI) + lane / G::CH;
            sbk = (lane % G::CH) ^ skey<G::CH>(js);
            srow = static_cast<const uint8_t*>(scales) +
                   (int64_t)rows_of[min(js, n - 1)] * NB_ * 4;
        }
    }
    // Issues the stage's loads into the slot at LDS address `slot`. Pieces
    // past a row's end are clamped to its last piece; their blocks read
    // scale 0, so they add nothing.
    __device__ __forceinline__ void issue(int c, uint32_t slot) const {
        const uint32_t wdst = slot + wave * G::WBYTES;
#pragma unroll
        for (int i = 0; i < G::WINSTR; ++i)
            dma_b128(wrow[i] + min(c * G::RB + wpo[i], rowb - 16), wdst + i * 1024);
        const uint32_t adst = slot + G::A_OFF + wave * AIW * 1024;
#pragma unroll
        for (int i = 0; i < AIW; ++i)
            dma_b128(arow[i] + min(c * G::ARB + apo[i], arowb - 16), adst + i * 1024);
        if (scl) {
            if (sx4) {
                // token j's scales land at D_OFF + 16 j, the layout of the
                // 4-byte loads (the swizzle key is 0 with 4-block stages)
                if ((int)(threadIdx.x & 63) < G::kTok)
                    dma_b128(srow + 4 * c * G::CH, slot + G::D_OFF);
            } else {
                const int b = c * G::CH + sbk;
                dma_b32(b < NB ? static_cast<const void*>(srow + 4 * b) : &kZeroScale,
                        slot + G::D_OFF + wave * TPI * G::CH * 4);
            }
        }
    }
};

// K loop: acc[t][g][i] = sum over blocks of d[token] * D(tile t, group g)[i].
// INT: the staged scales are the integer form (k_scale_int) and the sum is
// exact in int64 (one v_mad_i64_i32 per element and block), scaled by
// 2^ex[token] (etok[g]: this lane's token of group g) and rounded once at
// the end; else the scales are floats and the sum is fp64 (one conversion
// and one fma per element and block). TAP records the exact block dots of
// tile 0 for sampled rows.
template <int BITS, int KT, int NG, bool TAP, bool INT>
__device__ __forceinline__ void mm_loop(const Plan<BITS, KT, NG>& pl, uint8_t* smem,
                                        double (&acc)[2][KT / 16][4], const int (&etok)[KT / 16], int nst,
                                        const PfArgs& a, int tap_r0, int s0, int n) {
    typedef Geo<BITS, KT> G;
    constexpr int kMaxG = G::kMaxG;
    constexpr int LD = Plan<BITS, KT, NG>::LD;
    const int lane = threadIdx.x & 63;
    const int lr = lane & 15, q = lane >> 4;
    long acci[2][NG][4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int g = 0; g < kMaxG; ++g) acc[t][g][i] = 0.0;
#pragma unroll
            for (int g = 0; g < NG; ++g) acci[t][g][i] = 0;
        }
    // slot-relative lane bases of the operand reads; the block index of the
    // stage is XORed into the piece bits (no carries: the other terms have
    // those bits clear)
    int wq, wbx;  // piece bit from q, byte in the piece from q
    if (BITS == 4) { wq = 0; wbx = 4 * q; }
    else if (BITS == 8) { wq = q >> 1; wbx = 8 * (q & 1); }
    else { wq = 0; wbx = 4 * (q >> 1); }
    // Loop-invariant operand offsets of block bi inside a slot. Tile 1 sits
    // 16 RB above tile 0 and token group 1 16 ARB / 16 CH floats above group
    // 0 with equal swizzle keys (16 rows / tokens are a whole number of key
    // periods), so they are immediate offsets of the same address.
    const int r0k = wkey(lr, G::KS, G::NPC), a0k = wkey(lr, G::AKS, G::ANPC);
    const int wbase = pl.wave * G::WBYTES + lr * G::RB + ((wq ^ r0k) << 4) + wbx;
    const int abase = G::A_OFF + lr * G::ARB + (((q >> 1) ^ a0k) << 4) + 8 * (q & 1);
    const int dbase = G::D_OFF + lr * G::CH * 4 + 4 * skey<G::CH>(lr);
    int wo[G::CH], ao[G::CH], dof[G::CH];
#pragma unroll
    for (int bi = 0; bi < G::CH; ++bi) {
        const int pb = BITS == 4 ? bi : BITS == 8 ? 2 * bi : bi >> 1;  // piece bits of block bi
        const int ib = BITS == 2 ? 8 * (bi & 1) : 0;                   // byte in the piece
        wo[bi] = (wbase ^ (pb << 4)) + ib;
        ao[bi] = abase ^ (bi << 5);
        dof[bi] = dbase ^ (bi << 2);
    }
    const v4i zero = {0, 0, 0, 0};
    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void*)smem;

    pl.issue(0, lds0);
    if (nst > 1) pl.issue(1, lds0 + G::SLOT);
    // unrolled over the ring so that every slot offset is an immediate
#pragma unroll 1
    for (int cb = 0; cb < nst; cb += kSlots) {
#pragma unroll
        for (int sl = 0; sl < kSlots; ++sl) {
            const int c = cb + sl;
            if (c >= nst) break;
            const uint8_t* cur = smem + sl * G::SLOT;
            // this wave's loads of stage c are in (those of stage c + 1 may
            // not be); with TAP the stores of the taps share the counter and
            // need not complete in order with the loads, so that variant
            // waits for all
            if (c + 1 < nst && !TAP) {
                if (pl.scl) wait_vm<LD, false>();
                else wait_vm<LD - 1, false>();
            } else {
                wait_vm<0, false>();
            }
            stage_barrier();  // every wave's loads of stage c are in; slot c - 1 is free
            if (c + 2 < nst) pl.issue(c + 2, lds0 + ((sl + 2) % kSlots) * G::SLOT);
#pragma unroll
            for (int bi = 0; bi < G::CH; ++bi) {
                const long a0 = a_op<BITS>(cur + wo[bi], q);
                const long a1 = a_op<BITS>(cur + wo[bi] + 16 * G::RB, q);
#pragma unroll
                for (int g = 0; g < NG; ++g) {
                    const long bv =
                        *reinterpret_cast<const long*>(cur + ao[bi] + g * 16 * G::ARB);
                    const uint8_t* dp = cur + dof[bi] + g * 16 * G::CH * 4;
                    const v4i c0 = __builtin_amdgcn_mfma_i32_16x16x32_i8(a0, bv, zero, 0, 0, 0);
                    const v4i c1 = __builtin_amdgcn_mfma_i32_16x16x32_i8(a1, bv, zero, 0, 0, 0);
                    if constexpr (INT) {
                        const long dm = *reinterpret_cast<const int*>(dp);
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            acci[0][g][i] += dm * (long)c0[i];
                            acci[1][g][i] += dm * (long)c1[i];
                            asm volatile("" : "+v"(acci[0][g][i]), "+v"(acci[1][g][i]));
                        }
                    } else {
                        const double dd = (double)*reinterpret_cast<const float*>(dp);
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            acc[0][g][i] += dd * (double)c0[i];
                            acc[1][g][i] += dd * (double)c1[i];
                            asm volatile("" : "+v"(acc[0][g][i]), "+v"(acc[1][g][i]));
                        }
                    }
                    if (TAP) {
                        const int b = c * G::CH + bi, j = 16 * g + lr, BH = pl.NB;
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int r = tap_r0 + 4 * q + i;
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
                for (int i = 0; i < 4; ++i) acc[t][g][i] = ldexp((double)acci[t][g][i], etok[g]);
    }
}

// Element of a 32-block stored at byte p in activation order L (0 natural,
// 1 int4's 8-group order, 2 int2's 16-group order).
template <int L>
__device__ __forceinline__ constexpr int act_elem(int p) {
    return L == 0 ? p
         : L == 1 ? (p & ~7) + 2 * (p & 3) + ((p >> 2) & 1)
                  : (p & ~15) + 4 * (p & 3) + ((p >> 2) & 3);
}

// Gate/up + SwiGLU + Q8_0(h) for one item and 64 intermediate rows; Q8_0(h)
// is stored in the activation order of the down weights' width.
template <int BITS, int KT, bool TAP>
__global__ __launch_bounds__(256) void k_pf_gateup(PfArgs a) {
    typedef Geo<BITS, KT> G;
    constexpr int kMaxG = KT / 16;
    __shared__ __align__(1024) uint8_t smem[kSlots * G::SLOT];
    static_assert(kSlots * G::SLOT >= KT * (kRows + 1) * 4, "h reuses the ring");
    const int nrt = a.I / kRows;
    int it, rt;
    if (!work_of<KT>(a, nrt, it, rt)) return;
    const int e = a.item_e[it], s0 = a.item_s0[it], n = a.item_n[it];
    const int H = a.H, I = a.I, BH = H >> 5;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lr = lane & 15, q = lane >> 4;
    const int64_t rowb = (int64_t)H * BITS / 8;
    const uint8_t* gate = a.eq + (int64_t)e * a.blob_q;
    const uint8_t* up = gate + (int64_t)I * rowb;
    const int r0 = rt * kRows + wave * 16;
    const int nst = (BH + G::CH - 1) / G::CH;

    const uint8_t* const tiles[2] = {gate + (int64_t)r0 * rowb, up + (int64_t)r0 * rowb};
    const int nrow[2] = {16, 16};
    const int32_t* rows_of = a.slot_tok + s0;  // token of each of the item's slots
    // the row scales of this lane's results, loaded before the K loop so that
    // the epilogue does not wait for them
    const float* gs = a.es + (int64_t)e * a.blob_s;
    const float* us = gs + I;
    float gsr[4], usr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        gsr[i] = gs[r0 + 4 * q + i];
        usr[i] = us[r0 + 4 * q + i];
    }
    // integer scales unless the call has none (few tokens) or a token of the
    // item has none
    bool wide = a.ex == nullptr;
    int etok[kMaxG] = {};
    if (!wide) {
        const int tv = rows_of[min((int)threadIdx.x, n - 1)];
        wide = __syncthreads_or((int)threadIdx.x < n && a.ex[tv] == kWideRow);
#pragma unroll
        for (int g = 0; g < kMaxG; ++g) etok[g] = a.ex[rows_of[min(16 * g + lr, n - 1)]];
    }
    double acc[2][kMaxG][4];
    auto run = [&](auto ng, auto in) {
        constexpr int NG = decltype(ng)::value;
        constexpr bool INT = decltype(in)::value;
        Plan<BITS, KT, NG> pl;
        pl.init(tiles, nrow, rowb, a.qx, H, rows_of, n,
                INT ? static_cast<const void*>(a.mx) : static_cast<const void*>(a.dx), BH);
        mm_loop<BITS, KT, NG, TAP, INT>(pl, smem, acc, etok, nst, a, r0, s0, n);
    };
    typedef std::integral_constant<int, 1> G1;
    typedef std::integral_constant<int, 2> G2;
    typedef std::integral_constant<int, 4> G4;
    typedef std::integral_constant<bool, true> Int;
    typedef std::integral_constant<bool, false> F64;
    if (!wide) {
        if (n <= 16) run(G1{}, Int{});
        else if (KT == 32 || n <= 32) run(G2{}, Int{});
        else if constexpr (KT == 64) run(G4{}, Int{});
    } else {
        if (n <= 16) run(G1{}, F64{});
        else if (KT == 32 || n <= 32) run(G2{}, F64{});
        else if constexpr (KT == 64) run(G4{}, F64{});
    }
    __syncthreads();  // the ring is reused for h below
    float (*hbuf)[kRows + 1] = reinterpret_cast<float (*)[kRows + 1]>(smem);

    // SwiGLU (token groups that hold tokens only), then Q8_0 over each 32
    // consecutive h rows of a token
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int g = 0; g < kMaxG; ++g) {
            if (16 * g >= n) continue;  // uniform
            // the sums carry the multiplier of the weight codes: scale it away (exact)
            const float gv = (float)((double)gsr[i] * (acc[0][g][i] * G::InvScale));
            const float uv = (float)((double)usr[i] * (acc[1][g][i] * G::InvScale));
            hbuf[16 * g + lr][wave * 16 + 4 * q + i] = swiglu_f32(gv, uv);
        }
    }
    __syncthreads();
    // P consecutive threads per 32-row block of a token, each taking VPT of
    // its bytes (in the activation order of the down weights' width); the
    // block's amax is the maximum over the P threads
    constexpr int P = 256 / (2 * KT), VPT = 32 / P;
    static_assert(P == 2 || P == 4, "threads per h block");
    if ((int)threadIdx.x < 2 * P * n) {
        const int j = threadIdx.x / (2 * P), kb = (threadIdx.x / P) & 1, sp = threadIdx.x % P;
        const float* hv = &hbuf[j][32 * kb];
        float amax = 0.0f;
#pragma unroll
        for (int k = 0; k < VPT; ++k)
            amax = fmaxf(amax, fabsf(hv[act_elem<G::Layout>(VPT * sp + k)]));
#pragma unroll
        for (int o = 1; o < P; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
        const float d = amax / 127.0f;
        uint32_t w[VPT / 4];
#pragma unroll
        for (int i = 0; i < VPT / 4; ++i) {
            const int p0 = VPT * sp + 4 * i;
            w[i] = pack4_i8(q8_code(hv[act_elem<G::Layout>(p0)], d),
                            q8_code(hv[act_elem<G::Layout>(p0 + 1)], d),
                            q8_code(hv[act_elem<G::Layout>(p0 + 2)], d),
                            q8_code(hv[act_elem<G::Layout>(p0 + 3)], d));
        }
        int8_t* o = a.qh + (int64_t)(s0 + j) * I + rt * kRows + 32 * kb + VPT * sp;
        if constexpr (VPT == 8) {
            typedef unsigned v2u __attribute__((ext_vector_type(2)));
            *reinterpret_cast<v2u*>(o) = v2u{w[0], w[1]};
        } else {
            typedef unsigned v4u __attribute__((ext_vector_type(4)));
            *reinterpret_cast<v4u*>(o) = v4u{w[0], w[1], w[2], w[3]};
        }
        if (sp == 0) a.dh[(int64_t)(s0 + j) * (I >> 5) + rt * 2 + kb] = d;
    }
}

// Down projection for one item and 128 output rows: ye[slot, row] =
// fp32(s_down[row] * sum_b d_h,b * I_b). The last row tile may pass H (rows
// clamped for loading, not stored).
template <int BITS, int KT>
__global__ __launch_bounds__(256) void k_pf_down(PfArgs a) {
    typedef Geo<BITS, KT> G;
    constexpr int kMaxG = KT / 16;
    __shared__ __align__(1024) uint8_t smem[kSlots * G::SLOT];
    static_assert(kSlots * G::SLOT >= KT * (kDnRows + 1) * 4, "y reuses the ring");
    __shared__ int s_rows[KT];
    const int nrt = (a.H + kDnRows - 1) / kDnRows;
    const int it = blockIdx.x / nrt, rt = blockIdx.x - it * nrt;
    if (it >= *a.n_items) return;
    const int e = a.item_e[it], s0 = a.item_s0[it], n = a.item_n[it];
    const int H = a.H, I = a.I, BI = I >> 5;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lr = lane & 15, q = lane >> 4;
    const int64_t rowb = (int64_t)I * BITS / 8;
    const uint8_t* down = a.eq + (int64_t)e * a.blob_q + 2 * (int64_t)H * rowb;
    const int R0 = rt * kDnRows + wave * 32;
    const int nst = (BI + G::CH - 1) / G::CH;
    // the item's slots are consecutive rows of q_h
    if (threadIdx.x < KT) s_rows[threadIdx.x] = s0 + threadIdx.x;
    __syncthreads();

    // rows past H are clamped to H - 1 (tile bases stay inside the matrix)
    const int t0 = min(R0, H - 1), t1 = min(R0 + 16, H - 1);
    const uint8_t* const tiles[2] = {down + (int64_t)t0 * rowb, down + (int64_t)t1 * rowb};
    const int nrow[2] = {max(1, min(16, H - t0)), max(1, min(16, H - t1))};
    // integer scales unless the call has none (few tokens) or a slot of the
    // item has none
    bool wide = a.eh == nullptr;
    int etok[kMaxG] = {};
    if (!wide) {
        wide = __syncthreads_or((int)threadIdx.x < n &&
                                a.eh[s0 + min((int)threadIdx.x, n - 1)] == kWideRow);
#pragma unroll
        for (int g = 0; g < kMaxG; ++g) etok[g] = a.eh[s0 + min(16 * g + lr, n - 1)];
    }
    double acc[2][kMaxG][4];
    auto run = [&](auto ng, auto in) {
        constexpr int NG = decltype(ng)::value;
        constexpr bool INT = decltype(in)::value;
        Plan<BITS, KT, NG> pl;
        pl.init(tiles, nrow, rowb, a.qh, I, s_rows, n,
                INT ? static_cast<const void*>(a.mh) : static_cast<const void*>(a.dh), BI);
        mm_loop<BITS, KT, NG, false, INT>(pl, smem, acc, etok, nst, a, 0, s0, n);
    };
    typedef std::integral_constant<int, 1> G1;
    typedef std::integral_constant<int, 2> G2;
    typedef std::integral_constant<int, 4> G4;
    typedef std::integral_constant<bool, true> Int;
    typedef std::integral_constant<bool, false> F64;
    if (!wide) {
        if (n <= 16) run(G1{}, Int{});
        else if (KT == 32 || n <= 32) run(G2{}, Int{});
        else if constexpr (KT == 64) run(G4{}, Int{});
    } else {
        if (n <= 16) run(G1{}, F64{});
        else if (KT == 32 || n <= 32) run(G2{}, F64{});
        else if constexpr (KT == 64) run(G4{}, F64{});
    }
    __syncthreads();  // the ring is reused for y below
    float (*ybuf)[kDnRows + 1] = reinterpret_cast<float (*)[kDnRows + 1]>(smem);

    const float* ds = a.es + (int64_t)e * a.blob_s + 2 * I;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int rl = wave * 32 + 16 * t + 4 * q + i;
            const float dsr = ds[min(rt * kDnRows + rl, H - 1)];
#pragma unroll
            for (int g = 0; g < kMaxG; ++g)  // undo the multiplier of the weight codes
                ybuf[16 * g + lr][rl] = (float)((double)dsr * (acc[t][g][i] * G::InvScale));
        }
    __syncthreads();
    const int nr = min(kDnRows, H - rt * kDnRows);
    for (int v = threadIdx.x; v < n * kDnRows; v += 256) {
        const int j = v >> 7, r = v & 127;
        if (r < nr) a.ye[(int64_t)(s0 + j) * H + rt * kDnRows + r] = ybuf[j][r];
    }
}

}  // namespace pf
