// Grouped int8 MFMA kernels for many tokens (prefill, stacked layers).
//
// Work item = (expert, first slot, n <= 32 of its tokens). A workgroup takes
// one item and a tile of 64 output rows; wave w owns rows 16w .. 16w+15 of
// the tile (for gate/up: those gate rows and the matching up rows, so SwiGLU
// needs no exchange). Per 32-wide block b every wave issues
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
// Both operands go through LDS in chunks of 16 blocks (8 for int8), loaded one chunk
// ahead into registers with coalesced 16-byte loads: weight rows per wave
// (each wave reads only its own rows), the item's activation rows and block
// scales once per workgroup (all four waves use the same tokens). Pitches
// are padded so the operand reads hit distinct banks.
#pragma once

#include <type_traits>

#include "coli_common.h"

namespace pf {

typedef int v4i __attribute__((ext_vector_type(4)));
// plain vector type for 16-byte moves (HIP's uint4 struct copies become
// memcpy calls that keep staging arrays out of registers)
typedef unsigned v4u __attribute__((ext_vector_type(4)));

constexpr int kTok = 32;              // tokens per work item
constexpr int kRows = 64;             // output rows per workgroup

// Staging geometry and operand form of one weight width (2, 4 or 8 bits).
template <int BITS>
struct WFmt {
    static constexpr int CH = BITS == 8 ? 8 : 16;  // blocks staged per step
    static constexpr int WB = 4 * BITS;            // bytes of a 32-wide block of a row
    static constexpr int RB = CH * WB;             // bytes of a row per chunk
    static constexpr int PB = RB / 16;             // bytes per lane (16 lanes per row)
    static constexpr int Pitch = RB + 8;           // LDS bytes per staged row
    static constexpr int ActPitch = CH * 32 + 16;  // LDS bytes per staged activation row
    static constexpr int DPitch = CH + 1;          // floats per staged scale row
    static constexpr int ActBytes = kTok * ActPitch;
    static constexpr int DBytes = kTok * DPitch * 4;
    static constexpr int Scale = BITS == 4 ? 16 : BITS == 2 ? 64 : 1;  // code multiplier
    static constexpr double InvScale = 1.0 / Scale;                    // exact
    static constexpr int Layout = BITS == 4 ? 1 : BITS == 2 ? 2 : 0;   // activation order
};

struct PfArgs {
    const uint8_t* eq;
    const float* es;
    int64_t blob_q, blob_s;
    int H, I;
    const int8_t* qx;      // [T, H] Q8_0 codes of x (8-group order)
    const float* dx;       // [T, H/32]
    const int32_t* item_e;
    const int32_t* item_s0;
    const int32_t* item_n;
    const int32_t* n_items;
    const int32_t* slot_tok;
    int8_t* qh;            // [slots, I]
    float* dh;             // [slots, I/32]
    float* ye;             // [slots, H]
    int32_t* tap;
    int tap_rows, tap_stride;
};

__device__ __forceinline__ long a_operand(uint32_t w) {
    return (long)(uint32_t)nib_lo16(w) | ((long)(uint32_t)nib_hi16(w) << 32);
}

__device__ __forceinline__ uint32_t lds_u32(const uint8_t* p) {
    return *reinterpret_cast<const uint32_t*>(p);
}

// A operand (8 int8 values, k = 8q .. 8q+7 of the block's k order) of the
// staged block starting at blk, for lane group q.
template <int BITS>
__device__ __forceinline__ long a_op(const uint8_t* blk, int q) {
    if (BITS == 4) return a_operand(lds_u32(blk + 4 * q));
    if (BITS == 8) return *reinterpret_cast<const long*>(blk + 8 * q);
    const uint32_t x = lds_u32(blk + 4 * (q >> 1));
    const int s1 = (q & 1) ? 2 : 6;
    const uint32_t lo = (x << s1) & 0xC0C0C0C0u, hi = (x << (s1 - 2)) & 0xC0C0C0C0u;
    return (long)lo | ((long)hi << 32);
}

// Stages NR rows of one chunk: lane l loads PB bytes (16, int2: 8) of staged
// row (l >> 4) + 4k at piece (l & 15) of the chunk. Staged rows 16m .. 16m+15
// are rows 0..15 of matrix m, starting at base[m] (this lane's row l >> 4)
// with `stride` bytes between rows, `rowb` bytes per row.
template <int NR, int BITS>
struct Stager {
    typedef WFmt<BITS> F;
    typedef unsigned v2u __attribute__((ext_vector_type(2)));
    typedef typename std::conditional<F::PB == 16, v4u, v2u>::type piece_t;
    const uint8_t* base[NR / 16];
    int64_t stride;
    int rowb;
    __device__ __forceinline__ void issue(int c, piece_t (&v)[NR / 4]) const {
        const int off = min(c * F::RB + (int)(threadIdx.x & 15) * F::PB, rowb - F::PB);
#pragma unroll
        for (int k = 0; k < NR / 4; ++k)
            v[k] = *reinterpret_cast<const piece_t*>(base[k / 4] + (int64_t)(4 * (k % 4)) * stride +
                                                     off);
    }
    __device__ __forceinline__ void commit(uint8_t* lds, const piece_t (&v)[NR / 4]) const {
        const int r0 = (threadIdx.x & 63) >> 4, bi = threadIdx.x & 15;
#pragma unroll
        for (int k = 0; k < NR / 4; ++k) {
            uint8_t* d = lds + (r0 + 4 * k) * F::Pitch + bi * F::PB;
            if constexpr (F::PB == 16) {
                *reinterpret_cast<v2u*>(d) = v[k].xy;
                *reinterpret_cast<v2u*>(d + 8) = v[k].zw;
            } else {
                *reinterpret_cast<v2u*>(d) = v[k];
            }
        }
    }
};

// Activation rows of the item's 32 tokens (rows of a [*, NB * 32] int8
// matrix in the width's element order, with NB block scales per row), one
// chunk of CH blocks: thread tid loads the 16-byte half (tid & 1) of block
// (tid % 2CH) / 2 of token rows tid / 2CH + (256 / 2CH) k, and threads below
// 8 CH four block scales each.
template <int CH>
struct ActStager {
    static constexpr int TPR = 2 * CH;        // threads per token row
    static constexpr int RPP = 256 / TPR;     // token rows per pass
    static constexpr int NP = kTok / RPP;     // passes
    static constexpr int ActPitch = CH * 32 + 16, DPitch = CH + 1;
    const int8_t* row[NP];
    const float* drow;
    __device__ __forceinline__ void init(const int8_t* base, const float* dbase, int64_t pitch,
                                         int NB, const int32_t* rows_of, int n) {
        const int half = threadIdx.x & 1;
#pragma unroll
        for (int k = 0; k < NP; ++k) {
            const int j = min((int)(threadIdx.x / TPR) + RPP * k, n - 1);
            row[k] = base + (int64_t)rows_of[j] * pitch + 16 * half;
        }
        const int jd = min((int)((threadIdx.x % (8 * CH)) / (CH / 4)), n - 1);
        drow = dbase + (int64_t)rows_of[jd] * NB;
    }
    __device__ __forceinline__ void issue(int c, int NB, v4u (&v)[NP], float (&dv)[4]) const {
        const int b = min(c * CH + (int)((threadIdx.x % TPR) >> 1), NB - 1);
#pragma unroll
        for (int k = 0; k < NP; ++k) v[k] = *reinterpret_cast<const v4u*>(row[k] + b * 32);
        // every thread loads (threads >= 8 CH repeat rows of the first 8 CH, in
        // bounds), so the values stay in registers; only threads < 8 CH store
        const int b0 = c * CH + (threadIdx.x % (CH / 4)) * 4;
#pragma unroll
        for (int i = 0; i < 4; ++i) dv[i] = drow[min(b0 + i, NB - 1)];
    }
    // Scales of blocks past NB are stored as 0, so those blocks add nothing.
    __device__ __forceinline__ void commit(int c, int NB, uint8_t* act, float* dbuf,
                                           const v4u (&v)[NP], const float (&dv)[4]) const {
        const int blk = (threadIdx.x % TPR) >> 1, half = threadIdx.x & 1;
#pragma unroll
        for (int k = 0; k < NP; ++k) {
            const int j = threadIdx.x / TPR + RPP * k;
            *reinterpret_cast<v4u*>(act + j * ActPitch + blk * 32 + 16 * half) = v[k];
        }
        if (threadIdx.x < 8 * CH) {
            const int j = threadIdx.x / (CH / 4), b0 = (threadIdx.x % (CH / 4)) * 4;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                dbuf[j * DPitch + b0 + i] = (c * CH + b0 + i < NB) ? dv[i] : 0.0f;
        }
    }
};

// K loop of the gate/up kernel for NG 16-token groups: MFMA per block and
// group, fp64 epilogue. Inside a chunk there are no branches, so the
// compiler can overlap the next block's LDS reads and MFMAs with the current
// block's epilogue.
template <int BITS, int NG, bool TAP>
__device__ __forceinline__ void gateup_loop(const PfArgs& a, const Stager<32, BITS>& st,
                                            const ActStager<WFmt<BITS>::CH>& as, uint8_t* lds,
                                            uint8_t* act, float* dbuf, double (&accg)[2][4],
                                            double (&accu)[2][4], int BH, int r0, int q, int lr,
                                            int s0, int n) {
    typedef WFmt<BITS> F;
    constexpr int CH = F::CH;
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int i = 0; i < 4; ++i) accg[g][i] = accu[g][i] = 0.0;
    const v4i zero = {0, 0, 0, 0};
    const int nch = (BH + CH - 1) / CH;
    typename Stager<32, BITS>::piece_t wv[8];
    v4u av[ActStager<CH>::NP];
    float adv[4];
    st.issue(0, wv);
    as.issue(0, BH, av, adv);
    st.commit(lds, wv);
    as.commit(0, BH, act, dbuf, av, adv);
    __syncthreads();
#pragma unroll 1
    for (int c = 0; c < nch; ++c) {
        // unconditional (keeps the staging registers out of memory); after
        // the last chunk this re-reads that chunk, from cache
        const int cn = min(c + 1, nch - 1);
        st.issue(cn, wv);
        as.issue(cn, BH, av, adv);
#pragma unroll
        for (int bi = 0; bi < CH; ++bi) {
            const long ag = a_op<BITS>(lds + lr * F::Pitch + bi * F::WB, q);
            const long au = a_op<BITS>(lds + (16 + lr) * F::Pitch + bi * F::WB, q);
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                const int j = 16 * g + lr;
                const long bv =
                    *reinterpret_cast<const long*>(act + j * F::ActPitch + bi * 32 + 8 * q);
                const double dd = (double)dbuf[j * F::DPitch + bi];
                const v4i cg = __builtin_amdgcn_mfma_i32_16x16x32_i8(ag, bv, zero, 0, 0, 0);
                const v4i cu = __builtin_amdgcn_mfma_i32_16x16x32_i8(au, bv, zero, 0, 0, 0);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    accg[g][i] += dd * (double)cg[i];
                    accu[g][i] += dd * (double)cu[i];
                    asm volatile("" : "+v"(accg[g][i]), "+v"(accu[g][i]));
                }
                if (TAP) {
                    const int b = c * CH + bi;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int r = r0 + 4 * q + i;
                        if (j < n && b < BH && (r % a.tap_stride) == 0)
                            a.tap[((int64_t)(s0 + j) * a.tap_rows + r / a.tap_stride) * BH + b] =
                                cg[i] / F::Scale;
                    }
                }
            }
        }
        __syncthreads();
        st.commit(lds, wv);
        as.commit(cn, BH, act, dbuf, av, adv);
        __syncthreads();
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
template <int BITS, bool TAP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void k_pf_gateup(PfArgs a) {
    typedef WFmt<BITS> F;
    constexpr int kW = 32 * F::Pitch;  // per-wave weight staging (16 gate + 16 up rows)
    __shared__ __align__(16) uint8_t smem[4 * kW + F::ActBytes + F::DBytes];
    const int nrt = a.I / kRows;
    const int it = blockIdx.x / nrt, rt = blockIdx.x - it * nrt;
    if (it >= *a.n_items) return;
    const int e = a.item_e[it], s0 = a.item_s0[it], n = a.item_n[it];
    const int H = a.H, I = a.I, BH = H >> 5;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lr = lane & 15, q = lane >> 4;
    const int ng = (n + 15) >> 4;  // 16-token groups in use (1 or 2)
    const int64_t rowb = (int64_t)H * BITS / 8;
    const uint8_t* gate = a.eq + (int64_t)e * a.blob_q;
    const uint8_t* up = gate + (int64_t)I * rowb;
    const int r0 = rt * kRows + wave * 16;
    uint8_t* lds = smem + wave * kW;
    uint8_t* act = smem + 4 * kW;
    float* dbuf = reinterpret_cast<float*>(smem + 4 * kW + F::ActBytes);
    static_assert(F::ActBytes >= kTok * (kRows + 1) * 4, "h reuses the activation area");

    Stager<32, BITS> st;  // staged rows 0..15: gate rows r0.., 16..31: up rows r0..
    st.stride = rowb;
    st.rowb = (int)rowb;
    st.base[0] = gate + (int64_t)(r0 + q) * rowb;
    st.base[1] = up + (int64_t)(r0 + q) * rowb;
    ActStager<F::CH> as;
    as.init(a.qx, a.dx, H, BH, a.slot_tok + s0, n);

    double accg[2][4], accu[2][4];
    if (ng == 1)
        gateup_loop<BITS, 1, TAP>(a, st, as, lds, act, dbuf, accg, accu, BH, r0, q, lr, s0, n);
    else
        gateup_loop<BITS, 2, TAP>(a, st, as, lds, act, dbuf, accg, accu, BH, r0, q, lr, s0, n);
    __syncthreads();  // the activation area is reused for h below
    float (*hbuf)[kRows + 1] = reinterpret_cast<float (*)[kRows + 1]>(act);

    // SwiGLU, then Q8_0 over each 32 consecutive h rows of a token
    const float* gs = a.es + (int64_t)e * a.blob_s;
    const float* us = gs + I;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = r0 + 4 * q + i;
        const float gsr = gs[r], usr = us[r];
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            // the sums carry the multiplier of the weight codes: scale it away (exact)
            const float gv = (float)((double)gsr * (accg[g][i] * F::InvScale));
            const float uv = (float)((double)usr * (accu[g][i] * F::InvScale));
            hbuf[16 * g + lr][wave * 16 + 4 * q + i] = swiglu_f32(gv, uv);
        }
    }
    __syncthreads();
    if ((int)threadIdx.x < 2 * n) {
        const int j = threadIdx.x >> 1, kb = threadIdx.x & 1;
        const float* hv = &hbuf[j][32 * kb];
        float amax = 0.0f;
#pragma unroll
        for (int k = 0; k < 32; ++k) amax = fmaxf(amax, fabsf(hv[k]));
        const float d = amax / 127.0f;
        uint32_t w[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            w[i] = pack4_i8(q8_code(hv[act_elem<F::Layout>(4 * i)], d),
                            q8_code(hv[act_elem<F::Layout>(4 * i + 1)], d),
                            q8_code(hv[act_elem<F::Layout>(4 * i + 2)], d),
                            q8_code(hv[act_elem<F::Layout>(4 * i + 3)], d));
        v4u* o = reinterpret_cast<v4u*>(a.qh + (int64_t)(s0 + j) * I + rt * kRows + 32 * kb);
        o[0] = v4u{w[0], w[1], w[2], w[3]};
        o[1] = v4u{w[4], w[5], w[6], w[7]};
        a.dh[(int64_t)(s0 + j) * (I >> 5) + rt * 2 + kb] = d;
    }
}

// K loop of the down kernel (as gateup_loop, one weight matrix).
template <int BITS, int NG>
__device__ __forceinline__ void down_loop(const Stager<16, BITS>& st,
                                          const ActStager<WFmt<BITS>::CH>& as, uint8_t* lds,
                                          uint8_t* act, float* dbuf, double (&acc)[2][4],
                                          int BI, int q, int lr) {
    typedef WFmt<BITS> F;
    constexpr int CH = F::CH;
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[g][i] = 0.0;
    const v4i zero = {0, 0, 0, 0};
    const int nch = (BI + CH - 1) / CH;
    typename Stager<16, BITS>::piece_t wv[4];
    v4u av[ActStager<CH>::NP];
    float adv[4];
    st.issue(0, wv);
    as.issue(0, BI, av, adv);
    st.commit(lds, wv);
    as.commit(0, BI, act, dbuf, av, adv);
    __syncthreads();
#pragma unroll 1
    for (int c = 0; c < nch; ++c) {
        // unconditional (keeps the staging registers out of memory); after
        // the last chunk this re-reads that chunk, from cache
        const int cn = min(c + 1, nch - 1);
        st.issue(cn, wv);
        as.issue(cn, BI, av, adv);
#pragma unroll
        for (int bi = 0; bi < CH; ++bi) {
            const long aw = a_op<BITS>(lds + lr * F::Pitch + bi * F::WB, q);
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                const int j = 16 * g + lr;
                const long bv =
                    *reinterpret_cast<const long*>(act + j * F::ActPitch + bi * 32 + 8 * q);
                const double dd = (double)dbuf[j * F::DPitch + bi];
                const v4i cd = __builtin_amdgcn_mfma_i32_16x16x32_i8(aw, bv, zero, 0, 0, 0);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc[g][i] += dd * (double)cd[i];
                    asm volatile("" : "+v"(acc[g][i]));
                }
            }
        }
        __syncthreads();
        st.commit(lds, wv);
        as.commit(cn, BI, act, dbuf, av, adv);
        __syncthreads();
    }
}

// Down projection for one item and 64 output rows: ye[slot, row] =
// fp32(s_down[row] * sum_b d_h,b * I_b).
template <int BITS>
__global__ __launch_bounds__(256) void k_pf_down(PfArgs a) {
    typedef WFmt<BITS> F;
    constexpr int kW = 16 * F::Pitch;
    __shared__ __align__(16) uint8_t smem[4 * kW + F::ActBytes + F::DBytes];
    const int nrt = a.H / kRows;
    const int it = blockIdx.x / nrt, rt = blockIdx.x - it * nrt;
    if (it >= *a.n_items) return;
    const int e = a.item_e[it], s0 = a.item_s0[it], n = a.item_n[it];
    const int H = a.H, I = a.I, BI = I >> 5;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lr = lane & 15, q = lane >> 4;
    const int ng = (n + 15) >> 4;
    const int64_t rowb = (int64_t)I * BITS / 8;
    const uint8_t* down = a.eq + (int64_t)e * a.blob_q + 2 * (int64_t)H * I * BITS / 8;
    const int r0 = rt * kRows + wave * 16;
    uint8_t* lds = smem + wave * kW;
    uint8_t* act = smem + 4 * kW;
    float* dbuf = reinterpret_cast<float*>(smem + 4 * kW + F::ActBytes);
    static_assert(F::ActBytes >= kTok * (kRows + 1) * 4, "y reuses the activation area");

    Stager<16, BITS> st;
    st.stride = rowb;
    st.rowb = (int)rowb;
    st.base[0] = down + (int64_t)(r0 + q) * rowb;
    // the item's slots are consecutive rows of q_h
    __shared__ int s_rows[kTok];
    if (threadIdx.x < kTok) s_rows[threadIdx.x] = s0 + threadIdx.x;
    __syncthreads();
    ActStager<F::CH> as;
    as.init(a.qh, a.dh, I, BI, s_rows, n);

    double acc[2][4];
    if (ng == 1)
        down_loop<BITS, 1>(st, as, lds, act, dbuf, acc, BI, q, lr);
    else
        down_loop<BITS, 2>(st, as, lds, act, dbuf, acc, BI, q, lr);
    __syncthreads();  // the activation area is reused for y below
    float (*ybuf)[kRows + 1] = reinterpret_cast<float (*)[kRows + 1]>(act);

    const float* ds = a.es + (int64_t)e * a.blob_s + 2 * I;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int rl = wave * 16 + 4 * q + i;
        const float dsr = ds[rt * kRows + rl];
#pragma unroll
        for (int g = 0; g < 2; ++g)  // undo the multiplier of the weight codes
            ybuf[16 * g + lr][rl] = (float)((double)dsr * (acc[g][i] * F::InvScale));
    }
    __syncthreads();
    for (int v = threadIdx.x; v < n * kRows; v += 256) {
        const int j = v >> 6, r = v & 63;
        a.ye[(int64_t)(s0 + j) * H + rt * kRows + r] = ybuf[j][r];
    }
}

}  // namespace pf
