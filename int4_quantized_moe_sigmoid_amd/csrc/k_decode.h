// Fused path for few tokens (decode at batch 1, MTP verify): three launches.
//
//   A  router rows, one workgroup per expert (fp64 logits); workgroup 0 also
//      writes Q8_0(x).
//   B  gate/up + SwiGLU + Q8_0(h). The shared expert's h-blocks come first in
//      the grid: they need no routing, so they stream while the routed
//      workgroups each recompute the top-k and expert bucketing of the <= 4
//      tokens in LDS (a few hundred values; cheaper here than any grid-wide
//      hand-off, which on this GPU means an L2 write-back per workgroup).
//      Tokens that share an expert are served by one pass over its weights.
//   C  down projection of every expert in use plus the weighted combine,
//      written straight into y.
//
// Kernel boundaries are the only synchronisation. Weight streams use 16-byte
// nontemporal loads (each byte is used once); lane l owns blocks l, l+64,
// l+128 of a row so a wave instruction reads 1 KiB contiguous.
#pragma once

#include "coli_common.h"
#include "coli_args.h"

namespace dec {


typedef unsigned v4u __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 ldnt(const uint8_t* p) {
    const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

typedef unsigned v2u __attribute__((ext_vector_type(2)));

// Expert weight widths of the few-token kernels. A row holds 4 BITS bytes
// per 32-wide block (codes packed little end first). blk is one block in
// registers, dot its exact int32 product with 32 Q8_0 codes stored in the
// order kL (0 natural, 1 the 8-group order e0 e2 e4 e6 e1 e3 e5 e7, 2 the
// 16-group order e0 e4 e8 e12 e1 ...), times kDiv = 1 / kInv (the int4
// codes enter the dot as 16 q, int2 codes as 64 q, each shifted into the top
// of its byte).
// HR h-rows per gate/up step keep a step's loads at 3 KB per row pair of
// int4 (one int8 row pair, four int2 row pairs).
template <int BITS> struct DW;
template <> struct DW<4> {
    typedef uint4 blk;
    static constexpr int kL = 1, kDiv = 16, HR = 2;
    static constexpr double kInv = 0.0625;
    static __device__ __forceinline__ blk load(const uint8_t* p) { return ldnt(p); }
    static __device__ __forceinline__ int dot(const blk& w, uint4 a0, uint4 a1) {
        return dot_block16(w, a0, a1);
    }
};
template <> struct DW<8> {
    struct blk {
        v4u lo, hi;
    };
    static constexpr int kL = 0, kDiv = 1, HR = 1;
    static constexpr double kInv = 1.0;
    static __device__ __forceinline__ blk load(const uint8_t* p) {
        blk b;
        b.lo = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
        b.hi = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p + 16));
        return b;
    }
    static __device__ __forceinline__ int dot(const blk& w, uint4 a0, uint4 a1) {
        int acc = 0;
        acc = __builtin_amdgcn_sdot4((int)w.lo.x, (int)a0.x, acc, false);
        acc = __builtin_amdgcn_sdot4((int)w.lo.y, (int)a0.y, acc, false);
        acc = __builtin_amdgcn_sdot4((int)w.lo.z, (int)a0.z, acc, false);
        acc = __builtin_amdgcn_sdot4((int)w.lo.w, (int)a0.w, acc, false);
        acc = __builtin_amdgcn_sdot4((int)w.hi.x, (int)a1.x, acc, false);
        acc = __builtin_amdgcn_sdot4((int)w.hi.y, (int)a1.y, acc, false);
        acc = __builtin_amdgcn_sdot4((int)w.hi.z, (int)a1.z, acc, false);
        acc = __builtin_amdgcn_sdot4((int)w.hi.w, (int)a1.w, acc, false);
        return acc;
    }
};
template <> struct DW<2> {
    typedef v2u blk;
    static constexpr int kL = 2, kDiv = 64, HR = 4;
    static constexpr double kInv = 0.015625;
    static __device__ __forceinline__ blk load(const uint8_t* p) {
        return __builtin_nontemporal_load(reinterpret_cast<const v2u*>(p));
    }
    // (x << s) & 0xC0C0C0C0 puts code 4j + (6 - s) / 2 of dword x, times 64,
    // in byte j: s = 6, 4, 2, 0 give elements {0,4,8,12}, {1,5,9,13}, ...
    static __device__ __forceinline__ int dot(const blk& w, uint4 a0, uint4 a1) {
        constexpr unsigned M = 0xC0C0C0C0u;
        int acc = 0;
        acc = __builtin_amdgcn_sdot4((int)((w.x << 6) & M), (int)a0.x, acc, false);
        acc = __builtin_amdgcn_sdot4((int)((w.x << 4) & M), (int)a0.y, acc, false);
        acc = __builtin_amdgcn_sdot4((int)((w.x << 2) & M), (int)a0.z, acc, false);
        acc = __builtin_amdgcn_sdot4((int)(w.x & M), (int)a0.w, acc, false);
        acc = __builtin_amdgcn_sdot4((int)((w.y << 6) & M), (int)a1.x, acc, false);
        acc = __builtin_amdgcn_sdot4((int)((w.y << 4) & M), (int)a1.y, acc, false);
        acc = __builtin_amdgcn_sdot4((int)((w.y << 2) & M), (int)a1.z, acc, false);
        acc = __builtin_amdgcn_sdot4((int)(w.y & M), (int)a1.w, acc, false);
        return acc;
    }
};

// Position of element k (0..31) of a block in activation order L.
template <int L>
__device__ __forceinline__ int act_pos(int k) {
    if (L == 0) return k;
    if (L == 1) return q8_perm_pos(k);
    return (k & ~15) + 4 * (k & 3) + ((k >> 2) & 3);
}

// Transposed wave reduction of V values per lane: after log2(V) halving
// butterflies every lane holds one partial of value index (lane >> (6 -
// log2 V)); the remaining butterflies finish that sum. Returns the full sum
// of that value index.
template <int V>
__device__ __forceinline__ double wave_reduce_tr(double* v, int lane) {
    static_assert(V >= 1 && V <= 64 && (V & (V - 1)) == 0, "V: a power of two up to 64");
    int step = 0;
#pragma unroll
    for (int h = V; h > 1; h >>= 1) {
        const int mask = 32 >> step;
        const bool upper = (lane & mask) != 0;
#pragma unroll
        for (int i = 0; i < h / 2; ++i) {
            // the two candidates pass through an empty asm, so the compiler
            // cannot turn the lane-dependent choice into an array access with
            // a per-lane index (which puts the array in scratch memory)
            double lo = v[i], hi = v[i + h / 2];
            asm volatile("" : "+v"(lo), "+v"(hi));
            const double keep = upper ? hi : lo;
            const double send = upper ? lo : hi;
            v[i] = keep + __shfl_xor(send, mask, 64);
        }
        ++step;
    }
    double s = v[0];
#pragma unroll
    for (int mask = 32 >> step; mask > 0; mask >>= 1) s += __shfl_xor(s, mask, 64);
    return s;
}

// Routing of T <= 4 tokens, computed redundantly by every workgroup of B.
struct Route {
    int idx[kMaxTok][16];
    int flat[kMaxEntries];      // idx in (token, k) order: entry t * K + k
    float w[kMaxTok][16];
    int n_ent;                  // T * K entries, ordered by (expert, token)
    int ent_e[kMaxEntries];     // expert of sorted entry
    int ent_t[kMaxEntries];     // token of sorted entry
    float ent_w[kMaxEntries];   // gate weight of sorted entry
    int slot_of[kMaxTok][17];   // slot of (t, k); k == K: shared
    int n_uniq;
    int u_e[kMaxEntries];       // unique experts, ascending
    int u_s0[kMaxEntries];      // first sorted entry (= slot) of each
    int u_n[kMaxEntries];       // tokens of each
    int u_w0[kMaxEntries];      // several tokens: first work unit of each (below)
};

// LDS scratch of the top-k, dead once the routing is done.
struct TopkScratch {
    unsigned long long ckey[kMaxTok][256];
    int ce[kMaxTok][256];
    double cs[kMaxTok][256];
    double ssel[kMaxTok][16];
};

// Total order on doubles (no NaN) as unsigned integers.
__device__ __forceinline__ unsigned long long order_key(double c) {
    const long long b = __double_as_longlong(c);
    return (b < 0) ? ~(unsigned long long)b : ((unsigned long long)b | 0x8000000000000000ull);
}

// The two largest of the values held by n aligned lanes (n a power of two,
// <= 64), merged with xor shuffles; every lane of the n ends with the pair.
__device__ __forceinline__ void top2_lanes(double& a, double& b, int n) {
    for (int o = 1; o < n; o <<= 1) {
        const double oa = __shfl_xor(a, o, 64), ob = __shfl_xor(b, o, 64);
        b = fmax(fmin(a, oa), fmax(b, ob));
        a = fmax(a, oa);
    }
}

// Cross-lane moves of 64-bit values without LDS: a DPP move (CTRL: quad
// permute, half-row or row mirror) or a read of one lane into all lanes.
template <int CTRL>
__device__ __forceinline__ unsigned long long dpp64(unsigned long long v) {
    const int lo = __builtin_amdgcn_mov_dpp((int)(unsigned)v, CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_mov_dpp((int)(unsigned)(v >> 32), CTRL, 0xF, 0xF, false);
    return ((unsigned long long)(unsigned)hi << 32) | (unsigned)lo;
}
__device__ __forceinline__ unsigned long long readlane64(unsigned long long v, int l) {
    const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)v, l);
    const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(v >> 32), l);
    return ((unsigned long long)hi << 32) | lo;
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E;  // quad permutes [1,0,3,2], [2,3,0,1]
constexpr int kDppRowMirror = 0x140, kDppHalfMirror = 0x141;

// Top-k of token t by one wave, which uses only row t of the scratch: idx,
// flat entries t K + k and gates w of token t. Lane L holds experts 4L ..
// 4L+3 (E <= 256). The smallest of the 32-expert group maxima (8 lanes per
// group) is found with lane shuffles; the experts at or above it are
// compacted into LDS with ballots and ranked by who is ahead (c descending,
// index ascending); the gates are summed in k order. All LDS traffic stays
// within the wave, whose LDS operations complete in program order. With ONE
// (a single token) the wave also fills the sorted entries and the expert list.
template <bool ONE>
__device__ __forceinline__ void topk_wave(const double* sig, const double* cval, int E, int K,
                                          int S, int norm, double rho, GroupSel gsel, Route& R,
                                          TopkScratch& Z, int t) {
    const int lane = threadIdx.x & 63;
    {
        unsigned long long key[4];
        double sv[4], cv[4];
        bool ok[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = 4 * lane + j;
            ok[j] = e < E;
            sv[j] = ok[j] ? sig[e] : 0.0;
            const double c = ok[j] ? cval[e] : 0.0;
            key[j] = ok[j] ? order_key(c) : 0ull;
            cv[j] = ok[j] ? c : -__builtin_inf();
        }
        // group-limited selection: the experts of dropped groups leave the race.
        // Groups of 4 lpg experts (lpg a power of two: whole lanes) take their
        // two largest c from lane shuffles, and the smallest second-largest c
        // of the kept groups (2 tg >= K experts at or above it) bounds the K-th
        // largest from below; other group sizes go through LDS.
        unsigned long long gthr = 0ull;
        if (gsel.ng > 1) {
            const int lpg = gsel.gs >> 2;
            if ((gsel.gs & 3) == 0 && !(lpg & (lpg - 1))) {
                double a = fmax(cv[0], cv[1]), b2 = fmin(cv[0], cv[1]);
#pragma unroll
                for (int j = 2; j < 4; ++j) {
                    b2 = fmax(b2, fmin(a, cv[j]));
                    a = fmax(a, cv[j]);
                }
                top2_lanes(a, b2, lpg);
                const int g = lane / lpg;
                const bool head = (lane & (lpg - 1)) == 0 && g < gsel.ng;
                const double sc = head ? a + b2 : -__builtin_inf();
                int rank = 0;
                for (int j = 0; j < gsel.ng; ++j) {
                    const double o = __shfl(sc, j * lpg, 64);
                    rank += (o > sc || (o == sc && j < g)) ? 1 : 0;
                }
                const bool kept = head && rank < gsel.tg;
                const unsigned long long keepl = __ballot(kept);
                double tb = kept ? b2 : __builtin_inf();
#pragma unroll
                for (int o = 1; o < 64; o <<= 1) tb = fmin(tb, __shfl_xor(tb, o, 64));
                if (2 * gsel.tg >= K) gthr = order_key(tb);
                if (!((keepl >> (lane & ~(lpg - 1))) & 1ull)) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        ok[j] = false;
                        key[j] = 0ull;
                    }
                }
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (ok[j]) Z.cs[t][4 * lane + j] = cv[j];  // free until the compaction
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                const unsigned long long keep = group_keep_mask(Z.cs[t], gsel);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (ok[j] && !((keep >> ((4 * lane + j) / gsel.gs)) & 1ull)) {
                        ok[j] = false;
                        key[j] = 0ull;
                    }
            }
        }
        // the smallest maximum of >= K non-empty expert groups bounds the K-th
        // largest key from below: 32-expert groups (8 lanes), else with groups
        // 8-expert groups (2 lanes)
        // the smallest maximum of >= K non-empty expert groups bounds the K-th
        // largest key from below: 32-expert groups (8 lanes), else with groups
        // 8-expert groups (2 lanes). Group maxima by DPP moves (quad permutes,
        // then the half-row mirror pairs the two quads of 8 lanes), the
        // minimum by the row mirror (two groups of a 16-lane row) and one read
        // of each row.
        const int G = (E + 31) >> 5, G8 = (E + 7) >> 3;
        unsigned long long thr = gthr;
        const unsigned long long m4 = max(max(key[0], key[1]), max(key[2], key[3]));
        const unsigned long long q2 = max(m4, dpp64<kDppXor1>(m4));  // 2-lane maxima
        if (thr == 0ull && G >= K) {
            unsigned long long gm = max(q2, dpp64<kDppXor2>(q2));
            gm = max(gm, dpp64<kDppHalfMirror>(gm));
            const bool live = (lane >> 3) < G && gm != 0ull;
            const int cnt = __popcll(__ballot(live && (lane & 7) == 0));
            unsigned long long v = live ? gm : ~0ull;  // no (eligible) experts in this group
            v = min(v, dpp64<kDppRowMirror>(v));
            v = min(min(readlane64(v, 0), readlane64(v, 16)), min(readlane64(v, 32), readlane64(v, 48)));
            if (cnt >= K) thr = v;
        }
        if (thr == 0ull && gsel.ng > 1 && G8 >= K) {
            const bool live = (lane >> 1) < G8 && q2 != 0ull;
            const int cnt = __popcll(__ballot(live && (lane & 1) == 0));
            unsigned long long v = live ? q2 : ~0ull;
            v = min(v, dpp64<kDppXor2>(v));
            v = min(v, dpp64<kDppHalfMirror>(v));
            v = min(v, dpp64<kDppRowMirror>(v));
            v = min(min(readlane64(v, 0), readlane64(v, 16)), min(readlane64(v, 32), readlane64(v, 48)));
            if (cnt >= K) thr = v;
        }
        // candidates (keys at or above the threshold) compacted into LDS, then
        // each candidate's position = the number of candidates ahead of it (c
        // descending, index ascending)
        int base = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const bool c = ok[j] && key[j] >= thr;
            const unsigned long long bal = __ballot(c);
            if (c) {
                const int p = base + __popcll(bal & ((1ull << lane) - 1ull));
                Z.ckey[t][p] = key[j];
                Z.ce[t][p] = 4 * lane + j;
                Z.cs[t][p] = sv[j];
            }
            base += __popcll(bal);
        }
        const int m = base;
        if (m <= 64) {
            // one candidate per lane; the others broadcast from their lanes
            const bool has = lane < m;
            const unsigned long long ki = has ? Z.ckey[t][lane] : 0ull;
            const int ei = has ? Z.ce[t][lane] : 0x7fffffff;
            const double si = has ? Z.cs[t][lane] : 0.0;
            int rank = 0;
            for (int j = 0; j < m; ++j) {  // uniform
                const unsigned long long kj = readlane64(ki, j);
                const int ej = __builtin_amdgcn_readlane(ei, j);
                rank += (kj > ki || (kj == ki && ej < ei)) ? 1 : 0;
            }
            const bool sel = has && rank < K;
            // gate values summed in position order (k ascending)
            double sum = 0.0;
            for (int k = 0; k < K; ++k) {
                const int src = __builtin_ctzll(__ballot(sel && rank == k));
                const long long sb = (long long)readlane64((unsigned long long)__double_as_longlong(si), src);
                sum += __longlong_as_double(sb);
            }
            // the K experts are distinct: slot = number of chosen experts below
            const unsigned long long selm = __ballot(sel);
            int slot = 0;
            for (unsigned long long mm = selm; mm; mm &= mm - 1ull) {  // uniform, K steps
                const int ej = __builtin_amdgcn_readlane(ei, __builtin_ctzll(mm));
                slot += ej < ei ? 1 : 0;
            }
            if (sel) {
                double v = si;
                if (norm) v = v / sum;
                v = v * rho;
                const float w = (float)v;
                R.idx[t][rank] = ei;
                R.flat[t * K + rank] = ei;
                R.w[t][rank] = w;
                if (ONE) {  // one token: sorted entries = experts ascending
                    R.ent_e[slot] = ei;
                    R.ent_t[slot] = 0;
                    R.ent_w[slot] = w;
                    R.slot_of[0][rank] = slot;
                    R.u_e[slot] = ei;
                    R.u_s0[slot] = slot;
                    R.u_n[slot] = 1;
                }
            }
        } else {
            for (int i = lane; i < m; i += 64) {
                const unsigned long long ki = Z.ckey[t][i];
                const int ei = Z.ce[t][i];
                int rank = 0;
                for (int j0 = 0; j0 < m; j0 += 8) {
                    unsigned long long kj[8];
                    int ej[8];
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        const int j = min(j0 + u, m - 1);
                        kj[u] = Z.ckey[t][j];
                        ej[u] = Z.ce[t][j];
                    }
#pragma unroll
                    for (int u = 0; u < 8; ++u)
                        rank += (j0 + u < m && (kj[u] > ki || (kj[u] == ki && ej[u] < ei))) ? 1 : 0;
                }
                if (rank < K) {
                    R.idx[t][rank] = ei;
                    R.flat[t * K + rank] = ei;
                    Z.ssel[t][rank] = Z.cs[t][i];
                }
            }
            if (lane < K) {
                double ss[16];
                int ix[16];
#pragma unroll
                for (int kk = 0; kk < 16; ++kk) {
                    ss[kk] = Z.ssel[t][min(kk, K - 1)];
                    ix[kk] = R.idx[t][min(kk, K - 1)];
                }
                double sum = 0.0;
#pragma unroll
                for (int kk = 0; kk < 16; ++kk)
                    if (kk < K) sum += ss[kk];  // k ascending
                double v = Z.ssel[t][lane];
                if (norm) v = v / sum;
                v = v * rho;
                const float w = (float)v;
                R.w[t][lane] = w;
                if (ONE) {
                    // the K experts are distinct: slot = number of chosen experts below
                    const int e = R.idx[t][lane];
                    int slot = 0;
#pragma unroll
                    for (int kk = 0; kk < 16; ++kk)
                        if (kk < K && ix[kk] < e) ++slot;
                    R.ent_e[slot] = e;
                    R.ent_t[slot] = 0;
                    R.ent_w[slot] = w;
                    R.slot_of[0][lane] = slot;
                    R.u_e[slot] = e;
                    R.u_s0[slot] = slot;
                    R.u_n[slot] = 1;
                }
            }
        }
        if (ONE && lane == 0) {
            R.n_uniq = K;
            if (S) R.slot_of[0][K] = K;
        }
    }
}

// Routing of one token by wave 0 (the others wait at one barrier).
__device__ __forceinline__ void route_one(const double* sig, const double* cval, int E, int K,
                                          int S, int norm, double rho, GroupSel gsel, Route& R,
                                          TopkScratch& Z) {
    if (threadIdx.x < 64) topk_wave<true>(sig, cval, E, K, S, norm, rho, gsel, R, Z, 0);
    __syncthreads();
}

// Fills R (in LDS) for T <= 4 tokens; called by the whole workgroup.
__device__ __forceinline__ void route_small(const double* sig, const double* cval, int T, int E, int K, int S,
                            int norm, double rho, GroupSel gsel, Route& R, TopkScratch& Z) {
    // wave t routes token t (T <= 4 waves)
    const int wv = threadIdx.x >> 6;
    if (wv < T)
        topk_wave<false>(sig + (int64_t)wv * E, cval + (int64_t)wv * E, E, K, S, norm, rho, gsel,
                         R, Z, wv);
    __syncthreads();
    // Bucketing by wave 0: entry i = t K + k ((token, k) order, T K <= 64)
    // takes its sorted position (expert ascending, then token) from a bitonic
    // sort of the keys (e, t, k) over the wave's 64 lanes, absent entries
    // last, so that lane p ends up holding the p-th entry. An entry opens its
    // expert's run when the entry before it has another expert; the run's
    // list index is the number of runs opened before it (a ballot). No loop
    // over the entries.
    if (threadIdx.x < 64) {
        const int n = T * K;
        const int lane = threadIdx.x;
        unsigned key = 0xffffffffu;  // E <= 256, T <= 4, K <= 16: 14-bit keys
        if (lane < n) {
            const int t = lane / K, k = lane - t * K;
            key = ((unsigned)R.flat[lane] << 6) | ((unsigned)t << 4) | (unsigned)k;
        }
#pragma unroll
        for (int size = 2; size <= 64; size <<= 1)
#pragma unroll
            for (int stride = size >> 1; stride > 0; stride >>= 1) {
                const unsigned other = __shfl_xor(key, stride, 64);
                const bool keep_min = ((lane & stride) == 0) == ((lane & size) == 0);
                key = keep_min ? min(key, other) : max(key, other);
            }
        const bool has = lane < n;
        const int e = (int)(key >> 6), t = (int)((key >> 4) & 3), k = (int)(key & 15);
        const unsigned prev = __shfl_up(key, 1, 64);
        const bool first = has && (lane == 0 || (prev >> 6) != (key >> 6));
        const unsigned long long runs = __ballot(first);
        const int u = __popcll(runs & ((1ull << lane) - 1ull));
        const unsigned long long later = runs & ~((2ull << lane) - 1ull);
        const int next = later ? __builtin_ctzll(later) : n;  // where the next run opens
        if (has) {
            R.ent_e[lane] = e;
            R.ent_t[lane] = t;
            R.ent_w[lane] = R.w[t][k];
            R.slot_of[t][k] = lane;
            if (first) {
                R.u_e[u] = e;
                R.u_s0[u] = lane;
                R.u_n[u] = next - lane;
            }
        }
        if (lane == 0) R.n_uniq = __popcll(runs);
        if (lane < T && S) R.slot_of[lane][K] = n + lane;
        // gate/up work units (k_dec_gateup): an expert with one token takes
        // one unit, one with several (more arithmetic per weight byte) two
        const bool multi = first && next - lane > 1;
        const int mb = __popcll(__ballot(multi) & ((1ull << lane) - 1ull));
        if (first) R.u_w0[u] = u + mb;
    }
    __syncthreads();
}



// Gate/up GEMV for one expert, NT token slots and 32 intermediate rows
// (h-block hb), then SwiGLU and Q8_0(h) into qh/dh at slots slot0 + i.
// Activations: Q8_0 codes of x in the width's order (qx) and block scales
// (dx), rows of token tok[i]. Four waves; wave w owns h-rows w, w+4, ...,
// w+28, taken HR per step (HR gate + HR up rows), so the four waves read
// 4 HR consecutive rows of each matrix at a time; the loop is fully unrolled
// and every load unconditional (lanes past the last block read a clamped
// address and see zero activations), with two steps' loads in flight.
template <int NT, int NBJ, bool TAP, int BITS>
__device__ __forceinline__ void gateup_block(const DecArgs& a, int e, int hb, int n,
                                             const int* tok, int slot0, float (*hbuf)[32]) {
    typedef DW<BITS> F;
    typedef typename F::blk Blk;
    constexpr int HR = F::HR, RQ = 2 * HR, NS = 8 / HR;  // rows per step, steps
    const int H = a.H, I = a.I, BH = H >> 5;
    const int64_t rowb = (int64_t)H * BITS / 8;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint8_t* gate = a.eq + (int64_t)e * a.blob_q;
    const uint8_t* up = gate + (int64_t)I * rowb;
    const float* gs = a.es + (int64_t)e * a.blob_s;
    const float* us = gs + I;
    const int r0 = hb * 32 + wave;  // rows r0 + 4k, k = 0..7
    int boff[NBJ];
#pragma unroll
    for (int j = 0; j < NBJ; ++j) boff[j] = min(lane + 64 * j, BH - 1) * (4 * BITS);
    Blk wb[2][RQ][NBJ];
    // step p: gate rows r0 + 4 (HR p + q), q < HR, then the same up rows
    auto load_pair = [&](int p, Blk (&dst)[RQ][NBJ]) {
#pragma unroll
        for (int q = 0; q < RQ; ++q) {
            const int r = r0 + 4 * (HR * p + (q % HR));
            const uint8_t* row = ((q < HR) ? gate : up) + (int64_t)r * rowb;
#pragma unroll
            for (int j = 0; j < NBJ; ++j) dst[q][j] = F::load(row + boff[j]);
        }
    };
    load_pair(0, wb[0]);
    if (NS > 1) load_pair(1, wb[1]);
    // row scales, one per lane (lane k & 7 holds row r0 + 4 (k & 7))
    const float gsl = gs[r0 + 4 * (lane & 7)];
    const float usl = us[r0 + 4 * (lane & 7)];
    uint4 xa[NT][NBJ][2];
    double xd[NT][NBJ];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        const int t = tok[(i < n) ? i : 0];
#pragma unroll
        for (int j = 0; j < NBJ; ++j) {
            const int b = lane + 64 * j;
            const bool ok = i < n && b < BH;
            const int bb = min(b, BH - 1);
            const uint4* p = reinterpret_cast<const uint4*>(a.qx + (int64_t)t * H + bb * 32);
            const uint4 a0 = p[0], a1 = p[1];
            const float d = a.dx[(int64_t)t * BH + bb];
            xa[i][j][0] = ok ? a0 : make_uint4(0, 0, 0, 0);
            xa[i][j][1] = ok ? a1 : make_uint4(0, 0, 0, 0);
            xd[i][j] = ok ? (double)d * F::kInv : 0.0;  // undo the factor of the codes
        }
    }
    constexpr int V = RQ * NT;  // values per step, a power of two
    constexpr int kShift = 6 - ((V >= 32) ? 5 : (V >= 16) ? 4 : (V >= 8) ? 3 : (V >= 4) ? 2 : 1);
#pragma unroll
    for (int p = 0; p < NS; ++p) {
        if (p >= 1 && p < NS - 1) load_pair(p + 1, wb[(p + 1) & 1]);
        // keep the next step's loads issued ahead of this step's arithmetic
        __builtin_amdgcn_sched_barrier(0);
        const Blk (&wc)[RQ][NBJ] = wb[p & 1];
        // values ordered (row, token): rows q < HR are the gate rows of step p,
        // the others the up rows
        double v[V];
#pragma unroll
        for (int q = 0; q < RQ; ++q)
#pragma unroll
            for (int i = 0; i < NT; ++i) {
                double acc = 0.0;
#pragma unroll
                for (int j = 0; j < NBJ; ++j) {
                    const int dq = F::dot(wc[q][j], xa[i][j][0], xa[i][j][1]);
                    acc += xd[i][j] * (double)dq;
                    if (TAP && q < HR) {
                        const int r = r0 + 4 * (HR * p + q), b = lane + 64 * j;
                        if (i < n && b < BH && (r % a.tap_stride) == 0)
                            a.tap[((int64_t)(slot0 + i) * a.tap_rows + r / a.tap_stride) * BH + b] =
                                dq / F::kDiv;
                    }
                }
                v[q * NT + i] = acc;
            }
        const double sum = wave_reduce_tr<V>(v, lane);
        const double other = __shfl_xor(sum, 32, 64);  // up value for gate lanes
        const int vi = lane >> kShift;   // value index held by this lane
        const int kq = HR * p + ((vi < HR * NT) ? vi / NT : 0);
        const float gsk = __shfl(gsl, kq, 64), usk = __shfl(usl, kq, 64);
        if (vi < HR * NT && lane == (vi << kShift)) {
            const int q = vi / NT, i = vi - q * NT;   // q < HR: row r0 + 4(HR p + q)
            if (i < n) {
                const float g = (float)((double)gsk * sum);
                const float u = (float)((double)usk * other);
                hbuf[i][wave + 4 * (HR * p + q)] = swiglu_f32(g, u);
            }
        }
    }
    __syncthreads();
    if (threadIdx.x < NT * 32) {
        const int i = threadIdx.x >> 5, k = threadIdx.x & 31;
        const float val = (i < n) ? hbuf[i][k] : 0.0f;
        float amax = fabsf(val);
#pragma unroll
        for (int o = 16; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 32));
        const float dd = amax / 127.0f;
        const int c = q8_code(val, dd);
        if (i < n) {
            a.qh[(int64_t)(slot0 + i) * I + hb * 32 + act_pos<F::kL>(k)] = (int8_t)c;
            if (k == 0) a.dh[(int64_t)(slot0 + i) * (I >> 5) + hb] = dd;
        }
    }
}

// As gateup_block for experts with several tokens: the Q8_0 codes and
// scales of all T tokens are staged in LDS (xs: T rows of H bytes, xds: T
// rows of H/32 scales); the expert's n tokens are rows tok[0..n) and are read
// per step, one token at a time, so the activations do not occupy registers
// for the whole kernel.
template <int NT, int NBJ, bool TAP, int BITS>
__device__ __forceinline__ void gateup_block_lds(const DecArgs& a, int e, int hb, int n,
                                                 const int* tok, int slot0, const uint8_t* xs,
                                                 const float* xds, float (*hbuf)[32]) {
    typedef DW<BITS> F;
    typedef typename F::blk Blk;
    // half the one-token step: two steps of weight loads in flight stay within
    // the registers of three workgroups per CU
    constexpr int HR = (F::HR > 1) ? F::HR / 2 : 1, RQ = 2 * HR, NS = 8 / HR;
    const int H = a.H, I = a.I, BH = H >> 5;
    const int64_t rowb = (int64_t)H * BITS / 8;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint8_t* gate = a.eq + (int64_t)e * a.blob_q;
    const uint8_t* up = gate + (int64_t)I * rowb;
    const float* gs = a.es + (int64_t)e * a.blob_s;
    const float* us = gs + I;
    const int r0 = hb * 32 + wave;  // rows r0 + 4k, k = 0..7
    int boff[NBJ];
#pragma unroll
    for (int j = 0; j < NBJ; ++j) boff[j] = min(lane + 64 * j, BH - 1) * (4 * BITS);
    Blk wb[2][RQ][NBJ];
    auto load_pair = [&](int p, Blk (&dst)[RQ][NBJ]) {
#pragma unroll
        for (int q = 0; q < RQ; ++q) {
            const int r = r0 + 4 * (HR * p + (q % HR));
            const uint8_t* row = ((q < HR) ? gate : up) + (int64_t)r * rowb;
#pragma unroll
            for (int j = 0; j < NBJ; ++j) dst[q][j] = F::load(row + boff[j]);
        }
    };
    load_pair(0, wb[0]);
    if (NS > 1) load_pair(1, wb[1]);
    const float gsl = gs[r0 + 4 * (lane & 7)];
    const float usl = us[r0 + 4 * (lane & 7)];
    int tk[NT];  // staged row of the i-th token
#pragma unroll
    for (int i = 0; i < NT; ++i) tk[i] = __builtin_amdgcn_readfirstlane(tok[min(i, n - 1)]);
    constexpr int V = RQ * NT;  // values per step, a power of two
    constexpr int kShift = 6 - ((V >= 32) ? 5 : (V >= 16) ? 4 : (V >= 8) ? 3 : (V >= 4) ? 2 : 1);
#pragma unroll
    for (int p = 0; p < NS; ++p) {
        if (p >= 1 && p < NS - 1) load_pair(p + 1, wb[(p + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
        const Blk (&wc)[RQ][NBJ] = wb[p & 1];
        double v[V];
#pragma unroll
        for (int i = 0; i < NT; ++i) {
            double acc[RQ];
#pragma unroll
            for (int q = 0; q < RQ; ++q) acc[q] = 0.0;
            if (i < n) {
#pragma unroll
                for (int j = 0; j < NBJ; ++j) {
                    const int b = lane + 64 * j, bb = min(b, BH - 1);
                    const uint4* px = reinterpret_cast<const uint4*>(xs + tk[i] * H + bb * 32);
                    const uint4 x0 = px[0], x1 = px[1];
                    const double xd = (b < BH) ? (double)xds[tk[i] * BH + bb] * F::kInv : 0.0;
#pragma unroll
                    for (int q = 0; q < RQ; ++q) {
                        const int dq = F::dot(wc[q][j], x0, x1);
                        acc[q] += xd * (double)dq;
                        if (TAP && q < HR) {
                            const int r = r0 + 4 * (HR * p + q);
                            if (b < BH && (r % a.tap_stride) == 0)
                                a.tap[((int64_t)(slot0 + i) * a.tap_rows + r / a.tap_stride) * BH +
                                      b] = dq / F::kDiv;
                        }
                    }
                }
            }
#pragma unroll
            for (int q = 0; q < RQ; ++q) v[q * NT + i] = acc[q];
        }
        const double sum = wave_reduce_tr<V>(v, lane);
        const double other = __shfl_xor(sum, 32, 64);
        const int vi = lane >> kShift;
        const int kq = HR * p + ((vi < HR * NT) ? vi / NT : 0);
        const float gsk = __shfl(gsl, kq, 64), usk = __shfl(usl, kq, 64);
        if (vi < HR * NT && lane == (vi << kShift)) {
            const int q = vi / NT, i = vi - q * NT;
            if (i < n) {
                const float g = (float)((double)gsk * sum);
                const float u = (float)((double)usk * other);
                hbuf[i][wave + 4 * (HR * p + q)] = swiglu_f32(g, u);
            }
        }
    }
    __syncthreads();
    if (threadIdx.x < NT * 32) {
        const int i = threadIdx.x >> 5, k = threadIdx.x & 31;
        const float val = (i < n) ? hbuf[i][k] : 0.0f;
        float amax = fabsf(val);
#pragma unroll
        for (int o = 16; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 32));
        const float dd = amax / 127.0f;
        const int c = q8_code(val, dd);
        if (i < n) {
            a.qh[(int64_t)(slot0 + i) * I + hb * 32 + act_pos<F::kL>(k)] = (int8_t)c;
            if (k == 0) a.dh[(int64_t)(slot0 + i) * (I >> 5) + hb] = dd;
        }
    }
    __syncthreads();  // hbuf is reused by the workgroup's next h-block
}

// Copies the Q8_0 codes and scales of all T tokens into LDS rows xs[t]
// (H bytes) and xds[t] (H/32 scales), by threads tid0 .. tid0 + nt - 1.
__device__ __forceinline__ void stage_all_tokens(const DecArgs& a, uint8_t* xs, float* xds,
                                                 int tid0, int nt) {
    const int V = a.H >> 4, BH = a.H >> 5;  // 16-byte pieces and scales per row
    const int nq = a.T * V, nd = a.T * BH;   // rows are contiguous on both sides
    const int i0 = (int)threadIdx.x - tid0;
    for (int x = i0; x < nq; x += nt)
        reinterpret_cast<v4u*>(xs)[x] = reinterpret_cast<const v4u*>(a.qx)[x];
    for (int x = i0; x < nd; x += nt) xds[x] = a.dx[x];
}

// Publishes the routing computed in R (one workgroup of B) for C, the taps
// and the workspace layout.
__device__ void publish_route(const DecArgs& a, const Route& R) {
    const int T = a.T, K = a.K, E = a.E, S = a.S;
    const int n = T * K;
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
        const int t = i / K, k = i - t * K;
        a.idx[i] = R.idx[t][k];
        a.wts[i] = R.w[t][k];
        a.slot_tok[i] = R.ent_t[i];
        a.slot_of[t * (K + S) + k] = R.slot_of[t][k];
        reinterpret_cast<float*>(a.uinfo + kUinfoW)[i] = R.ent_w[i];
    }
    for (int t = threadIdx.x; t < T; t += blockDim.x)
        if (S) {
            a.slot_of[t * (K + S) + K] = n + t;
            a.slot_tok[n + t] = t;
        }
    for (int e = threadIdx.x; e < E + S; e += blockDim.x) {
        int cnt = (e < E) ? 0 : T, before = 0;
        for (int v = 0; v < R.n_uniq; ++v) {
            if (R.u_e[v] == e) cnt = R.u_n[v];
            if (R.u_e[v] < e) before += R.u_n[v];
        }
        a.counts[e] = cnt;
        a.offs[e] = (e < E) ? before : n;
    }
    if (threadIdx.x == 0) a.offs[E + S] = n + S * T;
    for (int v = threadIdx.x; v < R.n_uniq; v += blockDim.x) {
        a.uinfo[1 + 3 * v] = R.u_e[v];
        a.uinfo[2 + 3 * v] = R.u_s0[v];
        a.uinfo[3 + 3 * v] = R.u_n[v];
    }
    if (threadIdx.x == 0) a.uinfo[0] = R.n_uniq;
}

// A: router rows (one workgroup per expert) and Q8_0(x): workgroup e also
// quantises blocks 8e .. 8e+7 of the T x H/32 activation blocks (half a
// wave per block, lane k holding element k), while its router row loads are
// in flight.
template <int NT, int BITS>
__global__ __launch_bounds__(256) void k_dec_router(DecArgs a) {
    __shared__ double red[NT][4];
    const int e = blockIdx.x;  // grid: max(E, blocks / 8) workgroups
    const int T = a.T, H = a.H;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const bool router = e < a.E;
    const float* wrow = a.wr + (int64_t)min(e, a.E - 1) * H;
    constexpr int kIt = 6;  // H <= 6144 on this path: 6144 / (256 threads x 4)
    float4 wv[kIt];
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
        const int h = min((int)threadIdx.x * 4 + 1024 * it, H - 4);
        wv[it] = *reinterpret_cast<const float4*>(wrow + h);
    }
    // every token's activations requested with the router row (clamped,
    // unconditional loads), before any arithmetic
    float4 xv[NT][kIt];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int it = 0; it < kIt; ++it) {
            const int h = min((int)threadIdx.x * 4 + 1024 * it, H - 4);
            xv[t][it] = *reinterpret_cast<const float4*>(a.x + (int64_t)min(t, T - 1) * H + h);
        }
    {
        const int blk = e * 8 + (int)(threadIdx.x >> 5);
        const int k = threadIdx.x & 31;
        if (blk < T * (H >> 5)) {
            const float v = a.x[(int64_t)blk * 32 + k];
            float amax = fabsf(v);
#pragma unroll
            for (int o = 16; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 32));
            const float d = amax / 127.0f;
            a.qx[(int64_t)blk * 32 + act_pos<DW<BITS>::kL>(k)] = (int8_t)q8_code(v, d);
            if (k == 0) a.dx[blk] = d;
        }
    }
    double acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = 0.0;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        if (t < T) {
#pragma unroll
            for (int it = 0; it < kIt; ++it) {
                const int h = threadIdx.x * 4 + 1024 * it;
                if (h < H) {
                    acc[t] += (double)xv[t][it].x * (double)wv[it].x;
                    acc[t] += (double)xv[t][it].y * (double)wv[it].y;
                    acc[t] += (double)xv[t][it].z * (double)wv[it].z;
                    acc[t] += (double)xv[t][it].w * (double)wv[it].w;
                }
            }
        }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const double sm = wave_sum_f64(acc[t]);
        if (lane == 0) red[t][wave] = sm;
    }
    __syncthreads();
    if (router && (int)threadIdx.x < T) {
        const double* r = red[threadIdx.x];
        const double l = (r[0] + r[1]) + (r[2] + r[3]);
        const int64_t i = (int64_t)threadIdx.x * a.E + e;
        a.logits[i] = l;
        // the sigmoid and the selection score once per expert here, not in
        // every gate/up workgroup
        const double sg = 1.0 / (1.0 + exp(-l));
        a.sig[i] = sg;
        a.cval[i] = sg + (double)a.bias[e];
    }
}

// Sigmoid, correction bias and top-k for the many-token path (E <= 256,
// K <= 16): one wave per token runs topk_wave, the few-token selection
// (group maxima bound the K-th score from below; the experts at or above it
// are compacted and ranked), on its token's s and c staged in LDS. It picks
// the same experts in the same order, and sums and scales the same gates, as
// K rounds of a wave arg-max would.
__global__ __launch_bounds__(256) void k_topk_wave(const double* __restrict__ logits,
                                                   const float* __restrict__ bias, int T, int E,
                                                   int K, int norm, double rho, GroupSel gsel,
                                                   int32_t* __restrict__ idx,
                                                   float* __restrict__ wout) {
    __shared__ TopkScratch Z;
    __shared__ Route R;
    __shared__ double sc[2][kMaxTok][256];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int t = blockIdx.x * 4 + wave;
    if (t >= T) return;  // the whole wave; no workgroup barrier follows
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = lane + 64 * j;
        if (e < E) {
            const double l = logits[(int64_t)t * E + e];
            const double sg = 1.0 / (1.0 + exp(-l));
            sc[0][wave][e] = sg;
            sc[1][wave][e] = sg + (double)bias[e];
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    topk_wave<false>(sc[0][wave], sc[1][wave], E, K, 0, norm, rho, gsel, R, Z, wave);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (lane < K) {
        idx[(int64_t)t * K + lane] = R.idx[wave][lane];
        wout[(int64_t)t * K + lane] = R.w[wave][lane];
    }
}

// B: blocks [0, S*nrb) shared-expert h-blocks, then (u, hb) for the u-th
// expert in use (u < min(E, T*K)); block (u = 0, hb = 0) publishes routing.
template <int NT, int NBJ, bool TAP, int BITS>
__global__ __launch_bounds__(256) void k_dec_gateup(DecArgs a) {
    // several tokens: every token's Q8_0(x) staged in LDS beside the top-k
    // scratch, so that a wave with no token to route can stage it meanwhile;
    // H <= 6144 on this path
    constexpr int kAct = (NT > 1) ? NT * 6144 + NT * 192 * 4 : 16;
    __shared__ TopkScratch Z;
    __shared__ __align__(16) uint8_t act[kAct];
    __shared__ Route R;
    __shared__ float hbuf[NT][32];
    __shared__ int s_tok[NT];
    uint8_t* xs = act;
    float* xds = reinterpret_cast<float*>(act + NT * a.H);
    // One token: a workgroup per (expert, h-block of 32 rows). Several
    // tokens: work units of nrb / 2 workgroups; an expert holding one token
    // takes one unit (two h-blocks per workgroup, so fewer workgroups redo
    // the routing), one holding several (and the shared expert) takes two
    // (one h-block per workgroup: its steps carry the arithmetic of every
    // token and would otherwise make the tail). The grid covers the most
    // units a routing can produce (one per entry T K, two per expert).
    const int nrb = a.I >> 5;
    const int nw = (NT > 1) ? nrb / 2 : nrb;  // workgroups per unit / per expert
    int b = blockIdx.x;
    if (NT == 1) {
        if (a.S) {
            if (b < nrb) {
                if (threadIdx.x == 0) s_tok[0] = 0;
                __syncthreads();
                gateup_block<NT, NBJ, TAP, BITS>(a, a.E, b, a.T, s_tok, a.T * a.K, hbuf);
                return;
            }
            b -= nrb;
        }
        // routing latency sits on the path to this workgroup's first weight
        // load: the routing wave wins issue slots over co-resident streaming
        // waves
        __builtin_amdgcn_s_setprio(3);
        route_one(a.sig, a.cval, a.E, a.K, a.S, a.norm, a.rho, a.gsel, R, Z);
        __builtin_amdgcn_s_setprio(0);
        if (b == 0) publish_route(a, R);
        const int u = b / nw, hw = b - u * nw;
        if (u >= R.n_uniq) return;
        const int e = __builtin_amdgcn_readfirstlane(R.u_e[u]);
        const int s0 = __builtin_amdgcn_readfirstlane(R.u_s0[u]);
        const int n = __builtin_amdgcn_readfirstlane(R.u_n[u]);
        gateup_block<NT, NBJ, TAP, BITS>(a, e, hw, n, &R.ent_t[s0], s0, hbuf);
        return;
    }
    // several tokens: the work of this workgroup as (expert, first h-block,
    // h-blocks, tokens, their slots); one call site below
    int e, hb0, nhb, n, s0;
    const int* tok;
    bool staged = false;
    if (a.S && b < nrb) {
        if ((int)threadIdx.x < NT) s_tok[threadIdx.x] = min((int)threadIdx.x, a.T - 1);
        e = a.E;
        hb0 = b;
        nhb = 1;
        n = a.T;
        s0 = a.T * a.K;
        tok = s_tok;
    } else {
        if (a.S) b -= nrb;
        // with fewer than four tokens the last wave, which routes none, stages
        // the activations while the others route
        staged = a.T < 4;
        if (staged && threadIdx.x >= 192) stage_all_tokens(a, xs, xds, 192, 64);
        __builtin_amdgcn_s_setprio(3);
        route_small(a.sig, a.cval, a.T, a.E, a.K, a.S, a.norm, a.rho, a.gsel, R, Z);
        __builtin_amdgcn_s_setprio(0);
        if (b == 0) publish_route(a, R);
        // the expert whose units hold unit b / nw: lane v tests expert v (every
        // wave computes the same ballot)
        const int unit = b / nw, hw = b - unit * nw;
        const int lane = threadIdx.x & 63;
        const int nu = R.n_uniq;
        const int w0 = R.u_w0[min(lane, nu - 1)], nv = R.u_n[min(lane, nu - 1)];
        const unsigned long long hm =
            __ballot(lane < nu && unit >= w0 && unit < w0 + (nv > 1 ? 2 : 1));
        if (hm == 0ull) return;  // no expert: nothing to do
        const int u = __builtin_ctzll(hm);
        e = __builtin_amdgcn_readfirstlane(R.u_e[u]);
        s0 = __builtin_amdgcn_readfirstlane(R.u_s0[u]);
        n = __builtin_amdgcn_readfirstlane(R.u_n[u]);
        const int uw0 = __builtin_amdgcn_readfirstlane(R.u_w0[u]);
        hb0 = (n > 1) ? (unit - uw0) * nw + hw : 2 * hw;
        nhb = (n > 1) ? 1 : 2;
        tok = &R.ent_t[s0];
    }
    if (!staged) {
        stage_all_tokens(a, xs, xds, 0, 256);
        __syncthreads();
    }
#pragma unroll 1
    for (int h = 0; h < nhb; ++h)
        gateup_block_lds<NT, NBJ, TAP, BITS>(a, e, hb0 + h, n, tok, s0, xs, xds, hbuf);
}

// C: down projection of every expert in use and the weighted combine.
// Workgroup = 4 waves x RPW rows; lane l owns block l (+64 j) of a down row.
// Experts are taken NB at a time: all their rows and activation blocks are
// requested before any is used (unconditional loads, clamped indices), then
// reduced. Each wave accumulates its rows' combine in LDS (fp64), in
// ascending expert order with the shared expert last.
template <int NT, int NBJ, int RPW, int NB, int BITS>
__global__ __launch_bounds__(256) void k_dec_down(DecArgs a) {
    typedef DW<BITS> F;
    typedef typename F::blk Blk;
    __shared__ int s_e[kMaxEntries], s_s0[kMaxEntries], s_n[kMaxEntries];
    __shared__ float s_w[kMaxEntries + kMaxTok];
    __shared__ int s_t[kMaxEntries + kMaxTok];
    __shared__ double s_acc[4 * RPW][NT];
    const int T = a.T, K = a.K, E = a.E, S = a.S, H = a.H, I = a.I;
    const int BI = I >> 5;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n_ent = T * K;
    const int c0 = blockIdx.x * (4 * RPW) + wave * RPW;
    int bcl[NBJ];
#pragma unroll
    for (int j = 0; j < NBJ; ++j) bcl[j] = min(lane + 64 * j, BI - 1);
    constexpr int V = RPW * NT;
    constexpr int kLog = (V >= 16) ? 4 : (V >= 8) ? 3 : (V >= 4) ? 2 : (V >= 2) ? 1 : 0;
    constexpr int kShift = 6 - kLog;
    // one expert's operands for this wave's rows: weights, Q8_0(h) of its
    // tokens, row scales
    struct Operands {
        Blk w[RPW][NBJ];
        uint4 ha[NT][NBJ][2];
        float hdf[NT][NBJ];
        float dsv[RPW];
    };
    const int64_t rowb = (int64_t)I * BITS / 8;  // bytes per down row
    auto load_w = [&](int ev, Operands& o) {
        const uint8_t* down = a.eq + (int64_t)ev * a.blob_q + 2 * (int64_t)H * rowb;
#pragma unroll
        for (int r = 0; r < RPW; ++r)
#pragma unroll
            for (int j = 0; j < NBJ; ++j)
                o.w[r][j] = F::load(down + (int64_t)(c0 + r) * rowb + bcl[j] * (4 * BITS));
    };
    auto load_h = [&](int ev, int s0, int n, Operands& o) {
        const float* ds = a.es + (int64_t)ev * a.blob_s + 2 * I;
#pragma unroll
        for (int r = 0; r < RPW; ++r) o.dsv[r] = ds[c0 + r];
#pragma unroll
        for (int i = 0; i < NT; ++i) {
            const int sl = s0 + min(i, n - 1);
#pragma unroll
            for (int j = 0; j < NBJ; ++j) {
                const uint4* p = reinterpret_cast<const uint4*>(a.qh + (int64_t)sl * I + bcl[j] * 32);
                o.ha[i][j][0] = p[0];
                o.ha[i][j][1] = p[1];
                o.hdf[i][j] = a.dh[(int64_t)sl * BI + bcl[j]];
            }
        }
    };
    // y_e of this wave's rows for the n tokens of one expert, added with the
    // slot weights (callers go in ascending expert order, the shared expert
    // last): into s_acc, or with one token into racc, a register of the lane
    // that holds row r's value (no LDS round trip in the chain of experts)
    double racc = 0.0;
    auto compute = [&](const Operands& o, int s0, int n) {
        double vals[V];
#pragma unroll
        for (int r = 0; r < RPW; ++r)
#pragma unroll
            for (int i = 0; i < NT; ++i) {
                double p = 0.0;
                if (i < n) {  // n is wave-uniform: no dot products for absent tokens
#pragma unroll
                    for (int j = 0; j < NBJ; ++j) {
                        const bool ok = lane + 64 * j < BI;
                        const double hd = ok ? (double)o.hdf[i][j] * F::kInv : 0.0;
                        p += hd * (double)F::dot(o.w[r][j], o.ha[i][j][0], o.ha[i][j][1]);
                    }
                }
                vals[r * NT + i] = p;
            }
        const double sum = wave_reduce_tr<V>(vals, lane);
        const int vi = lane >> kShift;
        if (lane == (vi << kShift)) {
            const int r = vi / NT, i = vi - r * NT;
            if (i < n) {
                float dsr = o.dsv[0];
#pragma unroll
                for (int rr = 1; rr < RPW; ++rr)
                    if (r == rr) dsr = o.dsv[rr];
                const float yv = (float)((double)dsr * sum);
                if constexpr (NT == 1)
                    racc += (double)s_w[s0] * (double)yv;
                else
                    s_acc[wave * RPW + r][s_t[s0 + i]] += (double)s_w[s0 + i] * (double)yv;
            }
        }
    };
    // The published route (routed experts in use, their slots and weights)
    // comes in one round trip, which the shared expert's loads (its slots
    // follow the routed ones) overlap; they are issued after it so that the
    // wait for the route does not also wait for them.
    // Every load here is unconditional (no branch for the counter wait to
    // merge over); lanes past the used entries read in-bounds leftovers.
    const int nr = __builtin_amdgcn_readfirstlane(a.uinfo[0]);
    const int n_sl = n_ent + S * T;
    const int ue = a.uinfo[1 + 3 * lane];
    const int us0 = a.uinfo[2 + 3 * lane];
    const int un = a.uinfo[3 + 3 * lane];
    const int ti = threadIdx.x;
    const float wv = reinterpret_cast<const float*>(a.uinfo + kUinfoW)[min(ti, n_ent - 1)];
    const int tv = a.slot_tok[min(ti, n_sl - 1)];
    __builtin_amdgcn_sched_barrier(0);
    Operands sh;
    load_w(S ? E : 0, sh);
    load_h(S ? E : 0, n_ent, T, sh);
    __builtin_amdgcn_sched_barrier(0);
    if (wave == 0) {
        s_e[lane] = ue;
        s_s0[lane] = us0;
        s_n[lane] = un;
    }
    if (ti < n_sl) {
        s_w[ti] = (ti < n_ent) ? wv : 1.0f;
        s_t[ti] = tv;
    }
    if (ti < 4 * RPW * NT) (&s_acc[0][0])[ti] = 0.0;
    __syncthreads();
    // routed experts in batches of NB, the next batch's loads issued before
    // the current batch's arithmetic (two register buffers)
    struct Batch {
        Operands o[NB];
    };
    auto load = [&](int v0, Batch& bt) {
#pragma unroll
        for (int bi = 0; bi < NB; ++bi) {
            const int v = min(v0 + bi, nr - 1);
            load_w(__builtin_amdgcn_readfirstlane(s_e[v]), bt.o[bi]);
        }
#pragma unroll
        for (int bi = 0; bi < NB; ++bi) {
            const int v = min(v0 + bi, nr - 1);
            load_h(__builtin_amdgcn_readfirstlane(s_e[v]), __builtin_amdgcn_readfirstlane(s_s0[v]),
                   __builtin_amdgcn_readfirstlane(s_n[v]), bt.o[bi]);
        }
    };
    auto compute_batch = [&](int v0, const Batch& bt) {
#pragma unroll
        for (int bi = 0; bi < NB; ++bi) {
            const int v = v0 + bi;
            if (v >= nr) break;
            compute(bt.o[bi], __builtin_amdgcn_readfirstlane(s_s0[v]),
                    __builtin_amdgcn_readfirstlane(s_n[v]));
        }
    };
    Batch b0, b1;
    if (nr > 0) load(0, b0);
    if constexpr (NT == 1 && NB == 1) {
        // one token: the dot products of two experts, then one reduction of
        // their four row sums (the same addition tree per value as two
        // separate reductions, so the same results, in fewer dependent steps)
        auto partial = [&](const Operands& o, double (&pp)[RPW]) {
#pragma unroll
            for (int r = 0; r < RPW; ++r) {
                double p = 0.0;
#pragma unroll
                for (int j = 0; j < NBJ; ++j) {
                    const bool ok = lane + 64 * j < BI;
                    const double hd = ok ? (double)o.hdf[0][j] * F::kInv : 0.0;
                    p += hd * (double)F::dot(o.w[r][j], o.ha[0][j][0], o.ha[0][j][1]);
                }
                pp[r] = p;
            }
        };
        constexpr int V2 = 2 * RPW;
        constexpr int kShift2 = (V2 == 8) ? 3 : (V2 == 4) ? 4 : 5;
#pragma unroll 1
        for (int v0 = 0; v0 < nr; v0 += 2) {
            if (v0 + 1 >= nr) {  // odd count: the last one alone
                compute(b0.o[0], __builtin_amdgcn_readfirstlane(s_s0[v0]), 1);
                break;
            }
            load(v0 + 1, b1);
            __builtin_amdgcn_sched_barrier(0);
            double vals[V2];
            double pa[RPW], pb[RPW];
            partial(b0.o[0], pa);
            float dsa[RPW];
#pragma unroll
            for (int r = 0; r < RPW; ++r) dsa[r] = b0.o[0].dsv[r];
            // unconditional (the index is clamped: the last pair requests
            // expert nr - 1 again), so that the wait for b1 does not also wait
            // for these loads, as it would after a conditional issue
            load(v0 + 2, b0);
            __builtin_amdgcn_sched_barrier(0);
            partial(b1.o[0], pb);
#pragma unroll
            for (int r = 0; r < RPW; ++r) {
                vals[r] = pa[r];
                vals[RPW + r] = pb[r];
            }
            const double sum = wave_reduce_tr<V2>(vals, lane);
            // value (expert m, row r) sits in lanes (m RPW + r) << kShift2; row
            // r's combine lives in lane r << kShift: experts added in order
            const int r = lane >> kShift;
            float dsr_a = dsa[0], dsr_b = b1.o[0].dsv[0];
#pragma unroll
            for (int rr = 1; rr < RPW; ++rr)
                if (r == rr) {
                    dsr_a = dsa[rr];
                    dsr_b = b1.o[0].dsv[rr];
                }
            const double sa = __shfl(sum, r << kShift2, 64);
            const double sb = __shfl(sum, (RPW + r) << kShift2, 64);
            const float ya = (float)((double)dsr_a * sa);
            const float yb = (float)((double)dsr_b * sb);
            racc += (double)s_w[__builtin_amdgcn_readfirstlane(s_s0[v0])] * (double)ya;
            racc += (double)s_w[__builtin_amdgcn_readfirstlane(s_s0[v0 + 1])] * (double)yb;
        }
    } else {
#pragma unroll 1
        for (int v0 = 0; v0 < nr; v0 += 2 * NB) {
            if (v0 + NB < nr) load(v0 + NB, b1);
            __builtin_amdgcn_sched_barrier(0);
            compute_batch(v0, b0);
            if (v0 + NB >= nr) break;
            if (v0 + 2 * NB < nr) load(v0 + 2 * NB, b0);
            __builtin_amdgcn_sched_barrier(0);
            compute_batch(v0 + NB, b1);
        }
    }
    if (S) compute(sh, n_ent, T);
    if constexpr (NT == 1) {
        const int r = lane >> kShift;
        if (lane == (r << kShift) && T > 0) {
            float* out = a.y + c0 + r;
            const float yv = (float)racc;
            *out = a.accum ? *out + yv : yv;
        }
    } else if (lane < RPW * NT) {
        const int r = lane / NT, t = lane - r * NT;
        if (t < T) {
            float* out = a.y + (int64_t)t * H + c0 + r;
            const float yv = (float)s_acc[wave * RPW + r][t];
            *out = a.accum ? *out + yv : yv;
        }
    }
}


// C (expert-split variant): down projection and combine for 8 output rows
// per workgroup. Wave w takes the experts in use v = w, w+4, w+8, ... in
// batches of PB; a batch's 8 rows per expert and its activation blocks are
// all requested before any is used (at batch 1 with 9 experts in use this is
// the whole job: one memory round trip per wave). Per-(row, expert, token)
// results y_e = fp32(s_down * sum) go to LDS; the combine then runs in
// ascending expert order with the shared expert last.
template <int NT, int PB, int BITS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void k_dec_down_x(DecArgs a) {
    typedef DW<BITS> F;
    constexpr int RW = 8;                        // rows per workgroup
    constexpr int kSlots = kMaxEntries + kMaxTok;
    __shared__ int s_e[kMaxEntries + 1], s_s0[kMaxEntries + 1], s_n[kMaxEntries + 1];
    __shared__ float s_w[kSlots];
    __shared__ int s_t[kSlots];
    __shared__ float s_y[RW][kSlots];            // y_e of (row, slot)
    __shared__ int s_nu;
    const int T = a.T, K = a.K, E = a.E, S = a.S, H = a.H, I = a.I;
    const int BI = I >> 5;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n_ent = T * K;
    // the published route in one round trip: lane v of wave 0 reads entry v
    // (unconditionally: the entries past n_uniq are in-bounds leftovers)
    if (wave == 0) {
        const int nu = a.uinfo[0];
        const int ue = a.uinfo[1 + 3 * lane];
        const int us0 = a.uinfo[2 + 3 * lane];
        const int un = a.uinfo[3 + 3 * lane];
        if (lane < nu) {
            s_e[lane] = ue;
            s_s0[lane] = us0;
            s_n[lane] = un;
        }
        if (lane == 0) {
            if (S) {
                s_e[nu] = E;
                s_s0[nu] = n_ent;
                s_n[nu] = T;
            }
            s_nu = nu + (S ? 1 : 0);
        }
    }
    for (int i = threadIdx.x; i < n_ent + S * T; i += 256) {
        s_w[i] = (i < n_ent) ? reinterpret_cast<const float*>(a.uinfo + kUinfoW)[i] : 1.0f;
        s_t[i] = a.slot_tok[i];
    }
    __syncthreads();
    const int c0 = blockIdx.x * RW;
    const int nu = __builtin_amdgcn_readfirstlane(s_nu);
    const int bcl = min(lane, BI - 1);           // I <= 2048: one block per lane
#pragma unroll 1
    for (int v0 = wave; v0 < nu; v0 += 4 * PB) {
        typename F::blk w[PB][RW];
        uint4 ha[PB][NT][2];
        float hdf[PB][NT];
        int ev[PB];
#pragma unroll
        for (int m = 0; m < PB; ++m) {
            const int v = min(v0 + 4 * m, nu - 1);
            ev[m] = __builtin_amdgcn_readfirstlane(s_e[v]);
            const int64_t rowb = (int64_t)I * BITS / 8;
            const uint8_t* down = a.eq + (int64_t)ev[m] * a.blob_q + 2 * (int64_t)H * rowb;
#pragma unroll
            for (int r = 0; r < RW; ++r)
                w[m][r] = F::load(down + (int64_t)(c0 + r) * rowb + bcl * (4 * BITS));
        }
#pragma unroll
        for (int m = 0; m < PB; ++m) {
            const int v = min(v0 + 4 * m, nu - 1);
            const int s0 = __builtin_amdgcn_readfirstlane(s_s0[v]);
            const int n = __builtin_amdgcn_readfirstlane(s_n[v]);
#pragma unroll
            for (int i = 0; i < NT; ++i) {
                const int sl = s0 + min(i, n - 1);
                const uint4* p = reinterpret_cast<const uint4*>(a.qh + (int64_t)sl * I + bcl * 32);
                ha[m][i][0] = p[0];
                ha[m][i][1] = p[1];
                hdf[m][i] = a.dh[(int64_t)sl * BI + bcl];
            }
        }
        // row scales: lane r (< RW) of the wave holds expert m's scale of row c0 + r
        float dsm[PB];
#pragma unroll
        for (int m = 0; m < PB; ++m) dsm[m] = a.es[(int64_t)ev[m] * a.blob_s + 2 * I + c0 + (lane & (RW - 1))];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = 0; m < PB; ++m) {
            const int v = v0 + 4 * m;
            const int vc = min(v, nu - 1);
            const int n = __builtin_amdgcn_readfirstlane(s_n[vc]);
            const int s0 = __builtin_amdgcn_readfirstlane(s_s0[vc]);
#pragma unroll
            for (int i = 0; i < NT; ++i) {
                // the expert's tokens only (n is wave-uniform; most routed
                // experts of a few-token call hold one)
                if (v >= nu || i >= n) break;
                const bool ok = lane < BI;
                const double hd = ok ? (double)hdf[m][i] * F::kInv : 0.0;
                double vals[RW];
#pragma unroll
                for (int r = 0; r < RW; ++r)
                    vals[r] = hd * (double)F::dot(w[m][r], ha[m][i][0], ha[m][i][1]);
                const double sum = wave_reduce_tr<RW>(vals, lane);
                const int r = lane >> 3;  // 64 / RW lanes per value
                const float ds = __shfl(dsm[m], r, 64);
                if ((lane & 7) == 0) s_y[r][s0 + i] = (float)((double)ds * sum);
            }
        }
    }
    __syncthreads();
    if ((int)threadIdx.x < RW * T) {
        const int r = threadIdx.x / T, t = threadIdx.x - r * T;
        double acc = 0.0;
        for (int v = 0; v < nu; ++v) {
            const int s0 = s_s0[v], n = s_n[v];
            for (int i = 0; i < n; ++i)
                if (s_t[s0 + i] == t) acc += (double)s_w[s0 + i] * (double)s_y[r][s0 + i];
        }
        float* out = a.y + (int64_t)t * H + c0 + r;
        const float yv = (float)acc;
        *out = a.accum ? *out + yv : yv;
    }
}

}  // namespace dec
