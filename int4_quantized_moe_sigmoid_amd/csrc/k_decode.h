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

namespace dec {

constexpr int kMaxTok = 4;
constexpr int kMaxEntries = 64;  // T * K

typedef unsigned v4u __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 ldnt(const uint8_t* p) {
    const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Transposed wave reduction of V values per lane: after log2(V) halving
// butterflies every lane holds one partial of value index (lane >> (6 -
// log2 V)); the remaining butterflies finish that sum. Returns the full sum
// of that value index.
template <int V>
__device__ __forceinline__ double wave_reduce_tr(double* v, int lane) {
    int step = 0;
#pragma unroll
    for (int h = V; h > 1; h >>= 1) {
        const int mask = 32 >> step;
        const bool upper = (lane & mask) != 0;
#pragma unroll
        for (int i = 0; i < h / 2; ++i) {
            const double keep = upper ? v[i + h / 2] : v[i];
            const double send = upper ? v[i] : v[i + h / 2];
            v[i] = keep + __shfl_xor(send, mask, 64);
        }
        ++step;
    }
    double s = v[0];
#pragma unroll
    for (int mask = 32 >> step; mask > 0; mask >>= 1) s += __shfl_xor(s, mask, 64);
    return s;
}

// Q8_0 of block b of fp32 row x (32 values) into the 8-group order, in
// registers: a0/a1 hold the 32 codes, returns the block scale.
__device__ __forceinline__ float q8_block_regs(const float* x, uint4& a0, uint4& a1) {
    const float4* p = reinterpret_cast<const float4*>(x);
    float v[32];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float4 f = p[i];
        v[4 * i] = f.x;
        v[4 * i + 1] = f.y;
        v[4 * i + 2] = f.z;
        v[4 * i + 3] = f.w;
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
    const float d = amax / 127.0f;
    int c[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) c[i] = q8_code(v[i], d);
    uint32_t w[8];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        w[2 * g] = pack4_i8(c[8 * g], c[8 * g + 2], c[8 * g + 4], c[8 * g + 6]);
        w[2 * g + 1] = pack4_i8(c[8 * g + 1], c[8 * g + 3], c[8 * g + 5], c[8 * g + 7]);
    }
    a0 = make_uint4(w[0], w[1], w[2], w[3]);
    a1 = make_uint4(w[4], w[5], w[6], w[7]);
    return d;
}

// Routing of T <= 4 tokens, computed redundantly by every workgroup of B.
struct Route {
    int idx[kMaxTok][16];
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
    // top-k scratch
    unsigned long long gmax[kMaxTok][8];  // max key of each 32-expert group
    int ncand[kMaxTok];
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

// Sigmoid + bias + top-k + gate weights of T <= 4 tokens by the whole
// workgroup (thread e owns expert e, E <= blockDim.x). Selection order is c
// descending, expert index ascending among equal c; an expert's position is
// the number of experts ahead of it in that order. Only experts whose c is at
// least the smallest of the 32-expert group maxima can be among the K largest
// (when there are >= K groups those maxima are >= K distinct experts), so
// positions are counted among those few candidates only.
__device__ __forceinline__ void topk_wg(const double* logits, const float* bias, int T, int E, int K,
                                        int norm, double rho, Route& R) {
    const int e = threadIdx.x;
    const int G = (E + 31) >> 5;
    const bool filt = G >= K;
    if (threadIdx.x < kMaxTok * 8) (&R.gmax[0][0])[threadIdx.x] = 0ull;
    if (threadIdx.x < kMaxTok) R.ncand[threadIdx.x] = 0;
    double l[kMaxTok];
    float bb = 0.0f;
#pragma unroll
    for (int t = 0; t < kMaxTok; ++t) l[t] = (t < T && e < E) ? logits[(int64_t)t * E + e] : 0.0;
    if (e < E) bb = bias[e];
    __syncthreads();
    unsigned long long key[kMaxTok];
    double s[kMaxTok];
#pragma unroll
    for (int t = 0; t < kMaxTok; ++t) {
        s[t] = 1.0 / (1.0 + exp(-l[t]));
        key[t] = order_key(s[t] + (double)bb);
        if (filt && t < T && e < E) atomicMax(&R.gmax[t][e >> 5], key[t]);
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < kMaxTok; ++t) {
        if (t < T && e < E) {
            unsigned long long thr = 0ull;
            if (filt) {
                thr = ~0ull;
                for (int g = 0; g < G; ++g) thr = min(thr, R.gmax[t][g]);
            }
            if (key[t] >= thr) {
                const int p = atomicAdd(&R.ncand[t], 1);
                R.ckey[t][p] = key[t];
                R.ce[t][p] = e;
                R.cs[t][p] = s[t];
            }
        }
    }
    __syncthreads();
    for (int t = 0; t < T; ++t) {
        const int m = R.ncand[t];
        for (int i = threadIdx.x; i < m; i += blockDim.x) {
            const unsigned long long ki = R.ckey[t][i];
            const int ei = R.ce[t][i];
            int rank = 0;
            for (int j = 0; j < m; ++j) {
                const unsigned long long kj = R.ckey[t][j];
                rank += (kj > ki || (kj == ki && R.ce[t][j] < ei)) ? 1 : 0;
            }
            if (rank < K) {
                R.idx[t][rank] = ei;
                R.ssel[t][rank] = R.cs[t][i];
            }
        }
    }
    __syncthreads();
    if ((int)threadIdx.x < T * K) {
        const int t = threadIdx.x / K, k = threadIdx.x - t * K;
        double sum = 0.0;
        for (int kk = 0; kk < K; ++kk) sum += R.ssel[t][kk];
        double v = R.ssel[t][k];
        if (norm) v = v / sum;
        v = v * rho;
        R.w[t][k] = (float)v;
    }
}

// Fills R (in LDS) for T tokens; must be called by the whole workgroup
// (blockDim.x >= E).
__device__ __forceinline__ void route_small(const double* logits, const float* bias, int T, int E, int K, int S,
                            int norm, double rho, Route& R) {
    topk_wg(logits, bias, T, E, K, norm, rho, R);
    __syncthreads();
    const int n = T * K;
    const int i = threadIdx.x;
    int e = 0, t = 0, k = 0, rank = 0, first = 1, cnt = 0;
    if (i < n) {
        t = i / K;
        k = i - t * K;
        e = R.idx[t][k];
        for (int j = 0; j < n; ++j) {
            const int tj = j / K, ej = R.idx[tj][j - tj * K];
            if (ej < e || (ej == e && tj < t)) ++rank;
            if (ej == e) {
                ++cnt;
                if (tj < t) first = 0;
            }
        }
    }
    __syncthreads();
    if (i < n) {
        R.ent_e[rank] = e;
        R.ent_t[rank] = t;
        R.ent_w[rank] = R.w[t][k];
        R.slot_of[t][k] = rank;
    }
    if (i < T && S) R.slot_of[i][K] = n + i;
    __syncthreads();
    if (i < n && first) {
        int u = 0;
        for (int j = 0; j < n; ++j) {
            const int ej = R.ent_e[j];
            if ((j == 0 || R.ent_e[j - 1] != ej) && ej < e) ++u;
        }
        R.u_e[u] = e;
        R.u_s0[u] = rank;
        R.u_n[u] = cnt;
    }
    if (i == 0) {
        int u = 0;
        for (int j = 0; j < n; ++j)
            if (j == 0 || R.ent_e[j - 1] != R.ent_e[j]) ++u;
        R.n_uniq = u;
    }
    __syncthreads();
}

struct DecArgs {
    const float* x;
    const float* wr;
    const float* bias;
    const uint8_t* eq;
    const float* es;
    int64_t blob_q, blob_s;
    int T, H, I, E, K, S, norm;
    double rho;
    // workspace
    double* logits;
    int8_t* qx;
    float* dx;
    int32_t* idx;
    float* wts;
    int32_t* counts;
    int32_t* offs;
    int32_t* slot_of;
    int32_t* slot_tok;
    int32_t* uinfo;   // [0] = n_uniq, then (e, s0, n) triples, then slot weights
    int8_t* qh;
    float* dh;
    int32_t* tap;
    int tap_rows, tap_stride;
    float* y;
    int accum;
};

constexpr int kUinfoW = 1 + 3 * kMaxEntries;  // offset of the slot weights in uinfo


// Gate/up GEMV for one expert, NT token slots and 32 intermediate rows
// (h-block hb), then SwiGLU and Q8_0(h) into qh/dh at slots slot0 + i.
// Activations: Q8_0 codes of x in 8-group order (qx) and block scales (dx),
// rows of token tok[i]. Four waves; wave w owns h-rows w, w+4, ..., w+28,
// taken two per step (two gate + two up rows), so the four waves read 8
// consecutive rows of each matrix at a time; the loop is fully unrolled and
// every load unconditional (lanes past the last block read a clamped address
// and see zero activations), with two steps' loads in flight.
template <int NT, int NBJ, bool TAP>
__device__ __forceinline__ void gateup_block(const DecArgs& a, int e, int hb, int n,
                                             const int* tok, int slot0, float (*hbuf)[32]) {
    const int H = a.H, I = a.I, BH = H >> 5;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint8_t* gate = a.eq + (int64_t)e * a.blob_q;
    const uint8_t* up = gate + (int64_t)I * (H >> 1);
    const float* gs = a.es + (int64_t)e * a.blob_s;
    const float* us = gs + I;
    const int r0 = hb * 32 + wave;  // rows r0 + 4k, k = 0..7
    int boff[NBJ];
#pragma unroll
    for (int j = 0; j < NBJ; ++j) boff[j] = min(lane + 64 * j, BH - 1) * 16;
    uint4 wb[2][4][NBJ];
    auto load_pair = [&](int p, uint4 (&dst)[4][NBJ]) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = r0 + 4 * (2 * p + (q & 1));
            const uint8_t* row = ((q < 2) ? gate : up) + (int64_t)r * (H >> 1);
#pragma unroll
            for (int j = 0; j < NBJ; ++j) dst[q][j] = ldnt(row + boff[j]);
        }
    };
    load_pair(0, wb[0]);
    load_pair(1, wb[1]);
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
            xd[i][j] = ok ? (double)d * 0.0625 : 0.0;  // undo the x16 of the codes
        }
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        if (p >= 1 && p < 3) load_pair(p + 1, wb[(p + 1) & 1]);
        // keep the next step's loads issued ahead of this step's arithmetic
        __builtin_amdgcn_sched_barrier(0);
        const uint4 (&wc)[4][NBJ] = wb[p & 1];
        // values ordered (quad, token): quad 0/1 = gate rows of step p, 2/3 = up rows
        double v[4 * NT];
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int i = 0; i < NT; ++i) {
                double acc = 0.0;
#pragma unroll
                for (int j = 0; j < NBJ; ++j) {
                    const int d16 = dot_block16(wc[q][j], xa[i][j][0], xa[i][j][1]);
                    acc += xd[i][j] * (double)d16;
                    if (TAP && q < 2) {
                        const int r = r0 + 4 * (2 * p + q), b = lane + 64 * j;
                        if (i < n && b < BH && (r % a.tap_stride) == 0)
                            a.tap[((int64_t)(slot0 + i) * a.tap_rows + r / a.tap_stride) * BH + b] =
                                d16 / 16;
                    }
                }
                v[q * NT + i] = acc;
            }
        const double sum = wave_reduce_tr<4 * NT>(v, lane);
        const double other = __shfl_xor(sum, 32, 64);  // up value for gate lanes
        constexpr int kShift = (NT == 1) ? 4 : (NT == 2) ? 3 : 2;  // 6 - log2(4 NT)
        const int vi = lane >> kShift;   // value index held by this lane
        const int kq = 2 * p + ((vi < 2 * NT) ? vi / NT : 0);
        const float gsk = __shfl(gsl, kq, 64), usk = __shfl(usl, kq, 64);
        if (vi < 2 * NT && lane == (vi << kShift)) {
            const int q = vi / NT, i = vi - q * NT;   // q in {0, 1}: row r0 + 4(2p+q)
            if (i < n) {
                const float g = (float)((double)gsk * sum);
                const float u = (float)((double)usk * other);
                hbuf[i][wave + 4 * (2 * p + q)] = swiglu_f32(g, u);
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
            a.qh[(int64_t)(slot0 + i) * I + hb * 32 + q8_perm_pos(k)] = (int8_t)c;
            if (k == 0) a.dh[(int64_t)(slot0 + i) * (I >> 5) + hb] = dd;
        }
    }
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

// A: router rows (one workgroup per expert); workgroup 0 also writes Q8_0(x).
template <int NT>
__global__ __launch_bounds__(256) void k_dec_router(DecArgs a) {
    __shared__ double red[NT][4];
    const int e = blockIdx.x;
    const int T = a.T, H = a.H;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const float* wrow = a.wr + (int64_t)e * H;
    double acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = 0.0;
    for (int h = threadIdx.x * 4; h < H; h += 1024) {
        const float4 wv = *reinterpret_cast<const float4*>(wrow + h);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            if (t < T) {
                const float4 xv = *reinterpret_cast<const float4*>(a.x + (int64_t)t * H + h);
                acc[t] += (double)xv.x * (double)wv.x;
                acc[t] += (double)xv.y * (double)wv.y;
                acc[t] += (double)xv.z * (double)wv.z;
                acc[t] += (double)xv.w * (double)wv.w;
            }
        }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const double s = wave_sum_f64(acc[t]);
        if (lane == 0) red[t][wave] = s;
    }
    __syncthreads();
    if ((int)threadIdx.x < T) {
        const double* r = red[threadIdx.x];
        a.logits[(int64_t)threadIdx.x * a.E + e] = (r[0] + r[1]) + (r[2] + r[3]);
    }
    if (e == 0) {
        const int nblk = T * (H >> 5);
        for (int blk = threadIdx.x; blk < nblk; blk += 256) {
            uint4 q0, q1;
            const float d = q8_block_regs(a.x + (int64_t)blk * 32, q0, q1);
            uint4* o = reinterpret_cast<uint4*>(a.qx + (int64_t)blk * 32);
            o[0] = q0;
            o[1] = q1;
            a.dx[blk] = d;
        }
    }
}

// B: blocks [0, S*nrb) shared-expert h-blocks, then (u, hb) for the u-th
// expert in use (u < min(E, T*K)); block (u = 0, hb = 0) publishes routing.
template <int NT, int NBJ, bool TAP>
__global__ __launch_bounds__(256) void k_dec_gateup(DecArgs a) {
    __shared__ Route R;
    __shared__ float hbuf[NT][32];
    __shared__ int s_tok[NT];
    const int nrb = a.I >> 5;
    int b = blockIdx.x;
    if (a.S) {
        if (b < nrb) {
            if ((int)threadIdx.x < NT) s_tok[threadIdx.x] = threadIdx.x;
            __syncthreads();
            gateup_block<NT, NBJ, TAP>(a, a.E, b, a.T, s_tok, a.T * a.K, hbuf);
            return;
        }
        b -= nrb;
    }
    route_small(a.logits, a.bias, a.T, a.E, a.K, a.S, a.norm, a.rho, R);
    if (b == 0) publish_route(a, R);
    const int u = b / nrb, hb = b - u * nrb;
    if (u >= R.n_uniq) return;
    const int e = __builtin_amdgcn_readfirstlane(R.u_e[u]);
    const int s0 = __builtin_amdgcn_readfirstlane(R.u_s0[u]);
    const int n = __builtin_amdgcn_readfirstlane(R.u_n[u]);
    gateup_block<NT, NBJ, TAP>(a, e, hb, n, &R.ent_t[s0], s0, hbuf);
}

// C: down projection of every expert in use and the weighted combine.
// Workgroup = 4 waves x RPW rows; lane l owns block l (+64 j) of a down row.
// Experts are taken NB at a time: all their rows and activation blocks are
// requested before any is used (unconditional loads, clamped indices), then
// reduced. Each wave accumulates its rows' combine in LDS (fp64), in
// ascending expert order with the shared expert last.
template <int NT, int NBJ, int RPW, int NB>
__global__ __launch_bounds__(256) void k_dec_down(DecArgs a) {
    __shared__ int s_e[kMaxEntries + 1], s_s0[kMaxEntries + 1], s_n[kMaxEntries + 1];
    __shared__ float s_w[kMaxEntries + kMaxTok];
    __shared__ int s_t[kMaxEntries + kMaxTok];
    __shared__ double s_acc[4 * RPW][NT];
    __shared__ int s_nu;
    const int T = a.T, K = a.K, E = a.E, S = a.S, H = a.H, I = a.I;
    const int BI = I >> 5;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n_ent = T * K;
    if (threadIdx.x == 0) {
        int nu = a.uinfo[0];
        for (int v = 0; v < nu; ++v) {
            s_e[v] = a.uinfo[1 + 3 * v];
            s_s0[v] = a.uinfo[2 + 3 * v];
            s_n[v] = a.uinfo[3 + 3 * v];
        }
        if (S) {
            s_e[nu] = E;
            s_s0[nu] = n_ent;
            s_n[nu] = T;
            ++nu;
        }
        s_nu = nu;
    }
    for (int i = threadIdx.x; i < n_ent + S * T; i += 256) {
        s_w[i] = (i < n_ent) ? reinterpret_cast<const float*>(a.uinfo + kUinfoW)[i] : 1.0f;
        s_t[i] = a.slot_tok[i];
    }
    if (threadIdx.x < 4 * RPW * NT) (&s_acc[0][0])[threadIdx.x] = 0.0;
    __syncthreads();
    const int c0 = blockIdx.x * (4 * RPW) + wave * RPW;
    const int nu = __builtin_amdgcn_readfirstlane(s_nu);
    int bcl[NBJ];
#pragma unroll
    for (int j = 0; j < NBJ; ++j) bcl[j] = min(lane + 64 * j, BI - 1);
    constexpr int V = RPW * NT;
    constexpr int kLog = (V >= 16) ? 4 : (V >= 8) ? 3 : (V >= 4) ? 2 : (V >= 2) ? 1 : 0;
    constexpr int kShift = 6 - kLog;
#pragma unroll 1
    for (int v0 = 0; v0 < nu; v0 += NB) {
        uint4 w[NB][RPW][NBJ];
        uint4 ha[NB][NT][NBJ][2];
        float hdf[NB][NT][NBJ];
        float dsv[NB][RPW];
#pragma unroll
        for (int bi = 0; bi < NB; ++bi) {
            const int v = min(v0 + bi, nu - 1);
            const int ev = __builtin_amdgcn_readfirstlane(s_e[v]);
            const uint8_t* down = a.eq + (int64_t)ev * a.blob_q + (int64_t)I * H;
#pragma unroll
            for (int r = 0; r < RPW; ++r)
#pragma unroll
                for (int j = 0; j < NBJ; ++j)
                    w[bi][r][j] = ldnt(down + (int64_t)(c0 + r) * (I >> 1) + bcl[j] * 16);
        }
#pragma unroll
        for (int bi = 0; bi < NB; ++bi) {
            const int v = min(v0 + bi, nu - 1);
            const int ev = __builtin_amdgcn_readfirstlane(s_e[v]);
            const int s0 = __builtin_amdgcn_readfirstlane(s_s0[v]);
            const int n = __builtin_amdgcn_readfirstlane(s_n[v]);
            const float* ds = a.es + (int64_t)ev * a.blob_s + 2 * I;
#pragma unroll
            for (int r = 0; r < RPW; ++r) dsv[bi][r] = ds[c0 + r];
#pragma unroll
            for (int i = 0; i < NT; ++i) {
                const int sl = s0 + min(i, n - 1);
#pragma unroll
                for (int j = 0; j < NBJ; ++j) {
                    const uint4* p = reinterpret_cast<const uint4*>(a.qh + (int64_t)sl * I + bcl[j] * 32);
                    ha[bi][i][j][0] = p[0];
                    ha[bi][i][j][1] = p[1];
                    hdf[bi][i][j] = a.dh[(int64_t)sl * BI + bcl[j]];
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int bi = 0; bi < NB; ++bi) {
            const int v = v0 + bi;
            if (v >= nu) break;
            const int s0 = __builtin_amdgcn_readfirstlane(s_s0[v]);
            const int n = __builtin_amdgcn_readfirstlane(s_n[v]);
            double vals[V];
#pragma unroll
            for (int r = 0; r < RPW; ++r)
#pragma unroll
                for (int i = 0; i < NT; ++i) {
                    double p = 0.0;
#pragma unroll
                    for (int j = 0; j < NBJ; ++j) {
                        const bool ok = i < n && lane + 64 * j < BI;
                        const double hd = ok ? (double)hdf[bi][i][j] * 0.0625 : 0.0;
                        p += hd * (double)dot_block16(w[bi][r][j], ha[bi][i][j][0], ha[bi][i][j][1]);
                    }
                    vals[r * NT + i] = p;
                }
            const double sum = wave_reduce_tr<V>(vals, lane);
            const int vi = lane >> kShift;
            if (lane == (vi << kShift)) {
                const int r = vi / NT, i = vi - r * NT;
                if (i < n) {
                    float dsr = dsv[bi][0];
#pragma unroll
                    for (int rr = 1; rr < RPW; ++rr)
                        if (r == rr) dsr = dsv[bi][rr];
                    const float yv = (float)((double)dsr * sum);
                    s_acc[wave * RPW + r][s_t[s0 + i]] += (double)s_w[s0 + i] * (double)yv;
                }
            }
        }
    }
    if (lane < RPW * NT) {
        const int r = lane / NT, t = lane - r * NT;
        if (t < T) {
            float* out = a.y + (int64_t)t * H + c0 + r;
            const float yv = (float)s_acc[wave * RPW + r][t];
            *out = a.accum ? *out + yv : yv;
        }
    }
}

}  // namespace dec
