// Fused path for few tokens (decode at batch 1, MTP verify): three launches.
//
//   A  router rows (one workgroup per expert row, fp64 logits) and, in the
//      same grid, the shared expert's gate/up + SwiGLU + Q8_0(h): the shared
//      expert does not depend on routing, so its weights stream while the
//      router runs. The router workgroup that finishes last (a tagged
//      device-scope counter, see tagged_add) runs the top-k and the expert
//      bucketing of the <= 4 tokens once and publishes them.
//   B  routed gate/up + SwiGLU + Q8_0(h): one workgroup per (expert in use,
//      block of 32 intermediate rows); tokens that share an expert are served
//      by one pass over its weights.
//   C  down projection of every expert in use plus the weighted combine,
//      written straight into y.
//
// Weight streams use 16-byte nontemporal loads (each byte is used once);
// lane l owns blocks l, l+64, l+128 of a row so a wave instruction reads 1 KiB
// contiguous. Activations are quantised to Q8_0 in registers by each
// workgroup straight from fp32 x (bit-identical to the Q8_0 kernel).
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
};

// One wave per token: sigmoid + bias, K rounds of wave arg-max (c desc, index
// asc), gates normalised (k ascending) and scaled, as k_topk.
template <int EPL>
__device__ __forceinline__ void route_token_wave(const double* logits, const float* bias, int E, int K, int norm,
                                 double rho, int t, int lane, Route& R) {
    double c[EPL], s[EPL];
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
        const int e = lane + 64 * j;
        if (e < E) {
            // written by other workgroups of this grid: device-coherent load
            const double l = __hip_atomic_load(logits + (int64_t)t * E + e, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
            s[j] = 1.0 / (1.0 + exp(-l));
            c[j] = s[j] + (double)bias[e];
        } else {
            s[j] = 0.0;
            c[j] = -__builtin_inf();
        }
    }
    uint32_t taken = 0;
    int my_e = 0;
    double my_s = 0.0;
    for (int k = 0; k < K; ++k) {
        double bc = -__builtin_inf(), bs = 0.0;
        int be = 0x7fffffff;
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
            const int e = lane + 64 * j;
            if (e < E && !((taken >> j) & 1u) && (c[j] > bc || (c[j] == bc && e < be))) {
                bc = c[j];
                be = e;
                bs = s[j];
            }
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            const double oc = __shfl_xor(bc, o, 64);
            const int oe = __shfl_xor(be, o, 64);
            const double os = __shfl_xor(bs, o, 64);
            if (oc > bc || (oc == bc && oe < be)) {
                bc = oc;
                be = oe;
                bs = os;
            }
        }
        if ((be & 63) == lane) taken |= 1u << (be >> 6);
        if (lane == k) {
            my_e = be;
            my_s = bs;
        }
    }
    double sum = 0.0;
    for (int k = 0; k < K; ++k) sum += __shfl(my_s, k, 64);
    if (lane < K) {
        double v = my_s;
        if (norm) v = v / sum;
        v = v * rho;
        R.idx[t][lane] = my_e;
        R.w[t][lane] = (float)v;
    }
}

// Fills R (in LDS) for T tokens; must be called by the whole workgroup (>= 64
// threads, T <= 4 waves route).
template <int EPL>
__device__ __forceinline__ void route_small(const double* logits, const float* bias, int T, int E, int K, int S,
                            int norm, double rho, Route& R) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (wave < T) route_token_wave<EPL>(logits, bias, E, K, norm, rho, wave, lane, R);
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

// 64-bit counter in the workspace whose high word is a per-call tag and low
// word a count: the first increment of a call replaces a stale tag (left by
// an earlier call, or arbitrary memory) by compare-and-swap, so the counter
// needs no clearing between calls. Returns the count before this increment.
// The data a workgroup publishes before its increment is written with
// device-scope atomic stores (coherent across the chip's L2 slices without a
// cache write-back) and completed before the increment (the workgroup
// barrier waits for outstanding stores); the observer reads it back with
// device-scope atomic loads. Agent-scope release/acquire fences would instead
// write back and invalidate whole L2 slices, which costs microseconds each.
__device__ __forceinline__ uint32_t tagged_add(unsigned long long* c, uint32_t tag) {
    unsigned long long v = __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (;;) {
        if ((uint32_t)(v >> 32) == tag)
            return (uint32_t)__hip_atomic_fetch_add(c, 1ull, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
        const unsigned long long want = ((unsigned long long)tag << 32) | 1ull;
        if (__hip_atomic_compare_exchange_strong(c, &v, want, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT))
            return 0;
    }
}

// Gate/up GEMV for one expert, NT token slots and 32 intermediate rows
// (h-block hb), then SwiGLU and Q8_0(h) into qh/dh at slots slot0 + i.
// Activations (Q8_0 codes in 8-group order and block scales) are read from
// aq/ad, rows of token tok[i] with strides H and H/32 (global workspace or
// LDS). An 8-wave workgroup: wave w owns h-rows w, w+8, w+16, w+24, i.e. two
// steps of (two gate + two up) rows, and requests both steps' weights before
// any arithmetic, so a CU holding two such workgroups has all of its share of
// the expert's bytes in flight at once; at every step the eight waves read
// 16 consecutive rows of each matrix. Loads are unconditional (lanes past the
// last block read a clamped address and see zero activations).
template <int NT, int NBJ, bool TAP>
__device__ __forceinline__ void gateup_block(const uint8_t* gate, const uint8_t* up, const float* gs,
                                             const float* us, int H, int I, int hb, int n,
                                             const int8_t* aq, const float* ad, const int* tok,
                                             int slot0, int8_t* qh, float* dh, int32_t* tap,
                                             int tap_rows, int tap_stride, float (*hbuf)[32]) {
    const int BH = H >> 5;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r0 = hb * 32 + wave;  // rows r0 + 8k, k = 0..3
    int boff[NBJ];
#pragma unroll
    for (int j = 0; j < NBJ; ++j) boff[j] = min(lane + 64 * j, BH - 1) * 16;

    uint4 wb[2][4][NBJ];
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = r0 + 8 * (2 * p + (q & 1));
            const uint8_t* row = ((q < 2) ? gate : up) + (int64_t)r * (H >> 1);
#pragma unroll
            for (int j = 0; j < NBJ; ++j) wb[p][q][j] = ldnt(row + boff[j]);
        }
    float gsc[4], usc[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        gsc[k] = gs[r0 + 8 * k];
        usc[k] = us[r0 + 8 * k];
    }
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
            const uint4* p = reinterpret_cast<const uint4*>(aq + (int64_t)t * H + bb * 32);
            const uint4 a0 = p[0], a1 = p[1];
            const float d = ad[(int64_t)t * BH + bb];
            xa[i][j][0] = ok ? a0 : make_uint4(0, 0, 0, 0);
            xa[i][j][1] = ok ? a1 : make_uint4(0, 0, 0, 0);
            xd[i][j] = ok ? (double)d * 0.0625 : 0.0;  // undo the x16 of the codes
        }
    }
    __builtin_amdgcn_sched_barrier(0);

#pragma unroll
    for (int p = 0; p < 2; ++p) {
        // values ordered (quad, token): quad 0/1 = gate rows of step p, 2/3 = up rows
        double v[4 * NT];
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int i = 0; i < NT; ++i) {
                double acc = 0.0;
#pragma unroll
                for (int j = 0; j < NBJ; ++j) {
                    const int d16 = dot_block16(wb[p][q][j], xa[i][j][0], xa[i][j][1]);
                    acc += xd[i][j] * (double)d16;
                    if (TAP && q < 2) {
                        const int r = r0 + 8 * (2 * p + q), b = lane + 64 * j;
                        if (i < n && b < BH && (r % tap_stride) == 0)
                            tap[((int64_t)(slot0 + i) * tap_rows + r / tap_stride) * BH + b] = d16 / 16;
                    }
                }
                v[q * NT + i] = acc;
            }
        const double sum = wave_reduce_tr<4 * NT>(v, lane);
        const double other = __shfl_xor(sum, 32, 64);  // up value for gate lanes
        constexpr int kShift = (NT == 1) ? 4 : (NT == 2) ? 3 : 2;  // 6 - log2(4 NT)
        const int vi = lane >> kShift;   // value index held by this lane
        if (vi < 2 * NT && lane == (vi << kShift)) {
            const int q = vi / NT, i = vi - q * NT;   // q in {0, 1}: row r0 + 8(2p+q)
            if (i < n) {
                const int k = 2 * p + q;
                const float g = (float)((double)gsc[k] * sum);
                const float u = (float)((double)usc[k] * other);
                hbuf[i][wave + 8 * k] = swiglu_f32(g, u);
            }
        }
    }
    __syncthreads();
    if (threadIdx.x < NT * 32) {
        const int i = threadIdx.x >> 5, k = threadIdx.x & 31;
        const float val = (i < n) ? hbuf[i][k] : 0.0f;
        float a = fabsf(val);
#pragma unroll
        for (int o = 16; o > 0; o >>= 1) a = fmaxf(a, __shfl_xor(a, o, 32));
        const float dd = a / 127.0f;
        const int c = q8_code(val, dd);
        if (i < n) {
            qh[(int64_t)(slot0 + i) * I + hb * 32 + q8_perm_pos(k)] = (int8_t)c;
            if (k == 0) dh[(int64_t)(slot0 + i) * (I >> 5) + hb] = dd;
        }
    }
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
    unsigned long long* sync;  // tagged counters
    uint32_t tag;
};

constexpr int kUinfoW = 1 + 3 * kMaxEntries;  // offset of the slot weights in uinfo

// Publishes the routing computed in R (by the last router workgroup).
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

// A: blocks [0, E) router rows (the last one to finish also routes);
//    blocks [E, E + I/32) shared-expert h-blocks.
template <int NT, int NBJ, int EPL, bool TAP>
__global__ __launch_bounds__(512) void k_dec_router_shared(DecArgs a) {
    __shared__ float hbuf[NT][32];
    __shared__ double red[NT][8];
    __shared__ int s_last;
    __shared__ Route R;
    __shared__ uint4 s_q[NT * 8192 / 16];   // Q8_0 codes of x (8-group order)
    __shared__ float s_d[NT * 8192 / 32];
    const int b = blockIdx.x;
    const int T = a.T, H = a.H;
    if (b < a.E) {
        const int e = b;
        const float* wrow = a.wr + (int64_t)e * H;
        double acc[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t] = 0.0;
        for (int h = threadIdx.x * 4; h < H; h += 2048) {
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
            if ((threadIdx.x & 63) == 0) red[t][threadIdx.x >> 6] = s;
        }
        __syncthreads();
        if ((int)threadIdx.x < T) {
            const double* r = red[threadIdx.x];
            __hip_atomic_store(a.logits + (int64_t)threadIdx.x * a.E + e,
                               ((r[0] + r[1]) + (r[2] + r[3])) + ((r[4] + r[5]) + (r[6] + r[7])),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        if (e == 0) {
            // Q8_0(x) into the workspace for the routed gate/up kernel and the taps
            const int nblk = T * (H >> 5);
            for (int blk = threadIdx.x; blk < nblk; blk += 512) {
                uint4 q0, q1;
                const float d = q8_block_regs(a.x + (int64_t)blk * 32, q0, q1);
                uint4* o = reinterpret_cast<uint4*>(a.qx + (int64_t)blk * 32);
                o[0] = q0;
                o[1] = q1;
                a.dx[blk] = d;
            }
        }
        __syncthreads();
        if (threadIdx.x == 0) s_last = (tagged_add(a.sync, a.tag) == (uint32_t)(a.E - 1));
        __syncthreads();
        if (!s_last) return;
        // every router row is in memory: route the tokens once
        route_small<EPL>(a.logits, a.bias, a.T, a.E, a.K, a.S, a.norm, a.rho, R);
        publish_route(a, R);
        return;
    }
    // shared expert: quantise x into LDS cooperatively, then one h-block
    const int hb = b - a.E;
    const int se = a.E;
    const int BH = H >> 5;
    for (int blk = threadIdx.x; blk < T * BH; blk += 512) {
        uint4 q0, q1;
        s_d[blk] = q8_block_regs(a.x + (int64_t)blk * 32, q0, q1);
        s_q[2 * blk] = q0;
        s_q[2 * blk + 1] = q1;
    }
    __syncthreads();
    int tok[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) tok[i] = i;
    const uint8_t* gate = a.eq + (int64_t)se * a.blob_q;
    const uint8_t* up = gate + (int64_t)a.I * (H >> 1);
    const float* gs = a.es + (int64_t)se * a.blob_s;
    gateup_block<NT, NBJ, TAP>(gate, up, gs, gs + a.I, H, a.I, hb, T,
                               reinterpret_cast<const int8_t*>(s_q), s_d, tok, T * a.K, a.qh,
                               a.dh, a.tap, a.tap_rows, a.tap_stride, hbuf);
}

// B: routed gate/up, blocks = (unique expert u, h-block hb), u < min(E, T*K).
template <int NT, int NBJ, bool TAP>
__global__ __launch_bounds__(512) void k_dec_gateup(DecArgs a) {
    __shared__ float hbuf[NT][32];
    const int nrb = a.I >> 5;
    const int u = blockIdx.x / nrb, hb = blockIdx.x - u * nrb;
    const int nu = __builtin_amdgcn_readfirstlane(a.uinfo[0]);
    if (u >= nu) return;
    const int e = __builtin_amdgcn_readfirstlane(a.uinfo[1 + 3 * u]);
    const int s0 = __builtin_amdgcn_readfirstlane(a.uinfo[2 + 3 * u]);
    const int n = __builtin_amdgcn_readfirstlane(a.uinfo[3 + 3 * u]);
    int tok[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) tok[i] = (NT == 1) ? 0 : a.slot_tok[s0 + ((i < n) ? i : 0)];
    const uint8_t* gate = a.eq + (int64_t)e * a.blob_q;
    const uint8_t* up = gate + (int64_t)a.I * (a.H >> 1);
    const float* gs = a.es + (int64_t)e * a.blob_s;
    gateup_block<NT, NBJ, TAP>(gate, up, gs, gs + a.I, a.H, a.I, hb, n, a.qx, a.dx, tok, s0,
                               a.qh, a.dh, a.tap, a.tap_rows, a.tap_stride, hbuf);
}

// C: down projection of every expert in use and the weighted combine.
// A workgroup owns 8 output rows and has one wave per expert in use (up to
// 16; more are taken in rounds): each wave requests its expert's 8 rows and
// activation blocks at once, reduces 8 rows x NT tokens, and leaves the
// weighted fp64 contributions in LDS; the combine sums them per row in
// ascending expert order (shared expert last).
template <int NT, int NBJ>
__global__ __launch_bounds__(1024) void k_dec_down(DecArgs a) {
    constexpr int RPG = 8;
    __shared__ int s_e[kMaxEntries + 1], s_s0[kMaxEntries + 1], s_n[kMaxEntries + 1];
    __shared__ float s_w[kMaxEntries + kMaxTok];
    __shared__ int s_t[kMaxEntries + kMaxTok];
    __shared__ double s_part[kMaxEntries + 1][RPG][NT];
    __shared__ int s_nu;
    const int T = a.T, K = a.K, E = a.E, S = a.S, H = a.H, I = a.I;
    const int BI = I >> 5;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nwave = blockDim.x >> 6;
    const int n_ent = T * K;
    const int c0 = blockIdx.x * RPG;
    int bcl[NBJ];
#pragma unroll
    for (int j = 0; j < NBJ; ++j) bcl[j] = min(lane + 64 * j, BI - 1);
    // expert of this wave in round 0, straight from the workspace (no LDS round trip)
    const int nu_r = __builtin_amdgcn_readfirstlane(a.uinfo[0]);
    const int nu = nu_r + S;
    auto expert_of = [&](int v, int& e, int& s0, int& n) {
        if (v < nu_r) {
            e = __builtin_amdgcn_readfirstlane(a.uinfo[1 + 3 * v]);
            s0 = __builtin_amdgcn_readfirstlane(a.uinfo[2 + 3 * v]);
            n = __builtin_amdgcn_readfirstlane(a.uinfo[3 + 3 * v]);
        } else {
            e = E;
            s0 = n_ent;
            n = T;
        }
    };
    for (int i = threadIdx.x; i < n_ent + S * T; i += blockDim.x) {
        s_w[i] = (i < n_ent) ? reinterpret_cast<const float*>(a.uinfo + kUinfoW)[i] : 1.0f;
        s_t[i] = a.slot_tok[i];
    }
    for (int i = threadIdx.x; i < nu * RPG * NT; i += blockDim.x) (&s_part[0][0][0])[i] = 0.0;
    __syncthreads();
    constexpr int V = RPG * NT;
    constexpr int kLog = (V >= 32) ? 5 : (V >= 16) ? 4 : 3;
    constexpr int kShift = 6 - kLog;
#pragma unroll 1
    for (int v = wave; v < nu; v += nwave) {
        int e, s0, n;
        expert_of(v, e, s0, n);
        const uint8_t* down = a.eq + (int64_t)e * a.blob_q + (int64_t)I * H;
        uint4 w[RPG][NBJ];
#pragma unroll
        for (int r = 0; r < RPG; ++r)
#pragma unroll
            for (int j = 0; j < NBJ; ++j)
                w[r][j] = ldnt(down + (int64_t)(c0 + r) * (I >> 1) + bcl[j] * 16);
        const float* ds = a.es + (int64_t)e * a.blob_s + 2 * I;
        float dsv[RPG];
#pragma unroll
        for (int r = 0; r < RPG; ++r) dsv[r] = ds[c0 + r];
        uint4 ha[NT][NBJ][2];
        double hd[NT][NBJ];
#pragma unroll
        for (int i = 0; i < NT; ++i) {
            const int sl = s0 + min(i, n - 1);
#pragma unroll
            for (int j = 0; j < NBJ; ++j) {
                const bool ok = i < n && lane + 64 * j < BI;
                const uint4* p = reinterpret_cast<const uint4*>(a.qh + (int64_t)sl * I + bcl[j] * 32);
                ha[i][j][0] = p[0];
                ha[i][j][1] = p[1];
                const float d = a.dh[(int64_t)sl * BI + bcl[j]];
                hd[i][j] = ok ? (double)d * 0.0625 : 0.0;
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        double vals[V];
#pragma unroll
        for (int r = 0; r < RPG; ++r)
#pragma unroll
            for (int i = 0; i < NT; ++i) {
                double p = 0.0;
#pragma unroll
                for (int j = 0; j < NBJ; ++j)
                    p += hd[i][j] * (double)dot_block16(w[r][j], ha[i][j][0], ha[i][j][1]);
                vals[r * NT + i] = p;
            }
        const double sum = wave_reduce_tr<V>(vals, lane);
        const int vi = lane >> kShift;
        if (lane == (vi << kShift)) {
            const int r = vi / NT, i = vi - r * NT;
            float dsr = dsv[0];
#pragma unroll
            for (int rr = 1; rr < RPG; ++rr)
                if (r == rr) dsr = dsv[rr];
            const float yv = (float)((double)dsr * sum);
            if (i < n) s_part[v][r][s_t[s0 + i]] = (double)s_w[s0 + i] * (double)yv;
        }
    }
    __syncthreads();
    if (threadIdx.x < RPG * NT) {
        const int r = threadIdx.x / NT, t = threadIdx.x - r * NT;
        double acc = 0.0;
        for (int v = 0; v < nu; ++v) acc += s_part[v][r][t];
        if (t < T) {
            float* out = a.y + (int64_t)t * H + c0 + r;
            const float yv = (float)acc;
            *out = a.accum ? *out + yv : yv;
        }
    }
}

}  // namespace dec
