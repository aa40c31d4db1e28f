// One persistent kernel for the whole layer on few tokens (decode, MTP
// verify). Launch cost on this GPU is a few microseconds per kernel, close to
// a tenth of the layer at batch 1, and each phase boundary (router -> top-k
// -> gate/up -> down) would otherwise drain the machine. Here the phases are
// work items that overlap:
//
//   item ids   [0, E)                router row e (+ Q8_0(x) in item 0); the
//                                    last router item routes the tokens
//              [E, E+S*nrb)          shared-expert h-block (no routing needed)
//              [.., + UM*nrb)        routed h-block (u = expert in use, hb)
//              [.., + H/RPG)         down rows c0..c0+RPG-1 of every expert
//                                    in use + weighted combine into y
//
// A workgroup takes item blockIdx.x first, then the next unclaimed id from a
// queue counter, so ids are started in increasing order and an item only
// waits for items with smaller ids (its producers): the lowest unfinished
// item can always proceed, whatever the number of resident workgroups.
// Waits poll per-class counters (tagged counters, see tagged_add) and are
// bounded: a wait that exceeds its budget sets an error word and the item
// goes on with whatever data is present, so a fault in this protocol yields
// wrong numbers that the host reports, never a hang.
//
// Data passed between workgroups of the grid (logits, Q8_0(x), routing, q_h,
// d_h) is stored and loaded with device-scope atomic accesses, which stay
// coherent across the chip's L2 slices without cache-wide fences.
#pragma once

#include "k_decode.h"

namespace dec {

constexpr int kRPG = 8;              // down rows per item
constexpr int kCtrQueue = 0, kCtrRouter = 1, kCtrRoute = 2, kCtrQx = 3, kCtrH = 4;
constexpr int kCtrShared = kCtrH + kMaxEntries;   // shared expert h-blocks
constexpr int kSyncWords = kCtrShared + 1;
constexpr int kWaitBudget = 1 << 22;

__device__ __forceinline__ uint32_t ld_dev_u32(const void* p) {
    return __hip_atomic_load(reinterpret_cast<const uint32_t*>(p), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev_f32(const float* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint4 ld_dev16(const void* p) {
    const unsigned long long* q = reinterpret_cast<const unsigned long long*>(p);
    const unsigned long long a = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned long long b =
        __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return make_uint4((uint32_t)a, (uint32_t)(a >> 32), (uint32_t)b, (uint32_t)(b >> 32));
}
__device__ __forceinline__ void st_dev_u32(void* p, uint32_t v) {
    __hip_atomic_store(reinterpret_cast<uint32_t*>(p), v, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev_f32(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Bounded wait (whole wave) until the tagged counter reaches `target`.
__device__ __forceinline__ void wait_count(unsigned long long* c, uint32_t tag, uint32_t target,
                                           int32_t* err) {
    for (int it = 0; it < kWaitBudget; ++it) {
        const unsigned long long v =
            __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const bool done = ((uint32_t)(v >> 32) == tag) && ((uint32_t)v >= target);
        if (__builtin_amdgcn_readfirstlane((int)done)) return;
        __builtin_amdgcn_s_sleep(2);
    }
    st_dev_u32(err, 1u);
}

struct PArgs {
    DecArgs d;
    int32_t* err;
    int n_router, n_shared, n_routed, n_down, n_items;
    int grid;
};

// Gate/up h-block with device-coherent activation loads and q_h/d_h stores
// (the producer/consumer are other workgroups of the same grid). Four waves,
// 8 h-rows each, two steps in flight.
template <int NT, int NBJ, bool TAP>
__device__ __forceinline__ void p_gateup(const PArgs& P, int e, int hb, int n, const int* tok,
                                         int slot0, float (*hbuf)[32], int8_t (*qbuf)[32]) {
    const DecArgs& a = P.d;
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
    float gsc[8], usc[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        gsc[k] = gs[r0 + 4 * k];
        usc[k] = us[r0 + 4 * k];
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
            const int8_t* p = a.qx + (int64_t)t * H + bb * 32;
            const uint4 a0 = ld_dev16(p), a1 = ld_dev16(p + 16);
            const float d = ld_dev_f32(a.dx + (int64_t)t * BH + bb);
            xa[i][j][0] = ok ? a0 : make_uint4(0, 0, 0, 0);
            xa[i][j][1] = ok ? a1 : make_uint4(0, 0, 0, 0);
            xd[i][j] = ok ? (double)d * 0.0625 : 0.0;
        }
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        if (p >= 1 && p < 3) load_pair(p + 1, wb[(p + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
        const uint4 (&wc)[4][NBJ] = wb[p & 1];
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
        const double other = __shfl_xor(sum, 32, 64);
        constexpr int kShift = (NT == 1) ? 4 : (NT == 2) ? 3 : 2;
        const int vi = lane >> kShift;
        if (vi < 2 * NT && lane == (vi << kShift)) {
            const int q = vi / NT, i = vi - q * NT;
            if (i < n) {
                const int k = 2 * p + q;
                const float g = (float)((double)gsc[k] * sum);
                const float u = (float)((double)usc[k] * other);
                hbuf[i][wave + 4 * k] = swiglu_f32(g, u);
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
        qbuf[i][q8_perm_pos(k)] = (int8_t)q8_code(val, dd);
        if (i < n && k == 0) st_dev_f32(a.dh + (int64_t)(slot0 + i) * (I >> 5) + hb, dd);
    }
    __syncthreads();
    if (threadIdx.x < NT * 8) {
        const int i = threadIdx.x >> 3, w = threadIdx.x & 7;
        if (i < n)
            st_dev_u32(a.qh + (int64_t)(slot0 + i) * I + hb * 32 + 4 * w,
                       reinterpret_cast<const uint32_t*>(qbuf[i])[w]);
    }
}

template <int NT, int NBJH, int NBJI, int EPL, bool TAP>
__global__ __launch_bounds__(256) void k_dec_persist(PArgs P) {
    __shared__ int s_item;
    __shared__ double red[NT][4];
    __shared__ int s_last;
    __shared__ Route R;
    __shared__ float hbuf[NT][32];
    __shared__ uint32_t qbuf32[NT][8];
    __shared__ int s_tok[NT];
    __shared__ float s_w[kMaxEntries + kMaxTok];
    __shared__ int s_t[kMaxEntries + kMaxTok];
    __shared__ double s_part[kMaxEntries + 1][kRPG][NT];
    const DecArgs& a = P.d;
    const int T = a.T, H = a.H, I = a.I, E = a.E, K = a.K, S = a.S;
    const int nrb = I >> 5, BH = H >> 5, BI = I >> 5;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int b_shared = P.n_router, b_routed = b_shared + P.n_shared,
              b_down = b_routed + P.n_routed;
    unsigned long long* ctr = a.sync;
    const uint32_t tag = a.tag;

    int item = blockIdx.x;
    while (item < P.n_items) {
        if (item < b_shared) {
            // ------------------------------------------------ router row
            const int e = item;
            if (e == 0) {
                // Q8_0(x) for every gate/up item (and the taps)
                const int nblk = T * BH;
                for (int blk = threadIdx.x; blk < nblk; blk += 256) {
                    uint4 q0, q1;
                    const float d = q8_block_regs(a.x + (int64_t)blk * 32, q0, q1);
                    uint32_t* o = reinterpret_cast<uint32_t*>(a.qx + (int64_t)blk * 32);
                    st_dev_u32(o + 0, q0.x); st_dev_u32(o + 1, q0.y);
                    st_dev_u32(o + 2, q0.z); st_dev_u32(o + 3, q0.w);
                    st_dev_u32(o + 4, q1.x); st_dev_u32(o + 5, q1.y);
                    st_dev_u32(o + 6, q1.z); st_dev_u32(o + 7, q1.w);
                    st_dev_f32(a.dx + blk, d);
                }
                __syncthreads();
                if (threadIdx.x == 0) tagged_add(ctr + kCtrQx, tag);
            }
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
                __hip_atomic_store(a.logits + (int64_t)threadIdx.x * E + e,
                                   (r[0] + r[1]) + (r[2] + r[3]), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            }
            __syncthreads();
            if (threadIdx.x == 0) s_last = (tagged_add(ctr + kCtrRouter, tag) == (uint32_t)(E - 1));
            __syncthreads();
            if (s_last) {
                route_small<EPL>(a.logits, a.bias, T, E, K, S, a.norm, a.rho, R);
                // routing for the other items (device scope) and for the host
                const int n = T * K;
                for (int i = threadIdx.x; i < n; i += 256) {
                    const int t = i / K, k = i - t * K;
                    a.idx[i] = R.idx[t][k];
                    a.wts[i] = R.w[t][k];
                    a.slot_of[t * (K + S) + k] = R.slot_of[t][k];
                    st_dev_u32(a.slot_tok + i, (uint32_t)R.ent_t[i]);
                    st_dev_f32(reinterpret_cast<float*>(a.uinfo + kUinfoW) + i, R.ent_w[i]);
                }
                for (int t = threadIdx.x; t < T; t += 256)
                    if (S) {
                        a.slot_of[t * (K + S) + K] = n + t;
                        st_dev_u32(a.slot_tok + n + t, (uint32_t)t);
                    }
                for (int ee = threadIdx.x; ee < E + S; ee += 256) {
                    int cnt = (ee < E) ? 0 : T, before = 0;
                    for (int v = 0; v < R.n_uniq; ++v) {
                        if (R.u_e[v] == ee) cnt = R.u_n[v];
                        if (R.u_e[v] < ee) before += R.u_n[v];
                    }
                    a.counts[ee] = cnt;
                    a.offs[ee] = (ee < E) ? before : n;
                }
                if (threadIdx.x == 0) a.offs[E + S] = n + S * T;
                for (int v = threadIdx.x; v < R.n_uniq; v += 256) {
                    st_dev_u32(a.uinfo + 1 + 3 * v, (uint32_t)R.u_e[v]);
                    st_dev_u32(a.uinfo + 2 + 3 * v, (uint32_t)R.u_s0[v]);
                    st_dev_u32(a.uinfo + 3 + 3 * v, (uint32_t)R.u_n[v]);
                }
                if (threadIdx.x == 0) st_dev_u32(a.uinfo, (uint32_t)R.n_uniq);
                __syncthreads();
                if (threadIdx.x == 0) tagged_add(ctr + kCtrRoute, tag);
            }
        } else if (item < b_down) {
            // ------------------------------------------------ gate/up h-block
            const bool shared = item < b_routed;
            const int rel = shared ? item - b_shared : item - b_routed;
            const int u = rel / nrb, hb = rel - u * nrb;
            int e, s0, n;
            if (shared) {
                e = E;
                s0 = T * K;
                n = T;
                if (threadIdx.x < NT) s_tok[threadIdx.x] = threadIdx.x;
            } else {
                if (wave == 0) wait_count(ctr + kCtrRoute, tag, 1, P.err);
                __syncthreads();
                const int nu = __builtin_amdgcn_readfirstlane((int)ld_dev_u32(a.uinfo));
                if (u >= nu) goto next_item;   // uniform: whole workgroup skips
                e = __builtin_amdgcn_readfirstlane((int)ld_dev_u32(a.uinfo + 1 + 3 * u));
                s0 = __builtin_amdgcn_readfirstlane((int)ld_dev_u32(a.uinfo + 2 + 3 * u));
                n = __builtin_amdgcn_readfirstlane((int)ld_dev_u32(a.uinfo + 3 + 3 * u));
                if ((int)threadIdx.x < NT)
                    s_tok[threadIdx.x] = (int)ld_dev_u32(a.slot_tok + s0 + min((int)threadIdx.x, n - 1));
            }
            if (wave == 0) wait_count(ctr + kCtrQx, tag, 1, P.err);
            __syncthreads();
            p_gateup<NT, NBJH, TAP>(P, e, hb, n, s_tok, s0, hbuf,
                                    reinterpret_cast<int8_t(*)[32]>(qbuf32));
            __syncthreads();
            if (threadIdx.x == 0) tagged_add(ctr + (shared ? kCtrShared : kCtrH + u), tag);
        } else {
            // ------------------------------------------------ down rows + combine
            const int c0 = (item - b_down) * kRPG;
            if (wave == 0) wait_count(ctr + kCtrRoute, tag, 1, P.err);
            __syncthreads();
            const int nu_r = __builtin_amdgcn_readfirstlane((int)ld_dev_u32(a.uinfo));
            const int nu = nu_r + S;
            const int n_ent = T * K;
            for (int i = threadIdx.x; i < n_ent + S * T; i += 256) {
                s_w[i] = (i < n_ent) ? ld_dev_f32(reinterpret_cast<const float*>(a.uinfo + kUinfoW) + i)
                                     : 1.0f;
                s_t[i] = (i < n_ent) ? (int)ld_dev_u32(a.slot_tok + i) : i - n_ent;
            }
            for (int i = threadIdx.x; i < nu * kRPG * NT; i += 256) (&s_part[0][0][0])[i] = 0.0;
            __syncthreads();
            int bcl[NBJI];
#pragma unroll
            for (int j = 0; j < NBJI; ++j) bcl[j] = min(lane + 64 * j, BI - 1);
            constexpr int V = kRPG * NT;
            constexpr int kLog = (V >= 32) ? 5 : (V >= 16) ? 4 : 3;
            constexpr int kShift = 6 - kLog;
            // shared expert first: its h-blocks are produced earliest
            for (int q = wave; q < nu; q += 4) {
                const int v = (S && q == 0) ? nu_r : q - S;   // expert slot
                int ev, s0, n;
                unsigned long long* c;
                if (v == nu_r) {
                    ev = E; s0 = n_ent; n = T; c = ctr + kCtrShared;
                } else {
                    ev = __builtin_amdgcn_readfirstlane((int)ld_dev_u32(a.uinfo + 1 + 3 * v));
                    s0 = __builtin_amdgcn_readfirstlane((int)ld_dev_u32(a.uinfo + 2 + 3 * v));
                    n = __builtin_amdgcn_readfirstlane((int)ld_dev_u32(a.uinfo + 3 + 3 * v));
                    c = ctr + kCtrH + v;
                }
                const uint8_t* down = a.eq + (int64_t)ev * a.blob_q + (int64_t)I * H;
                uint4 w[kRPG][NBJI];
#pragma unroll
                for (int r = 0; r < kRPG; ++r)
#pragma unroll
                    for (int j = 0; j < NBJI; ++j)
                        w[r][j] = ldnt(down + (int64_t)(c0 + r) * (I >> 1) + bcl[j] * 16);
                const float* ds = a.es + (int64_t)ev * a.blob_s + 2 * I;
                float dsv[kRPG];
#pragma unroll
                for (int r = 0; r < kRPG; ++r) dsv[r] = ds[c0 + r];
                wait_count(c, tag, (uint32_t)nrb, P.err);
                uint4 ha[NT][NBJI][2];
                double hd[NT][NBJI];
#pragma unroll
                for (int i = 0; i < NT; ++i) {
                    const int sl = s0 + min(i, n - 1);
#pragma unroll
                    for (int j = 0; j < NBJI; ++j) {
                        const bool ok = i < n && lane + 64 * j < BI;
                        const int8_t* p = a.qh + (int64_t)sl * I + bcl[j] * 32;
                        ha[i][j][0] = ld_dev16(p);
                        ha[i][j][1] = ld_dev16(p + 16);
                        const float d = ld_dev_f32(a.dh + (int64_t)sl * BI + bcl[j]);
                        hd[i][j] = ok ? (double)d * 0.0625 : 0.0;
                    }
                }
                double vals[V];
#pragma unroll
                for (int r = 0; r < kRPG; ++r)
#pragma unroll
                    for (int i = 0; i < NT; ++i) {
                        double p = 0.0;
#pragma unroll
                        for (int j = 0; j < NBJI; ++j)
                            p += hd[i][j] * (double)dot_block16(w[r][j], ha[i][j][0], ha[i][j][1]);
                        vals[r * NT + i] = p;
                    }
                const double sum = wave_reduce_tr<V>(vals, lane);
                const int vi = lane >> kShift;
                if (lane == (vi << kShift)) {
                    const int r = vi / NT, i = vi - r * NT;
                    float dsr = dsv[0];
#pragma unroll
                    for (int rr = 1; rr < kRPG; ++rr)
                        if (r == rr) dsr = dsv[rr];
                    const float yv = (float)((double)dsr * sum);
                    if (i < n) s_part[v][r][s_t[s0 + i]] = (double)s_w[s0 + i] * (double)yv;
                }
            }
            __syncthreads();
            if (threadIdx.x < kRPG * NT) {
                const int r = threadIdx.x / NT, t = threadIdx.x - r * NT;
                double acc = 0.0;
                for (int v = 0; v < nu; ++v) acc += s_part[v][r][t];   // routed ascending, shared last
                if (t < T) {
                    float* out = a.y + (int64_t)t * H + c0 + r;
                    const float yv = (float)acc;
                    *out = a.accum ? *out + yv : yv;
                }
            }
        }
    next_item:
        __syncthreads();
        if (threadIdx.x == 0) s_item = P.grid + (int)tagged_add(ctr + kCtrQueue, tag);
        __syncthreads();
        item = s_item;
    }
}

}  // namespace dec
