// Router (fp32 inputs, fp64 accumulation), sigmoid + correction bias + top-k
// in wavefront registers, and token->expert bucketing by histogram and scan.
#pragma once

#include "coli_common.h"

// ---------------------------------------------------------------------------
// Router logits for few tokens: one workgroup per expert row streams its
// H floats once and dots them with every token (tokens come from L2). The
// row goes in chunks of kU float4 per thread; a chunk's loads (the row's and
// every token slot's, clamped and unconditional) are all issued before its
// arithmetic, so a 6144-wide row costs one round trip, not six.
// ---------------------------------------------------------------------------
template <int NT>
__global__ __launch_bounds__(256) void k_router_gemv(const float* __restrict__ x,
                                                     const float* __restrict__ wr, int T, int H,
                                                     int E, double* __restrict__ logits) {
    __shared__ double red[NT][4];
    constexpr int kU = 6;
    const int e = blockIdx.x;
    const float* wrow = wr + (int64_t)e * H;
    double acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = 0.0;
    for (int h0 = threadIdx.x * 4; h0 < H; h0 += 1024 * kU) {
        float4 wv[kU], xv[NT][kU];
#pragma unroll
        for (int u = 0; u < kU; ++u)
            wv[u] = *reinterpret_cast<const float4*>(wrow + min(h0 + 1024 * u, H - 4));
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int u = 0; u < kU; ++u)
                xv[t][u] = *reinterpret_cast<const float4*>(
                    x + (int64_t)min(t, T - 1) * H + min(h0 + 1024 * u, H - 4));
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            if (t < T) {
#pragma unroll
                for (int u = 0; u < kU; ++u) {
                    if (h0 + 1024 * u < H) {
                        acc[t] += (double)xv[t][u].x * (double)wv[u].x;
                        acc[t] += (double)xv[t][u].y * (double)wv[u].y;
                        acc[t] += (double)xv[t][u].z * (double)wv[u].z;
                        acc[t] += (double)xv[t][u].w * (double)wv[u].w;
                    }
                }
            }
        }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const double s = wave_sum_f64(acc[t]);
        if ((threadIdx.x & 63) == 0) red[t][threadIdx.x >> 6] = s;
    }
    __syncthreads();
    if (threadIdx.x < NT && (int)threadIdx.x < T) {
        const int t = threadIdx.x;
        logits[(int64_t)t * E + e] = (red[t][0] + red[t][1]) + (red[t][2] + red[t][3]);
    }
}

// Router logits for many tokens: a 64-token x 64-expert tile per workgroup
// over one of `ksplit` equal slices of the hidden dimension, on the fp64
// matrix cores: each wave computes a 32 x 32 quarter as 2 x 2 tiles of
// v_mfma_f64_16x16x4f64 (A: lane l holds token l % 16 at k = l / 16; B:
// expert l % 16 at k = l / 16; result register i of lane l is token
// l / 16 + 4 i, expert l % 16; checked on the device). Products of the fp32
// inputs are exact in fp64; the slice's sum is fp64, four terms per step.
// Operands are converted to fp64 in LDS ([row][k], pitch 33: the 16 rows x 4
// k of an operand read hit distinct banks per 16 lanes). Partial sums go to
// part[slice][t][e]; k_router_reduce adds the slices in order.
constexpr int kRouterTile = 64;
constexpr int kRouterK = 32;

typedef double v4d __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void k_router_gemm(const float* __restrict__ x,
                                                     const float* __restrict__ wr, int T, int H,
                                                     int E, int ksplit,
                                                     double* __restrict__ part) {
    __shared__ double xs[kRouterTile][kRouterK + 1];
    __shared__ double ws[kRouterTile][kRouterK + 1];
    const int t0 = blockIdx.x * kRouterTile, e0 = blockIdx.y * kRouterTile;
    const int kper = H / ksplit, kbeg = blockIdx.z * kper;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int tr = (wave >> 1) * 32, ec = (wave & 1) * 32;  // this wave's quarter
    const int r16 = lane & 15, kq = lane >> 4;
    v4d acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = v4d{0.0, 0.0, 0.0, 0.0};
    // this thread's two float4 of each operand chunk: rows li >> 3, columns
    // 4 (li & 7) of the 64 x 32 tile; the next chunk is requested right after
    // the current one is staged (unconditionally: the last chunk is requested
    // again at the end), so its latency overlaps the MFMA work
    const int kend = kbeg + kper;
    const float* xrow[2];
    const float* wrow[2];
    bool xok[2], wok[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int li = tid * 2 + i, row = li >> 3, c4 = li & 7;
        xok[i] = t0 + row < T;
        wok[i] = e0 + row < E;
        xrow[i] = x + (int64_t)min(t0 + row, T - 1) * H + c4 * 4;
        wrow[i] = wr + (int64_t)min(e0 + row, E - 1) * H + c4 * 4;
    }
    float4 nv[2], nw[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        nv[i] = *reinterpret_cast<const float4*>(xrow[i] + kbeg);
        nw[i] = *reinterpret_cast<const float4*>(wrow[i] + kbeg);
    }
    for (int k0 = kbeg; k0 < kend; k0 += kRouterK) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int li = tid * 2 + i, row = li >> 3, c4 = li & 7;
            const float4 v = xok[i] ? nv[i] : make_float4(0.f, 0.f, 0.f, 0.f);
            const float4 w = wok[i] ? nw[i] : make_float4(0.f, 0.f, 0.f, 0.f);
            xs[row][c4 * 4 + 0] = v.x;
            xs[row][c4 * 4 + 1] = v.y;
            xs[row][c4 * 4 + 2] = v.z;
            xs[row][c4 * 4 + 3] = v.w;
            ws[row][c4 * 4 + 0] = w.x;
            ws[row][c4 * 4 + 1] = w.y;
            ws[row][c4 * 4 + 2] = w.z;
            ws[row][c4 * 4 + 3] = w.w;
        }
        __syncthreads();
        const int kn = min(k0 + kRouterK, kend - kRouterK);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            nv[i] = *reinterpret_cast<const float4*>(xrow[i] + kn);
            nw[i] = *reinterpret_cast<const float4*>(wrow[i] + kn);
        }
#pragma unroll
        for (int k = 0; k < kRouterK; k += 4) {
            double av[2], bv[2];
#pragma unroll
            for (int a = 0; a < 2; ++a) av[a] = xs[tr + 16 * a + r16][k + kq];
#pragma unroll
            for (int b = 0; b < 2; ++b) bv[b] = ws[ec + 16 * b + r16][k + kq];
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[a], bv[b], acc[a][b], 0, 0, 0);
        }
        __syncthreads();
    }
    double* out = part + (int64_t)blockIdx.z * T * E;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = t0 + tr + 16 * a + kq + 4 * i, e = e0 + ec + 16 * b + r16;
                if (t < T && e < E) out[(int64_t)t * E + e] = acc[a][b][i];
            }
}

// logits[i] = sum over slices s = 0 .. ksplit-1 of part[s][i], in that order.
__global__ __launch_bounds__(256) void k_router_reduce(const double* __restrict__ part,
                                                       int ksplit, int64_t n,
                                                       double* __restrict__ logits) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    double v = part[i];
    for (int s = 1; s < ksplit; ++s) v += part[(int64_t)s * n + i];
    logits[i] = v;
}

// ---------------------------------------------------------------------------
// Sigmoid, correction bias and top-k for shapes beyond the wave selection of
// k_topk_wave (more than 256 experts or K > 16): one wave per token, EPL
// candidates per lane. K rounds of a wave arg-max under the total order (c
// desc, index asc); lane k keeps the k-th choice. Gate values: unbiased
// sigmoid, normalised by their sum (k ascending) when asked, times rho,
// rounded to fp32.
// ---------------------------------------------------------------------------
template <int EPL>
__global__ __launch_bounds__(256) void k_topk(const double* __restrict__ logits,
                                              const float* __restrict__ bias, int T, int E, int K,
                                              int norm, double rho, GroupSel gsel,
                                              int32_t* __restrict__ idx,
                                              float* __restrict__ wout) {
    extern __shared__ double c_stage[];  // [4][E] when gsel.ng > 1
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;  // whole wave leaves together
    double c[EPL], s[EPL];
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
        const int e = lane + 64 * j;
        if (e < E) {
            const double l = logits[(int64_t)t * E + e];
            s[j] = 1.0 / (1.0 + exp(-l));
            c[j] = s[j] + (double)bias[e];
        } else {
            s[j] = 0.0;
            c[j] = -__builtin_inf();
        }
    }
    if (gsel.ng > 1) {
        // group-limited selection: the experts of dropped groups leave the race
        double* cw = c_stage + (threadIdx.x >> 6) * E;
#pragma unroll
        for (int j = 0; j < EPL; ++j)
            if (lane + 64 * j < E) cw[lane + 64 * j] = c[j];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const unsigned long long keep = group_keep_mask(cw, gsel);
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
            const int e = lane + 64 * j;
            if (e < E && !((keep >> (e / gsel.gs)) & 1ull)) c[j] = -__builtin_inf();
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
        idx[(int64_t)t * K + lane] = my_e;
        wout[(int64_t)t * K + lane] = (float)v;
    }
}

// ---------------------------------------------------------------------------
// Bucketing, step 1: one workgroup per expert scans the [T, K] choices in
// token order and compacts the matching (t, k) entries (value t*(K+S)+k) into
// a fixed-capacity list; the shared expert (index E) takes every token. No
// atomics: ballot + popcount ranks inside a wave, LDS across waves, so the
// lists are in ascending token order and identical on every run.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_bucket_lists(const int32_t* __restrict__ idx, int T,
                                                      int K, int E, int S,
                                                      int32_t* __restrict__ lists,
                                                      int32_t* __restrict__ counts) {
    __shared__ int wave_cnt[4];
    const int e = blockIdx.x;
    const int KS = K + S;
    int32_t* out = lists + (int64_t)e * T;
    if (e == E) {
        for (int t = threadIdx.x; t < T; t += 256) out[t] = t * KS + K;
        if (threadIdx.x == 0) counts[e] = T;
        return;
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int base = 0;
    for (int t0 = 0; t0 < T; t0 += 256) {
        const int t = t0 + threadIdx.x;
        int kk = -1;
        if (t < T)
            for (int k = 0; k < K; ++k)
                if (idx[(int64_t)t * K + k] == e) kk = k;
        const uint64_t bal = __ballot(kk >= 0);
        const int pre = __popcll(bal & ((1ull << lane) - 1ull));
        if (lane == 0) wave_cnt[wave] = __popcll(bal);
        __syncthreads();
        int off = base;
        for (int w = 0; w < wave; ++w) off += wave_cnt[w];
        if (kk >= 0) out[off + pre] = t * KS + kk;
        base += wave_cnt[0] + wave_cnt[1] + wave_cnt[2] + wave_cnt[3];
        __syncthreads();
    }
    if (threadIdx.x == 0) counts[e] = base;
}

// ---------------------------------------------------------------------------
// Bucketing, step 2 (one workgroup per expert, E + S in all): expert e's
// first slot (the counts of the experts before it) and first item (their
// item counts, ceil(count / CH)) as sums over the count array, exact in any
// order; then its work items (expert, first slot, <= CH tokens) and, from its
// list, the slot <-> (t, k) maps. Experts are in ascending order, so slots
// and items follow expert order; the last workgroup writes the totals.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_bucket_fill(
    const int32_t* __restrict__ counts, const int32_t* __restrict__ lists, int T, int K, int E,
    int S, int CH, int32_t* __restrict__ offs, int32_t* __restrict__ slot_of,
    int32_t* __restrict__ slot_tok, int32_t* __restrict__ item_e, int32_t* __restrict__ item_s0,
    int32_t* __restrict__ item_n, int32_t* __restrict__ n_items) {
    __shared__ int red[2][4];
    const int NE = E + S, KS = K + S;
    const int e = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int so = 0, io = 0;
    for (int f = threadIdx.x; f < e; f += 256) {
        const int c = counts[f];
        so += c;
        io += (c + CH - 1) / CH;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        so += __shfl_xor(so, o, 64);
        io += __shfl_xor(io, o, 64);
    }
    if (lane == 0) {
        red[0][wave] = so;
        red[1][wave] = io;
    }
    __syncthreads();
    so = (red[0][0] + red[0][1]) + (red[0][2] + red[0][3]);
    io = (red[1][0] + red[1][1]) + (red[1][2] + red[1][3]);
    const int c = counts[e];
    const int ni = (c + CH - 1) / CH;
    if (threadIdx.x == 0) {
        offs[e] = so;
        if (e == NE - 1) {
            offs[NE] = so + c;
            *n_items = io + ni;
        }
    }
    for (int j = threadIdx.x; j < ni; j += 256) {
        item_e[io + j] = e;
        item_s0[io + j] = so + j * CH;
        item_n[io + j] = min(CH, c - j * CH);
    }
    for (int p = threadIdx.x; p < c; p += 256) {
        const int entry = lists[(int64_t)e * T + p];
        slot_of[entry] = so + p;
        slot_tok[so + p] = entry / KS;
    }
}
