// int4 x int8 GEMV kernels for small token groups (decode, MTP verify).
//
// HBM-bound: every weight byte is read once per item. Lane l of a wave owns
// 32-wide blocks b = l, l+64, l+128, ... of a row, so one 16-byte load per
// lane covers a whole block and a wave instruction reads 1 KiB contiguous.
// The activation blocks a lane needs never change across rows, so they stay
// in registers for the whole kernel. Block dots are exact int32 (sdot4 on
// int4 codes pre-scaled by 16), scaled by the fp64 block scale and summed in
// fp64; the fp64 sum is order-independent to ~1e-16, so any lane split gives
// the same fp32 result.
#pragma once

#include "coli_common.h"
#include "coli_args.h"


// Gate/up for one item (an expert and up to NT of its tokens) and one block
// of 32 intermediate rows, then SwiGLU and Q8_0 of the 32 h values per token.
// Four waves, eight rows each.
template <int NT, int NBJ>
__global__ __launch_bounds__(256) void k_gateup_gemv(
    const uint8_t* __restrict__ eq, const float* __restrict__ es, int64_t blob_q,
    int64_t blob_s, const int8_t* __restrict__ qx, const float* __restrict__ dx, ItemArgs items,
    const int32_t* __restrict__ slot_tok, int H, int I, int8_t* __restrict__ qh,
    float* __restrict__ dh, int32_t* __restrict__ tap, int tap_rows, int tap_stride) {
    __shared__ float hbuf[NT][32];
    const int nrb = I >> 5;
    const int it = blockIdx.x / nrb;
    const int hb = blockIdx.x - it * nrb;
    if (it >= *items.n_items) return;
    const int e = items.item_e[it], s0 = items.item_s0[it], n = items.item_n[it];
    const int BH = H >> 5;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint8_t* gate = eq + (int64_t)e * blob_q;
    const uint8_t* up = gate + (int64_t)I * (H >> 1);
    const float* gs = es + (int64_t)e * blob_s;
    const float* us = gs + I;

    uint4 xa[NT][NBJ][2];
    double xd[NT][NBJ];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        const int t = (i < n) ? slot_tok[s0 + i] : 0;
#pragma unroll
        for (int j = 0; j < NBJ; ++j) {
            const int b = lane + 64 * j;
            if (i < n && b < BH) {
                const uint4* p = reinterpret_cast<const uint4*>(qx + (int64_t)t * H + b * 32);
                xa[i][j][0] = p[0];
                xa[i][j][1] = p[1];
                xd[i][j] = (double)dx[(int64_t)t * BH + b] * 0.0625;  // undo the x16 of the codes
            } else {
                xa[i][j][0] = make_uint4(0, 0, 0, 0);
                xa[i][j][1] = make_uint4(0, 0, 0, 0);
                xd[i][j] = 0.0;
            }
        }
    }

    for (int rr = 0; rr < 8; ++rr) {
        const int r = hb * 32 + wave * 8 + rr;
        const uint8_t* grow = gate + (int64_t)r * (H >> 1);
        const uint8_t* urow = up + (int64_t)r * (H >> 1);
        uint4 wg[NBJ], wu[NBJ];
#pragma unroll
        for (int j = 0; j < NBJ; ++j) {
            const int b = lane + 64 * j;
            if (b < BH) {
                wg[j] = *reinterpret_cast<const uint4*>(grow + b * 16);
                wu[j] = *reinterpret_cast<const uint4*>(urow + b * 16);
            } else {
                wg[j] = make_uint4(0, 0, 0, 0);
                wu[j] = make_uint4(0, 0, 0, 0);
            }
        }
        const bool do_tap = tap != nullptr && (r % tap_stride) == 0;
        double pg[NT], pu[NT];
#pragma unroll
        for (int i = 0; i < NT; ++i) {
            pg[i] = 0.0;
            pu[i] = 0.0;
#pragma unroll
            for (int j = 0; j < NBJ; ++j) {
                const int dg = dot_block16(wg[j], xa[i][j][0], xa[i][j][1]);
                const int du = dot_block16(wu[j], xa[i][j][0], xa[i][j][1]);
                pg[i] += xd[i][j] * (double)dg;
                pu[i] += xd[i][j] * (double)du;
                const int b = lane + 64 * j;
                if (do_tap && i < n && b < BH)
                    tap[((int64_t)(s0 + i) * tap_rows + r / tap_stride) * BH + b] = dg / 16;
            }
            pg[i] = wave_sum_f64(pg[i]);
            pu[i] = wave_sum_f64(pu[i]);
        }
        if (lane == 0) {
#pragma unroll
            for (int i = 0; i < NT; ++i) {
                if (i < n) {
                    const float g = (float)((double)gs[r] * pg[i]);
                    const float u = (float)((double)us[r] * pu[i]);
                    hbuf[i][wave * 8 + rr] = swiglu_f32(g, u);
                }
            }
        }
    }
    __syncthreads();
    // Q8_0 of the 32 h values of each token: half a wave per token.
    if (threadIdx.x < NT * 32) {
        const int i = threadIdx.x >> 5, k = threadIdx.x & 31;
        const float v = (i < n) ? hbuf[i][k] : 0.0f;
        float a = fabsf(v);
#pragma unroll
        for (int o = 16; o > 0; o >>= 1) a = fmaxf(a, __shfl_xor(a, o, 32));
        const float dd = a / 127.0f;
        const int c = q8_code(v, dd);
        if (i < n) {
            qh[(int64_t)(s0 + i) * I + hb * 32 + q8_perm_pos(k)] = (int8_t)c;
            if (k == 0) dh[(int64_t)(s0 + i) * (I >> 5) + hb] = dd;
        }
    }
}

// Down projection for one item and 32 output rows: y_e[slot, c] in fp32.
template <int NT, int NBJ>
__global__ __launch_bounds__(256) void k_down_gemv(const uint8_t* __restrict__ eq,
                                                   const float* __restrict__ es, int64_t blob_q,
                                                   int64_t blob_s, const int8_t* __restrict__ qh,
                                                   const float* __restrict__ dh, ItemArgs items,
                                                   int H, int I, float* __restrict__ ye) {
    const int nrb = H >> 5;
    const int it = blockIdx.x / nrb;
    const int cb = blockIdx.x - it * nrb;
    if (it >= *items.n_items) return;
    const int e = items.item_e[it], s0 = items.item_s0[it], n = items.item_n[it];
    const int BI = I >> 5;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint8_t* down = eq + (int64_t)e * blob_q + (int64_t)I * H;
    const float* ds = es + (int64_t)e * blob_s + 2 * I;

    uint4 ha[NT][NBJ][2];
    double hd[NT][NBJ];
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
        for (int j = 0; j < NBJ; ++j) {
            const int b = lane + 64 * j;
            if (i < n && b < BI) {
                const uint4* p = reinterpret_cast<const uint4*>(qh + (int64_t)(s0 + i) * I + b * 32);
                ha[i][j][0] = p[0];
                ha[i][j][1] = p[1];
                hd[i][j] = (double)dh[(int64_t)(s0 + i) * BI + b] * 0.0625;
            } else {
                ha[i][j][0] = make_uint4(0, 0, 0, 0);
                ha[i][j][1] = make_uint4(0, 0, 0, 0);
                hd[i][j] = 0.0;
            }
        }

    for (int rr = 0; rr < 8; ++rr) {
        const int c = cb * 32 + wave * 8 + rr;
        const uint8_t* row = down + (int64_t)c * (I >> 1);
        uint4 w[NBJ];
#pragma unroll
        for (int j = 0; j < NBJ; ++j) {
            const int b = lane + 64 * j;
            w[j] = (b < BI) ? *reinterpret_cast<const uint4*>(row + b * 16) : make_uint4(0, 0, 0, 0);
        }
        double p[NT];
#pragma unroll
        for (int i = 0; i < NT; ++i) {
            p[i] = 0.0;
#pragma unroll
            for (int j = 0; j < NBJ; ++j)
                p[i] += hd[i][j] * (double)dot_block16(w[j], ha[i][j][0], ha[i][j][1]);
            p[i] = wave_sum_f64(p[i]);
        }
        if (lane == 0) {
#pragma unroll
            for (int i = 0; i < NT; ++i)
                if (i < n) ye[(int64_t)(s0 + i) * H + c] = (float)((double)ds[c] * p[i]);
        }
    }
}

// y[t] = fp32( sum_k w[t,k] * y_e[slot(t,k)] + y_e[slot(t,shared)] ), fp64, k ascending.
// A thread takes four consecutive columns of one token (H % 32 == 0) and
// issues the loads of up to eight slots before it adds them up.
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ ye,
                                                 const int32_t* __restrict__ slot_of,
                                                 const float* __restrict__ w, int K, int S, int H,
                                                 float* __restrict__ y, int accum) {
    const int nb = (H + 1023) >> 10;
    const int t = blockIdx.x / nb;
    const int c = ((blockIdx.x - t * nb) * 256 + threadIdx.x) * 4;
    if (c >= H) return;
    const int KS = K + S;
    const int32_t* so = slot_of + (int64_t)t * KS;
    const float* wt = w + (int64_t)t * K;
    double a[4] = {0.0, 0.0, 0.0, 0.0};
    constexpr int B = 8;
    for (int k0 = 0; k0 < K; k0 += B) {
        float4 v[B];
        double wk[B];
#pragma unroll
        for (int j = 0; j < B; ++j)
            if (k0 + j < K) {
                v[j] = *reinterpret_cast<const float4*>(ye + (int64_t)so[k0 + j] * H + c);
                wk[j] = (double)wt[k0 + j];
            }
#pragma unroll
        for (int j = 0; j < B; ++j)
            if (k0 + j < K) {
                a[0] += wk[j] * (double)v[j].x;
                a[1] += wk[j] * (double)v[j].y;
                a[2] += wk[j] * (double)v[j].z;
                a[3] += wk[j] * (double)v[j].w;
            }
    }
    if (S) {
        const float4 v = *reinterpret_cast<const float4*>(ye + (int64_t)so[K] * H + c);
        a[0] += (double)v.x;
        a[1] += (double)v.y;
        a[2] += (double)v.z;
        a[3] += (double)v.w;
    }
    float4 r = make_float4((float)a[0], (float)a[1], (float)a[2], (float)a[3]);
    float4* out = reinterpret_cast<float4*>(y + (int64_t)t * H + c);
    if (accum) {
        const float4 o = *out;
        r = make_float4(o.x + r.x, o.y + r.y, o.z + r.z, o.w + r.w);
    }
    *out = r;
}
