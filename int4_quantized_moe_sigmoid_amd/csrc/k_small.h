// Elementwise-class kernels: Q8_0 quantisation, int4 packing, RMSNorm.
// All three are HBM-bound streams: coalesced 16-byte loads, one pass.
#pragma once

#include "coli_common.h"

// Q8_0 over blocks of 32 consecutive fp32 values (a [T, dim] row-major array
// is a flat run of T*dim/32 blocks). Four lanes share a block, eight values
// each; the block max is a 2-step butterfly. PERM stores each group of 8 as
// (e0,e2,e4,e6,e1,e3,e5,e7), the order the int4 dot kernels consume.
template <bool PERM>
__global__ __launch_bounds__(256) void k_quant_q8(const float* __restrict__ x, int64_t nblk,
                                                  int8_t* __restrict__ q, float* __restrict__ d) {
    const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t blk = g >> 2;
    const int part = (int)(g & 3);
    float v[8];
    if (blk < nblk) {
        const float4* p = reinterpret_cast<const float4*>(x + blk * 32 + part * 8);
        const float4 a = p[0], b = p[1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = 0.0f;
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
    const float dd = amax / 127.0f;
    int c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = q8_code(v[i], dd);
    if (blk < nblk) {
        uint2 o;
        if (PERM) {
            o.x = pack4_i8(c[0], c[2], c[4], c[6]);
            o.y = pack4_i8(c[1], c[3], c[5], c[7]);
        } else {
            o.x = pack4_i8(c[0], c[1], c[2], c[3]);
            o.y = pack4_i8(c[4], c[5], c[6], c[7]);
        }
        *reinterpret_cast<uint2*>(q + blk * 32 + part * 8) = o;
        if (part == 0) d[blk] = dd;
    }
}

__device__ __forceinline__ int int4_code(float w, float s) {
    if (s == 0.0f) return 0;
    float r = __builtin_rintf(w / s);
    r = fminf(fmaxf(r, -7.0f), 7.0f);
    return (int)r;
}

// One workgroup per row: block max |w|, s = max/7, then 4 codes -> 2 bytes per lane.
__global__ __launch_bounds__(256) void k_pack_int4(const float* __restrict__ w, int64_t cols,
                                                   uint8_t* __restrict__ q,
                                                   float* __restrict__ scale) {
    __shared__ float red[4];
    const int64_t r = blockIdx.x;
    const float* row = w + r * cols;
    const int tid = threadIdx.x;
    float amax = 0.0f;
    for (int64_t j = (int64_t)tid * 4; j < cols; j += 1024) {
        const float4 v = *reinterpret_cast<const float4*>(row + j);
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    }
    amax = wave_max_f32(amax);
    if ((tid & 63) == 0) red[tid >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float s = amax / 7.0f;
    if (tid == 0) scale[r] = s;
    uint8_t* out = q + r * (cols / 2);
    for (int64_t j = (int64_t)tid * 4; j < cols; j += 1024) {
        const float4 v = *reinterpret_cast<const float4*>(row + j);
        const uint32_t b = (uint32_t)(int4_code(v.x, s) & 0xF) |
                           ((uint32_t)(int4_code(v.y, s) & 0xF) << 4) |
                           ((uint32_t)(int4_code(v.z, s) & 0xF) << 8) |
                           ((uint32_t)(int4_code(v.w, s) & 0xF) << 12);
        *reinterpret_cast<uint16_t*>(out + j / 2) = (uint16_t)b;
    }
}

// RMSNorm with unit gain, one workgroup per token, sums in fp64.
__global__ __launch_bounds__(256) void k_rmsnorm(const float* x, int64_t dim, double eps,
                                                 float* out) {
    __shared__ double red[4];
    const int64_t t = blockIdx.x;
    const float* row = x + t * dim;
    double ss = 0.0;
    for (int64_t i = threadIdx.x; i < dim; i += 256) {
        const double v = (double)row[i];
        ss += v * v;
    }
    ss = wave_sum_f64(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    const double tot = (red[0] + red[1]) + (red[2] + red[3]);
    const double rms = sqrt(tot / (double)dim + eps);
    for (int64_t i = threadIdx.x; i < dim; i += 256) out[t * dim + i] = (float)((double)row[i] / rms);
}
