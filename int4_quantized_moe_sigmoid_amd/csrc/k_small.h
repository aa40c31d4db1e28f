// Elementwise-class kernels: Q8_0 quantisation, int4 packing, RMSNorm.
// All three are HBM-bound streams: coalesced 16-byte loads, one pass.
#pragma once

#include "coli_common.h"

// Q8_0 over blocks of 32 consecutive fp32 values (a [T, dim] row-major array
// is a flat run of T*dim/32 blocks). Four lanes share a block, eight values
// each; the block max is a 2-step butterfly. LAYOUT 0 keeps the natural
// order (int8 weights); 1 stores each group of 8 as (e0,e2,e4,e6,e1,e3,e5,e7),
// the order the int4 dot kernels consume; 2 each group of 16 as (e0,e4,e8,
// e12,e1,e5,e9,e13,e2,e6,e10,e14,e3,e7,e11,e15), the int2 order.
template <int LAYOUT>
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
    // LAYOUT 2: a 16-element group spans this lane (part even: elements
    // 0..7, odd: 8..15) and its neighbour; the group's order is (e0 e4 e8 e12
    // e1 e5 e9 e13 | e2 e6 e10 e14 e3 e7 e11 e15), the even part writing the
    // first eight bytes
    int p[8];
    if (LAYOUT == 2) {
#pragma unroll
        for (int i = 0; i < 8; ++i) p[i] = __shfl_xor(c[i], 1, 64);
    }
    if (blk < nblk) {
        uint2 o;
        if (LAYOUT == 1) {
            o.x = pack4_i8(c[0], c[2], c[4], c[6]);
            o.y = pack4_i8(c[1], c[3], c[5], c[7]);
        } else if (LAYOUT == 2) {
            if ((part & 1) == 0) {
                o.x = pack4_i8(c[0], c[4], p[0], p[4]);
                o.y = pack4_i8(c[1], c[5], p[1], p[5]);
            } else {
                o.x = pack4_i8(p[2], p[6], c[2], c[6]);
                o.y = pack4_i8(p[3], p[7], c[3], c[7]);
            }
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

// Symmetric BITS-wide code of w under row scale s: clamp(rint(w / s), +-Q),
// Q = 2^(BITS-1) - 1; 0 when s = 0.
template <int BITS>
__device__ __forceinline__ int wcode(float w, float s) {
    constexpr float Q = (float)((1 << (BITS - 1)) - 1);
    if (s == 0.0f) return 0;
    float r = __builtin_rintf(w / s);
    r = fminf(fmaxf(r, -Q), Q);
    return (int)r;
}

// One workgroup per row: block max |w|, s = max / Q, then 4 codes per lane
// packed little end first (int4: 2 bytes, int8: 4 bytes, int2: 1 byte).
template <int BITS>
__global__ __launch_bounds__(256) void k_pack_bits(const float* __restrict__ w, int64_t cols,
                                                   uint8_t* __restrict__ q,
                                                   float* __restrict__ scale) {
    constexpr uint32_t M = (1u << BITS) - 1u;
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
    const float s = amax / (float)((1 << (BITS - 1)) - 1);
    if (tid == 0) scale[r] = s;
    uint8_t* out = q + r * (cols * BITS / 8);
    for (int64_t j = (int64_t)tid * 4; j < cols; j += 1024) {
        const float4 v = *reinterpret_cast<const float4*>(row + j);
        const uint32_t b = ((uint32_t)wcode<BITS>(v.x, s) & M) |
                           (((uint32_t)wcode<BITS>(v.y, s) & M) << BITS) |
                           (((uint32_t)wcode<BITS>(v.z, s) & M) << (2 * BITS)) |
                           (((uint32_t)wcode<BITS>(v.w, s) & M) << (3 * BITS));
        uint8_t* o = out + j * BITS / 8;
        if (BITS == 8) *reinterpret_cast<uint32_t*>(o) = b;
        else if (BITS == 4) *reinterpret_cast<uint16_t*>(o) = (uint16_t)b;
        else *o = (uint8_t)b;
    }
}

// RMSNorm with unit gain, one workgroup per token, sums in fp64.
// vec: dim a multiple of 4 up to 1024 kV (x and out 16-byte aligned); the
// row is then read once, as float4 loads all in flight together, and written
// from registers (out may alias x: every read of the row precedes the
// barrier, every write follows it).
__global__ __launch_bounds__(256) void k_rmsnorm(const float* x, int64_t dim, double eps,
                                                 float* out, int vec) {
    constexpr int kV = 8;
    __shared__ double red[4];
    const int64_t t = blockIdx.x;
    const float* row = x + t * dim;
    double ss = 0.0;
    float4 v[kV];
    if (vec) {
#pragma unroll
        for (int u = 0; u < kV; ++u) {
            const int64_t i = 4 * (int64_t)threadIdx.x + 1024 * u;
            v[u] = (i < dim) ? *reinterpret_cast<const float4*>(row + i) : make_float4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < kV; ++u)
            ss += (double)v[u].x * v[u].x + (double)v[u].y * v[u].y + (double)v[u].z * v[u].z +
                  (double)v[u].w * v[u].w;
    } else {
        for (int64_t i = threadIdx.x; i < dim; i += 256) {
            const double e = (double)row[i];
            ss += e * e;
        }
    }
    ss = wave_sum_f64(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    const double tot = (red[0] + red[1]) + (red[2] + red[3]);
    const double rms = sqrt(tot / (double)dim + eps);
    if (vec) {
#pragma unroll
        for (int u = 0; u < kV; ++u) {
            const int64_t i = 4 * (int64_t)threadIdx.x + 1024 * u;
            if (i < dim)
                *reinterpret_cast<float4*>(out + t * dim + i) =
                    make_float4((float)((double)v[u].x / rms), (float)((double)v[u].y / rms),
                                (float)((double)v[u].z / rms), (float)((double)v[u].w / rms));
        }
    } else {
        for (int64_t i = threadIdx.x; i < dim; i += 256)
            out[t * dim + i] = (float)((double)row[i] / rms);
    }
}

// Streaming read of n16 16-byte words (the HBM read ceiling the layer's
// kernels are compared with): every workgroup streams one contiguous chunk,
// sixteen nontemporal loads per lane in flight (a 64 KB window per
// workgroup); an XOR checksum per wave is folded into *sink so no load is
// dead. Few long streams (one workgroup per CU) read fastest: measured
// 7.2 TB/s against 5.9 TB/s for a grid-stride loop over 2048 workgroups.
typedef unsigned v4u_s __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(256) void k_stream_read(const v4u_s* __restrict__ p, int64_t n16,
                                                     uint32_t* sink) {
    constexpr int U = 16;
    const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const int64_t b0 = (int64_t)blockIdx.x * per;
    const int64_t b1 = b0 + per < n16 ? b0 + per : n16;
    v4u_s acc = {0u, 0u, 0u, 0u};
    int64_t i = b0 + threadIdx.x;
    for (; i + (U - 1) * 256 < b1; i += U * 256) {
        v4u_s v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(p + i + u * 256);
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u];
    }
    for (; i < b1; i += 256) acc ^= __builtin_nontemporal_load(p + i);
    uint32_t r = acc.x ^ acc.y ^ acc.z ^ acc.w;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) r ^= (uint32_t)__shfl_xor((int)r, o, 64);
    if ((threadIdx.x & 63) == 0) atomicXor(sink, r);
}

// FP8 e4m3 code -> fp32 (1 sign, 4 exponent bits with bias 7, 3 mantissa
// bits; exponent 0 is subnormal m * 2^-9; no infinities). The NaN code
// S.1111.111 converts to 0.
__device__ __forceinline__ float e4m3_value(uint32_t b) {
    const uint32_t sign = (b & 0x80u) << 24, e = (b >> 3) & 0xFu, m = b & 7u;
    if (e == 15u && m == 7u) return 0.0f;
    if (e == 0u) return __uint_as_float(sign | __float_as_uint((float)m * 0x1p-9f));
    return __uint_as_float(sign | ((e + 120u) << 23) | (m << 20));
}

// FP8 -> fp32 -> int4 for one row per workgroup: w = e4m3(q8) * bs[r/128][c/128]
// (one fp32 rounding), then the pack of k_pack_bits<4>. Four codes per thread.
__global__ __launch_bounds__(256) void k_pack_fp8_int4(const uint8_t* __restrict__ q8,
                                                       const float* __restrict__ bs,
                                                       int64_t cols, uint8_t* __restrict__ q,
                                                       float* __restrict__ scale) {
    __shared__ float red[4];
    const int64_t r = blockIdx.x;
    const uint8_t* row = q8 + r * cols;
    const float* bsr = bs + (r >> 7) * ((cols + 127) >> 7);
    const int tid = threadIdx.x;
    auto load4 = [&](int64_t j, float (&v)[4]) {
        const uint32_t c = *reinterpret_cast<const uint32_t*>(row + j);
        const float sc = bsr[j >> 7];  // the 4 codes share one 128-column block
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = e4m3_value((c >> (8 * i)) & 0xFFu) * sc;
    };
    float amax = 0.0f;
    for (int64_t j = (int64_t)tid * 4; j < cols; j += 1024) {
        float v[4];
        load4(j, v);
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
    }
    amax = wave_max_f32(amax);
    if ((tid & 63) == 0) red[tid >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float s = amax / 7.0f;
    if (tid == 0) scale[r] = s;
    uint8_t* out = q + r * (cols / 2);
    for (int64_t j = (int64_t)tid * 4; j < cols; j += 1024) {
        float v[4];
        load4(j, v);
        const uint32_t b = (uint32_t)(int4_code(v[0], s) & 0xF) |
                           ((uint32_t)(int4_code(v[1], s) & 0xF) << 4) |
                           ((uint32_t)(int4_code(v[2], s) & 0xF) << 8) |
                           ((uint32_t)(int4_code(v[3], s) & 0xF) << 12);
        *reinterpret_cast<uint16_t*>(out + j / 2) = (uint16_t)b;
    }
}

// Whether the int4 codes of a row with scale s can be taken from a product
// instead of the quotient w / s: s in [2^-100, 2^100] keeps 1/s a normal number.
__device__ __forceinline__ bool int4_fast_ok(float s) {
    return s >= 0x1p-100f && s <= 0x1p100f;
}

// Four e4m3 codes of a dword with the NaN codes (magnitude 0x7F) replaced by
// zero bytes, bytewise without branches: a magnitude byte plus one reaches
// 0x80 only for 0x7F, and no byte carries into the next.
__device__ __forceinline__ uint32_t e4m3_zero_nan4(uint32_t c) {
    const uint32_t nan = ((c & 0x7F7F7F7Fu) + 0x01010101u) & 0x80808080u;
    return c & ~(nan | (nan - (nan >> 7)));
}

// FP8 -> int4 for rows whose length is a multiple of 1024 codes, up to 8192:
// one wave per row (CPL 16-code chunks per lane), or 8 / CPL rows per wave
// when CPL divides 8, so every lane issues up to eight 16-byte loads at once.
// No LDS, no barrier. Same result as k_pack_fp8_int4, bit for bit:
//  * row maximum: e4m3 magnitudes order like their 7-bit codes and fp32
//    rounding is monotone, so max_j |fl(e_j * bs)| = |fl(max_j |e_j| * bs)|
//    within a 16-code chunk (one block scale): a packed 16-bit integer
//    maximum of the magnitude bytes, then one conversion and one product per
//    chunk, then a wave reduction;
//  * codes: t = fl(e * m + 8) with m = fl(bs * fl(1/s)) differs from
//    fl(w / s) + 8 by at most 7 * 4 * 2^-24 (three roundings in m and e * m,
//    one in w) + 2^-21 (the add) + 7 * 2^-24 (the quotient) < 2.6e-6, so when
//    t lies 4e-6 or more from every half-integer, rint(t) - 8 is the code.
//    Otherwise (rare), or when s is outside [2^-100, 2^100], the lane redoes
//    the chunk as clamp(rint(fl(e * bs) / s)). An all-zero row (s = 0) takes
//    the product path with 1/s replaced by 0;
//  * packing: rint(t) in [1, 15] is the offset-binary code, written into its
//    byte by a float -> u8 conversion (exact on integers); two bytes per nibble
//    pair are merged with a shift, eight codes gathered with one byte permute,
//    and xor 8 per nibble turns offset binary into two's complement.
template <int CPL>
__global__ __launch_bounds__(256) void k_pack_fp8_int4_wave(const uint8_t* __restrict__ q8,
                                                            const float* __restrict__ bs,
                                                            int64_t rows, uint8_t* __restrict__ q,
                                                            float* __restrict__ scale) {
    typedef unsigned v4u __attribute__((ext_vector_type(4)));
    typedef unsigned v2u __attribute__((ext_vector_type(2)));
    typedef unsigned short v2h __attribute__((ext_vector_type(2)));
    constexpr int RPW = (8 % CPL == 0) ? 8 / CPL : 1;  // rows per wave
    constexpr int NCH = RPW * CPL;                       // chunks per lane
    constexpr int64_t cols = 1024 * CPL;
    constexpr int nbc = (int)(cols / 128);
    const int lane = threadIdx.x & 63;
    const int64_t r0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * RPW;
    if (r0 >= rows) return;
    v4u c[NCH];
    float sc[NCH];
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int64_t r = min(r0 + i / CPL, rows - 1);  // a ragged last wave rereads its last row
        const int j = lane + 64 * (i % CPL);            // chunk within the row
        c[i] = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(q8 + r * cols) + j);
        sc[i] = bs[(r >> 7) * nbc + (j >> 3)];          // 16 codes inside one 128-column block
    }
#pragma unroll
    for (int i = 0; i < NCH; ++i)
#pragma unroll
        for (int d = 0; d < 4; ++d) c[i][d] = e4m3_zero_nan4(c[i][d]);
#pragma unroll
    for (int g = 0; g < RPW; ++g) {
        const int64_t r = r0 + g;
        float amax = 0.0f;
#pragma unroll
        for (int i = g * CPL; i < (g + 1) * CPL; ++i) {
            v2h ev = {0, 0}, od = {0, 0};
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                ev = __builtin_elementwise_max(ev, __builtin_bit_cast(v2h, c[i][d] & 0x007F007Fu));
                od = __builtin_elementwise_max(od, __builtin_bit_cast(v2h, c[i][d] & 0x7F007F00u));
            }
            const uint32_t mag = max(max((uint32_t)ev[0], (uint32_t)ev[1]),
                                     max((uint32_t)od[0], (uint32_t)od[1]) >> 8);
            amax = fmaxf(amax, fabsf(__builtin_amdgcn_cvt_f32_fp8((int)mag, 0) * sc[i]));
        }
        amax = wave_max_f32(amax);
        const float s = amax / 7.0f;
        if (r >= rows) break;
        if (lane == 0) scale[r] = s;
        const bool fast = s == 0.0f || int4_fast_ok(s);
        const float inv = (s == 0.0f || !fast) ? 0.0f : 1.0f / s;
        uint8_t* out = q + r * (cols / 2);
#pragma unroll
        for (int i = g * CPL; i < (g + 1) * CPL; ++i) {
            // a chunk of zeros may have bs far above s: keep m finite (any
            // chunk with a nonzero code has m <= 7 / 2^-9)
            const float m = fminf(sc[i] * inv, 0x1p100f);
            uint32_t b[4];
            float dmax = 0.0f;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[i][d], false);
                const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[i][d], true);
                const float e4[4] = {lo[0], lo[1], hi[0], hi[1]};
                uint32_t x = 0;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const float t = fmaf(e4[k], m, 8.0f);
                    const float rt = __builtin_rintf(t);
                    dmax = fmaxf(dmax, fabsf(t - rt));
                    x = __builtin_amdgcn_cvt_pk_u8_f32(rt, k, x);
                }
                b[d] = x;
            }
            if (!fast || dmax > 0.5f - 4e-6f) {  // s != 0 here
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[i][d], false);
                    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[i][d], true);
                    const float e4[4] = {lo[0], lo[1], hi[0], hi[1]};
                    uint32_t x = 0;
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const float w = e4[k] * sc[i];
                        const float cq = fminf(fmaxf(__builtin_rintf(w / s), -7.0f), 7.0f);
                        x = __builtin_amdgcn_cvt_pk_u8_f32(cq + 8.0f, k, x);
                    }
                    b[d] = x;
                }
            }
            v2u o;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t zl = b[2 * h] | (b[2 * h] >> 4);
                const uint32_t zh = b[2 * h + 1] | (b[2 * h + 1] >> 4);
                o[h] = __builtin_amdgcn_perm(zh, zl, 0x06040200u) ^ 0x88888888u;
            }
            reinterpret_cast<v2u*>(out)[lane + 64 * (i % CPL)] = o;
        }
    }
}
