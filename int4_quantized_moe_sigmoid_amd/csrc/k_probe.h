// Measurement kernels, not steps of the layer: issue rates of the int8 MFMA
// forms and of the per-block epilogue of the grouped kernels, each wave
// timing its own loop with the shader clock (s_memtime). They give the
// ceiling of an exact per-block epilogue: the epilogue work per MFMA result
// is fixed by the Q8_0 format (one scaled add per row, token and 32-block).
#pragma once

#include "coli_common.h"

namespace probe {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

// kind: 0 = 8 x v_mfma_i32_16x16x32_i8 per iteration, 1 = 8 x 16x16x64,
// 2 = 4 x 32x32x32, 3 = 16 x v_mad_i64_i32, 4 = 16 x (v_cvt_f64_i32 +
// v_fma_f64), 5 = 2 x 32x32x32 each followed by the int64 epilogue of its 16
// results, 6 = the same with the fp64 epilogue, 7 = 4 x 16x16x32 with the
// int64 epilogue of their 4 results.
template <int KIND>
__global__ __launch_bounds__(256) void k_mfma_probe(int iters, int seed, long long* cycles) {
    const int lane = threadIdx.x & 63;
    v4i a = {seed + lane, seed * 3 + lane, 7 * lane, lane ^ seed};
    v4i b = {lane * 5, seed, lane + 1, seed ^ 0x55};
    long aa = ((long)a.x << 32) | (unsigned)a.y, bb = ((long)b.x << 32) | (unsigned)b.y;
    long acc64[16];
    double accd[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        acc64[i] = i;
        accd[i] = i;
    }
    v4i c4[8];
    v16i c16[4];
#pragma unroll
    for (int i = 0; i < 8; ++i) c4[i] = v4i{i, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v16i z = {};
        z[0] = i;
        c16[i] = z;
    }
    const v4i zero4 = {0, 0, 0, 0};
    const v16i zero16 = {};
    int m = (seed | 1) + lane;
    const long long t0 = __builtin_amdgcn_s_memtime();
    for (int it = 0; it < iters; ++it) {
        if constexpr (KIND == 0) {
#pragma unroll
            for (int i = 0; i < 8; ++i) c4[i] = __builtin_amdgcn_mfma_i32_16x16x32_i8(aa, bb, c4[i], 0, 0, 0);
        } else if constexpr (KIND == 1) {
#pragma unroll
            for (int i = 0; i < 8; ++i) c4[i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c4[i], 0, 0, 0);
        } else if constexpr (KIND == 2) {
#pragma unroll
            for (int i = 0; i < 4; ++i) c16[i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c16[i], 0, 0, 0);
        } else if constexpr (KIND == 3) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                acc64[i] += (long)m * (long)(a.x + i);
                asm volatile("" : "+v"(acc64[i]));
            }
        } else if constexpr (KIND == 4) {
            const double dm = (double)m;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                accd[i] += dm * (double)(a.x + i);
                asm volatile("" : "+v"(accd[i]));
            }
        } else if constexpr (KIND == 5 || KIND == 6) {
            const v16i r0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, zero16, 0, 0, 0);
            const v16i r1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, a, zero16, 0, 0, 0);
            if constexpr (KIND == 5) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    acc64[i] += (long)m * (long)r0[i];
                    asm volatile("" : "+v"(acc64[i]));
                }
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    acc64[i] += (long)(m + 1) * (long)r1[i];
                    asm volatile("" : "+v"(acc64[i]));
                }
            } else {
                const double dm = (double)m, dm1 = (double)(m + 1);
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    accd[i] += dm * (double)r0[i];
                    asm volatile("" : "+v"(accd[i]));
                }
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    accd[i] += dm1 * (double)r1[i];
                    asm volatile("" : "+v"(accd[i]));
                }
            }
        } else {
            v4i r[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) r[j] = __builtin_amdgcn_mfma_i32_16x16x32_i8(aa + j, bb, zero4, 0, 0, 0);
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc64[4 * j + i] += (long)(m + j) * (long)r[j][i];
                    asm volatile("" : "+v"(acc64[4 * j + i]));
                }
        }
        m += 3;
        // operands opaque to the compiler: every iteration does its work
        asm volatile("" : "+v"(m), "+v"(a), "+v"(b), "+v"(aa), "+v"(bb));
    }
    const long long t1 = __builtin_amdgcn_s_memtime();
    long long s = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) s += c4[i].x + c4[i].w;
#pragma unroll
    for (int i = 0; i < 4; ++i) s += c16[i][0] + c16[i][15];
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc64[i] + (long long)accd[i];
    if (lane == 0) cycles[blockIdx.x * 4 + (threadIdx.x >> 6)] = t1 - t0;
    // the results stay live (the last entry is a sink that practically never
    // receives a store)
    if (s == 0x123456789ll) cycles[gridDim.x * 4] = s;
}

}  // namespace probe
