// Device helpers shared by the gfx950 kernels of the MoE layer library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define COLI_WAVE 64

// Wave-wide reductions (64 lanes, butterfly over ds_bpermute / DPP).
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

// Packed int4 nibbles -> int8 lanes scaled by 16 (no sign-extension work):
// for a dword holding 8 codes c0..c7 (byte m = c_2m | c_2m+1 << 4),
//   lo16 = bytes 16*(c0, c2, c4, c6), hi16 = bytes 16*(c1, c3, c5, c7)
// because moving a 4-bit two's complement code into the top nibble of a byte
// makes that byte the int8 value 16*code.
__device__ __forceinline__ int nib_lo16(uint32_t x) { return (int)((x << 4) & 0xF0F0F0F0u); }
__device__ __forceinline__ int nib_hi16(uint32_t x) { return (int)(x & 0xF0F0F0F0u); }

// 16 * (exact int32 dot of one 32-wide block): w holds the block's 32 int4
// codes as packed (16 bytes), a0/a1 hold the 32 int8 activations in the
// library's 8-group order (e0,e2,e4,e6,e1,e3,e5,e7 per group of 8).
__device__ __forceinline__ int dot_block16(uint4 w, uint4 a0, uint4 a1) {
    int acc = 0;
    acc = __builtin_amdgcn_sdot4(nib_lo16(w.x), (int)a0.x, acc, false);
    acc = __builtin_amdgcn_sdot4(nib_hi16(w.x), (int)a0.y, acc, false);
    acc = __builtin_amdgcn_sdot4(nib_lo16(w.y), (int)a0.z, acc, false);
    acc = __builtin_amdgcn_sdot4(nib_hi16(w.y), (int)a0.w, acc, false);
    acc = __builtin_amdgcn_sdot4(nib_lo16(w.z), (int)a1.x, acc, false);
    acc = __builtin_amdgcn_sdot4(nib_hi16(w.z), (int)a1.y, acc, false);
    acc = __builtin_amdgcn_sdot4(nib_lo16(w.w), (int)a1.z, acc, false);
    acc = __builtin_amdgcn_sdot4(nib_hi16(w.w), (int)a1.w, acc, false);
    return acc;
}

// Position of element k (0..31) of a block in the 8-group order.
__device__ __forceinline__ int q8_perm_pos(int k) {
    const int m = k & 7;
    return (k & ~7) + ((m & 1) ? 4 + (m >> 1) : (m >> 1));
}

// Q8_0 code of v for block scale d (d == 0 -> 0); IEEE division, rint.
__device__ __forceinline__ int q8_code(float v, float d) {
    if (d == 0.0f) return 0;
    float r = __builtin_rintf(v / d);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (int)r;
}

__device__ __forceinline__ uint32_t pack4_i8(int a, int b, int c, int d) {
    return (uint32_t)(a & 0xFF) | ((uint32_t)(b & 0xFF) << 8) | ((uint32_t)(c & 0xFF) << 16) |
           ((uint32_t)(d & 0xFF) << 24);
}

// SiLU(g) * u in double, rounded to fp32.
__device__ __forceinline__ float swiglu_f32(float g, float u) {
    const double z = (double)g;
    const double s = z / (1.0 + exp(-z));
    return (float)(s * (double)u);
}

// Group-limited expert selection (the topk_method knob of the GLM-5.2-colibri
// architecture page, section on routing options, read as DeepSeek-V3's
// group-limited routing). The E experts form ng groups of gs consecutive
// experts; a group's score is the sum of its two largest biased scores c (its
// only c when gs = 1); the tg groups with the largest scores stay eligible,
// ties to the lower group index. Called by one whole wave with the c of the E
// experts in c_lds (written by this wave); returns, in every lane, the bit
// mask of the kept groups (ng <= 64).
struct GroupSel {
    int ng, gs, tg;  // ng <= 1: no groups
};

__device__ __forceinline__ unsigned long long group_keep_mask(const double* c_lds, GroupSel g) {
    const int lane = threadIdx.x & 63;
    double score = -__builtin_inf();
    if (lane < g.ng) {
        const double* p = c_lds + lane * g.gs;
        double a = -__builtin_inf(), b = -__builtin_inf();
        for (int i0 = 0; i0 < g.gs; i0 += 8) {  // eight loads in flight per round
            double v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = p[min(i0 + u, g.gs - 1)];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                if (i0 + u >= g.gs) break;
                if (v[u] > a) {
                    b = a;
                    a = v[u];
                } else if (v[u] > b) {
                    b = v[u];
                }
            }
        }
        score = g.gs > 1 ? a + b : a;
    }
    int rank = 0;
    for (int j = 0; j < g.ng; ++j) {
        const double o = __shfl(score, j, 64);
        rank += (o > score || (o == score && j < lane)) ? 1 : 0;
    }
    return __ballot(lane < g.ng && rank < g.tg);
}
