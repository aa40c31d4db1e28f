// Host-side launch helpers shared by the library's translation units: the
// per-launch timing marks and the entry points of the kernel families, each
// defined in its own translation unit (the few-token kernels in
// launch_decode.hip, the grouped MFMA kernels in launch_prefill.hip, the
// GEMV kernels and the combine in launch_gemv.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include "coli_moe.h"
#include "coli_args.h"

// Optional per-launch timing (coli_moe_forward_profiled): mark() names the
// next launch; launch j then carries events 2j (start) and 2j + 1 (stop),
// which the packet processor stamps at the kernel's own begin and end.
struct Marks {
    hipStream_t s;
    void* const* ev = nullptr;
    const char** names = nullptr;
    int n = 0, used = 0;  // n events, used launches so far
    const char* pending = "";
    void mark(const char* name) { pending = name; }
    void take(hipEvent_t* e0, hipEvent_t* e1) {
        *e0 = *e1 = nullptr;
        if (ev && 2 * used + 1 < n) {
            *e0 = (hipEvent_t)ev[2 * used];
            *e1 = (hipEvent_t)ev[2 * used + 1];
            if (names) names[used] = pending;
        }
        ++used;
    }
};

// kernel<<<grid, block, shmem, s>>>(args...), with the launch's own start and
// stop events when profiling.
template <typename... P, typename... A>
void launch(Marks& mk, void (*kernel)(P...), dim3 grid, dim3 block, uint32_t shmem, hipStream_t s,
            A&&... args) {
    static_assert(sizeof...(P) == sizeof...(A), "kernel argument count");
    hipEvent_t e0, e1;
    mk.take(&e0, &e1);
    if (e0)
        hipExtLaunchKernelGGL(kernel, grid, block, shmem, s, e0, e1, 0u, static_cast<P>(args)...);
    else
        kernel<<<grid, block, shmem, s>>>(static_cast<P>(args)...);
}

// Width of the expert weight codes (0 reads as 4).
inline int weight_bits(const coli_moe_cfg& c) { return c.weight_bits ? c.weight_bits : 4; }

// Few-token path (up to four tokens; int2 up to two): router, fused
// gate/up + SwiGLU + Q8_0(h), down + combine.
bool small_path_fits(const coli_moe_cfg& c, int64_t T);
void launch_small(const dec::DecArgs& a, int bits, hipStream_t s, Marks& mk);

// Top-k of T tokens' logits with the few-token path's wave selection
// (launch_decode.hip); E <= 256, K <= 16.
void launch_topk_wave(const double* logits, const float* bias, int64_t T, int E, int K,
                      int norm, double rho, GroupSel gsel, int32_t* idx, float* wts,
                      hipStream_t s, Marks& mk);

// Grouped int8-MFMA gate/up and down over n_it work items of kt (32 or 64)
// tokens, with the integer block scales of x and h when pa.mx is set.
void launch_pf_path(const pf::PfArgs& pa, int bits, int kt, int64_t T, int64_t n_slots,
                    int64_t n_it, hipStream_t s, Marks& mk);

// GEMV gate/up and down (int4) over max_items items of up to 4 tokens.
void launch_gemv_path(const coli_moe_weights* w, int64_t blob_q, int64_t blob_s,
                      const int8_t* qx, const float* dx, ItemArgs it, const int32_t* slot_tok,
                      int8_t* qh, float* dh, float* ye, int32_t* tap, int tap_rows,
                      int tap_stride, int64_t T, int64_t max_items, hipStream_t s, Marks& mk);

// y = sum_k w_k ye[slot(t, k)] + ye[slot(t, shared)] (y += with accum).
void launch_combine(const float* ye, const int32_t* slot_of, const float* wts, int K, int S,
                    int H, float* y, int64_t T, int accum, hipStream_t s, Marks& mk);
