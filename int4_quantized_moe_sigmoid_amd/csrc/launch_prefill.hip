// Launches of the grouped int8-MFMA kernels (k_prefill.h).
#include "coli_launch.h"
#include "k_prefill.h"
#include "k_prefill32.h"

namespace {

// The grouped MFMA kernels of one weight width: gate/up (with debug taps or
// not), the integer form of the h scales, down; KT tokens per item.
template <int BITS, typename HS>
void launch_pf(int kt, bool tap, dim3 g1, dim3 g2, const pf::PfArgs& pa, HS h_scales,
               hipStream_t s, Marks& mk) {
    mk.mark("pf_gateup");
    if (kt == 64) {
        if (tap) launch(mk, pf::k_pf_gateup<BITS, 64, true>, g1, 256, 0, s, pa);
        else launch(mk, pf::k_pf_gateup<BITS, 64, false>, g1, 256, 0, s, pa);
    } else {
        if (tap) launch(mk, pf::k_pf_gateup<BITS, 32, true>, g1, 256, 0, s, pa);
        else launch(mk, pf::k_pf_gateup<BITS, 32, false>, g1, 256, 0, s, pa);
    }
    h_scales();
    mk.mark("pf_down");
    if (kt == 64) launch(mk, pf::k_pf_down<BITS, 64>, g2, 256, 0, s, pa);
    else launch(mk, pf::k_pf_down<BITS, 32>, g2, 256, 0, s, pa);
}

// 64-token items with int4 weights: gate/up on the 32x32x32 kernel (128 h
// rows per workgroup), down on the 16x16x32 kernel. Measured on the 8-layer
// stack at 4096 tokens: gate/up 2598 us against 2707 us; the 32x32 down
// kernel (256 rows per workgroup, 2 waves per SIMD) took 1576 us against
// 1467 us, and with 32-token items the 32x32 gate/up kernel loses to the
// 16x16 one at its higher occupancy (prefill T=512: 808 against 749 us).
template <typename HS>
void launch_pf32_64(bool tap, dim3 g1, dim3 g2, const pf::PfArgs& pa, HS h_scales, hipStream_t s,
                    Marks& mk) {
    mk.mark("pf_gateup");
    if (tap) launch(mk, pf::k_pf32_gateup<4, 64, true>, g1, 256, 0, s, pa);
    else launch(mk, pf::k_pf32_gateup<4, 64, false>, g1, 256, 0, s, pa);
    h_scales();
    mk.mark("pf_down");
    launch(mk, pf::k_pf_down<4, 64>, g2, 256, 0, s, pa);
}

// Grid of a gate/up kernel with nrt row tiles per item (pf::work_of): a
// multiple of 8 blocks covering every (item, row tile) of up to n_it items.
dim3 gateup_grid(int64_t nrt, int64_t n_it) { return dim3((unsigned)((nrt * n_it + 7) / 8 * 8)); }

}  // namespace

void launch_pf_path(const pf::PfArgs& pa, int bits, int kt, int64_t T, int64_t n_slots,
                    int64_t n_it, hipStream_t s, Marks& mk) {
    const int H = pa.H, I = pa.I;
    const bool int_scales = pa.mx != nullptr;
    if (int_scales) {
        mk.mark("scale_int_x");
        launch(mk, pf::k_scale_int, (unsigned)((T + 3) / 4), 256, 0, s, pa.dx, T, H / 32,
               const_cast<int32_t*>(pa.mx), const_cast<int32_t*>(pa.ex));
    }
    const dim3 g1 = gateup_grid(I / pf::kRows, n_it);
    const dim3 g2((unsigned)(((H + pf::kDnRows - 1) / pf::kDnRows) * n_it));
    auto h_scales = [&] {
        if (!int_scales) return;
        mk.mark("scale_int_h");
        launch(mk, pf::k_scale_int, (unsigned)((n_slots + 3) / 4), 256, 0, s, pa.dh, n_slots,
               I / 32, const_cast<int32_t*>(pa.mh), const_cast<int32_t*>(pa.eh));
    };
    const bool tap = pa.tap != nullptr;
    if (bits == 4 && kt == 64 && I % pf::kRows32 == 0) {
        const dim3 h1 = gateup_grid(I / pf::kRows32, n_it);
        launch_pf32_64(tap, h1, g2, pa, h_scales, s, mk);
    } else if (bits == 4) launch_pf<4>(kt, tap, g1, g2, pa, h_scales, s, mk);
    else if (bits == 8) launch_pf<8>(kt, tap, g1, g2, pa, h_scales, s, mk);
    else launch_pf<2>(kt, tap, g1, g2, pa, h_scales, s, mk);
}
