// Launches of the GEMV kernels and the combine (k_gemv.h).
#include "coli_launch.h"
#include "k_gemv.h"

namespace {

template <int NT>
void launch_gateup_nt(int nbj, dim3 grid, hipStream_t s, const coli_moe_weights* w,
                      int64_t blob_q, int64_t blob_s, const int8_t* qx, const float* dx,
                      ItemArgs it, const int32_t* slot_tok, int8_t* qh, float* dh, int32_t* tap,
                      int tap_rows, int tap_stride, Marks& mk) {
    const int H = w->cfg.hidden, I = w->cfg.inter;
#define COLI_GU(NBJ)                                                                          \
    launch(mk, k_gateup_gemv<NT, NBJ>, grid, 256, 0, s, w->experts_q, w->experts_scale, blob_q, blob_s, \
                                                qx, dx, it, slot_tok, H, I, qh, dh, tap,        \
                                                tap_rows, tap_stride)
    switch (nbj) {
        case 1: COLI_GU(1); break;
        case 2: COLI_GU(2); break;
        case 3: COLI_GU(3); break;
        default: COLI_GU(4); break;
    }
#undef COLI_GU
}

template <int NT>
void launch_down_nt(int nbj, dim3 grid, hipStream_t s, const coli_moe_weights* w,
                    int64_t blob_q, int64_t blob_s, const int8_t* qh, const float* dh,
                    ItemArgs it, float* ye, Marks& mk) {
    const int H = w->cfg.hidden, I = w->cfg.inter;
#define COLI_DN(NBJ)                                                                          \
    launch(mk, k_down_gemv<NT, NBJ>, grid, 256, 0, s, w->experts_q, w->experts_scale, blob_q, blob_s, \
                                              qh, dh, it, H, I, ye)
    switch (nbj) {
        case 1: COLI_DN(1); break;
        case 2: COLI_DN(2); break;
        case 3: COLI_DN(3); break;
        default: COLI_DN(4); break;
    }
#undef COLI_DN
}

}  // namespace

void launch_gemv_path(const coli_moe_weights* w, int64_t blob_q, int64_t blob_s,
                      const int8_t* qx, const float* dx, ItemArgs it, const int32_t* slot_tok,
                      int8_t* qh, float* dh, float* ye, int32_t* tap, int tap_rows,
                      int tap_stride, int64_t T, int64_t max_items, hipStream_t s, Marks& mk) {
    const int H = w->cfg.hidden, I = w->cfg.inter;
    const int ch = 4;                            // tokens per item
    const int nt = (T >= ch) ? ch : (int)T;      // tokens per item at most
    const int nbj_h = (H / 32 + 63) / 64;
    const int nbj_i = (I / 32 + 63) / 64;
    mk.mark("gateup");
    {
        dim3 grid((unsigned)((I / 32) * max_items));
        if (nt <= 1)
            launch_gateup_nt<1>(nbj_h, grid, s, w, blob_q, blob_s, qx, dx, it, slot_tok, qh, dh,
                                tap, tap_rows, tap_stride, mk);
        else if (nt <= 2)
            launch_gateup_nt<2>(nbj_h, grid, s, w, blob_q, blob_s, qx, dx, it, slot_tok, qh, dh,
                                tap, tap_rows, tap_stride, mk);
        else
            launch_gateup_nt<4>(nbj_h, grid, s, w, blob_q, blob_s, qx, dx, it, slot_tok, qh, dh,
                                tap, tap_rows, tap_stride, mk);
    }
    mk.mark("down");
    {
        dim3 grid((unsigned)((H / 32) * max_items));
        if (nt <= 1)
            launch_down_nt<1>(nbj_i, grid, s, w, blob_q, blob_s, qh, dh, it, ye, mk);
        else if (nt <= 2)
            launch_down_nt<2>(nbj_i, grid, s, w, blob_q, blob_s, qh, dh, it, ye, mk);
        else
            launch_down_nt<4>(nbj_i, grid, s, w, blob_q, blob_s, qh, dh, it, ye, mk);
    }
}

void launch_combine(const float* ye, const int32_t* slot_of, const float* wts, int K, int S,
                    int H, float* y, int64_t T, int accum, hipStream_t s, Marks& mk) {
    dim3 grid((unsigned)(((H + 1023) / 1024) * T));
    launch(mk, k_combine, grid, 256, 0, s, ye, slot_of, wts, K, S, H, y, accum);
}
