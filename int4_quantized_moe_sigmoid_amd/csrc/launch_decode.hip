// Launches of the few-token kernels (k_decode.h).
#include <algorithm>

#include "coli_launch.h"
#include "k_decode.h"

// Few-token path: three fused kernels (k_decode.h), every weight width.
// Shapes it covers: hidden <= 6144, intermediate <= 2048, <= 256 routed
// experts; up to four tokens (int2: two, where the grouped MFMA kernels
// overtake it, their code expansion being paid once per token there).
bool small_path_fits(const coli_moe_cfg& c, int64_t T) {
    const int max_tok = weight_bits(c) == 2 ? 2 : 4;
    return T <= max_tok && T * c.top_k <= dec::kMaxEntries && c.hidden <= 6144 &&
           c.inter <= 2048 && c.inter % 64 == 0 && c.n_experts <= 256;
}

template <int NT, int NBJH, bool TAP, int BITS>
void launch_small_tap(const dec::DecArgs& a, hipStream_t s, Marks& mk) {
    const int nrb = a.I / 32;
    mk.mark("dec_router");
    const int qb = (a.T * (a.H / 32) + 7) / 8;  // workgroups needed for Q8_0(x)
    launch(mk, dec::k_dec_router<NT, BITS>, (a.E > qb) ? a.E : qb, 256, 0, s, a);
    mk.mark("dec_gateup");
    const int um = (a.T * a.K < a.E) ? a.T * a.K : a.E;
    // one token: a workgroup per h-block of every expert that can be in use;
    // several: the shared expert's h-blocks, then work units of nrb / 2
    // workgroups (an expert with one token takes one unit, with several two,
    // so never more units than entries T K, nor than 2 E)
    const int gu = (NT > 1) ? a.S * nrb + std::min(a.T * a.K, 2 * a.E) * (nrb / 2)
                            : (a.S + um) * nrb;
    launch(mk, dec::k_dec_gateup<NT, NBJH, TAP, BITS>, gu, 256, 0, s, a);
    mk.mark("dec_down");
    if (NT == 4)
        launch(mk, dec::k_dec_down_x<NT, 1, BITS>, a.H / 8, 256, 0, s, a);
    else if (NT == 1)  // one expert per batch (1.1 us faster than two at decode shape)
        launch(mk, dec::k_dec_down<NT, 1, 2, 1, BITS>, a.H / 8, 256, 0, s, a);
    else
        launch(mk, dec::k_dec_down<NT, 1, 2, 2, BITS>, a.H / 8, 256, 0, s, a);
}

template <int NT, int BITS>
void launch_small_nt(const dec::DecArgs& a, hipStream_t s, Marks& mk) {
    if (a.H <= 2048) {
        if (a.tap) launch_small_tap<NT, 1, true, BITS>(a, s, mk);
        else launch_small_tap<NT, 1, false, BITS>(a, s, mk);
    } else {
        if (a.tap) launch_small_tap<NT, 3, true, BITS>(a, s, mk);
        else launch_small_tap<NT, 3, false, BITS>(a, s, mk);
    }
}

template <int BITS>
void launch_small_bits(const dec::DecArgs& a, hipStream_t s, Marks& mk) {
    if (a.T <= 1) launch_small_nt<1, BITS>(a, s, mk);
    else if (a.T <= 2) launch_small_nt<2, BITS>(a, s, mk);
    else launch_small_nt<4, BITS>(a, s, mk);
}

void launch_topk_wave(const double* logits, const float* bias, int64_t T, int E, int K,
                      int norm, double rho, GroupSel gsel, int32_t* idx, float* wts,
                      hipStream_t s, Marks& mk) {
    launch(mk, dec::k_topk_wave, (unsigned)((T + 3) / 4), 256, 0, s, logits, bias, (int)T, E, K,
           norm, rho, gsel, idx, wts);
}

void launch_small(const dec::DecArgs& a, int bits, hipStream_t s, Marks& mk) {
    if (bits == 8) launch_small_bits<8>(a, s, mk);
    else if (bits == 2) launch_small_bits<2>(a, s, mk);
    else launch_small_bits<4>(a, s, mk);
}

