// Argument blocks of the layer's kernel families, shared by the host code
// that fills them and the kernels that read them.
#pragma once

#include <stdint.h>

#include "coli_common.h"

// Work items of the many-token kernels: item i is expert item_e[i], its
// slots item_s0[i] .. item_s0[i] + item_n[i] - 1; *n_items items in all.
struct ItemArgs {
    int32_t* item_e;
    int32_t* item_s0;
    int32_t* item_n;
    int32_t* n_items;
};

namespace dec {

constexpr int kMaxTok = 4;
constexpr int kMaxEntries = 64;  // T * K

struct DecArgs {
    const float* x;
    const float* wr;
    const float* bias;
    const uint8_t* eq;
    const float* es;
    int64_t blob_q, blob_s;
    int T, H, I, E, K, S, norm;
    double rho;
    GroupSel gsel;  // group-limited selection (ng <= 1: none)
    // workspace
    double* logits;
    double* sig;   // [T, E] sigmoid of the logits (written by the router kernel)
    double* cval;  // [T, E] s + bias, the selection scores
    int8_t* qx;
    float* dx;
    int32_t* idx;
    float* wts;
    int32_t* counts;
    int32_t* offs;
    int32_t* slot_of;
    int32_t* slot_tok;
    int32_t* uinfo;   // [0] = n_uniq, then (e, s0, n) triples, then slot weights
    int8_t* qh;
    float* dh;
    int32_t* tap;
    int tap_rows, tap_stride;
    float* y;
    int accum;
};

constexpr int kUinfoW = 1 + 3 * kMaxEntries;  // offset of the slot weights in uinfo

}  // namespace dec

namespace pf {

constexpr int kRows = 64;     // gate/up: h rows per workgroup (16 per wave)
constexpr int kDnRows = 128;  // down: output rows per workgroup (32 per wave)

struct PfArgs {
    const uint8_t* eq;
    const float* es;
    int64_t blob_q, blob_s;
    int H, I;
    const int8_t* qx;      // [T, H] Q8_0 codes of x (in the weight width's element order)
    const float* dx;       // [T, H/32]
    const int32_t* item_e;
    const int32_t* item_s0;
    const int32_t* item_n;
    const int32_t* n_items;
    const int32_t* offs;   // [E + S + 1] first slot of each expert (its items follow it)
    const int32_t* slot_tok;
    int8_t* qh;            // [slots, I]
    float* dh;             // [slots, I/32]
    float* ye;             // [slots, H]
    int32_t* tap;
    int tap_rows, tap_stride;
    const int32_t* mx;     // integer form of dx (k_scale_int) and its exponents
    const int32_t* ex;
    const int32_t* mh;     // integer form of dh and its exponents
    const int32_t* eh;
};

}  // namespace pf
