// varq_device.h - launch-argument tables and small device helpers shared by the
// gfx950 kernels of the VAR-Q packed KV-cache library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "varq_quant_math.h"

#define VARQ_MAX_GROUPS_DEV 256

namespace varq {

// ---------------------------------------------------------------- arguments

// quantize+pack. Work unit = (batch, head, block, channel slice); `unit_start`
// is the prefix count of units per block, `slice_words` the words per slice of
// each block (slices tile the W words of a row; the last one may be shorter).
struct QuantPackArgs {
    const uint16_t *x;          // bf16 [B, L_in, H, D] at (sx_b, sx_l, sx_h), channel stride 1
    int64_t sx_b, sx_l, sx_h;
    uint32_t *packed;           // [B, H, W, L_cap]
    float *scales;              // [B, H, G_cap, D]
    int64_t L_cap, tok_start, G_cap, group_start;
    int B, H, D, W, G;
    int n_units;
    int32_t off[VARQ_MAX_GROUPS_DEV + 1];          // token offsets relative to x
    int32_t unit_start[VARQ_MAX_GROUPS_DEV + 1];   // prefix of units per block
    uint8_t slice_words[VARQ_MAX_GROUPS_DEV];      // words per slice, per block
};

struct UnpackArgs {
    const uint32_t *packed;     // [B, H, W, L_cap]
    const float *scales;        // [B, H, G_cap, D]
    uint16_t *out;              // bf16 [B, H, L, D]
    int64_t L_cap, G_cap, L;
    int B, H, D, W, G;
    int32_t off[VARQ_MAX_GROUPS_DEV + 1];
};

struct AttnArgs {
    const uint16_t *q;          // bf16 [B, Lq, H, D]
    int64_t sq_b, sq_l, sq_h;
    const uint32_t *pk, *pv;    // [B, H, W, L_cap]
    const float *sk, *sv;       // [B, H, G_cap, D]
    uint16_t *out;              // bf16 [B, Lq, H, D]
    int64_t so_b, so_l, so_h;
    int64_t L_cap, G_cap, L_kv, Lq;
    int B, H, W, G;
    int n_qtiles;
    float scale_log2;           // softmax_scale * log2(e)
    int32_t off[VARQ_MAX_GROUPS_DEV + 1];
};

// ---------------------------------------------------------------- helpers

// Work-groups of one launch are handed to the 8 XCDs round robin (block i runs
// on XCD i % 8). Remap so that consecutive logical ids run on the same XCD and
// share its L2: XCD x takes logical ids [x*per, (x+1)*per). Returns -1 for the
// padding ids of a grid rounded up to a multiple of 8.
__device__ inline int64_t xcd_logical_id(int64_t hw_id, int64_t n_logical) {
    const int64_t per = (n_logical + 7) / 8;
    const int64_t logical = (hw_id % 8) * per + hw_id / 8;
    return logical < n_logical ? logical : -1;
}

__device__ inline float bf16lo(uint32_t w) { return u2f(w << 16); }
__device__ inline float bf16hi(uint32_t w) { return u2f(w & 0xFFFF0000u); }

// Block g holding token t, searching upward from g0 (off[g0] <= t required).
__device__ inline int group_of(const int32_t *off, int g0, int64_t t) {
    int g = g0;
    while (off[g + 1] <= t) ++g;
    return g;
}

}  // namespace varq
