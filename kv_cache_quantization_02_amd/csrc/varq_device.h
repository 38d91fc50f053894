// varq_device.h - launch-argument tables and small device helpers shared by the
// gfx950 kernels of the VAR-Q packed KV-cache library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "varq_quant_math.h"

#define VARQ_MAX_GROUPS_DEV 256

namespace varq {

// ---------------------------------------------------------------- arguments

// quantize+pack. Work unit = up to chunk_rows token rows of one (batch, head):
// a chunk of a block longer than chunk_rows, or a pack of whole consecutive
// blocks. unit_start[g] is the index, within one (batch, head), of the first
// unit holding block g (blocks of one pack share it); units_per_bh = unit_start[G].
// When some block spans several chunks, `part`, `fin` and `sync` point to
// scratch: 64-bit (epoch << 32 | fp32 bits) slots for per-unit partial maxima
// [n_units, D] and block maxima [B*H*G, D], and sync = {epoch of the last
// launch, work-groups finished, timeout status}. Otherwise part == nullptr.
struct QuantPackArgs {
    const uint16_t *x;          // bf16 [B, L_in, H, D] at (sx_b, sx_l, sx_h), channel stride 1
    int64_t sx_b, sx_l, sx_h;
    uint32_t *packed;           // [B, H, W, L_cap]
    float *scales;              // [B, H, G_cap, D]
    // a second tensor of the same shape, block map and cache layout (V next
    // to K): units [n_units_one, n_units) are its units (non-split launches)
    const uint16_t *x2;
    int64_t sx2_b, sx2_l, sx2_h;
    uint32_t *packed2;
    float *scales2;
    int64_t n_units_one;        // units of one tensor (n_units when x2 is null)
    uint64_t *part;             // [n_units, D] (both tensors)
    uint64_t *fin;              // [T*B*H*G, D], T = 2 with x2
    uint32_t *sync;             // [3]
    int64_t L_cap, tok_start, G_cap, group_start;
    int64_t n_units;
    int B, H, D, W, G;
    int chunk_rows, rows_log2, units_per_bh;
    int lds_max, lds_s, lds_y, lds_codes, lds_off, lds_us, lds_bytes;   // dynamic LDS layout (bytes)
    int32_t off[VARQ_MAX_GROUPS_DEV + 1];          // token offsets relative to x
    int32_t unit_start[VARQ_MAX_GROUPS_DEV + 1];
};

// quantize+pack of blocks longer than one work-group's unit, one work-group
// per (tensor, batch, head, block, channel slab): the blocks [gb, G) of the
// call (all longer than a unit), slab = SW consecutive channels. The block
// table off[] is relative to x, as in QuantPackArgs.
struct SlabArgs {
    const uint16_t *x[2];       // bf16 [B, L_in, H, D] of K (and V), channel stride 1
    int64_t sx_b[2], sx_l[2], sx_h[2];
    uint32_t *packed[2];        // [B, H, W, L_cap]
    float *scales[2];           // [B, H, G_cap, D]
    int64_t L_cap, tok_start, G_cap, group_start;
    int64_t n_units;            // n_tensors * B * H * nbig * slabs
    int B, H, D, W;
    int gb, nbig, slabs;        // first slab block, slab blocks, slabs per row
    int32_t off[VARQ_MAX_GROUPS_DEV + 1];
};

struct UnpackArgs {
    const uint32_t *packed;     // [B, H, W, L_cap]
    const float *scales;        // [B, H, G_cap, D]
    uint16_t *out;              // bf16 [B, H, L, D]
    const float *rcos, *rsin;   // pre-RoPE: per-token rotation tables [L, D/2] (else null)
    int64_t L_cap, G_cap, L;
    int B, H, D, W, G;
    int32_t off[VARQ_MAX_GROUPS_DEV + 1];
};

struct GroupArgs {
    const uint16_t *x;          // bf16 [B, L, H, D] at (sx_b, sx_l, sx_h)
    int64_t sx_b, sx_l, sx_h;
    uint32_t *packed;           // [B, H, W, L_cap]
    uint32_t *absmax;           // the scale buffer: group maxima (fp32 bits), then scales
    int64_t L_cap;
    int B, L, H, D, W, G;
    int32_t off[VARQ_MAX_GROUPS_DEV + 1];
};

constexpr int VARQ_MAX_KV_SPLITS = 8;

struct AttnArgs {
    const uint16_t *q;          // bf16 [B, Lq, H, D]
    int64_t sq_b, sq_l, sq_h;
    const uint32_t *pk, *pv;    // [B, H, W, L_cap]
    const float *sk, *sv;       // [B, H, G_cap, D]
    const uint16_t *kd, *vd;    // dense bf16 [B, H, L_cap, D] (unfused baseline; pk/pv unused)
    const float *rcos, *rsin;   // pre-RoPE: per-token rotation tables [L_kv, D/2] (else null)
    uint16_t *out;              // bf16 [B, Lq, H, D]
    int64_t so_b, so_l, so_h;
    int64_t L_cap, G_cap, L_kv, Lq;
    int B, H, W, G;
    int n_qtiles;
    float scale_log2;           // softmax_scale * log2(e)
    // the KV tiles split into kv_splits ranges [split_t0[s], split_t0[s + 1])
    // (64-token tiles), split s starting in block split_g0[s]; with more than
    // one split every work-group writes its unnormalized O and its (m, l) to
    // part_o [S, B*H, Lq, D] and part_ml [S, B*H, Lq, 2] (fp32) for the merge
    int kv_splits;
    int32_t split_t0[VARQ_MAX_KV_SPLITS + 1];
    int32_t split_g0[VARQ_MAX_KV_SPLITS];
    float *part_o, *part_ml;
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
