/*
 * varq.h - C ABI of the MI355X (gfx950) VAR-Q packed KV-cache library.
 *
 * VAR-Q (project page "VAR-Q: Tuning-free KV Cache Quantization for Visual
 * Autoregressive Image and Video Generation") keeps one scale factor per
 * feature channel within each generation block (a resolution scale or a
 * frame), stores 2-8 bit codes packed into INT32 containers, and unpacks and
 * dequantizes them to BF16 for attention (project page: summary, "Next-block
 * prediction", "Quantization, bit packing, and retrieval" / Fig. 8). The README
 * section "Memory-Efficient Runtime" names the compiled operators this library
 * provides: quantize+pack, unpack+dequant and packed-KV attention, with compact
 * per-group scales and exact cache preallocation.
 *
 * Conventions for every entry point
 *  - Tensor pointers are DEVICE pointers owned by the caller. The library never
 *    frees them, keeps no reference after the call returns and allocates no
 *    device memory of its own. Calls that may need device scratch (the
 *    cross-work-group exchange of quantize+pack for blocks longer than one
 *    work-group, the partial results of attention launches split over KV
 *    ranges) take a caller-owned `workspace` of at least the bytes that the
 *    matching *_workspace query returns (NULL is accepted when it returns 0).
 *    Only varq_quantize_pack_kv_noalloc, for callers that cannot allocate,
 *    uses a fixed device array inside the library instead.
 *  - `group_offsets` is a HOST array of G+1 int32 prefix offsets
 *    0 = o_0 < o_1 < ... < o_G: block g covers tokens [o_g, o_{g+1}).
 *    G <= VARQ_MAX_GROUPS per call.
 *  - Strides are in elements and non-negative (VARQ_EINVAL otherwise). The
 *    channel (head_dim) stride is 1 ("BLHc" layout of the README's
 *    qkv_format: [batch, token, head, channel]).
 *  - `stream` is a hipStream_t (NULL = the default stream). Every compute call
 *    only enqueues work on that stream and returns; results are ready when the
 *    stream reaches them. No call synchronizes the stream except
 *    varq_quantize_pack_check, which exists to read a status back.
 *  - Arguments are validated on the host before anything is enqueued; on any
 *    error nothing is launched and a negative varq_status is returned.
 *    varq_last_error() then describes the failure (per calling thread).
 *  - Inputs must be finite (NaN/Inf are outside the contract).
 *
 * Data layout (this library's reading; the pages fix no layout)
 *  - bits b in 2..8; qmax = 2^(b-1) - 1; cpw = floor(32/b) codes per word;
 *    W = ceil(D / cpw) words per (batch, head, token).
 *  - Packed cache: int32 [B, H, W, L_cap]: plane w of (batch, head) holds word w
 *    of every token. Field i (bits [i*b, i*b+b)) of word w is the code of channel
 *    w*cpw + i in b-bit two's complement; unused fields and bits are zero.
 *  - Scales: fp32 [B, H, G_cap, D], one per (batch, head, block, channel),
 *    s = fp32(absmax / qmax); never expanded per token.
 *  - Codes: q = clamp(rint(fp32(x / s)), -qmax, qmax) with IEEE division and
 *    ties to even; q = 0 when s = 0. Dequantized value: bf16_rne(fp32(q) * s).
 */
#ifndef VARQ_H
#define VARQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum varq_status {
    VARQ_OK = 0,
    VARQ_EINVAL = -1,       /* bad size, count, stride, null pointer or group table */
    VARQ_EBITS = -2,        /* bits outside 2..8 */
    VARQ_EALIGN = -3,       /* pointer or stride not aligned as documented */
    VARQ_ECAPACITY = -4,    /* write or read range outside the preallocated cache */
    VARQ_ELAUNCH = -5,      /* the HIP runtime reported an error */
    VARQ_EUNSUPPORTED = -6, /* valid request the kernels do not implement (e.g. head_dim) */
    VARQ_EWORKSPACE = -7    /* workspace NULL or smaller than the workspace query's answer */
} varq_status;

#define VARQ_MAX_GROUPS 256

/* Codes of `bits` bits per INT32 container: floor(32/bits); 0 if bits is not
 * in 2..8. The project page's summary and Fig. 8 pack 2-8 bit codes into INT32
 * containers without naming a layout; whole fields per word is this library's
 * reading (it reproduces the Table 4 INT6 rows, which need 5 codes per word). */
int varq_codes_per_word(int bits);

/* INT32 words per (batch, head, token) row: ceil(head_dim / floor(32/bits));
 * 0 if bits is not in 2..8 or head_dim < 1. Packing runs along head_dim
 * (project page Fig. 8 packs each token's codes; the per-row word count with a
 * partly empty last word reproduces the Table 4 INT6 memory rows). */
int varq_words_per_row(int head_dim, int bits);

/*
 * Exact persistent size of ONE packed tensor (K or V) and of its scales, for
 * preallocation to the known generation length (README "Memory-Efficient
 * Runtime": expected_total_seq_len / preallocate_kv_cache):
 *   *packed_bytes = B*H*W*L_cap*4,  *scale_bytes = B*H*G_cap*head_dim*4.
 * Either output pointer may be NULL. Pure host arithmetic.
 */
int varq_cache_bytes(int B, int H, int head_dim, int64_t L_cap, int64_t G_cap, int bits,
                     int64_t *packed_bytes, int64_t *scale_bytes);

/*
 * quantize+pack (project page summary and Fig. 8; README "Memory-Efficient
 * Runtime"): for every (batch b, head h, block g, channel c) of the input,
 * a = max |x| over the block's tokens, s = fp32(a/qmax); every element gets the
 * code q defined above; codes are packed into INT32 words.
 *
 *  x            bf16 [B, L_in, H, D] at element strides (sx_b, sx_l, sx_h), channel
 *               stride 1. Pointer 16-byte aligned; strides multiples of 8.
 *  group_offsets host int32[G_in+1], block boundaries relative to x (o_{G_in} = L_in).
 *  packed       int32 [B, H, W, L_cap]; rows [tok_start, tok_start+L_in) of every
 *               plane are written, nothing else. 16-byte aligned; L_cap % 8 == 0.
 *  scales       fp32 [B, H, G_cap, D]; slots [group_start, group_start+G_in) are
 *               written, nothing else. 4-byte aligned.
 *  D            head_dim: a multiple of 8, 8 <= D <= 256.
 * Errors: VARQ_EBITS, VARQ_EINVAL, VARQ_EALIGN, VARQ_ECAPACITY
 * (tok_start+L_in > L_cap or group_start+G_in > G_cap), VARQ_EUNSUPPORTED (a
 * block of more 16384-element chunks than resident work-groups, or a token
 * stride or cache length beyond 32-bit byte offsets), VARQ_ELAUNCH.
 * Long blocks: a block longer than one work-group's 16384 elements (16384 / D
 * token rows) is handled whole by one work-group per channel slab when the
 * long blocks follow all the short ones and form at most 16 runs of
 * consecutive blocks that take one work-group shape (each block takes the
 * smallest that holds it), and either bits is 2, 4, 7 or 8, D a multiple of
 * 16 and no block over 8192 rows (16- or 32-channel slabs), or bits is 3, 5
 * or 6 and no block over 1612, 2688, 1612 rows (40-, 24-, 40-channel slabs,
 * any D); such calls need no workspace. Otherwise its chunks exchange per-channel
 * maxima through the caller's workspace (varq_quantize_pack_workspace gives
 * the size: 16 bytes of launch state plus 8 bytes per (chunk, channel) and per
 * (block, channel); it is 0 when no exchange is needed, and workspace may then
 * be NULL). The workspace must be
 * zero-filled once before its first use; every launch leaves it valid for the
 * next (each slot carries the tag of the launch that wrote it, and the launch
 * state advances the tag), so it is then reused without clearing, by calls of
 * any shape, as long as calls sharing it are ordered on one stream. Such
 * launches are cooperative (every work-group resident); a cross-work-group wait
 * is bounded in time and one cut short is reported by varq_quantize_pack_check.
 * Deterministic: the output does not depend on launch order or timing.
 */
int varq_quantize_pack(const void *x, int64_t sx_b, int64_t sx_l, int64_t sx_h,
                       int B, int H, int D, int64_t L_in,
                       const int32_t *group_offsets, int G_in, int bits,
                       int32_t *packed, int64_t L_cap, int64_t tok_start,
                       float *scales, int64_t G_cap, int64_t group_start,
                       void *workspace, int64_t workspace_bytes, void *stream);

/*
 * Workspace bytes that a quantize+pack call over n_tensors (1: varq_quantize_pack,
 * 2: varq_quantize_pack_kv) tensors of this shape and block map needs, in
 * *bytes: 0 when every block fits one work-group's rows. Pure host arithmetic.
 * Errors: VARQ_EBITS, VARQ_EINVAL.
 */
int varq_quantize_pack_workspace(int B, int H, int D, int64_t L_in, const int32_t *group_offsets, int G_in,
                                 int bits, int n_tensors, int64_t *bytes);

/*
 * quantize+pack of K and V together (project page Fig. 8: the new block's K
 * and V are both quantized and packed before attention reads them back): the
 * same result as varq_quantize_pack(k -> packed_k, scales_k) followed by
 * varq_quantize_pack(v -> packed_v, scales_v), with one shape, block map and
 * cache layout for both. k and v have strides of their own; packed_k/packed_v
 * and scales_k/scales_v are distinct buffers. Both tensors go through one
 * launch (the cooperative kernel when some block is longer than one
 * work-group's 16384 elements, with the workspace rules above counting the
 * chunks and blocks of both tensors: varq_quantize_pack_workspace with
 * n_tensors = 2).
 * Errors: those of varq_quantize_pack, for either tensor, and VARQ_EINVAL when
 * K and V share a cache buffer.
 */
int varq_quantize_pack_kv(const void *k, int64_t sk_b, int64_t sk_l, int64_t sk_h,
                          const void *v, int64_t sv_b, int64_t sv_l, int64_t sv_h,
                          int B, int H, int D, int64_t L_in,
                          const int32_t *group_offsets, int G_in, int bits,
                          int32_t *packed_k, float *scales_k, int32_t *packed_v, float *scales_v,
                          int64_t L_cap, int64_t tok_start, int64_t G_cap, int64_t group_start,
                          void *workspace, int64_t workspace_bytes, void *stream);

/*
 * varq_quantize_pack_kv for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same arguments without a workspace and the same outputs,
 * bit for bit. The cross-work-group exchange uses a fixed 16 MiB array inside
 * the library instead, one per device, kept until the process ends; the call
 * itself allocates nothing. A call whose exchange would need more than 16 MiB
 * (16 bytes + 8 bytes per (chunk, channel) and per (block, channel) of both
 * tensors, as varq_quantize_pack_workspace with n_tensors = 2 counts it)
 * returns VARQ_EWORKSPACE and launches nothing. The first call on a device
 * that needs the array enqueues a kernel zeroing it on `stream` before its own
 * launch. Every call on one device shares that device's array and leaves it
 * valid for the next, so calls that may overlap on one device (other streams,
 * other threads) race: order them on one stream. varq_quantize_pack_check
 * with a NULL workspace reports this array's status on the current device.
 */
int varq_quantize_pack_kv_noalloc(const void *k, int64_t sk_b, int64_t sk_l, int64_t sk_h,
                                  const void *v, int64_t sv_b, int64_t sv_l, int64_t sv_h,
                                  int B, int H, int D, int64_t L_in,
                                  const int32_t *group_offsets, int G_in, int bits,
                                  int32_t *packed_k, float *scales_k, int32_t *packed_v, float *scales_v,
                                  int64_t L_cap, int64_t tok_start, int64_t G_cap, int64_t group_start,
                                  void *stream);

/*
 * Pre-RoPE quantization (project page Appendix F / Table 7; Insight 03, Eq. 3):
 * the cache holds K quantized BEFORE the rotary embedding, and the rotation is
 * applied to the dequantized K. The schedule is a pair of fp32 tables
 * rope_cos, rope_sin [L, D/2] (row t = cache token t, column i = channel pair
 * (2i, 2i+1)), device pointers, 4-byte aligned, at least L (unpack) or L_kv
 * (attention) rows. For every pair of the dequantized bf16 values (a, b):
 *   a' = bf16_rne(fp32(fp32(a*c) - fp32(b*s))),  b' = bf16_rne(fp32(fp32(a*s) + fp32(b*c))).
 *
 * varq_unpack_dequant_rope: varq_unpack_dequant followed by that rotation
 * (the unfused pre-RoPE path; bit-exact). Same arguments and errors as
 * varq_unpack_dequant, plus VARQ_EINVAL for a NULL table and VARQ_EALIGN.
 *
 * varq_packed_attention_rope: varq_packed_attention with every dequantized K
 * tile rotated before the scores; q must already be rotated (it is not
 * cached). Same arguments, errors, workspace and tolerance as
 * varq_packed_attention, plus VARQ_EINVAL for a NULL table and VARQ_EALIGN.
 */
int varq_unpack_dequant_rope(const int32_t *packed, const float *scales,
                             int B, int H, int D, int64_t L_cap, int64_t G_cap, int64_t L,
                             const int32_t *group_offsets, int G, int bits,
                             const float *rope_cos, const float *rope_sin,
                             void *out, void *stream);

int varq_packed_attention_rope(const void *q, int64_t sq_b, int64_t sq_l, int64_t sq_h,
                               int B, int H, int D, int64_t Lq,
                               const int32_t *packed_k, const float *scales_k,
                               const int32_t *packed_v, const float *scales_v,
                               int64_t L_cap, int64_t G_cap, int64_t L_kv,
                               const int32_t *group_offsets, int G, int bits,
                               float softmax_scale,
                               void *out, int64_t so_b, int64_t so_l, int64_t so_h,
                               const float *rope_cos, const float *rope_sin,
                               void *workspace, int64_t workspace_bytes, void *stream);

/*
 * Scale groupings (project page, grouping ablation Table 5 and error table
 * Table 1). The "channel axis" is the hidden width H * D: a grouping without
 * it shares one scale across heads and head channels. Compact fp32 scale
 * layouts, one value per group:
 *   VARQ_GROUP_CHANNEL_BLOCK  [B, H, G, D]  the method (varq_quantize_pack)
 *   VARQ_GROUP_CHANNEL        [B, H, D]     "without block axis" (one block [0, L))
 *   VARQ_GROUP_BLOCK          [B, G]        "without channel axis"
 *   VARQ_GROUP_TOKEN_HEAD     [B, H, L]     "per-token & per-head"
 *   VARQ_GROUP_TOKEN          [B, L]        "per-token"
 *   VARQ_GROUP_TENSOR         [1]           "per-tensor" (Table 1)
 */
enum {
    VARQ_GROUP_CHANNEL_BLOCK = 0,
    VARQ_GROUP_CHANNEL = 1,
    VARQ_GROUP_BLOCK = 2,
    VARQ_GROUP_TOKEN_HEAD = 3,
    VARQ_GROUP_TOKEN = 4,
    VARQ_GROUP_TENSOR = 5
};

/* Number of scales of grouping `mode` for x [B, L, H, D] with G blocks
 * (the product of the layout above); -1 for an unknown mode or a negative size. */
int64_t varq_grouped_scale_count(int mode, int B, int64_t L, int H, int D, int G);

/*
 * quantize+pack with the scales of grouping `mode` (project page Table 5):
 * for every group, a = max |x| over its elements and s = fp32(a/qmax); codes,
 * packing and word layout are exactly those of varq_quantize_pack. Quantizes
 * one whole sequence window [0, L) (no append offsets).
 *
 *  x            bf16 [B, L, H, D] at element strides (sx_b, sx_l, sx_h), channel
 *               stride 1. Pointer 16-byte aligned; strides multiples of 8.
 *  group_offsets host int32[G+1] block boundaries (used by CHANNEL_BLOCK and
 *               BLOCK; the other groupings still require a valid table).
 *  packed       int32 [B, H, W, L_cap], rows [0, L) written. 16-byte aligned;
 *               L_cap % 8 == 0, L <= L_cap.
 *  scales       fp32, n_scales >= varq_grouped_scale_count(...) entries; the first
 *               count are written (compact layout above). 4-byte aligned. For
 *               BLOCK, TOKEN_HEAD, TOKEN and TENSOR the buffer first holds the
 *               groups' maxima while the call runs (stream-ordered).
 *  D            head_dim: a multiple of 8, 8 <= D <= 256.
 * CHANNEL_BLOCK and CHANNEL run varq_quantize_pack (its workspace rules apply,
 * with the table of the grouping: CHANNEL is one block [0, L)); the other
 * groupings run three passes over x and need no workspace.
 * Errors: VARQ_EBITS, VARQ_EINVAL (unknown mode, bad sizes or table),
 * VARQ_EALIGN, VARQ_ECAPACITY (L > L_cap or n_scales too small),
 * VARQ_EUNSUPPORTED (B*L*H*W or the scale count beyond 2^31 - 1), VARQ_ELAUNCH.
 * Deterministic.
 */
int varq_quantize_pack_grouped(const void *x, int64_t sx_b, int64_t sx_l, int64_t sx_h,
                               int B, int H, int D, int64_t L,
                               int mode, const int32_t *group_offsets, int G, int bits,
                               int32_t *packed, int64_t L_cap,
                               float *scales, int64_t n_scales,
                               void *workspace, int64_t workspace_bytes, void *stream);

/*
 * Packed-KV attention (project page "Next-block prediction": a block attends to
 * the cache of all earlier blocks and itself; README: packed-KV load, unpack and
 * dequant fused into attention). For every (b, h) and query row i:
 *   O[b,i,h,:] = softmax_j(Q[b,i,h,:] . K^[b,h,j,:] * softmax_scale) V^[b,h,j,:]
 * over the window j in [0, L_kv) with no mask, where K^, V^ are the dequantized
 * caches. Logits, softmax and accumulation in fp32; output rounded to bf16.
 *
 *  q            bf16 [B, Lq, H, D] at strides (sq_b, sq_l, sq_h); 16-byte aligned,
 *               strides multiples of 8.
 *  packed_k/v   int32 [B, H, W, L_cap] written by varq_quantize_pack (16-byte aligned).
 *  scales_k/v   fp32 [B, H, G_cap, D].
 *  group_offsets host int32[G+1]: the block boundaries in cache tokens used when
 *               the cache was written; o_G = L_kv <= L_cap, G <= G_cap.
 *  D            64 or 128.
 *  out          bf16 [B, Lq, H, D] at strides (so_b, so_l, so_h); 8-byte aligned,
 *               strides multiples of 4. Must not overlap q or the cache.
 * Errors: VARQ_EBITS, VARQ_EINVAL, VARQ_EALIGN, VARQ_ECAPACITY, VARQ_EUNSUPPORTED
 * (D not 64/128), VARQ_ELAUNCH.
 * Workspace: when (b, h, query tile) work-groups fill less than two rounds of
 * the device, the window's 64-token tiles run in up to 8 ranges (at least 8
 * tiles each) and a second kernel merges the ranges' unnormalized outputs and
 * (maximum, sum) pairs with log-sum-exp weights. The partials, S*B*H*Lq*(D+2)
 * fp32 for S ranges, live in the caller's workspace
 * (varq_packed_attention_workspace gives the size; 0 for one range, when
 * workspace may be NULL). Its contents on entry do not matter: every launch
 * writes each partial it reads. Calls sharing a workspace must be ordered on
 * one stream. The range count depends only on the shapes and the current
 * device's compute-unit count.
 */
int varq_packed_attention(const void *q, int64_t sq_b, int64_t sq_l, int64_t sq_h,
                          int B, int H, int D, int64_t Lq,
                          const int32_t *packed_k, const float *scales_k,
                          const int32_t *packed_v, const float *scales_v,
                          int64_t L_cap, int64_t G_cap, int64_t L_kv,
                          const int32_t *group_offsets, int G, int bits,
                          float softmax_scale,
                          void *out, int64_t so_b, int64_t so_l, int64_t so_h,
                          void *workspace, int64_t workspace_bytes, void *stream);

/*
 * Workspace bytes of a packed (or bf16) attention call of this shape on the
 * current device, in *bytes (0 when the window runs as one range). Host
 * arithmetic plus a query of the device's compute-unit count.
 * Errors: VARQ_EINVAL (bad sizes), VARQ_EUNSUPPORTED (D not 64/128),
 * VARQ_ELAUNCH (no device).
 */
int varq_packed_attention_workspace(int B, int H, int D, int64_t Lq, int64_t L_kv, int64_t *bytes);

/*
 * unpack+dequant (README "Memory-Efficient Runtime"; project page Fig. 8): the
 * dense bf16 view of tokens [0, L) of a packed cache,
 *   out[b, h, t, c] = bf16_rne(fp32(q[b,h,t,c]) * s[b,h,g(t),c]),
 * g(t) the block holding t. Used by the unfused attention path and by tests.
 *
 *  packed, scales as above; group_offsets host int32[G+1] with o_G = L <= L_cap.
 *  out          bf16 [B, H, L, D], contiguous, 16-byte aligned.
 *  D            a multiple of 8, 8 <= D <= 256.
 * Errors: as varq_quantize_pack.
 */
int varq_unpack_dequant(const int32_t *packed, const float *scales,
                        int B, int H, int D, int64_t L_cap, int64_t G_cap, int64_t L,
                        const int32_t *group_offsets, int G, int bits,
                        void *out, void *stream);

/*
 * Plain bf16 attention over dense K and V: the unfused baseline that the
 * fused varq_packed_attention is measured against (README "Deployment
 * Results": fusing packed-KV load, unpack and dequant into attention; the
 * unfused path first writes the dequantized cache with varq_unpack_dequant).
 * Same result definition as varq_packed_attention with K^, V^ given directly:
 *   O[b,i,h,:] = softmax_j(Q[b,i,h,:] . K[b,h,j,:] * softmax_scale) V[b,h,j,:],
 * j in [0, L_kv), no mask; logits, softmax and accumulation in fp32; bf16 out.
 *  q            bf16 [B, Lq, H, D] at strides (sq_b, sq_l, sq_h); 16-byte aligned,
 *               strides multiples of 8.
 *  k, v         bf16 [B, H, L_rows, D], contiguous (varq_unpack_dequant's output
 *               layout), 16-byte aligned; L_kv <= L_rows.
 *  D            64 or 128.
 *  out          bf16 [B, Lq, H, D] at strides (so_b, so_l, so_h); 8-byte aligned,
 *               strides multiples of 4. Must not overlap q, k or v.
 * Errors: VARQ_EINVAL, VARQ_EALIGN, VARQ_ECAPACITY (L_kv > L_rows),
 * VARQ_EUNSUPPORTED (D not 64/128), VARQ_ELAUNCH.
 * Workspace and KV ranges as for varq_packed_attention (same plan and the
 * same varq_packed_attention_workspace size for the same shapes, so both paths
 * compute in the same order).
 */
int varq_bf16_attention(const void *q, int64_t sq_b, int64_t sq_l, int64_t sq_h,
                        int B, int H, int D, int64_t Lq,
                        const void *k, const void *v, int64_t L_rows, int64_t L_kv,
                        float softmax_scale,
                        void *out, int64_t so_b, int64_t so_l, int64_t so_h,
                        void *workspace, int64_t workspace_bytes, void *stream);

/* Whether a quantize+pack call that used `workspace` since the previous check
 * ended a cross-work-group wait by its time bound (the cooperative launch used
 * when a block is longer than one work-group's rows). The kernel's waits end
 * by construction; the bound only keeps a faulty device from hanging, and a
 * wait cut short leaves that call's outputs invalid. Synchronizes `stream` (a
 * hipStream_t; NULL = the null stream; the stream the calls ran on) and reads
 * the status word in the workspace's launch state.
 * A NULL workspace means the fixed array of varq_quantize_pack_kv_noalloc on
 * the current device.
 * Returns VARQ_OK (also when no such launch used the workspace or array), or
 * VARQ_ELAUNCH after a timed-out wait (the status is then cleared) or when the
 * status cannot be read. */
int varq_quantize_pack_check(void *workspace, void *stream);

/* Text of the last error reported to the calling thread ("" if none). */
const char *varq_last_error(void);

/* Library version string. */
const char *varq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* VARQ_H */
