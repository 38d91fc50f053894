"""VAR-Q CPU oracle: the plain, slow definition of what the packed-KV path computes.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module. The GPU library never calls it and it
shares no code with the GPU library.

Sources (the VAR-Q project page "VAR-Q: Tuning-free KV Cache Quantization for
Visual Autoregressive Image and Video Generation", and the VAR-Q README):
  * project page, summary and "Next-block prediction": one scale factor per
    feature channel within each generation block (a scale or a frame); block
    boundaries come from the generation loop; 2-8 bit values packed into INT32
    containers; every block attends to the KV cache of all earlier blocks.
  * project page, "Quantization, bit packing, and retrieval" (Fig. 8): quantize
    K and V, pack into INT32 with scale factors, store, then unpack and
    dequantize to BF16 before attention.
  * README, "Memory-Efficient Runtime": scale metadata stored per group, never
    expanded per token; caches preallocated to the known generation length.

Readings where the pages are silent (each listed in the design notes):
  * symmetric quantizer, scale s = fp32(absmax / (2**(b-1) - 1)), no zero point;
  * code q = rint(fp32(x / s)) with ties to even (IEEE fp32 division, not a
    reciprocal multiply), clipped to [-qmax, qmax]; an all-zero group has s = 0
    and codes 0;
  * packing along head_dim, least-significant field first, two's complement
    fields of b bits, floor(32/b) fields per word, W = ceil(D / floor(32/b))
    words per (batch, head, token); unused fields are zero;
  * cache layout: words [B, H, W, L_cap] (one plane per word index), scales
    fp32 [B, H, G_cap, D];
  * dequantized value bf16_rne(fp32(q) * s);
  * attention over the whole window [0, L_kv) without a mask, logits scaled by
    the fp32 softmax scale (default fp32(1/sqrt(D))), computed here in fp64;
  * grouping variants (Table 5, Table 1): the "channel axis" is the hidden
    width H * D, so groupings without it share a scale across heads; scales
    are stored compactly, one fp32 per group;
  * pre-RoPE quantization (Appendix F, Table 7): K is quantized before the
    rotation; the dequantized bf16 K is rotated pairwise, (2i, 2i+1), by
    per-token cos/sin tables in fp32 (each product and the sum rounded) and
    rounded to bf16 again; the query arrives already rotated.

Array conventions: activations are float32 arrays holding bf16 values, in the
BLHc layout [B, L, H, D] (the README's qkv_format "BLHc"). Words are uint32.
"""

from __future__ import annotations

import math

import numpy as np

SUPPORTED_BITS = (2, 3, 4, 5, 6, 7, 8)


# --------------------------------------------------------------------------
# Code geometry (project page: "2-8 bit, packed into INT32 containers")
# --------------------------------------------------------------------------

def qmax(bits: int) -> int:
    """Largest code magnitude of a symmetric b-bit quantizer: 2**(b-1) - 1."""
    return (1 << (bits - 1)) - 1


def codes_per_word(bits: int) -> int:
    """Fields of b bits that fit one INT32 container: floor(32 / b)."""
    if bits not in SUPPORTED_BITS:
        raise ValueError(f"bits must be in 2..8, got {bits}")
    return 32 // bits


def words_per_row(head_dim: int, bits: int) -> int:
    """INT32 words per (batch, head, token) row: ceil(D / floor(32 / b))."""
    cpw = codes_per_word(bits)
    return -(-head_dim // cpw)


def cache_bytes(B, H, D, L_cap, G_cap, bits):
    """Persistent bytes of one packed tensor (K or V) and of its scales.

    README "Deployment Results" and "Memory-Efficient Runtime": the reduction
    counts persistent K/V storage including the compact per-group scale
    metadata. Returns (packed_bytes, scale_bytes)."""
    packed = B * H * words_per_row(D, bits) * L_cap * 4
    scales = B * H * G_cap * D * 4
    return packed, scales


def kv_reduction_percent(D, L, G, bits):
    """Cache-memory reduction versus bf16 for one (batch, head): 100*(1 - packed+scales / bf16)."""
    packed, scales = cache_bytes(1, 1, D, L, G, bits)
    return 100.0 * (1.0 - (packed + scales) / (L * D * 2))


# --------------------------------------------------------------------------
# bf16 rounding (project page, "Quantization, bit packing, and retrieval":
# cached values are dequantized to BF16 before attention)
# --------------------------------------------------------------------------

def bf16_round_f32(x) -> np.ndarray:
    """Round float32 values to the nearest bf16 value, ties to even, returned as
    float32. Works on the bit pattern: add 0x7FFF plus the lowest kept bit, then
    clear the 16 discarded bits (finite inputs only)."""
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)).astype(np.uint32)
    return r.view(np.float32)


def bf16_round_f64(x) -> np.ndarray:
    """Round float64 values straight to the nearest bf16 value (8 significant
    bits, ties to even, bf16 subnormal spacing 2**-133), returned as float32."""
    a = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(a)                      # a = m * 2**e, 0.5 <= |m| < 1
    # spacing of bf16 values around a: 2**(e-8) for normal values
    e_sp = np.maximum(e - 8, -133)
    scaled = np.ldexp(a, -e_sp)            # exact
    r = np.ldexp(np.rint(scaled), e_sp)    # rint: ties to even
    return r.astype(np.float32)


# --------------------------------------------------------------------------
# Channel x block grouping, scales and codes (project page summary and
# "Next-block prediction": one scale per feature channel within each block)
# --------------------------------------------------------------------------

def _check_offsets(offsets, L):
    off = [int(o) for o in offsets]
    if off[0] != 0 or off[-1] != L or any(b <= a for a, b in zip(off, off[1:])):
        raise ValueError("offsets must start at 0, end at L and strictly increase")
    return off


def group_absmax(x, offsets) -> np.ndarray:
    """a[b, h, g, c] = max over tokens t of block g of |x[b, t, h, c]|; float32 [B, H, G, D]."""
    x = np.asarray(x, dtype=np.float32)
    B, L, H, D = x.shape
    off = _check_offsets(offsets, L)
    G = len(off) - 1
    a = np.empty((B, H, G, D), dtype=np.float32)
    for g in range(G):
        a[:, :, g, :] = np.abs(x[:, off[g]:off[g + 1]]).max(axis=1)
    return a


def group_scales(x, offsets, bits) -> np.ndarray:
    """s = fp32(absmax / qmax) per (batch, head, block, channel); float32 [B, H, G, D]."""
    a = group_absmax(x, offsets)
    return (a / np.float32(qmax(bits))).astype(np.float32)


def quantize_codes(x, offsets, scales, bits) -> np.ndarray:
    """Codes q = clip(rint(fp32(x / s)), -qmax, qmax) (q = 0 where s = 0); int32 [B, H, L, D]."""
    x = np.asarray(x, dtype=np.float32)
    B, L, H, D = x.shape
    off = _check_offsets(offsets, L)
    qm = qmax(bits)
    q = np.empty((B, H, L, D), dtype=np.int32)
    for g in range(len(off) - 1):
        xg = x[:, off[g]:off[g + 1]].transpose(0, 2, 1, 3)            # [B, H, n, D]
        s = scales[:, :, g, None, :].astype(np.float32)                # [B, H, 1, D]
        safe = np.where(s == 0, np.float32(1), s)
        r = np.divide(xg, safe, dtype=np.float32)                      # IEEE fp32 division
        r = np.where(s == 0, np.float32(0), r)
        q[:, :, off[g]:off[g + 1], :] = np.clip(np.rint(r), -qm, qm).astype(np.int32)
    return q


# --------------------------------------------------------------------------
# INT32 container packing (project page summary; Fig. 8)
# --------------------------------------------------------------------------

def pack_codes(codes, bits) -> np.ndarray:
    """Codes int [B, H, L, D] -> words uint32 [B, H, W, L].

    Field i of word w of a (batch, head, token) row holds channel w*cpw + i,
    stored as its low b bits (two's complement) at bit offset i*b."""
    codes = np.asarray(codes)
    B, H, L, D = codes.shape
    cpw = codes_per_word(bits)
    W = words_per_row(D, bits)
    mask = np.uint32((1 << bits) - 1)
    u = (codes.astype(np.int64) & int(mask)).astype(np.uint32)
    pad = np.zeros((B, H, L, W * cpw), dtype=np.uint32)
    pad[..., :D] = u
    fields = pad.reshape(B, H, L, W, cpw)
    words = np.zeros((B, H, L, W), dtype=np.uint32)
    for i in range(cpw):
        words |= fields[..., i] << np.uint32(i * bits)
    return np.ascontiguousarray(words.transpose(0, 1, 3, 2))


def unpack_words(words, head_dim, bits) -> np.ndarray:
    """Words uint32 [B, H, W, L] -> sign-extended codes int32 [B, H, L, D]."""
    words = np.asarray(words, dtype=np.uint32)
    B, H, W, L = words.shape
    cpw = codes_per_word(bits)
    mask = np.uint32((1 << bits) - 1)
    half = 1 << (bits - 1)
    rows = words.transpose(0, 1, 3, 2)                                  # [B, H, L, W]
    out = np.empty((B, H, L, W, cpw), dtype=np.int32)
    for i in range(cpw):
        f = ((rows >> np.uint32(i * bits)) & mask).astype(np.int32)
        out[..., i] = np.where(f >= half, f - (1 << bits), f)
    return out.reshape(B, H, L, W * cpw)[..., :head_dim]


def dequantize(codes, scales, offsets) -> np.ndarray:
    """bf16_rne(fp32(q) * s) per element; float32 [B, H, L, D] holding bf16 values."""
    codes = np.asarray(codes)
    B, H, L, D = codes.shape
    off = _check_offsets(offsets, L)
    out = np.empty((B, H, L, D), dtype=np.float32)
    for g in range(len(off) - 1):
        prod = codes[:, :, off[g]:off[g + 1], :].astype(np.float32) * \
            scales[:, :, g, None, :].astype(np.float32)
        out[:, :, off[g]:off[g + 1], :] = bf16_round_f32(prod.astype(np.float32))
    return out


def quantize_pack(x, offsets, bits):
    """The quantize+pack operator: x [B, L, H, D] -> (words uint32 [B, H, W, L],
    scales float32 [B, H, G, D])."""
    s = group_scales(x, offsets, bits)
    q = quantize_codes(x, offsets, s, bits)
    return pack_codes(q, bits), s


def unpack_dequant(words, scales, offsets, head_dim, bits):
    """The unpack+dequant operator: words [B, H, W, L] + scales -> float32 [B, H, L, D] (bf16 values)."""
    return dequantize(unpack_words(words, head_dim, bits), scales, offsets)


# --------------------------------------------------------------------------
# Attention over the packed cache (project page, "Next-block prediction": a
# block attends to the cache of all earlier blocks; Fig. 8: unpack, then attend)
# --------------------------------------------------------------------------

def default_softmax_scale(D) -> np.float32:
    return np.float32(1.0 / math.sqrt(D))


def attention_fp64(q, khat, vhat, softmax_scale, bh=None):
    """Exact softmax(Q K^T * sigma) V in fp64 for every (batch, head) or the listed ones.

    q: [B, Lq, H, D] (bf16 values); khat, vhat: [B, H, L, D] (bf16 values);
    softmax_scale: the fp32 scale, used as its exact value.
    Returns (O fp64 [n, Lq, D], C fp64 [n, Lq, D], O rounded to bf16 [n, Lq, D])
    over the pairs in `bh` (default all, batch-major), where C = P |V| is the
    size of the weighted sum used by the attention tolerance."""
    q = np.asarray(q, dtype=np.float32)
    B, Lq, H, D = q.shape
    sig = float(np.float32(softmax_scale))
    pairs = bh if bh is not None else [(b, h) for b in range(B) for h in range(H)]
    O = np.empty((len(pairs), Lq, D))
    C = np.empty((len(pairs), Lq, D))
    for n, (b, h) in enumerate(pairs):
        qq = q[b, :, h, :].astype(np.float64)
        kk = np.asarray(khat[b, h], dtype=np.float64)
        vv = np.asarray(vhat[b, h], dtype=np.float64)
        s = (qq @ kk.T) * sig
        s -= s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        O[n] = p @ vv
        C[n] = p @ np.abs(vv)
    return O, C, bf16_round_f64(O)


def packed_attention(q, words_k, scales_k, words_v, scales_v, offsets, bits,
                     softmax_scale=None, bh=None):
    """Attention of q over the packed cache window [0, L_kv), L_kv = offsets[-1].

    words_*: uint32 [B, H, W, L_cap] (only the first L_kv tokens are read),
    scales_*: float32 [B, H, G_cap, D]; offsets: the G+1 block boundaries in
    cache tokens used when the cache was written."""
    q = np.asarray(q, dtype=np.float32)
    D = q.shape[-1]
    if softmax_scale is None:
        softmax_scale = default_softmax_scale(D)
    L_kv = int(offsets[-1])
    G = len(offsets) - 1
    wk = np.asarray(words_k)[..., :L_kv]
    wv = np.asarray(words_v)[..., :L_kv]
    if bh is not None:
        # decode only the (batch, head) pairs asked for
        idx_b = [b for b, _ in bh]
        idx_h = [h for _, h in bh]
        wk = wk[idx_b, idx_h][:, None]
        wv = wv[idx_b, idx_h][:, None]
        sk = np.asarray(scales_k)[idx_b, idx_h][:, None, :G]
        sv = np.asarray(scales_v)[idx_b, idx_h][:, None, :G]
        kh = unpack_dequant(wk, sk, offsets, D, bits)
        vh = unpack_dequant(wv, sv, offsets, D, bits)
        qsel = np.stack([q[b, :, h, :] for b, h in bh])[:, :, None, :]   # [n, Lq, 1, D]
        return attention_fp64(qsel, kh, vh, softmax_scale)
    kh = unpack_dequant(wk, np.asarray(scales_k)[:, :, :G], offsets, D, bits)
    vh = unpack_dequant(wv, np.asarray(scales_v)[:, :, :G], offsets, D, bits)
    return attention_fp64(q, kh, vh, softmax_scale)


def attention_error(o_test, o_ref_bf16, C):
    """The attention tolerance's error measure (a reading: the pages state no
    tolerance, and the absolute bound alone is below the bf16 spacing of
    outputs whose size exceeds 2): the elementwise |O_test - O_ref| divided by
    max(1, C), where C = P|V^| is the size of the weighted sum behind each
    output, reported as its max and mean, next to the raw max/mean absolute
    error. Where C <= 1 the normalised error is the absolute error."""
    d = np.abs(np.asarray(o_test, dtype=np.float64) - np.asarray(o_ref_bf16, dtype=np.float64))
    e = d / np.maximum(1.0, C)
    return {"max_norm": float(e.max()), "mean_norm": float(e.mean()),
            "max_abs": float(d.max()), "mean_abs": float(d.mean())}


# --------------------------------------------------------------------------
# Grouping variants of project page Table 5 (and Table 1): where one scale is
# shared. The "channel axis" is the whole hidden width H * D: a grouping
# without it shares a scale across heads as well as head channels. This is the
# reading that reproduces every VAR-d30 KV-cache size of Table 5 from its
# scale count (10.44 / 9.45 / 9.34 / 10.51 / 9.38 GB).
# --------------------------------------------------------------------------

GROUPINGS = ("channel_block", "channel", "block", "token_head", "token", "tensor")


def grouping_scale_shape(mode, B, L, H, D, G):
    """Compact scale layout of each grouping (one fp32 per group):
    channel_block [B, H, G, D] (VAR-Q, Table 5 "VAR-Q (full)"), channel [B, H, D]
    ("without block axis"), block [B, G] ("without channel axis"), token_head
    [B, H, L] ("per-token & per-head"), token [B, L] ("per-token"), tensor [1]
    (Table 1 "per-tensor")."""
    return {"channel_block": (B, H, G, D), "channel": (B, H, D), "block": (B, G),
            "token_head": (B, H, L), "token": (B, L), "tensor": (1,)}[mode]


def grouping_ids(mode, B, L, H, D, offsets) -> np.ndarray:
    """Flat index into the compact scale layout of every element of x [B, L, H, D];
    int64 [B, L, H, D]."""
    off = _check_offsets(offsets, L)
    G = len(off) - 1
    g_of_t = np.zeros(L, dtype=np.int64)
    for g in range(G):
        g_of_t[off[g]:off[g + 1]] = g
    b = np.arange(B, dtype=np.int64)[:, None, None, None]
    t = np.arange(L, dtype=np.int64)[None, :, None, None]
    h = np.arange(H, dtype=np.int64)[None, None, :, None]
    c = np.arange(D, dtype=np.int64)[None, None, None, :]
    g = g_of_t[None, :, None, None]
    ids = {"channel_block": ((b * H + h) * G + g) * D + c,
           "channel": (b * H + h) * D + c,
           "block": b * G + g + 0 * (h + c),
           "token_head": (b * H + h) * L + t + 0 * c,
           "token": b * L + t + 0 * (h + c),
           "tensor": 0 * (b + t + h + c)}[mode]
    return np.broadcast_to(ids, (B, L, H, D)).astype(np.int64)


def grouped_scales(x, mode, offsets, bits) -> np.ndarray:
    """s = fp32(absmax / qmax) per group of `mode`; float32 of grouping_scale_shape."""
    x = np.asarray(x, dtype=np.float32)
    B, L, H, D = x.shape
    G = len(_check_offsets(offsets, L)) - 1
    shape = grouping_scale_shape(mode, B, L, H, D, G)
    a = np.zeros(int(np.prod(shape)), dtype=np.float32)
    np.maximum.at(a, grouping_ids(mode, B, L, H, D, offsets).ravel(), np.abs(x).ravel())
    return (a / np.float32(qmax(bits))).astype(np.float32).reshape(shape)


def grouped_codes(x, mode, offsets, scales, bits) -> np.ndarray:
    """Codes q = clip(rint(fp32(x / s)), -qmax, qmax) with each element's group
    scale (q = 0 where s = 0); int32 [B, H, L, D]."""
    x = np.asarray(x, dtype=np.float32)
    B, L, H, D = x.shape
    s = np.asarray(scales, dtype=np.float32).ravel()[grouping_ids(mode, B, L, H, D, offsets)]
    safe = np.where(s == 0, np.float32(1), s)
    r = np.where(s == 0, np.float32(0), np.divide(x, safe, dtype=np.float32))
    qm = qmax(bits)
    return np.clip(np.rint(r), -qm, qm).astype(np.int32).transpose(0, 2, 1, 3)


def grouped_quantize_pack(x, mode, offsets, bits):
    """Quantize+pack with the scales of grouping `mode`: (words uint32 [B, H, W, L],
    scales float32 of grouping_scale_shape). The words are laid out exactly like
    the channel x block cache; only where a scale is shared differs."""
    s = grouped_scales(x, mode, offsets, bits)
    return pack_codes(grouped_codes(x, mode, offsets, s, bits), bits), s


def grouped_dequantize(words, scales, mode, offsets, head_dim, bits) -> np.ndarray:
    """bf16_rne(fp32(q) * s) with each element's group scale; float32 [B, L, H, D]."""
    q = unpack_words(words, head_dim, bits).transpose(0, 2, 1, 3)     # [B, L, H, D]
    B, L, H, D = q.shape
    s = np.asarray(scales, dtype=np.float32).ravel()[grouping_ids(mode, B, L, H, D, offsets)]
    return bf16_round_f32((q.astype(np.float32) * s).astype(np.float32))


def grouped_kv_gib(mode, seqs, L, C, D, G, bits, layers) -> float:
    """KV-cache size in GiB of `layers` K and V caches of `seqs` sequences of L
    tokens and C = H * D hidden channels: b-bit codes without padding plus one
    4-byte scale per group (project page, Table 5 "KV (GB)" columns)."""
    H = C // D
    n_scales = int(np.prod(grouping_scale_shape(mode, seqs, L, H, D, G)))
    return 2 * layers * (seqs * L * C * bits / 8 + 4 * n_scales) / 2 ** 30


# --------------------------------------------------------------------------
# Pre-RoPE quantization (project page, Appendix F / Table 7 and Insight 03,
# Eq. 3): K is quantized before the rotary embedding, and the rotation is
# applied to the dequantized K just before attention. RoPE rotates every
# channel pair (2i, 2i+1) by an angle that depends on the token's position;
# the schedule is given as per-token tables cos[t, i], sin[t, i].
# --------------------------------------------------------------------------

def rope_tables(positions, head_dim, base=10000.0):
    """The standard one-axis schedule: angle(t, i) = positions[t] * base^(-2i/D),
    cos and sin computed in fp64 and rounded to fp32; float32 [L, D/2] each."""
    pos = np.asarray(positions, dtype=np.float64)[:, None]
    inv = base ** (-2.0 * np.arange(head_dim // 2, dtype=np.float64) / head_dim)
    ang = pos * inv[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def apply_rope(x, cos, sin) -> np.ndarray:
    """Rotate the pairs (2i, 2i+1) of x [..., L, D] (bf16 values) by the table
    angles of each token: a' = a*c - b*s, b' = a*s + b*c, each product and the
    sum rounded to fp32, then the result rounded to bf16. float32 [..., L, D]."""
    x = np.asarray(x, dtype=np.float32)
    c = np.asarray(cos, dtype=np.float32)
    s = np.asarray(sin, dtype=np.float32)
    a, b = x[..., 0::2], x[..., 1::2]
    a2 = (a * c).astype(np.float32) - (b * s).astype(np.float32)
    b2 = (a * s).astype(np.float32) + (b * c).astype(np.float32)
    out = np.empty_like(x)
    out[..., 0::2] = bf16_round_f32(a2.astype(np.float32))
    out[..., 1::2] = bf16_round_f32(b2.astype(np.float32))
    return out


def packed_attention_rope(q, words_k, scales_k, words_v, scales_v, offsets, bits, cos, sin,
                          softmax_scale=None, bh=None):
    """Attention over a cache whose K was quantized before RoPE: K^ is
    dequantized, rotated by the tables (apply_rope) and only then used; q is
    the already rotated query. Returns what attention_fp64 returns."""
    B, Lq, H, D = np.asarray(q).shape
    khat = apply_rope(unpack_dequant(words_k, scales_k, offsets, D, bits), cos, sin)
    vhat = unpack_dequant(words_v, scales_v, offsets, D, bits)
    sig = default_softmax_scale(D) if softmax_scale is None else np.float32(softmax_scale)
    return attention_fp64(q, khat, vhat, sig, bh)
