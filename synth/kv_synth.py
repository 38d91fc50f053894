"""Seeded synthetic K/V/Q tensors with the pages' channel x block structure.

What the generators imitate (VAR-Q project page):
  * "Next-block prediction": a block is one resolution scale (next-scale models)
    or one frame (next-frame models); the cache is indexed by feature channel and
    generation block.
  * "Channel x block KV-cache quantization": a few channels carry large values
    and their magnitudes shift from block to block.
  * Observation 01 (Fig. 5): K outlier channels are architectural (shared across
    inputs), V outlier channels are input driven (drawn per sample).
  * Insight 03, Eq. 3: RoPE rotates each channel pair (2i, 2i+1) by the block
    index times the pair frequency; every token of a block shares the rotation,
    so the two channels of a fast pair trade magnitude across blocks.

Everything is drawn in float32 with torch generators and rounded once to bf16 by
torch's own conversion. Nothing here quantizes, packs or attends.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

# Resolution schedule of a VAR-style next-scale model (side lengths; a scale of
# side s emits s*s tokens): 680 tokens in 10 blocks.
VAR_SIDES = (1, 2, 3, 4, 5, 6, 8, 10, 13, 16)
# Infinity-style 1024px schedule: 10521 tokens in 13 blocks.
INFINITY_1024_SIDES = (1, 2, 4, 6, 8, 12, 16, 20, 24, 32, 40, 48, 64)
# Next-frame models: one latent frame is 1560 tokens; the default grouping unit
# of the README's "Configs" section is one frame.
FRAME_TOKENS = 1560


def scale_offsets(sides):
    """Prefix token offsets of a next-scale schedule (block j holds sides[j]**2 tokens)."""
    off = [0]
    for s in sides:
        off.append(off[-1] + int(s) * int(s))
    return off


def frame_offsets(n_groups, tokens_per_group=FRAME_TOKENS):
    """Prefix token offsets of n_groups equal frame groups."""
    return [i * tokens_per_group for i in range(n_groups + 1)]


def _gen(seed, stream, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1_000_003 + int(stream))
    return g


def _group_index(offsets, device):
    sizes = torch.tensor([offsets[i + 1] - offsets[i] for i in range(len(offsets) - 1)],
                         device=device)
    return torch.repeat_interleave(torch.arange(len(sizes), device=device), sizes)


def _outlier_multiplier(gen, n_sets, H, D, G, n_out, device, lo=20.0, hi=50.0,
                        drift_lo=0.5, drift_hi=2.0):
    """Per-(set, head, group, channel) multiplier: 1 off the outlier channels,
    base U(lo, hi) times a per-group log-uniform drift in [drift_lo, drift_hi] on
    n_out channels chosen per (set, head)."""
    mult = torch.ones(n_sets, H, G, D, device=device)
    if n_out <= 0:
        return mult
    pick = torch.rand(n_sets, H, D, generator=gen, device=device).argsort(dim=-1)[..., :n_out]
    base = lo + (hi - lo) * torch.rand(n_sets, H, n_out, generator=gen, device=device)
    ld = math.log(drift_lo) + (math.log(drift_hi) - math.log(drift_lo)) * torch.rand(
        n_sets, H, n_out, G, generator=gen, device=device)
    val = base[..., None] * torch.exp(ld)                      # [S, H, n_out, G]
    val = val.permute(0, 1, 3, 2)                               # [S, H, G, n_out]
    idx = pick[:, :, None, :].expand(n_sets, H, G, n_out)
    mult.scatter_(3, idx, val)
    return mult


def gen_next_scale_kv(B, H, D, offsets, n_out, seed, stream, device="cpu",
                      shared_across_batch=True):
    """bf16 [B, L, H, D]: N(0,1) values whose n_out outlier channels per head are
    scaled by U(20,50) x a per-block drift in [0.5, 2].

    shared_across_batch=True draws one outlier set for the whole batch (the K
    behaviour of Observation 01); False draws it per batch element (V)."""
    G = len(offsets) - 1
    L = offsets[-1]
    gen = _gen(seed, stream, device)
    x = torch.randn(B, L, H, D, generator=gen, device=device)
    n_sets = 1 if shared_across_batch else B
    mult = _outlier_multiplier(gen, n_sets, H, D, G, n_out, device)   # [S,H,G,D]
    gidx = _group_index(offsets, device)                               # [L]
    m = mult[:, :, gidx, :].permute(0, 2, 1, 3)                        # [S,L,H,D]
    x.mul_(m)
    return x.to(torch.bfloat16)


def _frame_k_pre(B, H, D, L, gen, device, n_fast_pairs, n_out_pairs, angle_jitter):
    """Pre-RoPE K of the next-frame generator, fp32 [B, L, H, D] (see gen_rope_frame_k)."""
    k = torch.randn(B, L, H, D, generator=gen, device=device)
    pairs = torch.rand(H, n_fast_pairs, generator=gen, device=device).argsort(-1)[:, :n_out_pairs]
    amp0 = 20.0 + 30.0 * torch.rand(H, n_out_pairs, generator=gen, device=device)
    phi0 = 2.0 * math.pi * torch.rand(H, n_out_pairs, generator=gen, device=device)
    amp = amp0 * (1.0 + 0.1 * torch.randn(B, L, H, n_out_pairs, generator=gen, device=device))
    ang = phi0 + angle_jitter * torch.randn(B, L, H, n_out_pairs, generator=gen, device=device)
    ch_even = (2 * pairs)                                             # [H, P]
    hidx = torch.arange(H, device=device)[:, None].expand_as(ch_even)
    k[:, :, hidx, ch_even] = amp * torch.cos(ang)
    k[:, :, hidx, ch_even + 1] = amp * torch.sin(ang)
    return k


def rope_frame_tables(L, D, device="cpu", frame_tokens=FRAME_TOKENS, rope_base=10000.0):
    """RoPE along the frame axis: cos and sin of frame(t) * omega_i, omega_i =
    base**(-2i/D), fp32 [L, D/2] each (all tokens of a frame share the angle)."""
    frame = (torch.arange(L, device=device) // frame_tokens).to(torch.float32)   # [L]
    i = torch.arange(D // 2, device=device, dtype=torch.float32)
    omega = rope_base ** (-2.0 * i / D)                                           # [D/2]
    theta = frame[:, None] * omega[None, :]                                       # [L, D/2]
    return torch.cos(theta), torch.sin(theta)


def gen_rope_frame_k(B, H, D, offsets, seed, stream, device="cpu", frame_tokens=FRAME_TOKENS,
                     n_fast_pairs=8, n_out_pairs=4, rope_base=10000.0, angle_jitter=0.1):
    """Post-RoPE K of a next-frame model, bf16 [B, L, H, D] (Insight 03, Eq. 3).

    Pre-RoPE K is N(0,1); in n_out_pairs of the n_fast_pairs lowest-index pairs of
    each head the pair has per-token amplitude M_t = U(20,50)*(1+0.1 N(0,1)) and
    angle phi_t = phi_{h,i} + angle_jitter * N(0,1). Every pair i of every token of frame f
    is then rotated by f*omega_i, omega_i = base**(-2i/D); all tokens of a frame
    share the angle. The frame index drives the rotation (blocks are frames)."""
    L = offsets[-1]
    gen = _gen(seed, stream, device)
    k = _frame_k_pre(B, H, D, L, gen, device, n_fast_pairs, n_out_pairs, angle_jitter)
    cos, sin = rope_frame_tables(L, D, device, frame_tokens, rope_base)
    c = cos[None, :, None, :]
    s = sin[None, :, None, :]
    ke, ko = k[..., 0::2], k[..., 1::2]
    re = ke * c - ko * s
    ro = ke * s + ko * c
    out = torch.stack((re, ro), dim=-1).reshape(B, L, H, D)
    return out.to(torch.bfloat16)


def gen_pre_rope_frame_k(B, H, D, offsets, seed, stream, device="cpu", frame_tokens=FRAME_TOKENS,
                         n_fast_pairs=8, n_out_pairs=4, rope_base=10000.0, angle_jitter=0.1):
    """The same draws as gen_rope_frame_k before the rotation: pre-RoPE K, bf16
    [B, L, H, D], and its rotation tables (cos, sin) fp32 [L, D/2] (inputs of the
    pre-RoPE path, project page Appendix F)."""
    L = offsets[-1]
    gen = _gen(seed, stream, device)
    k = _frame_k_pre(B, H, D, L, gen, device, n_fast_pairs, n_out_pairs, angle_jitter)
    cos, sin = rope_frame_tables(L, D, device, frame_tokens, rope_base)
    return k.to(torch.bfloat16), cos, sin


def gen_queries(B, Lq, H, D, seed, stream, device="cpu"):
    """Queries ~ N(0,1), bf16 [B, Lq, H, D] (the pages say nothing of Q's distribution)."""
    gen = _gen(seed, stream, device)
    return torch.randn(B, Lq, H, D, generator=gen, device=device).to(torch.bfloat16)


def gen_unit_v(B, L, H, D, seed, stream, device="cpu"):
    """V ~ N(0,1) without outlier channels (the unit-V twin of a workload)."""
    gen = _gen(seed, stream, device)
    return torch.randn(B, L, H, D, generator=gen, device=device).to(torch.bfloat16)


@dataclass(frozen=True)
class Workload:
    """One synthetic workload. `offsets` are the group (block) boundaries in cache
    tokens; `calls` lists the packed-attention calls as (q_start, q_len, L_kv)
    with queries taken from the cache-aligned block [q_start, q_start+q_len)."""
    name: str
    B: int
    H: int
    D: int
    offsets: tuple
    bits: tuple
    kind: str                 # "next_scale" | "next_frame"
    n_out_k: int
    n_out_v: int
    calls: tuple
    append_blocks: tuple = field(default=())   # next-frame: group offsets of each generation block
    description: str = ""

    @property
    def L(self):
        return self.offsets[-1]

    @property
    def G(self):
        return len(self.offsets) - 1


def _last_block_call(off):
    return ((off[-2], off[-1] - off[-2], off[-1]),)


_VAR_OFF = tuple(scale_offsets(VAR_SIDES))
_INF_OFF = tuple(scale_offsets(INFINITY_1024_SIDES))
_SF_OFF = tuple(frame_offsets(21))
_LL_OFF = tuple(frame_offsets(40))

WORKLOADS = {
    "tiny": Workload(
        name="tiny", B=1, H=16, D=64, offsets=_VAR_OFF, bits=(4,), kind="next_scale",
        n_out_k=8, n_out_v=8, calls=_last_block_call(_VAR_OFF),
        description="1 layer, batch 1, 16 heads x 64, 10 VAR scales (680 tokens), INT4"),
    "var_d30": Workload(
        name="var_d30", B=16, H=30, D=64, offsets=_VAR_OFF, bits=(4, 8), kind="next_scale",
        n_out_k=8, n_out_v=8, calls=_last_block_call(_VAR_OFF),
        description="VAR-d30-like: batch 16, 30 heads x 64, 10 scales (680 tokens), "
                    "last scale (256 queries) over the full packed cache; INT4 and INT8"),
    "infinity_8b": Workload(
        name="infinity_8b", B=8, H=32, D=128, offsets=_INF_OFF, bits=(4, 2), kind="next_scale",
        n_out_k=5, n_out_v=5, calls=_last_block_call(_INF_OFF),
        description="Infinity-8B-like 1024px: batch 4 x 2 (CFG), 32 heads x 128, 13 scales "
                    "(10521 tokens), last block 4096 queries; INT4 and INT2"),
    "self_forcing": Workload(
        name="self_forcing", B=12, H=12, D=128, offsets=_SF_OFF, bits=(4,), kind="next_frame",
        n_out_k=4, n_out_v=6,
        calls=tuple((4680 * j, 4680, 4680 * (j + 1)) for j in range(7)),
        append_blocks=tuple((3 * j, 3 * j + 3) for j in range(7)),
        description="Self-Forcing-like: batch 12, 12 heads x 128, 7 blocks of 3 frames x 1560 "
                    "tokens (32760 total); block j attends to all prior packed blocks and itself; INT4"),
    "longlive": Workload(
        name="longlive", B=4, H=12, D=128, offsets=_LL_OFF, bits=(3, 2), kind="next_frame",
        n_out_k=4, n_out_v=6, calls=((62400 - 1560, 1560, 62400),),
        append_blocks=tuple((j, j + 1) for j in range(40)),
        description="LongLive-like: batch 4, 12 heads x 128, 40 frame blocks x 1560 tokens "
                    "(62400-token cache); INT3 and INT2; 1560 queries over the full cache"),
}


def workload_inputs(wl: Workload, seed=0, device="cpu", unit_v=False, with_v=True):
    """K, V (bf16 [B, L, H, D]) and the queries of the workload's last attention
    call (bf16 [B, Lq, H, D]). Sub-streams: 1 = K, 2 = V, 3 = Q."""
    if wl.kind == "next_scale":
        k = gen_next_scale_kv(wl.B, wl.H, wl.D, wl.offsets, wl.n_out_k, seed, 1, device,
                              shared_across_batch=True)
    else:
        k = gen_rope_frame_k(wl.B, wl.H, wl.D, wl.offsets, seed, 1, device,
                             n_out_pairs=wl.n_out_k)
    v = None
    if with_v:
        if unit_v:
            v = gen_unit_v(wl.B, wl.L, wl.H, wl.D, seed, 2, device)
        else:
            v = gen_next_scale_kv(wl.B, wl.H, wl.D, wl.offsets, wl.n_out_v, seed, 2, device,
                                  shared_across_batch=False)
    q_len = wl.calls[-1][1]
    q = gen_queries(wl.B, q_len, wl.H, wl.D, seed, 3, device)
    return k, v, q
