"""The synthetic inputs have the structure the pages describe (CPU only)."""

import numpy as np
import torch

from synth import (INFINITY_1024_SIDES, VAR_SIDES, WORKLOADS, frame_offsets,
                   gen_next_scale_kv, gen_rope_frame_k, scale_offsets)


def test_block_schedules():
    assert scale_offsets(VAR_SIDES)[-1] == 680 and len(VAR_SIDES) == 10
    assert scale_offsets(INFINITY_1024_SIDES)[-1] == 10521 and len(INFINITY_1024_SIDES) == 13
    assert frame_offsets(21)[-1] == 32760 and frame_offsets(40)[-1] == 62400
    sf = WORKLOADS["self_forcing"]
    assert [c[2] for c in sf.calls] == [4680 * (j + 1) for j in range(7)]
    assert sf.calls[-1][:2] == (28080, 4680)
    assert WORKLOADS["infinity_8b"].calls[-1][1] == 4096
    assert WORKLOADS["var_d30"].calls[-1][1] == 256


def _top_channels(x, offsets, n):
    # x [B, L, H, D] -> per (b, h, g) the set of the n largest-absmax channels
    out = {}
    for g in range(len(offsets) - 1):
        a = x[:, offsets[g]:offsets[g + 1]].abs().amax(dim=1)          # [B, H, D]
        idx = a.topk(n, dim=-1).indices.sort(-1).values
        out[g] = idx
    return out


def test_k_outliers_shared_across_batch_v_outliers_per_sample():
    """Observation 01: K outlier channels are architectural, V's input driven."""
    off = scale_offsets(VAR_SIDES)
    k = gen_next_scale_kv(4, 3, 64, off, 8, seed=0, stream=1, shared_across_batch=True).float()
    v = gen_next_scale_kv(4, 3, 64, off, 8, seed=0, stream=2, shared_across_batch=False).float()
    g = len(off) - 2                                                     # a 169-token block
    tk = _top_channels(k, off, 8)[g]
    tv = _top_channels(v, off, 8)[g]
    assert all(torch.equal(tk[0], tk[b]) for b in range(1, 4))
    assert not all(torch.equal(tv[0], tv[b]) for b in range(1, 4))
    # outlier magnitudes shift from block to block (per-block drift)
    a = k.abs()
    per_block = torch.stack([a[:, off[i]:off[i + 1]].amax(1) for i in range(5, 10)])  # [5,B,H,D]
    ch = tk[0, 0]
    spread = per_block[:, 0, 0, ch].amax(0) / per_block[:, 0, 0, ch].amin(0)
    assert float(spread.max()) > 1.5


def test_rope_k_pair_envelope_flat_and_channels_trade_across_frames():
    """Insight 03, Eq. 3 and Appendix C (Eq. 4) on the next-frame K generator."""
    ft = 64
    off = frame_offsets(21, ft)
    k = gen_rope_frame_k(1, 2, 128, off, seed=0, stream=1, frame_tokens=ft).float()[0]  # [L,H,D]
    found_swap = False
    for h in range(2):
        for i in range(8):
            a, b = k[:, h, 2 * i], k[:, h, 2 * i + 1]
            if float(torch.maximum(a.abs(), b.abs()).max()) < 10:
                continue                                               # not an outlier pair
            env, ratio = [], []
            for f in range(21):
                af, bf = a[f * ft:(f + 1) * ft].double(), b[f * ft:(f + 1) * ft].double()
                m = torch.sqrt(af ** 2 + bf ** 2).sort(descending=True).values
                lhs = af.abs().max() ** 2 + bf.abs().max() ** 2
                # Eq. 4: M(1)^2 <= |a|_inf^2 + |b|_inf^2 <= M(1)^2 + M(2)^2
                assert m[0] ** 2 <= lhs * (1 + 1e-12) and lhs <= (m[0] ** 2 + m[1] ** 2) * (1 + 1e-12)
                env.append(float(lhs.sqrt()))
                ratio.append(float(af.abs().max() / bf.abs().max()))
            assert max(env) / min(env) < 1.6                             # flat pair envelope
            if max(ratio) > 2 and min(ratio) < 0.5:
                found_swap = True                                      # anti-phase trade
    assert found_swap


def test_generators_are_deterministic():
    off = scale_offsets(VAR_SIDES[:5])
    a = gen_next_scale_kv(2, 2, 64, off, 4, seed=3, stream=1)
    b = gen_next_scale_kv(2, 2, 64, off, 4, seed=3, stream=1)
    c = gen_next_scale_kv(2, 2, 64, off, 4, seed=4, stream=1)
    assert torch.equal(a, b) and not torch.equal(a, c)
    assert a.dtype == torch.bfloat16 and a.shape == (2, off[-1], 2, 64)
    assert np.isfinite(a.float().numpy()).all()


def test_pre_rope_generator_is_the_post_rope_one_before_rotation():
    """gen_pre_rope_frame_k draws exactly what gen_rope_frame_k draws, before
    the frame rotation: rotating its (bf16-rounded) K by its own tables gives the
    post-RoPE K within the bf16 rounding of the pair (errors scale with the
    pair's norm, since both channels of a pair mix)."""
    import numpy as np
    from oracle import varq_oracle as O
    from synth import gen_pre_rope_frame_k, gen_rope_frame_k
    from synth.kv_synth import FRAME_TOKENS
    off = [0, FRAME_TOKENS, 2 * FRAME_TOKENS]
    kpre, cos, sin = gen_pre_rope_frame_k(1, 2, 128, off, 0, 1)
    kpost = gen_rope_frame_k(1, 2, 128, off, 0, 1)
    rot = O.apply_rope(kpre.float().numpy().transpose(0, 2, 1, 3), cos.numpy(), sin.numpy()).transpose(0, 2, 1, 3)
    ref = kpost.float().numpy()
    pair = np.repeat(np.hypot(ref[..., 0::2], ref[..., 1::2]), 2, axis=-1)
    assert np.all(np.abs(rot - ref) <= 2 ** -6 * pair + 2 ** -6)
    # and the tables are the frame schedule: all tokens of a frame share the angle
    assert np.array_equal(cos[0].numpy(), np.ones(64, np.float32))
    assert np.array_equal(cos[FRAME_TOKENS - 1].numpy(), cos[0].numpy())
    assert not np.array_equal(cos[FRAME_TOKENS].numpy(), cos[0].numpy())
