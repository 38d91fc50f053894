"""Writes grouping_errors.json: relative Frobenius errors of every scale grouping
(project page Table 1 and Table 5 groupings) on the synthetic workloads, from
the oracle only.

For each workload, INT4, and each grouping:
  K, V       ||X - X'||_F / ||X||_F over the whole cache;
  attention  ||P - P'||_F / ||P||_F of the softmax weights and
  output     ||O - O'||_F / ||O||_F of the attention output,
over sampled (batch, head) pairs and queries, where P, O use the bf16 K, V and
P', O' the dequantized ones (fp64 arithmetic). Run from the repository root:
    python tests/golden/grouping_error_report.py
"""

import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import varq_oracle as O  # noqa: E402
from synth import WORKLOADS, gen_next_scale_kv, gen_queries, gen_rope_frame_k  # noqa: E402

BITS = 4
MODES = ("tensor", "block", "channel", "channel_block", "token", "token_head")


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / np.linalg.norm(a))


def _attn(q, k, v, sig):
    s = (q @ k.T) * sig
    s -= s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=1, keepdims=True)
    return p, p @ v


def inputs(name, seed=0):
    """K, V [B, L, H, D] and queries [B, Lq, H, D] (float32 holding bf16) at the report's size."""
    wl = WORKLOADS[name]
    if name == "infinity_8b":
        B, off, lq = 1, list(wl.offsets), 256            # one sequence, 256 of the last block's queries
    elif name == "self_forcing":
        B, off, lq = 1, list(wl.offsets)[:7], 256        # one sequence, the first two 3-frame blocks
    else:
        B, off, lq = wl.B, list(wl.offsets), wl.calls[-1][1]
    if wl.kind == "next_scale":
        k = gen_next_scale_kv(B, wl.H, wl.D, off, wl.n_out_k, seed, 1, shared_across_batch=True)
    else:
        k = gen_rope_frame_k(B, wl.H, wl.D, off, seed, 1, n_out_pairs=wl.n_out_k)
    v = gen_next_scale_kv(B, wl.H, wl.D, off, wl.n_out_v, seed, 2, shared_across_batch=False)
    q = gen_queries(B, lq, wl.H, wl.D, seed, 3)
    return k.float().numpy(), v.float().numpy(), q.float().numpy(), off


def report(name, pairs=4, seed=0):
    k, v, q, off = inputs(name, seed)
    B, L, H, D = k.shape
    sig = float(O.default_softmax_scale(D))
    rng = np.random.RandomState(seed)
    bh = [(int(rng.randint(B)), int(rng.randint(H))) for _ in range(pairs)]
    rows = {}
    for mode in MODES:
        wk, sk = O.grouped_quantize_pack(k, mode, off, BITS)
        wv, sv = O.grouped_quantize_pack(v, mode, off, BITS)
        kq = O.grouped_dequantize(wk, sk, mode, off, D, BITS)
        vq = O.grouped_dequantize(wv, sv, mode, off, D, BITS)
        pe, oe = [], []
        for (b, h) in bh:
            qq = q[b, :, h, :].astype(np.float64)
            p0, o0 = _attn(qq, k[b, :, h, :].astype(np.float64), v[b, :, h, :].astype(np.float64), sig)
            p1, o1 = _attn(qq, kq[b, :, h, :].astype(np.float64), vq[b, :, h, :].astype(np.float64), sig)
            pe.append((p0, p1))
            oe.append((o0, o1))
        rows[mode] = {
            "k": _rel(k, kq), "v": _rel(v, vq),
            "attention": _rel(np.concatenate([a for a, _ in pe]), np.concatenate([b for _, b in pe])),
            "output": _rel(np.concatenate([a for a, _ in oe]), np.concatenate([b for _, b in oe])),
            "scales_per_tensor": int(sk.size),
        }
    return {"shape": [B, L, H, D], "blocks": len(off) - 1, "pairs": bh, "queries": int(q.shape[1]),
            "errors": rows}


def frame_maps(L):
    """Group boundaries of a next-frame cache: 1560-token frames, the 4680-token
    chunk (compression ratio 3) and 1560-token frames shifted by half a frame
    (project page Table 6's misaligned placement). Written out here (not taken
    from the library's helper) so the report depends on the oracle only."""
    def frames(g, phase=0):
        inner = [b for b in range(phase if phase else g, L, g) if 0 < b < L]
        return [0] + inner + [L]
    return {"frames_1560": frames(1560), "chunk_4680": frames(4680), "frames_1560_misaligned": frames(1560, 780)}


def boundary_report(name="self_forcing", pairs=4, seed=0):
    k, v, q, _ = inputs(name, seed)
    B, L, H, D = k.shape
    sig = float(O.default_softmax_scale(D))
    rng = np.random.RandomState(seed)
    bh = [(int(rng.randint(B)), int(rng.randint(H))) for _ in range(pairs)]
    rows = {}
    for tag, off in frame_maps(L).items():
        wk, sk = O.quantize_pack(k, off, BITS)
        wv, sv = O.quantize_pack(v, off, BITS)
        kq = O.unpack_dequant(wk, sk, off, D, BITS).transpose(0, 2, 1, 3)
        vq = O.unpack_dequant(wv, sv, off, D, BITS).transpose(0, 2, 1, 3)
        oe = []
        for (b, h) in bh:
            qq = q[b, :, h, :].astype(np.float64)
            _, o0 = _attn(qq, k[b, :, h, :].astype(np.float64), v[b, :, h, :].astype(np.float64), sig)
            _, o1 = _attn(qq, kq[b, :, h, :].astype(np.float64), vq[b, :, h, :].astype(np.float64), sig)
            oe.append((o0, o1))
        rows[tag] = {"blocks": len(off) - 1, "k": _rel(k, kq), "v": _rel(v, vq),
                     "output": _rel(np.concatenate([a for a, _ in oe]), np.concatenate([b for _, b in oe]))}
    return {"shape": [B, L, H, D], "maps": rows}


def main():
    out = {"_about": "Relative Frobenius errors (fractions) of INT4 quantize-dequantize under each scale "
                     "grouping, computed by tests/golden/grouping_error_report.py from the oracle on the "
                     "synthetic workloads (project page Table 1 reports the same four quantities for "
                     "Infinity-2B; Table 5 the groupings).",
           "bits": BITS, "workloads": {}}
    for name in ("tiny", "var_d30", "infinity_8b", "self_forcing"):
        print("report", name, flush=True)
        out["workloads"][name] = report(name)
    print("report boundaries self_forcing", flush=True)
    out["boundaries"] = boundary_report()
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "grouping_errors.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print("wrote", path)


if __name__ == "__main__":
    main()
