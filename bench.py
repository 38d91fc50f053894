#!/usr/bin/env python3
"""Benchmark of the VAR-Q packed KV-cache hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
quantize+pack of K and V in one call (per-channel x per-block absmax, scales,
codes, INT32 words into a preallocated cache) followed by the packed-KV
attention call(s) of the workload (load packed words, unpack, dequantize,
QK^T, softmax, PV). The default workload is the Self-Forcing-like next-frame
loop, the largest configuration: seven generation blocks of 4680 tokens, each
quantized and packed and then attended by its 4680 queries over all blocks
so far.

Prints ONE JSON line. `value` is the step's algorithmic bytes (quant-pack:
bf16 in + words + scales out; attention: Q + O + packed K/V + scales) divided
by the step time, in GB/s. `roofline` reports the kernel with the largest
share of the step time against its bound (HBM for quant-pack, bf16 MFMA for
attention); its time is the timed steps' GPU time (two HIP events on the
launch stream around them) less the other kernel's, which comes from
kernel-only passes (the K steps with only that kernel's launches, back to
back, between two HIP events) just before and just after the timed steps.
`cpu_baseline` times the CPU oracle on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
DEFAULT_WORKLOAD = "self_forcing"
METRIC = "packed-KV attention GB/s + quant-pack GB/s, % of MI355X HBM peak"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD)
    p.add_argument("--bits", type=int, default=None)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-budget-s", type=float, default=15.0)
    p.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                   help="only run 5 plain device-to-device copies of BYTES bytes (counter calibration)")
    p.add_argument("--grouping-report", action="store_true",
                   help="only time quantize+pack of K under every scale grouping (one JSON line)")
    p.add_argument("--pre-rope-report", action="store_true",
                   help="only time the last attention call with K quantized before RoPE against the "
                        "plain (post-RoPE) kernel (one JSON line)")
    p.add_argument("--fusion-report", action="store_true",
                   help="only time the workload's last attention call fused (packed attention) against "
                        "unfused (unpack+dequant of K and V, then bf16 attention) per call (one JSON line)")
    p.add_argument("--batch", type=int, default=None,
                   help="with --fusion-report: sequences per call (default: the workload's batch)")
    return p.parse_args()


def copy_probe(nbytes):
    """Five plain device copies of a known size: the reference that scales the
    HBM byte counters (FETCH_SIZE / WRITE_SIZE) of the kernels."""
    import torch
    x = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(5):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes, "copies": 5}), flush=True)


# ---------------------------------------------------------------- algorithmic work

def qp_bytes(B, L, H, D, G, bits):
    cpw = 32 // bits
    W = -(-D // cpw)
    return B * L * H * D * 2 + B * H * W * L * 4 + B * H * G * D * 4


def attn_bytes(B, H, D, Lq, L_kv, G, bits):
    cpw = 32 // bits
    W = -(-D // cpw)
    return B * H * (2 * Lq * D * 2 + 2 * L_kv * W * 4 + 2 * G * D * 4)


def attn_flops(B, H, D, Lq, L_kv):
    return 4.0 * B * H * Lq * L_kv * D


def plan(wl, bits):
    """The step's launches: list of ('qp', t0, t1, g0, g1) and ('attn', call)."""
    off = list(wl.offsets)
    steps = []
    done_g = 0
    for (q0, ql, L_kv) in wl.calls:
        g1 = off.index(L_kv)
        if g1 > done_g:
            steps.append(("qp", off[done_g], L_kv, done_g, g1))
            done_g = g1
        steps.append(("attn", q0, ql, L_kv, g1))
    return steps


def kernel_hash(name):
    path = os.path.join(ROOT, "kv_cache_quantization_02_amd", "csrc", name)
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def load_traffic(kernel_file, workload, bits):
    """Measured HBM bytes per launch from committed rocprofv3 counter runs, if the
    kernel source is unchanged since they were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rows = json.load(f)
    for r in rows:
        if (r.get("kernel_file") == kernel_file and r.get("workload") == workload
                and r.get("bits") == bits and r.get("source_sha") == kernel_hash(kernel_file)):
            return r
    return None


# ---------------------------------------------------------------- CPU baseline

def cpu_baseline(wl, bits, budget_s, step_bytes, k, v, q):
    """The oracle as it stands on a bounded sample: whole-step (batch, head)
    slices, each the quantize+pack of that slice's K and V over the step's
    tokens and every attention call of the step for that (batch, head), until
    about budget_s seconds of CPU work. The rate is the slices' algorithmic
    bytes (the GPU step's bytes / (B * H) per slice) over the CPU time, in the
    unit of `value`; a whole step at that rate is extrapolated. k, v, q are
    the step's inputs (any device); each slice is copied to the host first,
    outside the timed CPU work."""
    import numpy as np

    from oracle import varq_oracle as O

    off = list(wl.offsets)
    launches = plan(wl, bits)
    rng = np.random.default_rng(0)
    per_slice = step_bytes / (wl.B * wl.H)
    nbytes = 0.0
    slices = []
    sig = O.default_softmax_scale(wl.D)
    dt = 0.0
    while dt < budget_s and len(slices) < wl.B * wl.H:
        b, h = int(rng.integers(wl.B)), int(rng.integers(wl.H))
        ks = k[b:b + 1, :, h:h + 1].float().cpu().numpy()
        vs = v[b:b + 1, :, h:h + 1].float().cpu().numpy()
        qs = q[b:b + 1, :, h:h + 1].float().cpu().numpy()
        t_start = time.perf_counter()
        W = O.words_per_row(wl.D, bits)
        wk = np.zeros((1, 1, W, wl.L), np.uint32)
        wv = np.zeros_like(wk)
        sk = np.zeros((1, 1, wl.G, wl.D), np.float32)
        sv = np.zeros_like(sk)
        for st in launches:
            if st[0] == "qp":
                _, t0, t1, g0, g1 = st
                rel = [o - t0 for o in off[g0:g1 + 1]]
                wk[..., t0:t1], sk[:, :, g0:g1] = O.quantize_pack(ks[:, t0:t1], rel, bits)
                wv[..., t0:t1], sv[:, :, g0:g1] = O.quantize_pack(vs[:, t0:t1], rel, bits)
            else:
                _, q0, ql, L_kv, g1 = st
                O.packed_attention(qs[:, :ql], wk, sk, wv, sv, off[:g1 + 1], bits, sig)
        dt += time.perf_counter() - t_start
        nbytes += per_slice
        slices.append((b, h))
    threads = len(os.sched_getaffinity(0))
    try:
        threads = min(threads, int(os.environ.get("OMP_NUM_THREADS", threads)))
    except ValueError:
        pass
    rate = nbytes / dt / 1e9
    return {"value": round(rate, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(slices)} whole-step (batch, head) slices of {wl.name} out of {wl.B * wl.H} "
                      f"(quantize+pack of the slice's K and V as the step does, then the step's "
                      f"{sum(1 for x in launches if x[0] != 'qp')} attention call(s)), {dt:.1f} s of CPU time; "
                      f"numpy/BLAS threads <= {threads}; a whole step at this rate: "
                      f"{step_bytes / (rate * 1e9):.0f} s (extrapolated)"}


# ---------------------------------------------------------------- unfused baseline

def unfused_compare(varq, torch, wl, bits, launches, off, q, pk, sk, pv, sv, args, fused_ms):
    """The attention calls of one step done the unfused way: unpack+dequant of
    K and V into bf16 workspaces, then plain bf16 attention, timed back to back
    per step with HIP events (same stream), outside the main timed region."""
    calls = [st for st in launches if st[0] != "qp"]
    if not calls:
        return None
    B, H, D = wl.B, wl.H, wl.D
    L_max = max(st[3] for st in calls)
    kd = torch.empty(B, H, L_max, D, dtype=torch.bfloat16, device=q.device)
    vd = torch.empty_like(kd)
    out = torch.empty_like(q)

    def one(st):
        _, q0, ql, L_kv, g1 = st
        # contiguous [B, H, L_kv, D] views at the start of the workspaces
        kw = kd.view(-1)[:B * H * L_kv * D].view(B, H, L_kv, D)
        vw = vd.view(-1)[:B * H * L_kv * D].view(B, H, L_kv, D)
        varq.unpack_dequant(pk, sk, off[:g1 + 1], bits, out=kw)
        varq.unpack_dequant(pv, sv, off[:g1 + 1], bits, out=vw)
        varq.bf16_attention(q, kw, vw, out=out)

    for _ in range(max(1, args.warmup)):
        for st in calls:
            one(st)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        for st in calls:
            one(st)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    return {"path": "unpack_dequant(K), unpack_dequant(V) into bf16, then bf16_attention",
            "timing": "the step's attention calls back to back, per step",
            "ms_per_step": round(ms, 5), "fused_ms_per_step": round(fused_ms, 5),
            "fused_speedup": round(ms / fused_ms, 3) if fused_ms else None,
            "dequant_workspace_bytes": int(kd.numel() * kd.element_size() * 2)}


def device_copy_rate(torch, nbytes=1 << 30, reps=5):
    """Read + write bytes per second of a plain device-to-device copy: the
    memory rate this device reaches on a streaming kernel, for context."""
    x = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    y.copy_(x)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        y.copy_(x)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del x, y
    return 2 * nbytes / (ms * 1e-3) / 1e9


# ---------------------------------------------------------------- grouping report

def grouping_report(varq, torch, wl, bits, k, args):
    """quantize+pack of the workload's K under each scale grouping of the
    project page's Table 5 / Table 1, event-timed per launch. Algorithmic bytes
    count one read of K plus the words and scales written (the groupings other
    than channel x block and channel read K twice)."""
    B, L, H, D = k.shape
    G = len(wl.offsets) - 1
    W = varq.words_per_row(D, bits)
    packed = torch.zeros(B, H, W, varq.round_capacity(L), dtype=torch.int32, device=k.device)
    modes = {}
    for mode in varq.GROUPINGS:
        scales = torch.zeros(varq.grouped_scale_shape(mode, B, L, H, D, G), dtype=torch.float32, device=k.device)
        fn = lambda: varq.quantize_pack_grouped(k, list(wl.offsets), bits, mode, packed, scales)
        for _ in range(max(1, args.warmup)):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for a, b in ev:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        ms = sum(a.elapsed_time(b) for a, b in ev) / len(ev)
        nbytes = B * L * H * D * 2 + B * H * W * L * 4 + scales.numel() * 4
        modes[mode] = {"avg_ms": round(ms, 5), "alg_bytes": nbytes, "scales": scales.numel(),
                       "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
                       "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    maps = {}
    if wl.kind == "next_frame":
        # channel x block with other boundary maps: the 4680-token chunk
        # (compression ratio 3) and 1560-token frames shifted by half a frame
        scales = torch.zeros(B, H, L // 780 + 2, D, dtype=torch.float32, device=k.device)
        for tag, off in (("frames_1560", varq.frame_group_offsets(L, 1560)),
                         ("chunk_4680", varq.frame_group_offsets(L, 4680)),
                         ("frames_1560_misaligned", varq.frame_group_offsets(L, 1560, phase=780))):
            fn = lambda: varq.quantize_pack(k, off, bits, packed, scales)
            for _ in range(max(1, args.warmup)):
                fn()
            torch.cuda.synchronize()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
            for a, b in ev:
                a.record()
                fn()
                b.record()
            torch.cuda.synchronize()
            ms = sum(a.elapsed_time(b) for a, b in ev) / len(ev)
            nbytes = qp_bytes(B, L, H, D, len(off) - 1, bits)
            maps[tag] = {"blocks": len(off) - 1, "avg_ms": round(ms, 5), "alg_bytes": nbytes,
                         "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1)}
    print(json.dumps({"grouping_report": {"workload": wl.name, "bits": bits, "tensor": "K",
                                          "shape": [B, L, H, D], "blocks": G, "steps": args.steps,
                                          "modes": modes, "boundary_maps": maps}}))


# ---------------------------------------------------------------- pre-RoPE report

def pre_rope_report(varq, torch, wl, bits, args):
    """The workload's last attention call three ways, event-timed per call: the
    plain packed attention (post-RoPE cache, the method's default), the same
    call on a cache quantized before RoPE with the rotation applied to every
    dequantized K tile (project page Appendix F / Table 7), and the unfused
    pre-RoPE path (unpack_dequant_rope + unpack_dequant + bf16_attention)."""
    from synth import gen_next_scale_kv, gen_pre_rope_frame_k, gen_queries, rope_frame_tables
    dev = torch.device("cuda:0")
    off = list(wl.offsets)
    if wl.kind == "next_frame":
        k, cos, sin = gen_pre_rope_frame_k(wl.B, wl.H, wl.D, off, 0, 1, dev)
    else:
        k = gen_next_scale_kv(wl.B, wl.H, wl.D, off, wl.n_out_k, 0, 1, dev, shared_across_batch=True)
        cos, sin = rope_frame_tables(wl.L, wl.D, dev)
    v = gen_next_scale_kv(wl.B, wl.H, wl.D, off, wl.n_out_v, 0, 2, dev, shared_across_batch=False)
    q0, ql, L_kv = wl.calls[-1]
    q = gen_queries(wl.B, ql, wl.H, wl.D, 0, 3, dev)
    B, H, D = wl.B, wl.H, wl.D
    pk, sk = varq.alloc_cache(B, H, D, wl.L, len(off) - 1, bits, device=dev)
    pv, sv = varq.alloc_cache(B, H, D, wl.L, len(off) - 1, bits, device=dev)
    varq.quantize_pack(k, off, bits, pk, sk)
    varq.quantize_pack(v, off, bits, pv, sv)
    del k, v
    goff = off[:off.index(L_kv) + 1]
    out = torch.empty_like(q)
    kd = torch.empty(B, H, L_kv, D, dtype=torch.bfloat16, device=dev)
    vd = torch.empty_like(kd)

    def timeit(fn):
        for _ in range(max(1, args.warmup)):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for a, b in ev:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in ev) / len(ev)

    def unfused():
        varq.unpack_dequant_rope(pk, sk, goff, bits, cos, sin, out=kd)
        varq.unpack_dequant(pv, sv, goff, bits, out=vd)
        varq.bf16_attention(q, kd, vd, out=out)

    t_post = timeit(lambda: varq.packed_attention(q, pk, sk, pv, sv, goff, bits, out=out))
    t_pre = timeit(lambda: varq.packed_attention_rope(q, pk, sk, pv, sv, goff, bits, cos, sin, out=out))
    t_unf = timeit(unfused)
    flops = attn_flops(B, H, D, ql, L_kv)
    rows = {name: {"avg_ms": round(t, 5), "TFLOP/s": round(flops / (t * 1e-3) / 1e12, 2)}
            for name, t in (("post_rope_fused", t_post), ("pre_rope_fused", t_pre), ("pre_rope_unfused", t_unf))}
    print(json.dumps({"pre_rope_report": {"workload": wl.name, "bits": bits, "call": [q0, ql, L_kv],
                                          "steps": args.steps, "calls": rows,
                                          "rotation_overhead": round(t_pre / t_post - 1.0, 4)}}))


# ---------------------------------------------------------------- fusion report

def fusion_report(varq, torch, wl, bits, args):
    """The workload's last attention call at `--batch` sequences, fused (packed
    attention reading the packed cache) against unfused (unpack+dequant of K
    and V into bf16, then bf16 attention), each timed back to back per call
    with HIP events (README "Deployment Results": the fused operator against
    the unfused path on Infinity-8B at batch 1)."""
    from synth import gen_next_scale_kv, gen_queries, gen_rope_frame_k
    dev = torch.device("cuda:0")
    B = args.batch or wl.B
    off = list(wl.offsets)
    q0, ql, L_kv = wl.calls[-1]
    goff = off[:off.index(L_kv) + 1]
    H, D = wl.H, wl.D
    if wl.kind == "next_frame":
        k = gen_rope_frame_k(B, H, D, goff, 0, 1, dev, n_out_pairs=wl.n_out_k)
    else:
        k = gen_next_scale_kv(B, H, D, goff, wl.n_out_k, 0, 1, dev, shared_across_batch=True)
    v = gen_next_scale_kv(B, H, D, goff, wl.n_out_v, 0, 2, dev, shared_across_batch=False)
    q = gen_queries(B, ql, H, D, 0, 3, dev)
    G = len(goff) - 1
    pk, sk = varq.alloc_cache(B, H, D, L_kv, G, bits, device=dev)
    pv, sv = varq.alloc_cache(B, H, D, L_kv, G, bits, device=dev)
    varq.quantize_pack_kv(k, v, goff, bits, pk, sk, pv, sv)
    varq.quantize_pack_check()
    del k, v
    out = torch.empty_like(q)
    kd = torch.empty(B, H, L_kv, D, dtype=torch.bfloat16, device=dev)
    vd = torch.empty_like(kd)

    def timeit(fn):
        for _ in range(max(1, args.warmup)):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    def fused():
        varq.packed_attention(q, pk, sk, pv, sv, goff, bits, out=out)

    def unfused():
        varq.unpack_dequant(pk, sk, goff, bits, out=kd)
        varq.unpack_dequant(pv, sv, goff, bits, out=vd)
        varq.bf16_attention(q, kd, vd, out=out)

    def unpack_only():
        varq.unpack_dequant(pk, sk, goff, bits, out=kd)
        varq.unpack_dequant(pv, sv, goff, bits, out=vd)

    t_f, t_u, t_d = timeit(fused), timeit(unfused), timeit(unpack_only)
    flops = attn_flops(B, H, D, ql, L_kv)
    print(json.dumps({"fusion_report": {
        "workload": wl.name, "bits": bits, "batch": B, "heads": H, "head_dim": D, "queries": ql, "window": L_kv,
        "steps": args.steps, "fused_ms": round(t_f, 5), "unfused_ms": round(t_u, 5),
        "unfused_unpack_ms": round(t_d, 5), "fused_speedup": round(t_u / t_f, 4),
        "fused_TFLOP/s": round(flops / (t_f * 1e-3) / 1e12, 2),
        "unfused_workspace_bytes": int(2 * kd.numel() * kd.element_size())}}), flush=True)


# ---------------------------------------------------------------- main

def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the multi-GPU sharding is "
              "described in the design notes but not built.", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    import torch

    from kv_cache_quantization_02_amd import varq
    from synth import WORKLOADS, workload_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    varq.lib()                      # fail loudly if the HIP library is missing
    wl = WORKLOADS[args.workload]
    bits = args.bits or wl.bits[0]
    dev = torch.device("cuda:0")
    if args.pre_rope_report:
        pre_rope_report(varq, torch, wl, bits, args)
        return
    if args.fusion_report:
        fusion_report(varq, torch, wl, bits, args)
        return
    if args.grouping_report:
        k, _, _ = workload_inputs(wl, seed=0, device=dev, with_v=False)
        grouping_report(varq, torch, wl, bits, k, args)
        return
    k, v, q = workload_inputs(wl, seed=0, device=dev)
    off = list(wl.offsets)
    B, H, D, L, G = wl.B, wl.H, wl.D, wl.L, wl.G
    pk, sk = varq.alloc_cache(B, H, D, L, G, bits, device=dev)
    pv, sv = varq.alloc_cache(B, H, D, L, G, bits, device=dev)
    out = torch.empty_like(q)
    launches = plan(wl, bits)

    step_bytes = 0.0
    qp_b, at_b, at_f = [], [], []
    for st in launches:
        if st[0] == "qp":
            _, t0, t1, g0, g1 = st
            b1 = qp_bytes(B, t1 - t0, H, D, g1 - g0, bits)
            qp_b.append(2 * b1)                 # K and V in one launch
            step_bytes += 2 * b1
        else:
            _, q0, ql, L_kv, g1 = st
            b1 = attn_bytes(B, H, D, ql, L_kv, g1, bits)
            at_b.append(b1)
            at_f.append(attn_flops(B, H, D, ql, L_kv))
            step_bytes += b1

    def run_launch(st):
        if st[0] == "qp":
            _, t0, t1, g0, g1 = st
            rel = [o - t0 for o in off[g0:g1 + 1]]
            varq.quantize_pack_kv(k[:, t0:t1], v[:, t0:t1], rel, bits, pk, sk, pv, sv, tok_start=t0, group_start=g0)
        else:
            _, q0, ql, L_kv, g1 = st
            varq.packed_attention(q, pk, sk, pv, sv, off[:g1 + 1], bits, out=out)

    def step(kinds=("qp", "attn")):
        for st in launches:
            if (st[0] == "qp" and "qp" in kinds) or (st[0] != "qp" and "attn" in kinds):
                run_launch(st)

    def exchange_check(when):
        # a cross-work-group wait cut short by its time bound would leave wrong
        # scales and a time that looks fast: no line is printed then
        try:
            varq.quantize_pack_check()
        except varq.VarqError as e:
            print(f"bench.py: quantize+pack exchange check failed {when}: {e}", file=sys.stderr)
            sys.exit(3)

    # per-kernel times: the K steps rerun with only one kernel's launches,
    # back to back on the launch stream between two events (the attention
    # calls read the cache the step wrote; re-quantizing a block rewrites the
    # same words), once just before and once just after the timed steps: the
    # clock drifts with the board's power and temperature, and the mean of
    # the two passes brackets the timed region
    def kind_ms(kind):
        if not any((st[0] == "qp") == (kind == "qp") for st in launches):
            return 0.0
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        step((kind,))
        e0.record()
        for _ in range(args.steps):
            step((kind,))
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    for _ in range(args.warmup):            # also allocates the calls' workspaces
        step()
    torch.cuda.synchronize()
    pre = (kind_ms("qp"), kind_ms("attn"))  # the cache stays as the steps leave it
    # timed region: K steps, wall clock between two synchronizations; two HIP
    # events on the launch stream bracket the steps (none between kernels: each
    # event leaves the GPU idle for a few microseconds)
    ev_t0, ev_t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev_t0.record()
    for _ in range(args.steps):
        step()
    ev_t1.record()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms_per_step = dt * 1e3 / args.steps
    gpu_step_ms = ev_t0.elapsed_time(ev_t1) / args.steps
    exchange_check("after the timed steps")

    post = (kind_ms("qp"), kind_ms("attn"))
    qp_pass_ms = 0.5 * (pre[0] + post[0])
    at_pass_ms = 0.5 * (pre[1] + post[1])
    # the dominant kernel's time comes from the timed steps themselves: their
    # GPU time less the other kernel's (kernel-only passes just before and just
    # after them, averaged); the two then add up to the steps' GPU time
    qp_dominant = qp_pass_ms >= at_pass_ms
    if qp_dominant:
        at_step_ms = at_pass_ms
        qp_step_ms = max(gpu_step_ms - at_step_ms, 1e-6)
    else:
        qp_step_ms = qp_pass_ms
        at_step_ms = max(gpu_step_ms - qp_step_ms, 1e-6)
    exchange_check("after the per-kernel passes")
    n_qp_per_step = max(1, len(qp_b))
    n_at_per_step = max(1, len(at_b))
    qp_avg_ms = qp_step_ms / n_qp_per_step
    at_avg_ms = at_step_ms / n_at_per_step
    qp_bytes_per_launch = sum(qp_b) / n_qp_per_step
    at_bytes_per_launch = sum(at_b) / n_at_per_step
    at_flops_per_launch = sum(at_f) / n_at_per_step
    qp_gbs = qp_bytes_per_launch / (qp_avg_ms * 1e-3) / 1e9 if qp_avg_ms else 0.0
    at_gbs = at_bytes_per_launch / (at_avg_ms * 1e-3) / 1e9 if at_avg_ms else 0.0
    at_tflops = at_flops_per_launch / (at_avg_ms * 1e-3) / 1e12 if at_avg_ms else 0.0

    kernels = {
        "timing": "per kernel: kernel-only passes (the K steps rerun with only that kernel's launches, back to "
                  "back, between two HIP events) just before and just after the timed steps (step_ms_before/"
                  "after, mean step_ms_passes); the smaller kernel's step_ms is that mean, the dominant kernel's "
                  "step_ms is the timed steps' GPU time (HIP events around them, gpu_step_ms) less it; "
                  "avg_ms = step_ms / launches",
        "quant_pack": {"avg_ms": round(qp_avg_ms, 5), "step_ms": round(qp_step_ms, 5),
                       "step_ms_passes": round(qp_pass_ms, 5),
                       "step_ms_before": round(pre[0], 5), "step_ms_after": round(post[0], 5),
                       "launches_per_step": len(qp_b),
                       "alg_bytes_per_launch": int(qp_bytes_per_launch), "GB/s": round(qp_gbs, 1),
                       "hbm_frac": round(qp_gbs / HBM_PEAK_GBS, 4)},
        "packed_attention": {"avg_ms": round(at_avg_ms, 5), "step_ms": round(at_step_ms, 5),
                             "step_ms_passes": round(at_pass_ms, 5),
                             "step_ms_before": round(pre[1], 5), "step_ms_after": round(post[1], 5),
                             "launches_per_step": len(at_b),
                             "alg_bytes_per_launch": int(at_bytes_per_launch),
                             "alg_flops_per_launch": at_flops_per_launch,
                             "GB/s": round(at_gbs, 1), "hbm_frac": round(at_gbs / HBM_PEAK_GBS, 4),
                             "TFLOP/s": round(at_tflops, 2),
                             "mfma_frac": round(at_tflops / MFMA_BF16_PEAK_TFLOPS, 4)},
        "sum_step_ms": round(qp_step_ms + at_step_ms, 5),
        "gpu_step_ms": round(gpu_step_ms, 5),
    }
    copy_gbs = device_copy_rate(torch)
    if qp_dominant:
        tr = load_traffic("quant_pack.hip", wl.name, bits)
        roof = {"kernel": "quant_pack", "bound": "hbm", "achieved": round(qp_gbs, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(qp_gbs / HBM_PEAK_GBS, 4),
                "traffic": (tr["fetch_bytes"] + tr["write_bytes"]) if tr else None,
                "timing": "HIP events on the launch stream around the timed steps, less the attention calls' "
                          "kernel-only time"}
    else:
        tr = load_traffic("packed_attention.hip", wl.name, bits)
        roof = {"kernel": "packed_attention", "bound": "mfma", "achieved": round(at_tflops, 2),
                "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(at_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": (tr["fetch_bytes"] + tr["write_bytes"]) if tr else None,
                "alg_flops_per_launch": at_flops_per_launch, "launches_per_step": len(at_b),
                "timing": "HIP events on the launch stream around the timed steps, less the quantize+pack calls' "
                          "kernel-only time"}
    if tr:
        roof["traffic_source"] = tr.get("profile")
    context = {"device_copy_GBs": round(copy_gbs, 1),
               "quant_pack_frac_of_device_copy": round(qp_gbs / copy_gbs, 4) if copy_gbs else None,
               "note": "peaks are the published nominal ones; a plain device copy (read + write) reaches "
                       "device_copy_GBs on this device"}

    fused_peak = torch.cuda.max_memory_allocated()
    unfused = unfused_compare(varq, torch, wl, bits, launches, off, q, pk, sk, pv, sv, args, at_pass_ms)
    # persistent cache sizes (exact preallocation) against the bf16 cache, and
    # the dequant workspace the unfused path needs (the fused path needs none)
    pb, sb = varq.cache_bytes(B, H, D, pk.shape[3], G, bits)
    bf16_bytes = B * L * H * D * 2
    memory = {"packed_bytes_per_tensor": int(pb), "scale_bytes_per_tensor": int(sb),
              "bf16_bytes_per_tensor": int(bf16_bytes),
              "cache_fraction_of_bf16": round((pb + sb) / bf16_bytes, 5),
              "fused_dequant_workspace_bytes": 0,
              "unfused_dequant_workspace_bytes": unfused["dequant_workspace_bytes"] if unfused else None,
              "device_peak_bytes_fused_step": int(fused_peak),
              "device_peak_bytes_with_unfused": int(torch.cuda.max_memory_allocated())}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, bits, args.cpu_budget_s, step_bytes, k, v, q)

    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "description": wl.description, "bits": bits,
                   "batch": B, "heads": H, "head_dim": D, "tokens": L, "blocks": G,
                   "attention_calls": [list(c) for c in wl.calls],
                   "step_alg_bytes": int(step_bytes),
                   "hbm_frac_of_step": round(value / HBM_PEAK_GBS, 4)},
        "roofline": roof,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "context": context,
        "unfused": unfused,
        "memory": memory,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
