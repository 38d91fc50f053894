"""The benchmark's algorithmic work per step, pinned to closed-form counts.

Per workload and bit width, worked out by hand from the per-unit rules:
quantize+pack of K and V reads 2 B per element and writes 4W B per (batch,
head, token) row plus 4 B per (batch, head, block, channel) scale; attention
moves Q and O (2 B per element each), the packed K and V windows (4W B per
row) and their scales, and performs 4 Lq L_kv D flops per (batch, head).
Values in MB (1e6 B) and GFLOP, as printed to the digits below.
"""

import pytest

import bench
from synth import WORKLOADS

# workload, bits: quant-pack K+V MB over the step, last attention call MB, its GFLOP
EXPECTED = [
    ("tiny", 4, 3.6, 1.83, 0.71),
    ("var_d30", 4, 106.9, 54.8, 21.4),
    ("var_d30", 8, 127.8, 75.7, 21.4),
    ("infinity_8b", 4, 1727, 885, 5648),
    ("infinity_8b", 2, 1555, 713, 5648),
    ("self_forcing", 4, 3022, 952, 11304),
    ("longlive", 3, 1847, 352, 2392),
    ("longlive", 2, 1727, 232, 2392),
]


def _digits(x):
    s = repr(x)
    return len(s.split(".")[1]) if "." in s else 0


@pytest.mark.parametrize("name,bits,qp_mb,attn_mb,gflop", EXPECTED)
def test_step_work_matches_closed_form(name, bits, qp_mb, attn_mb, gflop):
    wl = WORKLOADS[name]
    steps = bench.plan(wl, bits)
    qp = sum(2 * bench.qp_bytes(wl.B, t1 - t0, wl.H, wl.D, g1 - g0, bits)
             for (kind, t0, t1, g0, g1) in (s for s in steps if s[0] == "qp"))
    q0, lq, l_kv = wl.calls[-1]
    g = list(wl.offsets).index(l_kv)
    ab = bench.attn_bytes(wl.B, wl.H, wl.D, lq, l_kv, g, bits)
    af = bench.attn_flops(wl.B, wl.H, wl.D, lq, l_kv)
    assert round(qp / 1e6, _digits(qp_mb)) == qp_mb
    assert round(ab / 1e6, _digits(attn_mb)) == attn_mb
    assert round(af / 1e9, _digits(gflop)) == gflop


def test_plan_covers_every_block_once():
    """The step quantizes each block exactly once, before the first call that
    reads it, and every attention window ends on a block boundary."""
    for wl in WORKLOADS.values():
        steps = bench.plan(wl, wl.bits[0])
        done = 0
        for s in steps:
            if s[0] == "qp":
                _, t0, t1, g0, g1 = s
                assert g0 == done and g1 > g0 and wl.offsets[g0] == t0 and wl.offsets[g1] == t1
                done = g1
            else:
                _, q0, lq, l_kv, g1 = s
                assert wl.offsets[g1] == l_kv and g1 <= done
        assert done == len(wl.offsets) - 1
