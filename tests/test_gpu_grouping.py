"""GPU parity of quantize+pack under the grouping variants of the project
page's Table 5 and Table 1 (varq_quantize_pack_grouped), against the oracle's
grouped_quantize_pack: words and compact scales bit-exact."""

import sys

import numpy as np
import pytest
import torch

from oracle import varq_oracle as O
from synth import WORKLOADS, workload_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda"
MODES = ("channel_block", "channel", "block", "token_head", "token", "tensor")


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def V():
    from kv_cache_quantization_02_amd import varq
    varq.lib()
    return varq


def _gpu_grouped(V, x_dev, off, bits, mode, L_cap=None):
    B, L, H, D = x_dev.shape
    W = V.words_per_row(D, bits)
    L_cap = V.round_capacity(L_cap or L)
    packed = torch.full((B, H, W, L_cap), -1, dtype=torch.int32, device=DEV)     # sentinel past L
    shape = V.grouped_scale_shape(mode, B, L, H, D, len(off) - 1)
    scales = torch.full(shape, -1.0, dtype=torch.float32, device=DEV)
    V.quantize_pack_grouped(x_dev, off, bits, mode, packed, scales)
    torch.cuda.synchronize()
    return packed.cpu().numpy().view(np.uint32), scales.cpu().numpy()


def _check(V, x_cpu, off, bits, mode, x_dev=None, L_cap=None):
    x = x_cpu.float().numpy()
    B, L, H, D = x.shape
    w_ref, s_ref = O.grouped_quantize_pack(x, mode, off, bits)
    w, s = _gpu_grouped(V, x_cpu.to(DEV) if x_dev is None else x_dev, off, bits, mode, L_cap)
    assert s.shape == s_ref.shape
    assert np.array_equal(s.view(np.uint32), s_ref.view(np.uint32)), (mode, bits, "scales")
    assert np.array_equal(w[..., :L], w_ref), (mode, bits, "words")
    assert (w[..., L:] == 0xFFFFFFFF).all(), (mode, bits, "rows past L written")


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("mode", MODES)
def test_grouped_small_all_modes_all_bits(V, mode, bits):
    # head_dim 40: five 8-channel chunks per row, so rows and groups straddle waves
    _say(f"[grouped small {mode} b{bits}]")
    g = torch.Generator().manual_seed(100 + bits)
    B, L, H, D = 2, 37, 3, 40
    x = (torch.randn(B, L, H, D, generator=g) * 2).to(torch.bfloat16)
    x[1, 9:14, 2] = 0                                   # zero groups in several modes
    _check(V, x, [0, 1, 5, 14, 30, 37], bits, mode, L_cap=45)


@pytest.mark.parametrize("D", [8, 64, 128, 256])
@pytest.mark.parametrize("mode", ["block", "token_head", "token", "tensor"])
def test_grouped_head_dims(V, mode, D):
    _say(f"[grouped D={D} {mode}]")
    g = torch.Generator().manual_seed(D)
    B, L, H = 3, 70, 5
    x = torch.randn(B, L, H, D, generator=g).to(torch.bfloat16)
    _check(V, x, [0, 4, 13, 29, 70], 4, mode)


def test_grouped_strided_input(V):
    _say("[grouped strided]")
    g = torch.Generator().manual_seed(7)
    big = torch.randn(2, 50, 6, 64, generator=g).to(torch.bfloat16)
    xs = big[:, 5:45, 1:5]                              # token and head slices: non-contiguous
    for mode in ("block", "token_head", "token", "tensor"):
        _check(V, xs.contiguous(), [0, 3, 17, 40], 8, mode, x_dev=xs.to(DEV))


def test_grouped_repeat_is_deterministic(V):
    """Scale buffers are cleared inside the call: a second call with other data
    into the same buffers gives that data's result."""
    _say("[grouped repeat]")
    g = torch.Generator().manual_seed(11)
    B, L, H, D = 2, 30, 4, 64
    off = [0, 10, 30]
    x1 = (torch.randn(B, L, H, D, generator=g) * 5).to(torch.bfloat16)
    x2 = (torch.randn(B, L, H, D, generator=g) * 0.1).to(torch.bfloat16)
    for mode in ("block", "token", "tensor"):
        W = V.words_per_row(D, 4)
        packed = torch.zeros(B, H, W, V.round_capacity(L), dtype=torch.int32, device=DEV)
        scales = torch.zeros(V.grouped_scale_shape(mode, B, L, H, D, 2), dtype=torch.float32, device=DEV)
        V.quantize_pack_grouped(x1.to(DEV), off, 4, mode, packed, scales)
        V.quantize_pack_grouped(x2.to(DEV), off, 4, mode, packed, scales)
        w_ref, s_ref = O.grouped_quantize_pack(x2.float().numpy(), mode, off, 4)
        assert np.array_equal(scales.cpu().numpy().view(np.uint32), s_ref.view(np.uint32)), mode
        assert np.array_equal(packed.cpu().numpy().view(np.uint32)[..., :L], w_ref), mode


@pytest.mark.parametrize("mode", ["block", "token_head", "token", "tensor"])
def test_grouped_var_d30_full(V, mode):
    """The VAR-d30-like K cache at full size (16 x 680 tokens x 30 heads x 64)."""
    _say(f"[grouped var_d30 full {mode}]")
    wl = WORKLOADS["var_d30"]
    k, _, _ = workload_inputs(wl, seed=0, with_v=False)
    _check(V, k, list(wl.offsets), 4, mode)
