"""varq_quantize_pack_kv_noalloc through the C ABI: the same words and scales,
bit for bit, as varq_quantize_pack_kv with a workspace, on two calls in a
row (the second smaller, reusing the fixed exchange array the first left
behind), both at INT3 with blocks that no slab kernel takes (over 1612 rows,
or a short block after a long one) so that the exchange is used; a call
needing more than the fixed array is rejected.
A call whose long blocks take the slab kernel needs no exchange and also
matches."""

import ctypes
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def V():
    from kv_cache_quantization_02_amd import varq
    varq.lib()
    return varq


def _caches(V, B, H, D, L_cap, G_cap, bits):
    W = V.words_per_row(D, bits)
    pk = torch.full((B, H, W, V.round_capacity(L_cap)), -1, dtype=torch.int32, device=DEV)
    sk = torch.full((B, H, G_cap, D), -1.0, dtype=torch.float32, device=DEV)
    return pk, sk, torch.full_like(pk, -1), torch.full_like(sk, -1.0)


def _noalloc(V, k, v, off, bits, caches, tok_start=0, group_start=0):
    """One call of the no-allocation entry point through ctypes; returns the status."""
    pk, sk, pv, sv = caches
    B, L, H, D = k.shape
    arr = (ctypes.c_int32 * len(off))(*off)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return V.lib().varq_quantize_pack_kv_noalloc(
        k.data_ptr(), k.stride(0), k.stride(1), k.stride(2), v.data_ptr(), v.stride(0), v.stride(1), v.stride(2),
        B, H, D, L, arr, len(off) - 1, bits, pk.data_ptr(), sk.data_ptr(), pv.data_ptr(), sv.data_ptr(),
        pk.shape[3], tok_start, sk.shape[2], group_start, st)


def test_noalloc_equals_workspace_entry_point(V):
    g = torch.Generator(device=DEV).manual_seed(17)
    cases = [
        # (B, L, H, D, offsets, bits, tok_start, group_start, extra rows, extra groups)
        (2, 3400, 12, 128, [0, 1700, 3400], 3, 0, 0, 0, 0),          # two 1700-row blocks: 14 chunks each
        (1, 1500, 4, 64, [0, 700, 701, 1500], 3, 24, 2, 16, 1),      # smaller, at an offset of a larger cache
    ]
    for i, (B, L, H, D, off, bits, t0, g0, xr, xg) in enumerate(cases):
        _say(f"[noalloc call {i}: B={B} L={L} H={H} D={D} bits={bits}]")
        k = (torch.randn(B, L, H, D, generator=g, device=DEV) * 3).to(torch.bfloat16)
        v = torch.randn(B, L, H, D, generator=g, device=DEV).to(torch.bfloat16)
        G = len(off) - 1
        ref = _caches(V, B, H, D, t0 + L + xr, g0 + G + xg, bits)
        V.quantize_pack_kv(k, v, off, bits, *ref, tok_start=t0, group_start=g0)
        V.quantize_pack_check()
        got = _caches(V, B, H, D, t0 + L + xr, g0 + G + xg, bits)
        assert V.quantize_pack_workspace_bytes(B, H, D, off, bits, 2) > 0      # the exchange is used
        r = _noalloc(V, k, v, off, bits, got, t0, g0)
        assert r == 0, V.last_error()
        assert V.lib().varq_quantize_pack_check(None, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)) == 0
        torch.cuda.synchronize()
        for a, b in zip(got, ref):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32)), i


def test_noalloc_slab_calls_match(V):
    """INT4 next-frame block: the slab kernel, no scratch at all."""
    g = torch.Generator(device=DEV).manual_seed(23)
    B, L, H, D, off, bits = 2, 4680, 4, 128, [0, 1560, 3120, 4680], 4
    k = (torch.randn(B, L, H, D, generator=g, device=DEV) * 3).to(torch.bfloat16)
    v = torch.randn(B, L, H, D, generator=g, device=DEV).to(torch.bfloat16)
    assert V.quantize_pack_workspace_bytes(B, H, D, off, bits, 2) == 0
    ref = _caches(V, B, H, D, L, 3, bits)
    V.quantize_pack_kv(k, v, off, bits, *ref)
    got = _caches(V, B, H, D, L, 3, bits)
    assert _noalloc(V, k, v, off, bits, got) == 0, V.last_error()
    torch.cuda.synchronize()
    for a, b in zip(got, ref):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_noalloc_rejects_calls_beyond_the_fixed_array(V):
    """Infinity-8B-like K+V over all 13 scales at INT3 needs ~45 MB of exchange
    state: rejected with VARQ_EWORKSPACE before anything is launched (outputs
    untouched)."""
    from synth import WORKLOADS
    wl = WORKLOADS["infinity_8b"]
    B, H, D, bits = wl.B, wl.H, wl.D, 3
    off = list(wl.offsets)
    assert V.quantize_pack_workspace_bytes(B, H, D, off, bits, 2) > 16 << 20
    k = torch.zeros(B, wl.L, H, D, dtype=torch.bfloat16, device=DEV)
    caches = _caches(V, B, H, D, wl.L, wl.G, bits)
    r = _noalloc(V, k, k.clone(), off, bits, caches)
    assert r == -7 and "fixed" in V.last_error()
    torch.cuda.synchronize()
    assert bool((caches[0] == -1).all()) and bool((caches[1] == -1.0).all())
