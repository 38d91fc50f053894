"""Thin ctypes binding of libvarq.so (include/varq.h).

Each function marshals torch tensors into the C ABI's pointers, strides and
stream and calls the entry point of the same name (without the ``varq_``
prefix). All computation happens in the gfx950 kernels; if the library is not
built, every call raises. PyTorch supplies device memory and streams only:
the workspaces that some calls need are torch tensors, sized by the library's
workspace queries and kept here per (device, stream) unless the caller passes
one.
"""

from __future__ import annotations

import ctypes
import math
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libvarq.so")

VARQ_OK = 0
STATUS_NAMES = {0: "VARQ_OK", -1: "VARQ_EINVAL", -2: "VARQ_EBITS", -3: "VARQ_EALIGN",
                -4: "VARQ_ECAPACITY", -5: "VARQ_ELAUNCH", -6: "VARQ_EUNSUPPORTED", -7: "VARQ_EWORKSPACE"}
MAX_GROUPS = 256

_lib = None

_i32 = ctypes.c_int
_i64 = ctypes.c_int64
_vp = ctypes.c_void_p
_f32 = ctypes.c_float
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)

_SIGNATURES = {
    "varq_codes_per_word": (_i32, [_i32]),
    "varq_words_per_row": (_i32, [_i32, _i32]),
    "varq_cache_bytes": (_i32, [_i32, _i32, _i32, _i64, _i64, _i32, _i64p, _i64p]),
    "varq_quantize_pack": (_i32, [_vp, _i64, _i64, _i64, _i32, _i32, _i32, _i64, _i32p, _i32, _i32,
                                  _vp, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _vp]),
    "varq_quantize_pack_workspace": (_i32, [_i32, _i32, _i32, _i64, _i32p, _i32, _i32, _i32, _i64p]),
    "varq_quantize_pack_kv": (_i32, [_vp, _i64, _i64, _i64, _vp, _i64, _i64, _i64, _i32, _i32, _i32, _i64,
                                     _i32p, _i32, _i32, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64,
                                     _vp, _i64, _vp]),
    "varq_quantize_pack_kv_noalloc": (_i32, [_vp, _i64, _i64, _i64, _vp, _i64, _i64, _i64, _i32, _i32, _i32, _i64,
                                             _i32p, _i32, _i32, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _vp]),
    "varq_packed_attention": (_i32, [_vp, _i64, _i64, _i64, _i32, _i32, _i32, _i64,
                                     _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32p, _i32, _i32,
                                     _f32, _vp, _i64, _i64, _i64, _vp, _i64, _vp]),
    "varq_packed_attention_workspace": (_i32, [_i32, _i32, _i32, _i64, _i64, _i64p]),
    "varq_unpack_dequant": (_i32, [_vp, _vp, _i32, _i32, _i32, _i64, _i64, _i64, _i32p, _i32, _i32,
                                   _vp, _vp]),
    "varq_bf16_attention": (_i32, [_vp, _i64, _i64, _i64, _i32, _i32, _i32, _i64, _vp, _vp, _i64, _i64,
                                   _f32, _vp, _i64, _i64, _i64, _vp, _i64, _vp]),
    "varq_unpack_dequant_rope": (_i32, [_vp, _vp, _i32, _i32, _i32, _i64, _i64, _i64, _i32p, _i32, _i32,
                                        _vp, _vp, _vp, _vp]),
    "varq_packed_attention_rope": (_i32, [_vp, _i64, _i64, _i64, _i32, _i32, _i32, _i64,
                                          _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32p, _i32, _i32,
                                          _f32, _vp, _i64, _i64, _i64, _vp, _vp, _vp, _i64, _vp]),
    "varq_grouped_scale_count": (_i64, [_i32, _i32, _i64, _i32, _i32, _i32]),
    "varq_quantize_pack_grouped": (_i32, [_vp, _i64, _i64, _i64, _i32, _i32, _i32, _i64, _i32, _i32p, _i32,
                                          _i32, _vp, _i64, _vp, _i64, _vp, _i64, _vp]),
    "varq_quantize_pack_check": (_i32, [_vp, _vp]),
    "varq_last_error": (ctypes.c_char_p, []),
    "varq_version": (ctypes.c_char_p, []),
}


class VarqError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def lib():
    """The loaded libvarq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib = h
    return _lib


def _check(status):
    if status != VARQ_OK:
        raise VarqError(status, lib().varq_last_error().decode())


def _offsets(group_offsets):
    off = [int(o) for o in group_offsets]
    arr = (ctypes.c_int32 * len(off))(*off)
    return arr, len(off) - 1


def _stream(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, dtype, name):
    if not isinstance(t, torch.Tensor) or t.dtype != dtype or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA {dtype} tensor")


# Workspaces kept per (device, stream, kind): "qp" (quantize+pack exchange;
# zero-filled when allocated, then left to the library, which keeps it valid
# from call to call) and "attn" (attention partials; contents irrelevant).
_WS = {}


def _stream_obj(stream, device):
    return torch.cuda.current_stream(device) if stream is None else stream


def get_workspace(kind, nbytes, device, stream=None):
    """A cached workspace tensor of at least nbytes for calls of `kind` on
    `stream` (default: the device's current stream), or None if nbytes is 0.
    Growing allocates a new zero-filled tensor on that stream."""
    if nbytes <= 0:
        return None
    device = torch.device(device)
    if device.index is None:
        device = torch.device("cuda", torch.cuda.current_device())
    st = _stream_obj(stream, device)
    key = (device.index, st.cuda_stream, kind)
    ws = _WS.get(key)
    if ws is None or ws.numel() < nbytes:
        with torch.cuda.stream(st):
            ws = torch.zeros(int(nbytes), dtype=torch.uint8, device=device)
        _WS[key] = ws
    return ws


def _ws_args(ws):
    """(pointer, bytes) of a workspace tensor or None."""
    if ws is None:
        return None, 0
    if not isinstance(ws, torch.Tensor) or not ws.is_cuda or not ws.is_contiguous():
        raise TypeError("workspace must be a contiguous CUDA tensor")
    return ws.data_ptr(), ws.numel() * ws.element_size()


def quantize_pack_workspace_bytes(B, H, D, group_offsets, bits, n_tensors=1):
    """Workspace bytes of a quantize+pack call (0 when every block fits one work-group)."""
    off, G = _offsets(group_offsets)
    n = ctypes.c_int64()
    _check(lib().varq_quantize_pack_workspace(B, H, D, int(group_offsets[-1]), off, G, bits, n_tensors,
                                              ctypes.byref(n)))
    return n.value


def attention_workspace_bytes(B, H, D, Lq, L_kv):
    """Workspace bytes of a packed (or bf16) attention call on the current device."""
    n = ctypes.c_int64()
    _check(lib().varq_packed_attention_workspace(B, H, D, Lq, L_kv, ctypes.byref(n)))
    return n.value


def last_error() -> str:
    return lib().varq_last_error().decode()


def version() -> str:
    return lib().varq_version().decode()


def codes_per_word(bits: int) -> int:
    return lib().varq_codes_per_word(bits)


def words_per_row(head_dim: int, bits: int) -> int:
    return lib().varq_words_per_row(head_dim, bits)


def cache_bytes(B, H, head_dim, L_cap, G_cap, bits):
    """(packed_bytes, scale_bytes) of one packed tensor and its scales."""
    p, s = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().varq_cache_bytes(B, H, head_dim, L_cap, G_cap, bits, ctypes.byref(p), ctypes.byref(s)))
    return p.value, s.value


def round_capacity(L):
    """Token capacity accepted by the library: L rounded up to a multiple of 8."""
    return (int(L) + 7) // 8 * 8


def alloc_cache(B, H, head_dim, L_cap, G_cap, bits, device="cuda"):
    """Preallocate one packed tensor [B, H, W, L_cap] (int32) and its scales
    [B, H, G_cap, D] (fp32) with the exact sizes of cache_bytes()."""
    L_cap = round_capacity(L_cap)
    pb, sb = cache_bytes(B, H, head_dim, L_cap, G_cap, bits)
    W = words_per_row(head_dim, bits)
    packed = torch.zeros(B, H, W, L_cap, dtype=torch.int32, device=device)
    scales = torch.zeros(B, H, G_cap, head_dim, dtype=torch.float32, device=device)
    assert packed.numel() * 4 == pb and scales.numel() * 4 == sb
    return packed, scales


def quantize_pack(x, group_offsets, bits, packed, scales, tok_start=0, group_start=0, stream=None,
                  workspace=None):
    """x bf16 [B, L_in, H, D] (channel stride 1) -> rows [tok_start, tok_start+L_in)
    of `packed` [B, H, W, L_cap] and slots [group_start, group_start+G_in) of
    `scales` [B, H, G_cap, D]. `workspace`: a zero-filled (once) uint8 tensor
    of at least quantize_pack_workspace_bytes(); default: the stream's cached one."""
    _need(x, torch.bfloat16, "x")
    _need(packed, torch.int32, "packed")
    _need(scales, torch.float32, "scales")
    if x.dim() != 4 or x.stride(3) != 1:
        raise ValueError("x must be [B, L, H, D] with channel stride 1")
    if not packed.is_contiguous() or not scales.is_contiguous():
        raise ValueError("packed and scales must be contiguous")
    B, L, H, D = x.shape
    off, G = _offsets(group_offsets)
    if workspace is None and L > 0:
        workspace = get_workspace("qp", quantize_pack_workspace_bytes(B, H, D, group_offsets, bits, 1),
                                           x.device, stream)
    wp, wb = _ws_args(workspace)
    _check(lib().varq_quantize_pack(
        x.data_ptr(), x.stride(0), x.stride(1), x.stride(2), B, H, D, L, off, G, bits,
        packed.data_ptr(), packed.shape[3], tok_start, scales.data_ptr(), scales.shape[2],
        group_start, wp, wb, _stream(stream, x.device)))
    return packed, scales


def quantize_pack_kv(k, v, group_offsets, bits, packed_k, scales_k, packed_v, scales_v,
                     tok_start=0, group_start=0, stream=None, workspace=None):
    """quantize_pack of k and of v (same shape and block map, each bf16
    [B, L_in, H, D] with its own strides) into their own caches, in one launch."""
    for t, n in ((k, "k"), (v, "v")):
        _need(t, torch.bfloat16, n)
        if t.dim() != 4 or t.stride(3) != 1:
            raise ValueError(f"{n} must be [B, L, H, D] with channel stride 1")
    if k.shape != v.shape:
        raise ValueError("k and v must have one shape")
    for t, dt, n in ((packed_k, torch.int32, "packed_k"), (packed_v, torch.int32, "packed_v"),
                     (scales_k, torch.float32, "scales_k"), (scales_v, torch.float32, "scales_v")):
        _need(t, dt, n)
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
    if packed_k.shape != packed_v.shape or scales_k.shape != scales_v.shape:
        raise ValueError("K and V caches must have one layout")
    B, L, H, D = k.shape
    off, G = _offsets(group_offsets)
    if workspace is None and L > 0:
        workspace = get_workspace("qp", quantize_pack_workspace_bytes(B, H, D, group_offsets, bits, 2),
                                           k.device, stream)
    wp, wb = _ws_args(workspace)
    _check(lib().varq_quantize_pack_kv(
        k.data_ptr(), k.stride(0), k.stride(1), k.stride(2), v.data_ptr(), v.stride(0), v.stride(1), v.stride(2),
        B, H, D, L, off, G, bits, packed_k.data_ptr(), scales_k.data_ptr(), packed_v.data_ptr(), scales_v.data_ptr(),
        packed_k.shape[3], tok_start, scales_k.shape[2], group_start, wp, wb, _stream(stream, k.device)))
    return packed_k, scales_k, packed_v, scales_v


def quantize_pack_kv_noalloc(k, v, group_offsets, bits, packed_k, scales_k, packed_v, scales_v,
                             tok_start=0, group_start=0, stream=None):
    """quantize_pack_kv without a workspace: the library's fixed per-device
    exchange array (at most 16 MiB of exchange state) stands in for it, and
    nothing is allocated by the call."""
    for t, n in ((k, "k"), (v, "v")):
        _need(t, torch.bfloat16, n)
        if t.dim() != 4 or t.stride(3) != 1:
            raise ValueError(f"{n} must be [B, L, H, D] with channel stride 1")
    if k.shape != v.shape:
        raise ValueError("k and v must have one shape")
    for t, dt, n in ((packed_k, torch.int32, "packed_k"), (packed_v, torch.int32, "packed_v"),
                     (scales_k, torch.float32, "scales_k"), (scales_v, torch.float32, "scales_v")):
        _need(t, dt, n)
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
    if packed_k.shape != packed_v.shape or scales_k.shape != scales_v.shape:
        raise ValueError("K and V caches must have one layout")
    B, L, H, D = k.shape
    off, G = _offsets(group_offsets)
    _check(lib().varq_quantize_pack_kv_noalloc(
        k.data_ptr(), k.stride(0), k.stride(1), k.stride(2), v.data_ptr(), v.stride(0), v.stride(1), v.stride(2),
        B, H, D, L, off, G, bits, packed_k.data_ptr(), scales_k.data_ptr(), packed_v.data_ptr(), scales_v.data_ptr(),
        packed_k.shape[3], tok_start, scales_k.shape[2], group_start, _stream(stream, k.device)))
    return packed_k, scales_k, packed_v, scales_v


def quantize_pack_check(device=None, stream=None, workspace=None):
    """Raise VarqError if a quantize+pack call that used `workspace` (default:
    the cached workspace of the stream, itself defaulting to the current stream
    of `device`) since the previous check ended a cross-work-group wait by its
    time bound; synchronizes that stream."""
    dev = torch.device("cuda") if device is None else torch.device(device)
    if dev.index is None:
        dev = torch.device("cuda", torch.cuda.current_device())
    if workspace is None:
        workspace = _WS.get((dev.index, _stream_obj(stream, dev).cuda_stream, "qp"))
    wp, _ = _ws_args(workspace)
    _check(lib().varq_quantize_pack_check(wp, _stream(stream, dev)))


def frame_group_offsets(L, group_tokens, phase=0):
    """Block boundaries for a next-frame cache of L tokens in groups of
    `group_tokens` (project page: 1560-token frame groups; a compression ratio
    of 3 makes the whole 4680-token chunk one group). phase > 0 shifts every
    interior boundary by `phase` tokens (Table 6's misaligned placement uses
    half a group), which leaves a shorter group at each end."""
    L, g, phase = int(L), int(group_tokens), int(phase)
    if L < 1 or g < 1 or not 0 <= phase < g:
        raise ValueError("need L >= 1, group_tokens >= 1 and 0 <= phase < group_tokens")
    inner = list(range(phase if phase else g, L, g))
    return [0] + [b for b in inner if 0 < b < L] + [L]


# Scale groupings of the project page's Table 5 / Table 1 (include/varq.h VARQ_GROUP_*)
GROUPINGS = {"channel_block": 0, "channel": 1, "block": 2, "token_head": 3, "token": 4, "tensor": 5}


def grouped_scale_shape(mode, B, L, H, D, G):
    """Compact scale layout of a grouping (one fp32 per group)."""
    return {"channel_block": (B, H, G, D), "channel": (B, H, D), "block": (B, G),
            "token_head": (B, H, L), "token": (B, L), "tensor": (1,)}[mode]


def grouped_scale_count(mode, B, L, H, D, G):
    return lib().varq_grouped_scale_count(GROUPINGS[mode], B, L, H, D, G)


def quantize_pack_grouped(x, group_offsets, bits, mode, packed, scales, stream=None, workspace=None):
    """x bf16 [B, L, H, D] -> rows [0, L) of `packed` [B, H, W, L_cap] and the
    compact scales of grouping `mode` (a contiguous fp32 tensor of at least
    grouped_scale_count(...) elements)."""
    _need(x, torch.bfloat16, "x")
    _need(packed, torch.int32, "packed")
    _need(scales, torch.float32, "scales")
    if x.dim() != 4 or x.stride(3) != 1:
        raise ValueError("x must be [B, L, H, D] with channel stride 1")
    if not packed.is_contiguous() or not scales.is_contiguous():
        raise ValueError("packed and scales must be contiguous")
    B, L, H, D = x.shape
    off, G = _offsets(group_offsets)
    if workspace is None and mode in ("channel_block", "channel"):
        table = list(group_offsets) if mode == "channel_block" else [0, L]
        workspace = get_workspace("qp", quantize_pack_workspace_bytes(B, H, D, table, bits, 1),
                                           x.device, stream)
    wp, wb = _ws_args(workspace)
    _check(lib().varq_quantize_pack_grouped(
        x.data_ptr(), x.stride(0), x.stride(1), x.stride(2), B, H, D, L, GROUPINGS[mode], off, G, bits,
        packed.data_ptr(), packed.shape[3], scales.data_ptr(), scales.numel(), wp, wb, _stream(stream, x.device)))
    return packed, scales


def _attn_ws(workspace, B, H, D, Lq, L_kv, device, stream):
    if workspace is None:
        workspace = get_workspace("attn", attention_workspace_bytes(B, H, D, Lq, L_kv), device, stream)
    return _ws_args(workspace)


def packed_attention(q, packed_k, scales_k, packed_v, scales_v, group_offsets, bits,
                     softmax_scale=None, out=None, stream=None, workspace=None):
    """q bf16 [B, Lq, H, D] attends to cache tokens [0, group_offsets[-1]) ->
    out bf16 [B, Lq, H, D]."""
    _need(q, torch.bfloat16, "q")
    for t, n in ((packed_k, "packed_k"), (packed_v, "packed_v")):
        _need(t, torch.int32, n)
    for t, n in ((scales_k, "scales_k"), (scales_v, "scales_v")):
        _need(t, torch.float32, n)
    if q.dim() != 4 or q.stride(3) != 1:
        raise ValueError("q must be [B, Lq, H, D] with channel stride 1")
    for t in (packed_k, packed_v, scales_k, scales_v):
        if not t.is_contiguous():
            raise ValueError("packed caches and scales must be contiguous")
    if packed_k.shape != packed_v.shape or scales_k.shape != scales_v.shape:
        raise ValueError("K and V caches must have the same geometry")
    B, Lq, H, D = q.shape
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    softmax_scale = float(np.float32(softmax_scale))      # the fp32 value the kernel uses
    if out is None:
        out = torch.empty(B, Lq, H, D, dtype=torch.bfloat16, device=q.device)
    _need(out, torch.bfloat16, "out")
    if out.stride(3) != 1:
        raise ValueError("out must have channel stride 1")
    off, G = _offsets(group_offsets)
    L_kv = int(group_offsets[-1])
    wp, wb = _attn_ws(workspace, B, H, D, Lq, L_kv, q.device, stream)
    _check(lib().varq_packed_attention(
        q.data_ptr(), q.stride(0), q.stride(1), q.stride(2), B, H, D, Lq,
        packed_k.data_ptr(), scales_k.data_ptr(), packed_v.data_ptr(), scales_v.data_ptr(),
        packed_k.shape[3], scales_k.shape[2], L_kv, off, G, bits, softmax_scale,
        out.data_ptr(), out.stride(0), out.stride(1), out.stride(2), wp, wb, _stream(stream, q.device)))
    return out


def _rope_tables(rope_cos, rope_sin, rows, D):
    for t, n in ((rope_cos, "rope_cos"), (rope_sin, "rope_sin")):
        _need(t, torch.float32, n)
        if not t.is_contiguous() or t.dim() != 2 or t.shape[1] != D // 2 or t.shape[0] < rows:
            raise ValueError(f"{n} must be a contiguous fp32 [>= {rows}, {D // 2}] table")


def packed_attention_rope(q, packed_k, scales_k, packed_v, scales_v, group_offsets, bits, rope_cos, rope_sin,
                          softmax_scale=None, out=None, stream=None, workspace=None):
    """packed_attention over a cache whose K was quantized before RoPE: each
    dequantized K row t is rotated by rope_cos/rope_sin[t] (fp32 [>= L_kv, D/2])
    before the scores; q is already rotated."""
    _need(q, torch.bfloat16, "q")
    for t, n in ((packed_k, "packed_k"), (packed_v, "packed_v")):
        _need(t, torch.int32, n)
    for t, n in ((scales_k, "scales_k"), (scales_v, "scales_v")):
        _need(t, torch.float32, n)
    if q.dim() != 4 or q.stride(3) != 1:
        raise ValueError("q must be [B, Lq, H, D] with channel stride 1")
    for t in (packed_k, packed_v, scales_k, scales_v):
        if not t.is_contiguous():
            raise ValueError("packed caches and scales must be contiguous")
    if packed_k.shape != packed_v.shape or scales_k.shape != scales_v.shape:
        raise ValueError("K and V caches must have the same geometry")
    B, Lq, H, D = q.shape
    L_kv = int(group_offsets[-1])
    _rope_tables(rope_cos, rope_sin, L_kv, D)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    softmax_scale = float(np.float32(softmax_scale))
    if out is None:
        out = torch.empty(B, Lq, H, D, dtype=torch.bfloat16, device=q.device)
    _need(out, torch.bfloat16, "out")
    if out.stride(3) != 1:
        raise ValueError("out must have channel stride 1")
    off, G = _offsets(group_offsets)
    wp, wb = _attn_ws(workspace, B, H, D, Lq, L_kv, q.device, stream)
    _check(lib().varq_packed_attention_rope(
        q.data_ptr(), q.stride(0), q.stride(1), q.stride(2), B, H, D, Lq,
        packed_k.data_ptr(), scales_k.data_ptr(), packed_v.data_ptr(), scales_v.data_ptr(),
        packed_k.shape[3], scales_k.shape[2], L_kv, off, G, bits, softmax_scale,
        out.data_ptr(), out.stride(0), out.stride(1), out.stride(2),
        rope_cos.data_ptr(), rope_sin.data_ptr(), wp, wb, _stream(stream, q.device)))
    return out


def unpack_dequant_rope(packed, scales, group_offsets, bits, rope_cos, rope_sin, out=None, stream=None):
    """unpack_dequant followed by the pairwise rotation of each row t by
    rope_cos/rope_sin[t] (fp32 [>= L, D/2]): the dense post-RoPE K of a cache
    quantized before RoPE."""
    _need(packed, torch.int32, "packed")
    _need(scales, torch.float32, "scales")
    if not packed.is_contiguous() or not scales.is_contiguous():
        raise ValueError("packed and scales must be contiguous")
    B, H, _, L_cap = packed.shape
    D = scales.shape[3]
    L = int(group_offsets[-1])
    _rope_tables(rope_cos, rope_sin, L, D)
    if out is None:
        out = torch.empty(B, H, L, D, dtype=torch.bfloat16, device=packed.device)
    _need(out, torch.bfloat16, "out")
    if not out.is_contiguous():
        raise ValueError("out must be contiguous")
    off, G = _offsets(group_offsets)
    _check(lib().varq_unpack_dequant_rope(
        packed.data_ptr(), scales.data_ptr(), B, H, D, L_cap, scales.shape[2], L, off, G, bits,
        rope_cos.data_ptr(), rope_sin.data_ptr(), out.data_ptr(), _stream(stream, packed.device)))
    return out


def bf16_attention(q, k, v, L_kv=None, softmax_scale=None, out=None, stream=None, workspace=None):
    """Unfused baseline: q bf16 [B, Lq, H, D] attends to dense bf16 k, v
    [B, H, L_rows, D] (e.g. unpack_dequant's output) over rows [0, L_kv) ->
    out bf16 [B, Lq, H, D]."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, torch.bfloat16, n)
    if q.dim() != 4 or q.stride(3) != 1:
        raise ValueError("q must be [B, Lq, H, D] with channel stride 1")
    if not k.is_contiguous() or not v.is_contiguous() or k.shape != v.shape:
        raise ValueError("k and v must be contiguous [B, H, L_rows, D] of one shape")
    B, Lq, H, D = q.shape
    L_rows = k.shape[2]
    L_kv = L_rows if L_kv is None else int(L_kv)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    softmax_scale = float(np.float32(softmax_scale))
    if out is None:
        out = torch.empty(B, Lq, H, D, dtype=torch.bfloat16, device=q.device)
    _need(out, torch.bfloat16, "out")
    if out.stride(3) != 1:
        raise ValueError("out must have channel stride 1")
    wp, wb = _attn_ws(workspace, B, H, D, Lq, L_kv, q.device, stream)
    _check(lib().varq_bf16_attention(
        q.data_ptr(), q.stride(0), q.stride(1), q.stride(2), B, H, D, Lq,
        k.data_ptr(), v.data_ptr(), L_rows, L_kv, softmax_scale,
        out.data_ptr(), out.stride(0), out.stride(1), out.stride(2), wp, wb, _stream(stream, q.device)))
    return out


def unpack_dequant(packed, scales, group_offsets, bits, out=None, stream=None):
    """Dense bf16 [B, H, L, D] view of cache tokens [0, group_offsets[-1])."""
    _need(packed, torch.int32, "packed")
    _need(scales, torch.float32, "scales")
    if not packed.is_contiguous() or not scales.is_contiguous():
        raise ValueError("packed and scales must be contiguous")
    B, H, _, L_cap = packed.shape
    D = scales.shape[3]
    L = int(group_offsets[-1])
    if out is None:
        out = torch.empty(B, H, L, D, dtype=torch.bfloat16, device=packed.device)
    _need(out, torch.bfloat16, "out")
    if not out.is_contiguous():
        raise ValueError("out must be contiguous")
    off, G = _offsets(group_offsets)
    _check(lib().varq_unpack_dequant(
        packed.data_ptr(), scales.data_ptr(), B, H, D, L_cap, scales.shape[2], L, off, G, bits,
        out.data_ptr(), _stream(stream, packed.device)))
    return out
