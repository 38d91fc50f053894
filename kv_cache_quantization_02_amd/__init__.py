"""MI355X (gfx950) implementation of VAR-Q's packed KV-cache hot path.

The compute lives in libvarq.so (C ABI in include/varq.h): quantize+pack,
unpack+dequant and packed-KV attention as hand-written HIP kernels, plus a
plain bf16 attention over dense K/V for the unfused comparison. The module
`varq` is a thin ctypes binding over it.
"""

from . import varq  # noqa: F401
from .varq import (  # noqa: F401
    GROUPINGS,
    VarqError,
    alloc_cache,
    bf16_attention,
    cache_bytes,
    codes_per_word,
    frame_group_offsets,
    grouped_scale_count,
    grouped_scale_shape,
    packed_attention,
    packed_attention_rope,
    quantize_pack,
    quantize_pack_check,
    quantize_pack_grouped,
    quantize_pack_kv,
    unpack_dequant,
    unpack_dequant_rope,
    words_per_row,
)
