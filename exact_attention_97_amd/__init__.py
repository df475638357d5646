"""Exact fused scaled-dot-product attention for AMD MI355X (gfx950).

The compute lives in hand-written HIP kernels behind the C ABI of
``include/attn97.h`` (libattn97.so).  This package only loads that library
and marshals arguments: ``attn_fwd`` returns (O, LSE), ``attn_bwd`` returns
(dQ, dK, dV), ``attn_fwd_splitkv`` returns (O, LSE) for queries and keys of
different lengths by splitting the keys.
"""

from ._lib import (  # noqa: F401
    AttnError,
    attn_bwd,
    attn_fwd,
    attn_fwd_fp8,
    attn_fwd_fp8_quantized,
    attn_fwd_splitkv,
    bwd_workspace_bytes,
    fwd_splitkv_workspace_bytes,
    exp2_eval,
    fp8_buffer_bytes,
    fp8_buffer_views,
    fp8_quantize,
    load,
    prof_collect,
    prof_enable,
    prof_reset,
    set_variant,
    version,
)
