"""Sliding-window grouped-query attention for AMD Instinct MI355X (gfx950).

The work runs in hand-written HIP kernels behind the C ABI of ``libswa.so``
(``include/swa.h``); this package is the thin Python binding over it.

    from sliding_window_gqa_swa_amd import api
    out = api.prefill(q, k, v, cu_seqlens, window=1024)
"""
from . import api  # noqa: F401
from .api import (BLOCKWISE, CAUSAL, cache_append, cache_compact, cache_roll,  # noqa: F401
                  decode, decode_step, decode_workspace, decode_workspace_bytes, prefill,
                  prefill_backward, prefill_backward_workspace_bytes, prefill_chunk,
                  prefill_lse)
