"""Fused exact attention forward for MI355X (gfx950).

A thin ctypes binding over ``lib/libattn_fwd.so``, whose C ABI is declared in
``include/attn_fwd.h``.  The Python side only marshals arguments: every step
of the computation runs in the HIP kernels.  PyTorch is used for device memory
and streams.  There is no fallback: if the library is missing, every entry
point raises.

Entry points (same names as the C ABI): ``attn_fwd``, ``attn_fwd_ex``,
``attn_fwd_validate``, ``attn_fwd_plan``, ``attn_fwd_plan_ex``,
``attn_fwd_num_configs``, ``attn_fwd_config_desc``, ``attn_status_str``; and
the pages' convenience form ``flash_attn_forward(q, k, v, causal=True)``
("Lab 02 - Forward de flash attention en Triton", "Bloque A"), which also
returns the per-row log-sum-exp.

Split-KV ("Optimizaciones de Atencion", section "FlashDecoding"):
``attn_fwd_splitkv``, ``attn_fwd_splitkv_ex``, ``attn_fwd_splitkv_validate``,
``attn_fwd_splitkv_plan``, ``attn_fwd_splitkv_workspace_size`` and the
convenience ``flash_attn_forward_splitkv(q, k, v, causal=True)`` for Nq
queries against Nk keys (decoding); ``attn_fwd_splitkv_noalloc`` is the same
call with its partials in a fixed per-device array of the library, for
callers that cannot allocate.

Paged K/V ("00 - Por que la atencion domina la inferencia", section
"PagedAttention es un problema distinto"): ``attn_fwd_paged``,
``attn_fwd_paged_ex``, ``attn_fwd_paged_validate``, ``attn_fwd_paged_plan``,
``attn_fwd_paged_workspace_size`` and ``flash_attn_forward_paged``.

Backward (``include/attn_bwd.h``): ``attn_bwd``, ``attn_bwd_validate``,
``attn_bwd_workspace_size`` and ``flash_attn_backward(q, k, v, o, lse, dout)``,
the gradients of sum(dout * o) computed from the forward's log-sum-exp with
the scores recomputed tile by tile.
"""
from ._binding import (  # noqa: F401
    ATTN_BF16,
    ATTN_F16,
    ATTN_NOALLOC_SCRATCH_BYTES,
    STATUS,
    AttnError,
    attn_bwd,
    attn_bwd_validate,
    attn_bwd_workspace_size,
    attn_fwd,
    attn_fwd_autotune,
    attn_fwd_config_desc,
    attn_fwd_ex,
    attn_fwd_num_configs,
    attn_fwd_paged,
    attn_fwd_paged_ex,
    attn_fwd_paged_plan,
    attn_fwd_paged_validate,
    attn_fwd_paged_workspace_size,
    attn_fwd_plan,
    attn_fwd_plan_ex,
    attn_fwd_splitkv,
    attn_fwd_splitkv_ex,
    attn_fwd_splitkv_noalloc,
    attn_fwd_splitkv_plan,
    attn_fwd_splitkv_validate,
    attn_fwd_splitkv_workspace_size,
    attn_fwd_validate,
    attn_status_str,
    flash_attn_backward,
    flash_attn_forward,
    flash_attn_forward_paged,
    flash_attn_forward_splitkv,
    library_path,
    load_library,
    tuned_configs,
)
