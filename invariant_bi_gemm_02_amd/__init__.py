"""Batch-invariant forward kernels for MI355X (gfx950): Python binding.

Thin argument marshalling over the C-ABI library ``libbi.so`` (declared in
``include/bi.h``).  Every step of the computation runs in the library's HIP
kernels; torch supplies device memory and the current stream only.  There is
no CPU or library fallback: if the HIP library is missing, every call raises.
"""
from ._lib import (  # noqa: F401
    BiError,
    load,
    version,
    gemm,
    gemm_fast,
    gemm_noalloc,
    ceiling_mfma,
    ceiling_read,
    CEILING_READ_OUT_WORDS,
    gemm_workspace_bytes,
    gemm_fast_workspace_bytes,
    rmsnorm,
    rmsnorm_fast,
    add_rmsnorm,
    paged_decode_attn,
    paged_decode_attn_fast,
    attn_workspace_bytes,
    attn_fast_workspace_bytes,
    Workspace,
    embed,
    rope_table,
    rope,
    kv_append,
    silu_mul,
    add,
    paged_prefill_attn,
    gemm_segments,
    gemm_fold,
    sample,
    verify_commit,
)
