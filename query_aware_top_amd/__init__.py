"""Query-aware selective sparse attention (ESA and MoBA) for AMD MI355X.

Thin Python binding of the C ABI in include/qat.h (libqat.so, built from
query_aware_top_amd/csrc with hipcc for gfx950). The functions here only
marshal arguments: they check device, dtype and contiguity of torch tensors,
allocate outputs and the workspace with torch, and pass raw device pointers
and the current HIP stream to the library. Every step of the computation
runs in the library's HIP kernels; there is no fallback.
"""
from ._binding import (  # noqa: F401
    QatError,
    EsaParams,
    MobaParams,
    lib,
    lib_path,
    plan,
    abi_version,
    esa_params,
    moba_params,
    esa_workspace_size,
    esa_compress,
    esa_select,
    esa_select_heads,
    esa_sparse_attn,
    esa_bwd_workspace_size,
    esa_sparse_attn_bwd,
    moba_workspace_size,
    moba_block_select,
    moba_sparse_attn,
    moba_block_means,
    moba_decode_select,
    moba_decode_attn,
    moba_decode_attn_noalloc,
    moba_bwd_workspace_size,
    moba_sparse_attn_bwd,
    CcaParams,
    cca_params,
    cca_pool,
    cca_attn,
    EXPORTED_SYMBOLS,
    timing_enable,
    timing_select,
    timing_reset,
    timing_query,
)
