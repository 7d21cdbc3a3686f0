"""MI355X (gfx950) Multi-Head Latent Attention: absorbed decode over a latent
KV cache, the cache-row producer (latent and rotated RoPE key), causal
prefill in naive and absorbed form, and the output projection (with W_UV
folded in or not), as hand-written HIP kernels behind a C ABI
(include/mla.h).  This package is the thin Python binding over that library.
"""
from .binding import (  # noqa: F401
    EXPORTS,
    MLA_BF16,
    MLA_ERR_HIP,
    MLA_ERR_INVALID_ARG,
    MLA_ERR_UNSUPPORTED,
    MLA_ERR_WORKSPACE,
    MLA_F32,
    MLA_OK,
    NOALLOC_MAX_BYTES,
    AppendParams,
    DecodeParams,
    MLAError,
    PrefillParams,
    ProjParams,
    absorb_q,
    cache_append,
    decode,
    decode_latent,
    decode_noalloc,
    decode_num_splits,
    decode_params,
    decode_workspace_bytes,
    fold_value_output,
    kv_cache_bytes,
    output_proj,
    output_proj_workspace_bytes,
    prefill_absorbed,
    prefill_absorbed_num_splits,
    prefill_absorbed_workspace_bytes,
    prefill_naive,
    prefill_params,
    proj_params,
    prefill_workspace_bytes,
    status_string,
    version,
)
