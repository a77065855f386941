"""Absorbed Multi-Head Latent Attention decode for MI355X (gfx950).

A thin ctypes binding over ``libmla_absorbed.so``.  The functions carry the
names of the C ABI in ``include/mla_absorbed.h`` and only marshal arguments:
every step of the decode runs in the library's HIP kernels.  Tensors are
passed as torch tensors (their device pointers are used) or raw integer
device addresses; PyTorch serves only for device memory and streams.
"""
from .binding import (  # noqa: F401
    MLA_OK,
    MLA_ERR_INVALID_ARG,
    MLA_ERR_UNSUPPORTED,
    MLA_ERR_HIP,
    MLA_BF16,
    MLA_FP8_E4M3,
    MLA_FP16,
    MLA_FP32,
    MLA_TILE_TOKENS,
    MlaError,
    MlaShape,
    library,
    library_path,
    exported_symbols,
    mla_absorb_q,
    mla_decode_num_parts,
    mla_decode_paged,
    mla_combine_lse,
    mla_up_v,
    mla_combine_up_v,
    mla_append_kv,
    mla_append_kv_workspace_bytes,
    mla_append_kv_noalloc,
    MLA_APPEND_NOALLOC_MAX_BYTES,
    mla_prefill_workspace_bytes,
    mla_prefill_kv_elems,
    mla_prefill_kv,
    mla_prefill_attention,
    mla_tpla_split_weights,
    mla_tpla_rotate_cache,
    mla_tpla_reduce,
    mla_gqa_queries,
    mla_gqa_output,
    mla_probe_hbm_read,
    mla_probe_mfma,
    mla_probe_tile_copy,
    mla_validate_decode_inputs,
    mla_status_string,
    mla_last_error,
)
from .step import DecodeStep, GqaStep, PrefillStep, TplaStep, capture_steps, combine_up_supported, split_plan  # noqa: F401
