"""MLA decoding over a paged latent KV cache on MI355X (gfx950).

The compute lives in libmla.so (HIP kernels behind the C ABI of
include/mla.h); this package is its Python binding.
"""
from .binding import (  # noqa: F401
    BF16, F32, FP8_E4M3, Dims, MLAError, absorb_from_latent, absorb_from_latent_workspace_bytes, absorb_append, absorb_q,
    append_cache, cache_block_bytes, check_block_table, combine, combine_up_proj, decode,
    decode_needs_combine, decode_workspace_bytes, load_library, make_dims, prefill, prefill_paged,
    prefill_paged_workspace_bytes, prefill_workspace_bytes, project_down, project_down_workspace_bytes, up_proj,
)
from .pipeline import DecodeStep  # noqa: F401
