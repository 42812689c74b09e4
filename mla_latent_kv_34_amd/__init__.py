"""MI355X (gfx950) MLA hot path: paged latent cache append, weight-absorbed
split-KV decode (also from hidden states, with the projections in front of it)
and un-absorbed causal prefill (whole prompts or chunks over an existing
cache), as HIP kernels behind the C ABI in
include/mla.h.  This package is the thin Python binding."""
from ._lib import (  # noqa: F401
    Dims, MlaError, LibraryMissing, load, cache_append, decode, decode_step, decode_step_noalloc,
    decode_workspace_size,
    decode_hidden, decode_hidden_workspace_size, decode_layer, merge_query_weights,
    decode_hidden_merged, merge_output_weights, decode_layer_merged, prefill, prefill_workspace_size, prefill_chunk,
    prefill_chunk_workspace_size, LIB_PATH, EXPORTED,
    MLA_OK, MLA_ERR_INVALID_ARG, MLA_ERR_UNSUPPORTED, MLA_ERR_WORKSPACE, MLA_ERR_HIP,
    CHUNK_AUTO, CHUNK_EXPAND, CHUNK_ABSORB,
)
