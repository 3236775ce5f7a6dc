"""MI355X (gfx950) sparse-attention decode step: lightning-indexer scoring,
exact top-k selection and sparse multi-query attention as hand-written HIP
kernels behind the C ABI in include/dsa.h.

Importing the package loads libdsa.so and raises if it has not been built.
"""
from .binding import (  # noqa: F401
    DsaDims,
    DsaError,
    dsa_decode_step,
    dsa_decode_step_mt,
    dsa_decode_step_mt_workspace_bytes,
    NOALLOC_SCRATCH_BYTES,
    dsa_compress,
    dsa_decode_step_noalloc,
    dsa_decode_step_sink,
    dsa_decode_step_ragged,
    dsa_decode_step_workspace_bytes,
    dsa_indexer_qproj,
    dsa_indexer_score,
    dsa_indexer_score_mt,
    dsa_indexer_topk,
    dsa_indexer_topk_chunks,
    dsa_indexer_topk_workspace_bytes,
    dsa_sparse_attend,
    dsa_sparse_attend_mt,
    dsa_sparse_attend_sink,
    dsa_sparse_attend_workspace_bytes,
    dsa_topk,
    dsa_topk_ragged,
    dsa_topk_workspace_bytes,
    make_dims,
    status_string,
)
