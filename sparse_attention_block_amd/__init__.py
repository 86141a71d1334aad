"""MI355X-native MiniMax-M3 lightning-indexer decode pass.

The pass runs in hand-written HIP kernels for gfx950 behind the C ABI in
include/msa_indexer.h; this package holds the thin ctypes binding (same names as
the C entry points), the in-tree build, and the seeded input generators.
"""
from ._lib import (  # noqa: F401
    ENGINE_DEFAULT,
    ENGINE_MFMA,
    ENGINE_VALU,
    MsaError,
    bind_decode,
    bind_decode_multi,
    load,
    msa_indexer_block_scores,
    msa_indexer_block_scores_fp8,
    msa_indexer_block_scores_multi,
    msa_indexer_decode,
    msa_indexer_decode_fp8,
    msa_indexer_decode_multi,
    msa_indexer_decode_noalloc,
    msa_indexer_decode_pages,
    msa_indexer_expand_pages,
    msa_indexer_expand_pages_multi,
    msa_indexer_merge,
    msa_indexer_read_error,
    msa_indexer_split_topk,
    new_workspace,
    num_splits,
    plan,
    status_string,
    workspace_bytes,
    workspace_bytes_multi,
)
