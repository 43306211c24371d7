"""MI355X-native rank-share causal attention for context parallelism.

One context-parallel rank's share of causal attention, computed blockwise on one GPU with
hand-written gfx950 HIP kernels behind a C ABI (include/cpattn.h, libcpattn.so), plus the
layout companions of the all-gather and Ulysses variants.  This package is the thin
Python binding; build the library with ``python -m context_causal_attention_amd.build``.
"""
from ._binding import (  # noqa: F401
    BWD_WRITE_DKV,
    BWD_WRITE_DQ,
    HEADS_TO_SEQ,
    RANK_TO_SEQ,
    SEQ_TO_HEADS,
    SEQ_TO_RANK,
    CpattnError,
    attn_bwd_delta,
    block_bwd,
    block_fwd,
    block_fwd_merge,
    block_fwd_rows,
    header_entry_points,
    library_path,
    load_library,
    lse_merge,
    reorder_gathered,
    ring_blocks_bwd,
    ring_blocks_fwd,
    ring_share_bwd,
    ring_share_fwd,
    ulysses_heads_to_seq,
    ulysses_seq_to_heads,
    ulysses_share_fwd,
    usp_share_fwd,
    zigzag_index,
    zigzag_index_all,
)
