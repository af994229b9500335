"""CPU oracle for the QSA hot path.  TEST INFRASTRUCTURE ONLY.

Only the test-suite, the smoke check in ``__graft_entry__`` and the CPU
baseline leg of ``bench.py`` may import or call this package.  The product
path (the HIP library and its Python binding) never touches it, and it never
touches the product path: the two share no code.

See ``oracle/qsa_oracle.py`` for the definitions and their sources.
"""
from .qsa_oracle import (  # noqa: F401
    BLOCK, TOPK, IDX_HEADS, IDX_DIM, HEAD_DIM,
    bf16_bits_to_f64, f64_to_bf16_bits,
    compress_keys, block_scores, select_blocks, expand_tokens,
    attend, query_positions, qsa_forward, dense_decode,
    block_scores_rows, select_blocks_rows, select_rows,
    block_teacher, selection_recall, needle_survival,
    attend_backward, block_scores_backward, compress_keys_backward,
)
