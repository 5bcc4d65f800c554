"""CPU oracle for draft-token verification -- TEST INFRASTRUCTURE ONLY.

Only tests/, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the HIP library.
"""
from .verify import (  # noqa: F401
    FLAG_BAND, STATUS_BAD_LOGITS, STATUS_BAD_PARENT, STATUS_BAD_TOKEN,
    draw_from, greedy_chain, inverse_cdf, rank_order,
    row_is_valid, run_chain_batch, run_tree_batch, sample_chain, transform_row,
    tree_greedy,
)
from .calculator import (  # noqa: F401
    best_gamma, break_even_acceptance, expected_tokens_closed,
    expected_tokens_series, speedup, step_cost,
)
