"""CPU oracle (float64) for the Compressed-PagedAttention compression step.

Test infrastructure only: used by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the library itself.
"""
from .zipage_ref import *  # noqa: F401,F403
from .zipage_ref import (Params, Batch, Plan, BlockPool, UnitResult,  # noqa: F401
                         budget_tokens, widen, row_location, gather_rows,
                         window_positions, window_attention,
                         lightning_redundancy, combine_scores, pinned_mask,
                         select_keep, first_hole, compact_unit, update_global,
                         score_unit, compress, decode_attention, paged_decode)
