"""CPU oracle (fp64) for the attention forward pass.

Test infrastructure: imported only by the tests, the smoke check and the
bench's CPU-baseline leg. The GPU path does not import or call it.
"""
from .attention import (ROW_GROUP, finalize, merge_states, partial_state, sdpa_forward,
                        sdpa_rows, stream_fold)

__all__ = ["ROW_GROUP", "finalize", "merge_states", "partial_state", "sdpa_forward",
           "sdpa_rows", "stream_fold"]
