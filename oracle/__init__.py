"""CPU oracle for the exact attention forward (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import this
package. The product path (the HIP library and its Python binding) never does.
"""

from .attention import EmptyRowError, sdpa_reference, sdpa_reference_rows
from .recurrence import State, finish, merge_states, online_softmax_row

__all__ = [
    "EmptyRowError",
    "sdpa_reference",
    "sdpa_reference_rows",
    "State",
    "finish",
    "merge_states",
    "online_softmax_row",
]
