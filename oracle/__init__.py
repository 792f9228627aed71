"""CPU oracle for the exact attention forward and its gradients (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import this
package. The product path (the HIP library and its Python binding) never does.
"""

from .attention import EmptyRowError, sdpa_reference, sdpa_reference_rows
from .backward import sdpa_backward_reference, sdpa_backward_reference_sampled
from .recurrence import State, finish, merge_states, online_softmax_row

__all__ = [
    "EmptyRowError",
    "sdpa_reference",
    "sdpa_reference_rows",
    "sdpa_backward_reference",
    "sdpa_backward_reference_sampled",
    "State",
    "finish",
    "merge_states",
    "online_softmax_row",
]
