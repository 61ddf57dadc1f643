"""CPU float64 oracle of causal multi-head self-attention (test infrastructure).

Only the test suite, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg use this package. It shares no code with the HIP library.
"""

from .attention import (  # noqa: F401
    backward_packed,
    default_scale,
    forward_packed,
    head_backward,
    head_forward,
    split_packed_head,
)
