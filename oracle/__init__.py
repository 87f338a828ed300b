"""CPU float64 oracle for paged GQA decode — test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import this package. It shares no code with the
library in ``paged_kv_gqa_04_amd``.
"""

from .paged_gqa import (  # noqa: F401
    BF16,
    F16,
    bits_to_f64,
    decode,
    decode_case,
    gather_tokens,
    merge_states,
    range_state,
)
