"""fp64 CPU oracle for exact scaled-dot-product attention (test infrastructure).

This package is test infrastructure only. It may be imported by ``tests/``,
by ``__graft_entry__.smoke()`` and by the ``cpu_baseline`` leg of ``bench.py``,
and by nothing else. The GPU library never calls it and shares no code with
it.

Every function is the plain definition written out in float64. The softmax is
computed two-pass per row with the exact row maximum, not online. See
``oracle/attention.py`` for the definitions and the passages they follow.
"""
from .attention import (  # noqa: F401
    allowed_key_range,
    segment_bounds,
    attention_fwd,
    attention_fwd_rows,
    attention_bwd,
    attention_bwd_group,
    attention_dq_rows,
    attention_dkdv_rows,
    merge_partials,
    e4m3_decode,
)
