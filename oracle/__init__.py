"""fp64 CPU oracle for sliding-window attention (SWA).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, constants or
helpers with the HIP library; the only thing both sides see is the seeded
input generator in ``swa_inputs.py``, which holds no attention arithmetic.

Every function here is the plain definition written out in float64 numpy,
citing the page that defines it.  Every function is pinned by a CPU test
against something other than itself (values the pages print, closed forms,
library routines for the special cases, brute force); see
``tests/test_oracle_pins.py``.
"""

from .swa_ref import (  # noqa: F401
    CAUSAL,
    SYMMETRIC,
    allowed,
    band,
    window_mask,
    additive_mask,
    scores_per_layer,
    stacked_reach,
    kv_head,
    attention_loop,
    attention_dense,
    attention_banded,
    attention_rows,
    ring_append,
    decode,
    ring_append_chunk,
    prefill_chunk,
    dilated_mask,
    attention_dilated_dense,
    attention_dilated_rows,
    global_mask,
    attention_global_dense,
    attention_global_rows,
    decode_sinks,
)
