"""Test infrastructure: the fp64 CPU oracle and its brute-force cross-check.

Only the test suite, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may use this package.  It shares no code with the HIP
library and never imports it.
"""

from . import layer_oracle  # noqa: F401
from .longformer_oracle import (  # noqa: F401
    attention,
    attention_backward,
    attention_backward_bh,
    attention_bh,
    attention_global_proj,
    attention_global_proj_sampled,
    attention_lse,
    attention_lse_bh,
    attention_sampled,
    global_set,
    mask_count,
    mask_rows,
    window_member,
)
