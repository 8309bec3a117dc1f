"""fp64 CPU oracle for exact attention — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. It shares no code with the HIP library or
its Python binding and imports nothing from them.

Pins: every function here is checked by the ``-m "not gpu"`` tests against closed
forms, hand-derived golden values (``tests/golden``), invariants of softmax and a
pure-Python brute force (``oracle.brute``). No function is "parity unpinned".
"""
from .attention import (  # noqa: F401
    allowed_keys,
    attention,
    attention_backward,
    decode,
    gather_pages,
    merge_partials,
    online_attention_row,
    online_softmax_stats,
    scatter_pages,
    softmax_rows,
    two_pass_attention_row,
    window_mask,
)
