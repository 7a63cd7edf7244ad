"""Float64 CPU oracle for scaled-dot-product attention (test infrastructure only).

This package is the reference the GPU path is checked against. Only the test
suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import it; the library itself never does, and the two share no code.

Every public function here is pinned by ``tests/test_oracle_pins.py`` to
something other than itself (brute force, closed forms, special cases, the
pages' printed tables). None is "parity unpinned".
"""

from .attention import (  # noqa: F401
    visible,
    softmax_rows,
    attention,
    attention_lse,
    attention_bwd,
    attention_rows,
    attention_weights,
    sequence_pages,
    gather_sequence,
    decode_paged,
    decode_paged_window,
    kv_append,
    prefill_paged,
)
