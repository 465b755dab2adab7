"""CPU oracle for causal sliding-window attention (test infrastructure only).

This package is the slow, plain, fp64 definition that the HIP path is checked
against.  It is test infrastructure: only the test suite, the smoke check in
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or call it.  The product path (``sliding_window_causal_amd``) never
imports it and shares no code, table or helper with it.

Every function here is pinned by the CPU tests to values the source pages
print or to closed forms and library routines (see ``tests/test_oracle.py``);
none is "parity unpinned".
"""

from .swa_oracle import (  # noqa: F401
    band_mask,
    band_mask_max_form,
    swa_dense,
    swa_rows,
    swa_blocked,
    swa_loop,
    swa_lse,
    swa_backward,
    swa_backward_rows,
    mha_forward,
    mha_rows,
    ring_fill,
    ring_slot,
    swa_decode,
    swa_chunk,
)
