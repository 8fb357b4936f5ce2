"""CPU oracle for the fused scaled-dot-product attention forward.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only the tests, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP library (no kernels, helpers, tables or constants) and imports nothing
from ``scaled_dot_product_fwd_amd``.

The oracle is the plain definition of attention written out in float64 with the
score matrix materialised (row chunks bound the memory), i.e. the unfused
matmul-softmax-matmul sequence that the fused kernels replace.

Every function is pinned in ``tests/test_oracle.py`` against brute force on tiny
inputs, closed forms, invariants and a library special case.  No function here
is "parity unpinned".
"""

from .sdpa_ref import (  # noqa: F401
    MASK_KINDS,
    mask_array,
    visible_mask,
    visible_pairs,
    sdpa_ref,
    sdpa_ref_varlen,
    visible_offset,
    sdpa_ref_rows,
    sdpa_probs,
    sdpa_loop,
)
from .sdpa_bwd_ref import sdpa_bwd_ref, sdpa_bwd_ref_varlen  # noqa: F401
