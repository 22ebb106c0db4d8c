"""fp64 CPU oracle for exact attention and the row-wise softmax -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this package.  The HIP library and its Python binding never do,
and this package imports nothing from them.

Every function here is pinned by a ``-m "not gpu"`` test in
``tests/test_oracle_pins.py`` (closed forms, invariants, brute force on tiny
inputs, finite differences and a library special case); none is "parity unpinned".
"""
from .attention import backward, forward, forward_rows, probabilities, scores  # noqa: F401
from .online import chunk_merge, tiled_forward  # noqa: F401
from .softmax import softmax_rows  # noqa: F401
from .fp8 import decode_e4m3, forward_fp8  # noqa: F401
from .dropout import backward_dropout, forward_dropout, keep_mask, philox4x32_10  # noqa: F401
