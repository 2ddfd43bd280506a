"""Oracle package: plain fp64 CPU implementation of the Longformer combined
attention forward, of its gradients and of its input projections.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by
the benchmark's CPU-baseline leg, never by the product library.  It shares
no code with the HIP path.
"""
from .longformer_attention import (  # noqa: F401
    dense_bruteforce,
    forward,
    forward_rows,
    in_window,
    pair_count,
    pattern,
)
from .longformer_backward import backward, row_lse  # noqa: F401,E402
from .projections import project  # noqa: F401,E402
