"""fp64 CPU oracle for exact tiled attention.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the smoke check and by
the benchmark's CPU-baseline leg, never by the product package.  It shares no
code with the HIP path.
"""
from .ref import (  # noqa: F401
    scores, softmax_rows, head_forward, head_backward, head_panel,
    forward, backward, forward_backward,
)
