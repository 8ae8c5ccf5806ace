"""CPU oracle for the MonarchAttention forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call, link
or execute anything in this package: only the test suite, the smoke check and
the CPU-baseline leg of the benchmark use it.  It shares no code with the HIP
path (no kernels, headers, helpers or constant tables); the two meet only in
the seeded input generators, which hold none of the method's arithmetic.

Everything here is plain NumPy in float64 (the gradients in oracle.backward:
plain float64 PyTorch on the CPU, differentiated by torch.autograd), written
for a reader checking it against the pages by eye, not for speed.

Sources (cited by page title and section):
  [MA]    "MonarchAttention: Zero-Shot Conversion to Fast, Hardware-Aware
          Structured Attention" -- abstract (arXiv / OpenReview), the
          OpenReview reviews and author responses, and the scime atlas
          summary ("Proposal", "Approach").
  [MRT]   "MonarchRT: Efficient Attention for Real-Time Video Generation" --
          summary page, "Key claims" and "Method" (tiled Monarch, Theorem 4.1,
          the six aligned video block configurations).

Parity status of each public function is stated in its docstring; functions
whose results no pin fixes say "parity unpinned".
"""

from . import backward
from .layouts import LAYOUTS, grid_index, to_grid, from_grid
from .monarch import (
    forward_untiled,
    forward_tiled,
    forward,
    dense_from_factors,
    tile_of_rows,
    segment_of_cols,
    causal_allowed,
)
from .reference_attention import (
    exact_attention,
    dense_objective,
    row_entropy,
    logsumexp,
    softmax,
)

__all__ = [
    "LAYOUTS", "grid_index", "to_grid", "from_grid",
    "forward_untiled", "forward_tiled", "forward", "dense_from_factors",
    "tile_of_rows", "segment_of_cols", "causal_allowed",
    "exact_attention", "dense_objective", "row_entropy", "logsumexp", "softmax", "backward",
]
