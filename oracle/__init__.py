"""Plain float64 CPU oracle of the Tensor Cache memory and the delta rule.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import anything from this package.  The
HIP library never calls it, and it shares no code with the HIP path: every
function here is written from the pages' definitions, sequentially per token,
in float64 NumPy.

Sources (cited by page title and section):

* "Tensor Cache: Eviction-conditioned Associative Memory for Transformers"
  (gist.science summary), Methodology 1 (two-level architecture: L1 ring of
  the W most recent tokens, L2 outer-product matrix A, write, read, fusion)
  and Methodology 2 (parallel weighted-sum scan vs the chunk-mean shortcut);
  the capacity diagnostic of its results (``capacity``).
* "DeltaNet-family linear attention variants" (molayo1419.me), sections on the
  core identity, the additive-write problem, DeltaNet's prediction-error
  write, locality in key space and the reconstruction-loss derivation.
* "Hebbian memory MLP stores facts in Transformers without training"
  (mo.ai.kr), "a simple MLP construction": the classical memory W = sum v k^T,
  the gated feature map phi(x) = (A x) * (G x), the output matrix
  B = (1/F) sum v phi(k)^T and the storage definition (``hebbian``).

Every function is pinned by ``tests/test_oracle_*.py`` against closed forms,
brute-force sums, special cases and invariants; none is "parity unpinned".
"""
from . import tc, delta, hebbian, capacity  # noqa: F401
