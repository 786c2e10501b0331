"""CPU oracle for CompileMask's hot path: TEST INFRASTRUCTURE ONLY.

Only the test suite, the package's smoke check and the benchmark's CPU-baseline
leg may import this package.  The library's product path never calls it and has
no CPU fallback: it fails loudly when its HIP library is missing.

What it computes (numpy, float64, plain and slow on purpose):
  * ``masks``:      each mask family's visibility predicate, evaluated element
                    by element into a dense boolean mask, and the metadata
                    validity rules;
  * ``descriptor``: the Execution Descriptor read straight off that dense mask:
                    maximal visible runs per query row and per key column,
                    zero-length padding, tile states from visible counts, the
                    2-bit packing and the documented byte layout;
  * ``attention``:  dense masked softmax attention and its analytic backward.

CompileMask reaches exactly (up to rounding order) the result of dense masked
attention: skipping empty tiles and checking visibility only in partial tiles
changes the work, not the result (CompileMask paper summary, section 2.1
"Background" and section 3.3.2 "Descriptor-Guided Attention Execution").  So the
oracle is that plain definition written out.

It shares no code with ``runtime_metadata_attention_amd``; only the seeded
input generators in ``workloads`` serve both.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
(closed-form visible counts, a hand-derived worked example, brute-force
cross-checks, finite differences and textbook-library reductions).  None is
"parity unpinned".
"""
from . import masks, descriptor, attention  # noqa: F401
