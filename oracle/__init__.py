"""fp64 CPU oracle of the VerKV decode path (PoissonComp + KVFetch).

TEST INFRASTRUCTURE ONLY.  This package is the slow, plain reference that the
HIP path is checked against.  Only the test suite, the smoke check of the
package entry point and the CPU-baseline leg of the benchmark may import or run
it; the product path (the C-ABI library and its Python binding) never does, and
shares no code, table or helper with it.

Sources are the pages on "Verify Before You Fetch: Reliable KV Cache Compression
for LLM Inference" (arXiv 2611.11319): the paperdot.bitmofang.com abstract page
and the picx.dev summary page, whose section "Methodology" carries eqs. (3),
(5), (6), (7), (9), (10), Definition 2, Lemma 1 and the KVFetch steps 1-5.
Every function cites the passage it follows.  Where the pages are silent the
reading taken is stated in the function's docstring.

Precision: float64 throughout, Python integers where a sum must be exact.

Modules
  philox       Philox4x32-10 counter-based generator (Salmon et al., SC'11)
  poissoncomp  water-filling of inclusion probabilities and the Poisson sample
  kvfetch      sketch weights, shrinkage fixed point, Bernstein certificate,
               fetch ordering and k*, group union, estimator and refinement
  api          per-sequence mirrors of the library's compress / decode calls
"""
from . import philox, poissoncomp, kvfetch, api  # noqa: F401
