"""fp64 CPU oracle of the HSTU layer forward over a paged KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports this package; only
the tests, the smoke check and the benchmark's CPU-baseline leg use it.  It
shares no code with the HIP path: it is plain numpy (float64) and pure Python,
written from the method's definition, with no blocking, fusion or reordering
beyond bounding memory by processing query rows in blocks.

Sources (the pages this follows):
  * NVIDIA technical blog "Deploying an HSTU generative recommender with NVIDIA
    Dynamo-Triton" (Korean edition), sections "Why serving large sequential
    recommenders is hard" (jagged inputs; reuse of cached history K/V; a paged
    GPU KV data table with lookup/allocate/append/evict; an HSTU attention
    kernel that reads the paged cache) and "Benefits" (reuse cached K/V for the
    stable prefix and compute only the newly added tokens).
  * aitrends.kr summary article 100093, section "HSTU sequential modelling",
    and the news.bpdata.com Hungarian article, section "HSTU": softmax
    attention is replaced by SiLU weighting, a relative attention bias is
    added, and elementwise gating precedes the output projection.

The pages give no equation.  The exact layer (SiLU(X W1) split into U, V, Q,
K; pointwise SiLU(QK^T + bias) / N applied to V with a causal mask; LayerNorm
of each token's attention output row; gating by U; projection by W2) and each
reading taken where the pages are silent are listed in the project's design
notes and restated in each function's docstring.

Modules:
  buckets  -- integer log-linear relative-position bucket rule
  layer    -- jagged layer / stack (numpy fp64) and a padded-dense variant
  brute    -- scalar pure-Python brute force for tiny shapes
  paging   -- pool layout: append (scatter) and gather through a page table
  kvcache  -- reference model of the cache manager (LRU, host tier, trim)
  preprocess -- token rows: embeddings, interleave, context, positions
  beam     -- Semantic-ID beam-decode attention over a shared context KV
"""
from . import buckets, layer, brute, paging, preprocess, beam  # noqa: F401
