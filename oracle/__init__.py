"""CPU oracle for the paged KV cache hot path -- TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously-correct reference that the HIP
library is checked against.  It is written from the four web pages on
PagedAttention, cited in each function as

  [studynote 223]  "KV Cache PagedAttention" (agnusdei1207 brainscience study note 223)
  [studynote 528]  "vLLM PagedAttention KV cache optimization" (agnusdei1207 study note 528)
  [ch.09]          "09. PagedAttention" (119-ai-studio, LLM inference guide, chapter 9)
  [velog]          "Paged Attention" (velog.io/@junegood)

with the section or figure of the page.  Where the pages leave a step open,
the reading taken is stated at the function.

Rules this package obeys:
  * It imports nothing from the GPU package (paged_kv_cache_424_amd) and the
    GPU package imports nothing from here.  The two share no helper, table,
    layout function or constant generator.  Only the seeded input generators
    in ``workloads`` feed both sides.
  * Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
    ``bench.py`` may import it.  The product path never calls it.
  * Floating point is fp64 (the stored fp32/bf16 values are upcast exactly);
    indices and block bookkeeping are exact Python integers.

Modules:
  allocator  -- block allocator, sequences, fork/copy-on-write, block tables (O1)
  cache      -- the pool layout, cache write and block copy (O2, O3)
  attention  -- gather through the block table and naive softmax attention (O4)
  accounting -- fragmentation / capacity arithmetic used by the pages' examples
"""

from . import allocator, cache, attention, accounting  # noqa: F401
