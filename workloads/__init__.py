"""Seeded synthetic inputs shared by the tests, the bench and the oracle checks.

This module draws random numbers and builds allocator op scripts.  It holds
none of the method's arithmetic: no slot, layout, softmax or copy rule lives
here, so that the HIP path and the CPU oracle can both consume its output
while sharing no code with each other.
"""

from .configs import (  # noqa: F401
    Workload, CONFIG_NAMES, make, c1_tiny, c2_llama8b, c3_long, c4_shared_prefix, c4_prompt_cache, decode_batch,
    c5_mixed,
    NAN_FILL_BF16, NAN_FILL_F32, round_to_bf16_bits, relayout, subset,
)
