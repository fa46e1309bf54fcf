"""Plain fp64 CPU oracle of one dual-cache block-decoding iteration.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  It shares no code with the HIP path
(the ``block_wise_decoding_amd`` package) and imports nothing from it.
"""
from .dblock_oracle import (  # noqa: F401
    bf16_bits_to_f64,
    dual_cache_kv,
    attend,
    lm_logits,
    confidence_from_logits,
    lmhead_confidence,
    threshold_commit,
    iteration,
)
from .decoding import (  # noqa: F401
    threshold_commit_eos,
    decode_block,
    cache_append,
)
from .parity import (  # noqa: F401
    exclusion_set,
    attention_row_rel_err,
    compare_commit,
    block_schedule_violations,
    block_schedule_unambiguous,
)
