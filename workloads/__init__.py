"""Seeded synthetic inputs shared by the tests, the bench and the oracle runs.

Holds no step of the method itself: only scheduler-style metadata (lengths,
block tables, slot mappings) and random tensor contents.
"""

from .layout import ELEM_BYTES, StepLayout, build_layout, permute_requests  # noqa: F401
from .configs import (  # noqa: F401
    BENCH_CONFIGS,
    tiny_decode_fp32,
    llama3_8b_decode,
    llama3_8b_spec_verify,
    long_context_splitk,
    llama2_7b_mha_decode,
    mixed_step,
    mixed_step_prefill_only,
    small_decode,
    small_varlen,
)
