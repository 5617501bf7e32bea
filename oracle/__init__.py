"""Float64 CPU oracle for exact attention and the log-sum-exp merge.

TEST INFRASTRUCTURE, NOT PRODUCT CODE. Only the tests, the smoke check and the bench's CPU-baseline leg may
import this package. It shares no code with the HIP path (no kernels, headers, helpers, tables or constants) and
imports nothing from it; the HIP path never imports it.
"""
from .attention import (  # noqa: F401
    attention,
    attention_backward,
    lse_merge,
    lse_merge_many,
    lse_pair,
    visible,
)
