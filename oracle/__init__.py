"""FP64 CPU oracle for exact attention -- test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package. The library's own path never calls it, and it shares no code
with the HIP kernels or their host library.
"""
from .attention import (  # noqa: F401
    visible_mask, attention_forward, attention_backward, online_softmax_forward,
    merge_states, FullyMaskedRowError, attention_forward_varlen, attention_backward_varlen,
    philox4x32_10, dropout_threshold, dropout_keep_mask,
)
