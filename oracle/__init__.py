"""fp64 CPU oracle for exact softmax attention — TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import or run anything in this package.  The product path (the HIP library
and its Python binding) never calls it and must fail loudly rather than fall
back to it.

It shares no code with the HIP path: no kernels, headers, helpers, tables or
constants.  It is the plain definition of attention written out in float64
(materialising the score and probability rows), plus the online-softmax
recurrence the pages describe, plus a pure-Python brute force used to pin the
NumPy code on tiny inputs.

Modules:
  attention  - naive fp64 attention with causal/window masks, GQA/MQA head
               sharing, log-sum-exp, and the paged-cache decode and
               chunked-prefill oracles
  online     - the online softmax and the tiled recurrence (pages' algorithm)
  brute      - pure-Python loops with math.fsum, for n <= 16
  backward   - fp64 gradients dQ, dK, dV of the plain definition
  varlen     - the definition applied per sequence of a packed batch

Every function is pinned by the ``-m "not gpu"`` tests in ``tests/`` against
the pages' printed values, closed forms and invariants.
"""
from .attention import (attention, attention_head, decode_paged, gather_paged, prefill_paged,
                        visible_mask)
from .online import online_softmax, tiled_attention_head, merge_states
from .backward import attention_backward, attention_backward_head
from .varlen import attention_varlen, attention_varlen_backward

__all__ = [
    "attention",
    "attention_head",
    "decode_paged",
    "prefill_paged",
    "gather_paged",
    "visible_mask",
    "online_softmax",
    "tiled_attention_head",
    "merge_states",
    "attention_backward",
    "attention_backward_head",
    "attention_varlen",
    "attention_varlen_backward",
]
