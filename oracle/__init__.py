"""fp64 CPU oracle for exact attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the GPU library imports, calls or links this
package; only the tests, the smoke check and the benchmark's CPU-baseline leg may.
It shares no code with the HIP path.

Pages cited (by title and section):
  * "Phase 08 -- Inference Optimization at Depth", Concepts list and Lab 01
    (standard attention as the reference; the online-softmax recurrence in the
    Lab 01 talking points; O and the logsumexp L as the only stored outputs),
    Lab 03 step 4 (attention over non-contiguous KV pages via an indirection table).
  * screna.ai interview notes, FlashAttention block (S = QK^T, P = softmax(S))
    and MHA/MQA/GQA block (heads grouped, each group shares one K and V).

Every function is "pinned" by the CPU tests in tests/test_oracle.py and
tests/test_oracle_bwd.py (closed forms, brute force on tiny shapes, finite
differences, identities).  Nothing here is "parity unpinned".
"""

from .attention import (  # noqa: F401
    attention_ref,
    alibi_slopes_ref,
    decode_ref,
    prefill_paged_ref,
    dequant_pages_ref,
    decode_int8_ref,
    online_ref,
    lse_merge_ref,
    gather_pages_ref,
)
from .backward import attention_bwd_ref, attention_bwd_delta_ref  # noqa: F401
