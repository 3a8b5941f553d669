"""CPU oracle for the fused exact-attention forward pass.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import
anything from this package.  The product path (the HIP library and its Python
binding) never imports, calls or links it, and the two share no code.

Modules
-------
attention  plain two-pass fp64 attention (numpy), the reference every GPU
           result is compared with (also for decode steps, where the queries
           are the last positions of the cached sequence), plus the online-softmax recurrence in the
           pages' own step order (used only to pin the two-pass form).
backward   the gradients (dQ, dK, dV) of that forward, from the chain rule,
           for the GPU backward pass.
brute      the textbook softmax definition written as scalar loops over
           mpmath numbers, with no max-subtraction, for tiny inputs.

Pages cited (the text of three web pages on one subject):
  [CANN-FA]  "FlashAttention operator of the CANN ops-transformer repository:
             attention acceleration on the Ascend NPU", www.mooersco.com/news/1200175
  [FA-Dict]  hwcomputing.csdn.net tutorial page 6a0dbd08662f9a54cb75eb74
             (the "dictionary page by page" explanation of FlashAttention)
  [FA-Infer] gitcode.csdn.net page 6a0c62d2662f9a54cb75b31f (why Transformer
             inference is slow; FlashAttention on Ascend and CANN)

Parity status: every function here is pinned -- the forward and decode
functions by tests/test_oracle_pins.py (closed forms, invariants, brute
force, mutation tests), the backward by tests/test_oracle_bwd.py (finite
differences of the forward, torch autograd, invariants, mutation tests);
none is "parity unpinned".
"""

from .attention import (  # noqa: F401
    attention_decode_ref,
    attention_ref,
    attention_probs,
    online_attention,
    kv_head_of,
)
from .backward import attention_bwd_delta, attention_bwd_ref  # noqa: F401
