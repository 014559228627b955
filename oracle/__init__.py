"""CPU oracle for exact attention (float64, numpy and plain Python).

TEST INFRASTRUCTURE ONLY. This package is the slow, obviously correct
reference that the GPU library is checked against. Only the tests, the
smoke check and the benchmark's CPU-baseline leg may import it; the
library's product path never does, and it shares no code with the HIP
kernels.

Contents:
  softmax    -- safe softmax and the streaming normalizer recurrence
  attention  -- materialized forward (O, LSE) and textbook backward
  blockwise  -- the Q-stationary blockwise (m, d, O) update, a second route
  bruteforce -- scalar Python loops for tiny shapes, a third route
  fp8        -- e4m3 codes, the 128-row block quantizer (float32 recipe),
                dequantization and the forward on dequantized inputs

Every function is pinned by CPU tests against values and identities the
source pages and the mathematics fix (see tests/test_oracle.py); none is
"parity unpinned".
"""

from .softmax import safe_softmax, online_normalizer, logsumexp_from_state
from .attention import (fp32_scale, head_forward, head_probabilities, attention_forward,
                        head_backward, attention_backward, head_dq_rows)
from .blockwise import blockwise_head_forward, even_blocks, random_blocks
from .bruteforce import bruteforce_attention

__all__ = [
    "safe_softmax", "online_normalizer", "logsumexp_from_state",
    "fp32_scale", "head_forward", "head_probabilities", "attention_forward",
    "head_backward", "attention_backward", "head_dq_rows",
    "blockwise_head_forward", "even_blocks", "random_blocks",
    "bruteforce_attention",
]
