"""CPU oracle for exact attention -- TEST INFRASTRUCTURE ONLY.

This package is the slow, obviously correct definition that the GPU kernels
are checked against.  Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import it.  The product path (the HIP
library and its Python binding) never imports, calls or falls back to it, and
it shares no code, tables or helpers with that path.

Everything here is plain numpy in float64, following the attention equation
softmax(Q K^T / sqrt(d_k)) V as the pages state it ("FlashAttention (DE)",
section "Problematik der Standard-Attention"; the Russian page
"FlashAttention", section "Проблематика стандартного внимания"), computed the
naive way those sections describe: the full score matrix S is formed, a
two-pass softmax is taken over each whole row, and P is multiplied by V.
No tiling, no online softmax and no recomputation happen here.

Parity pins (tests/test_oracle.py, tests/golden/): every function below is
pinned by closed forms, invariants, brute force on tiny inputs, torch float64
cross-checks and finite differences.  No function in this package is
"parity unpinned".
"""

from .attention import (  # noqa: F401
    scores,
    causal_mask,
    softmax_rows,
    attention_forward,
    attention_forward_rows,
    attention_probs,
    attention_backward,
    attention_backward_from_probs,
    kv_head,
    group_sum,
    decode_positions,
    attention_decode,
    e4m3_to_float,
    attention_forward_fp8,
)
