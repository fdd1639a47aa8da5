"""fp64 CPU oracle for exact attention — TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the bench's CPU-baseline leg may
import this package.  The product path (the HIP library and its Python
binding) never imports, calls or links anything here, and this package never
imports the product path: the two share no code.

Parity is pinned for every function here by the CPU tests (invariants, closed
forms, library routines, brute force and a hand-worked example); no function
is "parity unpinned".
"""
from .attention import (  # noqa: F401
    attention_forward,
    attention_forward_rows,
    attention_backward,
    decode_paged,
    online_forward,
    attention_forward_gqa,
    attention_backward_gqa,
    attention_forward_varlen,
    attention_backward_varlen,
    prefill_paged,
    apply_rope,
    apply_rope_bf16,
    attention_forward_rope,
)
