"""CPU oracle (fp64) for exact attention.

TEST INFRASTRUCTURE ONLY: used by tests/, the smoke check and the benchmark's
CPU-baseline leg.  The product path (exact_attention_80_amd) never imports it.
"""

from .attention import (  # noqa: F401
    attention_backward,
    attention_flops,
    attention_forward,
    attention_probs,
    head_forward_backward,
    head_key_rows,
    head_query_rows,
    head_probs,
    varlen_backward,
    varlen_forward,
    varlen_qk_backward,
    varlen_qk_flops,
    varlen_qk_forward,
)
