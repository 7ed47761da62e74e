"""CPU fp64 oracle of the TokenGate gated-prefill path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import this package.  The product path (the
HIP kernels behind the C ABI and their Python binding) never calls it, and this
package never imports the product.

Source: "Researchers from Stanford and UC Berkeley Introduce TokenGate:
Token-Gated Attention Makes Long-Context Prefill Up to 11.3x Faster"
(MarkTechPost, October 2026), cited below as "the article" with its section
headings.  Every function is pinned by tests against something other than
itself (library routines, brute force, closed forms, invariants); none is
"parity unpinned".
"""

from .tokengate import (  # noqa: F401
    apply_rope,
    attention_rows_for_check,
    compact,
    decode_attention,
    gate_scores,
    gate_backward,
    gated_attention,
    gated_attention_backward,
    gated_attention_backward_columns,
    linear_residual,
    plan,
    pruned_layer,
    qkv_rope,
    random_k_keep,
    rms_norm,
    rope_inv_freq,
    round_f32,
    sample_budgets,
    score_grad_from_bias,
    select_topk,
    swiglu,
)
