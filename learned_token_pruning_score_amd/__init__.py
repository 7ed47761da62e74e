"""TokenGate gated-prefill hot path on MI355X (gfx950).

Python face of libtokengate.so: the C ABI calls under the same names
(``tg_plan``, ``tg_gate_score``, ``tg_select_topk``, ``tg_compact``,
``tg_gated_attn_fwd``, ``tg_gated_attn_bwd``, ``tg_rope_table``, ``tg_qkv_rope``, ``tg_rms_norm``,
``tg_linear_residual``, ``tg_swiglu``) taking torch device tensors, and ``GatedPrefill``,
which strings them together the way the three-phase prefill of the TokenGate
article ("How does TokenGate learned token pruning work?") does.  Every step
runs in the library's HIP kernels; without the built library or a GPU these
functions raise.
"""

from ._lib import (  # noqa: F401
    LIB_PATH,
    TG_BF16,
    TG_F32,
    SIGNATURES,
    TokenGateError,
    load_library,
    status_string,
    tg_abi_version,
    tg_compact,
    tg_compact_workspace,
    tg_gate_bwd,
    tg_gate_bwd_workspace,
    tg_gate_score,
    tg_gated_attn_bwd,
    tg_gated_attn_bwd_workspace,
    tg_gated_attn_fwd,
    tg_decode_attn,
    tg_decode_attn_workspace,
    tg_kv_append,
    tg_kv_scatter,
    tg_linear_residual,
    tg_plan,
    tg_qkv_rope,
    tg_rms_norm,
    tg_rope_table,
    tg_sample_budgets,
    tg_select_topk,
    tg_select_topk_noalloc,
    tg_select_topk_workspace,
    tg_swiglu,
)
from .pipeline import GatedPrefill  # noqa: F401
