"""Host orchestration of the gated prefill: gate -> top-K -> compaction ->
token-gated attention, on one stream, with every buffer allocated once.

The TokenGate article ("How does TokenGate learned token pruning work?")
splits prefill into a standard forward below the gate layer, the gate module
(score every token, keep the top-K document tokens and the whole question),
and a pruned forward over the kept tokens whose attention carries the score
bias ("What is token-gated attention?").  This class runs the gate module
(score, top-K, compaction), the rotary table of the kept rows' original
positions, the token-gated attention, and a whole pruned layer on the kept
rows (``pruned_layer``: RMSNorm, the fused q/k/v projection with the rotary
embedding, the gated attention, the output projection added to the residual,
RMSNorm and the SwiGLU MLP added to the residual).
The kept count is known on the host from the metadata (``tg_plan``), so no
step waits on the device.
"""

from __future__ import annotations

from typing import Optional, Sequence

import numpy as np
import torch

from . import _lib


class GatedPrefill:
    def __init__(self, cu_seqlens, doc_begin, doc_end, budget, D: int,
                 dtype: torch.dtype, device="cuda", with_index: bool = True):
        self.cu_seqlens_h = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
        self.doc_begin_h = np.ascontiguousarray(doc_begin, dtype=np.int32)
        self.doc_end_h = np.ascontiguousarray(doc_end, dtype=np.int32)
        self.budget_h = np.ascontiguousarray(budget, dtype=np.int32)
        self.cu_kept_h, self.max_kept_len = _lib.tg_plan(
            self.cu_seqlens_h, self.doc_begin_h, self.doc_end_h, self.budget_h)
        self.B = int(self.budget_h.shape[0])
        self.T = int(self.cu_seqlens_h[-1])
        self.Kt = int(self.cu_kept_h[-1])
        self.D = D
        self.dtype = dtype
        dev = torch.device(device)
        self.device = dev
        i32 = dict(dtype=torch.int32, device=dev)
        self.cu_seqlens = torch.from_numpy(self.cu_seqlens_h).to(dev)
        self.doc_begin = torch.from_numpy(self.doc_begin_h).to(dev)
        self.doc_end = torch.from_numpy(self.doc_end_h).to(dev)
        self.budget = torch.from_numpy(self.budget_h).to(dev)
        self.cu_kept = torch.from_numpy(self.cu_kept_h).to(dev)
        self.scores = torch.empty(self.T, dtype=torch.float32, device=dev)
        self.keep = torch.empty(self.T, dtype=torch.uint8, device=dev)
        self.hidden_k = torch.empty((self.Kt, D), dtype=dtype, device=dev)
        self.pos_k = torch.empty(self.Kt, **i32)
        self.bias_s = torch.empty(self.Kt, dtype=torch.float32, device=dev)
        self.kept_idx = torch.empty(self.Kt, **i32) if with_index else None
        self.rope_table = None
        self.ws_select = torch.empty(max(16, _lib.tg_select_topk_workspace(self.B, self.T)),
                                     dtype=torch.uint8, device=dev)
        self.ws_compact = torch.empty(max(16, _lib.tg_compact_workspace(self.B, self.T)),
                                      dtype=torch.uint8, device=dev)

    def gate_and_select(self, hidden: torch.Tensor, W1: torch.Tensor, b1: Optional[torch.Tensor],
                        w2: torch.Tensor, b2: float, pos: Optional[torch.Tensor] = None,
                        rand_keys: Optional[torch.Tensor] = None, stream=None) -> None:
        """Score every token, pick the kept set, compact rows/positions/biases.

        With ``rand_keys`` [T] (i.i.d. uniform draws, fp32) the kept set is
        random-K: the top-K of the random keys instead of the scores; the
        kept tokens' bias is still their score."""
        _lib.tg_gate_score(hidden, W1, b1, w2, b2, scores=self.scores, stream=stream)
        keys = self.scores if rand_keys is None else rand_keys
        _lib.tg_select_topk(keys, self.cu_seqlens, self.doc_begin, self.doc_end,
                            self.budget, keep=self.keep, workspace=self.ws_select, stream=stream)
        _lib.tg_compact(hidden, pos, self.scores, self.keep, self.cu_seqlens, self.doc_begin,
                        self.doc_end, self.Kt,
                        out=(self.hidden_k, self.pos_k, self.bias_s, self.kept_idx),
                        workspace=self.ws_compact, stream=stream)

    def rope(self, d: int, rope_theta: float, stream=None) -> torch.Tensor:
        """cos / sin table of the kept rows' original positions (after
        gate_and_select; shared by every pruned layer of the forward)."""
        if getattr(self, "rope_table", None) is None or self.rope_table.shape[1] != d // 2:
            self.rope_table = torch.empty((self.Kt, d // 2, 2), dtype=torch.float32,
                                          device=self.device)
        return _lib.tg_rope_table(self.pos_k, d, rope_theta, out=self.rope_table, stream=stream)

    def project_qkv(self, w_qkv: torch.Tensor, Hq: int, Hkv: int, d: int,
                    out: Optional[torch.Tensor] = None, x: Optional[torch.Tensor] = None,
                    stream=None):
        """q, k, v of a pruned layer from the kept rows x (default hidden_k;
        after rope()).  Returns (qkv, q, k, v) as tg_qkv_rope does; q, k and
        v feed attend() in place."""
        x = self.hidden_k if x is None else x
        return _lib.tg_qkv_rope(x, w_qkv, self.rope_table, Hq, Hkv, d, out=out, stream=stream)

    def pruned_layer(self, W_qkv: torch.Tensor, weights: dict, Hq: int, Hkv: int, d: int,
                     gain: torch.Tensor, tau: float, eps: float, x: Optional[torch.Tensor] = None,
                     stream=None) -> torch.Tensor:
        """One pre-norm layer above the gate on the kept rows x (default
        hidden_k), updated in place (after rope()):
            x += W_o . attention(rope(W_qkv . rms_norm(x)))
            x += W_down . (silu(W_gate . rms_norm(x)) * (W_up . rms_norm(x)))
        ``weights`` holds w_in, W_o, w_post, W_gate, W_up, W_down.  The
        intermediates live in buffers allocated on the first call."""
        x = self.hidden_k if x is None else x
        Kt, D = x.shape
        N = (Hq + 2 * Hkv) * d
        I = weights["W_gate"].shape[0]
        key = (Kt, D, N, Hq * d, I, x.dtype)
        if getattr(self, "_layer_key", None) != key:
            mk = lambda *shape: torch.empty(shape, dtype=x.dtype, device=x.device)  # noqa: E731
            self._layer_bufs = {"xn": mk(Kt, D), "qkv": mk(Kt, N), "att": mk(Kt, Hq, d),
                                "act": mk(Kt, I)}
            self._layer_key = key
        b = self._layer_bufs
        _lib.tg_rms_norm(x, weights["w_in"], eps, out=b["xn"], stream=stream)
        _, q, k, v = _lib.tg_qkv_rope(b["xn"], W_qkv, self.rope_table, Hq, Hkv, d, out=b["qkv"],
                                      stream=stream)
        self.attend(q, k, v, gain, tau, out=b["att"], stream=stream)
        _lib.tg_linear_residual(b["att"].view(Kt, Hq * d), weights["W_o"], x, out=x, stream=stream)
        _lib.tg_rms_norm(x, weights["w_post"], eps, out=b["xn"], stream=stream)
        _lib.tg_swiglu(b["xn"], weights["W_gate"], weights["W_up"], out=b["act"], stream=stream)
        _lib.tg_linear_residual(b["act"], weights["W_down"], x, out=x, stream=stream)
        return x

    def gate_backward(self, dbias: torch.Tensor, W1: torch.Tensor, b1: Optional[torch.Tensor],
                      w2: torch.Tensor, stream=None):
        """Backward of the gate MLP from the kept rows' bias gradient dbias
        [Kt] (summed over the pruned layers), after gate_and_select with
        with_index.  Returns (dhidden_k [Kt, D], dW1, db1, dw2, db2); the
        gradient of hidden at token kept_idx[r] is dhidden_k[r], zero at the
        other tokens."""
        return _lib.tg_gate_bwd(self.hidden_k, W1, b1, w2, dbias, self.kept_idx, self.cu_seqlens,
                                self.doc_begin, self.doc_end, stream=stream)

    def attend(self, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, gain: torch.Tensor,
               tau: float, out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
               stream=None):
        """Token-gated causal GQA attention of one layer over the kept tokens."""
        return _lib.tg_gated_attn_fwd(q, k, v, self.bias_s, gain, tau, self.cu_kept,
                                      self.max_kept_len, out=out, lse=lse, stream=stream)
