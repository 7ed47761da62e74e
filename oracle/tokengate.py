"""Plain, slow, obviously correct fp64 definitions of the gated-prefill steps.

TEST INFRASTRUCTURE ONLY (see the package docstring): never called by the
product path.

Citations name sections of the article "Researchers from Stanford and UC
Berkeley Introduce TokenGate: Token-Gated Attention Makes Long-Context Prefill
Up to 11.3x Faster" (MarkTechPost).  Where the article is silent the reading
taken is stated at the function; the article gives the ingredients of the
attention bias but no formula, so the formula used is
``logit_ij = tau * q_i . k_j / sqrt(d) + g_h * s_j`` with ``s_j = 0`` for keys
outside the document.

All floating-point work is numpy float64.  Inputs may be any real dtype
(bf16/fp32 values upcast exactly).  Integer and index results are exact.
"""

from __future__ import annotations

import math
from typing import Optional, Sequence, Tuple

import numpy as np

_ROW_CHUNK = 1024  # output rows evaluated per numpy call (memory bound only)


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _i64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.int64)


def plan(cu_seqlens, doc_begin, doc_end, budget) -> Tuple[np.ndarray, int]:
    """Kept-token count of every prompt, as an exclusive prefix ``cu_kept``.

    Article, "How does TokenGate learned token pruning work?": only the
    document may be pruned and the question is always kept; "How do you deploy
    TokenGate?": ``generate`` takes a budget on kept prefill tokens.  Reading:
    the budget counts document tokens, so prompt b keeps
    ``min(budget_b, doc_len_b)`` document tokens plus every token outside its
    document.  Returns (cu_kept int64 [B+1], longest kept prompt).
    """
    cu = _i64(cu_seqlens)
    db, de, bud = _i64(doc_begin), _i64(doc_end), _i64(budget)
    B = bud.shape[0]
    cu_kept = np.zeros(B + 1, dtype=np.int64)
    longest = 0
    for b in range(B):
        n = cu[b + 1] - cu[b]
        doc = de[b] - db[b]
        kept = min(bud[b], doc) + (n - doc)
        cu_kept[b + 1] = cu_kept[b] + kept
        longest = max(longest, int(kept))
    return cu_kept, longest


def gate_scores(hidden, W1, b1, w2, b2: float) -> np.ndarray:
    """Gate score of every token: ``s_t = b2 + sum_f w2_f SiLU(b1_f + W1[f] . h_t)``.

    Article, "How does TokenGate learned token pruning work?": an MLP scores
    each token from its post-attention residual at the gate layer; TL;DR: the
    gate is a small MLP.  Reading: one hidden layer with SiLU
    (``z = a / (1 + e^-a)``), biases on both linear maps, raw scalar output.
    Returns fp64 [T].  ``b1=None`` means zero bias.
    """
    h = _f64(hidden)
    W = _f64(W1)
    F = W.shape[0]
    bias1 = np.zeros(F) if b1 is None else _f64(b1)
    w = _f64(w2)
    out = np.empty(h.shape[0], dtype=np.float64)
    with np.errstate(over="ignore"):
        for lo in range(0, h.shape[0], 8192):
            a = h[lo:lo + 8192] @ W.T + bias1[None, :]
            z = a / (1.0 + np.exp(-a))
            out[lo:lo + 8192] = z @ w + float(b2)
    return out


def round_f32(x) -> np.ndarray:
    """Round to float32, nearest-even (the scores' storage precision)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def select_topk(scores, cu_seqlens, doc_begin, doc_end, budget) -> np.ndarray:
    """Keep flags: per prompt the ``min(budget, doc_len)`` best document tokens
    plus every non-document token.

    Article, "How does TokenGate learned token pruning work?": a top-K selector
    keeps the highest-scoring tokens, and only the document is prunable.
    Readings: ``doc_begin``/``doc_end`` are prompt-relative; order is (score
    descending, token index ascending), so equal scores go to the lower index;
    -0.0 equals +0.0; NaN ranks below every number (NaNs tied by index).
    ``scores`` is the fp32 array actually being selected on.  Returns uint8 [T].
    """
    s = np.asarray(scores)
    cu = _i64(cu_seqlens)
    db, de, bud = _i64(doc_begin), _i64(doc_end), _i64(budget)
    keep = np.zeros(s.shape[0], dtype=np.uint8)
    for b in range(bud.shape[0]):
        lo, hi = cu[b], cu[b + 1]
        keep[lo:hi] = 1
        dlo, dhi = lo + db[b], lo + de[b]
        keep[dlo:dhi] = 0
        idx = np.arange(dlo, dhi, dtype=np.int64)
        v = s[dlo:dhi].astype(np.float64) + 0.0  # -0.0 -> +0.0
        # lexsort: last key is primary.  -v ascending == v descending; NaN
        # stays NaN and numpy sorts NaN last.
        order = np.lexsort((idx, -v))
        k = int(min(bud[b], dhi - dlo))
        keep[idx[order[:k]]] = 1
    return keep


def compact(hidden, pos, scores, keep, cu_seqlens, doc_begin, doc_end):
    """Stable gather of the kept tokens.

    Article, "How does TokenGate learned token pruning work?": layers above
    the gate process only the kept tokens; "What is token-gated attention?":
    each kept token's score becomes its attention bias.  Readings: kept tokens
    keep their original order (prompt by prompt, ascending index) and original
    positions; a kept token outside the document has bias +0.0.
    Returns (hidden_k [Kt, D] same dtype as ``hidden``, pos_k int32 [Kt],
    bias_s float32 [Kt], kept_idx int64 [Kt]).
    """
    keep = np.asarray(keep)
    cu = _i64(cu_seqlens)
    db, de = _i64(doc_begin), _i64(doc_end)
    T = keep.shape[0]
    in_doc = np.zeros(T, dtype=bool)
    for b in range(db.shape[0]):
        in_doc[cu[b] + db[b]:cu[b] + de[b]] = True
    kept_idx = np.nonzero(keep)[0].astype(np.int64)
    hidden_k = np.asarray(hidden)[kept_idx]
    pos_k = np.asarray(pos, dtype=np.int32)[kept_idx]
    sc = np.asarray(scores, dtype=np.float32)[kept_idx]
    bias = np.where(in_doc[kept_idx], sc, np.float32(0.0)).astype(np.float32)
    return hidden_k, pos_k, bias, kept_idx


def gated_attention(q, k, v, bias, gain, tau: float, cu_kept,
                    rows: Optional[Sequence[int]] = None):
    """Causal GQA attention over the kept tokens with a per-key score bias.

    Article, "What is token-gated attention?": the kept token's gate score is
    an additive bias on attention logits, scaled by a learnable per-head gain,
    and a learnable temperature acts on the logits.  For prompt b, query head
    h (KV head ``h // (Hq / Hkv)``) and kept row i of that prompt:
    ``x_j = tau * q_i . k_j / sqrt(d) + gain_h * bias_j`` for the prompt's kept
    rows ``j <= i``; ``o_i = sum_j softmax(x)_j v_j``;
    ``lse_i = log sum_j exp(x_j)``.  ``gain=None`` drops the bias term.

    ``q`` [Kt, Hq, d], ``k``/``v`` [Kt, Hkv, d], ``bias`` [Kt].  ``rows``
    restricts evaluation to those global rows (others are NaN).  Returns fp64
    (o [Kt, Hq, d], lse [Hq, Kt]).
    """
    Q, K, V = _f64(q), _f64(k), _f64(v)
    Kt, Hq, d = Q.shape
    Hkv = K.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    group = Hq // Hkv
    s = np.zeros(Kt) if bias is None else _f64(bias)
    g = None if gain is None else _f64(gain)
    cu = _i64(cu_kept)
    o = np.full((Kt, Hq, d), np.nan)
    lse = np.full((Hq, Kt), np.nan)
    want = None if rows is None else np.unique(_i64(rows))
    scale = float(tau) / math.sqrt(d)
    for b in range(cu.shape[0] - 1):
        lo, hi = int(cu[b]), int(cu[b + 1])
        if hi == lo:
            continue
        if want is None:
            r = np.arange(lo, hi)
        else:
            r = want[(want >= lo) & (want < hi)]
        for c0 in range(0, r.shape[0], _ROW_CHUNK):
            rr = r[c0:c0 + _ROW_CHUNK]
            if rr.size == 0:
                continue
            i_rel = rr - lo
            n_keys = int(i_rel.max()) + 1
            visible = np.arange(n_keys)[None, :] <= i_rel[:, None]
            for h in range(Hq):
                kv = h // group
                x = scale * (Q[rr, h, :] @ K[lo:lo + n_keys, kv, :].T)
                if g is not None:
                    x = x + g[h] * s[lo:lo + n_keys][None, :]
                x = np.where(visible, x, -np.inf)
                m = x.max(axis=1)
                e = np.exp(x - m[:, None])
                z = e.sum(axis=1)
                o[rr, h, :] = (e @ V[lo:lo + n_keys, kv, :]) / z[:, None]
                lse[h, rr] = m + np.log(z)
    return o, lse


def attention_rows_for_check(cu_kept, per_prompt: int, seed: int = 0) -> np.ndarray:
    """A seeded sample of kept rows: each prompt's first and last row plus
    ``per_prompt`` rows drawn uniformly (for sizes too large to evaluate whole).
    Pure index sampling; it computes nothing of the method."""
    cu = _i64(cu_kept)
    g = np.random.default_rng(np.random.SeedSequence([int(seed), 7]))
    out = []
    for b in range(cu.shape[0] - 1):
        lo, hi = int(cu[b]), int(cu[b + 1])
        if hi == lo:
            continue
        out.extend([lo, hi - 1])
        n = min(per_prompt, hi - lo)
        out.extend(g.choice(np.arange(lo, hi), size=n, replace=False).tolist())
    return np.unique(np.asarray(out, dtype=np.int64))


def rope_inv_freq(d: int, theta: float) -> np.ndarray:
    """Rotary frequencies ``theta ** (-2 i / d)`` for i = 0 .. d/2 - 1, fp64.

    Reading (the article names Qwen3-1.7B as the model but not its position
    encoding): the rotary embedding of the Qwen3 family, in the rotate-half
    form, with its base ``theta`` (1e6 for Qwen3) as a parameter.
    """
    i = np.arange(d // 2, dtype=np.float64)
    return np.power(float(theta), -2.0 * i / d)


def apply_rope(x, pos, theta: float) -> np.ndarray:
    """Rotate every head vector of ``x`` [n, H, d] at its row's position.

    Article, "How does TokenGate learned token pruning work?": the layers
    above the gate run on the kept tokens only, which keep their original
    position ids.  Reading (rotate-half form): element i of a head is paired
    with element i + d/2, and the pair is rotated by the angle
    ``pos * theta ** (-2 i / d)``:
        y_i        = x_i cos(a_i) - x_{i+d/2} sin(a_i)
        y_{i+d/2}  = x_{i+d/2} cos(a_i) + x_i sin(a_i)
    """
    x = _f64(x)
    d = x.shape[-1]
    half = d // 2
    ang = _f64(pos)[:, None] * rope_inv_freq(d, theta)[None, :]  # [n, d/2]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def qkv_rope(hidden, W, pos, theta: float, Hq: int, Hkv: int, d: int):
    """Attention inputs of a pruned layer from the kept rows.

    Article, "How does TokenGate learned token pruning work?": above the gate
    the model processes only the kept tokens, at their original positions.
    Reading: ``y = hidden @ W.T`` with ``W`` [(Hq + 2 Hkv) d, D] whose rows are
    the q heads, then the k heads, then the v heads (no bias, no per-head
    normalisation); q and k are rotated at the rows' original positions,
    v is not.  Returns fp64 (q [n, Hq, d], k [n, Hkv, d], v [n, Hkv, d]).
    """
    y = _f64(hidden) @ _f64(W).T
    n = y.shape[0]
    q = y[:, :Hq * d].reshape(n, Hq, d)
    k = y[:, Hq * d:(Hq + Hkv) * d].reshape(n, Hkv, d)
    v = y[:, (Hq + Hkv) * d:].reshape(n, Hkv, d)
    return apply_rope(q, pos, theta), apply_rope(k, pos, theta), v


def rms_norm(x, weight, eps: float) -> np.ndarray:
    """RMSNorm of every row: ``y = weight * x / sqrt(mean(x^2) + eps)``.

    Article, "How does TokenGate learned token pruning work?": the layers
    above the gate run on the kept tokens.  Reading (the article names
    Qwen3-1.7B as the model but not its layer): a pre-norm layer of the
    Qwen3 family, with an RMSNorm (per-channel weight, eps 1e-6 there)
    before the attention and before the MLP.
    """
    x = _f64(x)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return _f64(weight) * x / np.sqrt(ms + float(eps))


def linear_residual(a, W, residual) -> np.ndarray:
    """``residual + a @ W.T``: the attention output projection (a = the
    heads' outputs [n, Hq d], W [D, Hq d]) and the MLP's down projection
    (a = the SwiGLU activation [n, I], W [D, I]), each added to the
    residual stream.  Reading as for rms_norm; no bias."""
    return _f64(residual) + _f64(a) @ _f64(W).T


def swiglu(h, W_gate, W_up) -> np.ndarray:
    """SwiGLU activation of the MLP: ``silu(h W_gate^T) * (h W_up^T)`` with
    ``silu(z) = z / (1 + exp(-z))``; W_gate and W_up [I, D].  Reading as for
    rms_norm (the Qwen3 MLP), no bias."""
    g = _f64(h) @ _f64(W_gate).T
    u = _f64(h) @ _f64(W_up).T
    return g / (1.0 + np.exp(-g)) * u


def pruned_layer(x, pos, cu_kept, bias, gain, tau: float, theta: float, eps: float,
                 w_in, W_qkv, Hq: int, Hkv: int, d: int, W_o, w_post, W_gate, W_up, W_down,
                 rows=None) -> np.ndarray:
    """One transformer layer above the gate, on the kept rows only.

    Article, "How does TokenGate learned token pruning work?": the layers
    above the gate see only the kept tokens, at their original positions;
    "What is token-gated attention?": their attention carries the gate's
    score bias.  Reading: the pre-norm layer
        a = x + O(attention(rope(QKV(rms_norm(x)))))
        y = a + Down(swiglu(rms_norm(a)))
    with the attention of ``gated_attention``.  ``rows`` limits the output
    to some rows (the attention still sees every earlier key).
    """
    x = _f64(x)
    n = x.shape[0]
    q, k, v = qkv_rope(rms_norm(x, w_in, eps), W_qkv, pos, theta, Hq, Hkv, d)
    o, _ = gated_attention(q, k, v, bias, gain, tau, cu_kept, rows=rows)
    sel = np.arange(n) if rows is None else np.asarray(rows)
    a = linear_residual(o[sel].reshape(len(sel), Hq * d), W_o, x[sel])
    return linear_residual(swiglu(rms_norm(a, w_post, eps), W_gate, W_up), W_down, a)


def gated_attention_backward(q, k, v, bias, gain, tau: float, cu_kept, dout,
                             rows: Optional[Sequence[int]] = None, out=None):
    """Gradients of ``sum(dout * o)``, o from ``gated_attention``.

    Article, "What is token-gated attention?": top-K is not differentiable,
    so the kept token's score enters the attention as a logit bias, which
    gives the loss a gradient path back to the scorer; the per-head gain and
    the temperature are learned as well.  With ``x_ij = tau q_i.k_j / sqrt(d)
    + g_h s_j`` over visible keys, ``P = softmax_j(x)``, ``o = P v``, the
    softmax derivative gives ``dx_ij = P_ij (dout_i.v_j - dout_i.o_i)`` and
        dq_i  = tau / sqrt(d) sum_j dx_ij k_j
        dk_j  = tau / sqrt(d) sum_(h in group, i) dx_ij q_i
        dv_j  = sum_(h in group, i) P_ij dout_i
        ds_j  = sum_h g_h sum_i dx_ij
        dg_h  = sum_ij dx_ij s_j
        dtau  = sum_(h, ij) dx_ij q_i.k_j / sqrt(d)
    Returns fp64 (dq [Kt, Hq, d], dk, dv [Kt, Hkv, d], ds [Kt], dg [Hq],
    dtau).  ``gain=None`` (no bias term): ds and dg are zero.  ``rows``
    restricts the work to dq of those global rows (each row's softmax needs
    only its own logits); the other results are then None and other dq rows
    NaN.  ``out`` [Kt, Hq, d]: the forward output as stored (e.g. rounded to
    bf16), used for ``D_i = dout_i . out_i`` in place of the exact o, as a
    backward that keeps the forward's output does.
    """
    if rows is not None:
        return _dq_rows(q, k, v, bias, gain, tau, cu_kept, dout, rows)
    Ost = None if out is None else _f64(out)
    Q, K, V, dO = _f64(q), _f64(k), _f64(v), _f64(dout)
    Kt, Hq, d = Q.shape
    Hkv = K.shape[1]
    group = Hq // Hkv
    s = np.zeros(Kt) if bias is None else _f64(bias)
    g = np.zeros(Hq) if gain is None else _f64(gain)
    cu = _i64(cu_kept)
    scale = float(tau) / math.sqrt(d)
    dq = np.zeros_like(Q)
    dk = np.zeros_like(K)
    dv = np.zeros_like(V)
    ds = np.zeros(Kt)
    dg = np.zeros(Hq)
    dtau = 0.0
    for b in range(cu.shape[0] - 1):
        lo, hi = int(cu[b]), int(cu[b + 1])
        if hi == lo:
            continue
        n = hi - lo
        visible = np.arange(n)[None, :] <= np.arange(n)[:, None]
        sb = s[lo:hi]
        for h in range(Hq):
            kv = h // group
            Qh, Kh, Vh, dOh = Q[lo:hi, h], K[lo:hi, kv], V[lo:hi, kv], dO[lo:hi, h]
            qk = Qh @ Kh.T
            x = scale * qk
            if gain is not None:
                x = x + g[h] * sb[None, :]
            x = np.where(visible, x, -np.inf)
            P = np.exp(x - x.max(axis=1, keepdims=True))
            P /= P.sum(axis=1, keepdims=True)
            O = P @ Vh if Ost is None else Ost[lo:hi, h]
            dP = dOh @ Vh.T
            dx = P * (dP - np.sum(dOh * O, axis=1, keepdims=True))
            dq[lo:hi, h] = scale * (dx @ Kh)
            dk[lo:hi, kv] += scale * (dx.T @ Qh)
            dv[lo:hi, kv] += P.T @ dOh
            if gain is not None:
                col = dx.sum(axis=0)
                ds[lo:hi] += g[h] * col
                dg[h] += float(col @ sb)
            dtau += float(np.sum(dx * qk)) / math.sqrt(d)
    return dq, dk, dv, ds, dg, dtau


def gated_attention_backward_columns(q, k, v, bias, gain, tau: float, cu_kept, dout, out, lse,
                                     cols: Sequence[int]):
    """dk, dv and the bias gradient of some key columns, given the forward's
    output and lse (the inputs the backward receives).

    Same formulas as ``gated_attention_backward`` ("What is token-gated
    attention?"), written per key column j of prompt b: over the visible
    queries i >= j of the prompt and the query heads h of j's KV group,
    ``P_ij = exp(x_ij - lse_hi)`` with the given lse, ``D_i = dout_i . out_i``
    with the given output, ``dx_ij = P_ij (dout_i . v_j - D_i)``;
        dk_j = tau / sqrt(d) sum_(h, i) dx_ij q_i
        dv_j = sum_(h, i) P_ij dout_i
        ds_j = sum_h g_h sum_i dx_ij        (all heads)
    ``out`` [Kt, Hq, d], ``lse`` [Hq, Kt].  Returns fp64 (dk [n, Hkv, d],
    dv [n, Hkv, d], ds [n]) for the n columns in ``cols`` order.
    """
    Q, K, V, dO = _f64(q), _f64(k), _f64(v), _f64(dout)
    O, L = _f64(out), _f64(lse)
    Kt, Hq, d = Q.shape
    Hkv = K.shape[1]
    group = Hq // Hkv
    s = np.zeros(Kt) if bias is None else _f64(bias)
    g = None if gain is None else _f64(gain)
    cu = _i64(cu_kept)
    scale = float(tau) / math.sqrt(d)
    cols = _i64(cols)
    dk = np.zeros((cols.shape[0], Hkv, d))
    dv = np.zeros((cols.shape[0], Hkv, d))
    ds = np.zeros(cols.shape[0])
    for n, j in enumerate(cols):
        b = int(np.searchsorted(cu, j, side="right")) - 1
        hi = int(cu[b + 1])
        for h in range(Hq):
            kv = h // group
            Qi, dOi = Q[j:hi, h], dO[j:hi, h]
            x = scale * (Qi @ K[j, kv])
            if g is not None:
                x = x + g[h] * s[j]
            P = np.exp(x - L[h, j:hi])
            D = np.sum(dOi * O[j:hi, h], axis=1)
            dx = P * (dOi @ V[j, kv] - D)
            dk[n, kv] += scale * (dx @ Qi)
            dv[n, kv] += P @ dOi
            if g is not None:
                ds[n] += g[h] * float(dx.sum())
    return dk, dv, ds


def _dq_rows(q, k, v, bias, gain, tau, cu_kept, dout, rows):
    """dq of some query rows: the same formulas as gated_attention_backward,
    one row at a time."""
    Q, K, V, dO = _f64(q), _f64(k), _f64(v), _f64(dout)
    Kt, Hq, d = Q.shape
    group = Hq // K.shape[1]
    s = np.zeros(Kt) if bias is None else _f64(bias)
    cu = _i64(cu_kept)
    scale = float(tau) / math.sqrt(d)
    dq = np.full_like(Q, np.nan)
    for i in np.unique(_i64(rows)):
        b = int(np.searchsorted(cu, i, side="right")) - 1
        lo = int(cu[b])
        for h in range(Hq):
            kv = h // group
            Kh, Vh = K[lo:i + 1, kv], V[lo:i + 1, kv]
            x = scale * (Kh @ Q[i, h])
            if gain is not None:
                x = x + _f64(gain)[h] * s[lo:i + 1]
            P = np.exp(x - x.max())
            P /= P.sum()
            dP = Vh @ dO[i, h]
            dx = P * (dP - dO[i, h] @ (P @ Vh))
            dq[i, h] = scale * (dx @ Kh)
    return dq, None, None, None, None, None


def gate_backward(hidden, W1, b1, w2, ds):
    """Gradients of ``sum(ds * s)`` for the gate score ``s`` of
    ``gate_scores`` (article, "What is token-gated attention?": the score
    bias is the scorer's gradient path).  With ``a = W1 h + b1``,
    ``z = silu(a)``, ``s = b2 + w2.z`` and ``silu'(a) = sig(a) (1 + a (1 - sig(a)))``:
        dw2 = sum_t ds_t z_t,   db2 = sum_t ds_t,
        da_t = ds_t w2 * silu'(a_t),   db1 = sum_t da_t,
        dW1 = sum_t da_t h_t^T,   dh_t = W1^T da_t.
    Returns fp64 (dh [T, D], dW1 [F, D], db1 [F], dw2 [F], db2).
    """
    H, W, w = _f64(hidden), _f64(W1), _f64(w2)
    g = _f64(ds)
    a = H @ W.T
    if b1 is not None:
        a = a + _f64(b1)[None, :]
    sig = 1.0 / (1.0 + np.exp(-a))
    z = a * sig
    da = g[:, None] * w[None, :] * sig * (1.0 + a * (1.0 - sig))
    return da @ W, da.T @ H, da.sum(axis=0), z.T @ g, float(g.sum())


def score_grad_from_bias(dbias, kept_idx, cu_seqlens, doc_begin, doc_end, T: int) -> np.ndarray:
    """Gradient of the loss with respect to every token's gate score, from
    the bias gradient of the kept rows (summed over the pruned layers).

    Article, "What is token-gated attention?": each kept token's score
    becomes its attention bias, so the bias is the scorer's gradient path;
    top-K passes none.  Reading (as in ``compact``): inside its prompt's
    document a kept token's bias is its score, outside it the bias is the
    constant 0.  Returns fp64 ds [T]: ``dbias[r]`` at token ``kept_idx[r]``
    when that token lies in its document, 0 for every other token.
    """
    g = np.zeros(int(T))
    cu = _i64(cu_seqlens)
    db, de = _i64(doc_begin), _i64(doc_end)
    for r, t in enumerate(_i64(kept_idx)):
        b = int(np.searchsorted(cu, t, side="right")) - 1
        rel = int(t - cu[b])
        if db[b] <= rel < de[b]:
            g[t] += float(dbias[r])
    return g


def decode_attention(q, k_cache, v_cache, bias_cache, start, lens, gain, tau: float):
    """One decode step of token-gated attention over the kept-only KV cache.

    Article, "How does TokenGate learned token pruning work?": layers above
    the gate never create KV entries for pruned tokens, so generation reads
    only the kept ones; "What is token-gated attention?": each kept token's
    score stays its bias.  Reading: the bias is persistent — document keys
    keep their gate score, question keys and generated keys carry 0 — and the
    new token sees every cached key of its sequence (including its own,
    appended before the step).  For sequence b, query head h (KV head
    ``h // (Hq / Hkv)``) and cache rows ``start[b] .. start[b] + lens[b]``:
    ``x_j = tau q.k_j / sqrt(d) + g_h bias_j``, ``o = softmax(x) v``,
    ``lse = log sum exp x``.  ``q`` [B, Hq, d]; caches [rows, Hkv, d] and
    [rows].  Returns fp64 (o [B, Hq, d], lse [B, Hq]); a sequence of length
    0 gives NaN.
    """
    Q, K, V = _f64(q), _f64(k_cache), _f64(v_cache)
    s = _f64(bias_cache)
    B, Hq, d = Q.shape
    group = Hq // K.shape[1]
    g = np.zeros(Hq) if gain is None else _f64(gain)
    scale = float(tau) / math.sqrt(d)
    o = np.full((B, Hq, d), np.nan)
    lse = np.full((B, Hq), np.nan)
    for b in range(B):
        lo, n = int(start[b]), int(lens[b])
        if n == 0:
            continue
        for h in range(Hq):
            kv = h // group
            x = scale * (K[lo:lo + n, kv] @ Q[b, h]) + g[h] * s[lo:lo + n]
            m = x.max()
            e = np.exp(x - m)
            o[b, h] = e @ V[lo:lo + n, kv] / e.sum()
            lse[b, h] = m + math.log(e.sum())
    return o, lse


def sample_budgets(doc_begin, doc_end, u, min_frac: float, max_frac: float) -> np.ndarray:
    """Random document budgets for a training step's random-budget loss.

    Article, "What is token-gated attention?": each training step averages a
    full-context loss and a random-budget loss, so one gate works across
    budgets.  Reading (the article gives no distribution): prompt b keeps the
    fraction ``f_b = min_frac + (max_frac - min_frac) u_b`` of its document,
    ``u_b`` in [0, 1) drawn by the caller, and its budget is
    ``floor(f_b * doc_len_b)`` (fp64).  The full-context loss is the budget
    ``doc_len_b`` (f = 1).
    """
    db, de = _i64(doc_begin), _i64(doc_end)
    uu = _f64(u)
    f = float(min_frac) + (float(max_frac) - float(min_frac)) * uu
    return np.floor(f * (de - db)).astype(np.int64)


def random_k_keep(rand_keys, cu_seqlens, doc_begin, doc_end, budget) -> np.ndarray:
    """Random-K selection (article, "How does TokenGate perform on
    benchmarks?": the ablation that keeps K random document tokens instead of
    the K best-scored ones).  Reading: with i.i.d. uniform keys ``rand_keys``
    [T] drawn by the caller, the top-K of the keys (``select_topk`` on them)
    is a uniformly random K-subset of each document; the question is kept as
    always.  The kept tokens' attention bias is still their gate score."""
    return select_topk(rand_keys, cu_seqlens, doc_begin, doc_end, budget)

