"""Seeded synthetic workloads shaped like the TokenGate gate layer.

The TokenGate article ("Researchers from Stanford and UC Berkeley Introduce
TokenGate: Token-Gated Attention Makes Long-Context Prefill Up to 11.3x
Faster", MarkTechPost) measures on NIAH, RepoBench-P, 2WikiMultihopQA,
MultiNews and BioDEX with Qwen3-1.7B (section "How does TokenGate perform on
benchmarks?").  None of that data or those weights exist here, so these
generators stand in for them: a long document followed by a short question,
a few planted "needle" tokens that the gate should prefer, and N(0, 1)
post-RoPE Q/K/V drawn directly at the kept shape.

Every tensor comes from its own counter-seeded numpy PCG64 stream,
``default_rng(SeedSequence([seed, stream]))``, so a tensor's values do not
depend on which other tensors a caller asks for.  Values are drawn in float32
and rounded to bfloat16 with torch on the CPU (round to nearest even).

Nothing here scores, selects, compacts or attends: the one piece of algebra is
the needle direction ``u = normalize(W1^T w2)``, which only shapes the input.
"""

from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

import numpy as np
import torch

# Stream ids of the counter-seeded generators.
_S_META = 0
_S_NEEDLE = 1
_S_HIDDEN = 2
_S_GATE = 3
_S_LAYER0 = 10
_S_QKV0 = 50
_S_DENSE = 99


@dataclass(frozen=True)
class WorkloadSpec:
    """Shape and value recipe of one workload.

    ``prompts`` lists fixed (document length, question length) pairs; when it
    is empty, ``ragged`` draws them.  ``budget_div`` gives each prompt's
    document budget as ``doc // div`` when ``budgets`` is empty.
    """

    name: str
    dtype: str  # "f32" or "bf16"
    D: int
    F: int
    Hq: int
    Hkv: int
    d: int
    tau: float
    layers: int
    needles_per_prompt: int
    prompts: Tuple[Tuple[int, int], ...] = ()
    budgets: Tuple[int, ...] = ()
    ragged_B: int = 0
    ragged_doc: Tuple[int, int] = (0, 0)
    ragged_q: Tuple[int, int] = (0, 0)
    ragged_divs: Tuple[int, ...] = ()
    dense_comparator: bool = False
    b2: float = 0.0
    rope_theta: float = 1e6  # rotary base of the Qwen3 family
    mlp_mult: int = 3        # MLP width I = mlp_mult * D (6144 for hidden 2048)
    norm_eps: float = 1e-6   # RMSNorm eps of the Qwen3 family


# The five workloads of the gated-prefill benchmark, plus small extra parity
# cases.  Qwen3-1.7B gate-layer shapes: hidden 2048, 16 query / 8 KV heads,
# head_dim 128; the gate is 2048 -> 256 -> 1.
CONFIGS: List[WorkloadSpec] = [
    WorkloadSpec(
        name="tiny_fp32_512", dtype="f32", D=256, F=64, Hq=4, Hkv=2, d=64,
        tau=1.1, layers=1, needles_per_prompt=8,
        prompts=((448, 64),), budgets=(128,)),
    WorkloadSpec(
        name="qwen3_1p7b_16k", dtype="bf16", D=2048, F=256, Hq=16, Hkv=8,
        d=128, tau=1.15, layers=1, needles_per_prompt=32,
        prompts=((16128, 256),), budgets=(2048,)),
    WorkloadSpec(
        name="qwen3_1p7b_32k", dtype="bf16", D=2048, F=256, Hq=16, Hkv=8,
        d=128, tau=1.15, layers=1, needles_per_prompt=32,
        prompts=((32512, 256),), budgets=(4096,), dense_comparator=True),
    WorkloadSpec(
        name="qwen3_1p7b_128k", dtype="bf16", D=2048, F=256, Hq=16, Hkv=8,
        d=128, tau=1.15, layers=4, needles_per_prompt=32,
        prompts=((130816, 256),), budgets=(8192,)),
    WorkloadSpec(
        name="ragged_8x_4k_32k", dtype="bf16", D=2048, F=256, Hq=16, Hkv=8,
        d=128, tau=1.15, layers=1, needles_per_prompt=4,
        ragged_B=8, ragged_doc=(4096, 32768), ragged_q=(64, 512),
        ragged_divs=(4, 8, 16)),
]

EXTRA: List[WorkloadSpec] = [
    # Ragged batch at the tiny shapes, fp32.
    WorkloadSpec(
        name="ragged_tiny_fp32", dtype="f32", D=256, F=64, Hq=4, Hkv=2, d=64,
        tau=1.1, layers=1, needles_per_prompt=2,
        ragged_B=5, ragged_doc=(1, 700), ragged_q=(1, 90),
        ragged_divs=(4, 8, 16)),
    # Ragged batch at the Qwen3-1.7B shapes, short prompts, bf16.
    WorkloadSpec(
        name="ragged_small_bf16", dtype="bf16", D=2048, F=256, Hq=16, Hkv=8,
        d=128, tau=1.15, layers=1, needles_per_prompt=4,
        ragged_B=4, ragged_doc=(200, 1800), ragged_q=(16, 300),
        ragged_divs=(4, 8, 16)),
    # Tiny shapes with b2 != 0.
    WorkloadSpec(
        name="tiny_fp32_b2", dtype="f32", D=256, F=64, Hq=4, Hkv=2, d=64,
        tau=1.1, layers=1, needles_per_prompt=8,
        prompts=((448, 64),), budgets=(128,), b2=0.5),
]


def spec(which) -> WorkloadSpec:
    """A spec by benchmark index (0..4) or by name."""
    if isinstance(which, WorkloadSpec):
        return which
    if isinstance(which, int):
        return CONFIGS[which]
    for s in CONFIGS + EXTRA:
        if s.name == which:
            return s
    raise KeyError(which)


def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(seed), int(stream)]))


def _torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def _round(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(_torch_dtype(dtype))


@dataclass
class Workload:
    """One batch of synthetic gate-layer inputs (torch CPU tensors).

    Prompts are packed back to back; prompt b owns tokens
    ``[cu_seqlens[b], cu_seqlens[b+1])`` and its document is the
    prompt-relative span ``[doc_begin[b], doc_end[b])``; the question follows
    the document.  Positions restart at 0 in every prompt.
    """

    spec: WorkloadSpec
    seed: int
    cu_seqlens: np.ndarray  # int32 [B+1]
    doc_begin: np.ndarray  # int32 [B], prompt-relative
    doc_end: np.ndarray  # int32 [B], prompt-relative
    budget: np.ndarray  # int32 [B], document-token budget
    needles: np.ndarray  # int64, global token indices of planted needles
    hidden: torch.Tensor  # [T, D] spec dtype
    W1: torch.Tensor  # [F, D] spec dtype
    b1: torch.Tensor  # [F] float32
    w2: torch.Tensor  # [F] float32
    b2: float

    @property
    def B(self) -> int:
        return int(self.cu_seqlens.shape[0] - 1)

    @property
    def T(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def dtype(self) -> torch.dtype:
        return _torch_dtype(self.spec.dtype)

    def positions(self) -> np.ndarray:
        """Prompt-relative position of every token, int32 [T]."""
        pos = np.empty(self.T, dtype=np.int32)
        for b in range(self.B):
            lo, hi = int(self.cu_seqlens[b]), int(self.cu_seqlens[b + 1])
            pos[lo:hi] = np.arange(hi - lo, dtype=np.int32)
        return pos


def _prompt_table(s: WorkloadSpec, seed: int):
    if s.prompts:
        docs = np.array([p[0] for p in s.prompts], dtype=np.int64)
        qs = np.array([p[1] for p in s.prompts], dtype=np.int64)
        budgets = np.array(s.budgets, dtype=np.int64)
        return docs, qs, budgets
    g = _rng(seed, _S_META)
    docs = g.integers(s.ragged_doc[0], s.ragged_doc[1], size=s.ragged_B, endpoint=True)
    qs = g.integers(s.ragged_q[0], s.ragged_q[1], size=s.ragged_B, endpoint=True)
    divs = g.choice(np.array(s.ragged_divs, dtype=np.int64), size=s.ragged_B)
    budgets = docs // divs
    return docs.astype(np.int64), qs.astype(np.int64), budgets.astype(np.int64)


def make_workload(which, seed: int = 0, with_hidden: bool = True) -> Workload:
    """Draw the gate-layer inputs of a workload.

    ``with_hidden=False`` skips the [T, D] hidden states (metadata and gate
    weights only), for callers that need shapes alone.
    """
    s = spec(which)
    docs, qs, budgets = _prompt_table(s, seed)
    B = len(docs)
    lens = docs + qs
    cu = np.zeros(B + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lens)
    T = int(cu[-1])

    # Needle positions: without replacement inside each document.
    gn = _rng(seed, _S_NEEDLE)
    needles = []
    for b in range(B):
        n = min(s.needles_per_prompt, int(docs[b]))
        if n > 0:
            rel = np.sort(gn.choice(int(docs[b]), size=n, replace=False))
            needles.append(cu[b] + rel)
    needles = np.concatenate(needles).astype(np.int64) if needles else np.zeros(0, np.int64)

    # Gate weights: W1 ~ N(0, 1/D), b1 ~ N(0, 0.1^2), w2 ~ N(0, 1/F).
    gw = _rng(seed, _S_GATE)
    W1f = gw.standard_normal((s.F, s.D), dtype=np.float32) * np.float32(1.0 / np.sqrt(s.D))
    b1 = (gw.standard_normal(s.F, dtype=np.float32) * np.float32(0.1)).astype(np.float32)
    w2 = (gw.standard_normal(s.F, dtype=np.float32) * np.float32(1.0 / np.sqrt(s.F))).astype(np.float32)
    W1 = _round(W1f, s.dtype)

    if with_hidden:
        gh = _rng(seed, _S_HIDDEN)
        h = gh.standard_normal((T, s.D), dtype=np.float32)
        if needles.size:
            # Planted needles: +3 sigma along the gate's first-order direction,
            # taken from the rounded weights.
            u = W1.to(torch.float64).numpy().T @ w2.astype(np.float64)
            u /= np.linalg.norm(u)
            h[needles] = (h[needles].astype(np.float64) + 3.0 * u[None, :]).astype(np.float32)
        hidden = _round(h, s.dtype)
        del h
    else:
        hidden = torch.empty((0, s.D), dtype=_torch_dtype(s.dtype))

    return Workload(
        spec=s, seed=seed,
        cu_seqlens=cu.astype(np.int32),
        doc_begin=np.zeros(B, dtype=np.int32),
        doc_end=docs.astype(np.int32),
        budget=budgets.astype(np.int32),
        needles=needles,
        hidden=hidden,
        W1=W1,
        b1=torch.from_numpy(b1),
        w2=torch.from_numpy(w2),
        b2=float(s.b2),
    )


def attention_inputs(which, layer: int, n_tokens: int, seed: int = 0):
    """Inputs of gated attention layer ``layer`` over ``n_tokens`` kept tokens.

    Returns (q [n, Hq, d], k [n, Hkv, d], v [n, Hkv, d], gain [Hq] float32).
    q/k/v are N(0, 1) "post-RoPE" values in the spec dtype; the per-head gain
    is U(0.5, 2).
    """
    s = spec(which)
    g = _rng(seed, _S_LAYER0 + int(layer))
    gain = g.uniform(0.5, 2.0, size=s.Hq).astype(np.float32)
    q = g.standard_normal((n_tokens, s.Hq, s.d), dtype=np.float32)
    k = g.standard_normal((n_tokens, s.Hkv, s.d), dtype=np.float32)
    v = g.standard_normal((n_tokens, s.Hkv, s.d), dtype=np.float32)
    return _round(q, s.dtype), _round(k, s.dtype), _round(v, s.dtype), torch.from_numpy(gain)


def qkv_weights(which, layer: int, seed: int = 0) -> torch.Tensor:
    """Fused q/k/v projection weight of pruned layer ``layer``.

    W_qkv [(Hq + 2 Hkv) d, D] in the spec dtype, rows: the q heads, then the
    k heads, then the v heads; entries N(0, 1/D), so projected values of
    N(0, 1) rows are about N(0, 1).
    """
    s = spec(which)
    g = _rng(seed, _S_QKV0 + int(layer))
    n = (s.Hq + 2 * s.Hkv) * s.d
    w = g.standard_normal((n, s.D), dtype=np.float32) * np.float32(1.0 / np.sqrt(s.D))
    return _round(w, s.dtype)


def layer_weights(which, layer: int, seed: int = 0) -> dict:
    """Weights of pruned layer ``layer`` besides W_qkv (``qkv_weights``).

    Pre-norm layer of the Qwen3 family: ``w_in`` and ``w_post`` the two
    RMSNorm weights [D] (float32, U(0.5, 1.5)); ``W_o`` [D, Hq d],
    ``W_gate`` and ``W_up`` [I, D], ``W_down`` [D, I] in the spec dtype,
    entries N(0, 1/fan_in).
    """
    s = spec(which)
    g = _rng(seed, _S_QKV0 + 20 + int(layer))
    D, I, HD = s.D, s.mlp_mult * s.D, s.Hq * s.d

    def w(rows, cols):
        return _round(g.standard_normal((rows, cols), dtype=np.float32) * np.float32(1.0 / np.sqrt(cols)), s.dtype)

    w_in = torch.from_numpy(g.uniform(0.5, 1.5, D).astype(np.float32))
    w_post = torch.from_numpy(g.uniform(0.5, 1.5, D).astype(np.float32))
    return {"w_in": w_in, "W_o": w(D, HD), "w_post": w_post, "W_gate": w(I, D), "W_up": w(I, D),
            "W_down": w(D, I)}


def dense_attention_inputs(which, n_tokens: int, seed: int = 0):
    """q/k/v over all ``n_tokens`` prompt tokens for the full-length causal
    attention that un-pruned prefill would run at the gate layer."""
    s = spec(which)
    g = _rng(seed, _S_DENSE)
    q = g.standard_normal((n_tokens, s.Hq, s.d), dtype=np.float32)
    k = g.standard_normal((n_tokens, s.Hkv, s.d), dtype=np.float32)
    v = g.standard_normal((n_tokens, s.Hkv, s.d), dtype=np.float32)
    return _round(q, s.dtype), _round(k, s.dtype), _round(v, s.dtype)


def with_overrides(which, **kw) -> WorkloadSpec:
    """A copy of a spec with some fields replaced (for extra test shapes)."""
    return dataclasses.replace(spec(which), **kw)
