"""Selection variants on the GPU: random-K selection (top-K over the
caller's uniform keys) and random document budgets (host sampler), against
the oracle.  Selection is a discontinuous decision, so flags and the
compacted rows are compared bit for bit on the same fp32 inputs (the keys,
and for the compaction the GPU's own gate scores, as for the top-K step).
"""

import numpy as np
import pytest
import torch

import learned_token_pruning_score_amd as tg
import oracle
import synth

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _note(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("name,quantize", [("ragged_8x_4k_32k", False), ("qwen3_1p7b_128k", False),
                                           ("ragged_8x_4k_32k", True)])
def test_random_k_flags(name, quantize):
    _note(f"[random-K] {name} quantize={quantize}")
    w = synth.make_workload(name, seed=6, with_hidden=False)
    T = w.T
    g = torch.Generator().manual_seed(6)
    keys = torch.rand(T, generator=g)
    if quantize:  # heavy ties: 64 distinct values
        keys = torch.floor(keys * 64) / 64
    ws = torch.empty(max(16, tg.tg_select_topk_workspace(w.B, T)), dtype=torch.uint8, device=DEV)
    keep = tg.tg_select_topk(keys.to(DEV), torch.from_numpy(w.cu_seqlens).to(DEV), torch.from_numpy(w.doc_begin).to(DEV),
                             torch.from_numpy(w.doc_end).to(DEV), torch.from_numpy(w.budget).to(DEV), workspace=ws)
    torch.cuda.synchronize()
    ref = oracle.random_k_keep(keys.numpy(), w.cu_seqlens, w.doc_begin, w.doc_end, w.budget)
    assert np.array_equal(keep.cpu().numpy().astype(bool), ref.astype(bool))


def test_random_k_pipeline_mode_keeps_score_bias():
    name = "ragged_small_bf16"
    _note(f"[random-K pipeline] {name}")
    w = synth.make_workload(name, seed=7)
    s = w.spec
    gp = tg.GatedPrefill(w.cu_seqlens, w.doc_begin, w.doc_end, w.budget, s.D, w.dtype)
    keys = torch.rand(w.T, generator=torch.Generator().manual_seed(7))
    hidden = w.hidden.to(DEV)
    gp.gate_and_select(hidden, w.W1.to(DEV), w.b1.to(DEV), w.w2.to(DEV), w.b2, rand_keys=keys.to(DEV))
    torch.cuda.synchronize()
    keep = gp.keep.cpu().numpy()
    ref_keep = oracle.random_k_keep(keys.numpy(), w.cu_seqlens, w.doc_begin, w.doc_end, w.budget)
    assert np.array_equal(keep.astype(bool), ref_keep.astype(bool))
    scores = gp.scores.cpu().numpy()
    hk, pk, bk, ik = oracle.compact(w.hidden.view(torch.int16).numpy(), w.positions(), scores, keep,
                                    w.cu_seqlens, w.doc_begin, w.doc_end)
    assert np.array_equal(gp.hidden_k.cpu().view(torch.int16).numpy(), hk)
    assert np.array_equal(gp.pos_k.cpu().numpy(), pk)
    assert np.array_equal(gp.bias_s.cpu().numpy().view(np.uint32), bk.view(np.uint32))
    assert np.array_equal(gp.kept_idx.cpu().numpy(), ik)


def test_random_budget_step():
    """Budgets from the host sampler drive a gated prefill: the kept count of
    every prompt is its sampled budget plus its question."""
    name = "ragged_8x_4k_32k"
    _note(f"[random budget] {name}")
    w = synth.make_workload(name, seed=8)
    s = w.spec
    u = np.random.default_rng(8).random(w.B).astype(np.float32)
    bud = tg.tg_sample_budgets(w.doc_begin, w.doc_end, u, 0.05, 0.5)
    assert np.array_equal(bud, oracle.sample_budgets(w.doc_begin, w.doc_end, u.astype(np.float64),
                                                     np.float32(0.05), np.float32(0.5)))
    gp = tg.GatedPrefill(w.cu_seqlens, w.doc_begin, w.doc_end, bud, s.D, w.dtype)
    gp.gate_and_select(w.hidden.to(DEV), w.W1.to(DEV), w.b1.to(DEV), w.w2.to(DEV), w.b2)
    torch.cuda.synchronize()
    keep = gp.keep.cpu().numpy()
    ref = oracle.select_topk(gp.scores.cpu().numpy(), w.cu_seqlens, w.doc_begin, w.doc_end, bud)
    assert np.array_equal(keep.astype(bool), ref.astype(bool))
    cu = w.cu_seqlens
    for b in range(w.B):
        doc = slice(cu[b] + w.doc_begin[b], cu[b] + w.doc_end[b])
        assert int(keep[doc].sum()) == int(bud[b])
        assert int(keep[cu[b]:cu[b + 1]].sum()) == int(bud[b]) + int(cu[b + 1] - cu[b] - (w.doc_end[b] - w.doc_begin[b]))
