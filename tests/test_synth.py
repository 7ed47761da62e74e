"""The seeded input generator: deterministic, shaped like the five benchmark
workloads, needles inside documents, budgets as the configs state them."""

import numpy as np
import torch

import synth


def test_shapes_of_benchmark_workloads():
    want_T = [512, 16384, 32768, 131072]
    want_budget = [128, 2048, 4096, 8192]
    for i in range(4):
        w = synth.make_workload(i, seed=0, with_hidden=False)
        assert w.T == want_T[i] and w.B == 1
        assert int(w.budget[0]) == want_budget[i]
        assert int(w.doc_end[0]) == want_T[i] - (64 if i == 0 else 256)
    w = synth.make_workload(4, seed=0, with_hidden=False)
    assert w.B == 8
    docs = w.doc_end - w.doc_begin
    qs = np.diff(w.cu_seqlens) - docs
    assert np.all((docs >= 4096) & (docs <= 32768))
    assert np.all((qs >= 64) & (qs <= 512))
    ratios = docs / np.maximum(w.budget, 1)
    for d, b in zip(docs, w.budget):
        assert b in (d // 4, d // 8, d // 16)


def test_deterministic_and_stream_independent():
    a = synth.make_workload(0, seed=0)
    b = synth.make_workload(0, seed=0)
    assert torch.equal(a.hidden, b.hidden) and torch.equal(a.W1, b.W1)
    c = synth.make_workload(0, seed=1)
    assert not torch.equal(a.hidden, c.hidden)
    q1, k1, v1, g1 = synth.attention_inputs(0, 0, 192)
    q2, k2, v2, g2 = synth.attention_inputs(0, 0, 192)
    assert torch.equal(q1, q2) and torch.equal(g1, g2)
    q3, *_ = synth.attention_inputs(0, 1, 192)
    assert not torch.equal(q1, q3)
    assert a.hidden.dtype == torch.float32
    assert synth.make_workload("ragged_small_bf16").hidden.dtype == torch.bfloat16


def test_needles_inside_documents():
    w = synth.make_workload("ragged_small_bf16", seed=0)
    assert len(np.unique(w.needles)) == len(w.needles)
    for t in w.needles:
        b = int(np.searchsorted(w.cu_seqlens, t, side="right") - 1)
        rel = t - w.cu_seqlens[b]
        assert w.doc_begin[b] <= rel < w.doc_end[b]


def test_gain_range_and_value_distribution():
    q, k, v, g = synth.attention_inputs(1, 0, 2304)
    assert q.shape == (2304, 16, 128) and k.shape == (2304, 8, 128)
    assert q.dtype == torch.bfloat16
    assert float(g.min()) >= 0.5 and float(g.max()) <= 2.0
    assert abs(float(q.float().std()) - 1.0) < 0.01
