"""The gated prefill captured in a HIP graph and replayed gives the eager
results, replay after replay, with eager work and synchronisations between
the replays (no memset nodes: workspaces are cleared by kernels)."""

import numpy as np
import pytest
import torch

import learned_token_pruning_score_amd as tg
import synth

pytestmark = pytest.mark.gpu


# a small batch (one-launch top-K, key-split attention) and a 113k-token
# ragged batch (four-kernel top-K, 256-row attention)
@pytest.mark.parametrize("name", ["ragged_small_bf16", "ragged_8x_4k_32k"])
def test_graph_replay_matches_eager(name):
    dev = "cuda"
    w = synth.make_workload(name, seed=3)
    s = w.spec
    gp = tg.GatedPrefill(w.cu_seqlens, w.doc_begin, w.doc_end, w.budget, s.D, w.dtype)
    hidden, W1, b1, w2 = (t.to(dev) for t in (w.hidden, w.W1, w.b1, w.w2))
    q, k, v, gain = (t.to(dev) for t in synth.attention_inputs(s, 0, gp.Kt, seed=3))
    out = torch.empty((gp.Kt, s.Hq, s.d), dtype=w.dtype, device=dev)

    def step():
        gp.gate_and_select(hidden, W1, b1, w2, w.b2)
        gp.attend(q, k, v, gain, s.tau, out=out)

    step()
    torch.cuda.synchronize()
    ref = [gp.scores.clone(), gp.keep.clone(), gp.hidden_k.clone(), gp.bias_s.clone(), out.clone()]

    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        step()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=cap):
            step()
    torch.cuda.synchronize()
    for rep in range(4):
        for t in (gp.scores, gp.hidden_k, gp.bias_s, out):  # scribble over the outputs
            t.fill_(7)
        gp.keep.fill_(3)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [gp.scores, gp.keep, gp.hidden_k, gp.bias_s, out]
        for a, b in zip(got, ref):
            assert torch.equal(a, b), f"replay {rep} differs"
        # eager work between replays
        step()
        torch.cuda.synchronize()
        assert torch.equal(out, ref[4])
