"""Gated-prefill throughput on one MI355X.

One step = one pass of the whole gated prefill over one synthetic batch:
gate MLP score of every token -> per-prompt top-K over the document ->
stable compaction of kept rows, positions and biases -> the stacked
token-gated causal GQA attention layers over the kept tokens.  Inputs are
resident in HBM before the timed region; every step re-runs all of it.  The
timed steps replay the step captured in a HIP graph (one launch per step);
the same step launched eagerly is timed too, with per-phase events, for the
per-kernel figures.  After the timed region, single steps each preceded by a
1 GiB write that evicts L2 and the last-level cache give the cold-cache
median (``cold_cache``), reported beside the back-to-back figure.

Prints one JSON line (stdout).  Progress goes to stderr.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="qwen3_1p7b_128k")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-phase-events", action="store_true",
                   help="time only whole steps (no per-phase events inside the timed region)")
    p.add_argument("--copy-probe-mib", type=int, default=0,
                   help="before the timed region, copy a buffer of this many MiB on the device "
                        "(a kernel of known traffic for calibrating memory counters)")
    p.add_argument("--eager-only", action="store_true",
                   help="time eager launches only (by default the timed steps are replays of the "
                        "step captured in a HIP graph, and the eager loop is reported beside them)")
    p.add_argument("--no-reference-points", action="store_true",
                   help="skip the reference timings taken after the timed region")
    p.add_argument("--flushed-reps", type=int, default=20,
                   help="after the timed region, time this many single steps, each after a 1 GiB "
                        "write that evicts L2 and the last-level cache, and report their median "
                        "beside the back-to-back figure (0: skip)")
    return p.parse_args()


def algorithmic_work(w, Kt, cu_kept):
    s = w.spec
    e = 2 if s.dtype == "bf16" else 4
    T, D, F = w.T, s.D, s.F
    lens = np.diff(cu_kept).astype(np.float64)
    attn_flop = 2.0 * s.d * s.Hq * float(np.sum(lens * (lens + 1)))
    return {
        "gate_bytes": T * D * e + F * D * e + 4 * T,
        "gate_flop": 2.0 * T * D * F,
        "select_bytes": 5 * T,
        "compact_bytes": T + 2 * Kt * D * e + 16 * Kt,
        "attn_flop_per_layer": attn_flop,
        "attn_bytes_per_layer": (2 * s.Hq + 2 * s.Hkv) * s.d * Kt * e,
    }


TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "gated_prefill_128k_hbm_traffic.md")


def measured_traffic(kernel, source):
    """HBM bytes per launch of `kernel` from the committed FETCH_SIZE /
    WRITE_SIZE summary, or None when the summary is missing or was taken on
    a different version of the kernel's source."""
    import hashlib
    try:
        with open(source, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
        with open(TRAFFIC_SUMMARY) as f:
            lines = f.read().splitlines()
    except OSError:
        return None
    for line in lines:
        if not line.startswith(kernel + " "):
            continue
        fields = dict(kv.split("=", 1) for kv in line[len(kernel) + 1:].split() if "=" in kv)
        if fields.get("source_sha256") == sha:
            return float(fields["traffic_bytes_per_launch"])
    return None


def time_launches(fn, stream, reps=5, n=5, before=None):
    """Median over `reps` of the mean time of `n` back-to-back calls of fn,
    from HIP events on `stream`; `before` runs untimed ahead of each rep."""
    import torch
    ts = []
    for _ in range(reps):
        if before is not None:
            before()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) / n)
    return float(np.median(ts))


def reference_points(tg, w, gp, layers, outs, hidden, W1, b1, w2, stream, dev):
    """Reference timings outside the timed region (each a median of event-timed
    repetitions on the launch stream):
      * the key-bias cost: the same attention launch with the bias and the
        temperature switched off (gain = NULL, tau = 1), as a ratio;
      * the dense comparator: full-length causal GQA attention (no pruning, no
        bias) at 32768 tokens with the same head shapes;
      * gate, top-K, compaction and attention launches, each after a 1 GiB
        write that evicts L2 and the last-level cache (the timed step runs
        them back to back);
      * a whole pruned layer on the kept rows, beside the step (seeded
        weights of the layer's shapes): the rotary table of the kept rows'
        positions, and per layer RMSNorm, the fused q/k/v projection with the
        rotary embedding, the gated attention, the output projection added to
        the residual, RMSNorm, the SwiGLU gate/up projection and the down
        projection added to the residual; each kernel timed alone too;
      * the backward of one gated attention layer (dq, dk, dv and the bias,
        gain and temperature gradients) on the step's kept rows, and the
        gate MLP's backward from the kept rows' bias gradient;
      * one decode step over the kept rows as a kept-only KV cache (one new
        query per prompt), with the bytes of cached keys and values it reads,
        and the scatter of the kept k, v and bias into such a cache;
      * one GPU's share of an 8-way split (KV heads a multiple of 8): the
        gate on an eighth of the tokens and the attention of an eighth of the
        KV heads (with their query heads) over all the kept rows;
      * what the chip reaches here on plain library work: a bf16 GEMM of
        8192^3 and a 1 GiB device copy."""
    import torch
    s = w.spec
    q, k, v, gain = layers[0]
    out = outs[0]
    gated = lambda: tg.tg_gated_attn_fwd(q, k, v, gp.bias_s, gain, s.tau, gp.cu_kept,  # noqa: E731
                                         gp.max_kept_len, out=out)
    plain = lambda: tg.tg_gated_attn_fwd(q, k, v, None, None, 1.0, gp.cu_kept,  # noqa: E731
                                         gp.max_kept_len, out=out)
    for _ in range(3):
        gated()
        plain()
    # alternate the two so that both see the same clock and temperature
    tp, tgt = [], []
    for _ in range(7):
        tp.append(time_launches(plain, stream, reps=1, n=5))
        tgt.append(time_launches(gated, stream, reps=1, n=5))
    t_plain, t_gated = float(np.median(tp)), float(np.median(tgt))
    work = algorithmic_work(w, gp.Kt, gp.cu_kept_h)
    r = {"attn_gated_us": t_gated * 1e3, "attn_no_bias_us": t_plain * 1e3,
         "key_bias_cost_ratio": t_gated / t_plain}

    import synth
    Kt, D, HD = gp.Kt, s.D, s.Hq * s.d
    Wqkv = synth.qkv_weights(s, 0, seed=0).to(dev)
    lw = {k_: v_.to(dev) for k_, v_ in synth.layer_weights(s, 0, seed=0).items()}
    I = lw["W_gate"].shape[0]
    nq = (s.Hq + 2 * s.Hkv) * s.d
    mk = lambda *shape: torch.empty(shape, dtype=Wqkv.dtype, device=dev)  # noqa: E731
    xk, xn, qkv_buf, att, act = mk(Kt, D), mk(Kt, D), mk(Kt, nq), mk(Kt, HD), mk(Kt, I)
    xk.copy_(gp.hidden_k)
    xn.copy_(gp.hidden_k)
    att.normal_()
    act.normal_()
    rope = lambda: gp.rope(s.d, s.rope_theta)  # noqa: E731
    rope()
    r["rope_table_us"] = time_launches(rope, stream, reps=7, n=5) * 1e3
    parts = {
        "rms_norm": (lambda: tg.tg_rms_norm(xk, lw["w_in"], s.norm_eps, out=xn), 0.0),
        "qkv_rope": (lambda: gp.project_qkv(Wqkv, s.Hq, s.Hkv, s.d, out=qkv_buf, x=xn), 2.0 * Kt * D * nq),
        "o_proj": (lambda: tg.tg_linear_residual(att, lw["W_o"], xk, out=xn), 2.0 * Kt * HD * D),
        "swiglu": (lambda: tg.tg_swiglu(xn, lw["W_gate"], lw["W_up"], out=act), 4.0 * Kt * D * I),
        "down_proj": (lambda: tg.tg_linear_residual(act, lw["W_down"], xk, out=xn), 2.0 * Kt * I * D),
    }
    for name, (fn, flop) in parts.items():
        fn()
        t = time_launches(fn, stream, reps=7, n=5)
        r[f"{name}_us"] = t * 1e3
        if flop:
            r[f"{name}_TFLOPs"] = flop / (t / 1e3) / 1e12
    r["rms_norm_GBps"] = 2.0 * Kt * D * xk.element_size() / (r["rms_norm_us"] / 1e6) / 1e9
    layer = lambda: gp.pruned_layer(Wqkv, lw, s.Hq, s.Hkv, s.d, gain, s.tau, s.norm_eps, x=xk)  # noqa: E731
    layer()
    t = time_launches(layer, stream, reps=5, n=3)
    r["pruned_layer_us"] = t * 1e3
    r["pruned_layer_TFLOPs"] = (2.0 * Kt * D * (nq + HD + 3 * I) + work["attn_flop_per_layer"]) / (t / 1e3) / 1e12
    del Wqkv, lw, xk, xn, qkv_buf, att, act

    # backward of one gated attention layer (seeded dout), on the step's
    # kept rows: algorithmic work 2.5x the forward's (S, dP, dQ, dK, dV)
    lse0 = torch.empty((s.Hq, Kt), dtype=torch.float32, device=dev)
    out0, _ = tg.tg_gated_attn_fwd(q, k, v, gp.bias_s, gain, s.tau, gp.cu_kept, gp.max_kept_len, lse=lse0)
    dout = torch.randn(out0.shape, device=dev).to(out0.dtype)
    wsb = torch.empty(max(16, tg.tg_gated_attn_bwd_workspace(gp.B, Kt, s.Hq, s.Hkv, s.d, q.dtype,
                                                             gp.max_kept_len)),
                      dtype=torch.uint8, device=dev)
    grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v),
             torch.empty(Kt, dtype=torch.float32, device=dev), torch.empty(s.Hq, dtype=torch.float32, device=dev),
             torch.empty(1, dtype=torch.float32, device=dev))
    bwd = lambda: tg.tg_gated_attn_bwd(q, k, v, gp.bias_s, gain, s.tau, gp.cu_kept, gp.max_kept_len,  # noqa: E731
                                       out0, lse0, dout, workspace=wsb, grads=grads)
    bwd()
    t = time_launches(bwd, stream, reps=5, n=3)
    r["attn_bwd_us"] = t * 1e3
    r["attn_bwd_TFLOPs"] = 2.5 * work["attn_flop_per_layer"] / (t / 1e3) / 1e12
    del lse0, out0, dout, wsb, grads

    # one decode step of one layer over the kept-only cache (every kept row
    # of the step, one new query per prompt): HBM-bound, reads each cached
    # key and value once
    lens = torch.from_numpy(np.diff(gp.cu_kept_h).astype(np.int32)).to(dev)
    qd = torch.randn((gp.B, s.Hq, s.d), device=dev).to(q.dtype)
    wsd = torch.empty(max(16, tg.tg_decode_attn_workspace(gp.B, s.Hq, s.d, gp.max_kept_len)), dtype=torch.uint8,
                      device=dev)
    outd = torch.empty_like(qd)
    dec = lambda: tg.tg_decode_attn(qd, k, v, gp.bias_s, gain, s.tau, gp.cu_kept[:-1], lens,  # noqa: E731
                                    gp.max_kept_len, out=outd, workspace=wsd)
    dec()
    t = time_launches(dec, stream, reps=7, n=10)
    r["decode_step_us"] = t * 1e3
    r["decode_step_GBps"] = 2.0 * Kt * s.Hkv * s.d * q.element_size() / (t / 1e3) / 1e9
    del lens, qd, wsd, outd
    # the prefill's kept k, v and bias into a cache with room for 16 new
    # tokens per sequence (read and written once)
    startc = (torch.from_numpy(gp.cu_kept_h[:-1].astype(np.int64)) + 16 * torch.arange(gp.B)).to(torch.int32).to(dev)
    kcache = torch.empty((Kt + 16 * gp.B, s.Hkv, s.d), dtype=q.dtype, device=dev)
    vcache = torch.empty_like(kcache)
    bcache = torch.empty(Kt + 16 * gp.B, dtype=torch.float32, device=dev)
    scat = lambda: tg.tg_kv_scatter(k, v, gp.bias_s, gp.cu_kept, kcache, vcache, bcache, startc)  # noqa: E731
    scat()
    t = time_launches(scat, stream, reps=5, n=5)
    r["kv_scatter_us"] = t * 1e3
    r["kv_scatter_GBps"] = (4.0 * Kt * s.Hkv * s.d * q.element_size() + 8.0 * Kt) / (t / 1e3) / 1e9
    del startc, kcache, vcache, bcache

    # gate MLP backward from the kept rows' bias gradient
    dbias = torch.randn(Kt, device=dev)
    wsg = torch.empty(max(16, tg.tg_gate_bwd_workspace(Kt, s.D, s.F, hidden.dtype)), dtype=torch.uint8,
                      device=dev)
    gbwd = lambda: tg.tg_gate_bwd(  # noqa: E731
        gp.hidden_k, W1, b1, w2, dbias, gp.kept_idx, gp.cu_seqlens, gp.doc_begin, gp.doc_end, workspace=wsg)
    gbwd()
    t = time_launches(gbwd, stream, reps=5, n=3)
    r["gate_bwd_us"] = t * 1e3
    r["gate_bwd_TFLOPs"] = 6.0 * Kt * s.D * s.F / (t / 1e3) / 1e12
    del dbias, wsg

    # one GPU's share of an 8-way split of the step: the gate on an eighth of
    # the tokens (rows shard with no exchange) and the attention of an eighth
    # of the KV heads (heads shard with no exchange once the kept rows are
    # gathered)
    if s.Hkv % 8 == 0:
        grp = s.Hq // s.Hkv * (s.Hkv // 8)  # the query heads of one GPU's KV heads
        kv8 = s.Hkv // 8
        T8 = w.T // 8
        gate8 = lambda: tg.tg_gate_score(hidden[:T8], W1, b1, w2, w.b2, scores=gp.scores[:T8])  # noqa: E731
        gate8()
        t = time_launches(gate8, stream, reps=5, n=5)
        r["shard8_gate_us"] = t * 1e3
        r["shard8_gate_GBps"] = (T8 * s.D * hidden.element_size() + 4 * T8) / (t / 1e3) / 1e9
        o1 = torch.empty((gp.Kt, grp, s.d), dtype=q.dtype, device=dev)
        attn1 = lambda: tg.tg_gated_attn_fwd(q[:, :grp], k[:, :kv8], v[:, :kv8], gp.bias_s, gain[:grp], s.tau,  # noqa: E731
                                             gp.cu_kept, gp.max_kept_len, out=o1)
        attn1()
        t = time_launches(attn1, stream, reps=5, n=5)
        r["shard8_attn_us"] = t * 1e3
        r["shard8_attn_TFLOPs"] = work["attn_flop_per_layer"] / 8 / (t / 1e3) / 1e12
        del o1

    flush_buf = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    flush = lambda: flush_buf.fill_(1)  # noqa: E731
    gate = lambda: tg.tg_gate_score(hidden, W1, b1, w2, w.b2, scores=gp.scores)  # noqa: E731
    sel = lambda: tg.tg_select_topk(gp.scores, gp.cu_seqlens, gp.doc_begin, gp.doc_end, gp.budget,  # noqa: E731
                                    keep=gp.keep, workspace=gp.ws_select)
    cmp = lambda: tg.tg_compact(hidden, None, gp.scores, gp.keep, gp.cu_seqlens, gp.doc_begin,  # noqa: E731
                                gp.doc_end, gp.Kt, out=(gp.hidden_k, gp.pos_k, gp.bias_s, gp.kept_idx),
                                workspace=gp.ws_compact)
    r["gate_us_after_cache_flush"] = time_launches(gate, stream, reps=7, n=1, before=flush) * 1e3
    r["select_us_after_cache_flush"] = time_launches(sel, stream, reps=7, n=1, before=flush) * 1e3
    r["compact_us_after_cache_flush"] = time_launches(cmp, stream, reps=7, n=1, before=flush) * 1e3
    r["attn_us_after_cache_flush"] = time_launches(gated, stream, reps=7, n=1, before=flush) * 1e3
    del flush_buf

    if s.dtype == "bf16":
        N = 32768
        g = torch.Generator(device="cpu").manual_seed(1)
        dq = torch.randn((N, s.Hq, s.d), generator=g).to(torch.bfloat16).to(dev)
        dk = torch.randn((N, s.Hkv, s.d), generator=g).to(torch.bfloat16).to(dev)
        dv = torch.randn((N, s.Hkv, s.d), generator=g).to(torch.bfloat16).to(dev)
        do = torch.empty_like(dq)
        cu = torch.tensor([0, N], dtype=torch.int32, device=dev)
        dense = lambda: tg.tg_gated_attn_fwd(dq, dk, dv, None, None, 1.0, cu, N, out=do)  # noqa: E731
        dense()
        t = time_launches(dense, stream, reps=3, n=3)
        flop = 2.0 * s.d * s.Hq * N * (N + 1)
        r["dense_causal_32k_us"] = t * 1e3
        r["dense_causal_32k_TFLOPs"] = flop / (t / 1e3) / 1e12
        del dq, dk, dv, do

        M = 8192
        A = torch.randn((M, M), device=dev, dtype=torch.bfloat16)
        B = torch.randn((M, M), device=dev, dtype=torch.bfloat16)
        C = torch.empty((M, M), device=dev, dtype=torch.bfloat16)
        mm = lambda: torch.matmul(A, B, out=C)  # noqa: E731
        mm()
        t = time_launches(mm, stream, reps=3, n=5)
        r["library_bf16_gemm_8192_TFLOPs"] = 2.0 * M ** 3 / (t / 1e3) / 1e12
        del A, B, C
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    cp = lambda: dst.copy_(src)  # noqa: E731
    cp()
    t = time_launches(cp, stream, reps=3, n=5)
    r["library_copy_1GiB_GBps"] = 2.0 * src.numel() / (t / 1e3) / 1e9
    del src, dst
    torch.cuda.synchronize()
    return r


def attn_kernel_name(dtype, Hq, d, Kt, n_cu):
    """The attention kernel a launch of this shape runs (the library's rule:
    fp32 on the vector-ALU path; bf16 on the key-split kernel when the
    256-row query tiles number fewer than twice the CUs, else the 256-row
    kernel)."""
    import torch
    if dtype == torch.float32:
        return f"attn_f32_kernel<{d}>"
    if Hq * ((Kt + 255) // 256) < 2 * n_cu:
        return f"attn_bf16_ks_kernel<{d}>"
    return f"attn_bf16_kernel<{d}, 8>"


def cpu_baseline(w, q_layers, cu_kept, Kt):
    """The fp64 oracle on a bounded sample of the same workload, scaled to the
    whole step: gate, top-K and compaction on all tokens; attention for one
    KV group (Hq/Hkv query heads) of one layer over every kept row, scaled by
    the number of KV groups and layers."""
    import torch
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    s = w.spec
    f64 = lambda t: t.to(torch.float64).numpy()  # noqa: E731
    W1, b1, w2 = f64(w.W1), f64(w.b1), f64(w.w2)
    t0 = time.perf_counter()
    s_full = oracle.round_f32(oracle.gate_scores(f64(w.hidden), W1, b1, w2, w.b2))
    t_gate = time.perf_counter() - t0
    t0 = time.perf_counter()
    keep = oracle.select_topk(s_full, w.cu_seqlens, w.doc_begin, w.doc_end, w.budget)
    t_sel = time.perf_counter() - t0
    t0 = time.perf_counter()
    bits = w.hidden.view(torch.int16 if s.dtype == "bf16" else torch.int32).numpy()
    _, _, bias, _ = oracle.compact(bits, w.positions(), s_full, keep, w.cu_seqlens, w.doc_begin,
                                   w.doc_end)
    t_cmp = time.perf_counter() - t0
    q, k, v, gain = q_layers[0]
    grp = s.Hq // s.Hkv
    t0 = time.perf_counter()
    oracle.gated_attention(f64(q[:, :grp]), f64(k[:, :1]), f64(v[:, :1]), bias,
                           f64(gain[:grp]), s.tau, cu_kept)
    t_attn = (time.perf_counter() - t0) * s.Hkv * s.layers
    total = t_gate + t_sel + t_cmp + t_attn
    return {
        "value": w.T / total, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
        "sample": (f"fp64 numpy oracle on the same workload: gate, top-K and compaction on all "
                   f"{w.T} tokens; attention for 1 of {s.Hkv} KV groups of 1 of {s.layers} "
                   f"layers over all {Kt} kept rows, scaled x{s.Hkv * s.layers}; estimated "
                   f"step {total:.1f} s"),
        "seconds": {"gate": t_gate, "select": t_sel, "compact": t_cmp, "attention": t_attn},
    }


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the gated prefill is measured on one MI355X "
              "and the library has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import learned_token_pruning_score_amd as tg

    if not torch.cuda.is_available():
        raise RuntimeError("bench.py needs a GPU")
    dev = "cuda:0"
    t_setup = time.perf_counter()
    w = synth.make_workload(args.workload, seed=0)
    s = w.spec
    gp = tg.GatedPrefill(w.cu_seqlens, w.doc_begin, w.doc_end, w.budget, s.D, w.dtype, device=dev)
    Kt = gp.Kt
    hidden, W1, b1, w2 = w.hidden.to(dev), w.W1.to(dev), w.b1.to(dev), w.w2.to(dev)
    layers_cpu = [synth.attention_inputs(s, l, Kt, seed=0) for l in range(s.layers)]
    layers = [tuple(t.to(dev) for t in L) for L in layers_cpu]
    outs = [torch.empty((Kt, s.Hq, s.d), dtype=w.dtype, device=dev) for _ in range(s.layers)]
    torch.cuda.synchronize()
    log(f"[bench] workload {s.name}: T={w.T} Kt={Kt} B={w.B} layers={s.layers} "
        f"setup {time.perf_counter() - t_setup:.1f}s")

    stream = torch.cuda.current_stream()
    phase_events = not args.no_phase_events
    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib * (1 << 20)
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.bitwise_not(src, out=dst)  # one elementwise kernel: reads n bytes, writes n bytes
        torch.cuda.synchronize()
        del src, dst
        log(f"[bench] copy probe: {args.copy_probe_mib} MiB")

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        tg.tg_gate_score(hidden, W1, b1, w2, w.b2, scores=gp.scores)
        if ev is not None:
            ev[1].record(stream)
        tg.tg_select_topk(gp.scores, gp.cu_seqlens, gp.doc_begin, gp.doc_end, gp.budget,
                          keep=gp.keep, workspace=gp.ws_select)
        if ev is not None:
            ev[2].record(stream)
        tg.tg_compact(hidden, None, gp.scores, gp.keep, gp.cu_seqlens, gp.doc_begin, gp.doc_end,
                      Kt, out=(gp.hidden_k, gp.pos_k, gp.bias_s, gp.kept_idx),
                      workspace=gp.ws_compact)
        if ev is not None:
            ev[3].record(stream)
        for l in range(s.layers):
            q, k, v, gain = layers[l]
            tg.tg_gated_attn_fwd(q, k, v, gp.bias_s, gain, s.tau, gp.cu_kept, gp.max_kept_len,
                                 out=outs[l])
            if ev is not None:
                ev[4 + l].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    n_ev = 4 + s.layers
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(args.steps)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        step(evs[i] if phase_events else None)
    end.record(stream)
    torch.cuda.synchronize()
    eager_ms = start.elapsed_time(end) / args.steps
    log(f"[bench] {args.steps} eager steps: {eager_ms:.4f} ms/step, "
        f"{w.T / (eager_ms / 1e3):.4g} tokens/s")

    graph_ms = None
    if not args.eager_only:
        # The timed steps: the same step captured once in a HIP graph and
        # replayed, one launch per step instead of one per kernel (the
        # kernels, inputs and buffers are the eager ones).
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        with torch.cuda.stream(cap):
            step()  # warm the capture stream
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=cap):
                step()
        torch.cuda.synchronize()
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        gs = torch.cuda.Event(enable_timing=True)
        ge = torch.cuda.Event(enable_timing=True)
        gs.record(stream)
        for _ in range(args.steps):
            g.replay()
        ge.record(stream)
        torch.cuda.synchronize()
        graph_ms = gs.elapsed_time(ge) / args.steps
        log(f"[bench] {args.steps} graph replays: {graph_ms:.4f} ms/step, "
            f"{w.T / (graph_ms / 1e3):.4g} tokens/s")
    ms_per_step = graph_ms if graph_ms is not None else eager_ms
    value = w.T / (ms_per_step / 1e3)

    # Cold-cache protocol: every rep writes 1 GiB (evicting L2 and the 256 MB
    # last-level cache), then one step runs between events; the median of the
    # reps is reported beside the back-to-back steps above (whose inputs stay
    # partly cache-resident from step to step).
    flushed = None
    if args.flushed_reps > 0:
        flush_buf = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        one = (lambda: g.replay()) if graph_ms is not None else (lambda: step())  # noqa: E731
        reps = []
        for _ in range(args.flushed_reps):
            flush_buf.fill_(1)
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            one()
            b.record(stream)
            torch.cuda.synchronize()
            reps.append(a.elapsed_time(b))
        del flush_buf
        med = float(np.median(reps))
        flushed = {"ms_per_step_median": med, "tokens_per_s": w.T / (med / 1e3),
                   "reps": args.flushed_reps, "min_ms": float(np.min(reps)),
                   "max_ms": float(np.max(reps)), "flush_bytes": 1 << 30,
                   "timing": "hip_graph_replay" if graph_ms is not None else "eager"}
        log(f"[bench] {args.flushed_reps} steps after a cache flush: median {med:.4f} ms/step, "
            f"{w.T / (med / 1e3):.4g} tokens/s")

    work = algorithmic_work(w, Kt, gp.cu_kept_h)
    phases = None
    roof = None
    if phase_events:
        def avg(i, j):
            return float(np.mean([evs[k][i].elapsed_time(evs[k][j]) for k in range(args.steps)]))
        gate_ms = avg(0, 1)
        sel_ms = avg(1, 2)
        cmp_ms = avg(2, 3)
        attn_ms = [avg(3 + l, 4 + l) for l in range(s.layers)]
        attn_avg = float(np.mean(attn_ms))
        sel_phase_ms = gate_ms + sel_ms + cmp_ms
        phases = {
            "gate_us": gate_ms * 1e3,
            "gate_GBps": work["gate_bytes"] / (gate_ms / 1e3) / 1e9,
            "gate_TFLOPs": work["gate_flop"] / (gate_ms / 1e3) / 1e12,
            "select_us": sel_ms * 1e3,
            "compact_us": cmp_ms * 1e3,
            "compact_GBps": work["compact_bytes"] / (cmp_ms / 1e3) / 1e9,
            "selection_phase_us": sel_phase_ms * 1e3,
            "selection_phase_GBps": (work["gate_bytes"] + work["select_bytes"] +
                                     work["compact_bytes"]) / (sel_phase_ms / 1e3) / 1e9,
            "attn_us_per_layer": attn_avg * 1e3,
            "attn_TFLOPs": work["attn_flop_per_layer"] / (attn_avg / 1e3) / 1e12,
            "attn_layers": s.layers,
        }
        achieved = work["attn_flop_per_layer"] / (attn_avg / 1e3) / 1e12
        traffic = None
        kname = attn_kernel_name(w.dtype, s.Hq, s.d, Kt, torch.cuda.get_device_properties(0).multi_processor_count)
        if s.name == "qwen3_1p7b_128k":
            traffic = measured_traffic(
                kname, os.path.join(ROOT, "learned_token_pruning_score_amd", "csrc", "attn.hip"))
        roof = {"bound": "mfma", "kernel": kname,
                "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic,
                "traffic_unit": "HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                "algorithmic_bytes_per_launch": work["attn_bytes_per_layer"],
                "per_launch_flop": work["attn_flop_per_layer"],
                "avg_launch_us": attn_avg * 1e3}
        log(f"[bench] phases: {json.dumps(phases)}")

    refs = None
    if not args.no_reference_points:
        refs = reference_points(tg, w, gp, layers, outs, hidden, W1, b1, w2, stream, dev)
        log(f"[bench] reference points: {json.dumps(refs)}")

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample ...")
        cpu = cpu_baseline(w, layers_cpu, gp.cu_kept_h, Kt)
        log(f"[bench] cpu baseline: {cpu['value']:.4g} tokens/s ({cpu['sample']})")

    line = {
        "metric": "gated prefill tokens/s at 128k (score+topK+compact+attn); % MFMA/HBM peak",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if s.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": s.name, "T": w.T, "kept": Kt, "prompts": w.B,
                   "hidden": s.D, "gate_hidden": s.F, "q_heads": s.Hq, "kv_heads": s.Hkv,
                   "head_dim": s.d, "gated_layers": s.layers, "tau": s.tau},
        "roofline": roof,
        "cpu_baseline": cpu,
        "phases": phases,
        "timing": "hip_graph_replay" if graph_ms is not None else "eager",
        "cold_cache": flushed,
        "eager_ms_per_step": eager_ms,
        "reference_points": refs,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
