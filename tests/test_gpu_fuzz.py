"""Seeded random end-to-end cases of the gated prefill through the C ABI
against the CPU fp64 oracle: random prompt counts and lengths (empty
prompts, empty documents, non-document tokens before and after the
document), budgets from 0 past the document length, hidden widths that are
and are not multiples of 64, gate widths 64/128/256, GQA shapes, head
dimensions 64/128, bf16 and fp32, with and without the score bias, implicit
and explicit (permuted) positions, and all-equal scores (W1 = 0: ties
decided by index alone).

Bars, per step, as in the fixed-workload parity tests: gate scores
|Δ| <= 1e-3 max(1, |s_ref|); keep flags, plan, compacted rows, positions,
biases and source indices bit-exact (the oracle on the GPU's own fp32
scores); attention max-abs 2e-2 (bf16 I/O) / 1e-4 (fp32) and lse 1e-3 /
1e-4 (the oracle on the GPU's own compacted biases), on every row of short
prompts and on a seeded sample plus every wave's first and last row of long
ones."""

import numpy as np
import pytest
import torch

import learned_token_pruning_score_amd as tg
import oracle

pytestmark = pytest.mark.gpu

DEV = "cuda"
ATTN_TOL = {torch.bfloat16: 2e-2, torch.float32: 1e-4}
LSE_TOL = {torch.bfloat16: 1e-3, torch.float32: 1e-4}
N_CASES = 120


def _f64(t):
    return t.detach().to("cpu").to(torch.float64).numpy()


def _case(seed):
    rng = np.random.default_rng(9000 + seed)
    dtype = torch.bfloat16 if rng.random() < 0.75 else torch.float32
    if dtype == torch.bfloat16:
        D = int(rng.choice([8, 64, 136, 512, 1000, 2048]))
    else:
        D = int(rng.choice([5, 64, 256]))
    F = int(rng.choice([64, 128, 256]))
    Hq, Hkv = [(4, 2), (8, 1), (16, 8), (6, 3), (2, 2)][int(rng.integers(0, 5))]
    d = int(rng.choice([64, 128]))
    B = int(rng.integers(1, 6))
    lens, dbs, des, buds = [], [], [], []
    for _ in range(B):
        pre = int(rng.integers(0, 20)) if rng.random() < 0.5 else 0
        doc = int(rng.integers(0, 2500)) if rng.random() < 0.9 else 0
        post = int(rng.integers(0, 300))
        if rng.random() < 0.08:
            pre = doc = post = 0  # an empty prompt
        lens.append(pre + doc + post)
        dbs.append(pre)
        des.append(pre + doc)
        buds.append(int(rng.integers(0, doc + 6)))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return dict(rng=rng, dtype=dtype, D=D, F=F, Hq=Hq, Hkv=Hkv, d=d, B=B, cu=cu,
                db=np.array(dbs, np.int32), de=np.array(des, np.int32), bud=np.array(buds, np.int32))


def _rows(cu_kept, rng):
    """All rows when every prompt is short; else 48 random rows per long
    prompt plus every 32-row block's first and last row (each wave's rows)."""
    rows = []
    for b in range(len(cu_kept) - 1):
        lo, hi = int(cu_kept[b]), int(cu_kept[b + 1])
        if hi - lo <= 700:
            rows.append(np.arange(lo, hi))
            continue
        first = np.arange(lo, hi, 32)
        rows += [rng.integers(lo, hi, 48), first, np.minimum(first + 31, hi - 1)]
    return np.unique(np.concatenate(rows)) if rows else np.zeros(0, np.int64)


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_gated_prefill(seed):
    c = _case(seed)
    rng, dt = c["rng"], c["dtype"]
    D, F, Hq, Hkv, d = c["D"], c["F"], c["Hq"], c["Hkv"], c["d"]
    T = int(c["cu"][-1])
    print(f"[fuzz {seed}] {dt} T={T} B={c['B']} D={D} F={F} heads {Hq}/{Hkv} d={d} "
          f"lens {np.diff(c['cu']).tolist()} budgets {c['bud'].tolist()}", flush=True)
    hidden = torch.from_numpy(rng.standard_normal((T, D)).astype(np.float32)).to(dt)
    W1 = torch.from_numpy((rng.standard_normal((F, D)) / np.sqrt(D)).astype(np.float32)).to(dt)
    b1 = torch.from_numpy((0.1 * rng.standard_normal(F)).astype(np.float32)) if rng.random() < 0.7 else None
    w2 = torch.from_numpy((rng.standard_normal(F) / np.sqrt(F)).astype(np.float32))
    b2 = float(rng.choice([0.0, 0.3]))
    if rng.random() < 0.15:  # every score equal: the kept set is decided by index alone
        W1.zero_()
    explicit = rng.random() < 0.4
    if explicit:  # a permutation of 0 .. len - 1 inside each prompt
        pos_h = np.concatenate([rng.permutation(n) for n in np.diff(c["cu"])] or [np.zeros(0)]).astype(np.int32)
    else:
        pos_h = np.concatenate([np.arange(n) for n in np.diff(c["cu"])] or [np.zeros(0)]).astype(np.int32)
    gp = tg.GatedPrefill(c["cu"], c["db"], c["de"], c["bud"], D, dt)
    gp.gate_and_select(hidden.to(DEV), W1.to(DEV), None if b1 is None else b1.to(DEV), w2.to(DEV), b2,
                       pos=torch.from_numpy(pos_h).to(DEV) if explicit else None)
    torch.cuda.synchronize()
    # gate scores
    s_gpu = gp.scores.cpu().numpy()
    s_ref = oracle.gate_scores(_f64(hidden), _f64(W1), None if b1 is None else _f64(b1), _f64(w2), b2)
    if T:
        err = np.abs(s_gpu.astype(np.float64) - s_ref) / np.maximum(1.0, np.abs(s_ref))
        assert err.max() <= 1e-3, f"score error {err.max()}"
    # plan, top-K and compaction, bit-exact on the GPU's scores
    cu_ref, mx_ref = oracle.plan(c["cu"], c["db"], c["de"], c["bud"])
    assert gp.cu_kept_h.tolist() == cu_ref.tolist() and gp.max_kept_len == mx_ref
    keep = gp.keep.cpu().numpy()
    assert np.array_equal(keep, oracle.select_topk(s_gpu, c["cu"], c["db"], c["de"], c["bud"]))
    ibits = torch.int16 if dt == torch.bfloat16 else torch.int32
    hk_ref, pk_ref, bk_ref, ik_ref = oracle.compact(hidden.view(ibits).numpy(), pos_h, s_gpu, keep, c["cu"],
                                                    c["db"], c["de"])
    assert np.array_equal(gp.hidden_k.cpu().view(ibits).numpy(), hk_ref)
    assert np.array_equal(gp.pos_k.cpu().numpy(), pk_ref)
    bk = gp.bias_s.cpu().numpy()
    assert np.array_equal(bk.view(np.uint32), bk_ref.view(np.uint32))
    assert np.array_equal(gp.kept_idx.cpu().numpy(), ik_ref)
    # token-gated attention over the kept rows
    Kt = gp.Kt
    if Kt == 0:
        return
    q = torch.from_numpy(rng.standard_normal((Kt, Hq, d)).astype(np.float32)).to(dt)
    k = torch.from_numpy(rng.standard_normal((Kt, Hkv, d)).astype(np.float32)).to(dt)
    v = torch.from_numpy(rng.standard_normal((Kt, Hkv, d)).astype(np.float32)).to(dt)
    tau = float(rng.uniform(0.5, 2.0))
    with_bias = rng.random() < 0.8
    gain = torch.from_numpy(rng.uniform(0.5, 2.0, Hq).astype(np.float32))
    o, lse = tg.tg_gated_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), gp.bias_s if with_bias else None,
                                  gain.to(DEV) if with_bias else None, tau, gp.cu_kept, gp.max_kept_len,
                                  lse=torch.empty((Hq, Kt), device=DEV))
    torch.cuda.synchronize()
    rows = _rows(gp.cu_kept_h, rng)
    o_ref, lse_ref = oracle.gated_attention(_f64(q), _f64(k), _f64(v), bk.astype(np.float64) if with_bias else None,
                                            _f64(gain) if with_bias else None, tau, gp.cu_kept_h, rows=rows)
    aerr = np.max(np.abs(_f64(o)[rows] - o_ref[rows]))
    lerr = np.max(np.abs(_f64(lse)[:, rows] - lse_ref[:, rows]))
    print(f"[fuzz {seed}] Kt={Kt} rows {len(rows)} attention max-abs {aerr:.2e} lse {lerr:.2e}", flush=True)
    assert aerr <= ATTN_TOL[dt] and lerr <= LSE_TOL[dt]
