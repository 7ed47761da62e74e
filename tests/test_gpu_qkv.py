"""GPU parity of the pruned layer's input step: the rotary table of the kept
rows' original positions and the fused q/k/v projection with the rotary
embedding, through the C ABI, against the CPU fp64 oracle.

Bars (written here):
  * rope table: |Δ| <= 1e-7 + |a| 2^-50 against cos / sin of the oracle's
    angles a (an fp32 rounding of an fp64 value of magnitude <= 1 is off by
    <= 2^-25; the fp64 angle itself is known to a few units of 2^-53
    relative, which matters only for positions far beyond any prompt).
  * q / k / v, bf16 I/O: |Δ| <= 2^-8 (1 + 2^-6) |ref| + (D + 4) 2^-23 S
    where S is sum_k |x_k| |W_nk| of the element (for a rotated element the
    sum over both members of its pair).  The first term is the one rounding
    to bf16 (unit roundoff 2^-8), the second twice the worst-case fp32
    accumulation bound (D + 3) 2^-24 S of the dot products, the rotation
    and the fp32 table entries.  The oracle gets exactly the GPU's bf16
    inputs.
  * q / k / v, fp32 I/O: |Δ| <= 2^-23 |ref| + (D + 4) 2^-23 S (no final
    rounding).
Full-size: the 128k-token workload's kept rows (8448) through the same
launches as the benchmark, on a seeded sample of rows.
"""

import numpy as np
import pytest
import torch

import learned_token_pruning_score_amd as tg
import oracle
import synth

pytestmark = pytest.mark.gpu

DEV = "cuda"
THETA = 1e6


def _note(msg):
    print(msg, flush=True)


def _f64(t):
    return t.detach().to("cpu").to(torch.float64).numpy()


def _pair_scale(S, H, d):
    """S [n, H d] -> per element, the sum of S over its rotation pair."""
    n = S.shape[0]
    Sh = S.reshape(n, H, d)
    half = d // 2
    p = Sh[..., :half] + Sh[..., half:]
    return np.concatenate([p, p], axis=-1)


def _check_qkv(qkv, x, W, pos, Hq, Hkv, d, dtype):
    """Compare the GPU's packed [n, (Hq + 2 Hkv) d] output with the oracle."""
    x64, W64 = _f64(x), _f64(W)
    D = x64.shape[1]
    q_ref, k_ref, v_ref = oracle.qkv_rope(x64, W64, pos, THETA, Hq, Hkv, d)
    S = np.abs(x64) @ np.abs(W64).T
    n = x64.shape[0]
    scales = (_pair_scale(S[:, :Hq * d], Hq, d),
              _pair_scale(S[:, Hq * d:(Hq + Hkv) * d], Hkv, d),
              S[:, (Hq + Hkv) * d:].reshape(n, Hkv, d))
    got = _f64(qkv)
    parts = (got[:, :Hq * d].reshape(n, Hq, d),
             got[:, Hq * d:(Hq + Hkv) * d].reshape(n, Hkv, d),
             got[:, (Hq + Hkv) * d:(Hq + 2 * Hkv) * d].reshape(n, Hkv, d))
    rel = 2.0 ** -8 * (1 + 2.0 ** -6) if dtype == torch.bfloat16 else 2.0 ** -23
    worst = 0.0
    for name, g, r, sc in zip("qkv", parts, (q_ref, k_ref, v_ref), scales):
        tol = rel * np.abs(r) + (D + 4) * 2.0 ** -23 * sc
        excess = np.abs(g - r) - tol
        i = np.unravel_index(np.argmax(excess), excess.shape)
        assert excess[i] <= 0, (f"{name}{tuple(int(j) for j in i)}: got {g[i]}, oracle {r[i]}, "
                                f"tol {tol[i]}")
        worst = max(worst, float(np.max(np.abs(g - r) / np.maximum(tol, 1e-30))))
    return worst


def _inputs(Kt, D, Hq, Hkv, d, dtype, seed, ld_pad=0, pos_max=131072):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((Kt, D + ld_pad), generator=g).to(dtype)
    N = (Hq + 2 * Hkv) * d
    W = (torch.randn((N, D), generator=g) / D ** 0.5).to(dtype)
    pos = torch.randint(0, pos_max, (Kt,), generator=g, dtype=torch.int32)
    return x, W, pos


@pytest.mark.parametrize("Kt,pos_max", [(1, 2), (700, 131072), (300, 1 << 24), (64, 2 ** 31 - 1)])
@pytest.mark.parametrize("d", [64, 128])
def test_rope_table(Kt, pos_max, d):
    _note(f"[rope_table] Kt={Kt} pos_max={pos_max} d={d}")
    g = torch.Generator().manual_seed(Kt + d)
    pos = torch.randint(0, pos_max, (Kt,), generator=g, dtype=torch.int32)
    pos[0] = 0
    tab = tg.tg_rope_table(pos.to(DEV), d, THETA)
    torch.cuda.synchronize()
    ang = pos.numpy().astype(np.float64)[:, None] * oracle.rope_inv_freq(d, THETA)[None, :]
    t = tab.cpu().numpy().astype(np.float64)
    tol = 1e-7 + np.abs(ang) * 2.0 ** -50
    assert np.all(np.abs(t[..., 0] - np.cos(ang)) <= tol)
    assert np.all(np.abs(t[..., 1] - np.sin(ang)) <= tol)
    assert np.all(t[0, :, 0] == 1.0) and np.all(t[0, :, 1] == 0.0)


# (Kt, D, Hq, Hkv, d, ld_pad, out_pad): the benchmark head shapes over four
# row tiles with a ragged last one; d = 64 with strided rows and a padded
# output; q/k/v boundaries inside a 256-column tile and a half-empty last
# column tile; one row; D of three 64-column stages.
BF16_SHAPES = [
    (1000, 2048, 16, 8, 128, 0, 0),
    (300, 256, 4, 2, 64, 64, 8),
    (77, 512, 3, 1, 128, 0, 0),
    (1, 64, 1, 1, 64, 0, 0),
    (513, 192, 2, 2, 128, 0, 0),
    (260, 128, 5, 1, 64, 0, 0),
]


@pytest.mark.parametrize("shape", BF16_SHAPES)
def test_qkv_rope_bf16(shape):
    Kt, D, Hq, Hkv, d, ld_pad, out_pad = shape
    _note(f"[qkv bf16] {shape}")
    x, W, pos = _inputs(Kt, D, Hq, Hkv, d, torch.bfloat16, seed=sum(shape))
    N = (Hq + 2 * Hkv) * d
    xd = x.to(DEV)[:, :D]
    tab = tg.tg_rope_table(pos.to(DEV), d, THETA)
    out = torch.full((Kt, N + out_pad), 7.0, dtype=torch.bfloat16, device=DEV)
    qkv, q, k, v = tg.tg_qkv_rope(xd, W.to(DEV), tab, Hq, Hkv, d, out=out[:, :N])
    torch.cuda.synchronize()
    assert q.shape == (Kt, Hq, d) and k.shape == (Kt, Hkv, d) and v.shape == (Kt, Hkv, d)
    _check_qkv(qkv.cpu(), x[:, :D], W, pos.numpy(), Hq, Hkv, d, torch.bfloat16)
    if out_pad:
        assert torch.all(out[:, N:].cpu() == 7.0), "padding columns written"
    # bit-reproducible
    qkv2, _, _, _ = tg.tg_qkv_rope(xd, W.to(DEV), tab, Hq, Hkv, d)
    torch.cuda.synchronize()
    assert torch.equal(qkv2, qkv)


# With 256 CUs: 128 tiles of 256 x 256 run as one launch of the tile kernel;
# 272 tiles as one full round of it plus 16 tiles cut into 64-row sub-tiles
# (the layout of the 128k kept rows: 528 tiles = two rounds + 16).  The
# small shapes above (at most 64 tiles) run on sub-tiles alone.
@pytest.mark.parametrize("Kt", [2000, 4352])
def test_qkv_rope_bf16_tile_and_subtile_launches(Kt):
    D, Hq, Hkv, d = 2048, 16, 8, 128
    _note(f"[qkv bf16 launches] Kt={Kt}")
    x, W, pos = _inputs(Kt, D, Hq, Hkv, d, torch.bfloat16, seed=Kt)
    tab = tg.tg_rope_table(pos.to(DEV), d, THETA)
    qkv, _, _, _ = tg.tg_qkv_rope(x.to(DEV), W.to(DEV), tab, Hq, Hkv, d)
    torch.cuda.synchronize()
    g = np.random.default_rng(Kt)
    rows = np.unique(np.concatenate([[0, 255, 256, Kt - 257, Kt - 256, Kt - 1],
                                     g.integers(0, Kt, 120), g.integers(Kt - 256, Kt, 40)]))
    idx = torch.from_numpy(rows)
    _check_qkv(qkv.cpu()[idx], x[idx], W, pos.numpy()[rows], Hq, Hkv, d, torch.bfloat16)


@pytest.mark.parametrize("shape", [(50, 256, 4, 2, 64), (33, 128, 2, 1, 128), (1, 64, 1, 1, 64)])
def test_qkv_rope_f32(shape):
    Kt, D, Hq, Hkv, d = shape
    _note(f"[qkv f32] {shape}")
    x, W, pos = _inputs(Kt, D, Hq, Hkv, d, torch.float32, seed=sum(shape))
    tab = tg.tg_rope_table(pos.to(DEV), d, THETA)
    qkv, _, _, _ = tg.tg_qkv_rope(x.to(DEV), W.to(DEV), tab, Hq, Hkv, d)
    torch.cuda.synchronize()
    _check_qkv(qkv.cpu(), x, W, pos.numpy(), Hq, Hkv, d, torch.float32)


def test_qkv_rope_empty_and_rejects():
    _note("[qkv] empty and invalid calls")
    x = torch.zeros((0, 128), dtype=torch.bfloat16, device=DEV)
    W = torch.zeros((4 * 64, 128), dtype=torch.bfloat16, device=DEV)
    tab = tg.tg_rope_table(torch.zeros(0, dtype=torch.int32, device=DEV), 64, THETA)
    qkv, q, _, _ = tg.tg_qkv_rope(x, W, tab, 2, 1, 64)
    assert qkv.shape == (0, 256) and q.shape == (0, 2, 64)
    # D not a multiple of 64 on the bf16 path
    x = torch.zeros((4, 96), dtype=torch.bfloat16, device=DEV)
    W = torch.zeros((4 * 64, 96), dtype=torch.bfloat16, device=DEV)
    tab = torch.zeros((4, 32, 2), dtype=torch.float32, device=DEV)
    with pytest.raises(tg.TokenGateError):
        tg.tg_qkv_rope(x, W, tab, 2, 1, 64)
    with pytest.raises(tg.TokenGateError):  # head size without a kernel
        tg.tg_rope_table(torch.zeros(4, dtype=torch.int32, device=DEV), 96, THETA)
    with pytest.raises(tg.TokenGateError):  # a rotary base must exceed 1
        tg.tg_rope_table(torch.zeros(4, dtype=torch.int32, device=DEV), 64, 1.0)


def test_qkv_feeds_attention_in_place():
    """compaction -> rope table -> q/k/v -> attention reading the packed
    buffer with its token stride gives the result of contiguous copies."""
    name = "ragged_small_bf16"
    _note(f"[qkv chain] {name}")
    w = synth.make_workload(name, seed=5)
    s = w.spec
    gp = tg.GatedPrefill(w.cu_seqlens, w.doc_begin, w.doc_end, w.budget, s.D, w.dtype)
    gp.gate_and_select(w.hidden.to(DEV), w.W1.to(DEV), w.b1.to(DEV), w.w2.to(DEV), w.b2)
    gp.rope(s.d, s.rope_theta)
    W = synth.qkv_weights(name, 0, seed=5)
    qkv, q, k, v = gp.project_qkv(W.to(DEV), s.Hq, s.Hkv, s.d)
    gain = torch.linspace(0.5, 2.0, s.Hq, device=DEV)
    o1, l1 = gp.attend(q, k, v, gain, s.tau, lse=torch.empty((s.Hq, gp.Kt), device=DEV))
    o2, l2 = gp.attend(q.contiguous(), k.contiguous(), v.contiguous(), gain, s.tau,
                       lse=torch.empty((s.Hq, gp.Kt), device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # the projection of the compacted rows at the compacted positions
    hk, pk = gp.hidden_k.cpu(), gp.pos_k.cpu().numpy()
    pos_ref = w.positions()[gp.kept_idx.cpu().numpy()]
    assert np.array_equal(pk, pos_ref)
    rows = np.unique(np.concatenate([[0, gp.Kt - 1], np.random.default_rng(5).integers(0, gp.Kt, 200)]))
    _check_qkv(qkv.cpu()[rows], hk[rows], W, pk[rows], s.Hq, s.Hkv, s.d, torch.bfloat16)


def test_qkv_rope_full_size_128k():
    """The 128k-token workload's 8448 kept rows, in the benchmark's launch
    configuration; a seeded sample of rows (each prompt's first and last
    kept row included) against the oracle."""
    name = "qwen3_1p7b_128k"
    _note(f"[qkv full] {name}")
    w = synth.make_workload(name, seed=0)
    s = w.spec
    gp = tg.GatedPrefill(w.cu_seqlens, w.doc_begin, w.doc_end, w.budget, s.D, w.dtype)
    gp.gate_and_select(w.hidden.to(DEV), w.W1.to(DEV), w.b1.to(DEV), w.w2.to(DEV), w.b2)
    del w.hidden
    gp.rope(s.d, s.rope_theta)
    W = synth.qkv_weights(name, 0, seed=0)
    qkv, _, _, _ = gp.project_qkv(W.to(DEV), s.Hq, s.Hkv, s.d)
    torch.cuda.synchronize()
    cu = gp.cu_kept_h
    rows = np.unique(np.concatenate([cu[:-1], cu[1:] - 1,
                                     np.random.default_rng(0).integers(0, gp.Kt, 96)]))
    rows = rows[(rows >= 0) & (rows < gp.Kt)]
    hk = gp.hidden_k[torch.from_numpy(rows).to(DEV)].cpu()
    pk = gp.pos_k.cpu().numpy()[rows]
    worst = _check_qkv(qkv[torch.from_numpy(rows).to(DEV)].cpu(), hk, W, pk, s.Hq, s.Hkv, s.d,
                       torch.bfloat16)
    _note(f"  Kt={gp.Kt} rows={rows.size} worst error / tolerance = {worst:.3f}")
