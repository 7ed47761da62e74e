"""GPU parity: the HIP path through the C ABI against the CPU fp64 oracle.

Bars (written here, per step):
  * gate scores: |s_gpu - s_ref| <= 1e-3 * max(1, |s_ref|)
  * top-K keep flags and compaction outputs: bit-exact given the same fp32
    scores; end-to-end kept sets (each side on its own scores) may differ
    only for tokens whose oracle score is within 1e-3 * max(1, |theta|) of
    the prompt's k-th best document score theta
  * attention output: max-abs 2e-2 for bf16 I/O, 1e-4 for fp32 I/O; lse
    max-abs 1e-3 (bf16) / 1e-4 (fp32); the oracle gets exactly the GPU's
    compacted biases, so kept-set ties cannot leak into this comparison
  * determinism: a second run is byte-identical.
Large workloads check every score and flag, and attention on a seeded sample
of rows (every prompt's first and last kept row included).
"""

import math

import numpy as np
import pytest
import torch

import learned_token_pruning_score_amd as tg
import oracle
import synth

pytestmark = pytest.mark.gpu

DEV = "cuda"
ATTN_TOL = {torch.bfloat16: 2e-2, torch.float32: 1e-4}
LSE_TOL = {torch.bfloat16: 1e-3, torch.float32: 1e-4}
SAMPLE_ROWS = 256  # random rows per prompt, for kept lengths above FULL_ROWS
FULL_ROWS = 3000
WAVE_ROWS = 32  # query rows per wave in both bf16 attention schedules


def _f64(t):
    return t.detach().to("cpu").to(torch.float64).numpy()


def _note(msg):
    print(msg, flush=True)


class Case:
    """GPU pipeline and oracle results for one workload, computed once."""

    def __init__(self, name):
        _note(f"[case] {name}")
        w = synth.make_workload(name, seed=0)
        self.w = w
        s = w.spec
        self.gp = tg.GatedPrefill(w.cu_seqlens, w.doc_begin, w.doc_end, w.budget, s.D, w.dtype)
        self.hidden = w.hidden.to(DEV)
        self.W1 = w.W1.to(DEV)
        self.b1 = w.b1.to(DEV)
        self.w2 = w.w2.to(DEV)
        self.gp.gate_and_select(self.hidden, self.W1, self.b1, self.w2, w.b2)
        torch.cuda.synchronize()
        gp = self.gp
        self.s_gpu = gp.scores.cpu().numpy()
        self.keep_gpu = gp.keep.cpu().numpy()
        self.hk = gp.hidden_k.cpu()
        self.pk = gp.pos_k.cpu().numpy()
        self.bk = gp.bias_s.cpu().numpy()
        self.ik = gp.kept_idx.cpu().numpy()
        self.s_ref = oracle.gate_scores(_f64(w.hidden), _f64(w.W1), _f64(w.b1), _f64(w.w2), w.b2)
        self.layers = {}

    def layer(self, l):
        if l not in self.layers:
            s = self.w.spec
            q, k, v, gain = synth.attention_inputs(s, l, self.gp.Kt, seed=0)
            qd, kd, vd, gd = q.to(DEV), k.to(DEV), v.to(DEV), gain.to(DEV)
            o, lse = self.gp.attend(qd, kd, vd, gd, s.tau,
                                    lse=torch.empty((s.Hq, self.gp.Kt), device=DEV))
            torch.cuda.synchronize()
            self.layers[l] = dict(q=q, k=k, v=v, gain=gain, dev=(qd, kd, vd, gd),
                                  o=o.cpu(), lse=lse.cpu())
        return self.layers[l]


_CASES = {}


def case(name):
    if name not in _CASES:
        _CASES.clear()  # hold one workload's device buffers at a time
        torch.cuda.empty_cache()
        _CASES[name] = Case(name)
    return _CASES[name]


NAMES = ["tiny_fp32_512", "tiny_fp32_b2", "ragged_tiny_fp32", "ragged_small_bf16",
         "qwen3_1p7b_16k", "qwen3_1p7b_32k", "ragged_8x_4k_32k", "qwen3_1p7b_128k"]


def _rows(cu_kept, boundaries=False):
    """None (every row) for short prompts; else SAMPLE_ROWS random rows per
    prompt plus its first and last, and with ``boundaries`` the first and last
    row of every 32-row block of a prompt (each wave's rows: the rows on both
    sides of every 64-key tile's diagonal and of every 128- and 256-row query
    tile edge)."""
    if int(np.max(np.diff(cu_kept), initial=0)) <= FULL_ROWS:
        return None
    rows = [oracle.attention_rows_for_check(cu_kept, SAMPLE_ROWS, seed=0)]
    if boundaries:
        for b in range(len(cu_kept) - 1):
            lo, hi = int(cu_kept[b]), int(cu_kept[b + 1])
            first = np.arange(lo, hi, WAVE_ROWS)
            rows += [first, np.minimum(first + WAVE_ROWS - 1, hi - 1)]
    return np.unique(np.concatenate(rows))


def _attn_check(o_gpu, lse_gpu, q, k, v, bias, gain, tau, cu_kept, dtype, rows):
    o_ref, lse_ref = oracle.gated_attention(_f64(q), _f64(k), _f64(v), bias, gain, tau, cu_kept,
                                            rows=rows)
    og = o_gpu.to(torch.float64).numpy()
    sel = slice(None) if rows is None else rows
    err = np.max(np.abs(og[sel] - o_ref[sel]))
    assert err <= ATTN_TOL[dtype], f"attention max-abs error {err}"
    if lse_gpu is not None:
        lg = lse_gpu.to(torch.float64).numpy()
        lerr = np.max(np.abs(lg[:, sel] - lse_ref[:, sel]))
        assert lerr <= LSE_TOL[dtype], f"lse max-abs error {lerr}"
    return err


@pytest.mark.parametrize("name", NAMES)
def test_pipeline_parity(name):
    c = case(name)
    w, gp = c.w, c.gp
    # gate scores
    err = np.abs(c.s_gpu.astype(np.float64) - c.s_ref) / np.maximum(1.0, np.abs(c.s_ref))
    assert err.max() <= 1e-3, f"score error {err.max()}"
    # selection, bit-exact on the GPU's own scores
    keep_ref = oracle.select_topk(c.s_gpu, w.cu_seqlens, w.doc_begin, w.doc_end, w.budget)
    assert np.array_equal(c.keep_gpu, keep_ref)
    # kept counts agree with the plan
    cu_ref, mx_ref = oracle.plan(w.cu_seqlens, w.doc_begin, w.doc_end, w.budget)
    assert gp.cu_kept_h.tolist() == cu_ref.tolist() and gp.max_kept_len == mx_ref
    # end-to-end kept sets: differences only inside the 1e-3 band around theta
    s32 = oracle.round_f32(c.s_ref)
    keep_e2e = oracle.select_topk(s32, w.cu_seqlens, w.doc_begin, w.doc_end, w.budget)
    diff = np.nonzero(keep_e2e != c.keep_gpu)[0]
    for b in range(w.B):
        lo = int(w.cu_seqlens[b])
        dlo, dhi = lo + int(w.doc_begin[b]), lo + int(w.doc_end[b])
        kk = min(int(w.budget[b]), dhi - dlo)
        mine = diff[(diff >= dlo) & (diff < dhi)]
        if mine.size == 0:
            continue
        theta = np.sort(c.s_ref[dlo:dhi])[::-1][kk - 1]
        band = 1e-3 * max(1.0, abs(theta))
        assert np.all(np.abs(c.s_ref[mine] - theta) <= band), (b, mine)
    # compaction, bit-exact
    hk_ref, pk_ref, bk_ref, ik_ref = oracle.compact(
        w.hidden.view(torch.int16 if w.dtype == torch.bfloat16 else torch.int32).numpy(),
        w.positions(), c.s_gpu, c.keep_gpu, w.cu_seqlens, w.doc_begin, w.doc_end)
    hk_bits = c.hk.view(torch.int16 if w.dtype == torch.bfloat16 else torch.int32).numpy()
    assert np.array_equal(hk_bits, hk_ref)
    assert np.array_equal(c.pk, pk_ref)
    assert np.array_equal(c.bk.view(np.uint32), bk_ref.view(np.uint32))
    assert np.array_equal(c.ik, ik_ref)
    # needle recall is reported, not graded
    _note(f"[{name}] T={w.T} Kt={gp.Kt} needle recall {c.keep_gpu[w.needles].mean():.3f}")


@pytest.mark.parametrize("name", NAMES)
def test_attention_parity(name):
    c = case(name)
    s = c.w.spec
    for l in range(s.layers):
        # the first layer also checks every wave's first and last row
        rows = _rows(c.gp.cu_kept_h, boundaries=(l == 0))
        L = c.layer(l)
        err = _attn_check(L["o"], L["lse"], L["q"], L["k"], L["v"], c.bk, _f64(L["gain"]),
                          s.tau, c.gp.cu_kept_h, c.w.dtype, rows)
        _note(f"[{name}] layer {l}: {'all' if rows is None else len(rows)} rows, max-abs {err:.2e}")


@pytest.mark.parametrize("name", ["tiny_fp32_512", "ragged_small_bf16", "qwen3_1p7b_16k"])
def test_determinism(name):
    c = case(name)
    gp = c.gp
    gp.gate_and_select(c.hidden, c.W1, c.b1, c.w2, c.w.b2)
    L = c.layer(0)
    qd, kd, vd, gd = L["dev"]
    o2, lse2 = gp.attend(qd, kd, vd, gd, c.w.spec.tau,
                         lse=torch.empty((c.w.spec.Hq, gp.Kt), device=DEV))
    torch.cuda.synchronize()
    assert np.array_equal(gp.scores.cpu().numpy().view(np.uint32), c.s_gpu.view(np.uint32))
    assert np.array_equal(gp.keep.cpu().numpy(), c.keep_gpu)
    assert torch.equal(gp.hidden_k.cpu(), c.hk)
    assert torch.equal(o2.cpu().view(torch.int16 if o2.dtype == torch.bfloat16 else torch.int32),
                       L["o"].view(torch.int16 if o2.dtype == torch.bfloat16 else torch.int32))
    assert torch.equal(lse2.cpu(), L["lse"])


def test_dense_comparator_parity():
    """Full-length causal attention at the 32k gate layer (no bias, tau = 1),
    the un-pruned prefill's attention."""
    s = synth.spec("qwen3_1p7b_32k")
    N = 32768
    q, k, v = synth.dense_attention_inputs(s, N, seed=0)
    cu = np.array([0, N], dtype=np.int32)
    o, lse = tg.tg_gated_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), None, None, 1.0,
                                  torch.from_numpy(cu).to(DEV), N, want_lse=True)
    torch.cuda.synchronize()
    rows = oracle.attention_rows_for_check(cu, 24, seed=1)
    err = _attn_check(o.cpu(), lse.cpu(), q, k, v, None, None, 1.0, cu, torch.bfloat16, rows)
    _note(f"[dense 32k] max-abs {err:.2e}")


# ------------------------------------------------------------------ edge cases

def _select_gpu(scores_np, cu, db, de, bud):
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(DEV)  # noqa: E731
    keep = tg.tg_select_topk(torch.from_numpy(np.ascontiguousarray(scores_np, np.float32)).to(DEV),
                             d(cu), d(db), d(de), d(bud))
    torch.cuda.synchronize()
    return keep.cpu().numpy()


def test_select_hand_worked_and_specials_on_gpu():
    import json, os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "select_hand_worked.json")))
    s = np.array([float(x) if isinstance(x, str) else x for x in g["scores"]], dtype=np.float32)
    for cs in g["cases"]:
        keep = _select_gpu(s, g["cu_seqlens"], g["doc_begin"], g["doc_end"], cs["budget"])
        assert np.nonzero(keep)[0].tolist() == cs["kept"], cs


# the first two inputs (115005 tokens) take the one-workgroup-per-prompt
# path, the last (315005 tokens) the chunked four-kernel path
@pytest.mark.parametrize("seed,long_len", [(0, 70001), (1, 70001), (2, 270001)])
def test_select_heavy_ties_and_ragged(seed, long_len):
    rng = np.random.default_rng(100 + seed)
    B = 6
    lens = np.array([0, 1, 5000, long_len, 3, 40000])
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    db = np.array([0, 0, 100, 7, 0, 39990])
    de = np.array([0, 1, 4900, long_len, 3, 40000])
    bud = np.array([5, 0, 1234, 9000, 7, 4])
    T = int(cu[-1])
    # few distinct values -> long runs of equal keys, plus specials
    s = rng.integers(-3, 4, size=T).astype(np.float32) * np.float32(0.5)
    s[rng.integers(0, T, 200)] = -0.0
    s[rng.integers(0, T, 50)] = np.nan
    s[rng.integers(0, T, 20)] = np.inf
    s[rng.integers(0, T, 20)] = -np.inf
    keep = _select_gpu(s, cu, db, de, bud)
    assert np.array_equal(keep, oracle.select_topk(s, cu, db, de, bud))
    # every budget regime on one prompt
    for kk in [0, 1, 2, 4999, 5000, 5001, 100000]:
        keep = _select_gpu(s[:5000], [0, 5000], [0], [5000], [kk])
        assert np.array_equal(keep, oracle.select_topk(s[:5000], [0, 5000], [0], [5000], [kk])), kk


def test_select_distinct_random_scores_large():
    rng = np.random.default_rng(7)
    T = 300000
    s = rng.standard_normal(T).astype(np.float32)
    for kk in [1, 8192, 150000, 299999]:
        keep = _select_gpu(s, [0, T], [0], [T], [kk])
        assert np.array_equal(keep, oracle.select_topk(s, [0, T], [0], [T], [kk])), kk


@pytest.mark.parametrize("T,D,F,ld_pad,dtype", [
    (1000, 2048, 256, 0, torch.bfloat16), (257, 1024, 128, 64, torch.bfloat16),
    (1, 128, 64, 0, torch.bfloat16), (300, 192, 256, 0, torch.bfloat16),
    (130, 320, 128, 16, torch.bfloat16),
    # more tiles than CUs: workgroups loop over tiles, loads run across tile ends
    (70001, 320, 256, 8, torch.bfloat16), (66000, 128, 64, 0, torch.bfloat16),
    # shorter inputs: F split over 2 or 4 waves per token group (128- and
    # 64-token tiles), the last one with more tiles than CUs
    (40000, 256, 256, 8, torch.bfloat16), (40000, 192, 128, 0, torch.bfloat16),
    (20000, 128, 256, 0, torch.bfloat16), (9000, 64, 64, 0, torch.bfloat16),
    # D % 64 != 0 (a partial last stage of 8..56 columns), with row padding
    # that holds NaN so that a read past column D would show
    (1000, 72, 256, 8, torch.bfloat16), (300, 8, 64, 0, torch.bfloat16),
    (2000, 2040, 256, 24, torch.bfloat16), (777, 200, 128, 56, torch.bfloat16),
    (70001, 1000, 256, 8, torch.bfloat16), (40000, 136, 128, 0, torch.bfloat16),
    (513, 256, 64, 8, torch.float32),
    (77, 100, 30, 3, torch.float32)])
def test_gate_shapes(T, D, F, ld_pad, dtype):
    rng = np.random.default_rng(T + D)
    h = torch.from_numpy(rng.standard_normal((T, D + ld_pad)).astype(np.float32)).to(dtype)
    if D % 64:
        h[:, D:] = float("nan")
    W1 = torch.from_numpy((rng.standard_normal((F, D)) / math.sqrt(D)).astype(np.float32)).to(dtype)
    b1 = torch.from_numpy((0.1 * rng.standard_normal(F)).astype(np.float32))
    w2 = torch.from_numpy((rng.standard_normal(F) / math.sqrt(F)).astype(np.float32))
    hd = h.to(DEV)[:, :D]
    for bb in [b1, None]:
        s = tg.tg_gate_score(hd, W1.to(DEV), None if bb is None else bb.to(DEV), w2.to(DEV), -0.25)
        torch.cuda.synchronize()
        ref = oracle.gate_scores(_f64(h[:, :D]), _f64(W1), None if bb is None else _f64(bb),
                                 _f64(w2), -0.25)
        err = np.abs(s.cpu().numpy() - ref) / np.maximum(1, np.abs(ref))
        assert err.max() <= 1e-3


@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 2048), (torch.float32, 37), (torch.bfloat16, 9)])
def test_compact_explicit_positions_and_copy_modes(dtype, D):
    rng = np.random.default_rng(D)
    lens = np.array([300, 0, 2500, 1])
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    db = np.array([10, 0, 0, 0]); de = np.array([290, 0, 2400, 1]); bud = np.array([30, 3, 100, 0])
    T = int(cu[-1])
    h = torch.from_numpy(rng.standard_normal((T, D)).astype(np.float32)).to(dtype)
    s = rng.standard_normal(T).astype(np.float32)
    pos = rng.permutation(T).astype(np.int32)  # arbitrary explicit positions
    keep = oracle.select_topk(s, cu, db, de, bud)
    cu_kept, _ = oracle.plan(cu, db, de, bud)
    Kt = int(cu_kept[-1])
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(DEV)  # noqa: E731
    hk, pk, bk, ik = tg.tg_compact(h.to(DEV), d(pos), torch.from_numpy(s).to(DEV),
                                   torch.from_numpy(keep).to(DEV), d(cu), d(db), d(de), Kt)
    torch.cuda.synchronize()
    iv = torch.int16 if dtype == torch.bfloat16 else torch.int32
    hr, pr, br, ir = oracle.compact(h.view(iv).numpy(), pos, s, keep, cu, db, de)
    assert np.array_equal(hk.cpu().view(iv).numpy(), hr)
    assert np.array_equal(pk.cpu().numpy(), pr)
    assert np.array_equal(bk.cpu().numpy().view(np.uint32), br.view(np.uint32))
    assert np.array_equal(ik.cpu().numpy(), ir)


@pytest.mark.parametrize("lens,unaligned_keep", [
    ([600000, 3, 500000], False),   # more than 2^20 tokens
    ([5000, 7, 20000], True),       # keep flags not 16-byte aligned
    ([4095, 1, 70000, 4097], False)])  # chunks straddling prompts
def test_compact_sizes_and_alignment(lens, unaligned_keep):
    rng = np.random.default_rng(len(lens) + sum(lens))
    lens = np.array(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    db = np.minimum(lens, 2); de = np.maximum(db, lens - 1); bud = lens // 7
    T, D = int(cu[-1]), 16
    h = torch.from_numpy(rng.standard_normal((T, D)).astype(np.float32)).to(torch.bfloat16)
    s = rng.standard_normal(T).astype(np.float32)
    keep = oracle.select_topk(s, cu, db, de, bud)
    cu_kept, _ = oracle.plan(cu, db, de, bud)
    Kt = int(cu_kept[-1])
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(DEV)  # noqa: E731
    kd = torch.from_numpy(keep).to(DEV)
    if unaligned_keep:
        buf = torch.zeros(T + 1, dtype=torch.uint8, device=DEV)
        buf[1:] = kd
        kd = buf[1:]
        assert kd.data_ptr() % 16 != 0
    hk, pk, bk, ik = tg.tg_compact(h.to(DEV), None, torch.from_numpy(s).to(DEV), kd, d(cu), d(db),
                                   d(de), Kt)
    torch.cuda.synchronize()
    pos = np.concatenate([np.arange(n) for n in lens]).astype(np.int32)
    hr, pr, br, ir = oracle.compact(h.view(torch.int16).numpy(), pos, s, keep, cu, db, de)
    assert np.array_equal(hk.cpu().view(torch.int16).numpy(), hr)
    assert np.array_equal(pk.cpu().numpy(), pr)
    assert np.array_equal(bk.cpu().numpy().view(np.uint32), br.view(np.uint32))
    assert np.array_equal(ik.cpu().numpy(), ir)


def _attn_inputs(rng, lens, Hq, Hkv, d, dtype):
    Kt = int(sum(lens))
    mk = lambda *shape: torch.from_numpy(rng.standard_normal(shape).astype(np.float32)).to(dtype)  # noqa: E731
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return cu, mk(Kt, Hq, d), mk(Kt, Hkv, d), mk(Kt, Hkv, d), \
        (2 * rng.standard_normal(Kt)).astype(np.float32), rng.uniform(0.5, 2, Hq).astype(np.float32)


@pytest.mark.parametrize("dtype,d,Hq,Hkv", [
    (torch.bfloat16, 128, 16, 8), (torch.bfloat16, 64, 4, 2), (torch.bfloat16, 128, 4, 1),
    (torch.bfloat16, 128, 3, 3), (torch.float32, 64, 4, 2), (torch.float32, 128, 2, 1)])
def test_attention_ragged_edges(dtype, d, Hq, Hkv):
    rng = np.random.default_rng(d + Hq)
    lens = [1, 2, 63, 64, 65, 0, 127, 128, 129, 300, 31, 33]
    cu, q, k, v, bias, gain = _attn_inputs(rng, lens, Hq, Hkv, d, dtype)
    cud = torch.from_numpy(cu).to(DEV)
    for tau, gg in [(1.15, gain), (1.0, None), (0.5, gain)]:
        o, lse = tg.tg_gated_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV),
                                      torch.from_numpy(bias).to(DEV),
                                      None if gg is None else torch.from_numpy(gg).to(DEV), tau,
                                      cud, max(lens), want_lse=True)
        torch.cuda.synchronize()
        _attn_check(o.cpu(), lse.cpu(), q, k, v, bias if gg is not None else None,
                    None if gg is None else gg.astype(np.float64), tau, cu, dtype, None)


# The same edge prompts next to one long prompt, so that the query tiles are
# many enough for the 256-row schedule (the short batches above take the
# key-split schedule); the oracle checks every edge row and a sample of the
# long prompt.
@pytest.mark.parametrize("d,Hq,Hkv,long_len", [
    (128, 16, 8, 8300), (64, 4, 2, 33000), (128, 3, 3, 44000)])
def test_attention_ragged_edges_long_batch(d, Hq, Hkv, long_len):
    rng = np.random.default_rng(d + Hq + 1)
    lens = [1, 2, 63, 64, 65, 0, 127, 128, 129, 300, 31, 33, long_len]
    cu, q, k, v, bias, gain = _attn_inputs(rng, lens, Hq, Hkv, d, torch.bfloat16)
    assert Hq * ((int(cu[-1]) + 255) // 256) >= 512
    cud = torch.from_numpy(cu).to(DEV)
    lo = int(cu[-2])
    rows = np.concatenate([np.arange(lo), lo + np.array([0, 1, 63, 64, 255, 256, 257, 4000]),
                           lo + long_len - 1 - np.arange(40)])
    rows = np.unique(rows[rows < int(cu[-1])])
    for tau, gg in [(1.15, gain), (1.0, None)]:
        o, lse = tg.tg_gated_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV),
                                      torch.from_numpy(bias).to(DEV),
                                      None if gg is None else torch.from_numpy(gg).to(DEV), tau,
                                      cud, max(lens), want_lse=True)
        torch.cuda.synchronize()
        _attn_check(o.cpu(), lse.cpu(), q, k, v, bias if gg is not None else None,
                    None if gg is None else gg.astype(np.float64), tau, cu, torch.bfloat16, rows)


# More prompts than one wave's lanes (100): both bf16 kernels' dispatch order
# counts each tile index's prompts 64 at a time (a ballot per group of 64
# prompts), so the second group and its empty prompts are exercised here, on
# the 256-row kernel (longer prompts) and on the key-split one (short
# prompts); every row is checked.
@pytest.mark.parametrize("max_len,big", [(260, True), (40, False)])
def test_attention_many_prompts(max_len, big):
    rng = np.random.default_rng(4242 + max_len)
    lens = [int(x) for x in rng.integers(0, max_len, 100)]
    lens[3] = lens[64] = lens[99] = 0
    lens[70] = 2 * max_len - 9
    cu, q, k, v, bias, gain = _attn_inputs(rng, lens, 16, 8, 128, torch.bfloat16)
    assert (16 * ((int(cu[-1]) + 255) // 256) >= 512) == big  # which kernel runs
    cud = torch.from_numpy(cu).to(DEV)
    o, lse = tg.tg_gated_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), torch.from_numpy(bias).to(DEV),
                                  torch.from_numpy(gain).to(DEV), 1.15, cud, max(lens), want_lse=True)
    torch.cuda.synchronize()
    _attn_check(o.cpu(), lse.cpu(), q, k, v, bias, gain.astype(np.float64), 1.15, cu, torch.bfloat16, None)


# Seeded random large batches (1-12 prompts up to 12000 rows, GQA shapes,
# d 64/128, bf16): mostly the 256-row kernel; every prompt's first and last
# 40 rows, each 256-row tile's first and last row and 300 random rows.
@pytest.mark.parametrize("seed", range(8))
def test_attention_large_random(seed):
    rng = np.random.default_rng(31000 + seed)
    Hq, Hkv = [(16, 8), (8, 1), (32, 8), (12, 4)][int(rng.integers(0, 4))]
    d = int(rng.choice([64, 128]))
    B = int(rng.integers(1, 13))
    lens = [int(x) for x in rng.integers(0, 12001, B)]
    if sum(lens) < 256:
        lens[0] = 5000
    print(f"[attn large {seed}] heads {Hq}/{Hkv} d={d} lens {lens}", flush=True)
    cu, q, k, v, bias, gain = _attn_inputs(rng, lens, Hq, Hkv, d, torch.bfloat16)
    Kt = int(cu[-1])
    rows = [rng.integers(0, Kt, 300)]
    for b in range(B):
        lo, hi = int(cu[b]), int(cu[b + 1])
        if hi > lo:
            t0 = np.arange(lo, hi, 256)
            rows += [np.arange(lo, min(hi, lo + 40)), np.arange(max(lo, hi - 40), hi), t0, np.minimum(t0 + 255, hi - 1)]
    rows = np.unique(np.concatenate(rows))
    tau = float(rng.uniform(0.6, 1.6))
    o, lse = tg.tg_gated_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), torch.from_numpy(bias).to(DEV),
                                  torch.from_numpy(gain).to(DEV), tau, torch.from_numpy(cu).to(DEV), max(lens),
                                  want_lse=True)
    torch.cuda.synchronize()
    _attn_check(o.cpu(), lse.cpu(), q, k, v, bias, gain.astype(np.float64), tau, cu, torch.bfloat16, rows)


def test_attention_properties_on_gpu():
    rng = np.random.default_rng(5)
    lens = [700, 1, 1500]
    Hq, Hkv, d = 16, 8, 128
    cu, q, k, v, bias, gain = _attn_inputs(rng, lens, Hq, Hkv, d, torch.bfloat16)
    cud = torch.from_numpy(cu).to(DEV)
    args = lambda vv, bb: (q.to(DEV), k.to(DEV), vv.to(DEV), torch.from_numpy(bb).to(DEV),  # noqa: E731
                           torch.from_numpy(gain).to(DEV), 1.15, cud, max(lens))
    # V = 1 -> O = 1 (softmax rows sum to one)
    o1, _ = tg.tg_gated_attn_fwd(*args(torch.ones_like(v), bias))
    torch.cuda.synchronize()
    assert torch.max(torch.abs(o1.cpu().float() - 1.0)).item() <= 2 ** -7
    # lse consistency: sum_j exp(x_j - lse) = 1, x recomputed in fp64 from the inputs
    o, lse = tg.tg_gated_attn_fwd(*args(v, bias), want_lse=True)
    torch.cuda.synchronize()
    lse = lse.cpu().numpy().astype(np.float64)
    Q, K = _f64(q), _f64(k)
    for r in [0, 5, 699, 700, 701, 2200]:
        b = int(np.searchsorted(cu, r, side="right") - 1)
        lo = int(cu[b])
        for h in [0, 7, 15]:
            x = 1.15 * (K[lo:r + 1, h // 2] @ Q[r, h]) / math.sqrt(d) + gain[h] * bias[lo:r + 1]
            assert abs(np.exp(x - lse[h, r]).sum() - 1.0) <= 1e-3
    # first kept row of each prompt sees only itself
    oc = o.cpu().float()
    for b in range(3):
        r = int(cu[b])
        assert torch.max(torch.abs(oc[r] - v[r].float().repeat_interleave(2, dim=0))).item() <= 2 ** -7
    # shifting every bias by c leaves O unchanged and moves each head's lse by
    # g_h c.  Against the GPU's own unshifted run: lse within 1e-4 of
    # lse + g_h c; O within 2e-3 plus what re-rounding can move (the two runs
    # compute each p in fp32 from different arguments, so a p near a bf16
    # rounding boundary may round the other way, one bf16 ulp, at most 2^-7
    # of p: 2^-7 sum_j P_j |v_j| in all; then the output's own rounding, one
    # bf16 ulp of the value); the mean difference below 1e-4 (a flip is rare);
    # and both runs within the bf16 bar of the oracle
    lse_t = torch.from_numpy(lse).float()
    ulp = lambda x: torch.exp2(torch.floor(torch.log2(x.abs().clamp_min(2.0 ** -126))) - 7)  # noqa: E731
    pv_abs, _ = oracle.gated_attention(_f64(q), _f64(k), np.abs(_f64(v)), bias, gain.astype(np.float64),
                                       1.15, cu)
    flip = torch.from_numpy(2.0 ** -7 * pv_abs).float()
    for c in [-7.5, 3.0]:
        oc2, lse2 = tg.tg_gated_attn_fwd(*args(v, (bias + c).astype(np.float32)), want_lse=True)
        torch.cuda.synchronize()
        _attn_check(oc2.cpu(), None, q, k, v, (bias + c).astype(np.float32), gain.astype(np.float64),
                    1.15, cu, torch.bfloat16, None)
        shift = torch.from_numpy((gain.astype(np.float64) * c)).float()[:, None]
        d_l = torch.abs(lse2.cpu() - lse_t - shift)
        assert d_l.max().item() <= 1e-4, d_l.max().item()
        d_o = torch.abs(oc2.cpu().float() - oc)
        assert torch.all(d_o <= 2e-3 + ulp(oc) + flip), (d_o - ulp(oc) - flip).max().item()
        assert d_o.mean().item() <= 1e-4, d_o.mean().item()
        _note(f"[shift {c}] lse max {d_l.max().item():.2e}, O max {d_o.max().item():.2e} "
              f"mean {d_o.mean().item():.2e}")
