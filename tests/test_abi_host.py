"""Host side of the C ABI, on the CPU: the library loads, exports every symbol
that include/tg.h declares, plans kept sizes like the oracle, and rejects
invalid calls with the documented status before any device work.

Only calls that return during argument checking are made here (no GPU in
this container): each one fails a check that comes before the launch.
"""

import ctypes
import os
import re

import numpy as np
import pytest

import learned_token_pruning_score_amd as tg
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tg.h")

TG_OK, TG_ERR_NULL, TG_ERR_SHAPE, TG_ERR_DTYPE, TG_ERR_RANGE = 0, -1, -2, -3, -4
TG_ERR_ALIGN, TG_ERR_UNSUPPORTED, TG_ERR_WORKSPACE = -5, -6, -7

FAKE = 0x100000  # 16-byte aligned, never dereferenced: every call below fails a check first


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tg_\w+)\s*\(", src)))


def test_every_declared_symbol_is_exported_and_typed():
    lib = tg.load_library()
    names = _declared()
    assert "tg_sample_budgets" in names and "tg_swiglu" in names and len(names) == 24
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(tg.SIGNATURES)


def test_abi_version_and_status_strings():
    assert tg.tg_abi_version() == 1
    for s in range(-8, 1):
        assert tg.status_string(s) and tg.status_string(s) != "unknown status"
    assert tg.status_string(-99) == "unknown status"


def test_plan_matches_oracle_on_random_batches():
    rng = np.random.default_rng(0)
    for _ in range(200):
        B = int(rng.integers(1, 9))
        lens = rng.integers(0, 5000, size=B)
        cu = np.concatenate([[0], np.cumsum(lens)])
        db = np.array([rng.integers(0, n + 1) for n in lens])
        de = np.array([rng.integers(a, n + 1) for a, n in zip(db, lens)])
        bud = rng.integers(0, 6000, size=B)
        got, mx = tg.tg_plan(cu, db, de, bud)
        want, wmx = oracle.plan(cu, db, de, bud)
        assert got.tolist() == want.tolist() and mx == wmx


def _plan_status(cu, db, de, bud):
    lib = tg.load_library()
    cu = np.ascontiguousarray(cu, np.int32)
    db = np.ascontiguousarray(db, np.int32)
    de = np.ascontiguousarray(de, np.int32)
    bud = np.ascontiguousarray(bud, np.int32)
    out = np.full(len(bud) + 1, -7, np.int32)
    mx = ctypes.c_int32(-7)
    p = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))  # noqa: E731
    st = lib.tg_plan(len(bud), p(cu), p(db), p(de), p(bud), p(out), ctypes.byref(mx))
    return st, out, mx.value


def test_plan_rejects_bad_metadata_without_writing():
    cases = [
        ([1, 10], [0], [5], [3]),        # cu_seqlens[0] != 0
        ([0, 10, 5], [0, 0], [5, 0], [3, 1]),  # decreasing
        ([0, 10], [6], [5], [3]),        # doc_end < doc_begin
        ([0, 10], [0], [11], [3]),       # doc past prompt end
        ([0, 10], [-1], [5], [3]),       # negative begin
        ([0, 10], [0], [5], [-1]),       # negative budget
    ]
    for cu, db, de, bud in cases:
        st, out, mx = _plan_status(cu, db, de, bud)
        assert st == TG_ERR_SHAPE, (cu, db, de, bud)
        assert np.all(out == -7) and mx == -7  # no side effects
    lib = tg.load_library()
    assert lib.tg_plan(-1, None, None, None, None, None, None) == TG_ERR_SHAPE
    assert lib.tg_plan(1, None, None, None, None, None, None) == TG_ERR_NULL


def test_gate_score_argument_checks():
    lib = tg.load_library()
    f = lib.tg_gate_score
    # (hidden, ld, T, D, W1, b1, w2, b2, F, dtype, scores, stream)
    assert f(FAKE, 2048, 10, 2048, FAKE, None, FAKE, 0.0, 256, 7, FAKE, None) == TG_ERR_DTYPE
    assert f(FAKE, 100, 10, 2048, FAKE, None, FAKE, 0.0, 256, 1, FAKE, None) == TG_ERR_SHAPE
    assert f(FAKE, 2048, -1, 2048, FAKE, None, FAKE, 0.0, 256, 1, FAKE, None) == TG_ERR_SHAPE
    assert f(FAKE, 2048, 10, 2048, FAKE, None, FAKE, float("nan"), 256, 1, FAKE, None) == TG_ERR_RANGE
    assert f(None, 2048, 10, 2048, FAKE, None, FAKE, 0.0, 256, 1, FAKE, None) == TG_ERR_NULL
    assert f(FAKE, 2048, 10, 2048, FAKE, None, None, 0.0, 256, 1, FAKE, None) == TG_ERR_NULL
    assert f(FAKE, 2048, 10, 2048, FAKE, None, FAKE, 0.0, 100, 1, FAKE, None) == TG_ERR_UNSUPPORTED
    # bf16 needs D % 8 == 0 (whole 16-byte chunks); any D for fp32
    assert f(FAKE, 2048, 10, 1004, FAKE, None, FAKE, 0.0, 256, 1, FAKE, None) == TG_ERR_UNSUPPORTED
    assert f(FAKE, 2048, 10, 1, FAKE, None, FAKE, 0.0, 256, 1, FAKE, None) == TG_ERR_UNSUPPORTED
    assert f(FAKE + 2, 2048, 10, 2048, FAKE, None, FAKE, 0.0, 256, 1, FAKE, None) == TG_ERR_ALIGN
    assert f(FAKE, 2049 + 3, 10, 2048, FAKE, None, FAKE, 0.0, 256, 1, FAKE, None) == TG_ERR_ALIGN
    assert f(FAKE, 256, 10, 256, FAKE, None, FAKE, 0.0, 2000, 0, FAKE, None) == TG_ERR_UNSUPPORTED
    # T == 0 is a valid no-op with no device work
    assert f(None, 2048, 0, 2048, None, None, None, 0.0, 256, 1, None, None) == TG_OK


def test_select_and_compact_argument_checks():
    lib = tg.load_library()
    need = tg.tg_select_topk_workspace(3, 1000)
    assert need >= 3 * 2048 * 4
    s = lib.tg_select_topk
    # (scores, cu, db, de, budget, B, T, keep, ws, ws_bytes, stream)
    assert s(FAKE, FAKE, FAKE, FAKE, FAKE, -1, 10, FAKE, FAKE, need, None) == TG_ERR_SHAPE
    assert s(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 10, FAKE, FAKE, need, None) == TG_ERR_SHAPE
    assert s(FAKE, None, FAKE, FAKE, FAKE, 3, 1000, FAKE, FAKE, need, None) == TG_ERR_NULL
    assert s(FAKE, FAKE, FAKE, FAKE, FAKE, 3, 1000, FAKE, FAKE, need - 1, None) == TG_ERR_WORKSPACE
    assert s(FAKE, FAKE, FAKE, FAKE, FAKE, 3, 1000, FAKE, None, need, None) == TG_ERR_WORKSPACE
    assert s(FAKE, FAKE, FAKE, FAKE, FAKE, 3, 1000, FAKE, FAKE + 4, need, None) == TG_ERR_ALIGN
    assert s(None, None, None, None, None, 0, 0, None, None, 0, None) == TG_OK
    big = tg.tg_select_topk_workspace(65536, 70000)
    assert s(FAKE, FAKE, FAKE, FAKE, FAKE, 65536, 70000, FAKE, FAKE, big, None) == TG_ERR_UNSUPPORTED
    cneed = tg.tg_compact_workspace(3, 1000)
    c = lib.tg_compact
    # (hidden, ld, D, dtype, pos, scores, keep, cu, db, de, B, T, Kt, hk, pk, bk, ik, ws, wsb, stream)
    args = [FAKE, 2048, 2048, 1, None, FAKE, FAKE, FAKE, FAKE, FAKE, 3, 1000, 100, FAKE, FAKE,
            FAKE, None, FAKE, cneed, None]

    def call(**kw):
        a = list(args)
        names = ["hidden", "ld", "D", "dtype", "pos", "scores", "keep", "cu", "db", "de", "B",
                 "T", "Kt", "hk", "pk", "bk", "ik", "ws", "wsb", "stream"]
        for k, v in kw.items():
            a[names.index(k)] = v
        return c(*a)

    assert call(dtype=5) == TG_ERR_DTYPE
    assert call(Kt=1001) == TG_ERR_SHAPE
    assert call(ld=100) == TG_ERR_SHAPE
    assert call(keep=None) == TG_ERR_NULL
    assert call(hk=None) == TG_ERR_NULL
    assert call(wsb=cneed - 1) == TG_ERR_WORKSPACE
    assert call(hidden=FAKE + 1) == TG_ERR_ALIGN
    assert call(hk=FAKE + 3, dtype=0, D=2048) == TG_ERR_ALIGN


def test_attention_argument_checks():
    lib = tg.load_library()
    a = lib.tg_gated_attn_fwd
    # (q, k, v, qs, ks, vs, bias, gain, tau, cu, B, maxlen, Kt, Hq, Hkv, d, dtype, out, lse, stream)
    base = [FAKE, FAKE, FAKE, 2048, 1024, 1024, FAKE, FAKE, 1.15, FAKE, 1, 100, 100, 16, 8, 128,
            1, FAKE, None, None]
    names = ["q", "k", "v", "qs", "ks", "vs", "bias", "gain", "tau", "cu", "B", "maxlen", "Kt",
             "Hq", "Hkv", "d", "dtype", "out", "lse", "stream"]

    def call(**kw):
        x = list(base)
        for k, v in kw.items():
            x[names.index(k)] = v
        return a(*x)

    assert call(dtype=9) == TG_ERR_DTYPE
    assert call(Hkv=6) == TG_ERR_SHAPE
    assert call(qs=2000) == TG_ERR_SHAPE
    assert call(maxlen=101) == TG_ERR_SHAPE
    assert call(tau=float("inf")) == TG_ERR_RANGE
    assert call(tau=0.0) == TG_ERR_RANGE and call(tau=-1.0) == TG_ERR_RANGE
    assert call(d=96, qs=96 * 16, ks=96 * 8, vs=96 * 8) == TG_ERR_UNSUPPORTED
    assert call(q=None) == TG_ERR_NULL
    assert call(bias=None) == TG_ERR_NULL  # gain given without bias
    assert call(k=FAKE + 2) == TG_ERR_ALIGN
    assert call(vs=1028) == TG_ERR_ALIGN
    assert call(B=0) == TG_OK and call(Kt=0, maxlen=0) == TG_OK  # valid no-ops
    # launch-grid limits: prompts, 256-row query tiles (bf16), heads (fp32)
    assert call(B=65536, Kt=70000, maxlen=100) == TG_ERR_UNSUPPORTED
    assert call(Kt=65536 * 256 + 1, maxlen=65536 * 256 + 1) == TG_ERR_UNSUPPORTED
    assert call(dtype=0, Hq=65536, Hkv=1, qs=65536 * 128) == TG_ERR_UNSUPPORTED


def test_rope_table_and_qkv_argument_checks():
    lib = tg.load_library()
    r = lib.tg_rope_table
    # (pos, Kt, d, theta, table, stream)
    assert r(FAKE, -1, 128, 1e6, FAKE, None) == TG_ERR_SHAPE
    assert r(FAKE, 10, 127, 1e6, FAKE, None) == TG_ERR_SHAPE
    assert r(FAKE, 10, 128, float("nan"), FAKE, None) == TG_ERR_RANGE
    assert r(FAKE, 10, 128, 1.0, FAKE, None) == TG_ERR_RANGE
    assert r(FAKE, 10, 96, 1e6, FAKE, None) == TG_ERR_UNSUPPORTED
    assert r(None, 10, 128, 1e6, FAKE, None) == TG_ERR_NULL
    assert r(FAKE, 10, 128, 1e6, FAKE + 8, None) == TG_ERR_ALIGN
    assert r(None, 0, 128, 1e6, None, None) == TG_OK  # empty: no device work

    q = lib.tg_qkv_rope
    # (x, ld_x, Kt, D, w, table, Hq, Hkv, d, dtype, qkv, ld_qkv, stream)
    base = [FAKE, 2048, 100, 2048, FAKE, FAKE, 16, 8, 128, 1, FAKE, 4096, None]
    names = ["x", "ld_x", "Kt", "D", "w", "table", "Hq", "Hkv", "d", "dtype", "qkv", "ld_qkv",
             "stream"]

    def call(**kw):
        a = list(base)
        for k, v in kw.items():
            a[names.index(k)] = v
        return q(*a)

    assert call(dtype=5) == TG_ERR_DTYPE
    assert call(ld_x=2000) == TG_ERR_SHAPE
    assert call(ld_qkv=4095) == TG_ERR_SHAPE
    assert call(Hkv=0) == TG_ERR_SHAPE and call(Kt=-1) == TG_ERR_SHAPE
    assert call(d=96, ld_qkv=4096) == TG_ERR_UNSUPPORTED
    assert call(D=1000, ld_x=1000) == TG_ERR_UNSUPPORTED  # bf16: D % 64
    assert call(ld_x=1 << 22) == TG_ERR_UNSUPPORTED  # 32-bit stage offsets
    assert call(dtype=0, Kt=1 << 20) == TG_ERR_UNSUPPORTED  # fp32: one thread per output
    assert call(x=None) == TG_ERR_NULL and call(table=None) == TG_ERR_NULL
    assert call(qkv=None) == TG_ERR_NULL and call(w=None) == TG_ERR_NULL
    assert call(x=FAKE + 2) == TG_ERR_ALIGN and call(table=FAKE + 4) == TG_ERR_ALIGN
    assert call(ld_x=2052) == TG_ERR_ALIGN and call(ld_qkv=4100) == TG_ERR_ALIGN
    assert call(Kt=0, x=None, w=None, table=None, qkv=None) == TG_OK  # empty: no device work


def test_layer_argument_checks():
    lib = tg.load_library()
    r = lib.tg_rms_norm
    # (x, ld_x, n, D, weight, eps, dtype, out, ld_out, stream)
    assert r(FAKE, 2048, 10, 2048, FAKE, 1e-6, 4, FAKE, 2048, None) == TG_ERR_DTYPE
    assert r(FAKE, 2000, 10, 2048, FAKE, 1e-6, 1, FAKE, 2048, None) == TG_ERR_SHAPE
    assert r(FAKE, 2048, 10, 2048, FAKE, -1.0, 1, FAKE, 2048, None) == TG_ERR_RANGE
    assert r(FAKE, 2048, 10, 2048, FAKE, float("nan"), 1, FAKE, 2048, None) == TG_ERR_RANGE
    assert r(FAKE, 2044, 10, 2044, FAKE, 1e-6, 1, FAKE, 2044, None) == TG_ERR_UNSUPPORTED
    assert r(FAKE, 2048, 10, 2048, None, 1e-6, 1, FAKE, 2048, None) == TG_ERR_NULL
    assert r(FAKE, 2048, 10, 2048, FAKE, 1e-6, 1, FAKE, 4096, None) == TG_ERR_SHAPE  # aliased, other stride
    assert r(FAKE, 2050, 10, 2048, FAKE, 1e-6, 0, FAKE + 64 * 1024, 2048, None) == TG_ERR_ALIGN
    assert r(None, 2048, 0, 2048, None, 1e-6, 1, None, 2048, None) == TG_OK

    lr = lib.tg_linear_residual
    # (a, ld_a, n, K, W, N, res, ld_res, dtype, out, ld_out, stream)
    assert lr(FAKE, 2048, 10, 2048, FAKE, 2048, FAKE, 2048, 2, FAKE, 2048, None) == TG_ERR_DTYPE
    assert lr(FAKE, 1000, 10, 2048, FAKE, 2048, FAKE, 2048, 1, FAKE, 2048, None) == TG_ERR_SHAPE
    assert lr(FAKE, 2048, 10, 2048, FAKE, 2048, FAKE, 2000, 1, FAKE + 4096, 2048, None) == TG_ERR_SHAPE
    assert lr(FAKE, 2048, 10, 2048, FAKE, 2016, FAKE, 2048, 1, FAKE + 4096, 2048, None) == TG_ERR_UNSUPPORTED
    assert lr(FAKE, 2000, 10, 2000, FAKE, 2048, FAKE, 2048, 1, FAKE + 4096, 2048, None) == TG_ERR_UNSUPPORTED
    assert lr(FAKE, 2048, 10, 2048, FAKE, 2048, FAKE, 2048, 1, FAKE, 4096, None) == TG_ERR_SHAPE  # aliased
    assert lr(FAKE, 2048, 10, 2048, None, 2048, FAKE, 2048, 1, FAKE + 4096, 2048, None) == TG_ERR_NULL
    assert lr(FAKE, 2052, 10, 2048, FAKE, 2048, FAKE, 2048, 1, FAKE + 4096, 2048, None) == TG_ERR_ALIGN
    assert lr(FAKE, 2048, 1 << 20, 2048, FAKE, 4096, FAKE, 4096, 0, FAKE + 64, 4096, None) == TG_ERR_UNSUPPORTED
    assert lr(None, 2048, 0, 2048, None, 2048, None, 2048, 1, None, 2048, None) == TG_OK

    sw = lib.tg_swiglu
    # (h, ld_h, n, D, w_gate, w_up, I, dtype, out, ld_out, stream)
    assert sw(FAKE, 2048, 10, 2048, FAKE, FAKE, 6144, 3, FAKE, 6144, None) == TG_ERR_DTYPE
    assert sw(FAKE, 2048, 10, 2048, FAKE, FAKE, 6144, 1, FAKE, 6000, None) == TG_ERR_SHAPE
    assert sw(FAKE, 2048, 10, 2048, FAKE, FAKE, 6000, 1, FAKE, 6000, None) == TG_ERR_UNSUPPORTED
    assert sw(FAKE, 2048, 10, 2048, FAKE, None, 6144, 1, FAKE, 6144, None) == TG_ERR_NULL
    assert sw(FAKE, 2048, 10, 2048, FAKE, FAKE + 8, 6144, 1, FAKE, 6144, None) == TG_ERR_ALIGN
    assert sw(None, 2048, 0, 2048, None, None, 6144, 1, None, 6144, None) == TG_OK



def test_sample_budgets_matches_oracle_and_rejects():
    rng = np.random.default_rng(61)
    B = 300
    db = rng.integers(0, 100, B).astype(np.int32)
    de = (db + rng.integers(0, 40000, B)).astype(np.int32)
    u = rng.random(B).astype(np.float32)
    for lo, hi in ((0.0, 1.0), (0.05, 0.3), (1.0, 1.0), (0.5, 0.5)):
        got = tg.tg_sample_budgets(db, de, u, lo, hi)
        exp = oracle.sample_budgets(db, de, u.astype(np.float64), np.float32(lo), np.float32(hi))
        assert np.array_equal(got, exp), (lo, hi)
    lib = tg.load_library()
    f = lib.tg_sample_budgets
    one = (ctypes.c_int32 * 1)(0)
    ten = (ctypes.c_int32 * 1)(10)
    uu = (ctypes.c_float * 1)(0.5)
    out = (ctypes.c_int32 * 1)(-7)
    assert f(1, one, ten, uu, 0.6, 0.4, out) == TG_ERR_RANGE and out[0] == -7
    assert f(1, one, ten, uu, -0.1, 0.4, out) == TG_ERR_RANGE
    assert f(1, one, ten, (ctypes.c_float * 1)(1.0), 0.1, 0.4, out) == TG_ERR_RANGE
    assert f(1, ten, one, uu, 0.1, 0.4, out) == TG_ERR_SHAPE
    assert f(1, None, ten, uu, 0.1, 0.4, out) == TG_ERR_NULL
    assert f(0, None, None, None, 0.1, 0.4, None) == TG_OK


def test_attention_backward_workspace_and_argument_checks():
    import torch
    lib = tg.load_library()
    # bf16 with several query heads per KV head adds the per-head fp32 dK and
    # dV sums (2 Hq Kt d floats); one head per group and fp32 need none
    w_g2 = tg.tg_gated_attn_bwd_workspace(1, 1000, 4, 2, 128, torch.bfloat16, 1000)
    w_g1 = tg.tg_gated_attn_bwd_workspace(1, 1000, 4, 4, 128, torch.bfloat16, 1000)
    w_f32 = tg.tg_gated_attn_bwd_workspace(1, 1000, 4, 2, 128, torch.float32, 1000)
    assert w_g2 - w_g1 == 2 * 4 * 1000 * 128 * 4
    assert w_f32 == w_g1
    with pytest.raises(tg.TokenGateError):
        tg.tg_gated_attn_bwd_workspace(1, 1000, 4, 3, 128, torch.bfloat16, 1000)
    with pytest.raises(TypeError):
        tg.tg_gated_attn_bwd_workspace(1, 1000, 4, 2, 128, torch.float16, 1000)
    n = ctypes.c_size_t(0)
    assert lib.tg_gated_attn_bwd_workspace(1, 1000, 4, 2, 128, 7, 1000, ctypes.byref(n)) == TG_ERR_DTYPE
    assert lib.tg_gated_attn_bwd_workspace(1, 1000, 4, 2, 128, 1, 1000, None) == TG_ERR_NULL

    need = tg.tg_gated_attn_bwd_workspace(1, 100, 16, 8, 128, torch.bfloat16, 100)
    f = lib.tg_gated_attn_bwd
    names = ["q", "k", "v", "qs", "ks", "vs", "bias", "gain", "tau", "cu", "B", "maxlen", "Kt", "Hq", "Hkv",
             "d", "dtype", "out", "lse", "dout", "dq", "dk", "dv", "dbias", "dgain", "dtau", "ws", "wsb",
             "stream"]
    base = [FAKE, FAKE, FAKE, 2048, 1024, 1024, FAKE, FAKE, 1.15, FAKE, 1, 100, 100, 16, 8, 128, 1, FAKE,
            FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None, FAKE, need, None]

    def call(**kw):
        x = list(base)
        for k, v in kw.items():
            x[names.index(k)] = v
        return f(*x)

    assert call(dtype=9) == TG_ERR_DTYPE
    assert call(Hkv=6) == TG_ERR_SHAPE
    assert call(qs=2000) == TG_ERR_SHAPE
    assert call(maxlen=101) == TG_ERR_SHAPE
    assert call(tau=float("nan")) == TG_ERR_RANGE and call(tau=0.0) == TG_ERR_RANGE
    assert call(d=96, qs=96 * 16, ks=96 * 8, vs=96 * 8) == TG_ERR_UNSUPPORTED
    assert call(B=0) == TG_OK and call(Kt=0, maxlen=0) == TG_OK  # valid no-ops
    assert call(dout=None) == TG_ERR_NULL
    assert call(bias=None) == TG_ERR_NULL  # gain given without bias
    assert call(wsb=need - 1) == TG_ERR_WORKSPACE and call(ws=None) == TG_ERR_WORKSPACE
    assert call(ws=FAKE + 8) == TG_ERR_ALIGN
    assert call(dk=FAKE + 2) == TG_ERR_ALIGN
    assert call(ks=1028) == TG_ERR_ALIGN


def test_gate_backward_argument_checks():
    import torch
    lib = tg.load_library()
    need = tg.tg_gate_bwd_workspace(500, 2048, 256, torch.bfloat16)
    assert need > 0
    # no kept rows: a finite workspace (an earlier layout divided by a zero chunk size)
    assert tg.tg_gate_bwd_workspace(0, 2048, 256, torch.bfloat16) >= 0
    assert tg.tg_gate_bwd_workspace(0, 2048, 256, torch.float32) >= 0
    with pytest.raises(TypeError):
        tg.tg_gate_bwd_workspace(500, 2048, 256, torch.float16)
    f = lib.tg_gate_bwd
    names = ["h", "ld", "Kt", "D", "W1", "b1", "w2", "F", "dbias", "kidx", "cu", "db", "de", "B", "dtype",
             "dh", "dW1", "db1", "dw2", "db2", "ws", "wsb", "stream"]
    base = [FAKE, 2048, 500, 2048, FAKE, FAKE, FAKE, 256, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, FAKE, FAKE,
            FAKE, FAKE, FAKE, FAKE, need, None]

    def call(**kw):
        x = list(base)
        for k, v in kw.items():
            x[names.index(k)] = v
        return f(*x)

    assert call(dtype=9) == TG_ERR_DTYPE
    assert call(ld=1000) == TG_ERR_SHAPE
    assert call(B=0) == TG_ERR_SHAPE  # rows but no prompts
    assert call(F=100) == TG_ERR_UNSUPPORTED
    assert call(D=100, ld=100) == TG_ERR_UNSUPPORTED  # bf16 needs D % 64 == 0
    assert call(W1=None) == TG_ERR_NULL and call(db2=None) == TG_ERR_NULL
    assert call(wsb=need - 1) == TG_ERR_WORKSPACE
    assert call(kidx=None) == TG_ERR_NULL
    assert call(w2=FAKE + 4) == TG_ERR_ALIGN
    assert call(h=FAKE + 2) == TG_ERR_ALIGN and call(ld=2052) == TG_ERR_ALIGN


def test_workspace_queries_at_zero_sizes():
    import torch
    assert tg.tg_select_topk_workspace(0, 0) >= 0 and tg.tg_select_topk_workspace(3, 0) >= 0
    assert tg.tg_compact_workspace(0, 0) >= 0
    assert tg.tg_gated_attn_bwd_workspace(0, 0, 4, 2, 128, torch.bfloat16, 0) >= 0
    assert tg.tg_decode_attn_workspace(0, 4, 128, 0) >= 0 and tg.tg_decode_attn_workspace(2, 4, 64, 0) >= 0


def test_decode_argument_checks():
    lib = tg.load_library()
    sc = lib.tg_kv_scatter
    # (k, v, ks, vs, bias, cu, B, Kt, Hkv, d, dtype, kc, vc, cks, cvs, bc, start, stream)
    assert sc(FAKE, FAKE, 1024, 1024, None, FAKE, 1, 10, 8, 128, 9, FAKE, FAKE, 1024, 1024, FAKE, FAKE, None) \
        == TG_ERR_DTYPE
    assert sc(FAKE, FAKE, 1000, 1024, None, FAKE, 1, 10, 8, 128, 1, FAKE, FAKE, 1024, 1024, FAKE, FAKE, None) \
        == TG_ERR_SHAPE
    assert sc(FAKE, FAKE, 1024, 1024, None, FAKE, 0, 10, 8, 128, 1, FAKE, FAKE, 1024, 1024, FAKE, FAKE, None) \
        == TG_ERR_SHAPE
    assert sc(FAKE, FAKE, 1024, 1024, None, FAKE, 1, 0, 8, 128, 1, FAKE, FAKE, 1024, 1024, FAKE, FAKE, None) \
        == TG_OK
    assert sc(FAKE, FAKE, 1024, 1024, None, FAKE, 1, 10, 8, 128, 1, FAKE, FAKE, 1024, 1024, None, FAKE, None) \
        == TG_ERR_NULL
    ap = lib.tg_kv_append
    # (k_new, v_new, B, Hkv, d, dtype, kc, vc, cks, cvs, bc, start, pos, stream)
    assert ap(FAKE, FAKE, 2, 8, 128, 9, FAKE, FAKE, 1024, 1024, FAKE, FAKE, FAKE, None) == TG_ERR_DTYPE
    assert ap(FAKE, FAKE, 2, 8, 128, 1, FAKE, FAKE, 1000, 1024, FAKE, FAKE, FAKE, None) == TG_ERR_SHAPE
    assert ap(FAKE, FAKE, 0, 8, 128, 1, FAKE, FAKE, 1024, 1024, FAKE, FAKE, FAKE, None) == TG_OK
    assert ap(FAKE, FAKE, 2, 8, 128, 1, FAKE, FAKE, 1024, 1024, FAKE, FAKE, None, None) == TG_ERR_NULL
    need = tg.tg_decode_attn_workspace(2, 16, 128, 5000)
    assert need > 0
    de = lib.tg_decode_attn
    names = ["q", "kc", "vc", "cks", "cvs", "bc", "gain", "tau", "start", "lens", "B", "maxlen", "Hq", "Hkv",
             "d", "dtype", "out", "lse", "ws", "wsb", "stream"]
    base = [FAKE, FAKE, FAKE, 1024, 1024, FAKE, FAKE, 1.15, FAKE, FAKE, 2, 5000, 16, 8, 128, 1, FAKE, None,
            FAKE, need, None]

    def call(**kw):
        x = list(base)
        for k, v in kw.items():
            x[names.index(k)] = v
        return de(*x)

    assert call(dtype=9) == TG_ERR_DTYPE
    assert call(Hkv=6) == TG_ERR_SHAPE and call(cks=1000) == TG_ERR_SHAPE
    assert call(tau=0.0) == TG_ERR_RANGE
    assert call(d=96, cks=768, cvs=768) == TG_ERR_UNSUPPORTED
    assert call(Hq=32, Hkv=2, cks=256, cvs=256) == TG_ERR_UNSUPPORTED  # 16 query heads per KV head
    assert call(B=0) == TG_OK
    assert call(q=None) == TG_ERR_NULL and call(bc=None) == TG_ERR_NULL  # gain without bias
    assert call(wsb=need - 1) == TG_ERR_WORKSPACE
    assert call(q=FAKE + 2) == TG_ERR_ALIGN and call(cks=1028) == TG_ERR_ALIGN


def test_select_noalloc_argument_checks():
    lib = tg.load_library()
    f = FAKE
    # same checks as tg_select_topk, all before any device work
    assert lib.tg_select_topk_noalloc(f, None, f, f, f, 1, 100, f, None) == TG_ERR_NULL
    assert lib.tg_select_topk_noalloc(None, f, f, f, f, 1, 100, f, None) == TG_ERR_NULL
    assert lib.tg_select_topk_noalloc(f, f, f, f, f, 1, 100, None, None) == TG_ERR_NULL
    assert lib.tg_select_topk_noalloc(f, f, f, f, f, -1, 100, f, None) == TG_ERR_SHAPE
    assert lib.tg_select_topk_noalloc(f, f, f, f, f, 0, 100, f, None) == TG_ERR_SHAPE
    assert lib.tg_select_topk_noalloc(f, f, f, f, f, 1, 1 << 31, f, None) == TG_ERR_SHAPE
    assert lib.tg_select_topk_noalloc(f, f, f, f, f, 70000, 100000, f, None) == TG_ERR_UNSUPPORTED
    assert lib.tg_select_topk_noalloc(None, None, None, None, None, 0, 0, None, None) == TG_OK
    # the static scratch holds 4 MiB: 300 prompts over 40000 tokens need the
    # chunked path's 4.96 MB workspace and are rejected before any launch
    assert tg.tg_select_topk_workspace(300, 40000) > (4 << 20)
    assert lib.tg_select_topk_noalloc(f, f, f, f, f, 300, 40000, f, None) == TG_ERR_WORKSPACE
    # the largest single-prompt workspace (64 chunks) fits
    assert tg.tg_select_topk_workspace(1, 1 << 30) <= (4 << 20)
