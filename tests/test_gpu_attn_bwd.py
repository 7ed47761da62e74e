"""GPU parity of the token-gated attention backward through the C ABI
against the CPU fp64 oracle.

Parity cases feed the backward the oracle's forward output stored in the
input dtype (and its lse in fp32), and the oracle's backward uses the same
stored output for D_i = dout_i . out_i, as any backward that keeps the
forward's output does.  What is left between the two is the kernel's own
arithmetic, bounded per element from the exact P and dx of the same inputs:
  E_ij = P_ij [(2d + 8) 2^-24 (sum_e |dout_ie| |v_je| + sum_e |dout_ie| |out_ie|)
               + 2^-16 (|dout_i . v_j| + |D_i|)]
the absolute error of the kernel's fp32 dx_ij (the fp32 accumulation of its
two dot products, and P = exp2 of an fp32 argument less an fp32 lse, both up
to about 30, good to about 2^-17, doubled); r = 2^-8 for bf16 (P and dx are
rounded to bf16, unit roundoff 2^-9, before the second products; doubled), 0
for fp32; o = 2^-8 (bf16) or 2^-22 (fp32) for the output's own rounding;
c = tau / sqrt(d):
  dq_i:  c sum_j (E_ij + r |dx_ij|) |k_j| + o |ref|
  dk_j:  c sum_(h,i) (E_ij + r |dx_ij|) |q_i| + o |ref|
  dv_j:  sum_(h,i) (r + 2^-16) P_ij |dout_i| + o |ref|
  ds_j:  sum_h |g_h| sum_i (E_ij + 2^-16 |dx_ij|)
  dg_h:  sum_ij (E_ij + 2^-16 |dx_ij|) |s_j|
  dtau:  sum_(h,ij) (E_ij + 2^-16 |dx_ij|) |q_i.k_j| / sqrt(d)
Full size (the 128k workload's 8448 kept rows, 16 heads, GPU forward then
GPU backward): dq of sampled rows against the oracle's exact dq, the bar
adding c sum_j P_ij |delta_i| |k_j| for the forward output's own error
delta_i = dout_i . (out_i - o_i) at that row; dk, dv and dbias of sampled key
columns (tile edges and random) against the oracle's column form given the
GPU forward's output and lse, with the bars above restricted to the column;
and identities that hold at any size: sum_j dv_j = sum_(h in group, i)
dout_i, sum_j ds_j = 0, sum q.dq = sum k.dk = tau dtau.
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


def _note(msg):
    print(msg, flush=True)


def _f64(t):
    return t.detach().to("cpu").to(torch.float64).numpy()


def _scales(q, k, v, bias, gain, tau, cu, dout, out, r):
    """The bars above, from the exact P and dx (D from the stored output)."""
    Kt, Hq, d = q.shape
    Hkv = k.shape[1]
    grp = Hq // Hkv
    c = tau / math.sqrt(d)
    g = np.zeros(Hq) if gain is None else gain
    u16 = 2.0 ** -16
    t_dq = np.zeros((Kt, Hq, d))
    t_dk = np.zeros((Kt, Hkv, d))
    t_dv = np.zeros((Kt, Hkv, d))
    t_ds = np.zeros(Kt)
    t_dg = np.zeros(Hq)
    t_tau = 0.0
    for b in range(len(cu) - 1):
        lo, hi = cu[b], cu[b + 1]
        n = hi - lo
        if n == 0:
            continue
        vis = np.arange(n)[None, :] <= np.arange(n)[:, None]
        for h in range(Hq):
            kv = h // grp
            Q, K, V, G, O = q[lo:hi, h], k[lo:hi, kv], v[lo:hi, kv], dout[lo:hi, h], out[lo:hi, h]
            qk = Q @ K.T
            x = np.where(vis, c * qk + g[h] * bias[lo:hi][None, :], -np.inf)
            P = np.exp(x - x.max(axis=1, keepdims=True))
            P /= P.sum(axis=1, keepdims=True)
            dP = G @ V.T
            D = np.sum(G * O, axis=1, keepdims=True)
            adx = np.abs(P * (dP - D))
            E = P * ((2 * d + 8) * 2.0 ** -24 * (np.abs(G) @ np.abs(V).T + np.sum(np.abs(G) * np.abs(O), axis=1, keepdims=True))
                     + u16 * (np.abs(dP) + np.abs(D)))
            A = E + r * adx
            t_dq[lo:hi, h] = c * (A @ np.abs(K))
            t_dk[lo:hi, kv] += c * (A.T @ np.abs(Q))
            t_dv[lo:hi, kv] += (r + u16) * (P.T @ np.abs(G))
            B = E + u16 * adx
            t_ds[lo:hi] += abs(g[h]) * B.sum(axis=0)
            t_dg[h] += float(np.sum(B * np.abs(bias[lo:hi])[None, :]))
            t_tau += float(np.sum(B * np.abs(qk))) / math.sqrt(d)
    return t_dq, t_dk, t_dv, t_ds, t_dg, t_tau


def _inputs(lens, Hq, Hkv, d, dtype, seed, with_bias=True):
    g = torch.Generator().manual_seed(seed)
    Kt = int(sum(lens))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q = torch.randn((Kt, Hq, d), generator=g).to(dtype)
    k = torch.randn((Kt, Hkv, d), generator=g).to(dtype)
    v = torch.randn((Kt, Hkv, d), generator=g).to(dtype)
    dout = torch.randn((Kt, Hq, d), generator=g).to(dtype)
    bias = torch.randn(Kt, generator=g)
    bias[::7] = 0.0
    gain = (torch.rand(Hq, generator=g) * 1.5 + 0.5) if with_bias else None
    return cu, q, k, v, dout, bias, gain


def _dev_args(cu, q, k, v, dout, bias, gain):
    cud = torch.from_numpy(cu).to(DEV)
    mx = int(np.max(np.diff(cu), initial=0))
    gnd = None if gain is None else gain.to(DEV)
    return cud, mx, q.to(DEV), k.to(DEV), v.to(DEV), dout.to(DEV), bias.to(DEV), gnd


def _run_stored(cu, q, k, v, dout, bias, gain, tau, out, lse):
    """GPU backward on the given stored forward output and lse."""
    cud, mx, qd, kd, vd, gd, bd, gnd = _dev_args(cu, q, k, v, dout, bias, gain)
    grads = tg.tg_gated_attn_bwd(qd, kd, vd, bd, gnd, tau, cud, mx, out.to(DEV), lse.to(DEV), gd)
    torch.cuda.synchronize()
    return grads


def _run_chain(cu, q, k, v, dout, bias, gain, tau):
    """GPU forward, then GPU backward on its output."""
    cud, mx, qd, kd, vd, gd, bd, gnd = _dev_args(cu, q, k, v, dout, bias, gain)
    Kt, Hq = q.shape[0], q.shape[1]
    out, lse = tg.tg_gated_attn_fwd(qd, kd, vd, bd, gnd, tau, cud, mx,
                                    lse=torch.empty((Hq, Kt), device=DEV))
    grads = tg.tg_gated_attn_bwd(qd, kd, vd, bd, gnd, tau, cud, mx, out, lse, gd)
    torch.cuda.synchronize()
    return out, lse, grads


def _check_all(cu, q, k, v, dout, bias, gain, tau, grads, out_st, dtype):
    q64, k64, v64, g64, o64 = _f64(q), _f64(k), _f64(v), _f64(dout), _f64(out_st)
    b64 = _f64(bias)
    gn = None if gain is None else _f64(gain)
    ref = oracle.gated_attention_backward(q64, k64, v64, b64, gn, tau, cu, g64, out=o64)
    bf = dtype == torch.bfloat16
    r, o_r = (2.0 ** -8, 2.0 ** -8) if bf else (0.0, 2.0 ** -22)
    t = _scales(q64, k64, v64, b64, gn, tau, cu, g64, o64, r)
    names = ["dq", "dk", "dv", "dbias", "dgain", "dtau"]
    worst = {}
    for i, (name, got, exp, sc) in enumerate(zip(names, grads, ref, t)):
        got = _f64(got).reshape(np.shape(exp))
        exp = np.asarray(exp, dtype=np.float64)
        tol = (sc + o_r * np.abs(exp)) if i < 3 else np.asarray(sc) + 1e-6
        excess = np.abs(got - exp) - tol
        j = np.unravel_index(np.argmax(excess), excess.shape) if excess.ndim else ()
        assert excess[j] <= 0, f"{name}{j}: got {got[j]}, oracle {exp[j]}, tol {tol[j]}"
        worst[name] = float(np.max(np.abs(got - exp) / np.maximum(tol, 1e-30)))
    _note(f"  worst error / bar: {worst}")


# prompt lengths: ragged with a 1-row and an empty prompt, several 128-key
# and 64-row tiles per prompt; GQA groups of 1, 2, 3 and 8; d = 128 and 64
CASES = [
    ([300, 1, 399, 0, 300], 4, 2, 128, torch.bfloat16, True),
    ([130, 257], 3, 1, 64, torch.bfloat16, True),
    ([200, 77], 4, 4, 128, torch.bfloat16, False),
    ([20, 45], 4, 2, 64, torch.float32, True),
    ([33], 2, 1, 128, torch.float32, False),
    # GQA group 8 (one KV head): eight per-head partial sums per key in the
    # fixed-order group sum; a 64-row tail and a 128-key tile boundary
    ([320, 129], 8, 1, 128, torch.bfloat16, True),
    ([200], 8, 2, 64, torch.bfloat16, True),
]


@pytest.mark.parametrize("lens,Hq,Hkv,d,dtype,with_bias", CASES)
def test_attn_bwd_parity(lens, Hq, Hkv, d, dtype, with_bias):
    _note(f"[attn bwd] lens={lens} Hq={Hq} Hkv={Hkv} d={d} {dtype} bias={with_bias}")
    cu, q, k, v, dout, bias, gain = _inputs(lens, Hq, Hkv, d, dtype, seed=sum(lens) + d, with_bias=with_bias)
    tau = 1.15
    o, lse = oracle.gated_attention(_f64(q), _f64(k), _f64(v), _f64(bias),
                                    None if gain is None else _f64(gain), tau, cu)
    out_st = torch.from_numpy(np.nan_to_num(o)).to(dtype)
    lse_st = torch.from_numpy(np.nan_to_num(lse)).to(torch.float32)
    grads = _run_stored(cu, q, k, v, dout, bias, gain, tau, out_st, lse_st)
    _check_all(cu, q, k, v, dout, bias, gain, tau, grads, out_st, dtype)
    # bit-reproducible
    grads2 = _run_stored(cu, q, k, v, dout, bias, gain, tau, out_st, lse_st)
    for a, b in zip(grads, grads2):
        assert torch.equal(a, b)


@pytest.mark.parametrize("seed", range(12))
def test_attn_bwd_random(seed):
    """Seeded random shapes: 1-4 prompts of 0-420 rows, GQA groups 1-8, d
    64/128, bf16 and fp32, with and without the bias, tau 0.5-2."""
    rng = np.random.default_rng(7000 + seed)
    Hq, Hkv = [(4, 2), (8, 1), (6, 3), (2, 2), (16, 8)][int(rng.integers(0, 5))]
    d = int(rng.choice([64, 128]))
    dtype = torch.bfloat16 if rng.random() < 0.7 else torch.float32
    with_bias = bool(rng.random() < 0.75)
    lens = [int(x) for x in rng.integers(0, 421, int(rng.integers(1, 5)))]
    if sum(lens) == 0:
        lens[0] = 1
    tau = float(rng.uniform(0.5, 2.0))
    _note(f"[attn bwd random {seed}] lens={lens} Hq={Hq} Hkv={Hkv} d={d} {dtype} bias={with_bias} tau={tau:.3f}")
    cu, q, k, v, dout, bias, gain = _inputs(lens, Hq, Hkv, d, dtype, seed=100 + seed, with_bias=with_bias)
    o, lse = oracle.gated_attention(_f64(q), _f64(k), _f64(v), _f64(bias),
                                    None if gain is None else _f64(gain), tau, cu)
    out_st = torch.from_numpy(np.nan_to_num(o)).to(dtype)
    lse_st = torch.from_numpy(np.nan_to_num(lse)).to(torch.float32)
    grads = _run_stored(cu, q, k, v, dout, bias, gain, tau, out_st, lse_st)
    _check_all(cu, q, k, v, dout, bias, gain, tau, grads, out_st, dtype)


def test_attn_bwd_many_prompts():
    """100 prompts (three empty): the query- and key-parallel passes map
    their slots over the prompts 64 at a time, so the second group is
    exercised; every gradient element is checked."""
    rng = np.random.default_rng(99)
    lens = [int(x) for x in rng.integers(0, 200, 100)]
    lens[0] = lens[64] = lens[99] = 0
    lens[80] = 300
    _note(f"[attn bwd many] {len(lens)} prompts, {sum(lens)} rows")
    cu, q, k, v, dout, bias, gain = _inputs(lens, 4, 2, 64, torch.bfloat16, seed=77, with_bias=True)
    tau = 0.9
    o, lse = oracle.gated_attention(_f64(q), _f64(k), _f64(v), _f64(bias), _f64(gain), tau, cu)
    out_st = torch.from_numpy(np.nan_to_num(o)).to(torch.bfloat16)
    lse_st = torch.from_numpy(np.nan_to_num(lse)).to(torch.float32)
    grads = _run_stored(cu, q, k, v, dout, bias, gain, tau, out_st, lse_st)
    _check_all(cu, q, k, v, dout, bias, gain, tau, grads, out_st, torch.bfloat16)


def test_attn_bwd_full_size_128k():
    """The 128k workload's kept rows (one prompt of 8448 rows), 16 heads."""
    name = "qwen3_1p7b_128k"
    _note(f"[attn bwd full] {name}")
    w = synth.make_workload(name, seed=0, with_hidden=False)
    s = w.spec
    cu_kept, mx = oracle.plan(w.cu_seqlens, w.doc_begin, w.doc_end, w.budget)
    cu = np.asarray(cu_kept, dtype=np.int32)
    Kt = int(cu[-1])
    q, k, v, gain = synth.attention_inputs(s, 0, Kt, seed=0)
    g = torch.Generator().manual_seed(5)
    dout = torch.randn((Kt, s.Hq, s.d), generator=g).to(q.dtype)
    bias = torch.randn(Kt, generator=g)
    out, lse, grads = _run_chain(cu, q, k, v, dout, bias, gain, s.tau)
    dq, dk, dv, ds, dg, dt = (_f64(x) for x in grads)
    q64, k64, v64, g64, o64 = _f64(q), _f64(k), _f64(v), _f64(dout), _f64(out)
    b64, gn = _f64(bias), _f64(gain)
    # dq of sampled rows against the exact oracle
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 127, 128, Kt - 1], np.random.default_rng(0).integers(0, Kt, 40)]))
    ref = oracle.gated_attention_backward(q64, k64, v64, b64, gn, s.tau, cu, g64, rows=rows)[0]
    o_rows, _ = oracle.gated_attention(q64, k64, v64, b64, gn, s.tau, cu, rows=rows)
    c = s.tau / math.sqrt(s.d)
    grp = s.Hq // s.Hkv
    for i in rows:
        for h in range(s.Hq):
            K = k64[:i + 1, h // grp]
            x = c * (K @ q64[i, h]) + gn[h] * b64[:i + 1]
            P = np.exp(x - x.max())
            P /= P.sum()
            V = v64[:i + 1, h // grp]
            G = g64[i, h]
            dP, D = V @ G, float(G @ o_rows[i, h])
            dx = P * (dP - D)
            delta = abs(float(G @ (o64[i, h] - o_rows[i, h])))
            E = P * ((2 * s.d + 8) * 2.0 ** -24 * (np.abs(V) @ np.abs(G) + float(np.abs(G) @ np.abs(o64[i, h])))
                     + 2.0 ** -16 * (np.abs(dP) + abs(D)) + delta)
            tol = c * ((E + 2.0 ** -8 * np.abs(dx)) @ np.abs(K)) + 2.0 ** -8 * np.abs(ref[i, h])
            err = np.abs(dq[i, h] - ref[i, h])
            assert np.all(err <= tol), f"dq row {i} head {h}: max err {err.max()}, bar {tol[np.argmax(err)]}"
    # dk, dv and the bias gradient of sampled key columns, element by element,
    # against the oracle's column form given the GPU forward's stored output
    # and lse (what the backward receives); bars as in _scales, per column
    cols = np.unique(np.concatenate([[0, 1, 63, 64, 127, 128, 4095, 4096, Kt - 65, Kt - 64, Kt - 2, Kt - 1],
                                     np.random.default_rng(1).integers(0, Kt, 20)]))
    lse64 = _f64(lse)
    rk, rv, rs = oracle.gated_attention_backward_columns(q64, k64, v64, b64, gn, s.tau, cu, g64, o64,
                                                         lse64, cols)
    r = 2.0 ** -8
    for n, j in enumerate(cols):
        t_k = np.zeros((s.Hkv, s.d))
        t_v = np.zeros((s.Hkv, s.d))
        t_s = 0.0
        for h in range(s.Hq):
            kv = h // grp
            Q, G, O = q64[j:, h], g64[j:, h], o64[j:, h]
            x = c * (Q @ k64[j, kv]) + gn[h] * b64[j]
            P = np.exp(x - lse64[h, j:])
            dP, D = G @ v64[j, kv], np.sum(G * O, axis=1)
            adx = np.abs(P * (dP - D))
            E = P * ((2 * s.d + 8) * 2.0 ** -24 * (np.abs(G) @ np.abs(v64[j, kv]) + np.sum(np.abs(G) * np.abs(O), axis=1))
                     + 2.0 ** -16 * (np.abs(dP) + np.abs(D)))
            t_k[kv] += c * ((E + r * adx) @ np.abs(Q))
            t_v[kv] += (r + 2.0 ** -16) * (P @ np.abs(G))
            t_s += abs(gn[h]) * float(np.sum(E + 2.0 ** -16 * adx))
        for name, got, ref_, bar in (("dk", dk[j], rk[n], t_k + r * np.abs(rk[n])),
                                     ("dv", dv[j], rv[n], t_v + r * np.abs(rv[n])),
                                     ("dbias", ds[j], rs[n], t_s + 1e-6)):
            err = np.abs(got - ref_)
            assert np.all(err <= bar), f"{name} column {j}: max err {np.max(err)}, bar {np.min(bar)}"
    _note(f"  columns {len(cols)}: dk, dv, dbias element-wise within their bars")
    # identities that hold at any size
    for kv in range(s.Hkv):
        lhs = dv[:, kv].sum(axis=0)
        rhs = g64[:, kv * grp:(kv + 1) * grp].sum(axis=(0, 1))
        bar = 2.0 ** -7 * (np.abs(g64[:, kv * grp:(kv + 1) * grp]).sum(axis=(0, 1)) + np.abs(dv[:, kv]).sum(axis=0))
        assert np.all(np.abs(lhs - rhs) <= bar), f"sum dv, kv head {kv}"
    # each row of dx sums to zero up to the stored output's error in D_i
    assert abs(ds.sum()) <= 1e-2 * float(np.abs(ds).sum()), (ds.sum(), np.abs(ds).sum())
    tq = float(np.sum(q64 * dq))
    tk = float(np.sum(k64 * dk))
    tt = s.tau * float(dt[0])
    scale = float(np.sum(np.abs(q64) * np.abs(dq)))
    assert abs(tq - tt) <= 2e-2 * scale and abs(tk - tt) <= 2e-2 * scale, (tq, tk, tt, scale)
    _note(f"  tau*dtau {tt:.4g}, sum q.dq {tq:.4g}, sum k.dk {tk:.4g}")
