"""GPU parity of the rest of a pruned layer (RMSNorm, the projection added
to the residual, the SwiGLU activation) through the C ABI, against the CPU
fp64 oracle, each kernel on the GPU's own inputs; and a whole pruned layer
chained on the device.

Bars (written here; u = 2^-24 the fp32 unit roundoff, "bf16 term"
2^-8 (1 + 2^-6) |ref| the one rounding of the output, absent for fp32):
  * rms_norm: |Δ| <= bf16 term + (D + 16) u |ref|  (fp32 sum of squares
    over D terms, root, division and two products).
  * linear_residual: |Δ| <= bf16 term + 2 (K + 4) u (S + |r|), S the sum
    of |a_k| |W_nk| and r the residual: twice the worst-case fp32
    accumulation bound of the dot product and the residual add.
  * swiglu: |Δ| <= bf16 term + 1.1 |u_j| E_g + |silu(g_j)| E_u + 2^-19 |ref|,
    E_g, E_u = 2 (D + 4) u S_g, S_u the accumulation bounds of the two dot
    products (|silu'| <= 1.1), 2^-19 for the exponential and reciprocal.
  * whole layer (bf16 intermediates rounded at every step): the relative
    2-norm error of the layer's update y - x below 3e-2 against the fp64
    oracle layer; and step by step, each intermediate element-wise at its
    own step's bar against the oracle step fed the GPU's previous output
    (q/k/v and attention at the bars of their own tests), with the in-place
    pipeline layer bit-identical to the steps.
Full size: the 128k-token workload's 8448 kept rows at the Qwen3-1.7B
shapes (D 2048, Hq d 2048, I 6144), in the benchmark's launch
configuration, on sampled rows.
"""

import numpy as np
import pytest
import torch

import learned_token_pruning_score_amd as tg
import oracle
import synth

pytestmark = pytest.mark.gpu

DEV = "cuda"
U = 2.0 ** -24


def _note(msg):
    print(msg, flush=True)


def _f64(t):
    return t.detach().to("cpu").to(torch.float64).numpy()


def _rel(dtype):
    return 2.0 ** -8 * (1 + 2.0 ** -6) if dtype == torch.bfloat16 else 0.0


def _assert_within(got, ref, tol, what):
    excess = np.abs(got - ref) - tol
    i = np.unravel_index(np.argmax(excess), excess.shape)
    assert excess[i] <= 0, f"{what}{tuple(int(j) for j in i)}: got {got[i]}, oracle {ref[i]}, tol {tol[i]}"


def _rand(shape, dtype, g, scale=1.0):
    return (torch.randn(shape, generator=g) * scale).to(dtype)


# ------------------------------------------------------------------ rms_norm

@pytest.mark.parametrize("n,D,dtype,mode", [
    (1000, 2048, torch.bfloat16, "plain"), (37, 256, torch.float32, "plain"),
    (300, 520, torch.bfloat16, "strided"), (9, 8, torch.float32, "inplace"),
    (64, 2048, torch.bfloat16, "inplace")])
def test_rms_norm(n, D, dtype, mode):
    _note(f"[rms_norm] n={n} D={D} {dtype} {mode}")
    g = torch.Generator().manual_seed(n + D)
    pad = 24 if mode == "strided" else 0
    x = _rand((n, D + pad), dtype, g) * torch.exp(torch.randn((n, 1), generator=g)).to(dtype)
    x[0, :] = 0  # a zero row normalises to zero
    if n > 2:
        x[1, :D] = (x[1, :D].float() * 1e4).to(dtype)
    w = torch.rand(D, generator=g) + 0.5
    eps = 1e-6
    xd = x.to(DEV)[:, :D]
    if mode == "inplace":
        y = tg.tg_rms_norm(xd, w.to(DEV), eps, out=xd)
    else:
        y = tg.tg_rms_norm(xd, w.to(DEV), eps)
    torch.cuda.synchronize()
    ref = oracle.rms_norm(_f64(x[:, :D]), _f64(w), eps)
    tol = _rel(dtype) * np.abs(ref) + (D + 16) * U * np.abs(ref)
    _assert_within(_f64(y), ref, tol, "rms_norm")
    assert torch.all(y[0] == 0)


# ----------------------------------------------------------- linear_residual

def _lr_check(got, a, W, r, dtype):
    a64, W64, r64 = _f64(a), _f64(W), _f64(r)
    ref = oracle.linear_residual(a64, W64, r64)
    S = np.abs(a64) @ np.abs(W64).T
    K = a64.shape[1]
    tol = _rel(dtype) * np.abs(ref) + 2 * (K + 4) * U * (S + np.abs(r64))
    _assert_within(_f64(got), ref, tol, "linear_residual")


# (n, K, N, mode): the attention output projection at 1000 rows (32 tiles:
# sub-tiles only) and at the 128k kept rows (264 tiles: a full round plus 8
# tiles as sub-tiles); the down projection (K = 6144) at 1200 rows (40
# tiles); 4352 rows (136 tiles: tile kernel only); small and in-place cases.
@pytest.mark.parametrize("n,K,N,mode", [
    (1000, 2048, 2048, "plain"), (8448, 2048, 2048, "sampled"), (1200, 6144, 2048, "plain"),
    (4352, 2048, 2048, "sampled"), (77, 128, 64, "plain"), (300, 256, 192, "inplace")])
def test_linear_residual_bf16(n, K, N, mode):
    _note(f"[linear_residual] n={n} K={K} N={N} {mode}")
    g = torch.Generator().manual_seed(n + K + N)
    a = _rand((n, K), torch.bfloat16, g)
    W = _rand((N, K), torch.bfloat16, g, K ** -0.5)
    r = _rand((n, N), torch.bfloat16, g, 2.0)
    rd = r.to(DEV)
    if mode == "inplace":
        y = tg.tg_linear_residual(a.to(DEV), W.to(DEV), rd, out=rd)
    else:
        y = tg.tg_linear_residual(a.to(DEV), W.to(DEV), rd)
    torch.cuda.synchronize()
    if mode == "sampled":
        rows = np.unique(np.concatenate([[0, 255, n - 257, n - 256, n - 1],
                                         np.random.default_rng(n).integers(0, n, 100),
                                         np.random.default_rng(n + 1).integers(n - 256, n, 30)]))
        idx = torch.from_numpy(rows)
        _lr_check(y.cpu()[idx], a[idx], W, r[idx], torch.bfloat16)
    else:
        _lr_check(y.cpu(), a, W, r, torch.bfloat16)
    y2 = tg.tg_linear_residual(a.to(DEV), W.to(DEV), r.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(y2, y)  # bit-reproducible, in place or not


@pytest.mark.parametrize("n,K,N", [(40, 256, 64), (3, 96, 5)])
def test_linear_residual_f32(n, K, N):
    g = torch.Generator().manual_seed(n)
    a, W, r = _rand((n, K), torch.float32, g), _rand((N, K), torch.float32, g), _rand((n, N), torch.float32, g)
    y = tg.tg_linear_residual(a.to(DEV), W.to(DEV), r.to(DEV))
    torch.cuda.synchronize()
    _lr_check(y.cpu(), a, W, r, torch.float32)


# -------------------------------------------------------------------- swiglu

def _sw_check(got, h, Wg, Wu, dtype):
    h64, g64, u64 = _f64(h), _f64(Wg), _f64(Wu)
    ref = oracle.swiglu(h64, g64, u64)
    gv, uv = h64 @ g64.T, h64 @ u64.T
    D = h64.shape[1]
    Eg = 2 * (D + 4) * U * (np.abs(h64) @ np.abs(g64).T)
    Eu = 2 * (D + 4) * U * (np.abs(h64) @ np.abs(u64).T)
    silu = gv / (1 + np.exp(-gv))
    tol = _rel(dtype) * np.abs(ref) + 1.1 * np.abs(uv) * Eg + np.abs(silu) * Eu + 2.0 ** -19 * np.abs(ref)
    _assert_within(_f64(got), ref, tol, "swiglu")


# (n, D, I): the MLP shape at 1000 rows (192 tiles: tile kernel only) and at
# the 128k kept rows (1584 tiles: six rounds plus 48 tiles as sub-tiles);
# I = 96 (a partial 128-row weight tile); small.
@pytest.mark.parametrize("n,D,I,sampled", [
    (1000, 2048, 6144, False), (8448, 2048, 6144, True), (70, 64, 96, False), (260, 512, 160, False)])
def test_swiglu_bf16(n, D, I, sampled):
    _note(f"[swiglu] n={n} D={D} I={I}")
    g = torch.Generator().manual_seed(n + D + I)
    h = _rand((n, D), torch.bfloat16, g)
    Wg = _rand((I, D), torch.bfloat16, g, 2 * D ** -0.5)
    Wu = _rand((I, D), torch.bfloat16, g, D ** -0.5)
    y = tg.tg_swiglu(h.to(DEV), Wg.to(DEV), Wu.to(DEV))
    torch.cuda.synchronize()
    if sampled:
        rows = np.unique(np.concatenate([[0, n - 1], np.random.default_rng(n).integers(0, n, 60),
                                         np.random.default_rng(n + 1).integers(n - 256, n, 30)]))
        idx = torch.from_numpy(rows)
        _sw_check(y.cpu()[idx], h[idx], Wg, Wu, torch.bfloat16)
    else:
        _sw_check(y.cpu(), h, Wg, Wu, torch.bfloat16)


@pytest.mark.parametrize("n,D,I", [(30, 256, 96), (2, 8, 3)])
def test_swiglu_f32(n, D, I):
    g = torch.Generator().manual_seed(n + I)
    h, Wg, Wu = _rand((n, D), torch.float32, g), _rand((I, D), torch.float32, g), _rand((I, D), torch.float32, g)
    y = tg.tg_swiglu(h.to(DEV), Wg.to(DEV), Wu.to(DEV))
    torch.cuda.synchronize()
    _sw_check(y.cpu(), h, Wg, Wu, torch.float32)


# ------------------------------------------------------------- whole layer

@pytest.mark.parametrize("name", ["ragged_small_bf16", "ragged_tiny_fp32"])
def test_pruned_layer_chain(name):
    _note(f"[pruned layer] {name}")
    w = synth.make_workload(name, seed=2)
    s = w.spec
    gp = tg.GatedPrefill(w.cu_seqlens, w.doc_begin, w.doc_end, w.budget, s.D, w.dtype)
    gp.gate_and_select(w.hidden.to(DEV), w.W1.to(DEV), w.b1.to(DEV), w.w2.to(DEV), w.b2)
    gp.rope(s.d, s.rope_theta)
    Wqkv = synth.qkv_weights(name, 0, seed=2)
    lw = synth.layer_weights(name, 0, seed=2)
    gain = torch.linspace(0.5, 2.0, s.Hq)
    x0 = gp.hidden_k.cpu()
    y = gp.pruned_layer(Wqkv.to(DEV), {k: v.to(DEV) for k, v in lw.items()}, s.Hq, s.Hkv, s.d,
                        gain.to(DEV), s.tau, s.norm_eps)
    torch.cuda.synchronize()
    Kt = gp.Kt
    rows = np.unique(np.concatenate([[0, Kt - 1], np.random.default_rng(2).integers(0, Kt, 150)]))
    ref = oracle.pruned_layer(_f64(x0), gp.pos_k.cpu().numpy(), gp.cu_kept_h, gp.bias_s.cpu().numpy(),
                              _f64(gain), s.tau, s.rope_theta, s.norm_eps, _f64(lw["w_in"]),
                              _f64(Wqkv), s.Hq, s.Hkv, s.d, _f64(lw["W_o"]), _f64(lw["w_post"]),
                              _f64(lw["W_gate"]), _f64(lw["W_up"]), _f64(lw["W_down"]), rows=rows)
    upd_ref = ref - _f64(x0)[rows]
    upd = _f64(y.cpu())[rows] - _f64(x0)[rows]
    err = np.linalg.norm(upd - upd_ref) / np.linalg.norm(upd_ref)
    _note(f"  relative error of the layer update: {err:.2e}")
    assert err <= 3e-2


@pytest.mark.parametrize("name", ["ragged_small_bf16", "ragged_tiny_fp32"])
def test_pruned_layer_steps(name):
    """The layer one call at a time, every intermediate in its own buffer:
    each step checked element-wise against the oracle step fed the GPU's
    previous output, at the bars above (q/k/v and attention at their own
    tests' bars), and the in-place pipeline bit-identical to the steps."""
    from test_gpu_parity import _attn_check
    from test_gpu_qkv import THETA, _check_qkv
    _note(f"[pruned layer, step by step] {name}")
    w = synth.make_workload(name, seed=3)
    s = w.spec
    assert s.rope_theta == THETA
    dt = w.dtype
    gp = tg.GatedPrefill(w.cu_seqlens, w.doc_begin, w.doc_end, w.budget, s.D, dt)
    gp.gate_and_select(w.hidden.to(DEV), w.W1.to(DEV), w.b1.to(DEV), w.w2.to(DEV), w.b2)
    gp.rope(s.d, s.rope_theta)
    Wqkv = synth.qkv_weights(name, 0, seed=3).to(DEV)
    lw = {k: v.to(DEV) for k, v in synth.layer_weights(name, 0, seed=3).items()}
    gain = torch.linspace(0.5, 2.0, s.Hq)
    Kt, Hq, Hkv, d = gp.Kt, s.Hq, s.Hkv, s.d
    x0 = gp.hidden_k.clone()
    xn1 = tg.tg_rms_norm(x0, lw["w_in"], s.norm_eps)
    qkv, q, k, v = tg.tg_qkv_rope(xn1, Wqkv, gp.rope_table, Hq, Hkv, d)
    att, lse = gp.attend(q, k, v, gain.to(DEV), s.tau, lse=torch.empty((Hq, Kt), device=DEV))
    x1 = tg.tg_linear_residual(att.view(Kt, Hq * d), lw["W_o"], x0)
    xn2 = tg.tg_rms_norm(x1, lw["w_post"], s.norm_eps)
    act = tg.tg_swiglu(xn2, lw["W_gate"], lw["W_up"])
    y = tg.tg_linear_residual(act, lw["W_down"], x1)
    torch.cuda.synchronize()
    cpu = {n: t.cpu() for n, t in dict(x0=x0, xn1=xn1, qkv=qkv, q=q, k=k, v=v, att=att, lse=lse, x1=x1,
                                       xn2=xn2, act=act, y=y).items()}
    for xin, wn, xout in (("x0", "w_in", "xn1"), ("x1", "w_post", "xn2")):
        ref = oracle.rms_norm(_f64(cpu[xin]), _f64(lw[wn]), s.norm_eps)
        tol = _rel(dt) * np.abs(ref) + (s.D + 16) * U * np.abs(ref)
        _assert_within(_f64(cpu[xout]), ref, tol, f"rms_norm {xout}")
    _check_qkv(cpu["qkv"], cpu["xn1"], Wqkv.cpu(), gp.pos_k.cpu().numpy(), Hq, Hkv, d, dt)
    _attn_check(cpu["att"], cpu["lse"], cpu["q"], cpu["k"], cpu["v"], gp.bias_s.cpu().numpy().astype(np.float64),
                _f64(gain), s.tau, gp.cu_kept_h, dt, None)
    _lr_check(cpu["x1"], cpu["att"].reshape(Kt, Hq * d), lw["W_o"].cpu(), cpu["x0"], dt)
    _sw_check(cpu["act"], cpu["xn2"], lw["W_gate"].cpu(), lw["W_up"].cpu(), dt)
    _lr_check(cpu["y"], cpu["act"], lw["W_down"].cpu(), cpu["x1"], dt)
    # the pipeline's in-place layer runs the same launches on the same inputs
    x_pipe = x0.clone()
    y_pipe = gp.pruned_layer(Wqkv, lw, Hq, Hkv, d, gain.to(DEV), s.tau, s.norm_eps, x=x_pipe)
    torch.cuda.synchronize()
    assert torch.equal(y_pipe, y)
