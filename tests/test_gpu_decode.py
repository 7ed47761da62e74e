"""GPU parity of decode over the kept-only KV cache through the C ABI
against the CPU fp64 oracle: the cache copies (bit-exact) and the decode
attention step.

Decode bar per element (the kernel works in fp32 throughout: an exp2 of an
fp32 logit and fp32 sums, good to about 2^-17 of sum_j P_j |v_j|; the output
is then rounded once):
  out:  |Δ| <= 2^-16 sum_j P_j |v_j| + r |ref|   (r = 2^-8 (1 + 2^-6) bf16, 2^-22 fp32)
  lse:  |Δ| <= 2^-16 max(1, |lse|)
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


def _check_decode(out, lse, q, kc, vc, bc, start, lens, gain, tau, dtype):
    o_ref, lse_ref = oracle.decode_attention(_f64(q), _f64(kc), _f64(vc), _f64(bc), start, lens,
                                             None if gain is None else _f64(gain), tau)
    Q, K, V, S = _f64(q), _f64(kc), _f64(vc), _f64(bc)
    B, Hq, d = Q.shape
    grp = Hq // K.shape[1]
    g = np.zeros(Hq) if gain is None else _f64(gain)
    r = 2.0 ** -8 * (1 + 2.0 ** -6) if dtype == torch.bfloat16 else 2.0 ** -22
    got, gl = _f64(out), _f64(lse)
    worst = 0.0
    for b in range(B):
        lo, n = int(start[b]), int(lens[b])
        for h in range(Hq):
            x = tau / math.sqrt(d) * (K[lo:lo + n, h // grp] @ Q[b, h]) + g[h] * S[lo:lo + n]
            P = np.exp(x - x.max())
            P /= P.sum()
            tol = 2.0 ** -16 * (P @ np.abs(V[lo:lo + n, h // grp])) + r * np.abs(o_ref[b, h])
            err = np.abs(got[b, h] - o_ref[b, h])
            assert np.all(err <= tol), f"out[{b},{h}]: max err {err.max()}, bar {tol[np.argmax(err)]}"
            worst = max(worst, float(np.max(err / tol)))
            assert abs(gl[b, h] - lse_ref[b, h]) <= 2.0 ** -16 * max(1.0, abs(lse_ref[b, h])), (b, h)
    return worst


def _cache(rows, Hkv, d, dtype, g):
    kc = torch.randn((rows, Hkv, d), generator=g).to(dtype)
    vc = torch.randn((rows, Hkv, d), generator=g).to(dtype)
    bc = torch.randn(rows, generator=g)
    bc[::5] = 0.0
    return kc, vc, bc


# (sequence lengths, Hq, Hkv, d, dtype): ragged with a one-key sequence and
# split boundaries (256 keys); GQA groups 1, 2, 3, 8; d 128 and 64; fp32
CASES = [
    ([700, 1, 300], 16, 8, 128, torch.bfloat16, True),
    ([257, 1024], 6, 2, 64, torch.bfloat16, True),
    ([5000], 8, 1, 128, torch.bfloat16, False),
    ([33, 260], 4, 4, 64, torch.float32, True),
]


@pytest.mark.parametrize("lens,Hq,Hkv,d,dtype,with_bias", CASES)
def test_decode_attn_parity(lens, Hq, Hkv, d, dtype, with_bias):
    _note(f"[decode] lens={lens} Hq={Hq} Hkv={Hkv} d={d} {dtype}")
    g = torch.Generator().manual_seed(sum(lens) + Hq)
    gap = 37
    start = np.cumsum([0] + [n + gap for n in lens[:-1]]).astype(np.int32)
    rows = int(start[-1] + lens[-1] + gap)
    kc, vc, bc = _cache(rows, Hkv, d, dtype, g)
    q = torch.randn((len(lens), Hq, d), generator=g).to(dtype)
    gain = torch.rand(Hq, generator=g) * 1.5 + 0.5 if with_bias else None
    tau = 1.15
    out, lse = tg.tg_decode_attn(q.to(DEV), kc.to(DEV), vc.to(DEV), bc.to(DEV),
                                 None if gain is None else gain.to(DEV), tau,
                                 torch.from_numpy(start).to(DEV), torch.tensor(lens, dtype=torch.int32, device=DEV),
                                 max(lens), lse=torch.empty((len(lens), Hq), device=DEV))
    torch.cuda.synchronize()
    w = _check_decode(out, lse, q, kc, vc, bc if with_bias else torch.zeros_like(bc), start, lens, gain, tau, dtype)
    _note(f"  worst error / bar {w:.3f}")


@pytest.mark.parametrize("seed", range(12))
def test_decode_attn_random(seed):
    """Seeded random caches: 1-40 sequences of 1-3000 keys (some at split
    boundaries), random gaps between them, GQA groups 1-8, d 64/128, bf16 and
    fp32, with and without the bias, tau 0.5-2."""
    rng = np.random.default_rng(8000 + seed)
    Hq, Hkv = [(16, 8), (8, 1), (6, 3), (4, 4), (2, 1)][int(rng.integers(0, 5))]
    d = int(rng.choice([64, 128]))
    dtype = torch.bfloat16 if rng.random() < 0.7 else torch.float32
    with_bias = bool(rng.random() < 0.75)
    B = int(rng.integers(1, 41))
    lens = [int(x) for x in rng.integers(1, 3001, B)]
    for j in range(B):
        if rng.random() < 0.15:
            lens[j] = int(rng.choice([1, 128, 129, 255, 256, 257, 512]))
    gaps = [int(x) for x in rng.integers(0, 50, B)]
    start = np.cumsum([0] + [n + gp for n, gp in zip(lens[:-1], gaps[:-1])]).astype(np.int32)
    rows = int(start[-1] + lens[-1] + gaps[-1])
    tau = float(rng.uniform(0.5, 2.0))
    _note(f"[decode random {seed}] B={B} max len {max(lens)} Hq={Hq} Hkv={Hkv} d={d} {dtype} bias={with_bias}")
    g = torch.Generator().manual_seed(300 + seed)
    kc, vc, bc = _cache(rows, Hkv, d, dtype, g)
    q = torch.randn((B, Hq, d), generator=g).to(dtype)
    gain = torch.rand(Hq, generator=g) * 1.5 + 0.5 if with_bias else None
    out, lse = tg.tg_decode_attn(q.to(DEV), kc.to(DEV), vc.to(DEV), bc.to(DEV),
                                 None if gain is None else gain.to(DEV), tau,
                                 torch.from_numpy(start).to(DEV), torch.tensor(lens, dtype=torch.int32, device=DEV),
                                 max(lens), lse=torch.empty((B, Hq), device=DEV))
    torch.cuda.synchronize()
    w = _check_decode(out, lse, q, kc, vc, bc if with_bias else torch.zeros_like(bc), start, lens, gain, tau, dtype)
    _note(f"  worst error / bar {w:.3f}")


@pytest.mark.parametrize("dtype,d,pad_src,pad_dst,offset", [
    (torch.bfloat16, 128, 0, 0, 0),   # 16-byte units
    (torch.bfloat16, 64, 8, 16, 0),   # padded rows, still whole 16-byte units
    (torch.bfloat16, 128, 4, 0, 0),   # source rows 8 bytes past a unit: element copy
    (torch.bfloat16, 64, 0, 0, 1),    # cache one element off 16-byte alignment: element copy
    (torch.float32, 64, 0, 4, 0),     # fp32, 16-byte units
    (torch.float32, 128, 1, 0, 0),    # fp32, source stride 4 bytes past a unit: element copy
])
def test_kv_scatter_layouts(dtype, d, pad_src, pad_dst, offset):
    """tg_kv_scatter against the cache built on the host, bit for bit, for
    the 16-byte copy and the element copy it falls back to."""
    rng = np.random.default_rng(d + pad_src + pad_dst + offset)
    Hkv = 4
    lens = [int(x) for x in rng.integers(0, 300, 7)]
    lens[2] = 0
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    Kt, B = int(cu[-1]), len(lens)
    room = 5
    start = (cu[:-1] + np.arange(B) * room).astype(np.int32)
    rows = Kt + B * room
    row = Hkv * d
    g = torch.Generator().manual_seed(3)
    ksrc = torch.randn((Kt, row + pad_src), generator=g).to(dtype)
    vsrc = torch.randn((Kt, row + pad_src), generator=g).to(dtype)
    bias = torch.randn(Kt, generator=g)
    view = lambda t: t.as_strided((Kt, Hkv, d), (row + pad_src, d, 1))  # noqa: E731  token rows of row + pad_src
    k, v = view(ksrc), view(vsrc)
    kd, vd = view(ksrc.to(DEV)), view(vsrc.to(DEV))
    n_el = rows * (row + pad_dst) + offset
    kbuf = torch.full((n_el,), 7, dtype=dtype, device=DEV)
    vbuf = torch.full((n_el,), 7, dtype=dtype, device=DEV)
    kc = kbuf[offset:].as_strided((rows, Hkv, d), (row + pad_dst, d, 1))
    vc = vbuf[offset:].as_strided((rows, Hkv, d), (row + pad_dst, d, 1))
    bc = torch.full((rows,), 9.0, device=DEV)
    tg.tg_kv_scatter(kd, vd, bias.to(DEV), torch.from_numpy(cu).to(DEV), kc, vc, bc, torch.from_numpy(start).to(DEV))
    torch.cuda.synchronize()
    Kh = torch.full((rows, Hkv, d), 7, dtype=dtype)
    Vh = torch.full((rows, Hkv, d), 7, dtype=dtype)
    Bh = torch.full((rows,), 9.0)
    for b in range(B):
        n = lens[b]
        Kh[start[b]:start[b] + n] = k[cu[b]:cu[b + 1]]
        Vh[start[b]:start[b] + n] = v[cu[b]:cu[b + 1]]
        Bh[start[b]:start[b] + n] = bias[cu[b]:cu[b + 1]]
    bits = torch.int16 if dtype == torch.bfloat16 else torch.int32
    assert torch.equal(kc.cpu().view(bits), Kh.view(bits))
    assert torch.equal(vc.cpu().view(bits), Vh.view(bits))
    assert torch.equal(bc.cpu(), Bh)
    if pad_dst:  # the padding between cache rows is untouched
        pad = kbuf.cpu()[offset:].reshape(rows, row + pad_dst)[:, row:]
        assert torch.all(pad.float() == 7.0)


def test_decode_steps_from_prefill_cache():
    """The ragged workload's kept layout: the prefill's kept k, v and bias
    scattered into a cache with room per sequence, then 5 decode steps each
    appending a token (bias 0) and attending over the whole cache."""
    name = "ragged_small_bf16"
    _note(f"[decode steps] {name}")
    w = synth.make_workload(name, seed=4, with_hidden=False)
    s = w.spec
    cu_kept, _ = oracle.plan(w.cu_seqlens, w.doc_begin, w.doc_end, w.budget)
    cu = np.asarray(cu_kept, dtype=np.int64)
    B, Kt = len(cu) - 1, int(cu[-1])
    q0, k0, v0, gain = synth.attention_inputs(s, 0, Kt, seed=4)
    g = torch.Generator().manual_seed(4)
    bias0 = torch.randn(Kt, generator=g)
    steps = 5
    start = (cu[:-1] + np.arange(B) * steps).astype(np.int32)
    rows = Kt + B * steps
    kc = torch.zeros((rows, s.Hkv, s.d), dtype=k0.dtype, device=DEV)
    vc = torch.zeros_like(kc)
    bc = torch.full((rows,), 9.0, device=DEV)
    startd = torch.from_numpy(start).to(DEV)
    tg.tg_kv_scatter(k0.to(DEV), v0.to(DEV), bias0.to(DEV), torch.from_numpy(cu.astype(np.int32)).to(DEV),
                     kc, vc, bc, startd)
    # the same cache built on the host
    Kh = torch.zeros((rows, s.Hkv, s.d), dtype=k0.dtype)
    Vh = torch.zeros_like(Kh)
    Bh = torch.full((rows,), 9.0)
    for b in range(B):
        n = int(cu[b + 1] - cu[b])
        Kh[start[b]:start[b] + n] = k0[cu[b]:cu[b + 1]]
        Vh[start[b]:start[b] + n] = v0[cu[b]:cu[b + 1]]
        Bh[start[b]:start[b] + n] = bias0[cu[b]:cu[b + 1]]
    lens = np.diff(cu).astype(np.int32)
    for step in range(steps):
        kn = torch.randn((B, s.Hkv, s.d), generator=g).to(k0.dtype)
        vn = torch.randn((B, s.Hkv, s.d), generator=g).to(k0.dtype)
        qn = torch.randn((B, s.Hq, s.d), generator=g).to(k0.dtype)
        tg.tg_kv_append(kn.to(DEV), vn.to(DEV), kc, vc, bc, startd, torch.from_numpy(lens).to(DEV))
        for b in range(B):
            Kh[start[b] + lens[b]] = kn[b]
            Vh[start[b] + lens[b]] = vn[b]
            Bh[start[b] + lens[b]] = 0.0
        lens = lens + 1
        out, lse = tg.tg_decode_attn(qn.to(DEV), kc, vc, bc, gain.to(DEV), s.tau, startd,
                                     torch.from_numpy(lens).to(DEV), int(lens.max()),
                                     lse=torch.empty((B, s.Hq), device=DEV))
        torch.cuda.synchronize()
        assert torch.equal(kc.cpu(), Kh) and torch.equal(vc.cpu(), Vh) and torch.equal(bc.cpu(), Bh), step
        _check_decode(out, lse, qn, Kh, Vh, Bh, start, lens, gain, s.tau, k0.dtype)


def test_decode_long_splits():
    """32 sequences of 3000-4096 keys over 4 KV heads: enough workgroups that
    the step takes 256-key splits (one partial per 256 keys)."""
    _note("[decode] 32 sequences, 256-key splits")
    g = torch.Generator().manual_seed(12)
    lens = [4096 - 37 * i for i in range(32)]
    Hq, Hkv, d = 8, 4, 64
    start = np.cumsum([0] + lens[:-1]).astype(np.int32)
    rows = int(start[-1] + lens[-1])
    kc, vc, bc = _cache(rows, Hkv, d, torch.bfloat16, g)
    q = torch.randn((len(lens), Hq, d), generator=g).to(torch.bfloat16)
    gain = torch.rand(Hq, generator=g) + 0.5
    out, lse = tg.tg_decode_attn(q.to(DEV), kc.to(DEV), vc.to(DEV), bc.to(DEV), gain.to(DEV), 1.15,
                                 torch.from_numpy(start).to(DEV), torch.tensor(lens, dtype=torch.int32, device=DEV),
                                 max(lens), lse=torch.empty((len(lens), Hq), device=DEV))
    torch.cuda.synchronize()
    w = _check_decode(out, lse, q, kc, vc, bc, start, lens, gain, 1.15, torch.bfloat16)
    _note(f"  worst error / bar {w:.3f}")


@pytest.mark.parametrize("n,Hq,Hkv,d,dtype", [
    (65536, 16, 8, 128, torch.bfloat16),   # one long sequence at the 1.7B head shapes
    (131072, 8, 4, 64, torch.float32),
])
def test_decode_long_splits_one_sequence(n, Hq, Hkv, d, dtype):
    """One sequence long enough for 256-key splits (Hkv * n / 256 >= 2048
    workgroups), d = 128 and fp32."""
    _note(f"[decode] one sequence of {n} keys, {Hq}/{Hkv} heads, d={d}, {dtype}")
    assert Hkv * (n // 256) >= 2048
    g = torch.Generator().manual_seed(n + d)
    kc, vc, bc = _cache(n, Hkv, d, dtype, g)
    q = torch.randn((1, Hq, d), generator=g).to(dtype)
    gain = torch.rand(Hq, generator=g) + 0.5
    start, lens = np.array([0], dtype=np.int32), [n]
    out, lse = tg.tg_decode_attn(q.to(DEV), kc.to(DEV), vc.to(DEV), bc.to(DEV), gain.to(DEV), 1.15,
                                 torch.from_numpy(start).to(DEV), torch.tensor(lens, dtype=torch.int32, device=DEV),
                                 n, lse=torch.empty((1, Hq), device=DEV))
    torch.cuda.synchronize()
    w = _check_decode(out, lse, q, kc, vc, bc, start, lens, gain, 1.15, dtype)
    _note(f"  worst error / bar {w:.3f}")


def test_decode_full_size_128k():
    """One decode step over the 128k workload's 8448 kept keys, 16 heads."""
    _note("[decode full] 8448 keys")
    g = torch.Generator().manual_seed(8)
    n, Hq, Hkv, d = 8448, 16, 8, 128
    kc, vc, bc = _cache(n + 64, Hkv, d, torch.bfloat16, g)
    q = torch.randn((1, Hq, d), generator=g).to(torch.bfloat16)
    gain = torch.rand(Hq, generator=g) + 0.5
    start, lens = np.array([0], dtype=np.int32), [n]
    out, lse = tg.tg_decode_attn(q.to(DEV), kc.to(DEV), vc.to(DEV), bc.to(DEV), gain.to(DEV), 1.15,
                                 torch.from_numpy(start).to(DEV), torch.tensor(lens, dtype=torch.int32, device=DEV),
                                 n, lse=torch.empty((1, Hq), device=DEV))
    torch.cuda.synchronize()
    w = _check_decode(out, lse, q, kc, vc, bc, start, lens, gain, 1.15, torch.bfloat16)
    _note(f"  worst error / bar {w:.3f}")
