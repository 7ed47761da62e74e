"""GPU parity of the gate-MLP backward through the C ABI against the CPU
fp64 oracle (score gradient from the kept rows' bias gradient, then the
MLP's backward).

Bars per element (u = 2^-24; with the exact a = W1 h + b1 and
Ea = 2 (D + 4) u sum_k |W1_fk| |h_k| the accumulation bound of the
recomputed a, the kernel's da is off by at most
E_da = |ds| |w2| (0.5 Ea + 2^-20) since |silu''| <= 0.5; r = 2^-8 for the
bf16 rounding of da before the two products, 0 for fp32):
  dhidden_k:  sum_f (E_da + r |da|) |W1_fd| + o |ref|   (o = 2^-8 bf16 output, 2^-22 fp32)
  dW1:        sum_t (E_da + r |da|) |h_td| + 2^-20 sum_t |da| |h_td|
  db1:        sum_t E_da + 2^-20 sum_t |da|
  dw2:        sum_t |ds| 1.1 Ea + 2^-20 sum_t |ds silu(a)|
  db2:        2^-20 sum_t |ds|
"""

import numpy as np
import pytest
import torch

import learned_token_pruning_score_amd as tg
import oracle

pytestmark = pytest.mark.gpu

DEV = "cuda"
U = 2.0 ** -24


def _note(msg):
    print(msg, flush=True)


def _f64(t):
    return t.detach().to("cpu").to(torch.float64).numpy()


def _case(T_lens, docs, D, F, dtype, seed, keep_frac=0.4, with_b1=True):
    """Prompts of the given lengths with document spans; a seeded kept set
    (every question token plus a fraction of each document)."""
    g = np.random.default_rng(seed)
    cu = np.concatenate([[0], np.cumsum(T_lens)]).astype(np.int32)
    T = int(cu[-1])
    db = np.array([d0 for d0, _ in docs], dtype=np.int32)
    de = np.array([d1 for _, d1 in docs], dtype=np.int32)
    keep = np.zeros(T, dtype=bool)
    for b in range(len(T_lens)):
        lo, hi = cu[b], cu[b + 1]
        keep[lo:hi] = True
        doc = np.arange(lo + db[b], lo + de[b])
        keep[doc] = g.random(doc.size) < keep_frac
    kept = np.nonzero(keep)[0].astype(np.int32)
    tg_ = torch.Generator().manual_seed(seed)
    hk = torch.randn((kept.size, D), generator=tg_).to(dtype)  # the kept rows of hidden
    W1 = (torch.randn((F, D), generator=tg_) / D ** 0.5).to(dtype)
    b1 = (torch.randn(F, generator=tg_) * 0.1) if with_b1 else None
    w2 = torch.randn(F, generator=tg_) / F ** 0.5
    dbias = torch.randn(kept.size, generator=tg_) * 2.0
    return cu, db, de, kept, hk, W1, b1, w2, dbias, T


def _check(cu, db, de, kept, hk, W1, b1, w2, dbias, T, dtype, res):
    """The oracle's score gradient over all T tokens, then its MLP backward
    over the kept rows (every other token has a zero score gradient and adds
    nothing to the sums)."""
    dh, dW1, db1, dw2, db2 = (None if x is None else _f64(x) for x in res)
    D = hk.shape[1]
    Hk = _f64(hk)
    Wd, w2d = _f64(W1), _f64(w2)
    b1d = None if b1 is None else _f64(b1)
    ds_full = oracle.score_grad_from_bias(_f64(dbias), kept, cu, db, de, T)
    dsk = ds_full[kept]
    r_dh, r_dW1, r_db1, r_dw2, r_db2 = oracle.gate_backward(Hk, Wd, b1d, w2d, dsk)
    a = Hk @ Wd.T + (0.0 if b1d is None else b1d[None, :])
    sg = 1 / (1 + np.exp(-a))
    da = dsk[:, None] * w2d[None, :] * sg * (1 + a * (1 - sg))
    Ea = 2 * (D + 4) * U * (np.abs(Hk) @ np.abs(Wd).T)
    Eda = np.abs(dsk)[:, None] * np.abs(w2d)[None, :] * (0.5 * Ea + 2.0 ** -20)
    bf = dtype == torch.bfloat16
    r = 2.0 ** -8 if bf else 0.0
    o = 2.0 ** -8 if bf else 2.0 ** -22
    A = Eda + r * np.abs(da)
    checks = [
        ("dhidden_k", dh, r_dh, A @ np.abs(Wd) + o * np.abs(r_dh)),
        ("dW1", dW1, r_dW1, A.T @ np.abs(Hk) + 2.0 ** -20 * (np.abs(da).T @ np.abs(Hk))),
        ("dw2", dw2, r_dw2, (np.abs(dsk)[:, None] * 1.1 * Ea).sum(axis=0)
         + 2.0 ** -20 * np.abs(dsk[:, None] * a * sg).sum(axis=0)),
        ("db2", db2.reshape(()), np.asarray(r_db2), np.asarray(2.0 ** -20 * np.abs(dsk).sum())),
    ]
    if b1 is not None:
        checks.append(("db1", db1, r_db1, Eda.sum(axis=0) + 2.0 ** -20 * np.abs(da).sum(axis=0)))
    worst = {}
    for name, got, exp, tol in checks:
        tol = tol + 1e-7
        excess = np.abs(got - exp) - tol
        j = np.unravel_index(np.argmax(excess), excess.shape) if excess.ndim else ()
        assert excess[j] <= 0, f"{name}{j}: got {got[j]}, oracle {exp[j]}, tol {tol[j]}"
        worst[name] = float(np.max(np.abs(got - exp) / tol))
    _note(f"  worst error / bar: {worst}")


def _run(cu, db, de, kept, hk, W1, b1, w2, dbias, T):
    res = tg.tg_gate_bwd(hk.to(DEV), W1.to(DEV), None if b1 is None else b1.to(DEV), w2.to(DEV), dbias.to(DEV),
                         torch.from_numpy(kept).to(DEV), torch.from_numpy(cu).to(DEV),
                         torch.from_numpy(db).to(DEV), torch.from_numpy(de).to(DEV))
    torch.cuda.synchronize()
    return res


# (prompt lengths, document spans, D, F, dtype, b1): a ragged batch with an
# empty document and an empty prompt; F = 256 / 128 / 64; fp32
CASES = [
    ([3000, 40, 0, 2500], [(0, 2900), (0, 0), (0, 0), (100, 2400)], 2048, 256, torch.bfloat16, True),
    ([1200, 900], [(0, 1100), (50, 800)], 512, 128, torch.bfloat16, False),
    ([700], [(0, 650)], 256, 64, torch.bfloat16, True),
    ([200, 90], [(0, 180), (0, 60)], 256, 64, torch.float32, True),
]


@pytest.mark.parametrize("lens,docs,D,F,dtype,with_b1", CASES)
def test_gate_bwd_parity(lens, docs, D, F, dtype, with_b1):
    _note(f"[gate bwd] lens={lens} D={D} F={F} {dtype} b1={with_b1}")
    case = _case(lens, docs, D, F, dtype, seed=sum(lens) + F, with_b1=with_b1)
    res = _run(*case)
    _check(*case, dtype, res)
    res2 = _run(*case)
    for a, b in zip(res, res2):
        if a is not None:
            assert torch.equal(a, b)  # bit-reproducible


def test_gate_bwd_full_size_128k():
    """The 128k workload's shape: one prompt of 131072 tokens, a 130k-token
    document kept at 1/16 and the question whole (8448 kept rows of 2048),
    gate 2048 -> 256."""
    _note("[gate bwd full] 131072 tokens, 8448 kept")
    g = np.random.default_rng(7)
    T, doc_end, D, F = 131072, 130816, 2048, 256
    cu = np.array([0, T], dtype=np.int32)
    db, de = np.array([0], dtype=np.int32), np.array([doc_end], dtype=np.int32)
    doc_kept = np.sort(g.choice(doc_end, size=8192, replace=False))
    kept = np.concatenate([doc_kept, np.arange(doc_end, T)]).astype(np.int32)
    tg_ = torch.Generator().manual_seed(7)
    hk = torch.randn((kept.size, D), generator=tg_).to(torch.bfloat16)
    W1 = (torch.randn((F, D), generator=tg_) / D ** 0.5).to(torch.bfloat16)
    b1 = torch.randn(F, generator=tg_) * 0.1
    w2 = torch.randn(F, generator=tg_) / F ** 0.5
    dbias = torch.randn(kept.size, generator=tg_) * 2.0
    case = (cu, db, de, kept, hk, W1, b1, w2, dbias, T)
    res = _run(*case)
    _check(*case, torch.bfloat16, res)


def test_gate_bwd_no_kept_rows():
    """No kept rows (one empty prompt): every gradient is zero, with no
    kernel reading the empty inputs."""
    _note("[gate bwd] no kept rows")
    tg_ = torch.Generator().manual_seed(3)
    D, F = 256, 64
    W1 = (torch.randn((F, D), generator=tg_) / D ** 0.5).to(torch.bfloat16)
    b1 = torch.randn(F, generator=tg_) * 0.1
    w2 = torch.randn(F, generator=tg_)
    i32 = dict(dtype=torch.int32, device=DEV)
    dh, dW1, db1, dw2, db2 = tg.tg_gate_bwd(
        torch.empty((0, D), dtype=torch.bfloat16, device=DEV), W1.to(DEV), b1.to(DEV), w2.to(DEV),
        torch.empty(0, device=DEV), torch.empty(0, **i32), torch.zeros(2, **i32), torch.zeros(1, **i32),
        torch.zeros(1, **i32))
    torch.cuda.synchronize()
    assert dh.shape == (0, D)
    for t in (dW1, db1, dw2, db2):
        assert torch.count_nonzero(t).item() == 0
