"""The allocation-free top-K entry point (tg_select_topk_noalloc, for callers
that cannot allocate device memory) against tg_select_topk with a caller
workspace, through the C ABI: bit-identical keep flags on consecutive calls,
the second on a smaller input (the static scratch keeps the first call's
contents), and on the one-workgroup path that uses no scratch."""

import numpy as np
import pytest
import torch

import learned_token_pruning_score_amd as tg
import oracle

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _both(s, cu, db, de, bud):
    print(f"[no_alloc] T={len(s)} B={len(bud)}", flush=True)
    st = torch.from_numpy(np.ascontiguousarray(s, np.float32)).to(DEV)
    meta = [torch.tensor(np.asarray(a, np.int32), device=DEV) for a in (cu, db, de, bud)]
    keep_ws = tg.tg_select_topk(st, *meta)
    keep_na = torch.full((len(s),), 7, dtype=torch.uint8, device=DEV)
    tg.tg_select_topk_noalloc(st, *meta, keep=keep_na)
    torch.cuda.synchronize()
    return keep_ws.cpu().numpy(), keep_na.cpu().numpy()


def _ties(rng, T):
    s = rng.integers(-40, 41, size=T).astype(np.float32) * np.float32(0.25)
    s[rng.integers(0, T, 64)] = -0.0
    s[rng.integers(0, T, 16)] = np.nan
    return s


def test_noalloc_matches_workspace_call_twice_then_smaller():
    rng = np.random.default_rng(2024)
    # first call: the 128k shape (one prompt, chunked path, static scratch)
    T = 131072
    s = rng.standard_normal(T).astype(np.float32)
    s[rng.integers(0, T, 4096)] = np.float32(0.5)  # a run of equal keys at the threshold's level
    cu, db, de, bud = [0, T], [0], [T - 256], [8192]
    a, b = _both(s, cu, db, de, bud)
    assert np.array_equal(a, b)
    assert np.array_equal(b, oracle.select_topk(s, cu, db, de, bud))
    # second call, smaller and ragged (still chunked: T > 32768), with heavy ties
    lens = np.array([30000, 1, 25000, 9000])
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    s = _ties(rng, T)
    db, de, bud = [100, 0, 0, 8000], [29900, 1, 25000, 9000], [3000, 1, 24999, 0]
    a, b = _both(s, cu, db, de, bud)
    assert np.array_equal(a, b)
    assert np.array_equal(b, oracle.select_topk(s, cu, db, de, bud))
    # third call: one-workgroup path (T <= 32768), no scratch involved
    T = 5000
    s = _ties(rng, T)
    a, b = _both(s, [0, T], [10], [4990], [777])
    assert np.array_equal(a, b)
    assert np.array_equal(b, oracle.select_topk(s, [0, T], [10], [4990], [777]))


def test_noalloc_rejects_oversized_before_any_work():
    st = torch.zeros(40000, dtype=torch.float32, device=DEV)
    keep = torch.full((40000,), 9, dtype=torch.uint8, device=DEV)
    B = 300
    cu = torch.tensor(np.linspace(0, 40000, B + 1).astype(np.int32), device=DEV)
    z = torch.zeros(B, dtype=torch.int32, device=DEV)
    with pytest.raises(tg.TokenGateError) as e:
        tg.tg_select_topk_noalloc(st, cu, z, z, z, keep=keep)
    assert e.value.status == -7
    torch.cuda.synchronize()
    assert int(keep.min()) == 9 and int(keep.max()) == 9  # nothing written


def test_noalloc_on_a_created_stream():
    # the scratch is looked up for the stream's device (hipStreamGetDevice)
    rng = np.random.default_rng(77)
    T = 70000
    s = rng.standard_normal(T).astype(np.float32)
    cu, db, de, bud = [0, T], [0], [T - 100], [5000]
    st = torch.from_numpy(s).to(DEV)
    meta = [torch.tensor(np.asarray(a, np.int32), device=DEV) for a in (cu, db, de, bud)]
    keep = torch.full((T,), 7, dtype=torch.uint8, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        tg.tg_select_topk_noalloc(st, *meta, keep=keep)
    side.synchronize()
    assert np.array_equal(keep.cpu().numpy(), oracle.select_topk(s, cu, db, de, bud))
