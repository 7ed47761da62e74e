"""ctypes binding of libtokengate.so (C ABI declared in include/tg.h).

Argument marshalling only: every function takes torch tensors (device memory
that torch allocated), checks dtypes and shapes that ctypes cannot see, and
passes raw pointers plus the current HIP stream.  All computation happens in
the library's HIP kernels; nothing here has a CPU fallback.  A missing
library or a missing GPU raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import numpy as np
import torch

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libtokengate.so")

TG_OK = 0
TG_F32 = 0
TG_BF16 = 1

_c_i64 = ctypes.c_int64
_c_i32 = ctypes.c_int32
_c_int = ctypes.c_int
_c_f32 = ctypes.c_float
_c_vp = ctypes.c_void_p
_c_size_p = ctypes.POINTER(ctypes.c_size_t)
_c_i32_p = ctypes.POINTER(ctypes.c_int32)

# Every exported symbol of include/tg.h with its ctypes signature.
SIGNATURES = {
    "tg_abi_version": (_c_int, []),
    "tg_status_string": (ctypes.c_char_p, [_c_int]),
    "tg_plan": (_c_int, [_c_int, _c_i32_p, _c_i32_p, _c_i32_p, _c_i32_p, _c_i32_p, _c_i32_p]),
    "tg_gate_score": (_c_int, [_c_vp, _c_i64, _c_i64, _c_int, _c_vp, _c_vp, _c_vp, _c_f32,
                               _c_int, _c_int, _c_vp, _c_vp]),
    "tg_select_topk_workspace": (_c_int, [_c_int, _c_i64, _c_size_p]),
    "tg_select_topk": (_c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_int, _c_i64, _c_vp,
                                _c_vp, ctypes.c_size_t, _c_vp]),
    "tg_select_topk_noalloc": (_c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_int, _c_i64, _c_vp,
                                        _c_vp]),
    "tg_compact_workspace": (_c_int, [_c_int, _c_i64, _c_size_p]),
    "tg_compact": (_c_int, [_c_vp, _c_i64, _c_int, _c_int, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp,
                            _c_vp, _c_int, _c_i64, _c_i64, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp,
                            ctypes.c_size_t, _c_vp]),
    "tg_gated_attn_fwd": (_c_int, [_c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64, _c_vp, _c_vp,
                                   _c_f32, _c_vp, _c_int, _c_int, _c_i64, _c_int, _c_int, _c_int,
                                   _c_int, _c_vp, _c_vp, _c_vp]),
    "tg_gated_attn_bwd_workspace": (_c_int, [_c_int, _c_i64, _c_int, _c_int, _c_int, _c_int, _c_int, _c_size_p]),
    "tg_gated_attn_bwd": (_c_int, [_c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64, _c_vp, _c_vp,
                                   _c_f32, _c_vp, _c_int, _c_int, _c_i64, _c_int, _c_int, _c_int,
                                   _c_int, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp,
                                   _c_vp, _c_vp, ctypes.c_size_t, _c_vp]),
    "tg_gate_bwd_workspace": (_c_int, [_c_i64, _c_int, _c_int, _c_int, _c_size_p]),
    "tg_gate_bwd": (_c_int, [_c_vp, _c_i64, _c_i64, _c_int, _c_vp, _c_vp, _c_vp, _c_int, _c_vp, _c_vp,
                             _c_vp, _c_vp, _c_vp, _c_int, _c_int, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp,
                             _c_vp, ctypes.c_size_t, _c_vp]),
    "tg_kv_scatter": (_c_int, [_c_vp, _c_vp, _c_i64, _c_i64, _c_vp, _c_vp, _c_int, _c_i64, _c_int, _c_int,
                               _c_int, _c_vp, _c_vp, _c_i64, _c_i64, _c_vp, _c_vp, _c_vp]),
    "tg_kv_append": (_c_int, [_c_vp, _c_vp, _c_int, _c_int, _c_int, _c_int, _c_vp, _c_vp, _c_i64, _c_i64,
                              _c_vp, _c_vp, _c_vp, _c_vp]),
    "tg_decode_attn_workspace": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_size_p]),
    "tg_decode_attn": (_c_int, [_c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_vp, _c_vp, _c_f32, _c_vp, _c_vp,
                                _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_vp, _c_vp, _c_vp,
                                ctypes.c_size_t, _c_vp]),
    "tg_sample_budgets": (_c_int, [_c_int, _c_i32_p, _c_i32_p, ctypes.POINTER(ctypes.c_float), _c_f32, _c_f32,
                                   _c_i32_p]),
    "tg_rope_table": (_c_int, [_c_vp, _c_i64, _c_int, ctypes.c_double, _c_vp, _c_vp]),
    "tg_qkv_rope": (_c_int, [_c_vp, _c_i64, _c_i64, _c_int, _c_vp, _c_vp, _c_int, _c_int, _c_int,
                             _c_int, _c_vp, _c_i64, _c_vp]),
    "tg_rms_norm": (_c_int, [_c_vp, _c_i64, _c_i64, _c_int, _c_vp, _c_f32, _c_int, _c_vp, _c_i64,
                             _c_vp]),
    "tg_linear_residual": (_c_int, [_c_vp, _c_i64, _c_i64, _c_int, _c_vp, _c_int, _c_vp, _c_i64,
                                    _c_int, _c_vp, _c_i64, _c_vp]),
    "tg_swiglu": (_c_int, [_c_vp, _c_i64, _c_i64, _c_int, _c_vp, _c_vp, _c_int, _c_int, _c_vp,
                           _c_i64, _c_vp]),
}

_lib = None


class TokenGateError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status} ({status_string(status)})")


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load (once) and type the shared library; raises if it was not built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(
            f"{p} not found: build it with `python -m learned_token_pruning_score_amd.build`")
    lib = ctypes.CDLL(p)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().tg_status_string(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != TG_OK:
        raise TokenGateError(fn, status)


def _dtype_code_of(dtype: torch.dtype) -> int:
    if dtype == torch.bfloat16:
        return TG_BF16
    if dtype == torch.float32:
        return TG_F32
    raise TypeError(f"unsupported dtype {dtype}")


def _dtype_code(t: torch.Tensor) -> int:
    return _dtype_code_of(t.dtype)


def _dev(t: Optional[torch.Tensor], name: str, dtype=None) -> int:
    if t is None:
        return 0
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _require_gpu() -> None:
    if not torch.cuda.is_available():
        raise RuntimeError("the TokenGate kernels need a ROCm GPU (gfx950); none is visible")


# ---------------------------------------------------------------- entry points

def tg_abi_version() -> int:
    return int(load_library().tg_abi_version())


def tg_plan(cu_seqlens, doc_begin, doc_end, budget) -> Tuple[np.ndarray, int]:
    """Host-only kept sizes: returns (cu_kept int32 [B+1], max kept length)."""
    lib = load_library()
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    db = np.ascontiguousarray(doc_begin, dtype=np.int32)
    de = np.ascontiguousarray(doc_end, dtype=np.int32)
    bud = np.ascontiguousarray(budget, dtype=np.int32)
    B = int(bud.shape[0])
    if cu.shape[0] != B + 1 or db.shape[0] != B or de.shape[0] != B:
        raise ValueError("cu_seqlens must have B+1 entries and the others B")
    out = np.zeros(B + 1, dtype=np.int32)
    mx = ctypes.c_int32(0)
    p = lambda a: a.ctypes.data_as(_c_i32_p)  # noqa: E731
    _check("tg_plan", lib.tg_plan(B, p(cu), p(db), p(de), p(bud), p(out), ctypes.byref(mx)))
    return out, int(mx.value)


def tg_gate_score(hidden: torch.Tensor, W1: torch.Tensor, b1: Optional[torch.Tensor],
                  w2: torch.Tensor, b2: float, scores: Optional[torch.Tensor] = None,
                  stream=None) -> torch.Tensor:
    """Gate scores [T] fp32 of ``hidden`` [T, D] (row stride may exceed D)."""
    _require_gpu()
    lib = load_library()
    T, D = hidden.shape
    F = W1.shape[0]
    if not _unit_cols(hidden) or not W1.is_contiguous() or W1.shape[1] != D:
        raise ValueError("hidden must have unit column stride and W1 must be [F, D] contiguous")
    if W1.dtype != hidden.dtype:
        raise TypeError("W1 and hidden must share a dtype")
    if scores is None:
        scores = torch.empty(T, dtype=torch.float32, device=hidden.device)
    _check("tg_gate_score", lib.tg_gate_score(
        _dev(hidden, "hidden"), hidden.stride(0) if T > 0 else D, T, D, _dev(W1, "W1"),
        _dev(b1, "b1", torch.float32), _dev(w2, "w2", torch.float32), float(b2), F,
        _dtype_code(hidden), _dev(scores, "scores", torch.float32), _stream(stream)))
    return scores


def tg_select_topk_workspace(B: int, T: int) -> int:
    n = ctypes.c_size_t(0)
    _check("tg_select_topk_workspace", load_library().tg_select_topk_workspace(B, T, ctypes.byref(n)))
    return int(n.value)


def tg_compact_workspace(B: int, T: int) -> int:
    n = ctypes.c_size_t(0)
    _check("tg_compact_workspace", load_library().tg_compact_workspace(B, T, ctypes.byref(n)))
    return int(n.value)


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)


def tg_select_topk(scores: torch.Tensor, cu_seqlens: torch.Tensor, doc_begin: torch.Tensor,
                   doc_end: torch.Tensor, budget: torch.Tensor, keep: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Keep flags uint8 [T] (metadata tensors are int32 on the device)."""
    _require_gpu()
    lib = load_library()
    T = scores.shape[0]
    B = budget.shape[0]
    if keep is None:
        keep = torch.empty(T, dtype=torch.uint8, device=scores.device)
    need = tg_select_topk_workspace(B, T)
    if workspace is None:
        workspace = _workspace(need, scores.device)
    _check("tg_select_topk", lib.tg_select_topk(
        _dev(scores, "scores", torch.float32), _dev(cu_seqlens, "cu_seqlens", torch.int32),
        _dev(doc_begin, "doc_begin", torch.int32), _dev(doc_end, "doc_end", torch.int32),
        _dev(budget, "budget", torch.int32), B, T, _dev(keep, "keep", torch.uint8),
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _stream(stream)))
    return keep


def tg_select_topk_noalloc(scores: torch.Tensor, cu_seqlens: torch.Tensor, doc_begin: torch.Tensor,
                           doc_end: torch.Tensor, budget: torch.Tensor, keep: torch.Tensor,
                           stream=None) -> torch.Tensor:
    """tg_select_topk on the library's static scratch: no workspace argument and
    no allocation (``keep`` must be given)."""
    _require_gpu()
    lib = load_library()
    T = scores.shape[0]
    B = budget.shape[0]
    _check("tg_select_topk_noalloc", lib.tg_select_topk_noalloc(
        _dev(scores, "scores", torch.float32), _dev(cu_seqlens, "cu_seqlens", torch.int32),
        _dev(doc_begin, "doc_begin", torch.int32), _dev(doc_end, "doc_end", torch.int32),
        _dev(budget, "budget", torch.int32), B, T, _dev(keep, "keep", torch.uint8), _stream(stream)))
    return keep


def tg_compact(hidden: torch.Tensor, pos: Optional[torch.Tensor], scores: torch.Tensor,
               keep: torch.Tensor, cu_seqlens: torch.Tensor, doc_begin: torch.Tensor,
               doc_end: torch.Tensor, Kt: int, out: Optional[tuple] = None,
               with_index: bool = True, workspace: Optional[torch.Tensor] = None, stream=None):
    """Returns (hidden_k [Kt, D], pos_k int32 [Kt], bias_s fp32 [Kt], kept_idx int32 [Kt] or None)."""
    _require_gpu()
    lib = load_library()
    T, D = hidden.shape
    B = doc_begin.shape[0]
    dev = hidden.device
    if not _unit_cols(hidden):
        raise ValueError("hidden must have unit column stride")
    if out is None:
        hk = torch.empty((Kt, D), dtype=hidden.dtype, device=dev)
        pk = torch.empty(Kt, dtype=torch.int32, device=dev)
        bk = torch.empty(Kt, dtype=torch.float32, device=dev)
        ik = torch.empty(Kt, dtype=torch.int32, device=dev) if with_index else None
    else:
        hk, pk, bk, ik = out
    need = tg_compact_workspace(B, T)
    if workspace is None:
        workspace = _workspace(need, dev)
    _check("tg_compact", lib.tg_compact(
        _dev(hidden, "hidden"), hidden.stride(0) if T > 0 else D, D, _dtype_code(hidden),
        _dev(pos, "pos", torch.int32), _dev(scores, "scores", torch.float32),
        _dev(keep, "keep", torch.uint8), _dev(cu_seqlens, "cu_seqlens", torch.int32),
        _dev(doc_begin, "doc_begin", torch.int32), _dev(doc_end, "doc_end", torch.int32), B, T, Kt,
        _dev(hk, "hidden_out"), _dev(pk, "pos_out", torch.int32),
        _dev(bk, "bias_out", torch.float32), _dev(ik, "kept_idx_out", torch.int32),
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _stream(stream)))
    return hk, pk, bk, ik


def tg_gated_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                      bias_s: Optional[torch.Tensor], gain: Optional[torch.Tensor], tau: float,
                      cu_kept: torch.Tensor, max_kept_len: int, out: Optional[torch.Tensor] = None,
                      lse: Optional[torch.Tensor] = None, want_lse: bool = False, stream=None):
    """Token-gated causal GQA attention; q [Kt, Hq, d], k/v [Kt, Hkv, d].

    Returns (out [Kt, Hq, d], lse [Hq, Kt] fp32 or None).
    """
    _require_gpu()
    lib = load_library()
    Kt, Hq, d = q.shape
    Hkv = k.shape[1]
    for name, t, H in (("q", q, Hq), ("k", k, Hkv), ("v", v, Hkv)):
        if t.dim() != 3 or t.shape[0] != Kt or t.shape[2] != d or t.shape[1] != H:
            raise ValueError(f"{name} has shape {tuple(t.shape)}")
        if t.numel() and (t.stride(2) != 1 or t.stride(1) != d):
            raise ValueError(f"{name} must have heads contiguous inside a token")
        if t.dtype != q.dtype:
            raise TypeError("q, k, v must share a dtype")
    B = cu_kept.shape[0] - 1
    if out is None:
        out = torch.empty((Kt, Hq, d), dtype=q.dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((Hq, Kt), dtype=torch.float32, device=q.device)
    _check("tg_gated_attn_fwd", lib.tg_gated_attn_fwd(
        _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), q.stride(0) if Kt else Hq * d,
        k.stride(0) if Kt else Hkv * d, v.stride(0) if Kt else Hkv * d,
        _dev(bias_s, "bias_s", torch.float32), _dev(gain, "gain", torch.float32), float(tau),
        _dev(cu_kept, "cu_kept", torch.int32), B, int(max_kept_len), Kt, Hq, Hkv, d,
        _dtype_code(q), _dev(out, "out"), _dev(lse, "lse", torch.float32), _stream(stream)))
    return out, lse


def tg_rope_table(pos: torch.Tensor, d: int, rope_theta: float,
                  out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """cos / sin of the rotary embedding at positions pos [Kt] int32.

    Returns table [Kt, d/2, 2] fp32: (cos, sin) of pos * rope_theta^(-2 i / d).
    """
    _require_gpu()
    lib = load_library()
    if pos.dim() != 1:
        raise ValueError("pos must be 1-D")
    Kt = pos.shape[0]
    if out is None:
        out = torch.empty((Kt, d // 2, 2), dtype=torch.float32, device=pos.device)
    elif tuple(out.shape) != (Kt, d // 2, 2) or not out.is_contiguous():
        raise ValueError(f"out has shape {tuple(out.shape)}")
    _check("tg_rope_table", lib.tg_rope_table(
        _dev(pos, "pos", torch.int32), Kt, int(d), float(rope_theta),
        _dev(out, "out", torch.float32), _stream(stream)))
    return out


def tg_qkv_rope(x: torch.Tensor, w_qkv: torch.Tensor, rope_table: torch.Tensor, Hq: int, Hkv: int,
                d: int, out: Optional[torch.Tensor] = None, stream=None):
    """Fused q/k/v projection of the rows of x [Kt, D], q and k rotated.

    w_qkv [(Hq + 2 Hkv) d, D] (q heads, k heads, v heads); rope_table from
    tg_rope_table.  Returns (qkv [Kt, (Hq + 2 Hkv) d], q [Kt, Hq, d],
    k [Kt, Hkv, d], v [Kt, Hkv, d]), the last three views into qkv.
    """
    _require_gpu()
    lib = load_library()
    if x.dim() != 2 or not _unit_cols(x):
        raise ValueError("x must be [Kt, D] with unit column stride")
    Kt, D = x.shape
    N = (Hq + 2 * Hkv) * d
    if tuple(w_qkv.shape) != (N, D) or not w_qkv.is_contiguous() or w_qkv.dtype != x.dtype:
        raise ValueError(f"w_qkv must be packed [{N}, {D}] of the dtype of x")
    if tuple(rope_table.shape) != (Kt, d // 2, 2) or not rope_table.is_contiguous():
        raise ValueError(f"rope_table has shape {tuple(rope_table.shape)}")
    if out is None:
        out = torch.empty((Kt, N), dtype=x.dtype, device=x.device)
    elif out.dim() != 2 or out.shape[0] != Kt or out.shape[1] < N or not _unit_cols(out):
        raise ValueError(f"out has shape {tuple(out.shape)}")
    if out.dtype != x.dtype:
        raise TypeError("out must have the dtype of x")
    _check("tg_qkv_rope", lib.tg_qkv_rope(
        _dev(x, "x"), x.stride(0) if Kt else D, Kt, D, _dev(w_qkv, "w_qkv"),
        _dev(rope_table, "rope_table", torch.float32), int(Hq), int(Hkv), int(d),
        _dtype_code(x), _dev(out, "out"), out.stride(0) if Kt else N, _stream(stream)))
    q = out[:, :Hq * d].unflatten(1, (Hq, d))
    k = out[:, Hq * d:(Hq + Hkv) * d].unflatten(1, (Hkv, d))
    v = out[:, (Hq + Hkv) * d:N].unflatten(1, (Hkv, d))
    return out, q, k, v


def _unit_cols(t: torch.Tensor) -> bool:
    """Unit stride along the last dimension (any strides for an empty
    tensor: it is never read)."""
    return t.numel() == 0 or t.stride(-1) == 1


def _rows2d(t: torch.Tensor, name: str) -> None:
    if t.dim() != 2 or not _unit_cols(t):
        raise ValueError(f"{name} must be 2-D with unit column stride")


def tg_rms_norm(x: torch.Tensor, weight: torch.Tensor, eps: float,
                out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """RMSNorm of the rows of x [n, D] with an fp32 weight [D]; out may be x."""
    _require_gpu()
    lib = load_library()
    _rows2d(x, "x")
    n, D = x.shape
    if tuple(weight.shape) != (D,) or not weight.is_contiguous():
        raise ValueError("weight must be a packed [D] vector")
    if out is None:
        out = torch.empty((n, D), dtype=x.dtype, device=x.device)
    _rows2d(out, "out")
    if tuple(out.shape) != (n, D) or out.dtype != x.dtype:
        raise ValueError("out must match x")
    _check("tg_rms_norm", lib.tg_rms_norm(
        _dev(x, "x"), x.stride(0) if n else D, n, D, _dev(weight, "weight", torch.float32),
        float(eps), _dtype_code(x), _dev(out, "out"), out.stride(0) if n else D, _stream(stream)))
    return out


def tg_linear_residual(a: torch.Tensor, W: torch.Tensor, residual: torch.Tensor,
                       out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """residual + a @ W.T: a [n, K], W [N, K], residual [n, N]; out may be residual."""
    _require_gpu()
    lib = load_library()
    _rows2d(a, "a")
    _rows2d(residual, "residual")
    n, K = a.shape
    N = W.shape[0]
    if tuple(W.shape) != (N, K) or not W.is_contiguous():
        raise ValueError(f"W must be packed [N, {K}]")
    if tuple(residual.shape) != (n, N):
        raise ValueError("residual must be [n, N]")
    for t, nm in ((W, "W"), (residual, "residual")):
        if t.dtype != a.dtype:
            raise TypeError(f"{nm} must have the dtype of a")
    if out is None:
        out = torch.empty((n, N), dtype=a.dtype, device=a.device)
    _rows2d(out, "out")
    if tuple(out.shape) != (n, N) or out.dtype != a.dtype:
        raise ValueError("out must be [n, N] of the dtype of a")
    _check("tg_linear_residual", lib.tg_linear_residual(
        _dev(a, "a"), a.stride(0) if n else K, n, K, _dev(W, "W"), N, _dev(residual, "residual"),
        residual.stride(0) if n else N, _dtype_code(a), _dev(out, "out"),
        out.stride(0) if n else N, _stream(stream)))
    return out


def tg_swiglu(h: torch.Tensor, w_gate: torch.Tensor, w_up: torch.Tensor,
              out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """silu(h @ w_gate.T) * (h @ w_up.T): h [n, D], w_gate / w_up [I, D]."""
    _require_gpu()
    lib = load_library()
    _rows2d(h, "h")
    n, D = h.shape
    I = w_gate.shape[0]
    for t, nm in ((w_gate, "w_gate"), (w_up, "w_up")):
        if tuple(t.shape) != (I, D) or not t.is_contiguous() or t.dtype != h.dtype:
            raise ValueError(f"{nm} must be packed [{I}, {D}] of the dtype of h")
    if out is None:
        out = torch.empty((n, I), dtype=h.dtype, device=h.device)
    _rows2d(out, "out")
    if tuple(out.shape) != (n, I) or out.dtype != h.dtype:
        raise ValueError("out must be [n, I] of the dtype of h")
    _check("tg_swiglu", lib.tg_swiglu(
        _dev(h, "h"), h.stride(0) if n else D, n, D, _dev(w_gate, "w_gate"), _dev(w_up, "w_up"), I,
        _dtype_code(h), _dev(out, "out"), out.stride(0) if n else I, _stream(stream)))
    return out


def tg_gated_attn_bwd_workspace(B: int, Kt: int, Hq: int, Hkv: int, d: int, dtype: torch.dtype,
                                max_kept_len: int) -> int:
    n = ctypes.c_size_t(0)
    _check("tg_gated_attn_bwd_workspace",
           load_library().tg_gated_attn_bwd_workspace(B, Kt, Hq, Hkv, d, _dtype_code_of(dtype), max_kept_len,
                                                      ctypes.byref(n)))
    return int(n.value)


def tg_gated_attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                      bias_s: Optional[torch.Tensor], gain: Optional[torch.Tensor], tau: float,
                      cu_kept: torch.Tensor, max_kept_len: int, out: torch.Tensor,
                      lse: torch.Tensor, dout: torch.Tensor, workspace: Optional[torch.Tensor] = None,
                      grads=None, stream=None):
    """Backward of tg_gated_attn_fwd.  Returns (dq, dk, dv, dbias [Kt],
    dgain [Hq], dtau [1]); ``grads`` may supply those six output tensors."""
    _require_gpu()
    lib = load_library()
    Kt, Hq, d = q.shape
    Hkv = k.shape[1]
    B = cu_kept.shape[0] - 1
    for name, t in (("out", out), ("dout", dout)):
        if tuple(t.shape) != (Kt, Hq, d) or not t.is_contiguous() or t.dtype != q.dtype:
            raise ValueError(f"{name} must be packed [Kt, Hq, d] of the dtype of q")
    if tuple(lse.shape) != (Hq, Kt) or lse.dtype != torch.float32:
        raise ValueError("lse must be [Hq, Kt] fp32")
    if grads is None:
        dev = q.device
        grads = (torch.empty((Kt, Hq, d), dtype=q.dtype, device=dev),
                 torch.empty((Kt, Hkv, d), dtype=q.dtype, device=dev),
                 torch.empty((Kt, Hkv, d), dtype=q.dtype, device=dev),
                 torch.empty(Kt, dtype=torch.float32, device=dev),
                 torch.empty(Hq, dtype=torch.float32, device=dev),
                 torch.empty(1, dtype=torch.float32, device=dev))
    dq, dk, dv, db, dg, dt = grads
    if workspace is None:
        workspace = torch.empty(max(16, tg_gated_attn_bwd_workspace(B, Kt, Hq, Hkv, d, q.dtype, max_kept_len)),
                                dtype=torch.uint8, device=q.device)
    _check("tg_gated_attn_bwd", lib.tg_gated_attn_bwd(
        _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), q.stride(0) if Kt else Hq * d,
        k.stride(0) if Kt else Hkv * d, v.stride(0) if Kt else Hkv * d,
        _dev(bias_s, "bias_s", torch.float32), _dev(gain, "gain", torch.float32), float(tau),
        _dev(cu_kept, "cu_kept", torch.int32), B, int(max_kept_len), Kt, Hq, Hkv, d,
        _dtype_code(q), _dev(out, "out"), _dev(lse, "lse", torch.float32), _dev(dout, "dout"),
        _dev(dq, "dq"), _dev(dk, "dk"), _dev(dv, "dv"), _dev(db, "dbias", torch.float32),
        _dev(dg, "dgain", torch.float32), _dev(dt, "dtau", torch.float32), _dev(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return dq, dk, dv, db, dg, dt


def tg_gate_bwd_workspace(Kt: int, D: int, F: int, dtype: torch.dtype) -> int:
    n = ctypes.c_size_t(0)
    _check("tg_gate_bwd_workspace", load_library().tg_gate_bwd_workspace(Kt, D, F, _dtype_code_of(dtype), ctypes.byref(n)))
    return int(n.value)


def tg_gate_bwd(hidden_k: torch.Tensor, W1: torch.Tensor, b1: Optional[torch.Tensor], w2: torch.Tensor,
                dbias: torch.Tensor, kept_idx: torch.Tensor, cu_seqlens: torch.Tensor,
                doc_begin: torch.Tensor, doc_end: torch.Tensor, workspace: Optional[torch.Tensor] = None,
                stream=None):
    """Backward of the gate MLP over the kept rows.  Returns (dhidden_k
    [Kt, D], dW1 [F, D] fp32, db1 [F] fp32, dw2 [F] fp32, db2 [1] fp32)."""
    _require_gpu()
    lib = load_library()
    if hidden_k.dim() != 2 or not _unit_cols(hidden_k):
        raise ValueError("hidden_k must be [Kt, D] with unit column stride")
    Kt, D = hidden_k.shape
    F = W1.shape[0]
    if tuple(W1.shape) != (F, D) or not W1.is_contiguous() or W1.dtype != hidden_k.dtype:
        raise ValueError("W1 must be packed [F, D] of the dtype of hidden_k")
    B = cu_seqlens.shape[0] - 1
    dev = hidden_k.device
    dh = torch.empty((Kt, D), dtype=hidden_k.dtype, device=dev)
    dW1 = torch.empty((F, D), dtype=torch.float32, device=dev)
    db1 = torch.empty(F, dtype=torch.float32, device=dev) if b1 is not None else None
    dw2 = torch.empty(F, dtype=torch.float32, device=dev)
    db2 = torch.empty(1, dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = torch.empty(max(16, tg_gate_bwd_workspace(Kt, D, F, hidden_k.dtype)),
                                dtype=torch.uint8, device=dev)
    _check("tg_gate_bwd", lib.tg_gate_bwd(
        _dev(hidden_k, "hidden_k"), hidden_k.stride(0) if Kt else D, Kt, D, _dev(W1, "W1"),
        _dev(b1, "b1", torch.float32), _dev(w2, "w2", torch.float32), F,
        _dev(dbias, "dbias", torch.float32), _dev(kept_idx, "kept_idx", torch.int32),
        _dev(cu_seqlens, "cu_seqlens", torch.int32), _dev(doc_begin, "doc_begin", torch.int32),
        _dev(doc_end, "doc_end", torch.int32), B, _dtype_code(hidden_k), _dev(dh, "dhidden_k"),
        _dev(dW1, "dW1"), _dev(db1, "db1"), _dev(dw2, "dw2"), _dev(db2, "db2"),
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream(stream)))
    return dh, dW1, db1, dw2, db2


def tg_kv_scatter(k: torch.Tensor, v: torch.Tensor, bias_s: Optional[torch.Tensor], cu_kept: torch.Tensor,
                  k_cache: torch.Tensor, v_cache: torch.Tensor, bias_cache: torch.Tensor, start: torch.Tensor,
                  stream=None) -> None:
    """Kept rows k, v [Kt, Hkv, d] (ragged by cu_kept) into caches [rows, Hkv, d]
    at rows start[b] + (r - cu_kept[b]), with their bias."""
    _require_gpu()
    Kt, Hkv, d = k.shape
    B = cu_kept.shape[0] - 1
    _check("tg_kv_scatter", load_library().tg_kv_scatter(
        _dev(k, "k"), _dev(v, "v"), k.stride(0) if Kt else Hkv * d, v.stride(0) if Kt else Hkv * d,
        _dev(bias_s, "bias_s", torch.float32), _dev(cu_kept, "cu_kept", torch.int32), B, Kt, Hkv, d,
        _dtype_code(k), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), k_cache.stride(0),
        v_cache.stride(0), _dev(bias_cache, "bias_cache", torch.float32), _dev(start, "start", torch.int32),
        _stream(stream)))


def tg_kv_append(k_new: torch.Tensor, v_new: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                 bias_cache: torch.Tensor, start: torch.Tensor, pos: torch.Tensor, stream=None) -> None:
    """New k, v [B, Hkv, d] into cache rows start[b] + pos[b], bias 0."""
    _require_gpu()
    B, Hkv, d = k_new.shape
    _check("tg_kv_append", load_library().tg_kv_append(
        _dev(k_new, "k_new"), _dev(v_new, "v_new"), B, Hkv, d, _dtype_code(k_new), _dev(k_cache, "k_cache"),
        _dev(v_cache, "v_cache"), k_cache.stride(0), v_cache.stride(0),
        _dev(bias_cache, "bias_cache", torch.float32), _dev(start, "start", torch.int32),
        _dev(pos, "pos", torch.int32), _stream(stream)))


def tg_decode_attn_workspace(B: int, Hq: int, d: int, max_len: int) -> int:
    n = ctypes.c_size_t(0)
    _check("tg_decode_attn_workspace",
           load_library().tg_decode_attn_workspace(B, Hq, d, max_len, ctypes.byref(n)))
    return int(n.value)


def tg_decode_attn(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                   bias_cache: Optional[torch.Tensor], gain: Optional[torch.Tensor], tau: float,
                   start: torch.Tensor, lens: torch.Tensor, max_len: int, out: Optional[torch.Tensor] = None,
                   lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None, stream=None):
    """One decode step; q [B, Hq, d].  Returns (out [B, Hq, d], lse [B, Hq] or None)."""
    _require_gpu()
    B, Hq, d = q.shape
    Hkv = k_cache.shape[1]
    if not q.is_contiguous():
        raise ValueError("q must be packed [B, Hq, d]")
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = torch.empty(max(16, tg_decode_attn_workspace(B, Hq, d, max_len)), dtype=torch.uint8,
                                device=q.device)
    _check("tg_decode_attn", load_library().tg_decode_attn(
        _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), k_cache.stride(0), v_cache.stride(0),
        _dev(bias_cache, "bias_cache", torch.float32), _dev(gain, "gain", torch.float32), float(tau),
        _dev(start, "start", torch.int32), _dev(lens, "lens", torch.int32), B, int(max_len), Hq, Hkv, d,
        _dtype_code(q), _dev(out, "out"), _dev(lse, "lse", torch.float32), _dev(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return out, lse


def tg_sample_budgets(doc_begin, doc_end, u, min_frac: float, max_frac: float) -> np.ndarray:
    """Random document budgets (host): floor((min_frac + (max_frac -
    min_frac) u_b) * doc_len_b) for the caller's uniform draws u in [0, 1)."""
    db = np.ascontiguousarray(doc_begin, dtype=np.int32)
    de = np.ascontiguousarray(doc_end, dtype=np.int32)
    uu = np.ascontiguousarray(u, dtype=np.float32)
    out = np.empty(db.shape[0], dtype=np.int32)
    p = lambda a, t: a.ctypes.data_as(ctypes.POINTER(t))  # noqa: E731
    _check("tg_sample_budgets", load_library().tg_sample_budgets(
        int(db.shape[0]), p(db, ctypes.c_int32), p(de, ctypes.c_int32), p(uu, ctypes.c_float),
        float(min_frac), float(max_frac), p(out, ctypes.c_int32)))
    return out

