"""Python binding of libsparsekv (sparse top-K KV decode attention on MI355X).

Argument marshalling only: every step runs in the HIP kernels of
``libsparsekv.so`` (built from ``csrc/`` by ``sparse_top_kv_amd.build``).  The
functions carry the C names (``skv_score``, ``skv_select``,
``skv_attend_sparse``, ``skv_attend_sparse_noalloc``, ``skv_attend_dense``,
``skv_verify``, ``skv_topk_step``, ``skv_gather``, ``skv_select_topp``, ``skv_budgets``)
and take torch tensors on a ROCm device; torch provides device memory and the
current stream, nothing else.  A missing library raises at the first call.

Layouts (see ``include/sparsekv.h``): K and V are ``[Hkv][n_cap][d]`` with
any row/head strides that keep 16-byte alignment; queries are
``[rows][Hq][d]`` contiguous (a single decode query may be ``[Hq][d]``);
outputs are fp32.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsparsekv.so")

SKV_OK, SKV_ERR_INVALID_ARG, SKV_ERR_UNSUPPORTED, SKV_ERR_WORKSPACE, SKV_ERR_HIP = range(5)
SKV_F32, SKV_BF16 = 0, 1
SKV_WS_HEADER_BYTES = 1048576
SKV_NOALLOC_SCRATCH_BYTES = 16 * 1048576
SKV_TOPK_ERROR_OFFSET = SKV_WS_HEADER_BYTES - 64 * 128 - 128
_ALIGN = 256

_lib = None


class SkvError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        msg = _load().skv_status_string(status).decode()
        super().__init__(f"{what}: {msg} (status {status})")


class Problem(ctypes.Structure):
    _fields_ = [("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("scale", ctypes.c_float), ("reserved", ctypes.c_int32),
                ("kv_head_stride", ctypes.c_int64), ("kv_pos_stride", ctypes.c_int64)]


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libsparsekv.so is not built ({LIB_PATH}); run "
                               "`python -m sparse_top_kv_amd.build` or __graft_entry__.build()")
        lib = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        P = ctypes.POINTER(Problem)
        lib.skv_status_string.restype = ctypes.c_char_p
        lib.skv_status_string.argtypes = [ctypes.c_int]
        lib.skv_version.restype = i32
        lib.skv_workspace_size.restype = sz
        lib.skv_workspace_size.argtypes = [P, i64, i32]
        lib.skv_workspace_init.argtypes = [vp, sz, vp]
        lib.skv_score.argtypes = [P, vp, i32, vp, i64, vp, i64, vp, sz, vp]
        lib.skv_select.argtypes = [P, vp, i64, i64, i32, i32, vp, i32, i32, vp, i64, vp, vp, sz, vp]
        lib.skv_attend_sparse.argtypes = [P, vp, vp, vp, i64, vp, i64, vp, i64, vp, vp, vp, sz, vp]
        lib.skv_attend_sparse_noalloc.argtypes = [P, vp, vp, vp, i64, vp, i64, vp, i64, vp, vp, vp]
        lib.skv_attend_dense.argtypes = [P, vp, vp, vp, i64, vp, vp, vp, sz, vp]
        lib.skv_topk_step.argtypes = [P, vp, vp, vp, i64, i32, i32, i32, vp, i64, vp, i64, vp, vp, vp,
                                      vp, sz, vp]
        lib.skv_verify.argtypes = [P, vp, i32, vp, vp, i64, vp, vp, vp, sz, vp]
        dbl = ctypes.c_double
        lib.skv_select_topp.argtypes = [P, vp, i64, i64, i32, i32, dbl, dbl, i32, i32, vp, i64, vp,
                                        vp, vp, sz, vp]
        lib.skv_gather.argtypes = [P, vp, vp, i64, vp, i64, vp, i64, vp, vp, i64, i64, vp, vp]
        lib.skv_budgets.argtypes = [vp, i32, ctypes.c_double, i32, ctypes.c_double, i64, vp, vp]
        for f in ("skv_workspace_init", "skv_score", "skv_select", "skv_attend_sparse",
                  "skv_attend_sparse_noalloc", "skv_topk_step",
                  "skv_attend_dense", "skv_verify", "skv_gather", "skv_select_topp", "skv_budgets"):
            getattr(lib, f).restype = ctypes.c_int
        _lib = lib
    return _lib


def library_path() -> str:
    return LIB_PATH


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return SKV_BF16
    if t.dtype == torch.float32:
        return SKV_F32
    raise TypeError(f"q/K/V must be bfloat16 or float32, got {t.dtype}")


def _stream(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _check_dev(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("libsparsekv takes device tensors")


def problem(q_heads: int, kv_heads: int, head_dim: int, dtype: int, kv_head_stride: int,
            kv_pos_stride: int, scale: float = 0.0) -> Problem:
    return Problem(q_heads, kv_heads, head_dim, dtype, float(scale), 0, kv_head_stride,
                   kv_pos_stride)


def problem_for(q, k, scale: float = 0.0) -> Problem:
    """Problem descriptor from a query tensor [..][Hq][d] and a cache [Hkv][cap][d]."""
    if k.dim() != 3 or k.stride(2) != 1:
        raise ValueError("cache must be [Hkv][n_cap][d] with contiguous channels")
    if q.dtype != k.dtype:
        raise TypeError("q and the cache must share a dtype")
    return problem(q.shape[-2], k.shape[0], k.shape[2], _dtype_code(k), k.stride(0),
                   k.stride(1), scale)


def skv_workspace_size(p: Problem, n_max: int, rows_max: int = 1) -> int:
    return int(_load().skv_workspace_size(ctypes.byref(p), n_max, rows_max))


class Workspace:
    """Device scratch for libsparsekv calls (torch-allocated, 256-byte aligned,
    reserved header zeroed once; every call leaves it zero).  Calls sharing it
    must be ordered on one stream."""

    def __init__(self, nbytes: int, device=None, stream=None):
        torch = _torch()
        if nbytes <= 0:
            raise ValueError("workspace size must be positive (invalid problem?)")
        self._buf = torch.empty(nbytes + _ALIGN, dtype=torch.uint8, device=device or "cuda")
        off = (-self._buf.data_ptr()) % _ALIGN
        self.tensor = self._buf[off:off + nbytes]
        self.nbytes = nbytes
        st = _load().skv_workspace_init(_ptr(self.tensor), nbytes, _stream(stream))
        if st != SKV_OK:
            raise SkvError(st, "skv_workspace_init")

    @property
    def ptr(self):
        return _ptr(self.tensor)

    @classmethod
    def for_problem(cls, p: Problem, n_max: int, rows_max: int = 1, device=None, stream=None):
        return cls(skv_workspace_size(p, n_max, rows_max), device, stream)


def skv_workspace_init(ws: Workspace, stream=None):
    st = _load().skv_workspace_init(ws.ptr, ws.nbytes, _stream(stream))
    if st != SKV_OK:
        raise SkvError(st, "skv_workspace_init")


def _idx_stride(idx):
    # an empty index list [Hkv][0] has no row stride to speak of
    return idx.stride(0) if idx.shape[-1] > 0 else 0


def _rows(q, hq):
    return q.shape[0] if q.dim() == 3 else 1


def skv_score(q, k, n: int, score, ws: Workspace, scale: float = 0.0, stream=None):
    """score[h][j] for j < n from window queries q [W][Hq][d] (or a decode query [Hq][d])."""
    _check_dev(q, k, score)
    if not q.is_contiguous() or score.dtype != _torch().float32 or score.stride(1) != 1:
        raise ValueError("q must be contiguous and score fp32 [Hkv][>=n]")
    p = problem_for(q, k, scale)
    st = _load().skv_score(ctypes.byref(p), _ptr(q), _rows(q, p.n_q_heads), _ptr(k), n,
                           _ptr(score), score.stride(0), ws.ptr, ws.nbytes, _stream(stream))
    if st != SKV_OK:
        raise SkvError(st, "skv_score")
    return score


def skv_select(score, n: int, n_sink: int, n_recent: int, k_uniform: int, idx, count,
               ws: Workspace, k_per_head=None, k_max: int | None = None, stream=None):
    """Sinks + top-K per kv head on an fp32 score [Hkv][>=n]; writes idx, count (int32)."""
    torch = _torch()
    _check_dev(score, idx, count, k_per_head)
    for t in (idx, count) + ((k_per_head,) if k_per_head is not None else ()):
        if t.dtype != torch.int32:
            raise TypeError("idx, count and k_per_head are int32")
    if k_max is None:
        k_max = k_uniform if k_per_head is None else idx.shape[1] - n_sink
    p = problem(score.shape[0], score.shape[0], 128, SKV_BF16, 128, 128)
    st = _load().skv_select(ctypes.byref(p), _ptr(score), score.stride(0), n, n_sink, n_recent,
                            _ptr(k_per_head), k_uniform, k_max, _ptr(idx), idx.stride(0),
                            _ptr(count), ws.ptr, ws.nbytes, _stream(stream))
    if st != SKV_OK:
        raise SkvError(st, "skv_select")
    return idx, count


def skv_select_topp(score, n: int, n_sink: int, n_recent: int, lam: float, prune: float, idx,
                    count, ws: Workspace, count_r=None, pooled: bool = False, fill_mode: int = 0,
                    stream=None):
    """SpecVLM selection on an fp32 score [rows][>=n]: top-P retention (mass >= lam of the
    total) plus a uniform fill; writes idx, count and (optionally) count_r = |V_R|."""
    torch = _torch()
    _check_dev(score, idx, count, count_r)
    for t in (idx, count) + ((count_r,) if count_r is not None else ()):
        if t.dtype != torch.int32:
            raise TypeError("idx, count and count_r are int32")
    if score.dtype != torch.float32 or score.stride(1) != 1:
        raise ValueError("score must be fp32 [rows][>=n]")
    p = problem(score.shape[0], score.shape[0], 128, SKV_BF16, 128, 128)
    st = _load().skv_select_topp(ctypes.byref(p), _ptr(score), score.stride(0), n, n_sink,
                                 n_recent, float(lam), float(prune), int(pooled), fill_mode,
                                 _ptr(idx), idx.stride(0), _ptr(count), _ptr(count_r), ws.ptr,
                                 ws.nbytes, _stream(stream))
    if st != SKV_OK:
        raise SkvError(st, "skv_select_topp")
    return idx, count


def skv_attend_sparse(q, k, v, n: int, idx, count, tail_start: int, out, lse, ws: Workspace,
                      scale: float = 0.0, stream=None):
    """Decode attention over idx[h][:count[h]] and the tail [tail_start, n)."""
    _check_dev(q, k, v, idx, count, out, lse)
    if k.stride() != v.stride():
        raise ValueError("K and V must share strides")
    p = problem_for(q, k, scale)
    st = _load().skv_attend_sparse(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), n, _ptr(idx),
                                   _idx_stride(idx), _ptr(count), tail_start, _ptr(out), _ptr(lse),
                                   ws.ptr, ws.nbytes, _stream(stream))
    if st != SKV_OK:
        raise SkvError(st, "skv_attend_sparse")
    return out, lse


def skv_attend_sparse_noalloc(q, k, v, n: int, idx, count, tail_start: int, out, lse,
                              scale: float = 0.0, stream=None):
    """skv_attend_sparse on the library's fixed per-GPU scratch (no workspace)."""
    _check_dev(q, k, v, idx, count, out, lse)
    if k.stride() != v.stride():
        raise ValueError("K and V must share strides")
    p = problem_for(q, k, scale)
    st = _load().skv_attend_sparse_noalloc(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), n,
                                           _ptr(idx), _idx_stride(idx), _ptr(count), tail_start,
                                           _ptr(out), _ptr(lse), _stream(stream))
    if st != SKV_OK:
        raise SkvError(st, "skv_attend_sparse_noalloc")
    return out, lse


def skv_topk_step(q, k, v, n: int, n_sink: int, n_recent: int, k_top: int, score, idx, count, out,
                  lse, ws: Workspace, scale: float = 0.0, stream=None):
    """Per-step top-K decode step: score of the decode query q [Hq][d], sinks + top-K +
    recent run, attention over that set (score, idx, count, out, lse written)."""
    torch = _torch()
    _check_dev(q, k, v, score, idx, count, out, lse)
    if k.stride() != v.stride():
        raise ValueError("K and V must share strides")
    if score.dtype != torch.float32 or score.stride(1) != 1:
        raise ValueError("score must be fp32 [Hkv][>=n]")
    for t in (idx, count):
        if t.dtype != torch.int32:
            raise TypeError("idx and count are int32")
    p = problem_for(q, k, scale)
    st = _load().skv_topk_step(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), n, n_sink, n_recent, k_top,
                               _ptr(score), score.stride(0), _ptr(idx), _idx_stride(idx), _ptr(count),
                               _ptr(out), _ptr(lse), ws.ptr, ws.nbytes, _stream(stream))
    if st != SKV_OK:
        raise SkvError(st, "skv_topk_step")
    return out, lse


def skv_attend_dense(q, k, v, n: int, out, lse, ws: Workspace, scale: float = 0.0, stream=None):
    """Decode attention of q [Hq][d] over keys [0, n)."""
    _check_dev(q, k, v, out, lse)
    if k.stride() != v.stride():
        raise ValueError("K and V must share strides")
    p = problem_for(q, k, scale)
    st = _load().skv_attend_dense(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), n, _ptr(out),
                                  _ptr(lse), ws.ptr, ws.nbytes, _stream(stream))
    if st != SKV_OK:
        raise SkvError(st, "skv_attend_dense")
    return out, lse


def skv_verify(q, k, v, n: int, out, lse, ws: Workspace, scale: float = 0.0, stream=None):
    """Causal verify of q [gamma][Hq][d]; the gamma new entries end at n."""
    _check_dev(q, k, v, out, lse)
    if k.stride() != v.stride():
        raise ValueError("K and V must share strides")
    p = problem_for(q, k, scale)
    st = _load().skv_verify(ctypes.byref(p), _ptr(q), q.shape[0], _ptr(k), _ptr(v), n,
                            _ptr(out), _ptr(lse), ws.ptr, ws.nbytes, _stream(stream))
    if st != SKV_OK:
        raise SkvError(st, "skv_verify")
    return out, lse


def skv_gather(k, v, n: int, idx, count, tail_start: int, k_out, v_out, rows_out=None,
               stream=None):
    """Copy each kv head's idx[h][:count[h]] rows and the tail [tail_start, n) of K and V
    into k_out / v_out ([Hkv][>= rows_max][d], same dtype); rows_out[h] = rows copied."""
    torch = _torch()
    _check_dev(k, v, idx, count, k_out, v_out, rows_out)
    if k.stride() != v.stride() or k_out.stride() != v_out.stride():
        raise ValueError("K and V (and their outputs) must share strides")
    if k_out.dtype != k.dtype or v.dtype != k.dtype or k_out.stride(2) != 1:
        raise ValueError("outputs must match the cache dtype with contiguous channels")
    for t in (idx, count) + ((rows_out,) if rows_out is not None else ()):
        if t.dtype != torch.int32:
            raise TypeError("idx, count and rows_out are int32")
    p = problem(k.shape[0], k.shape[0], k.shape[2], _dtype_code(k), k.stride(0), k.stride(1))
    st = _load().skv_gather(ctypes.byref(p), _ptr(k), _ptr(v), n, _ptr(idx), _idx_stride(idx),
                            _ptr(count), tail_start, _ptr(k_out), _ptr(v_out), k_out.stride(0),
                            k_out.stride(1), _ptr(rows_out), _stream(stream))
    if st != SKV_OK:
        raise SkvError(st, "skv_gather")
    return k_out, v_out


def skv_budgets(s, total_budget: float, window: int, rho: float, n_cand: int):
    """SparseMM per-head budgets (host): returns (K per head int32, b per head float64)."""
    s = np.ascontiguousarray(s, dtype=np.float64)
    k_out = np.zeros(s.shape[0], np.int32)
    b_out = np.zeros(s.shape[0], np.float64)
    st = _load().skv_budgets(s.ctypes.data, s.shape[0], float(total_budget), window, float(rho),
                             n_cand, k_out.ctypes.data, b_out.ctypes.data)
    if st != SKV_OK:
        raise SkvError(st, "skv_budgets")
    return k_out, b_out


def skv_version() -> int:
    return int(_load().skv_version())
