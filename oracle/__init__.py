"""fp64 CPU oracle for sparse top-K KV decode attention -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (``sparse_top_kv_amd``)
never does, and shares no code with it.

This module only marshals numpy arrays into ``liboracle_skv.so`` (built from
``skv_oracle.cpp`` with g++, no fast-math, ``-ffp-contract=off``); every piece of
arithmetic lives in that C++ file, which cites the passages it follows.

Array conventions (all C-contiguous):
  * bf16 tensors are ``numpy.uint16`` arrays of raw bf16 bits, fp32 tensors are
    ``numpy.float32``;
  * K and V are ``[Hkv][n_cap][d]``; a decode query is ``[Hq][d]``; a window of
    W observation queries (or gamma verify queries) is ``[W][Hq][d]``;
  * outputs are fp64 (``out``, ``lse``, ``score64``) plus the fp32 score array.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "skv_oracle.cpp")
_SO = os.path.join(_HERE, "liboracle_skv.so")
_lib = None

F32, BF16 = 0, 1


def build() -> str:
    """Compile the oracle library in-tree with g++ (CPU only)."""
    cmd = ["g++", "-O2", "-std=c++17", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-pthread", "-Wall", "-o", _SO + ".tmp", _SRC]
    subprocess.check_call(cmd)
    os.replace(_SO + ".tmp", _SO)
    global _lib
    _lib = None
    return _SO


class _Problem(ctypes.Structure):
    _fields_ = [("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("scale", ctypes.c_float), ("pad_", ctypes.c_int32),
                ("kv_head_stride", ctypes.c_int64), ("kv_pos_stride", ctypes.c_int64)]


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
            build()
        _lib = ctypes.CDLL(_SO)
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float32:
        return F32
    raise TypeError(f"oracle inputs must be uint16 (bf16 bits) or float32, got {a.dtype}")


def _problem(q: np.ndarray, k: np.ndarray, scale) -> _Problem:
    if k.ndim != 3 or q.shape[-1] != k.shape[2]:
        raise ValueError("K must be [Hkv][n_cap][d] and q [...][Hq][d]")
    if not (q.flags.c_contiguous and k.flags.c_contiguous):
        raise ValueError("oracle inputs must be C-contiguous")
    code = _dtype_code(k)
    if _dtype_code(q) != code:
        raise TypeError("q and K must share a dtype")
    d = k.shape[2]
    sc = np.float32(1.0 / np.sqrt(d) if scale is None or scale <= 0 else scale)
    return _Problem(q.shape[-2], k.shape[0], d, code, float(sc), 0,
                    k.shape[1] * d, d)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (code {rc})")


def score(q_obs: np.ndarray, k: np.ndarray, n: int, scale=None, nthreads=None):
    """Group-summed, window-averaged causal softmax score per kv head.

    q_obs is ``[W][Hq][d]`` (W = 1: a decode query at position n-1).  Returns
    ``(score64 [Hkv][n] float64, score32 [Hkv][n] float32)``.
    """
    lib = _load()
    q_obs = np.ascontiguousarray(q_obs)
    if q_obs.ndim == 2:
        q_obs = q_obs[None]
    p = _problem(q_obs, k, scale)
    hkv = k.shape[0]
    s64 = np.zeros((hkv, n), np.float64)
    s32 = np.zeros((hkv, n), np.float32)
    rc = lib.ora_score(ctypes.byref(p), _ptr(q_obs), ctypes.c_int32(q_obs.shape[0]),
                       _ptr(k), ctypes.c_int64(n), _ptr(s64), _ptr(s32),
                       ctypes.c_int64(n), ctypes.c_int32(nthreads or default_threads()))
    _check(rc, "score")
    return s64, s32


def select(score32: np.ndarray, n_sink: int, n_recent: int, k_per_head, idx_stride=None):
    """Sinks + top-K by (score desc, index asc); returns (idx [Hkv][stride], count)."""
    lib = _load()
    score32 = np.ascontiguousarray(score32, dtype=np.float32)
    hkv, n = score32.shape
    kh = np.ascontiguousarray(np.broadcast_to(np.asarray(k_per_head, np.int32), (hkv,)))
    if idx_stride is None:
        idx_stride = max(1, n_sink + int(kh.max(initial=0)))
    idx = np.full((hkv, idx_stride), -1, np.int32)
    cnt = np.zeros(hkv, np.int32)
    rc = lib.ora_select(_ptr(score32), ctypes.c_int64(n), ctypes.c_int32(hkv),
                        ctypes.c_int64(n), ctypes.c_int32(n_sink), ctypes.c_int32(n_recent),
                        _ptr(kh), _ptr(idx), ctypes.c_int64(idx_stride), _ptr(cnt))
    _check(rc, "select")
    return idx, cnt


def select_topp(score32: np.ndarray, n_sink: int, n_recent: int, lam: float, prune: float,
                pooled: bool = False, fill_mode: int = 0, idx_stride=None):
    """SpecVLM two-stage selection (top-P retention, then uniform fill).
    Returns (idx [H][stride], count [H], count_r [H] = |V_R|)."""
    lib = _load()
    score32 = np.ascontiguousarray(score32, dtype=np.float32)
    h, n = score32.shape
    if idx_stride is None:
        idx_stride = max(1, n - n_recent if n - n_recent > 0 else 1)
    idx = np.full((h, idx_stride), -1, np.int32)
    cnt = np.zeros(h, np.int32)
    cnt_r = np.zeros(h, np.int32)
    rc = lib.ora_select_topp(_ptr(score32), ctypes.c_int64(n), ctypes.c_int32(h), ctypes.c_int64(n),
                             ctypes.c_int32(n_sink), ctypes.c_int32(n_recent), ctypes.c_double(lam),
                             ctypes.c_double(prune), ctypes.c_int32(int(pooled)),
                             ctypes.c_int32(fill_mode), _ptr(idx), ctypes.c_int64(idx_stride),
                             _ptr(cnt), _ptr(cnt_r))
    _check(rc, "select_topp")
    return idx, cnt, cnt_r


def attend_dense(q: np.ndarray, k: np.ndarray, v: np.ndarray, n: int, scale=None,
                 nthreads=None):
    """Exact attention of q [Hq][d] over keys [0, n); returns (out [Hq][d], lse [Hq])."""
    lib = _load()
    q = np.ascontiguousarray(q)
    p = _problem(q, k, scale)
    out = np.zeros((q.shape[0], q.shape[1]), np.float64)
    lse = np.zeros(q.shape[0], np.float64)
    rc = lib.ora_attend_dense(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), ctypes.c_int64(n),
                              _ptr(out), _ptr(lse), ctypes.c_int32(nthreads or default_threads()))
    _check(rc, "attend_dense")
    return out, lse


def attend_sparse(q: np.ndarray, k: np.ndarray, v: np.ndarray, n: int, idx: np.ndarray,
                  count: np.ndarray, tail_start: int, scale=None, nthreads=None):
    """Exact attention over idx[h][:count[h]] followed by [tail_start, n)."""
    lib = _load()
    q = np.ascontiguousarray(q)
    p = _problem(q, k, scale)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    count = np.ascontiguousarray(count, dtype=np.int32)
    out = np.zeros((q.shape[0], q.shape[1]), np.float64)
    lse = np.zeros(q.shape[0], np.float64)
    rc = lib.ora_attend_sparse(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), ctypes.c_int64(n),
                               _ptr(idx), ctypes.c_int64(idx.shape[1]), _ptr(count),
                               ctypes.c_int64(tail_start), _ptr(out), _ptr(lse),
                               ctypes.c_int32(nthreads or default_threads()))
    _check(rc, "attend_sparse")
    return out, lse


def verify(q: np.ndarray, k: np.ndarray, v: np.ndarray, n: int, scale=None, nthreads=None):
    """Causal verify of gamma queries q [gamma][Hq][d] over a cache of length n."""
    lib = _load()
    q = np.ascontiguousarray(q)
    p = _problem(q, k, scale)
    gamma = q.shape[0]
    out = np.zeros(q.shape, np.float64)
    lse = np.zeros(q.shape[:2], np.float64)
    rc = lib.ora_verify(ctypes.byref(p), _ptr(q), ctypes.c_int32(gamma), _ptr(k), _ptr(v),
                        ctypes.c_int64(n), _ptr(out), _ptr(lse),
                        ctypes.c_int32(nthreads or default_threads()))
    _check(rc, "verify")
    return out, lse


def budgets(s: np.ndarray, total_budget: float, window: int, rho: float, n_cand: int):
    """Per-head top-K counts K_i and totals b_i from head scores s (length N)."""
    lib = _load()
    s = np.ascontiguousarray(s, dtype=np.float64)
    k_out = np.zeros(s.shape[0], np.int32)
    b_out = np.zeros(s.shape[0], np.float64)
    rc = lib.ora_budgets(_ptr(s), ctypes.c_int32(s.shape[0]), ctypes.c_double(total_budget),
                         ctypes.c_int32(window), ctypes.c_double(rho), ctypes.c_int64(n_cand),
                         _ptr(k_out), _ptr(b_out))
    _check(rc, "budgets")
    return k_out, b_out
