"""Host-side checks of the C ABI: every declared entry point is exported, and
argument validation rejects bad calls before anything reaches the GPU (all
calls here fail validation, so they run on a CPU-only host)."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import sparse_top_kv_amd as skv

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "sparsekv.h")
FAKE = 0x7F0000000000  # aligned, never dereferenced: validation fails first


def _declared():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"\b(skv_[a-z_]+)\s*\(", txt)))


def test_header_declares_the_five_calls_and_library_exports_all():
    names = _declared()
    for f in ("skv_score", "skv_select", "skv_attend_sparse", "skv_attend_dense", "skv_verify"):
        assert f in names
    lib = ctypes.CDLL(skv.library_path())
    for f in names:
        assert hasattr(lib, f), f


def _p(hq=32, hkv=8, d=128, dtype=skv.SKV_BF16, n_cap=4096):
    return skv.problem(hq, hkv, d, dtype, n_cap * d, d)


def _vp(x):
    return ctypes.c_void_p(x)


def _dense(p, n=1000, q=FAKE, ws_bytes=1 << 30, ws=FAKE):
    lib = skv._load()
    return lib.skv_attend_dense(ctypes.byref(p), _vp(q), _vp(FAKE), _vp(FAKE), n, _vp(FAKE), _vp(0),
                                _vp(ws), ws_bytes, _vp(0))


def test_problem_validation():
    assert _dense(_p(hq=30, hkv=8)) == skv.SKV_ERR_INVALID_ARG      # Hq % Hkv
    assert _dense(_p(hq=72, hkv=8)) == skv.SKV_ERR_UNSUPPORTED      # G = 9
    assert _dense(_p(d=96)) == skv.SKV_ERR_UNSUPPORTED
    assert _dense(_p(dtype=7)) == skv.SKV_ERR_INVALID_ARG
    assert _dense(_p(), q=0) == skv.SKV_ERR_INVALID_ARG             # null
    assert _dense(_p(), q=FAKE + 8) == skv.SKV_ERR_INVALID_ARG      # misaligned
    assert _dense(_p(), n=0) == skv.SKV_ERR_INVALID_ARG
    assert _dense(_p(n_cap=512), n=1000) == skv.SKV_ERR_INVALID_ARG  # heads overlap
    assert _dense(_p(), ws_bytes=1024) == skv.SKV_ERR_WORKSPACE
    assert _dense(_p(), ws=FAKE + 64) == skv.SKV_ERR_INVALID_ARG    # ws alignment
    p = _p()
    p.reserved = 1
    assert _dense(p) == skv.SKV_ERR_INVALID_ARG


def test_sparse_select_score_verify_validation():
    lib = skv._load()
    p = _p()
    b = ctypes.byref(p)
    big = 1 << 30
    # tail_start outside [0, n]
    assert lib.skv_attend_sparse(b, _vp(FAKE), _vp(FAKE), _vp(FAKE), 100, _vp(FAKE), 10, _vp(FAKE), 101,
                                 _vp(FAKE), _vp(0), _vp(FAKE), big, _vp(0)) == skv.SKV_ERR_INVALID_ARG
    # idx_stride < n_sink + k_max
    assert lib.skv_select(b, _vp(FAKE), 100, 100, 4, 8, _vp(0), 10, 10, _vp(FAKE), 13, _vp(FAKE),
                          _vp(FAKE), big, _vp(0)) == skv.SKV_ERR_INVALID_ARG
    # k_uniform > k_max
    assert lib.skv_select(b, _vp(FAKE), 100, 100, 4, 8, _vp(0), 11, 10, _vp(FAKE), 14, _vp(FAKE),
                          _vp(FAKE), big, _vp(0)) == skv.SKV_ERR_INVALID_ARG
    # score_stride < n, n_obs > n
    assert lib.skv_score(b, _vp(FAKE), 1, _vp(FAKE), 100, _vp(FAKE), 99, _vp(FAKE), big,
                         _vp(0)) == skv.SKV_ERR_INVALID_ARG
    assert lib.skv_score(b, _vp(FAKE), 101, _vp(FAKE), 100, _vp(FAKE), 100, _vp(FAKE), big,
                         _vp(0)) == skv.SKV_ERR_INVALID_ARG
    # fp32 window scoring and verify (composed from the vector kernels) check
    # their workspace before anything is enqueued
    pf = _p(dtype=skv.SKV_F32)
    assert lib.skv_score(ctypes.byref(pf), _vp(FAKE), 4, _vp(FAKE), 100, _vp(FAKE), 100, _vp(FAKE), 4096,
                         _vp(0)) == skv.SKV_ERR_WORKSPACE
    assert lib.skv_verify(ctypes.byref(pf), _vp(FAKE), 4, _vp(FAKE), _vp(FAKE), 100, _vp(FAKE), _vp(0),
                          _vp(FAKE), 4096, _vp(0)) == skv.SKV_ERR_WORKSPACE
    # gamma > n, gamma above 16
    assert lib.skv_verify(b, _vp(FAKE), 8, _vp(FAKE), _vp(FAKE), 5, _vp(FAKE), _vp(0), _vp(FAKE), big,
                          _vp(0)) == skv.SKV_ERR_INVALID_ARG
    assert lib.skv_verify(b, _vp(FAKE), 17, _vp(FAKE), _vp(FAKE), 100, _vp(FAKE), _vp(0), _vp(FAKE), big,
                          _vp(0)) == skv.SKV_ERR_INVALID_ARG
    # more than 64 rows per kv head run in passes; the workspace covers every gamma
    p7 = _p(hq=56, hkv=8)
    need = skv.skv_workspace_size(p7, 100, 16)
    for g in (9, 10, 13, 16):
        assert lib.skv_verify(ctypes.byref(p7), _vp(FAKE), g, _vp(FAKE), _vp(FAKE), 100, _vp(FAKE), _vp(0),
                              _vp(FAKE), 1024, _vp(0)) == skv.SKV_ERR_WORKSPACE
    assert need > skv.SKV_WS_HEADER_BYTES


def test_workspace_size_is_monotone_and_zero_for_bad_problems():
    p = _p(n_cap=131072)
    sizes = [skv.skv_workspace_size(p, n, 32) for n in (1, 100, 2048, 32768, 131072)]
    assert all(a <= b for a, b in zip(sizes, sizes[1:]))
    assert sizes[0] >= skv.SKV_WS_HEADER_BYTES
    assert skv.skv_workspace_size(_p(hq=72), 100, 1) == 0  # G = 9


def test_budgets_entry_point_equals_oracle():
    rng = np.random.default_rng(5)
    s = rng.exponential(1.0, 1024)
    s[rng.choice(1024, 51, replace=False)] *= 20
    k1, b1 = skv.skv_budgets(s, 1024 * 256, 32, 0.1, 32768 - 32)
    k2, b2 = oracle.budgets(s, 1024 * 256, 32, 0.1, 32768 - 32)
    assert np.array_equal(k1, k2)
    np.testing.assert_allclose(b1, b2, rtol=1e-15)
    with pytest.raises(skv.SkvError):
        skv.skv_budgets(np.array([1.0, -1.0]), 10, 1, 0.1, 5)


def test_gather_validation():
    lib = skv._load()
    p = _p()
    b = ctypes.byref(p)

    def g(n=100, idx_stride=20, tail=90, out=FAKE, ohs=4096 * 128, ops=128, count=FAKE):
        return lib.skv_gather(b, _vp(FAKE), _vp(FAKE), n, _vp(FAKE), idx_stride, _vp(count), tail,
                              _vp(out), _vp(FAKE), ohs, ops, _vp(0), _vp(0))

    assert g(tail=101) == skv.SKV_ERR_INVALID_ARG                 # tail_start > n
    assert g(count=0) == skv.SKV_ERR_INVALID_ARG                  # null count
    assert g(out=0) == skv.SKV_ERR_INVALID_ARG                    # null output
    assert g(out=FAKE + 8) == skv.SKV_ERR_INVALID_ARG             # misaligned output
    assert g(ops=64) == skv.SKV_ERR_INVALID_ARG                   # row stride < d
    assert g(ops=132) == skv.SKV_ERR_INVALID_ARG                  # row stride not 16-byte
    assert g(ohs=29 * 128) == skv.SKV_ERR_INVALID_ARG             # heads overlap: 20 + 10 rows
    assert g(n=0, tail=0) == skv.SKV_ERR_INVALID_ARG
    assert g(idx_stride=0, tail=100) == skv.SKV_ERR_INVALID_ARG   # nothing to copy


def test_binding_constants_match_the_header():
    """The Python binding's copies of the header's constants (workspace header
    size, status and dtype codes) agree with include/sparsekv.h."""
    txt = open(HEADER).read()
    m = re.search(r"#define\s+SKV_WS_HEADER_BYTES\s+(\d+)", txt)
    assert m and int(m.group(1)) == skv.SKV_WS_HEADER_BYTES
    for name in ("SKV_OK", "SKV_F32", "SKV_BF16"):
        mm = re.search(rf"\b{name}\s*=\s*(\d+)", txt)
        assert mm and int(mm.group(1)) == getattr(skv, name), name


def _noalloc(p, n=1000, q=FAKE, idx_stride=64, tail=900):
    lib = skv._load()
    return lib.skv_attend_sparse_noalloc(ctypes.byref(p), _vp(q), _vp(FAKE), _vp(FAKE), n, _vp(FAKE),
                                         idx_stride, _vp(FAKE), tail, _vp(FAKE), _vp(0), _vp(0))


def test_noalloc_entry_point_validates_and_bounds_its_scratch():
    """skv_attend_sparse_noalloc checks its arguments like skv_attend_sparse
    and refuses, before touching any device, a call whose split-K partials do
    not fit its fixed scratch (4096 kv heads x 10,000 rows: about 40 MB)."""
    assert _noalloc(_p(), q=0) == skv.SKV_ERR_INVALID_ARG
    assert _noalloc(_p(), tail=1001) == skv.SKV_ERR_INVALID_ARG
    assert _noalloc(_p(hq=72, hkv=8)) == skv.SKV_ERR_UNSUPPORTED
    big = skv.problem(4096, 4096, 128, skv.SKV_BF16, 10000 * 128, 128)
    assert _noalloc(big, n=10000, idx_stride=9968, tail=9968) == skv.SKV_ERR_WORKSPACE
    # the same call with a caller workspace would need more than the fixed size
    assert skv.skv_workspace_size(big, 10000) > skv.SKV_NOALLOC_SCRATCH_BYTES


def _topk(p, n=1000, q=FAKE, score=FAKE, score_stride=1000, S=4, R=64, K=256, idx_stride=260, count=FAKE):
    lib = skv._load()
    return lib.skv_topk_step(ctypes.byref(p), _vp(q), _vp(FAKE), _vp(FAKE), ctypes.c_int64(n), S, R, K,
                             _vp(score), ctypes.c_int64(score_stride), _vp(FAKE), ctypes.c_int64(idx_stride),
                             _vp(count), _vp(FAKE), _vp(0), _vp(FAKE), ctypes.c_size_t(1 << 30), _vp(0))


def test_topk_step_validation():
    """skv_topk_step rejects, before any device call, what the three calls it
    stands for would reject: a missing score row (required), a score stride
    below n, an index row too short for the sinks and K, negative counts."""
    assert _topk(_p(), score=0) == skv.SKV_ERR_INVALID_ARG
    assert _topk(_p(), score_stride=999) == skv.SKV_ERR_INVALID_ARG
    assert _topk(_p(), idx_stride=259) == skv.SKV_ERR_INVALID_ARG
    assert _topk(_p(), K=-1) == skv.SKV_ERR_INVALID_ARG
    assert _topk(_p(), S=-1) == skv.SKV_ERR_INVALID_ARG
    assert _topk(_p(), count=0) == skv.SKV_ERR_INVALID_ARG
    assert _topk(_p(), n=0) == skv.SKV_ERR_INVALID_ARG
    assert _topk(_p(), q=FAKE + 4) == skv.SKV_ERR_INVALID_ARG
    assert _topk(_p(hq=72, hkv=8)) == skv.SKV_ERR_UNSUPPORTED


def test_topk_error_word_offset_matches_the_header():
    txt = open(HEADER).read()
    m = re.search(r"#define\s+SKV_TOPK_ERROR_OFFSET\s+\(SKV_WS_HEADER_BYTES\s*-\s*(\d+)\s*\*\s*(\d+)\s*-\s*(\d+)\)", txt)
    assert m, "SKV_TOPK_ERROR_OFFSET"
    off = skv.SKV_WS_HEADER_BYTES - int(m.group(1)) * int(m.group(2)) - int(m.group(3))
    assert off == skv.SKV_TOPK_ERROR_OFFSET
