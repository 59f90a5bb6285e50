"""Full-size workloads through the C ABI against the fp64 oracle.

Each test runs one workload at its real shape in the launch configuration the
bench times, and checks (a) selection bit-exact when fed the oracle's fp32
scores, (b) end-to-end selection equal up to swaps of near-tied entries,
(c) planted structure (heavy hitters, needle) kept, (d) attention within the
bf16 tolerance against the oracle on the GPU's own kept set.  Outputs the
oracle cannot afford at full size are checked on a seeded sample of heads.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_top_kv_amd as skv
import synth
from gpu_util import banner, dev, host, need_gpu

pytestmark = pytest.mark.gpu
ATOL, LSE_ATOL = 2e-3, 1e-4
TINY = np.finfo(np.float32).tiny


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _near_tie_ok(gi, gc, o_idx, o_cnt, s64, lo, hi, K, forced=()):
    """GPU kept set vs oracle kept set for one head: equal sizes, and every
    differing candidate within 1e-5 (relative) of the oracle's K-th score."""
    assert gc == o_cnt
    gs, os_ = set(gi[:gc].tolist()), set(o_idx[:o_cnt].tolist())
    if K > 0 and gs != os_:
        tau = np.sort(s64[lo:hi])[::-1][K - 1]
        for j in gs ^ os_:
            assert abs(s64[j] - tau) <= 1e-5 * tau + TINY, (j, s64[j], tau)
    return gs


def _select_gpu(score, n, S, R, K, stride, ws, kph=None):
    H = score.shape[0]
    idx = torch.full((H, stride), -1, dtype=torch.int32, device="cuda")
    cnt = torch.zeros(H, dtype=torch.int32, device="cuda")
    skv.skv_select(score, n, S, R, K, idx, cnt, ws, k_per_head=kph,
                   k_max=(stride - S) if kph is not None else None)
    return idx, cnt


def _bitexact_select(s32, S, R, K, ws, kph=None):
    o_idx, o_cnt = oracle.select(s32, S, R, K if kph is None else kph)
    n = s32.shape[1]
    idx, cnt = _select_gpu(dev(s32), n, S, R, K if kph is None else 0, o_idx.shape[1], ws,
                           None if kph is None else dev(np.asarray(kph, np.int32)))
    torch.cuda.synchronize()
    gi, gc = host(idx), host(cnt)
    assert np.array_equal(gc, o_cnt)
    for h in range(s32.shape[0]):
        assert np.array_equal(gi[h, :gc[h]], o_idx[h, :o_cnt[h]])
    return o_idx, o_cnt


def test_llama_32k_window_selection_and_sparse_step():
    banner("llama 32K: generate")
    w = synth.llama_obs()
    n, S, R, K, H, Hkv, d = w.n, w.n_sink, w.n_recent, w.k_top, w.n_q_heads, w.n_kv_heads, w.head_dim
    banner("llama 32K: oracle window score")
    s64, s32 = oracle.score(w.q_obs, w.k, n)
    qo, q, kt, vt = dev(w.q_obs), dev(w.q), dev(w.k), dev(w.v)
    ws = skv.Workspace.for_problem(skv.problem_for(qo, kt), n, w.q_obs.shape[0])
    banner("llama 32K: GPU window score + select")
    score = torch.empty((Hkv, n), device="cuda")
    skv.skv_score(qo, kt, n, score, ws)
    idx, cnt = _select_gpu(score, n, S, R, K, S + K, ws)
    torch.cuda.synchronize()
    g = host(score)
    assert np.all(np.abs(g - s64) <= 1e-4 * s64 + 1e-12)
    o_idx, o_cnt = _bitexact_select(s32, S, R, K, ws)
    gi, gc = host(idx), host(cnt)
    for h in range(Hkv):
        gs = _near_tie_ok(gi[h], gc[h], o_idx[h], o_cnt[h], s64[h], S, n - R, K)
        assert set(w.extra["heavy"][h].tolist()) <= gs
    banner("llama 32K: sparse + dense step")
    out = torch.empty((H, d), device="cuda")
    lse = torch.empty(H, device="cuda")
    skv.skv_attend_sparse(q, kt, vt, n, idx, cnt, n - R, out, lse, ws)
    outd = torch.empty((H, d), device="cuda")
    lsed = torch.empty(H, device="cuda")
    skv.skv_attend_dense(q, kt, vt, n, outd, lsed, ws)
    torch.cuda.synchronize()
    ro, rl = oracle.attend_sparse(w.q, w.k, w.v, n, gi, gc, n - R)
    assert np.abs(host(out) - ro).max() <= ATOL and np.abs(host(lse) - rl).max() <= LSE_ATOL
    ro2, rl2 = oracle.attend_sparse(w.q, w.k, w.v, n, o_idx, o_cnt, n - R)
    assert np.abs(host(out) - ro2).max() <= 5 * ATOL  # against the oracle's own kept set
    rd, rdl = oracle.attend_dense(w.q, w.k, w.v, n)
    assert np.abs(host(outd) - rd).max() <= ATOL and np.abs(host(lsed) - rdl).max() <= LSE_ATOL


def test_llama_128k_per_step_topk_with_needle():
    banner("llama 128K: generate")
    w = synth.llama_needle()
    n, S, R, K, H, Hkv, d = w.n, w.n_sink, w.n_recent, w.k_top, w.n_q_heads, w.n_kv_heads, w.head_dim
    p_needle = w.extra["needle"]
    banner("llama 128K: oracle step score")
    s64, s32 = oracle.score(w.q[None], w.k, n)
    q, kt, vt = dev(w.q), dev(w.k), dev(w.v)
    ws = skv.Workspace.for_problem(skv.problem_for(q, kt), n)
    banner("llama 128K: GPU score -> select -> sparse attend")
    score = torch.empty((Hkv, n), device="cuda")
    skv.skv_score(q, kt, n, score, ws)
    idx, cnt = _select_gpu(score, n, S, R, K, S + K, ws)
    out = torch.empty((H, d), device="cuda")
    lse = torch.empty(H, device="cuda")
    skv.skv_attend_sparse(q, kt, vt, n, idx, cnt, n - R, out, lse, ws)
    torch.cuda.synchronize()
    assert np.all(np.abs(host(score) - s64) <= 1e-4 * s64 + 1e-12)
    o_idx, o_cnt = _bitexact_select(s32, S, R, K, ws)
    gi, gc = host(idx), host(cnt)
    for h in range(Hkv):
        gs = _near_tie_ok(gi[h], gc[h], o_idx[h], o_cnt[h], s64[h], S, n - R, K)
        assert p_needle in gs
    ro, rl = oracle.attend_sparse(w.q, w.k, w.v, n, gi, gc, n - R)
    assert np.abs(host(out) - ro).max() <= ATOL and np.abs(host(lse) - rl).max() <= LSE_ATOL
    banner("llama 128K: dense sweep 2K / 8K / 32K / 128K")
    for nn in (2048, 8192, 32768, n):
        od = torch.empty((H, d), device="cuda")
        ld = torch.empty(H, device="cuda")
        skv.skv_attend_dense(q, kt, vt, nn, od, ld, ws)
        torch.cuda.synchronize()
        rd, rdl = oracle.attend_dense(w.q, w.k, w.v, nn)
        assert np.abs(host(od) - rd).max() <= ATOL and np.abs(host(ld) - rdl).max() <= LSE_ATOL


@pytest.mark.parametrize("frac", [0.1, 0.5, 0.9])
def test_llama_128k_needle_sweep(frac):
    n = 131072
    pos = int(frac * n)
    banner(f"needle sweep at {pos}")
    w = synth.llama_needle(needle_pos=pos, trial=1)
    q, kt = dev(w.q), dev(w.k)
    ws = skv.Workspace.for_problem(skv.problem_for(q, kt), n)
    score = torch.empty((w.n_kv_heads, n), device="cuda")
    skv.skv_score(q, kt, n, score, ws)
    idx, cnt = _select_gpu(score, n, w.n_sink, w.n_recent, w.k_top, w.n_sink + w.k_top, ws)
    torch.cuda.synchronize()
    gi, gc = host(idx), host(cnt)
    for h in range(w.n_kv_heads):
        assert pos in set(gi[h, :gc[h]].tolist())


def test_qwen_video_sparse_to_dense_round():
    banner("qwen StD: generate")
    w = synth.qwen_std()
    m_v, m_t, gamma = w.extra["m_v"], w.extra["m_t"], w.extra["gamma"]
    m = m_v + m_t
    H, Hkv, d, K = w.n_q_heads, w.n_kv_heads, w.head_dim, w.k_top
    banner("qwen StD: oracle text-window score (W = 512)")
    s64, s32 = oracle.score(w.q_obs, w.k, m)
    qo, kt, vt = dev(w.q_obs), dev(w.k), dev(w.v)
    ws = skv.Workspace.for_problem(skv.problem_for(qo, kt), m + gamma, m_t)
    banner("qwen StD: GPU score + select")
    score = torch.empty((Hkv, m), device="cuda")
    skv.skv_score(qo, kt, m, score, ws)
    idx, cnt = _select_gpu(score, m, 0, m_t, K, K, ws)
    torch.cuda.synchronize()
    assert np.all(np.abs(host(score) - s64) <= 1e-4 * s64 + 1e-12)
    o_idx, o_cnt = _bitexact_select(s32, 0, m_t, K, ws)
    gi, gc = host(idx), host(cnt)
    for h in range(Hkv):
        _near_tie_ok(gi[h], gc[h], o_idx[h], o_cnt[h], s64[h], 0, m_v, K)
        assert gi[h, :gc[h]].max() < m_v
    banner("qwen StD: SpecVLM top-P + uniform fill on the oracle's scores")
    s32t = dev(s32)
    vidx = torch.empty((Hkv, m_v), dtype=torch.int32, device="cuda")
    vcnt = torch.empty(Hkv, dtype=torch.int32, device="cuda")
    vcr = torch.empty(Hkv, dtype=torch.int32, device="cuda")
    for pooled in (False, True):
        skv.skv_select_topp(s32t, m, 0, m_t, 0.5, 0.9, vidx, vcnt, ws, count_r=vcr, pooled=pooled)
        torch.cuda.synchronize()
        t_idx, t_cnt, t_cr = oracle.select_topp(s32, 0, m_t, 0.5, 0.9, pooled=pooled, idx_stride=m_v)
        vi, vc = host(vidx), host(vcnt)
        assert np.array_equal(vc, t_cnt) and np.array_equal(host(vcr), t_cr)
        assert all(np.array_equal(vi[h, :vc[h]], t_idx[h, :t_cnt[h]]) for h in range(Hkv))
        budget = int(np.floor((1.0 - 0.9) * m_v + 0.5))  # r = 90 %: 10 % of the video tokens
        assert np.array_equal(vc, np.maximum(t_cr, budget))
    qt = dev(np.ascontiguousarray(w.extra["q_draft"][0]))
    out = torch.empty((H, d), device="cuda")
    lse = torch.empty(H, device="cuda")
    skv.skv_attend_sparse(qt, kt, vt, m + 1, vidx, vcnt, m_v, out, lse, ws)
    torch.cuda.synchronize()
    ro, rl = oracle.attend_sparse(np.ascontiguousarray(w.extra["q_draft"][0]), w.k, w.v, m + 1,
                                  t_idx, t_cnt, m_v)
    assert np.abs(host(out) - ro).max() <= ATOL and np.abs(host(lse) - rl).max() <= LSE_ATOL
    banner("qwen StD: 5 draft steps + verify")
    qd = w.extra["q_draft"]
    for t in range(gamma):
        nt = m + t + 1
        qt = dev(np.ascontiguousarray(qd[t]))
        out = torch.empty((H, d), device="cuda")
        lse = torch.empty(H, device="cuda")
        skv.skv_attend_sparse(qt, kt, vt, nt, idx, cnt, m_v, out, lse, ws)
        torch.cuda.synchronize()
        ro, rl = oracle.attend_sparse(np.ascontiguousarray(qd[t]), w.k, w.v, nt, gi, gc, m_v)
        assert np.abs(host(out) - ro).max() <= ATOL and np.abs(host(lse) - rl).max() <= LSE_ATOL
    qv = w.extra["q_verify"]
    n = m + gamma
    out = torch.empty((gamma, H, d), device="cuda")
    lse = torch.empty((gamma, H), device="cuda")
    skv.skv_verify(dev(qv), kt, vt, n, out, lse, ws)
    torch.cuda.synchronize()
    ro, rl = oracle.verify(qv, w.k, w.v, n)
    assert np.abs(host(out) - ro).max() <= ATOL and np.abs(host(lse) - rl).max() <= LSE_ATOL


@pytest.mark.timeout(900)
def test_sparsemm_1024_heads_budgets_and_batched_step():
    banner("sparsemm: generate 1024 heads x 32K (host)")
    w = synth.sparsemm_heads()
    n, H, d, R = w.n, w.n_q_heads, w.head_dim, w.n_recent
    ex = w.extra
    banner("sparsemm: upload")
    qo, q, kt, vt = dev(w.q_obs), dev(w.q), dev(w.k), dev(w.v)
    ws = skv.Workspace.for_problem(skv.problem_for(qo, kt), n, ex["W"])
    banner("sparsemm: budgets")
    k_gpu, b_gpu = skv.skv_budgets(ex["head_scores"], ex["total_budget"], ex["window"], ex["rho"], n - R)
    k_ora, b_ora = oracle.budgets(ex["head_scores"], ex["total_budget"], ex["window"], ex["rho"], n - R)
    assert np.array_equal(k_gpu, k_ora)
    np.testing.assert_allclose(b_gpu, b_ora, rtol=1e-15)
    banner("sparsemm: GPU window score, ragged select, batched sparse step")
    score = torch.empty((H, n), device="cuda")
    skv.skv_score(qo, kt, n, score, ws)
    stride = int(k_gpu.max())
    idx, cnt = _select_gpu(score, n, 0, R, 0, stride, ws, kph=dev(k_gpu))
    out = torch.empty((H, d), device="cuda")
    lse = torch.empty(H, device="cuda")
    skv.skv_attend_sparse(q, kt, vt, n, idx, cnt, n - R, out, lse, ws)
    torch.cuda.synchronize()
    gi, gc = host(idx), host(cnt)
    assert np.array_equal(gc, k_gpu)
    del kt, vt, qo
    sample = np.sort(np.concatenate([
        synth.rng(5, 99).choice(H, 56, replace=False), ex["visual_heads"][:8]]))
    sample = np.unique(sample)
    banner(f"sparsemm: oracle on {len(sample)} sampled heads")
    sub = synth.sparsemm_heads(head_subset=sample)
    s64, s32 = oracle.score(sub.q_obs, sub.k, n)
    g = host(score)[sample]
    assert np.all(np.abs(g - s64) <= 1e-4 * s64 + 1e-12)
    _bitexact_select(s32, 0, R, 0, ws, kph=k_gpu[sample])
    o_idx, o_cnt = oracle.select(s32, 0, R, k_gpu[sample])
    for i, h in enumerate(sample):
        _near_tie_ok(gi[h], gc[h], o_idx[i], o_cnt[i], s64[i], 0, n - R, int(k_gpu[h]))
    ro, rl = oracle.attend_sparse(sub.q, sub.k, sub.v, n, gi[sample], gc[sample], n - R)
    assert np.abs(host(out)[sample] - ro).max() <= ATOL
    assert np.abs(host(lse)[sample] - rl).max() <= LSE_ATOL
