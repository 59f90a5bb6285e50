"""GPU parity of the MFMA kernels (causal verify, observation-window score)
against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import sparse_top_kv_amd as skv
import synth
from gpu_util import banner, dev, host, need_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _rand(shape, seed):
    return synth.bf16_bits(np.random.default_rng(seed).standard_normal(shape).astype(np.float32))


@pytest.mark.parametrize("hq,hkv,d", [(28, 4, 128), (32, 8, 128), (8, 8, 64), (16, 2, 64)])
@pytest.mark.parametrize("gamma,n", [(5, 5), (5, 300), (1, 77), (5, 3001), (8, 1000), (13, 2000), (16, 777)])
def test_verify_matches_oracle(hq, hkv, d, gamma, n):
    # gamma * G above 64 rows per kv head runs as several passes
    _check_verify(hq, hkv, d, gamma, n)


@pytest.mark.parametrize("hq,hkv,d,gamma,n", [(16, 4, 128, 9, 700), (16, 4, 64, 9, 1500), (28, 4, 64, 5, 1200),
                                              (28, 4, 128, 6, 900), (16, 2, 128, 5, 2500), (15, 3, 64, 7, 600)])
def test_verify_fold_rounds(hq, hkv, d, gamma, n):
    """35 and 36 rows per kv head fold in one round (the third row group's
    single row quad parked beside the ring); 40 and 42 rows take two."""
    _check_verify(hq, hkv, d, gamma, n)


@pytest.mark.parametrize("hq,hkv,d,gamma,n", [(32, 2, 128, 4, 500), (32, 2, 128, 9, 1000), (18, 3, 128, 5, 800),
                                              (24, 8, 64, 13, 700)])
def test_verify_other_group_sizes(hq, hkv, d, gamma, n):
    """Groups of 16 (four queries per pass: one pass, then three), 6 and 3."""
    _check_verify(hq, hkv, d, gamma, n)


def _check_verify(hq, hkv, d, gamma, n):
    banner(f"verify hq={hq} hkv={hkv} d={d} gamma={gamma} n={n}")
    q = _rand((gamma, hq, d), 1)
    k = _rand((hkv, n + 2, d), 2)
    v = _rand((hkv, n + 2, d), 3)
    ref_o, ref_l = oracle.verify(q, k, v, n)
    qt, kt, vt = dev(q), dev(k), dev(v)
    out = torch.full((gamma, hq, d), float("nan"), device="cuda")
    lse = torch.full((gamma, hq), float("nan"), device="cuda")
    ws = skv.Workspace.for_problem(skv.problem_for(qt, kt), n, gamma)
    skv.skv_verify(qt, kt, vt, n, out, lse, ws)
    torch.cuda.synchronize()
    assert np.abs(host(out) - ref_o).max() <= 2e-3
    assert np.abs(host(lse) - ref_l).max() <= 1e-4
    # each verify row equals the dense step at its own prefix
    for t in range(gamma):
        od = torch.empty((hq, d), device="cuda")
        ld = torch.empty(hq, device="cuda")
        skv.skv_attend_dense(qt[t].contiguous(), kt, vt, n - gamma + t + 1, od, ld, ws)
        torch.cuda.synchronize()
        assert (od - out[t]).abs().max().item() <= 2e-3


@pytest.mark.parametrize("hq,hkv,d", [(28, 4, 128), (32, 8, 128), (8, 8, 64)])
@pytest.mark.parametrize("gamma,n", [(16, 777), (5, 300), (13, 2000)])
def test_verify_with_every_logit_far_below_zero(hq, hkv, d, gamma, n):
    """Softmax is shift-invariant: with every logit near -100 a row whose
    wave saw no visible key in its first tile must still take its reference
    from the keys it does see (a stand-in reference of 0 would underflow every
    probability to zero and return out = 0, lse = -inf)."""
    banner(f"verify logits near -100 hq={hq} hkv={hkv} d={d} gamma={gamma} n={n}")
    rng = np.random.default_rng(31)
    u = rng.standard_normal(d).astype(np.float32)
    u /= np.linalg.norm(u)
    kf = 4.0 * u + 0.05 * rng.standard_normal((hkv, n + 2, d)).astype(np.float32)
    # q . k * d^-0.5 ~= -100 for every key: q = -c u with 4 c d^-0.5 = 100
    c = 100.0 * np.sqrt(d) / 4.0
    qf = -c * u + 0.05 * rng.standard_normal((gamma, hq, d)).astype(np.float32)
    q, k = synth.bf16_bits(qf.astype(np.float32)), synth.bf16_bits(kf.astype(np.float32))
    v = _rand((hkv, n + 2, d), 32)
    ref_o, ref_l = oracle.verify(q, k, v, n)
    assert ref_l.max() < -80.0  # every row's normaliser is far below zero
    qt, kt, vt = dev(q), dev(k), dev(v)
    out = torch.full((gamma, hq, d), float("nan"), device="cuda")
    lse = torch.full((gamma, hq), float("nan"), device="cuda")
    ws = skv.Workspace.for_problem(skv.problem_for(qt, kt), n, gamma)
    skv.skv_verify(qt, kt, vt, n, out, lse, ws)
    torch.cuda.synchronize()
    assert np.all(np.isfinite(host(lse)))
    assert np.abs(host(out) - ref_o).max() <= 2e-3
    assert np.abs(host(lse) - ref_l).max() <= 1e-4


@pytest.mark.parametrize("hq,hkv,d", [(32, 8, 128), (28, 4, 128), (4, 4, 64), (8, 1, 128), (24, 8, 128), (32, 2, 64)])
@pytest.mark.parametrize("W,n", [(32, 32), (32, 1000), (2, 300), (32, 4097), (20, 257)])
def test_obs_score_matches_oracle(hq, hkv, d, W, n):
    banner(f"obs score hq={hq} hkv={hkv} d={d} W={W} n={n}")
    q = _rand((W, hq, d), 4)
    k = _rand((hkv, n, d), 5)
    s64, s32 = oracle.score(q, k, n)
    qt, kt = dev(q), dev(k)
    score = torch.full((hkv, n + 3), float("nan"), device="cuda")
    ws = skv.Workspace.for_problem(skv.problem_for(qt, kt), n, W)
    skv.skv_score(qt, kt, n, score, ws)
    torch.cuda.synchronize()
    g = host(score)[:, :n]
    assert np.all(np.isfinite(g))
    assert np.all(np.abs(g - s64) <= 1e-4 * s64 + 1e-12)
    np.testing.assert_allclose(g.sum(1), hq // hkv, rtol=1e-4)


@pytest.mark.parametrize("hq,hkv,W,n", [(7, 1, 80, 70000), (28, 4, 64, 3000)])
def test_obs_score_row_groups(hq, hkv, W, n):
    """Few (kv head, key block) workgroups and many window rows: the rows are
    split into groups whose key sums are added at the end.  The first case has
    5 chunks of 128 rows over 4 groups of 2 (the last group holds none)."""
    banner(f"obs score row groups hq={hq} hkv={hkv} W={W} n={n}")
    d = 128
    q = _rand((W, hq, d), 6)
    k = _rand((hkv, n, d), 7)
    s64, _ = oracle.score(q, k, n)
    qt, kt = dev(q), dev(k)
    score = torch.full((hkv, n + 3), float("nan"), device="cuda")
    ws = skv.Workspace.for_problem(skv.problem_for(qt, kt), n, W)
    skv.skv_score(qt, kt, n, score, ws)
    torch.cuda.synchronize()
    g = host(score)[:, :n]
    assert np.all(np.isfinite(g))
    assert np.all(np.abs(g - s64) <= 1e-4 * s64 + 1e-12)
    np.testing.assert_allclose(g.sum(1), hq // hkv, rtol=1e-4)


def test_window_select_end_to_end_near_ties():
    """Window score on the GPU -> select on the GPU; the kept set may differ from
    the oracle's only by swaps of near-tied entries at the threshold."""
    banner("obs score -> select end to end")
    w = synth.llama_obs(n=4096)
    n, S, R = w.n, w.n_sink, w.n_recent
    K = int(0.3 * n) - S - R
    s64, s32 = oracle.score(w.q_obs, w.k, n)
    o_idx, o_cnt = oracle.select(s32, S, R, K)
    qt, kt = dev(w.q_obs), dev(w.k)
    ws = skv.Workspace.for_problem(skv.problem_for(qt, kt), n, w.q_obs.shape[0])
    score = torch.empty((w.n_kv_heads, n), device="cuda")
    skv.skv_score(qt, kt, n, score, ws)
    idx = torch.empty((w.n_kv_heads, S + K), dtype=torch.int32, device="cuda")
    cnt = torch.empty(w.n_kv_heads, dtype=torch.int32, device="cuda")
    skv.skv_select(score, n, S, R, K, idx, cnt, ws)
    torch.cuda.synchronize()
    gi, gc = host(idx), host(cnt)
    assert np.array_equal(gc, o_cnt)
    for h in range(w.n_kv_heads):
        gs, os_ = set(gi[h, :gc[h]]), set(o_idx[h, :o_cnt[h]])
        tau = np.sort(s64[h, S:n - R])[::-1][K - 1]
        for j in gs ^ os_:
            assert abs(s64[h, j] - tau) <= 1e-5 * tau + np.finfo(np.float32).tiny
        assert set(w.extra["heavy"][h].tolist()) <= gs


@pytest.mark.parametrize("hq,hkv,d,gamma,n", [(28, 4, 128, 5, 300), (32, 8, 64, 16, 777), (8, 8, 128, 1, 77),
                                              (32, 2, 128, 9, 1000)])
def test_verify_f32_matches_oracle(hq, hkv, d, gamma, n):
    """fp32 caches: one decode step per drafted query over its prefix."""
    banner(f"verify f32 hq={hq} hkv={hkv} d={d} gamma={gamma} n={n}")
    rng = np.random.default_rng(21)
    q = rng.standard_normal((gamma, hq, d)).astype(np.float32)
    k = rng.standard_normal((hkv, n + 2, d)).astype(np.float32)
    v = rng.standard_normal((hkv, n + 2, d)).astype(np.float32)
    ref_o, ref_l = oracle.verify(q, k, v, n)
    qt, kt, vt = dev(q), dev(k), dev(v)
    out = torch.full((gamma, hq, d), float("nan"), device="cuda")
    lse = torch.full((gamma, hq), float("nan"), device="cuda")
    ws = skv.Workspace.for_problem(skv.problem_for(qt, kt), n, gamma)
    skv.skv_verify(qt, kt, vt, n, out, lse, ws)
    torch.cuda.synchronize()
    assert np.abs(host(out) - ref_o).max() <= 1e-5
    assert np.abs(host(lse) - ref_l).max() <= 1e-5


@pytest.mark.parametrize("hq,hkv,d,W,n", [(32, 8, 128, 32, 1000), (28, 4, 64, 20, 257), (8, 1, 128, 2, 300),
                                          (16, 1, 64, 5, 4097), (24, 8, 128, 7, 7)])
def test_obs_score_f32_matches_oracle(hq, hkv, d, W, n):
    """fp32 window: one per-step score per window row over its prefix, added
    in row order."""
    banner(f"obs score f32 hq={hq} hkv={hkv} d={d} W={W} n={n}")
    rng = np.random.default_rng(22)
    q = rng.standard_normal((W, hq, d)).astype(np.float32)
    k = rng.standard_normal((hkv, n, d)).astype(np.float32)
    s64, _ = oracle.score(q, k, n)
    qt, kt = dev(q), dev(k)
    score = torch.full((hkv, n + 3), float("nan"), device="cuda")
    ws = skv.Workspace.for_problem(skv.problem_for(qt, kt), n, W)
    skv.skv_score(qt, kt, n, score, ws)
    torch.cuda.synchronize()
    g = host(score)[:, :n]
    assert np.all(np.isfinite(g))
    assert np.all(np.abs(g - s64) <= 1e-4 * s64 + 1e-12)
    np.testing.assert_allclose(g.sum(1), hq // hkv, rtol=1e-4)
