"""GPU parity of skv_topk_step, the per-step top-K decode step in one call
("Sparse-to-Dense ..." Sec. 3.2 top-K attention; "Where Activation Sparsity
and KV-Cache Sparsity Cross ...", "Speedup Across Context": sinks, selected
history and recent run).

For every case: the scores equal skv_score's bit for bit and the oracle's
within 1e-4 (relative); the kept set equals the oracle's selection on the
GPU's own fp32 scores bit for bit; out and lse match the oracle's attention
over that kept set (2e-3 / 1e-4 for bf16, 1e-5 for fp32); a repeated call is
bit-identical; the step's error word stays zero.  Shapes cover the one-launch
form (several chunks per kv head, a ragged last chunk, K = 0, K at and past
the candidate count, exact ties, head dims 64 and 128, groups 1, 4 and 7) and
the three-call form it falls back to (fp32 caches, caches too long for the
chunk logits to stay on chip)."""
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


def _rand(shape, seed, dtype):
    x = np.random.default_rng(seed).standard_normal(shape).astype(np.float32)
    return synth.bf16_bits(x) if dtype == "bf16" else x


def _run_step(q, k, v, n, S, R, K, ws):
    hq, d = q.shape[-2], q.shape[-1]
    hkv = k.shape[0]
    score = torch.full((hkv, n + 3), float("nan"), device="cuda")
    stride = max(S + K, 1)
    idx = torch.full((hkv, stride), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((hkv,), -7, dtype=torch.int32, device="cuda")
    out = torch.full((hq, d), float("nan"), device="cuda")
    lse = torch.full((hq,), float("nan"), device="cuda")
    skv.skv_topk_step(q, k, v, n, S, R, K, score, idx, cnt, out, lse, ws)
    return score, idx, cnt, out, lse


def _check(q, k, v, n, S, R, K, dtype, tag):
    banner(f"topk step {tag}: hq={q.shape[0]} hkv={k.shape[0]} d={q.shape[1]} n={n} S={S} R={R} K={K}")
    qt, kt, vt = dev(q), dev(k), dev(v)
    ws = skv.Workspace.for_problem(skv.problem_for(qt, kt), n)
    score, idx, cnt, out, lse = _run_step(qt, kt, vt, n, S, R, K, ws)
    # the three calls on the same inputs
    hkv = k.shape[0]
    sc3 = torch.full((hkv, n + 3), float("nan"), device="cuda")
    skv.skv_score(qt, kt, n, sc3, ws)
    score2, idx2, cnt2, out2, lse2 = _run_step(qt, kt, vt, n, S, R, K, ws)
    torch.cuda.synchronize()
    err = int(ws.tensor[skv.SKV_TOPK_ERROR_OFFSET:skv.SKV_TOPK_ERROR_OFFSET + 4].view(torch.int32).item())
    assert err == 0
    assert torch.equal(score[:, :n], sc3[:, :n])
    for a, b in ((score[:, :n], score2[:, :n]), (idx, idx2), (cnt, cnt2), (out, out2), (lse, lse2)):
        assert torch.equal(a, b)  # (the score rows' padding past n stays NaN)
    s32 = host(score)[:, :n]
    s64, _ = oracle.score(q[None], k, n)
    assert np.all(np.abs(s32 - s64) <= 1e-4 * s64 + 1e-12)
    o_idx, o_cnt = oracle.select(np.ascontiguousarray(s32), S, R, K, idx_stride=idx.shape[1])
    gi, gc = host(idx), host(cnt)
    assert np.array_equal(gc, o_cnt)
    for h in range(hkv):
        assert np.array_equal(gi[h, :gc[h]], o_idx[h, :o_cnt[h]]), h
    tail = max(n - R, 0)
    ro, rl = oracle.attend_sparse(q, k, v, n, gi, gc, tail)
    to, tl = (2e-3, 1e-4) if dtype == "bf16" else (1e-5, 1e-5)
    assert np.abs(host(out) - ro).max() <= to
    assert np.abs(host(lse) - rl).max() <= tl
    return gi, gc, s64


@pytest.mark.parametrize("hq,hkv,d,n,S,R,K", [
    (32, 8, 128, 131072, 4, 64, 4096),   # the Llama-3.1-8B per-step shape at 128K
    (32, 8, 128, 5000, 4, 64, 1000),     # ragged chunks
    (28, 4, 128, 20000, 0, 512, 1024),   # Qwen2-7B groups of seven
    (8, 8, 64, 2048, 4, 32, 256),        # MHA, head dim 64
    (32, 8, 128, 3000, 4, 64, 0),        # nothing selected: sinks and recent run only
    (32, 8, 128, 3000, 4, 64, 2932),     # every candidate
    (32, 8, 128, 3000, 4, 64, 5000),     # K past the candidate count
    (16, 2, 128, 777, 6, 9, 300),        # few kv heads, one short chunk each
    (16, 8, 128, 30000, 4, 64, 2000),    # groups of two
    (8, 8, 128, 60000, 2, 16, 3000),     # MHA at head dim 128: 32 keys per thread
    (32, 8, 64, 50000, 4, 64, 4096),     # head dim 64, groups of four
    # no threshold search (K = 0, K = every candidate) on full chunks: every
    # wave reads the lse of every query head
    (32, 8, 128, 131072, 4, 64, 0),
    (32, 8, 128, 70000, 4, 64, 70000),
    # groups of 3 (11 keys per thread), 5, 6 and 16 query heads
    (24, 8, 128, 40000, 4, 64, 3000),
    (20, 4, 64, 30000, 4, 64, 2000),
    (12, 2, 128, 9000, 4, 32, 700),
    (32, 2, 128, 20000, 4, 64, 1500),
])
def test_topk_step_matches_oracle(hq, hkv, d, n, S, R, K):
    q = _rand((hq, d), n + 1, "bf16")
    k = _rand((hkv, n + 2, d), n + 2, "bf16")
    v = _rand((hkv, n + 2, d), n + 3, "bf16")
    _check(q, k, v, n, S, R, K, "bf16", "one launch")


def test_topk_step_without_lse():
    """lse may be NULL; out is unchanged by leaving it out."""
    hq, hkv, d, n, S, R, K = 32, 8, 128, 9000, 4, 64, 700
    q = dev(_rand((hq, d), 31, "bf16"))
    k = dev(_rand((hkv, n, d), 32, "bf16"))
    v = dev(_rand((hkv, n, d), 33, "bf16"))
    ws = skv.Workspace.for_problem(skv.problem_for(q, k), n)
    score, idx, cnt, out, lse = _run_step(q, k, v, n, S, R, K, ws)
    out2 = torch.full_like(out, float("nan"))
    skv.skv_topk_step(q, k, v, n, S, R, K, score, idx, cnt, out2, None, ws)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)


def test_topk_step_exact_ties_keep_the_lowest_indices():
    """Identical keys give identical scores: the selection keeps the first K
    candidates, and every chunk's share of the ties is counted in order."""
    hq, hkv, d, n, S, R, K = 32, 8, 128, 40000, 4, 64, 7000
    q = _rand((hq, d), 5, "bf16")
    k = np.tile(_rand((hkv, 1, d), 6, "bf16"), (1, n, 1))
    v = _rand((hkv, n, d), 7, "bf16")
    gi, gc, _ = _check(q, k, v, n, S, R, K, "bf16", "ties")
    for h in range(hkv):
        assert np.array_equal(gi[h, :gc[h]], np.arange(S + K))


def test_topk_step_repeated_keys_across_chunks():
    """Keys drawn from 48 distinct rows: the scores take 48 values per kv head,
    each repeated in every chunk, so the threshold's bin holds runs of equal
    keys spread over all chunks (the path that resolves T in LDS)."""
    hq, hkv, d, n, S, R, K = 32, 8, 128, 24000, 4, 64, 3000
    rng = np.random.default_rng(21)
    base = _rand((hkv, 48, d), 22, "bf16")
    pick = rng.integers(0, 48, size=n)
    k = np.ascontiguousarray(base[:, pick, :])
    q = _rand((hq, d), 23, "bf16")
    v = _rand((hkv, n, d), 24, "bf16")
    _check(q, k, v, n, S, R, K, "bf16", "repeated keys")


@pytest.mark.parametrize("case", ["fp32", "too long"])
def test_topk_step_three_call_form(case):
    if case == "fp32":
        q, k, v = _rand((8, 64), 8, "f32"), _rand((8, 2048, 64), 9, "f32"), _rand((8, 2048, 64), 10, "f32")
        _check(q, k, v, 2048, 4, 32, 256, "f32", "fp32 caches")
    else:  # 8 kv heads x 300K keys: a chunk's logits no longer fit on chip
        n = 300000
        q = _rand((32, 128), 11, "bf16")
        k = _rand((8, n, 128), 12, "bf16")
        v = _rand((8, n, 128), 13, "bf16")
        _check(q, k, v, n, 4, 64, 4096, "bf16", "long cache")


def test_topk_step_llama_128k_needle():
    """The 128K needle workload: the planted key is kept in every kv head."""
    w = synth.llama_needle()
    gi, gc, _ = _check(w.q, w.k, w.v, w.n, w.n_sink, w.n_recent, w.k_top, "bf16", "128K needle")
    for h in range(w.n_kv_heads):
        assert w.extra["needle"] in set(gi[h, :gc[h]].tolist())
