"""Pins for the fp64 oracle: each check ties it to something other than itself
(closed forms, invariants, brute force, or an independent library routine), so
that a dropped term, a wrong sign or index, or a transposed operand fails here.

No GPU is needed; these run on the CPU in a few seconds.
"""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")


def _rand(shape, seed, dtype="f32", sd=1.0):
    x = np.random.default_rng(seed).standard_normal(shape).astype(np.float32) * np.float32(sd)
    return synth.bf16_bits(x) if dtype == "bf16" else x


def _f64(a):
    return synth.bf16_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)


def _sdpa(q, k, v, n, scale, causal_rows=None):
    """torch SDPA on CPU in float64 with GQA expanded by repeat_interleave.

    q [R][Hq][d] (R query positions), k/v [Hkv][cap][d].  causal_rows gives
    each query row's last visible key position (None: all n keys)."""
    qt = torch.from_numpy(_f64(q)).permute(1, 0, 2)  # [Hq][R][d]
    kt = torch.from_numpy(_f64(k)[:, :n])
    vt = torch.from_numpy(_f64(v)[:, :n])
    G = q.shape[1] // k.shape[0]
    kt = kt.repeat_interleave(G, dim=0)
    vt = vt.repeat_interleave(G, dim=0)
    mask = None
    if causal_rows is not None:
        pos = torch.arange(n)[None, :]
        last = torch.as_tensor(causal_rows)[:, None]
        mask = (pos <= last)[None]  # [1][R][n]
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    return out.permute(1, 0, 2).numpy()  # [R][Hq][d]


# ----------------------------------------------------------------------------
# attention
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("hq,hkv,d", [(8, 8, 64), (8, 2, 64), (7, 1, 128), (12, 4, 128)])
def test_dense_matches_torch_sdpa_fp64(dtype, hq, hkv, d):
    n = 301
    q = _rand((hq, d), 1, dtype)
    k = _rand((hkv, n + 7, d), 2, dtype)
    v = _rand((hkv, n + 7, d), 3, dtype)
    out, lse = oracle.attend_dense(q, k, v, n)
    scale = float(np.float32(1 / math.sqrt(d)))
    ref = _sdpa(q[None], k, v, n, scale)[0]
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    # lse against a library log-sum-exp over the same logits
    G = hq // hkv
    lg = np.einsum("gd,gjd->gj", _f64(q), np.repeat(_f64(k)[:, :n], G, axis=0)) * scale
    np.testing.assert_allclose(lse, torch.logsumexp(torch.from_numpy(lg), dim=1).numpy(), atol=1e-12)


def test_single_key_returns_its_value():
    q = _rand((4, 64), 5)
    k = _rand((4, 3, 64), 6)
    v = _rand((4, 3, 64), 7)
    out, lse = oracle.attend_dense(q, k, v, 1)
    np.testing.assert_array_equal(out, v[:, 0].astype(np.float64))
    l0 = (q.astype(np.float64) * k[:, 0].astype(np.float64)).sum(1) * float(np.float32(1 / 8))
    np.testing.assert_allclose(lse, l0, atol=1e-12)


def test_two_keys_sigmoid_closed_form():
    q = _rand((2, 64), 8)
    k = _rand((2, 2, 64), 9)
    v = _rand((2, 2, 64), 10)
    sc = float(np.float32(0.3))  # the scale argument is an fp32 value
    out, _ = oracle.attend_dense(q, k, v, 2, scale=sc)
    for h in range(2):
        l0 = sc * float(np.dot(q[h].astype(np.float64), k[h, 0].astype(np.float64)))
        l1 = sc * float(np.dot(q[h].astype(np.float64), k[h, 1].astype(np.float64)))
        s0 = 1 / (1 + math.exp(l1 - l0))
        s1 = 1 / (1 + math.exp(l0 - l1))
        v64 = v[h].astype(np.float64)  # keep the check in fp64 (a Python float times fp32 stays fp32)
        np.testing.assert_allclose(out[h], s0 * v64[0] + s1 * v64[1], atol=1e-12)


def test_uniform_keys_give_mean_of_values():
    hq, hkv, d, n = 8, 2, 64, 97
    q = _rand((hq, d), 11)
    k = np.broadcast_to(_rand((hkv, 1, d), 12), (hkv, n, d)).copy()
    v = _rand((hkv, n, d), 13)
    out, _ = oracle.attend_dense(q, k, v, n)
    G = hq // hkv
    np.testing.assert_allclose(out, np.repeat(v.astype(np.float64).mean(1), G, axis=0), atol=1e-12)
    # sparse over a subset: mean over exactly that subset + tail
    idx = np.array([[0, 5, 9, 40, -1], [3, 4, 50, 60, 61]], np.int32)
    cnt = np.array([4, 5], np.int32)
    out_s, _ = oracle.attend_sparse(q, k, v, n, idx, cnt, tail_start=90)
    for h in range(hkv):
        rows = list(idx[h, :cnt[h]]) + list(range(90, n))
        for g in range(h * G, (h + 1) * G):
            np.testing.assert_allclose(out_s[g], v[h, rows].astype(np.float64).mean(0), atol=1e-12)


def test_sparse_with_all_candidates_is_bit_identical_to_dense():
    w = synth.tiny_mha(n=512)
    n = w.n
    s64, s32 = oracle.score(w.q[None], w.k, n)
    ncand = n - w.n_sink - w.n_recent
    idx, cnt = oracle.select(s32, w.n_sink, w.n_recent, ncand)
    assert (cnt == n - w.n_recent).all()
    out_s, lse_s = oracle.attend_sparse(w.q, w.k, w.v, n, idx, cnt, n - w.n_recent)
    out_d, lse_d = oracle.attend_dense(w.q, w.k, w.v, n)
    np.testing.assert_array_equal(out_s, out_d)
    np.testing.assert_array_equal(lse_s, lse_d)


def test_empty_set_is_merge_identity():
    q = _rand((2, 64), 14)
    k = _rand((2, 8, 64), 15)
    idx = np.zeros((2, 1), np.int32)
    cnt = np.zeros(2, np.int32)
    out, lse = oracle.attend_sparse(q, k, k, 8, idx, cnt, tail_start=8)
    assert (out == 0).all() and np.isneginf(lse).all()


def test_lse_merge_of_random_partitions_equals_whole():
    hq, hkv, d, n = 8, 2, 128, 400
    q = _rand((hq, d), 16, "bf16")
    k = _rand((hkv, n, d), 17, "bf16")
    v = _rand((hkv, n, d), 18, "bf16")
    out, lse = oracle.attend_dense(q, k, v, n)
    rng = np.random.default_rng(19)
    perm = rng.permutation(n)
    cuts = np.sort(rng.choice(np.arange(1, n), 5, replace=False))
    parts = np.split(perm, cuts)
    outs, lses = [], []
    for part in parts:
        srt = np.sort(part).astype(np.int32)
        idx = np.tile(srt, (hkv, 1))
        o, l = oracle.attend_sparse(q, k, v, n, idx, np.full(hkv, len(srt), np.int32), tail_start=n)
        outs.append(o)
        lses.append(l)
    L = np.stack(lses)               # [parts][Hq]
    M = L.max(0)
    wts = np.exp(L - M)
    merged = (wts[..., None] * np.stack(outs)).sum(0) / wts.sum(0)[..., None]
    np.testing.assert_allclose(merged, out, atol=1e-13)
    np.testing.assert_allclose(M + np.log(wts.sum(0)), lse, atol=1e-13)


@pytest.mark.parametrize("hq,hkv", [(4, 4), (28, 4)])
def test_verify_matches_causal_sdpa_and_dense_prefixes(hq, hkv):
    d, n, gamma = 128, 257, 5
    q = _rand((gamma, hq, d), 20, "bf16")
    k = _rand((hkv, n, d), 21, "bf16")
    v = _rand((hkv, n, d), 22, "bf16")
    out, lse = oracle.verify(q, k, v, n)
    last = [n - gamma + t for t in range(gamma)]
    ref = _sdpa(q, k, v, n, float(np.float32(1 / math.sqrt(d))), causal_rows=last)
    np.testing.assert_allclose(out, ref, atol=1e-12)
    for t in range(gamma):
        od, ld = oracle.attend_dense(np.ascontiguousarray(q[t]), k, v, n - gamma + t + 1)
        np.testing.assert_array_equal(out[t], od)
        np.testing.assert_array_equal(lse[t], ld)


# ----------------------------------------------------------------------------
# score
# ----------------------------------------------------------------------------
def test_score_single_query_mha_is_the_softmax_row():
    hq, d, n = 4, 64, 333
    q = _rand((hq, d), 23)
    k = _rand((hq, n, d), 24)
    s64, s32 = oracle.score(q[None], k, n)
    sc = float(np.float32(1 / 8))
    lg = torch.from_numpy(np.einsum("hd,hjd->hj", q.astype(np.float64), k.astype(np.float64)) * sc)
    np.testing.assert_allclose(s64, torch.softmax(lg, dim=1).numpy(), atol=1e-15)
    np.testing.assert_array_equal(s32, s64.astype(np.float32))


@pytest.mark.parametrize("W,hq,hkv", [(1, 8, 2), (6, 8, 2), (5, 7, 1), (32, 4, 4)])
def test_score_window_matches_library_softmax(W, hq, hkv):
    d, n = 64, 150
    q = _rand((W, hq, d), 25, "bf16")
    k = _rand((hkv, n, d), 26, "bf16")
    s64, _ = oracle.score(q, k, n)
    G = hq // hkv
    sc = float(np.float32(1 / 8))
    qt = torch.from_numpy(_f64(q))                      # [W][Hq][d]
    kt = torch.from_numpy(_f64(k)).repeat_interleave(G, 0)  # [Hq][n][d]
    lg = torch.einsum("whd,hjd->whj", qt, kt) * sc
    pos = torch.arange(n)
    visible = pos[None, :] <= (n - W + torch.arange(W))[:, None]  # [W][n]
    lg = lg.masked_fill(~visible[:, None, :], float("-inf"))
    p = torch.softmax(lg, dim=2)                         # [W][Hq][n]
    ref = p.sum(0).reshape(hkv, G, n).sum(1) / W
    np.testing.assert_allclose(s64, ref.numpy(), atol=1e-14)
    # invariant: each kv head's scores sum to its group size
    np.testing.assert_allclose(s64.sum(1), G, atol=1e-12)


def test_score_uniform_keys_closed_form():
    W, hq, hkv, d, n = 8, 6, 2, 64, 40
    G = hq // hkv
    q = _rand((W, hq, d), 27)
    k = np.broadcast_to(_rand((hkv, 1, d), 28), (hkv, n, d)).copy()
    s64, _ = oracle.score(q, k, n)
    p_i = n - W + np.arange(W)  # positions of the window rows
    expect = np.array([(G / W) * sum(1.0 / (p + 1) for p in p_i if p >= j) for j in range(n)])
    for h in range(hkv):
        np.testing.assert_allclose(s64[h], expect, atol=1e-14)


# ----------------------------------------------------------------------------
# select
# ----------------------------------------------------------------------------
def _brute_force_topk(s, cand, K):
    """The unique K-subset T of cand with every member ranked before every
    non-member under (score desc, index asc), found by exhaustive search."""
    found = []
    for T in itertools.combinations(cand, K):
        Ts = set(T)
        rest = [j for j in cand if j not in Ts]
        if all((s[i] > s[j]) or (s[i] == s[j] and i < j) for i in T for j in rest):
            found.append(T)
    assert len(found) == 1
    return list(found[0])


def test_select_brute_force_tiny_with_ties():
    rng = np.random.default_rng(30)
    for trial in range(25):
        n = int(rng.integers(1, 13))
        vals = np.array([0.0, -0.0, 0.25, 0.5, 1.0, 3.0], np.float32)
        s = rng.choice(vals, size=(1, n)).astype(np.float32)
        for S in range(0, 3):
            for R in range(0, 3):
                tail = max(n - R, 0)
                cand = list(range(S, n - R)) if S < n - R else []
                for K in range(0, len(cand) + 2):
                    idx, cnt = oracle.select(s, S, R, K, idx_stride=16)
                    kk = min(K, len(cand))
                    expect = sorted(list(range(min(S, tail))) + _brute_force_topk(s[0], cand, kk))
                    assert cnt[0] == len(expect)
                    assert list(idx[0, :cnt[0]]) == expect


def test_select_matches_numpy_stable_argsort():
    rng = np.random.default_rng(31)
    hkv, n = 4, 5000
    s = rng.exponential(1.0, (hkv, n)).astype(np.float32)
    s[:, ::7] = s[:, 3:4]  # many exact ties
    S, R = 4, 64
    ks = np.array([0, 17, 1000, 9000], np.int32)
    idx, cnt = oracle.select(s, S, R, ks)
    for h in range(hkv):
        c = np.arange(S, n - R)
        order = c[np.argsort(-s[h, c], kind="stable")]
        kk = min(int(ks[h]), len(c))
        expect = np.sort(np.concatenate([np.arange(S), order[:kk]]))
        assert cnt[h] == S + kk
        np.testing.assert_array_equal(idx[h, :cnt[h]], expect)


def test_select_uniform_scores_take_lowest_indices():
    n, S, R, K = 1000, 4, 32, 100
    s = np.full((3, n), 0.001, np.float32)
    idx, cnt = oracle.select(s, S, R, K)
    for h in range(3):
        np.testing.assert_array_equal(idx[h, :cnt[h]], np.arange(S + K))


def test_select_window_overlap_edges():
    s = np.arange(10, dtype=np.float32)[None]
    idx, cnt = oracle.select(s, 4, 8, 5, idx_stride=8)   # recent [2,10) swallows sinks 2,3
    assert cnt[0] == 2 and list(idx[0, :2]) == [0, 1]
    idx, cnt = oracle.select(s, 4, 20, 5, idx_stride=8)  # recent window is everything
    assert cnt[0] == 0


def test_planted_heavy_hitters_are_selected():
    w = synth.tiny_mha()
    _, s32 = oracle.score(w.q[None], w.k, w.n)
    idx, cnt = oracle.select(s32, w.n_sink, w.n_recent, w.k_top)
    for h in range(w.n_kv_heads):
        assert set(w.extra["heavy"].tolist()) <= set(idx[h, :cnt[h]].tolist())


# ----------------------------------------------------------------------------
# budgets
# ----------------------------------------------------------------------------
def test_budgets_sparsemm_closed_forms():
    N, B, w, rho = 1024, 1024 * 256, 32, 0.1
    s = np.ones(N)
    k, b = oracle.budgets(s, B, w, rho, n_cand=32768)
    np.testing.assert_allclose(b, 256.0, atol=1e-9)     # equal scores: every head gets B/N
    r = 22.4
    b_remain = 206438.4
    assert (k == math.floor(r + b_remain / N)).all()
    s = synth.sparsemm_heads(head_subset=[]).extra["head_scores"]
    k, b = oracle.budgets(s, B, w, rho, n_cand=32768 - 32)
    np.testing.assert_allclose(b.sum(), B, rtol=1e-12)  # the three parts add up to B
    np.testing.assert_array_equal(k, np.floor(r + b_remain * s / s.sum()).astype(np.int32))
    assert k.min() >= 22 and k.max() < 32768


def test_budgets_clamp_to_candidates():
    s = np.array([1.0, 1000.0])
    k, _ = oracle.budgets(s, 2 * 5000, 0, 0.0, n_cand=3000)
    assert k[1] == 3000 and k[0] == math.floor(10000 / 1001)  # no redistribution of the clamped excess
