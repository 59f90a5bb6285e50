"""GPU parity of the compaction call (skv_gather) and of the dense step over a
compacted cache.

The copy is checked byte for byte against numpy fancy indexing of the same
cache (its definition: row i of head h is idx[h][i] for i < count[h], then the
tail).  The dense step over the compacted cache is checked against the oracle's
sparse attention over the same kept set."""
import numpy as np
import pytest
import torch

import oracle
import sparse_top_kv_amd as skv
import synth
from gpu_util import banner, dev, host, need_gpu

pytestmark = pytest.mark.gpu

TOL = {"f32": (1e-5, 1e-5), "bf16": (2e-3, 1e-4)}


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _rand(shape, seed, dtype):
    x = np.random.default_rng(seed).standard_normal(shape).astype(np.float32)
    return synth.bf16_bits(x) if dtype == "bf16" else x


def _sets(hkv, tail_start, stride, seed, counts):
    rng = np.random.default_rng(seed)
    idx = np.full((hkv, stride), -1, np.int32)
    for h in range(hkv):
        c = min(int(counts[h]), tail_start, stride)
        idx[h, :c] = np.sort(rng.choice(tail_start, size=c, replace=False))
    return idx


def _expected_rows(x, idx, cnt, tail_start, n, stride):
    """Numpy definition of the compacted rows of one head-major cache."""
    rows = []
    for h in range(x.shape[0]):
        c = max(0, min(int(cnt[h]), stride))
        rows.append(np.concatenate([x[h, idx[h, :c]], x[h, tail_start:n]]))
    return rows


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("hkv,d,n,tail,stride,pad", [
    (8, 128, 5000, 4936, 1500, 0),     # several workgroups per head, ragged last one
    (3, 64, 777, 700, 700, 32),        # padded output rows, full-width index list
    (2, 128, 100, 100, 40, 0),         # no tail
    (4, 64, 300, 0, 0, 0),             # tail only
])
def test_gather_is_exact_numpy_indexing(dtype, hkv, d, n, tail, stride, pad):
    banner(f"gather {dtype} hkv={hkv} d={d} n={n} tail={tail} stride={stride} pad={pad}")
    k = _rand((hkv, n + 5, d), 1, dtype)
    v = _rand((hkv, n + 5, d), 2, dtype)
    rng = np.random.default_rng(3)
    cnt = rng.integers(0, min(stride, tail) + 1, size=hkv).astype(np.int32)
    if hkv > 2 and stride > 0:
        cnt[0] = 0                       # empty indexed part
        cnt[1] = min(stride, tail)       # full index list
    idx = _sets(hkv, tail, stride, 4, cnt)
    if hkv > 3 and stride > 0:
        cnt[2] = stride + 7              # above idx_stride: clamped to idx_stride
        idx[2] = np.sort(rng.choice(tail, size=stride, replace=False))
    rows_max = min(stride, tail) + (n - tail)
    kt, vt = dev(k), dev(v)
    sentinel = 0x7F7F if dtype == "bf16" else 1.0e30
    shape = (hkv, rows_max + 3, d + pad)
    if dtype == "bf16":
        ko = torch.full(shape, 0, dtype=torch.int16, device="cuda").fill_(sentinel).view(torch.bfloat16)
        vo = ko.clone()
    else:
        ko = torch.full(shape, sentinel, device="cuda")
        vo = ko.clone()
    ko_view, vo_view = ko[:, :, :d], vo[:, :, :d]
    rows = torch.full((hkv,), -1, dtype=torch.int32, device="cuda")
    skv.skv_gather(kt, vt, n, dev(idx), dev(cnt), tail, ko_view, vo_view, rows)
    torch.cuda.synchronize()
    as_bits = (lambda t: host(t.view(torch.int16)).view(np.uint16)) if dtype == "bf16" else host
    gk, gv = as_bits(ko), as_bits(vo)
    ek, ev = _expected_rows(k, idx, cnt, tail, n, stride), _expected_rows(v, idx, cnt, tail, n, stride)
    for h in range(hkv):
        r = ek[h].shape[0]
        assert host(rows)[h] == r
        assert np.array_equal(gk[h, :r, :d], ek[h]) and np.array_equal(gv[h, :r, :d], ev[h])
        # rows past the head's count, and the padding of every row, are untouched
        sent = np.array(sentinel, dtype=gk.dtype)
        assert np.all(gk[h, r:] == sent) and np.all(gv[h, r:] == sent)
        if pad:
            assert np.all(gk[h, :, d:] == sent) and np.all(gv[h, :, d:] == sent)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("hq,hkv,d,n,tail,stride", [(32, 8, 128, 6000, 5936, 1800), (28, 4, 64, 900, 880, 300),
                                                    (16, 2, 128, 70, 64, 64)])
def test_dense_step_over_compacted_cache_matches_oracle(dtype, hq, hkv, d, n, tail, stride):
    banner(f"gather + dense {dtype} hq={hq} hkv={hkv} d={d} n={n}")
    q = _rand((hq, d), 5, dtype)
    k = _rand((hkv, n, d), 6, dtype)
    v = _rand((hkv, n, d), 7, dtype)
    cnt = np.full(hkv, min(stride, tail), np.int32)  # one kept count for every head
    idx = _sets(hkv, tail, stride, 8, cnt)
    ref_o, ref_l = oracle.attend_sparse(q, k, v, n, idx, cnt, tail)
    rows = int(cnt[0]) + n - tail
    qt, kt, vt = dev(q), dev(k), dev(v)
    kc = torch.empty((hkv, rows, d), dtype=kt.dtype, device="cuda")
    vc = torch.empty_like(kc)
    skv.skv_gather(kt, vt, n, dev(idx), dev(cnt), tail, kc, vc)
    out = torch.full((hq, d), float("nan"), device="cuda")
    lse = torch.full((hq,), float("nan"), device="cuda")
    ws = skv.Workspace.for_problem(skv.problem_for(qt, kc), rows)
    skv.skv_attend_dense(qt, kc, vc, rows, out, lse, ws)
    torch.cuda.synchronize()
    to, tl = TOL[dtype]
    assert np.abs(host(out) - ref_o).max() <= to
    assert np.abs(host(lse) - ref_l).max() <= tl


def test_llama_32k_compacted_step_matches_in_place_sparse_step():
    """Full-size kept set (4 sinks, the highest 30 % less sinks and recent run,
    64 recent entries) of the Llama-3.1-8B 32K workload: the dense step over the
    compacted cache and the in-place sparse step both match the oracle."""
    banner("llama 32K compaction: generate")
    w = synth.llama_obs()
    n, S, R, K, H, Hkv, d = w.n, w.n_sink, w.n_recent, w.k_top, w.n_q_heads, w.n_kv_heads, w.head_dim
    rng = np.random.default_rng(9)
    idx = np.zeros((Hkv, S + K), np.int32)
    for h in range(Hkv):
        kept = np.sort(rng.choice(np.arange(S, n - R), size=K, replace=False))
        idx[h] = np.concatenate([np.arange(S), kept])
    cnt = np.full(Hkv, S + K, np.int32)
    banner("llama 32K compaction: GPU gather + dense, sparse in place")
    q, kt, vt = dev(w.q), dev(w.k), dev(w.v)
    rows = S + K + R
    kc = torch.empty((Hkv, rows, d), dtype=torch.bfloat16, device="cuda")
    vc = torch.empty_like(kc)
    it, ct = dev(idx), dev(cnt)
    skv.skv_gather(kt, vt, n, it, ct, n - R, kc, vc)
    ws = skv.Workspace.for_problem(skv.problem_for(q, kt), n)
    out_c, lse_c = torch.empty((H, d), device="cuda"), torch.empty(H, device="cuda")
    out_s, lse_s = torch.empty((H, d), device="cuda"), torch.empty(H, device="cuda")
    skv.skv_attend_dense(q, kc, vc, rows, out_c, lse_c, ws)
    skv.skv_attend_sparse(q, kt, vt, n, it, ct, n - R, out_s, lse_s, ws)
    torch.cuda.synchronize()
    # sampled rows of the compacted cache, byte for byte
    kb = host(kc.view(torch.int16)).view(np.uint16)
    for h in range(Hkv):
        sample = rng.choice(rows, size=256, replace=False)
        src = np.where(sample < S + K, idx[h, np.minimum(sample, S + K - 1)], n - R + (sample - S - K))
        assert np.array_equal(kb[h, sample], w.k[h, src])
    banner("llama 32K compaction: oracle")
    ro, rl = oracle.attend_sparse(w.q, w.k, w.v, n, idx, cnt, n - R)
    to, tl = TOL["bf16"]
    for o, l in ((out_c, lse_c), (out_s, lse_s)):
        assert np.abs(host(o) - ro).max() <= to and np.abs(host(l) - rl).max() <= tl
