"""GPU parity of the SpecVLM selection (skv_select_topp) against the oracle:
index sets and counts bit-exact on identical fp32 scores, including scores
whose masses span the whole fp32 range (Stage I compares exact sums)."""
import numpy as np
import pytest
import torch

import oracle
import sparse_top_kv_amd as skv
from gpu_util import banner, dev, host, need_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _attn_like(rows, n, seed, heavy=0.01, zeros=0.0, quant=None):
    """Heavy-tailed non-negative scores: a flat floor plus planted large entries."""
    rng = np.random.default_rng(seed)
    s = rng.exponential(1e-4, (rows, n))
    nh = max(1, int(heavy * n))
    for h in range(rows):
        s[h, rng.choice(n, nh, replace=False)] += rng.exponential(0.02, nh)
    if zeros:
        s[rng.random((rows, n)) < zeros] = 0.0
    if quant:
        s = np.round(s / quant) * quant  # many exact ties
    return s.astype(np.float32)


def _run(s, n, S, R, lam, prune, pooled, mode, ws=None):
    rows = s.shape[0]
    tail = max(n - R, 0)
    ncand = max(n - R - S, 0)
    stride = max(1, min(S, tail) + ncand)
    st = dev(np.ascontiguousarray(s))
    idx = torch.full((rows, stride), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((rows,), -7, dtype=torch.int32, device="cuda")
    cr = torch.full((rows,), -7, dtype=torch.int32, device="cuda")
    if ws is None:
        ws = skv.Workspace.for_problem(skv.problem(rows, rows, 128, skv.SKV_BF16, 128, 128), n)
    skv.skv_select_topp(st, n, S, R, lam, prune, idx, cnt, ws, count_r=cr, pooled=pooled,
                        fill_mode=mode)
    torch.cuda.synchronize()
    o_idx, o_cnt, o_cr = oracle.select_topp(s[:, :n], S, R, lam, prune, pooled=pooled,
                                            fill_mode=mode, idx_stride=stride)
    gi, gc, gr = host(idx), host(cnt), host(cr)
    assert np.array_equal(gc, o_cnt) and np.array_equal(gr, o_cr)
    for h in range(rows):
        assert np.array_equal(gi[h, :gc[h]], o_idx[h, :o_cnt[h]])
    return gi, gc, gr


@pytest.mark.parametrize("pooled", [False, True])
@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("lam,prune", [(0.4, 0.9), (0.5, 0.9), (0.0, 0.5), (1.0, 0.0), (0.9, 1.0)])
def test_topp_matches_oracle(pooled, mode, lam, prune):
    banner(f"topp pooled={pooled} mode={mode} lam={lam} prune={prune}")
    s = _attn_like(4, 5000, 1, zeros=0.05)
    _run(s, 5000, 2, 64, lam, prune, pooled, mode)


@pytest.mark.parametrize("rows,n,S,R", [(1, 1, 0, 0), (3, 70, 4, 8), (8, 1024, 0, 0), (2, 1025, 1, 1),
                                        (5, 40000, 4, 512), (2, 10, 6, 6), (1, 300, 400, 0),
                                        (2, 32768 + 68, 4, 64), (2, 32769 + 68, 4, 64)])
def test_topp_shapes_and_ragged_tails(rows, n, S, R):
    banner(f"topp shape rows={rows} n={n} S={S} R={R}")
    s = _attn_like(rows, n, 2)
    for pooled in (False, True):
        _run(s, n, S, R, 0.5, 0.9, pooled, 0)


def test_topp_ties_zeros_and_tiny_scores():
    banner("topp ties / zeros / subnormal scores")
    s = _attn_like(3, 3000, 3, zeros=0.3, quant=1e-3)  # heavy ties at the crossing value
    for lam in (0.3, 0.5, 0.77):
        _run(s, 3000, 0, 0, lam, 0.8, False, 0)
        _run(s, 3000, 0, 0, lam, 0.8, True, 1)
    _run(np.zeros((2, 500), np.float32), 500, 4, 16, 0.5, 0.5, False, 0)  # no mass
    tiny = (_attn_like(2, 800, 4) * np.float32(1e-38)).astype(np.float32)  # subnormal range
    _run(tiny, 800, 0, 0, 0.5, 0.9, False, 0)
    big = (_attn_like(2, 800, 5) * np.float32(1e30)).astype(np.float32)
    _run(big, 800, 0, 0, 0.5, 0.9, True, 0)
    one = np.ones((2, 777), np.float32)  # every candidate ties
    _run(one, 777, 0, 0, 0.5, 0.9, False, 0)


def test_topp_many_rows_pooled_and_repeatable():
    banner("topp 64 rows pooled, twice")
    s = _attn_like(64, 8192, 6)
    a = _run(s, 8192, 0, 32, 0.5, 0.9, True, 0)
    b = _run(s, 8192, 0, 32, 0.5, 0.9, True, 0)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))


def _wide(rng, shape, zeros=0.1):
    """Binary exponents over about 2^-149 .. 2^20 in one row (subnormals included)."""
    e = rng.integers(-150, 21, shape).astype(np.float64)
    x = rng.random(shape) * np.exp2(e)
    x[rng.random(shape) < zeros] = 0.0
    return x.astype(np.float32)


@pytest.mark.parametrize("n", [3000, 40000])
def test_topp_exact_masses_over_the_fp32_range(n):
    """Register-resident rows (3000) and re-read rows (40000 candidates): the
    crossing may sit in any exponent bin, and lambda = 1 must keep every
    positive score, subnormals included."""
    banner(f"topp wide dynamic range n={n}")
    rng = np.random.default_rng(n)
    s = _wide(rng, (3, n))
    for lam in (1.0, 0.5, 0.37, 1e-300, float(np.nextafter(0.5, 1.0))):
        for pooled in (False, True):
            gi, gc, gr = _run(s, n, 2, 16, lam, 0.9, pooled, 0)
    gi, gc, gr = _run(s, n, 0, 0, 1.0, 1.0, False, 0)
    for h in range(3):
        assert np.array_equal(gi[h, :gc[h]], np.flatnonzero(s[h] > 0))


def test_topp_threshold_a_tiny_mass_past_a_prefix():
    banner("topp threshold 2^-91 past a prefix")
    s = np.zeros((2, 1000), np.float32)
    s[:, 10] = 1.0
    s[:, 500] = 1.0
    s[0, 700] = 2.0 ** -90   # half the total is 1 + 2^-91: both ones are needed
    _, _, gr = _run(s, 1000, 0, 0, 0.5, 1.0, False, 0)
    assert gr.tolist() == [2, 1]
