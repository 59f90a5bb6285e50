"""The longest cache a call accepts, end to end on the GPU: rows of one kv head
are addressed with 32-bit byte offsets, so n + 16 rows (one masked tile past
the end) must span less than 4 GiB, i.e. n <= 16,777,199 for bf16 and
8,388,591 for fp32 at head dim 128.  At that n the oracle cannot run, so the
checks use closed forms that hold at any size.  With every key zero all logits
are equal and softmax is uniform:
  - dense step: out = mean of V over [0, n), lse = ln n;
  - sparse step: out = mean of V over the kept rows, lse = ln(#rows);
  - verify: query t sees [0, n - gamma + t], so out_t is the mean over those
    n - gamma + t + 1 rows and lse_t = ln(n - gamma + t + 1);
  - per-step score: every key gets G / n (G query heads, each uniform);
  - select on those equal scores keeps the lowest candidate indices.
V is built as a[j] + b[t] with a[j] = (7 j mod 11) - 5 and b[t] = (t mod 3) - 1
(small integers, exact in bf16), so every mean is exact in fp64 on the host.
One past the largest n is refused before anything is enqueued."""
import math

import numpy as np
import pytest
import torch

import sparse_top_kv_amd as skv
from gpu_util import banner, host, need_gpu

pytestmark = pytest.mark.gpu

D, HQ, HKV = 128, 4, 1
G = HQ // HKV


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()
    yield
    torch.cuda.empty_cache()


def max_n(elem_bytes):
    return (1 << 32) // (D * elem_bytes) - 17


def a_of(j):
    return (7 * np.asarray(j, np.int64)) % 11 - 5


def a_prefix_sum(m):
    """sum of a[j] for j < m: every run of 11 consecutive j sums to zero."""
    return int(a_of(np.arange(m % 11)).sum())


B = (np.arange(D) % 3 - 1).astype(np.float64)


def build_cache(cap, dtype):
    k = torch.zeros((HKV, cap, D), dtype=dtype, device="cuda")
    a = ((torch.arange(cap, device="cuda", dtype=torch.int64) * 7) % 11 - 5).to(dtype)
    b = torch.from_numpy(B.astype(np.float32)).to(device="cuda", dtype=dtype)
    v = (a[:, None] + b[None, :]).unsqueeze(0)
    del a
    return k, v


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_longest_cache_end_to_end(dtype):
    elem = 2 if dtype == torch.bfloat16 else 4
    n = max_n(elem)
    banner(f"max context {dtype} n={n}")
    k, v = build_cache(n + 1, dtype)  # room for the refused call's extra row
    q = torch.randn((HQ, D), device="cuda").to(dtype)
    p = skv.problem_for(q, k)
    ws = skv.Workspace.for_problem(p, n, 8)
    out = torch.full((HQ, D), float("nan"), device="cuda")
    lse = torch.full((HQ,), float("nan"), device="cuda")

    # one past the limit is refused on the host
    with pytest.raises(skv.SkvError):
        skv.skv_attend_dense(q, k, v, n + 1, out, lse, ws)

    # dense step: uniform softmax over all n rows
    skv.skv_attend_dense(q, k, v, n, out, lse, ws)
    torch.cuda.synchronize()
    want = a_prefix_sum(n) / n + B
    assert np.abs(host(out) - want[None, :]).max() <= 1e-5
    assert np.abs(host(lse) - math.log(n)).max() <= 2e-5 * math.log(n)

    # sparse step: every 4099th row below the tail, then the last 64 rows
    R = 64
    tail = n - R
    idx_np = np.arange(0, tail, 4099, dtype=np.int64)
    idx = torch.from_numpy(idx_np.astype(np.int32)).cuda()[None, :]
    cnt = torch.tensor([idx_np.size], dtype=torch.int32, device="cuda")
    out.fill_(float("nan"))
    skv.skv_attend_sparse(q, k, v, n, idx, cnt, tail, out, lse, ws)
    torch.cuda.synchronize()
    rows = idx_np.size + R
    s_rows = int(a_of(idx_np).sum()) + int(a_of(np.arange(tail, n)).sum())
    assert np.abs(host(out) - (s_rows / rows + B)[None, :]).max() <= 1e-5
    assert np.abs(host(lse) - math.log(rows)).max() <= 2e-5 * math.log(rows)

    # verify: causal limits over the longest cache (bf16 only: the matrix-core pass)
    if dtype == torch.bfloat16:
        gamma = 5
        qv = torch.randn((gamma, HQ, D), device="cuda").to(dtype)
        ov = torch.full((gamma, HQ, D), float("nan"), device="cuda")
        lv = torch.full((gamma, HQ), float("nan"), device="cuda")
        skv.skv_verify(qv, k, v, n, ov, lv, ws)
        torch.cuda.synchronize()
        o, l = host(ov), host(lv)
        for t in range(gamma):
            m = n - gamma + t + 1
            assert np.abs(o[t] - (a_prefix_sum(m) / m + B)[None, :]).max() <= 1e-5
            assert np.abs(l[t] - math.log(m)).max() <= 2e-5 * math.log(m)

    # per-step score: G / n everywhere; then select keeps the lowest candidates
    score = torch.full((HKV, n), float("nan"), device="cuda")
    skv.skv_score(q, k, n, score, ws)
    torch.cuda.synchronize()
    rel = float(((score - G / n).abs().max() / (G / n)).item())
    assert rel <= 1e-5
    S, K = 4, 1000
    sel_idx = torch.full((HKV, S + K), -7, dtype=torch.int32, device="cuda")
    sel_cnt = torch.zeros(HKV, dtype=torch.int32, device="cuda")
    # equal scores: ties go to the lowest index, whatever the last bits hold
    skv.skv_select(torch.full_like(score, G / n), n, S, R, K, sel_idx, sel_cnt, ws)
    torch.cuda.synchronize()
    assert host(sel_cnt).tolist() == [S + K]
    assert np.array_equal(host(sel_idx)[0], np.arange(S + K))
