"""skv_attend_sparse_noalloc, the gathered-rows decode call for callers that
cannot allocate (its scratch is a fixed per-GPU array inside the library),
against skv_attend_sparse with a caller workspace: two calls in a row, the
second with a smaller input, each bit-identical to the workspace call (same
plan and kernels) and within the bf16 attention bound of the oracle."""
import numpy as np
import pytest
import torch

import oracle
import sparse_top_kv_amd as skv
import synth
from gpu_util import banner, dev, host, need_gpu

pytestmark = pytest.mark.gpu


def _case(hq, hkv, d, n, tail, keep, seed):
    rng = np.random.default_rng(seed)
    q = synth.bf16_bits(rng.standard_normal((hq, d)).astype(np.float32))
    k = synth.bf16_bits(rng.standard_normal((hkv, n, d)).astype(np.float32))
    v = synth.bf16_bits(rng.standard_normal((hkv, n, d)).astype(np.float32))
    idx = np.full((hkv, keep), -1, np.int32)
    cnt = np.zeros(hkv, np.int32)
    for h in range(hkv):
        c = keep if h else 0  # head 0: only the tail
        idx[h, :c] = np.sort(rng.choice(tail, c, replace=False))
        cnt[h] = c
    return q, k, v, idx, cnt


def test_noalloc_matches_the_workspace_call_on_two_calls_in_a_row():
    need_gpu()
    # Llama-3.1-8B shape at 32K with 30 % kept, then a smaller Qwen2-7B-shaped call
    cases = [(32, 8, 128, 32768, 32768 - 64, 9766, 1), (28, 4, 128, 3000, 2900, 700, 2)]
    for hq, hkv, d, n, tail, keep, seed in cases:
        banner(f"noalloc hq={hq} hkv={hkv} d={d} n={n} keep={keep}")
        q, k, v, idx, cnt = _case(hq, hkv, d, n, tail, keep, seed)
        qt, kt, vt, it, ct = dev(q), dev(k), dev(v), dev(idx), dev(cnt)
        ws = skv.Workspace.for_problem(skv.problem_for(qt, kt), n)
        o_ws = torch.full((hq, d), float("nan"), device="cuda")
        l_ws = torch.full((hq,), float("nan"), device="cuda")
        o_na = torch.full((hq, d), float("nan"), device="cuda")
        l_na = torch.full((hq,), float("nan"), device="cuda")
        skv.skv_attend_sparse(qt, kt, vt, n, it, ct, tail, o_ws, l_ws, ws)
        skv.skv_attend_sparse_noalloc(qt, kt, vt, n, it, ct, tail, o_na, l_na)
        torch.cuda.synchronize()
        assert torch.equal(o_ws, o_na) and torch.equal(l_ws, l_na)
        ref_o, ref_l = oracle.attend_sparse(q, k, v, n, idx, cnt, tail)
        assert np.abs(host(o_na) - ref_o).max() <= 2e-3
        assert np.abs(host(l_na) - ref_l).max() <= 1e-4
