"""Every call of the library inside a captured HIP graph: replays, with eager
work and synchronisations between them, give bit-identical results to the
eager calls (all kernels are deterministic and nothing in a call uses a
memset node)."""
import numpy as np
import pytest
import torch

import sparse_top_kv_amd as skv
import synth
from gpu_util import banner, dev, host, need_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _rand(shape, seed):
    return dev(synth.bf16_bits(np.random.default_rng(seed).standard_normal(shape).astype(np.float32)))


def _replay_matches(run, outs, replays=3):
    """run() enqueues the calls writing `outs`; eager result, then graph replays.
    Outputs are reset to a sentinel before every run, so entries a call leaves
    untouched (index rows past a head's count) compare equal too."""
    def reset():
        for o in outs:
            o.fill_(float("nan") if o.dtype.is_floating_point else -7)

    reset()
    run()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        run()  # warm the side stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run()
    for r in range(replays):
        reset()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, ref):  # bitwise (NaN sentinels compare equal)
            assert torch.equal(o.view(torch.uint8), e.view(torch.uint8)), f"replay {r}"
        run()  # eager work between replays
        torch.cuda.synchronize()


def test_per_step_topk_pipeline_in_a_graph():
    banner("graph: per-step score -> block select -> sparse attend; dense; gather")
    hq, hkv, d, n, S, R, K = 32, 8, 128, 20000, 4, 64, 2000
    q, k, v = _rand((hq, d), 1), _rand((hkv, n, d), 2), _rand((hkv, n, d), 3)
    ws = skv.Workspace.for_problem(skv.problem_for(q, k), n)
    score = torch.empty((hkv, n), device="cuda")
    idx = torch.empty((hkv, S + K), dtype=torch.int32, device="cuda")
    cnt = torch.empty(hkv, dtype=torch.int32, device="cuda")
    out = torch.empty((hq, d), device="cuda")
    lse = torch.empty(hq, device="cuda")
    outd = torch.empty((hq, d), device="cuda")
    lsed = torch.empty(hq, device="cuda")
    kc = torch.empty((hkv, S + K + R, d), dtype=torch.bfloat16, device="cuda")
    vc = torch.empty_like(kc)

    def run():
        skv.skv_score(q, k, n, score, ws)
        skv.skv_select(score, n, S, R, K, idx, cnt, ws)
        skv.skv_attend_sparse(q, k, v, n, idx, cnt, n - R, out, lse, ws)
        skv.skv_attend_dense(q, k, v, 3000, outd, lsed, ws)  # a small (narrow) dense call
        skv.skv_gather(k, v, n, idx, cnt, n - R, kc, vc)

    _replay_matches(run, [score, idx, cnt, out, lse, outd, lsed, kc, vc])


def test_window_score_verify_and_specvlm_select_in_a_graph():
    banner("graph: window score, multi-pass verify, top-P select")
    hq, hkv, d, n, W, gamma = 28, 4, 128, 6000, 64, 13
    qo, k, v = _rand((W, hq, d), 4), _rand((hkv, n, d), 5), _rand((hkv, n, d), 6)
    qv = _rand((gamma, hq, d), 7)
    ws = skv.Workspace.for_problem(skv.problem_for(qo, k), n, W)
    score = torch.empty((hkv, n), device="cuda")
    idx = torch.empty((hkv, n), dtype=torch.int32, device="cuda")
    cnt = torch.empty(hkv, dtype=torch.int32, device="cuda")
    cr = torch.empty(hkv, dtype=torch.int32, device="cuda")
    ov = torch.empty((gamma, hq, d), device="cuda")
    lv = torch.empty((gamma, hq), device="cuda")

    def run():
        skv.skv_score(qo, k, n, score, ws)
        skv.skv_select_topp(score, n, 0, 512, 0.5, 0.9, idx, cnt, ws, count_r=cr, pooled=True)
        skv.skv_verify(qv, k, v, n, ov, lv, ws)  # 91 rows per kv head: two passes

    _replay_matches(run, [score, idx, cnt, cr, ov, lv])


def test_many_head_work_list_in_a_graph():
    banner("graph: 600 kv heads, ragged counts (work-list mode)")
    hq = hkv = 600
    d, n, tail = 128, 3000, 2968
    rng = np.random.default_rng(8)
    counts = np.minimum(rng.exponential(60, hkv).astype(np.int64), tail)
    counts[:4] = tail
    idx = np.full((hkv, int(counts.max())), -1, np.int32)
    for h in range(hkv):
        idx[h, :counts[h]] = np.sort(rng.choice(tail, counts[h], replace=False))
    q, k, v = _rand((hq, d), 9), _rand((hkv, n, d), 10), _rand((hkv, n, d), 11)
    it, ct = dev(idx), dev(counts.astype(np.int32))
    ws = skv.Workspace.for_problem(skv.problem_for(q, k), n)
    out = torch.empty((hq, d), device="cuda")
    lse = torch.empty(hq, device="cuda")
    _replay_matches(lambda: skv.skv_attend_sparse(q, k, v, n, it, ct, tail, out, lse, ws), [out, lse])


def test_one_call_topk_step_in_a_graph():
    """skv_topk_step keeps its per-head arrival counters and chunk tickets in
    the workspace header and resets them at each step's last arrival: two
    steps per replay (one through the published-key exchange, one through the
    global radix levels, which many tied keys force) replay bit for bit."""
    banner("graph: two one-call top-K steps per replay")
    hq, hkv, d, n, S, R, K = 32, 8, 128, 40000, 4, 64, 3000
    q, k, v = _rand((hq, d), 4), _rand((hkv, n, d), 5), _rand((hkv, n, d), 6)
    kt = _rand((hkv, 1, d), 7).repeat(1, n, 1).contiguous()  # every key equal: ties
    ws = skv.Workspace.for_problem(skv.problem_for(q, k), n)
    score = torch.empty((hkv, n), device="cuda")
    idx = torch.empty((hkv, S + K), dtype=torch.int32, device="cuda")
    cnt = torch.empty(hkv, dtype=torch.int32, device="cuda")
    out = torch.empty((hq, d), device="cuda")
    lse = torch.empty(hq, device="cuda")
    score2 = torch.empty_like(score)
    idx2 = torch.empty_like(idx)
    cnt2 = torch.empty_like(cnt)
    out2 = torch.empty_like(out)
    lse2 = torch.empty_like(lse)

    def run():
        skv.skv_topk_step(q, k, v, n, S, R, K, score, idx, cnt, out, lse, ws)
        skv.skv_topk_step(q, kt, v, n, S, R, K, score2, idx2, cnt2, out2, lse2, ws)

    _replay_matches(run, [score, idx, cnt, out, lse, score2, idx2, cnt2, out2, lse2])
    err = int(ws.tensor[skv.SKV_TOPK_ERROR_OFFSET:skv.SKV_TOPK_ERROR_OFFSET + 4].view(torch.int32).item())
    assert err == 0
    assert torch.equal(idx2[:, S:].cpu(), torch.arange(S, S + K, dtype=torch.int32).repeat(hkv, 1))
