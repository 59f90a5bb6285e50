#!/usr/bin/env python3
"""Decode-attention bench for libsparsekv on one MI355X.

Headline (the JSON `value`): microseconds per top-K sparse decode-attention
step for the Llama-3.1-8B shape at 32K context (32 query heads, 8 kv heads,
head dim 128, bf16), 30 % of the cache kept (4 sinks + 64 recent + 9762
entries per kv head chosen once by the 32-query observation-window score).
The same step over the whole cache (dense split-K) runs beside it.

Timing ("Locating the Crossing" protocol of the ByteCross page: five blocks,
each in a fresh process, averaged, with a 95 % interval): the headline sparse
and dense steps are timed in `--blocks` child processes that the parent starts
one after another before it makes any GPU call.  In each child, W untimed
warm-up steps run, then K steps are captured once into a HIP graph and replayed
between two HIP events on the launch stream, with a device synchronise on both
sides; each step reads a different one of L "layers" (distinct caches, about
1 GB at 32K) so the 256 MB Infinity Cache cannot serve the working set.
`value` is the mean over the blocks (median and the t-interval beside it).
Inputs are resident in HBM before the timed region.  A decode-attention step is two kernels: the split-K
partial kernel (the dominant one) and the small log-sum-exp merge; the
roofline figure divides the algorithmic bytes by the whole step time, so the
merge counts against it.  Eager (one host launch per call) times are reported
beside the graph times.

Also reported in `details` (default sections): the tiny fp32 MHA parity
configuration (per-step top-K and dense at 2K), the 30 % sink-plus-recent
window against dense decoding through masked, fused and split-K attention
(2K-128K; the masked and fused paths are PyTorch baselines), compaction of the 32K kept
sets into contiguous caches (gather once, then the dense step over them),
dense steps at 2K-128K, the
per-step top-K pipeline at 128K (score -> select -> gathered attention), the
Sparse-to-Dense round of the Qwen2-7B video workload (5 sparse drafts + one
gamma=5 verify), the SpecVLM selection on it (top-P 0.5 + uniform fill to
10 % of the video tokens) and the round over that set, sweeps of the round
over gamma = 1..13 and over K (measured vs I/O-model break-even acceptance), one-time selection costs, and the byte-count speedup bounds.
The 1024-head SparseMM batched step (17 GB of cache) is part of the default
sections.
`--sections mfma`, `--sections hbm` and `--sections valu` are profiling modes
(no bench line): the Qwen2-7B matrix-core calls; three eager calls of each
streaming kernel at 32K and 128K; the 32K dense step through the matrix-core
kernel (bf16) and the vector-ALU kernel (fp32 caches); for runs under
rocprofv3 counters.

cpu_baseline: the fp64 oracle (test infrastructure) timed on this host on a
bounded sample of the headline step.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attn µs/step and % HBM roofline at 32K/128K ctx, dense vs top-K"
# FETCH_SIZE / WRITE_SIZE of the headline step, taken with rocprofv3 --pmc
COUNTERS = os.path.join(ROOT, "profiles", "attend_sparse_llama32k_hbm_counters.md")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# Dense decode baselines of "Where Activation Sparsity and KV-Cache Sparsity
# Cross in LLM Decoding", "The Attention Baseline": the same attention read
# through an eager masked implementation (matmul, explicit mask, softmax,
# matmul) and through one fused attention kernel with no split over the
# sequence (PyTorch SDPA, flash backend).  Both are PyTorch's own kernels,
# timed only as baselines.  q [Hq][d] bf16; k, v [Hkv][n_cap][d] bf16 (rows
# [0, L) are read); returns [Hkv][G][d] in bf16 for query head h * G + g.

def masked_decode(q, k, v, L, scale, mask=None):
    import torch
    hkv, d = k.shape[0], k.shape[2]
    G = q.shape[0] // hkv
    qg = q.view(hkv, G, d).transpose(1, 2).contiguous()                 # [Hkv][d][G]
    lg = torch.matmul(k[:, :L], qg).float() * scale                      # [Hkv][L][G]
    if mask is not None:
        lg = lg + mask
    pr = torch.softmax(lg, dim=1).to(q.dtype).transpose(1, 2).contiguous()
    return torch.matmul(pr, v[:, :L])                                   # [Hkv][G][d]


def fused_decode(q, k, v, L, scale):
    import torch.nn.functional as F
    from torch.nn.attention import SDPBackend, sdpa_kernel
    hkv, d = k.shape[0], k.shape[2]
    G = q.shape[0] // hkv
    with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
        o = F.scaled_dot_product_attention(q.view(1, hkv, G, d), k[None, :, :L], v[None, :, :L], scale=scale)
    return o[0]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--layers", type=int, default=8, help="distinct caches rotated at 32K")
    ap.add_argument("--blocks", type=int, default=5, help="timed blocks (median reported)")
    ap.add_argument("--sections", default="default",
                    help="headline | default | all | mfma (profiling: only the Qwen2-7B matrix-core "
                         "calls, no bench line) | hbm (profiling: three eager calls of each "
                         "streaming kernel at 32K and 128K, no bench line) | valu (profiling: the 32K "
                         "dense step through the matrix-core and the vector-ALU kernels, no bench line)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run one 512 MiB device copy (counter calibration under a profiler)")
    ap.add_argument("--child-block", action="store_true",
                    help="internal: time one block of the headline steps and print it as JSON")
    return ap.parse_args()


def run_blocks(args):
    """Time the headline steps in args.blocks fresh child processes, one after
    another (this process has made no GPU call yet).  Returns the children's
    JSON results."""
    import subprocess
    res = []
    for b in range(args.blocks):
        log(f"fresh-process block {b + 1}/{args.blocks}")
        cmd = [sys.executable, os.path.abspath(__file__), "--child-block", "--steps", str(args.steps),
               "--warmup", str(args.warmup), "--layers", str(args.layers)]
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
        if r.returncode != 0:
            sys.stderr.write(r.stderr[-4000:])
            raise SystemExit(f"block {b + 1} failed with status {r.returncode}")
        res.append(json.loads(r.stdout.strip().splitlines()[-1]))
    return res


def interval95(xs):
    """(mean, half-width of the two-sided 95 % Student-t interval of the mean)."""
    from scipy import stats
    x = np.asarray(xs, np.float64)
    if len(x) < 2:
        return float(x.mean()), None
    return float(x.mean()), float(stats.t.ppf(0.975, len(x) - 1) * x.std(ddof=1) / math.sqrt(len(x)))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: the decode "
              "step shards by kv head with no exchange, so one GPU's throughput is the "
              "per-GPU figure", file=sys.stderr)
        sys.exit(2)
    blocks = None
    if not args.child_block and args.sections in ("headline", "default", "all"):
        blocks = run_blocks(args)  # before this process touches the GPU
    import torch

    import sparse_top_kv_amd as skv
    from sparse_top_kv_amd import roofline as rf
    import synth

    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    details = {}

    def dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    def host_list(t):
        return [int(x) for x in t.cpu().tolist()]

    def time_steps(step, nsteps, warmup, blocks, graph=True):
        """Median over blocks of (elapsed / nsteps) in microseconds, timed with HIP
        events on the launch stream.  step(i) enqueues step i.  With graph=True the
        nsteps launches are captured once into a HIP graph and each block replays
        it, so host-side launch cost does not leak into the GPU time."""
        for i in range(warmup):
            step(i)
        torch.cuda.synchronize()
        g = None
        if graph:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(nsteps):
                    step(i)
            g.replay()
            torch.cuda.synchronize()
        per = []
        for b in range(blocks):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            if g is not None:
                g.replay()
            else:
                for i in range(nsteps):
                    step(i)
            e1.record(stream)
            torch.cuda.synchronize()
            per.append(e0.elapsed_time(e1) * 1000.0 / nsteps)
        per.sort()
        return per[len(per) // 2], per

    def attention_baselines(big, hq, hkv, d, out, lse):
        """The same 30 % sink-plus-recent window against dense decoding when
        both read the cache through masked (eager ops with an explicit mask),
        fused (one attention kernel, no split over the sequence) or split-K
        attention ("Where Activation Sparsity and KV-Cache Sparsity Cross",
        "The Attention Baseline").  The masked and fused paths are PyTorch's
        own (matmul + softmax, and SDPA's flash kernel); they are baselines
        only.  Returns speedups, each path's HBM fraction and the byte bounds."""
        scale = 1.0 / math.sqrt(d)
        res = {}
        for nn in (2048, 8192, 32768, 131072):
            w = int(round(0.3 * nn))
            recent = w - 4
            # window caches as a sink cache would hold them (contiguous)
            win = [(torch.cat([b["k"][:, :4], b["k"][:, nn - recent:nn]], 1).contiguous(),
                    torch.cat([b["v"][:, :4], b["v"][:, nn - recent:nn]], 1).contiguous()) for b in big]
            mask = {L: torch.zeros((L, 1), device="cuda") for L in (nn, w)}
            sink_idx = torch.arange(4, dtype=torch.int32, device="cuda").repeat(hkv, 1).contiguous()
            sink_cnt = torch.full((hkv,), 4, dtype=torch.int32, device="cuda")

            def masked(q, k, v, L):
                return masked_decode(q, k, v, L, scale, mask[L])

            def fused(q, k, v, L):
                return fused_decode(q, k, v, L, scale)

            paths = {
                "masked": (lambda i: masked(big[i % 2]["q"], big[i % 2]["k"], big[i % 2]["v"], nn),
                           lambda i: masked(big[i % 2]["q"], win[i % 2][0], win[i % 2][1], w), False),
                "fused": (lambda i: fused(big[i % 2]["q"], big[i % 2]["k"], big[i % 2]["v"], nn),
                          lambda i: fused(big[i % 2]["q"], win[i % 2][0], win[i % 2][1], w), False),
                "split_k": (lambda i: skv.skv_attend_dense(big[i % 2]["q"], big[i % 2]["k"], big[i % 2]["v"],
                                                           nn, out, lse, ws),
                            lambda i: skv.skv_attend_sparse(big[i % 2]["q"], big[i % 2]["k"], big[i % 2]["v"],
                                                            nn, sink_idx, sink_cnt, nn - recent, out, lse,
                                                            ws), True),
            }
            by_d = rf.dense_step_bytes(hq, hkv, d, nn, "bf16")
            by_w = rf.dense_step_bytes(hq, hkv, d, w, "bf16")
            layer = 2 * rf.projection_params(4096, 14336) + rf.kv_bytes_per_layer(nn)
            entry = {"window": w, "byte_bound_attention": round(by_d / by_w, 3),
                     "byte_bound_layer_with_projections": round(
                         rf.speedup_bound(layer, rf.kv_bytes_per_layer(nn) - rf.kv_bytes_per_layer(w)), 3)}
            for name, (dstep, wstep, graph) in paths.items():
                try:
                    nst = 20 if nn < 131072 else 10
                    td, _ = time_steps(dstep, nst, 3, 3, graph=graph)
                    tw, _ = time_steps(wstep, nst, 3, 3, graph=graph)
                    entry[name] = {"dense_us": round(td, 2), "window_us": round(tw, 2),
                                   "speedup": round(td / tw, 3),
                                   "dense_hbm_frac": round(rf.roofline_fraction(by_d, td * 1e-6), 4)}
                    if graph:
                        te, _ = time_steps(dstep, nst, 3, 1, graph=False)
                        tew, _ = time_steps(wstep, nst, 3, 1, graph=False)
                        entry[name]["eager_speedup"] = round(te / tew, 3)
                except RuntimeError as e:  # e.g. no flash kernel for this shape
                    entry[name] = {"error": str(e).splitlines()[0][:160]}
            res[str(nn)] = entry
            del win
        return res

    if args.sections == "mfma":
        # profiling mode for counter runs: the two matrix-core calls of the
        # Qwen2-7B workload (text-window score, W = 512; gamma = 5 verify)
        wq = synth.qwen_std()
        m = wq.extra["m_v"] + wq.extra["m_t"]
        gq = wq.extra["gamma"]
        qo4, k4, v4 = dev(wq.q_obs), dev(wq.k), dev(wq.v)
        qv4 = dev(wq.extra["q_verify"])
        ws4 = skv.Workspace.for_problem(skv.problem_for(qo4, k4), m + gq, wq.extra["m_t"])
        sc4 = torch.empty((wq.n_kv_heads, m), device="cuda")
        ov = torch.empty((gq, wq.n_q_heads, wq.head_dim), device="cuda")
        lv = torch.empty((gq, wq.n_q_heads), device="cuda")
        sc_us, _ = time_steps(lambda i: skv.skv_score(qo4, k4, m, sc4, ws4), 3, 1, 1, graph=False)
        v_us, _ = time_steps(lambda i: skv.skv_verify(qv4, k4, v4, m + gq, ov, lv, ws4), 20, 2, 1,
                             graph=False)
        print(json.dumps({"sections": "mfma", "text_window_score_us": round(sc_us, 1),
                          "verify_us": round(v_us, 2)}), flush=True)
        return

    if args.sections == "valu":
        # profiling mode for the matrix-core choice: the 32K dense decode step of
        # the Llama-3.1-8B shape through the matrix-core kernel (bf16 caches)
        # and, on the same shape with fp32 caches, through the vector-ALU kernel
        w = synth.llama_obs(layer=0)
        n = w.n
        q, k, v = dev(w.q), dev(w.k), dev(w.v)
        res = {}
        for name, (qq, kk, vv) in (("bf16_mfma", (q, k, v)),
                                   ("fp32_valu", (q.float(), k.float(), v.float()))):
            wsv = skv.Workspace.for_problem(skv.problem_for(qq, kk), n)
            o = torch.empty((w.n_q_heads, w.head_dim), device="cuda")
            ls = torch.empty(w.n_q_heads, device="cuda")
            us, _ = time_steps(lambda i: skv.skv_attend_dense(qq, kk, vv, n, o, ls, wsv), 20, 2, 1, graph=False)
            res[name] = {"eager_us": round(us, 2), "keys": w.n_kv_heads * n}
            del wsv
        print(json.dumps({"sections": "valu", **res}), flush=True)
        return

    if args.sections == "hbm":
        # profiling mode for HBM counter runs: each call three times, eagerly, in
        # a fixed order (32K: window score, select, gather, sparse and dense
        # step; 128K: per-step score, select, sparse and dense step)
        out_t = {}

        def timed(name, fn, reps=3):
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            out_t[name] = round(e0.elapsed_time(e1) * 1000.0 / reps, 2)

        w = synth.llama_obs(layer=0)
        q, qo, k, v = dev(w.q), dev(w.q_obs), dev(w.k), dev(w.v)
        n, S, R, K = w.n, w.n_sink, w.n_recent, w.k_top
        hq, hkv, d = w.n_q_heads, w.n_kv_heads, w.head_dim
        ws = skv.Workspace.for_problem(skv.problem_for(qo, k), 131072, 512)
        sc = torch.empty((hkv, n), device="cuda")
        idx = torch.empty((hkv, S + K), dtype=torch.int32, device="cuda")
        cnt = torch.empty(hkv, dtype=torch.int32, device="cuda")
        out = torch.empty((hq, d), device="cuda")
        lse = torch.empty(hq, device="cuda")
        kc = torch.empty((hkv, S + K + R, d), dtype=torch.bfloat16, device="cuda")
        vc = torch.empty_like(kc)
        timed("32k_window_score", lambda: skv.skv_score(qo, k, n, sc, ws))
        timed("32k_select", lambda: skv.skv_select(sc, n, S, R, K, idx, cnt, ws))
        timed("32k_gather", lambda: skv.skv_gather(k, v, n, idx, cnt, n - R, kc, vc))
        timed("32k_sparse_step", lambda: skv.skv_attend_sparse(q, k, v, n, idx, cnt, n - R, out, lse, ws))
        timed("32k_dense_step", lambda: skv.skv_attend_dense(q, k, v, n, out, lse, ws))
        del k, v, kc, vc
        w3 = synth.llama_needle(layer=0)
        q3, k3, v3 = dev(w3.q), dev(w3.k), dev(w3.v)
        n3, K3 = w3.n, w3.k_top
        sc3 = torch.empty((hkv, n3), device="cuda")
        idx3 = torch.empty((hkv, S + K3), dtype=torch.int32, device="cuda")
        timed("128k_step_score", lambda: skv.skv_score(q3, k3, n3, sc3, ws))
        timed("128k_select", lambda: skv.skv_select(sc3, n3, S, R, K3, idx3, cnt, ws))
        timed("128k_sparse_step", lambda: skv.skv_attend_sparse(q3, k3, v3, n3, idx3, cnt, n3 - R, out, lse, ws))
        timed("128k_dense_step", lambda: skv.skv_attend_dense(q3, k3, v3, n3, out, lse, ws))
        timed("128k_topk_step", lambda: skv.skv_topk_step(q3, k3, v3, n3, S, R, K3, sc3, idx3, cnt, out, lse, ws))
        if args.calib_copy:  # known traffic for the counters' scale: 512 MiB read, 512 MiB written
            src = torch.ones(512 << 20, dtype=torch.uint8, device="cuda")
            dst = torch.empty_like(src)
            torch.cuda.synchronize()
            dst.copy_(src)
            torch.cuda.synchronize()
        print(json.dumps({"sections": "hbm", "eager_us": out_t}), flush=True)
        return

    # ------------------------------------------------------------------
    # headline: Llama-3.1-8B shape, 32K, 30 % kept via window score once
    # ------------------------------------------------------------------
    L = args.layers
    log(f"generating {L} layers of the 32K Llama-shape workload")
    layers = []
    for l in range(L):
        w = synth.llama_obs(layer=l)
        layers.append(dict(q=dev(w.q), qo=dev(w.q_obs), k=dev(w.k), v=dev(w.v)))
    n, S, R, K = w.n, w.n_sink, w.n_recent, w.k_top
    hq, hkv, d = w.n_q_heads, w.n_kv_heads, w.head_dim
    p = skv.problem_for(layers[0]["qo"], layers[0]["k"])
    ws = skv.Workspace.for_problem(p, 131072, 512)
    for lay in layers:
        lay["score"] = torch.empty((hkv, n), device="cuda")
        lay["idx"] = torch.empty((hkv, S + K), dtype=torch.int32, device="cuda")
        lay["cnt"] = torch.empty(hkv, dtype=torch.int32, device="cuda")
        lay["out"] = torch.empty((hq, d), device="cuda")
        lay["lse"] = torch.empty(hq, device="cuda")

    def select_once(i):
        lay = layers[i % L]
        skv.skv_score(lay["qo"], lay["k"], n, lay["score"], ws)
        skv.skv_select(lay["score"], n, S, R, K, lay["idx"], lay["cnt"], ws)

    sel_us, _ = time_steps(select_once, L, 1, 1, graph=False)
    details["llama32k_window_score_plus_select_once_us"] = round(sel_us, 2)
    tail = n - R

    def sparse_step(i):
        lay = layers[i % L]
        skv.skv_attend_sparse(lay["q"], lay["k"], lay["v"], n, lay["idx"], lay["cnt"], tail,
                              lay["out"], lay["lse"], ws)

    def dense_step(i):
        lay = layers[i % L]
        skv.skv_attend_dense(lay["q"], lay["k"], lay["v"], n, lay["out"], lay["lse"], ws)

    if args.child_block:
        sp1, _ = time_steps(sparse_step, args.steps, args.warmup, 1)
        de1, _ = time_steps(dense_step, args.steps, args.warmup, 1)
        print(json.dumps({"sparse_us": sp1, "dense_us": de1}), flush=True)
        return
    sp_blocks = sorted(b["sparse_us"] for b in blocks)
    de_blocks = sorted(b["dense_us"] for b in blocks)
    sp_us, sp_ci = interval95(sp_blocks)
    de_us, de_ci = interval95(de_blocks)
    sp_eager, _ = time_steps(sparse_step, args.steps, 2, 1, graph=False)
    de_eager, _ = time_steps(dense_step, args.steps, 2, 1, graph=False)
    # the same steps on one layer only: its cache stays in the 256 MB Infinity
    # Cache (labelled MALL-warm; not the headline)
    sp_warm, _ = time_steps(lambda i: sparse_step(0), args.steps, args.warmup, 3)
    de_warm, _ = time_steps(lambda i: dense_step(0), args.steps, args.warmup, 3)
    details["llama32k_sparse_us_mall_warm"] = round(sp_warm, 3)
    details["llama32k_dense_us_mall_warm"] = round(de_warm, 3)
    details["llama32k_sparse_us_eager_launches"] = round(sp_eager, 3)
    details["llama32k_dense_us_eager_launches"] = round(de_eager, 3)
    rows = S + K + R
    sp_bytes = rf.sparse_step_bytes(hq, hkv, d, rows, S + K, "bf16")
    de_bytes = rf.dense_step_bytes(hq, hkv, d, n, "bf16")
    details["llama32k_sparse_us"] = round(sp_us, 3)
    details["llama32k_sparse_ci95_us"] = None if sp_ci is None else [round(sp_us - sp_ci, 3), round(sp_us + sp_ci, 3)]
    details["llama32k_sparse_median_us"] = round(float(np.median(sp_blocks)), 3)
    details["llama32k_sparse_blocks_us"] = [round(x, 3) for x in sp_blocks]
    details["llama32k_dense_us"] = round(de_us, 3)
    details["llama32k_dense_ci95_us"] = None if de_ci is None else [round(de_us - de_ci, 3), round(de_us + de_ci, 3)]
    details["llama32k_dense_median_us"] = round(float(np.median(de_blocks)), 3)
    details["llama32k_dense_blocks_us"] = [round(x, 3) for x in de_blocks]
    details["llama32k_dense_hbm_frac"] = round(rf.roofline_fraction(de_bytes, de_us * 1e-6), 4)
    details["llama32k_sparse_hbm_frac"] = round(rf.roofline_fraction(sp_bytes, sp_us * 1e-6), 4)
    details["llama32k_speedup_measured"] = round(de_us / sp_us, 3)
    details["llama32k_speedup_byte_bound"] = round(de_bytes / sp_bytes, 3)
    details["llama32k_bytes"] = {"sparse": sp_bytes, "dense": de_bytes}

    if args.sections != "headline":
        # compaction: gather each layer's kept set once into a contiguous cache,
        # then run the dense step over it (against the in-place sparse step above)
        for lay in layers:
            lay["kc"] = torch.empty((hkv, rows, d), dtype=torch.bfloat16, device="cuda")
            lay["vc"] = torch.empty_like(lay["kc"])

        def gather_once(i):
            lay = layers[i % L]
            skv.skv_gather(lay["k"], lay["v"], n, lay["idx"], lay["cnt"], tail, lay["kc"], lay["vc"])

        def compact_step(i):
            lay = layers[i % L]
            skv.skv_attend_dense(lay["q"], lay["kc"], lay["vc"], rows, lay["out"], lay["lse"], ws)

        log("timing compaction and the dense step over the compacted caches")
        ga_us, _ = time_steps(gather_once, L, 2, args.blocks)
        cs_us, _ = time_steps(compact_step, args.steps, args.warmup, args.blocks)
        ga_bytes = 2 * 2 * hkv * rows * d * 2 + hkv * (S + K) * 4  # K+V rows read and written, indices
        cs_bytes = rf.dense_step_bytes(hq, hkv, d, rows, "bf16")
        gain = sp_us - cs_us
        details["llama32k_compaction"] = {
            "gather_once_us": round(ga_us, 3),
            "gather_hbm_frac": round(rf.roofline_fraction(ga_bytes, ga_us * 1e-6), 4),
            "compacted_dense_step_us": round(cs_us, 3),
            "compacted_dense_step_hbm_frac": round(rf.roofline_fraction(cs_bytes, cs_us * 1e-6), 4),
            "in_place_sparse_step_us": round(sp_us, 3),
            "steps_to_repay_gather": round(ga_us / gain, 1) if gain > 0 else None,
        }
        for lay in layers:
            del lay["kc"], lay["vc"]

    if args.calib_copy:
        src = torch.ones(512 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        details["calib_copy_bytes"] = {"read": src.numel(), "written": dst.numel()}
        del src, dst

    # streaming ceiling of this machine: a 1 GiB device-to-device copy (read + write)
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(5):
        dst.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize()
    ceil_gbps = 2 * src.numel() * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    details["copy_ceiling_GBps"] = round(ceil_gbps, 1)
    details["llama32k_sparse_frac_of_copy_ceiling"] = round(sp_bytes / (sp_us * 1e-6) / 1e9 / ceil_gbps, 4)
    details["llama32k_dense_frac_of_copy_ceiling"] = round(de_bytes / (de_us * 1e-6) / 1e9 / ceil_gbps, 4)
    del src, dst
    # streaming-read ceiling: libskvprobe's read kernel (one workgroup per CU,
    # 16-byte non-temporal loads) over two alternating 1 GiB buffers
    probe = ctypes.CDLL(os.path.join(os.path.dirname(skv.LIB_PATH), "libskvprobe.so"))
    probe.skv_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    rbufs = [torch.ones(1 << 28, dtype=torch.float32, device="cuda") for _ in range(2)]
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")

    def read_once(i):
        if probe.skv_probe_read(rbufs[i % 2].data_ptr(), 1 << 30, sink.data_ptr(), 256,
                                ctypes.c_void_p(stream.cuda_stream)) != 0:
            raise RuntimeError("skv_probe_read failed")

    for i in range(4):
        read_once(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(10):
        read_once(i)
    e1.record(stream)
    torch.cuda.synchronize()
    read_gbps = (1 << 30) * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    details["read_ceiling_GBps"] = round(read_gbps, 1)
    details["llama32k_sparse_frac_of_read_ceiling"] = round(sp_bytes / (sp_us * 1e-6) / 1e9 / read_gbps, 4)
    details["llama32k_dense_frac_of_read_ceiling"] = round(de_bytes / (de_us * 1e-6) / 1e9 / read_gbps, 4)
    del rbufs, sink
    torch.cuda.empty_cache()

    if args.sections != "headline":
        del layers
        torch.cuda.empty_cache()
        # ------------------------------------------------------------------
        # 128K: dense sweep and the per-step top-K pipeline with a needle
        # ------------------------------------------------------------------
        log("generating 2 layers of the 128K Llama-shape workload")
        big = []
        for l in range(2):
            w3 = synth.llama_needle(layer=l)
            big.append(dict(q=dev(w3.q), k=dev(w3.k), v=dev(w3.v)))
        n3, K3 = w3.n, w3.k_top
        out = torch.empty((hq, d), device="cuda")
        lse = torch.empty(hq, device="cuda")
        sweep = {}
        for nn in (2048, 8192, 32768, 131072):
            # windows at different offsets of the two 128K caches: distinct memory per step
            nwin = max(1, min(64, n3 // nn))

            def dstep(i, nn=nn, nwin=nwin):
                b = big[i % 2]
                off = ((i // 2) % nwin) * nn
                skv.skv_attend_dense(b["q"], b["k"][:, off:], b["v"][:, off:], nn, out, lse, ws)

            us, _ = time_steps(dstep, args.steps, args.warmup, 3)
            by = rf.dense_step_bytes(hq, hkv, d, nn, "bf16")
            sweep[str(nn)] = {"us": round(us, 3), "hbm_frac": round(rf.roofline_fraction(by, us * 1e-6), 4)}
        details["dense_sweep"] = sweep
        details["attention_baselines"] = attention_baselines(big, hq, hkv, d, out, lse)
        score3 = torch.empty((hkv, n3), device="cuda")
        idx3 = torch.empty((hkv, S + K3), dtype=torch.int32, device="cuda")
        cnt3 = torch.empty(hkv, dtype=torch.int32, device="cuda")

        def topk_step(i):  # the step as one call
            b = big[i % 2]
            skv.skv_topk_step(b["q"], b["k"], b["v"], n3, S, R, K3, score3, idx3, cnt3, out, lse, ws)

        def topk_three(i):  # the same step as score -> select -> attend_sparse
            b = big[i % 2]
            skv.skv_score(b["q"], b["k"], n3, score3, ws)
            skv.skv_select(score3, n3, S, R, K3, idx3, cnt3, ws)
            skv.skv_attend_sparse(b["q"], b["k"], b["v"], n3, idx3, cnt3, n3 - R, out, lse, ws)

        log("timing the 128K per-step top-K pipeline")
        ts_us, _ = time_steps(topk_step, max(20, args.steps // 4), 5, 3)
        t3_us, _ = time_steps(topk_three, max(20, args.steps // 4), 5, 3)
        # one call: K once, the kept V rows, the fp32 scores out
        ts_bytes = hkv * n3 * d * 2 + hkv * (S + K3 + R) * d * 2 + hkv * n3 * 4
        t3_bytes = (hkv * n3 * d * 2 + rf.sparse_step_bytes(hq, hkv, d, S + K3 + R, S + K3, "bf16"))
        details["llama128k_topk_step_us"] = round(ts_us, 2)
        details["llama128k_topk_step_hbm_frac"] = round(rf.roofline_fraction(ts_bytes, ts_us * 1e-6), 4)
        details["llama128k_topk_three_call_us"] = round(t3_us, 2)
        details["llama128k_topk_three_call_hbm_frac"] = round(rf.roofline_fraction(t3_bytes, t3_us * 1e-6), 4)
        details["llama128k_topk_speedup_measured"] = round(sweep["131072"]["us"] / ts_us, 3)
        details["llama128k_topk_speedup_three_call"] = round(sweep["131072"]["us"] / t3_us, 3)
        details["llama128k_topk_speedup_byte_bound"] = round(
            rf.dense_step_bytes(hq, hkv, d, n3, "bf16") / ts_bytes, 3)
        # the three calls of that step timed on their own (same inputs)
        nst = max(20, args.steps // 4)
        part = {}
        part["score_us"], _ = time_steps(
            lambda i: skv.skv_score(big[i % 2]["q"], big[i % 2]["k"], n3, score3, ws), nst, 5, 3)
        part["select_us"], _ = time_steps(
            lambda i: skv.skv_select(score3, n3, S, R, K3, idx3, cnt3, ws), nst, 5, 3)
        part["attend_sparse_us"], _ = time_steps(
            lambda i: skv.skv_attend_sparse(big[i % 2]["q"], big[i % 2]["k"], big[i % 2]["v"], n3, idx3, cnt3,
                                            n3 - R, out, lse, ws), nst, 5, 3)
        details["llama128k_topk_step_parts_us"] = {k: round(v, 2) for k, v in part.items()}
        del big, score3
        torch.cuda.empty_cache()
        # ------------------------------------------------------------------
        # Qwen2-7B video Sparse-to-Dense round: 5 sparse drafts + 1 verify
        # ------------------------------------------------------------------
        # tiny MHA fp32 (the parity configuration): per-step top-K and dense
        wt = synth.tiny_mha()
        qt1, kt1, vt1 = dev(wt.q), dev(wt.k), dev(wt.v)
        wst = skv.Workspace.for_problem(skv.problem_for(qt1, kt1), wt.n)
        sct = torch.empty((wt.n_kv_heads, wt.n), device="cuda")
        idxt = torch.empty((wt.n_kv_heads, wt.n_sink + wt.k_top), dtype=torch.int32, device="cuda")
        cntt = torch.empty(wt.n_kv_heads, dtype=torch.int32, device="cuda")
        ot = torch.empty((wt.n_q_heads, wt.head_dim), device="cuda")
        lt = torch.empty(wt.n_q_heads, device="cuda")

        def tiny_topk(i):
            skv.skv_score(qt1, kt1, wt.n, sct, wst)
            skv.skv_select(sct, wt.n, wt.n_sink, wt.n_recent, wt.k_top, idxt, cntt, wst)
            skv.skv_attend_sparse(qt1, kt1, vt1, wt.n, idxt, cntt, wt.n - wt.n_recent, ot, lt, wst)

        tk_us, _ = time_steps(tiny_topk, args.steps, args.warmup, 3)
        td_us, _ = time_steps(lambda i: skv.skv_attend_dense(qt1, kt1, vt1, wt.n, ot, lt, wst),
                              args.steps, args.warmup, 3)
        details["tiny_mha_fp32_2k"] = {"topk_step_us": round(tk_us, 2), "dense_step_us": round(td_us, 2),
                                       "note": "launch-bound parity configuration (8 heads, d = 64, fp32)"}
        del qt1, kt1, vt1

        log("generating the Qwen2-7B video workload")
        wq = synth.qwen_std()
        m_v, m_t, gamma = wq.extra["m_v"], wq.extra["m_t"], wq.extra["gamma"]
        m = m_v + m_t
        hq4, hkv4 = wq.n_q_heads, wq.n_kv_heads
        L4 = 12  # 12 x 52 MB of K+V: beyond the Infinity Cache
        # room for up to 16 drafted entries (the gamma sweep below)
        pad = synth.bf16_bits(np.random.default_rng(5).standard_normal(
            (hkv4, m + 16 - wq.k.shape[1], d)).astype(np.float32))
        k4h, v4h = np.concatenate([wq.k, pad], axis=1), np.concatenate([wq.v, pad], axis=1)
        kv4 = [(dev(k4h), dev(v4h))] + [(dev(np.roll(k4h, l, axis=1)), dev(np.roll(v4h, l, axis=1)))
                                        for l in range(1, L4)]
        qo4 = dev(wq.q_obs)
        qd4 = [dev(np.ascontiguousarray(wq.extra["q_draft"][t])) for t in range(gamma)]
        qv4 = dev(wq.extra["q_verify"])
        ws4 = skv.Workspace.for_problem(skv.problem_for(qo4, kv4[0][0]), m + 16, m_t)
        sc4 = torch.empty((hkv4, m), device="cuda")
        idx4 = torch.empty((hkv4, wq.k_top), dtype=torch.int32, device="cuda")
        cnt4 = torch.empty(hkv4, dtype=torch.int32, device="cuda")

        def sel4(i):
            k4 = kv4[i % L4][0]
            skv.skv_score(qo4, k4, m, sc4, ws4)
            skv.skv_select(sc4, m, 0, m_t, wq.k_top, idx4, cnt4, ws4)

        sel4_us, _ = time_steps(sel4, 4, 1, 1, graph=False)
        obs4_us, _ = time_steps(lambda i: skv.skv_score(qo4, kv4[i % L4][0], m, sc4, ws4), 4, 1, 3)
        obs4_flops = rf.obs_score_flops(hq4, m, d, m_t)
        o4 = torch.empty((hq4, d), device="cuda")
        l4 = torch.empty(hq4, device="cuda")
        ov = torch.empty((gamma, hq4, d), device="cuda")
        lv = torch.empty((gamma, hq4), device="cuda")

        def round_std(i):
            k4, v4 = kv4[i % L4]
            for t in range(gamma):
                skv.skv_attend_sparse(qd4[t], k4, v4, m + t + 1, idx4, cnt4, m_v, o4, l4, ws4)
            skv.skv_verify(qv4, k4, v4, m + gamma, ov, lv, ws4)

        def round_dense(i):
            k4, v4 = kv4[i % L4]
            for t in range(gamma):
                skv.skv_attend_dense(qd4[t], k4, v4, m + t + 1, o4, l4, ws4)

        def verify_only(i):
            k4, v4 = kv4[i % L4]
            skv.skv_verify(qv4, k4, v4, m + gamma, ov, lv, ws4)

        # SpecVLM selection on the same text-window score: top-P retention
        # (lambda 0.5) + uniform fill to 10 % of the video tokens (r = 90 %)
        vidx4 = torch.empty((hkv4, m_v), dtype=torch.int32, device="cuda")
        vcnt4 = torch.empty(hkv4, dtype=torch.int32, device="cuda")
        vcr4 = torch.empty(hkv4, dtype=torch.int32, device="cuda")

        def topp4(i):
            skv.skv_select_topp(sc4, m, 0, m_t, 0.5, 0.9, vidx4, vcnt4, ws4, count_r=vcr4)

        def topp4_pooled(i):
            skv.skv_select_topp(sc4, m, 0, m_t, 0.5, 0.9, vidx4, vcnt4, ws4, count_r=vcr4, pooled=True)

        sel4(0)
        tp_pool_us, _ = time_steps(topp4_pooled, 8, 2, 3)
        tp_us, _ = time_steps(topp4, 8, 2, 3)
        torch.cuda.synchronize()
        v_kept = host_list(vcnt4)
        v_ret = host_list(vcr4)

        def round_specvlm(i):
            k4, v4 = kv4[i % L4]
            for t in range(gamma):
                skv.skv_attend_sparse(qd4[t], k4, v4, m + t + 1, vidx4, vcnt4, m_v, o4, l4, ws4)
            skv.skv_verify(qv4, k4, v4, m + gamma, ov, lv, ws4)

        log("timing the Sparse-to-Dense round")
        r_us, _ = time_steps(round_std, max(20, args.steps // 4), 5, 3)
        rv_us, _ = time_steps(round_specvlm, max(20, args.steps // 4), 5, 3)
        rd_us, _ = time_steps(round_dense, max(20, args.steps // 4), 5, 3)
        v_us, _ = time_steps(verify_only, args.steps, args.warmup, 3)
        v_bytes = rf.verify_bytes(hq4, hkv4, d, m + gamma, gamma, "bf16")
        draft_bytes = sum(rf.sparse_step_bytes(hq4, hkv4, d, wq.k_top + m_t + t + 1, wq.k_top, "bf16")
                          for t in range(gamma))
        dense_round_bytes = sum(rf.dense_step_bytes(hq4, hkv4, d, m + t + 1, "bf16") for t in range(gamma))
        details["qwen_std"] = {
            "text_window_score_plus_select_once_us": round(sel4_us, 1),
            "text_window_score_us": round(obs4_us, 1),
            "text_window_score_tflops": round(obs4_flops / (obs4_us * 1e-6) / 1e12, 1),
            "text_window_score_mfma_frac_of_bf16_peak": round(obs4_flops / (obs4_us * 1e-6) / 2.5e15, 4),
            "round_5_drafts_plus_verify_us": round(r_us, 2),
            "dense_5_steps_us": round(rd_us, 2),
            "verify_us": round(v_us, 3),
            "verify_hbm_frac": round(rf.roofline_fraction(v_bytes, v_us * 1e-6), 4),
            "verify_tflops": round(rf.verify_flops(hq4, m + gamma, d, gamma) / (v_us * 1e-6) / 1e12, 2),
            "verify_mfma_frac_of_bf16_peak": round(
                rf.verify_flops(hq4, m + gamma, d, gamma) / (v_us * 1e-6) / 2.5e15, 5),
            "round_speedup_measured_alpha1": round(rd_us / r_us, 3),
            "specvlm_topp_select_us": round(tp_us, 2),
            "specvlm_topp_select_pooled_us": round(tp_pool_us, 2),
            "specvlm_kept_per_head": v_kept,
            "specvlm_top_p_retained_per_head": v_ret,
            "specvlm_round_5_drafts_plus_verify_us": round(rv_us, 2),
            "round_speedup_byte_bound_alpha1": round(dense_round_bytes / (draft_bytes + v_bytes), 3),
        }
        # Sparse-to-Dense sweeps: draft length gamma (K fixed) and kept K
        # (gamma = 5).  Per accepted token a round costs T_round / (alpha gamma)
        # against T_dense for vanilla decoding, so the measured break-even
        # acceptance is T_round / (gamma T_dense); the I/O model's is
        # (K + m_t) / (m_v + m_t) + 1 / gamma.
        log("Sparse-to-Dense sweeps over gamma and K")
        dense1_us, _ = time_steps(lambda i: skv.skv_attend_dense(qd4[0], kv4[i % L4][0], kv4[i % L4][1],
                                                                m + 1, o4, l4, ws4),
                                  args.steps, args.warmup, 3)
        rng4 = np.random.default_rng(7)
        qv_all = dev(synth.bf16_bits(rng4.standard_normal((16, hq4, d)).astype(np.float32)))
        ov16 = torch.empty((16, hq4, d), device="cuda")
        lv16 = torch.empty((16, hq4), device="cuda")

        def round_g(gam, kidx, kcnt):
            def step(i):
                k4, v4 = kv4[i % L4]
                for t in range(gam):
                    skv.skv_attend_sparse(qd4[t % gamma], k4, v4, m + t + 1, kidx, kcnt, m_v, o4, l4, ws4)
                skv.skv_verify(qv_all[:gam], k4, v4, m + gam, ov16[:gam], lv16[:gam], ws4)
            return step

        def sweep_entry(gam, k_sel, kidx, kcnt):
            us, _ = time_steps(round_g(gam, kidx, kcnt), 10, 2, 3)
            vus, _ = time_steps(lambda i: skv.skv_verify(qv_all[:gam], kv4[i % L4][0], kv4[i % L4][1], m + gam,
                                                         ov16[:gam], lv16[:gam], ws4), 20, 2, 3)
            return {"round_us": round(us, 2), "verify_us": round(vus, 2),
                    "alpha_break_even_measured": round(us / (gam * dense1_us), 3),
                    "alpha_break_even_io_model": round(rf.std_break_even_alpha(gam, k_sel, m_t, m_v), 3)}

        g_sweep = {str(g): sweep_entry(g, wq.k_top, idx4, cnt4) for g in range(1, 14)}
        k_sweep = {}
        for frac in (0.05, 0.1, 0.2, 0.3, 0.5):
            kk = int(frac * m_v)
            kidx = torch.empty((hkv4, kk), dtype=torch.int32, device="cuda")
            kcnt = torch.empty(hkv4, dtype=torch.int32, device="cuda")
            skv.skv_score(qo4, kv4[0][0], m, sc4, ws4)
            skv.skv_select(sc4, m, 0, m_t, kk, kidx, kcnt, ws4)
            k_sweep[str(kk)] = sweep_entry(gamma, kk, kidx, kcnt)
        details["qwen_std_sweeps"] = {"dense_step_us": round(dense1_us, 3), "gamma": g_sweep,
                                      "K_at_gamma5": k_sweep}
        del kv4
        torch.cuda.empty_cache()

    if args.sections in ("default", "all"):
        log("generating the 1024-head SparseMM workload (17 GB)")
        w5 = synth.sparsemm_heads()
        n5, H5, R5 = w5.n, w5.n_q_heads, w5.n_recent
        ex = w5.extra
        q5, qo5, k5, v5 = dev(w5.q), dev(w5.q_obs), dev(w5.k), dev(w5.v)
        del w5
        ws5 = skv.Workspace.for_problem(skv.problem_for(qo5, k5), n5, ex["W"])
        kb, _ = skv.skv_budgets(ex["head_scores"], ex["total_budget"], ex["window"], ex["rho"], n5 - R5)
        kdev = dev(kb)
        sc5 = torch.empty((H5, n5), device="cuda")
        idx5 = torch.empty((H5, int(kb.max())), dtype=torch.int32, device="cuda")
        cnt5 = torch.empty(H5, dtype=torch.int32, device="cuda")

        def sel5(i):
            skv.skv_score(qo5, k5, n5, sc5, ws5)
            skv.skv_select(sc5, n5, 0, R5, 0, idx5, cnt5, ws5, k_per_head=kdev, k_max=int(kb.max()))

        s5_us, _ = time_steps(sel5, 2, 1, 1, graph=False)
        o5 = torch.empty((H5, d), device="cuda")
        l5 = torch.empty(H5, device="cuda")

        def step5(i):
            skv.skv_attend_sparse(q5, k5, v5, n5, idx5, cnt5, n5 - R5, o5, l5, ws5)

        st5_us, _ = time_steps(step5, args.steps, args.warmup, 3)
        b5 = rf.sparse_step_bytes(H5, H5, d, [int(x) + R5 for x in kb], [int(x) for x in kb], "bf16")
        details["sparsemm_1024h"] = {
            "window_score_plus_select_once_us": round(s5_us, 1),
            "batched_sparse_step_us": round(st5_us, 2),
            "hbm_frac": round(rf.roofline_fraction(b5, st5_us * 1e-6), 4),
            "byte_bound_vs_dense": round(rf.dense_step_bytes(H5, H5, d, n5, "bf16") / b5, 1),
        }

    # ------------------------------------------------------------------
    # CPU baseline: the oracle on a bounded sample of the headline step
    # ------------------------------------------------------------------
    import oracle
    log("timing the fp64 oracle on the host")
    w0 = synth.llama_obs(layer=0)
    _, s32 = oracle.score(w0.q_obs, w0.k, n)
    oi, oc = oracle.select(s32, S, R, K)
    threads = oracle.default_threads()
    t0 = time.perf_counter()
    reps = 0
    while True:
        oracle.attend_sparse(w0.q, w0.k, w0.v, n, oi, oc, tail, nthreads=threads)
        reps += 1
        if time.perf_counter() - t0 >= args.cpu_seconds:
            break
    cpu_us = (time.perf_counter() - t0) / reps * 1e6
    # single thread, same step (a few runs)
    t0 = time.perf_counter()
    reps1 = 0
    while True:
        oracle.attend_sparse(w0.q, w0.k, w0.v, n, oi, oc, tail, nthreads=1)
        reps1 += 1
        if time.perf_counter() - t0 >= max(1.0, args.cpu_seconds / 5):
            break
    cpu1_us = (time.perf_counter() - t0) / reps1 * 1e6
    t0 = time.perf_counter()
    oracle.attend_dense(w0.q, w0.k, w0.v, n, nthreads=threads)
    cpu_dense_us = (time.perf_counter() - t0) * 1e6
    cpu_score_select_us = None
    if args.sections != "headline":
        # per-step score + select of the 128K workload (one run)
        w3c = synth.llama_needle(layer=0)
        t0 = time.perf_counter()
        _, s3 = oracle.score(w3c.q[None], w3c.k, w3c.n, nthreads=threads)
        oracle.select(s3, w3c.n_sink, w3c.n_recent, w3c.k_top)
        cpu_score_select_us = round((time.perf_counter() - t0) * 1e6, 1)
        del w3c, s3
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass

    line = {
        "metric": METRIC,
        "value": round(sp_us, 3),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(sp_us / 1000.0, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "Llama-3.1-8B-shape single-sequence decode attention, 32K context, top-K sparse "
                        "step over 30% of the cache (4 sinks + 64 recent + 9762 by 32-query window score)",
            "q_heads": hq, "kv_heads": hkv, "head_dim": d, "context": n, "kept_rows_per_kv_head": rows,
            "layers_rotated": L,
            "timing": f"mean of {args.blocks} blocks x {args.steps} graph-replayed steps, each block in a "
                      "fresh process; 95 % t-interval in details",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(sp_bytes / (sp_us * 1e-6) / 1e9, 1),
            "peak": 8000.0,
            "unit": "GB/s",
            "frac": round(rf.roofline_fraction(sp_bytes, sp_us * 1e-6), 4),
            "traffic": rf.counter_traffic(COUNTERS),
            "kernel": "skv_attend_sparse step = attend_mfma_kernel<d=128, one 16-row group, sparse> + merge_kernel",
            "algorithmic_bytes_per_launch": sp_bytes,
        },
        "cpu_baseline": {
            "value": round(cpu_us, 1),
            "unit": "us/step",
            "cores": threads,
            "kind": "oracle",
            "sample": f"{reps} fp64 oracle runs of the headline sparse step (32 heads x {rows} kept rows) "
                      f"on one layer, {args.cpu_seconds:.0f} s budget",
            "single_thread_value": round(cpu1_us, 1),
            "dense_step_us": round(cpu_dense_us, 1),
            "score_select_128k_us": cpu_score_select_us,
            "cpu_model": cpu_model,
        },
        "details": details,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
