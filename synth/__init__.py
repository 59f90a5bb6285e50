"""Seeded synthetic inputs for the five sparse top-K decode-attention workloads.

This module is shared by the tests, the oracle-side checks and the bench.  It
holds no arithmetic of the method itself (no logits, softmax, selection or
attention): only random draws, bf16 rounding of the drawn values and the
planting rules that give the inputs their structure.

Every stream is ``numpy.random.Generator(PCG64(SeedSequence([workload, tag,
head, trial])))`` so any kv head of any workload can be regenerated on its own.
Values are drawn in fp32 and rounded to bf16 with round-to-nearest-even on the
bit pattern; bf16 tensors are returned as ``uint16`` arrays of raw bits.

Workload shapes follow the pages: Llama-3.1-8B (32 query heads, 8 kv heads,
head dim 128), Qwen2-7B (28/4/128), 196 visual tokens per video frame, four
attention sinks, a 30 % keep ratio, SparseMM's w=32, rho=0.1 and a budget of
256 entries per head.  The benchmark datasets the pages time on are not used;
these draws stand in for them.
"""
from __future__ import annotations

import concurrent.futures as _cf
import math
import os
from dataclasses import dataclass, field

import numpy as np

# stream tags
T_K, T_V, T_Q, T_QOBS, T_NOISE, T_POS, T_HEADSCORE, T_FRAME, T_QDRAFT, T_QVERIFY, T_TOPIC, T_NEW = range(12)


def rng(workload: int, tag: int, head: int = 0, trial: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([workload, tag, head, trial])))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bits, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    t = np.right_shift(u, 16)
    np.bitwise_and(t, 1, out=t)
    t += 0x7FFF
    t += u
    np.right_shift(t, 16, out=t)
    return t.astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bits -> fp32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _unit(x: np.ndarray) -> np.ndarray:
    return (x / np.linalg.norm(x, axis=-1, keepdims=True)).astype(np.float32)


def _pool_map(fn, items):
    workers = min(16, max(1, len(os.sched_getaffinity(0))))
    with _cf.ThreadPoolExecutor(workers) as ex:
        return list(ex.map(fn, items))


@dataclass
class Workload:
    """One synthetic decode-attention problem plus its policy knobs."""
    name: str
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: str                  # "bf16" or "f32"
    n: int                      # cache length the step reads
    k: np.ndarray               # [Hkv][n_cap][d]
    v: np.ndarray               # [Hkv][n_cap][d]
    q: np.ndarray               # decode query [Hq][d]
    q_obs: np.ndarray | None = None   # observation window [W][Hq][d]
    n_sink: int = 0
    n_recent: int = 0
    k_top: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads


def _normal(workload, tag, head, trial, shape, sd=1.0):
    return rng(workload, tag, head, trial).standard_normal(shape, dtype=np.float32) * np.float32(sd)


# ----------------------------------------------------------------------------
# 1. tiny MHA, fp32, per-step top-K
# ----------------------------------------------------------------------------
def tiny_mha(trial: int = 0, n: int = 2048, heads: int = 8, d: int = 64,
             frac_heavy: float = 0.02, k_top: int = 256, n_sink: int = 4,
             n_recent: int = 32) -> Workload:
    """MHA, fp32.  q, K, V ~ N(0,1); round(frac_heavy*n) positions drawn from the
    candidate range get keys 4 q_h/|q_h| + 0.1 N(0, I) in every head."""
    W = 1
    q = _normal(1, T_Q, 0, trial, (heads, d))
    k = np.stack([_normal(1, T_K, h, trial, (n, d)) for h in range(heads)])
    v = np.stack([_normal(1, T_V, h, trial, (n, d)) for h in range(heads)])
    cand = np.arange(n_sink, n - n_recent)
    nh = int(round(frac_heavy * n))
    heavy = np.sort(rng(1, T_POS, 0, trial).choice(cand, size=nh, replace=False))
    qu = _unit(q)
    for h in range(heads):
        noise = _normal(1, T_NOISE, h, trial, (nh, d), 0.1)
        k[h, heavy] = 4.0 * qu[h] + noise
    return Workload("tiny_mha_fp32", heads, heads, d, "f32", n, k, v, q, None,
                    n_sink, n_recent, k_top, {"heavy": heavy, "W": W})


# ----------------------------------------------------------------------------
# 2. Llama-3.1-8B shape at 32K, observation-window selection once (30 % keep)
# ----------------------------------------------------------------------------
def llama_obs(trial: int = 0, n: int = 32768, hq: int = 32, hkv: int = 8, d: int = 128,
              W: int = 32, keep: float = 0.30, n_sink: int = 4, n_recent: int = 64,
              frac_heavy: float = 0.01, layer: int = 0) -> Workload:
    """K, V ~ N(0,1).  Each kv head h has a unit topic u_h; its window and
    decode queries are sqrt(d) u_h + N(0, I).  round(frac_heavy*n) candidate
    positions per kv head get keys 4 u_h + 0.1 N(0, I).  K counts only the
    score-selected entries: floor(keep*n) - sinks - recent."""
    G = hq // hkv
    wl = 2
    topic = np.stack([_unit(_normal(wl, T_TOPIC, h, trial + 1000 * layer, (d,))) for h in range(hkv)])

    k = np.empty((hkv, n, d), np.uint16)
    v = np.empty((hkv, n, d), np.uint16)

    def head_kv(h):
        kh = _normal(wl, T_K, h, trial + 1000 * layer, (n, d))
        cand = np.arange(n_sink, n - n_recent)
        nh = int(round(frac_heavy * n))
        pos = np.sort(rng(wl, T_POS, h, trial + 1000 * layer).choice(cand, size=nh, replace=False))
        kh[pos] = 4.0 * topic[h] + _normal(wl, T_NOISE, h, trial + 1000 * layer, (nh, d), 0.1)
        k[h] = bf16_bits(kh)
        v[h] = bf16_bits(_normal(wl, T_V, h, trial + 1000 * layer, (n, d)))
        return pos

    heavy = _pool_map(head_kv, range(hkv))
    ut = np.repeat(topic, G, axis=0)  # [Hq][d]
    q_obs = math.sqrt(d) * ut[None] + _normal(wl, T_QOBS, 0, trial + 1000 * layer, (W, hq, d))
    q = math.sqrt(d) * ut + _normal(wl, T_Q, 0, trial + 1000 * layer, (hq, d))
    k_top = int(math.floor(keep * n)) - n_sink - n_recent
    return Workload("llama8b_32k_obs", hq, hkv, d, "bf16", n, k, v, bf16_bits(q),
                    bf16_bits(q_obs), n_sink, n_recent, k_top,
                    {"heavy": heavy, "W": W, "keep": keep})


# ----------------------------------------------------------------------------
# 3. Llama-3.1-8B shape at 128K, per-step top-K with a planted needle
# ----------------------------------------------------------------------------
def llama_needle(trial: int = 0, n: int = 131072, hq: int = 32, hkv: int = 8, d: int = 128,
                 k_top: int = 4096, n_sink: int = 4, n_recent: int = 64,
                 needle_pos: int | None = None, layer: int = 0) -> Workload:
    """K, V, q ~ N(0,1).  One needle position p (the same in every kv head) gets
    the key 16 c_h + 0.1 N(0, I), c_h the unit sum of the group's unit queries."""
    G = hq // hkv
    wl = 3
    q = bf16_bits(_normal(wl, T_Q, 0, trial + 1000 * layer, (hq, d)))
    qf = bf16_to_f32(q)
    if needle_pos is None:
        needle_pos = int(rng(wl, T_POS, 0, trial + 1000 * layer).integers(n_sink, n - n_recent))

    k = np.empty((hkv, n, d), np.uint16)
    v = np.empty((hkv, n, d), np.uint16)

    def head_kv(h):
        kh = _normal(wl, T_K, h, trial + 1000 * layer, (n, d))
        c = _unit(_unit(qf[h * G:(h + 1) * G]).sum(axis=0))
        kh[needle_pos] = 16.0 * c + _normal(wl, T_NOISE, h, trial + 1000 * layer, (d,), 0.1)
        k[h] = bf16_bits(kh)
        v[h] = bf16_bits(_normal(wl, T_V, h, trial + 1000 * layer, (n, d)))

    _pool_map(head_kv, range(hkv))
    return Workload("llama8b_128k_needle", hq, hkv, d, "bf16", n, k, v, q, None,
                    n_sink, n_recent, k_top, {"needle": needle_pos, "W": 1})


# ----------------------------------------------------------------------------
# 4. Qwen2-7B video Sparse-to-Dense round
# ----------------------------------------------------------------------------
def qwen_std(trial: int = 0, frames: int = 128, per_frame: int = 196, m_t: int = 512,
             hq: int = 28, hkv: int = 4, d: int = 128, k_top: int = 1024,
             gamma: int = 5) -> Workload:
    """Visual keys of frame f: mu_{h,f} + 0.5 N(0, I), mu_{h,f} ~ N(0, I); text
    keys, values, all queries and the gamma new entries ~ N(0, 1).  The cache
    holds m_v + m_t prompt entries plus room for the gamma drafted entries."""
    wl = 4
    m_v = frames * per_frame
    m = m_v + m_t
    cap = m + gamma

    k = np.empty((hkv, cap, d), np.uint16)
    v = np.empty((hkv, cap, d), np.uint16)

    def head_kv(h):
        mu = _normal(wl, T_FRAME, h, trial, (frames, d))
        kv_vis = np.repeat(mu, per_frame, axis=0) + _normal(wl, T_K, h, trial, (m_v, d), 0.5)
        k_text = _normal(wl, T_K, h + 10_000, trial, (m_t, d))
        k_new = _normal(wl, T_NEW, h, trial, (gamma, d))
        k[h] = bf16_bits(np.concatenate([kv_vis, k_text, k_new]))
        v[h] = bf16_bits(_normal(wl, T_V, h, trial, (cap, d)))

    _pool_map(head_kv, range(hkv))
    q_obs = bf16_bits(_normal(wl, T_QOBS, 0, trial, (m_t, hq, d)))
    q_draft = bf16_bits(_normal(wl, T_QDRAFT, 0, trial, (gamma, hq, d)))
    q_verify = bf16_bits(_normal(wl, T_QVERIFY, 0, trial, (gamma, hq, d)))
    return Workload("qwen2_7b_std_video", hq, hkv, d, "bf16", m, k, v, q_draft[0], q_obs,
                    0, m_t, k_top,
                    {"m_v": m_v, "m_t": m_t, "gamma": gamma, "q_draft": q_draft,
                     "q_verify": q_verify, "W": m_t})


# ----------------------------------------------------------------------------
# 5. SparseMM per-head budgets over 32 layers x 32 heads (flattened)
# ----------------------------------------------------------------------------
def sparsemm_heads(trial: int = 0, layers: int = 32, heads: int = 32, n: int = 32768,
                   d: int = 128, W: int = 32, mean_budget: int = 256, window: int = 32,
                   rho: float = 0.1, frac_visual: float = 0.05, visual_mult: float = 20.0,
                   head_subset=None) -> Workload:
    """MHA, every (layer, head) flattened into one head index.  K, V, q ~ N(0,1)
    per head; head visual scores s ~ Exp(1) with round(frac_visual*N) seeded
    heads scaled by visual_mult.  ``head_subset`` regenerates only those heads
    (K, V, q, q_obs in subset order) for oracle checks on a sample."""
    wl = 5
    N = layers * heads
    s = rng(wl, T_HEADSCORE, 0, trial).exponential(1.0, N)
    vis = rng(wl, T_POS, 0, trial).choice(N, size=int(round(frac_visual * N)), replace=False)
    s[vis] *= visual_mult
    hs = list(range(N)) if head_subset is None else [int(h) for h in head_subset]

    H = len(hs)
    k = np.empty((H, n, d), np.uint16)
    v = np.empty((H, n, d), np.uint16)
    q = np.empty((H, d), np.uint16)
    q_obs = np.empty((W, H, d), np.uint16)

    def head_all(i):
        h = hs[i]
        k[i] = bf16_bits(_normal(wl, T_K, h, trial, (n, d)))
        v[i] = bf16_bits(_normal(wl, T_V, h, trial, (n, d)))
        q[i] = bf16_bits(_normal(wl, T_Q, h, trial, (d,)))
        q_obs[:, i] = bf16_bits(_normal(wl, T_QOBS, h, trial, (W, d)))

    _pool_map(head_all, range(H))
    return Workload("sparsemm_1024heads_32k", len(hs), len(hs), d, "bf16", n, k, v, q, q_obs,
                    0, window, 0,
                    {"head_scores": s, "visual_heads": np.sort(vis), "total_budget": N * mean_budget,
                     "window": window, "rho": rho, "W": W, "heads": np.asarray(hs)})
