"""Byte account of a decode-attention step (host arithmetic only).

The KV read of one layer is ``2 * h_kv * d_h * elem * n`` bytes: keys and values
of every kv head, ``4096 n`` bytes for Llama-3.1-8B in fp16/bf16 ("Where
Activation Sparsity and KV-Cache Sparsity Cross in LLM Decoding", section "The
Byte Crossover").  The same section gives the projection parameter count
``P = 3 d d_ff + 2 d^2 + 2 d h_kv d_h``, the crossover length
``n* = P (1 - r_P) / (2 h_kv d_h (1 - r_KV))`` and the bandwidth-bound speedup
limit ``B / (B - dB)``; the Sparse-to-Dense paper (Sec. 3.3 I/O complexity
analysis) gives the per-token I/O of a draft/verify round.

"Algorithmic bytes" of a call are the bytes the method itself must move:
cache rows it reads, the query, the indices of a kept set, and its outputs.
Scratch traffic (partials, logits, histograms) is excluded, so it counts
against the achieved fraction of the roofline.
"""
from __future__ import annotations

HBM_PEAK_BYTES_PER_S = 8.0e12  # MI355X HBM3E, published peak


def elem_bytes(dtype: str) -> int:
    return {"bf16": 2, "f32": 4}[dtype]


# ---------------------------------------------------------------------------
# the pages' byte account (host formulas, pinned against printed values)
# ---------------------------------------------------------------------------
def kv_bytes_per_layer(n: int, h_kv: int = 8, d_h: int = 128, elem: int = 2) -> int:
    """Bytes of K and V one decode step reads for one layer at context n."""
    return 2 * h_kv * d_h * elem * n


def projection_params(d: int, d_ff: int, h_kv: int = 8, d_h: int = 128) -> int:
    """Parameters of the seven projections of a layer (3 feed-forward, 4 attention)."""
    return 3 * d * d_ff + 2 * d * d + 2 * d * h_kv * d_h


def crossover_tokens(d: int, d_ff: int, r_p: float, r_kv: float, h_kv: int = 8,
                     d_h: int = 128, ff_only: bool = False) -> float:
    """Context length where projection and KV savings are equal (element size cancels)."""
    p = 3 * d * d_ff if ff_only else projection_params(d, d_ff, h_kv, d_h)
    return p * (1.0 - r_p) / (2.0 * h_kv * d_h * (1.0 - r_kv))


def speedup_bound(total_bytes: float, saved_bytes: float) -> float:
    """Upper bound on a bandwidth-bound step's speedup when saved_bytes are skipped."""
    return total_bytes / (total_bytes - saved_bytes)


def std_io_average(gamma: int, k: int, m_t: int, m_v: int, alpha: float) -> float:
    """Per accepted token I/O (in cache entries) of a Sparse-to-Dense round."""
    return (gamma * (k + m_t) + m_v + m_t) / (alpha * gamma)


def std_break_even_alpha(gamma: int, k: int, m_t: int, m_v: int) -> float:
    """Acceptance ratio above which the round reads less than vanilla decoding."""
    return (k + m_t) / (m_v + m_t) + 1.0 / gamma


# ---------------------------------------------------------------------------
# algorithmic bytes of each library call
# ---------------------------------------------------------------------------
def dense_step_bytes(hq: int, hkv: int, d: int, n: int, dtype: str) -> int:
    e = elem_bytes(dtype)
    return 2 * hkv * n * d * e + hq * d * e + hq * d * 4 + hq * 4


def sparse_step_bytes(hq: int, hkv: int, d: int, rows_per_head, n_indexed_per_head,
                      dtype: str) -> int:
    """rows_per_head: kept rows read per kv head (indexed + tail), summed over heads
    if a sequence is given; n_indexed_per_head: how many of them came by index."""
    e = elem_bytes(dtype)
    rows = sum(rows_per_head) if hasattr(rows_per_head, "__iter__") else rows_per_head * hkv
    nidx = (sum(n_indexed_per_head) if hasattr(n_indexed_per_head, "__iter__")
            else n_indexed_per_head * hkv)
    return 2 * rows * d * e + 4 * nidx + 4 * hkv + hq * d * e + hq * d * 4 + hq * 4


def score_bytes(hq: int, hkv: int, d: int, n: int, n_obs: int, dtype: str) -> int:
    """One read of K, the window queries and the fp32 score output."""
    e = elem_bytes(dtype)
    return hkv * n * d * e + n_obs * hq * d * e + hkv * n * 4


def select_bytes(hkv: int, n: int, kept_indices: int) -> int:
    """One read of the score array plus the written indices and counts."""
    return hkv * n * 4 + 4 * kept_indices + 4 * hkv


def verify_bytes(hq: int, hkv: int, d: int, n: int, gamma: int, dtype: str) -> int:
    e = elem_bytes(dtype)
    return 2 * hkv * n * d * e + gamma * hq * d * e + gamma * hq * (d + 1) * 4


def verify_flops(hq: int, n: int, d: int, gamma: int) -> int:
    """q.k and p.v multiply-adds of the causal verify pass (2 flops each)."""
    keys = sum(n - gamma + t + 1 for t in range(gamma))  # keys seen per query head
    return 2 * 2 * hq * d * keys


def obs_score_flops(hq: int, n: int, d: int, n_obs: int) -> int:
    """q.k multiply-adds of the observation-window score: every window row of
    every query head against every key, computed twice (the two passes)."""
    return 2 * 2 * hq * n_obs * n * d


def roofline_fraction(nbytes: float, seconds: float, peak: float = HBM_PEAK_BYTES_PER_S) -> float:
    return nbytes / seconds / peak


# ---------------------------------------------------------------------------
# measured HBM traffic (hardware counters), valid only for unchanged kernels
# ---------------------------------------------------------------------------
# Sources whose change alters what one sparse decode step moves: the split-K
# partial kernels (matrix-core for bf16, vector for fp32), the merge kernel,
# their shared helpers and the host-side planner.
STEP_SOURCES = ("api.hip", "attend.hip", "attend_mfma.hip", "merge.hip", "skv_common.h",
                "skv_kernels.h", "skv_mfma.h", "skv_tile.h")


def step_source_digest() -> str:
    """sha256 (first 16 hex digits) over the step's sources, in STEP_SOURCES order."""
    import hashlib
    import os
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
    h = hashlib.sha256()
    for name in STEP_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counter_traffic(summary_path: str):
    """HBM bytes per step recorded in a counter summary, or None if the summary is
    missing or was taken on other step sources than the ones in the tree.  The
    summary holds the lines `source_sha256: <digest>` and
    `traffic_bytes_per_step: <int>`."""
    import os
    if not os.path.exists(summary_path):
        return None
    fields = {}
    with open(summary_path) as f:
        for line in f:
            key, sep, val = line.strip().strip("`").partition(":")
            if sep:
                fields[key.strip()] = val.strip().strip("`")
    if fields.get("source_sha256") != step_source_digest():
        return None
    try:
        return int(fields["traffic_bytes_per_step"])
    except (KeyError, ValueError):
        return None
