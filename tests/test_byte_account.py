"""Pins of the host byte account against figures the pages print."""
import json
import math
import os

import pytest

from sparse_top_kv_amd import roofline as rf

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_kv_bytes_per_layer_matches_page():
    g = _load("bytecross_byte_account.json")
    assert rf.kv_bytes_per_layer(1) == g["layer_kv_bytes_per_token_llama8b"]
    for n, printed, rel in g["layer_kv_bytes"]:
        assert rf.kv_bytes_per_layer(n) == pytest.approx(printed, rel=rel)
    # projection weights of one Llama-3.1-8B layer in a 2-byte format
    assert 2 * rf.projection_params(4096, 14336) == pytest.approx(g["layer_projection_bytes_llama8b_fp16"], rel=0.005)


def test_crossover_table():
    g = _load("bytecross_byte_account.json")
    for row in g["crossover_table"]:
        n_star = rf.crossover_tokens(row["d"], row["d_ff"], 0.5, 0.3) / 1024
        n_ff = rf.crossover_tokens(row["d"], row["d_ff"], 0.5, 0.3, ff_only=True) / 1024
        assert round(n_star, 1) == row["n_star_K"], row["model"]
        assert round(n_ff, 1) == row["n_star_ff_K"], row["model"]
    for row in g["crossing_table_llama8b"]:
        n_star = rf.crossover_tokens(4096, 14336, row["r_p"], row["r_kv"]) / 1024
        assert round(n_star, 1) == row["n_star_K"]


def test_std_io_break_even_is_where_the_round_equals_vanilla():
    g = _load("std_io_and_video_tokens.json")
    for frames, tokens in g["frames_to_tokens"]:
        assert frames * g["tokens_per_frame"] == tokens
    gamma, k, m_t, m_v = 5, 1024, 512, 25088
    a = rf.std_break_even_alpha(gamma, k, m_t, m_v)
    assert rf.std_io_average(gamma, k, m_t, m_v, a) == pytest.approx(m_v + m_t, rel=1e-12)
    assert rf.std_io_average(gamma, k, m_t, m_v, 1.0) < m_v + m_t
    assert rf.std_io_average(gamma, k, m_t, m_v, a * 0.9) > m_v + m_t


def test_step_byte_counts_for_the_llama_shape():
    # dense 32K: 134.2 MB of cache plus the query and outputs
    b = rf.dense_step_bytes(32, 8, 128, 32768, "bf16")
    assert b - rf.kv_bytes_per_layer(32768) == 32 * 128 * 2 + 32 * 129 * 4
    # 30% keep at 32K: 9830 rows per kv head, 9766 of them by index
    s = rf.sparse_step_bytes(32, 8, 128, 9830, 9766, "bf16")
    assert s == 2 * 8 * 9830 * 256 + 4 * 8 * 9766 + 32 + 32 * 256 + 32 * 129 * 4
    assert rf.speedup_bound(b, b - s) == pytest.approx(b / s)


def test_counter_traffic_only_for_unchanged_step_sources(tmp_path):
    """Measured traffic is reported only while the step's kernel sources match the
    digest the counters were taken on."""
    from sparse_top_kv_amd import roofline as rf
    good = tmp_path / "good.md"
    good.write_text(f"# counters\nsource_sha256: `{rf.step_source_digest()}`\n"
                    "traffic_bytes_per_step: `41234567`\n")
    assert rf.counter_traffic(str(good)) == 41234567
    stale = tmp_path / "stale.md"
    stale.write_text("source_sha256: 0123456789abcdef\ntraffic_bytes_per_step: 5\n")
    assert rf.counter_traffic(str(stale)) is None
    assert rf.counter_traffic(str(tmp_path / "missing.md")) is None
