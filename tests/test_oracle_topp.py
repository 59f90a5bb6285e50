"""Pins of the oracle's SpecVLM selection (Stage I top-P retention, Stage II
uniform reduction; SpecVLM blog, "The SpecVLM Method").

The oracle measures mass in exact fixed point; these checks use exact rational
arithmetic on the fp32 scores themselves (fractions.Fraction), closed forms of
the special cases and invariants of the two stages, so a wrong order, a wrong
threshold comparison, an off-by-one in the prefix or a wrong walk through the
leftovers fails one of them."""
from fractions import Fraction

import numpy as np
import pytest

import oracle


def _budget(prune, n_cand):
    """(1 - r) n_cand, product in double, rounded half away from zero (exactly)."""
    return int(Fraction((1.0 - prune) * n_cand) + Fraction(1, 2)) if n_cand else 0


def _brute(row, n_sink, n_recent, lam, prune, fill_mode):
    """Exact-rational definition of one selection (no fixed point)."""
    n = len(row)
    tail = max(n - n_recent, 0)
    sinks = list(range(min(n_sink, tail)))
    cand = list(range(n_sink, n - n_recent)) if n_sink < n - n_recent else []
    a = {j: Fraction(float(row[j])) for j in cand}
    order = sorted(cand, key=lambda j: (-a[j], j))
    total = sum(a.values(), Fraction(0))
    target = Fraction(lam) * total
    c = 0
    while c < len(order) and sum((a[j] for j in order[:c]), Fraction(0)) < target:
        c += 1
    vr = set(order[:c])
    left = [j for j in cand if j not in vr]
    b = _budget(prune, len(cand))
    n_u = min(max(b - c, 0), len(left)) if fill_mode == 0 else min(b, len(left))
    vu = set()
    if n_u:
        interval = Fraction(len(left), n_u)
        vu = {left[int(k * interval)] for k in range(n_u)}
    return sorted(set(sinks) | vr | vu), c


def _check(s, n_sink, n_recent, lam, prune, fill_mode=0):
    idx, cnt, cr = oracle.select_topp(s, n_sink, n_recent, lam, prune, fill_mode=fill_mode)
    for h in range(s.shape[0]):
        want, c = _brute(s[h], n_sink, n_recent, lam, prune, fill_mode)
        assert cr[h] == c
        assert idx[h, :cnt[h]].tolist() == want
    return idx, cnt, cr


def test_hand_worked_example():
    # masses 0.1 0.4 0.2 0.3, lambda 0.5: 0.4 alone is short of half of 1.0,
    # 0.4 + 0.3 reaches it, so V_R = {1, 3}; r = 0.5 keeps 2, so nothing is added
    s = np.array([[0.1, 0.4, 0.2, 0.3]], np.float32)
    idx, cnt, cr = oracle.select_topp(s, 0, 0, 0.5, 0.5)
    assert cr[0] == 2 and idx[0, :cnt[0]].tolist() == [1, 3]
    # r = 0: keep everything (the two leftovers are walked at interval 1)
    idx, cnt, _ = oracle.select_topp(s, 0, 0, 0.5, 0.0)
    assert idx[0, :cnt[0]].tolist() == [0, 1, 2, 3]
    # lambda exactly at a prefix boundary: 0.4 + 0.3 = 0.7 of the mass
    s2 = np.array([[1.0, 4.0, 2.0, 3.0]], np.float32)
    _, _, cr = oracle.select_topp(s2, 0, 0, 0.7, 1.0)
    assert cr[0] == 2
    _, _, cr = oracle.select_topp(s2, 0, 0, np.nextafter(0.7, 1.0), 1.0)
    assert cr[0] == 3


@pytest.mark.parametrize("seed", range(12))
def test_brute_force_tiny(seed):
    rng = np.random.default_rng(seed)
    h, n = 3, int(rng.integers(1, 40))
    s = rng.exponential(1.0, (h, n)).astype(np.float32)
    s[rng.random((h, n)) < 0.2] = 0.0
    S, R = int(rng.integers(0, 4)), int(rng.integers(0, 6))
    lam = float(rng.choice([0.0, 0.3, 0.4, 0.5, 0.9, 1.0]))
    prune = float(rng.choice([0.0, 0.5, 0.9, 1.0]))
    for mode in (0, 1):
        _check(s, S, R, lam, prune, mode)


def test_lambda_zero_is_a_pure_uniform_walk():
    s = np.random.default_rng(1).random((2, 100)).astype(np.float32)
    idx, cnt, cr = oracle.select_topp(s, 0, 0, 0.0, 0.9)
    assert cr.tolist() == [0, 0]
    for h in range(2):
        assert idx[h, :cnt[h]].tolist() == list(range(0, 100, 10))


def test_lambda_one_keeps_every_candidate_with_mass():
    rng = np.random.default_rng(2)
    s = rng.random((2, 500)).astype(np.float32) + 0.01
    s[:, rng.choice(500, 60, replace=False)] = 0.0
    idx, cnt, cr = oracle.select_topp(s, 0, 0, 1.0, 1.0)
    for h in range(2):
        assert idx[h, :cnt[h]].tolist() == np.flatnonzero(s[h] > 0).tolist()


def test_all_zero_scores_and_empty_candidates():
    s = np.zeros((2, 50), np.float32)
    idx, cnt, cr = oracle.select_topp(s, 4, 6, 0.5, 0.5)
    assert cr.tolist() == [0, 0] and cnt.tolist() == [4 + 20] * 2
    # sinks and recent cover everything: only sinks are written
    idx, cnt, cr = oracle.select_topp(np.ones((1, 8), np.float32), 4, 6, 0.5, 0.5, idx_stride=8)
    assert cnt.tolist() == [2] and idx[0, :2].tolist() == [0, 1]


@pytest.mark.parametrize("lam,prune", [(0.4, 0.9), (0.5, 0.9), (0.5, 0.5), (0.9, 0.95)])
def test_stage_invariants_on_attention_like_scores(lam, prune):
    """Heavy-tailed scores (a few planted large entries over a flat floor), the
    shape of verifier attention over video tokens."""
    rng = np.random.default_rng(3)
    n = 3000
    s = (rng.exponential(1e-4, (2, n))).astype(np.float32)
    s[:, rng.choice(n, 40, replace=False)] += rng.exponential(0.01, (2, 40)).astype(np.float32)
    for mode in (0, 1):
        idx, cnt, cr = oracle.select_topp(s, 0, 0, lam, prune, fill_mode=mode)
        b = _budget(prune, n)
        for h in range(2):
            a = [Fraction(float(x)) for x in s[h]]
            order = sorted(range(n), key=lambda j: (-a[j], j))
            total = sum(a, Fraction(0))
            c = int(cr[h])
            vr = order[:c]
            mass = sum((a[j] for j in vr), Fraction(0))
            assert mass >= Fraction(lam) * total
            assert c == 0 or mass - a[vr[-1]] < Fraction(lam) * total
            kept = idx[h, :cnt[h]].tolist()
            assert kept == sorted(kept) and set(vr) <= set(kept)
            left = [j for j in range(n) if j not in set(vr)]
            vu = [r for r, j in enumerate(left) if j in set(kept)]
            want_u = min(max(b - c, 0), len(left)) if mode == 0 else min(b, len(left))
            assert len(vu) == want_u and len(kept) == c + want_u
            if mode == 0:
                assert len(kept) == max(c, b)
            gaps = np.diff(vu)
            if len(gaps):
                lo, hi = len(left) // want_u, -(-len(left) // want_u)
                assert vu[0] == 0 and gaps.min() >= lo and gaps.max() <= hi


def test_pooled_equals_selection_on_the_summed_row():
    # dyadic scores: the row sums are exact in fp32, so pooling is the same as
    # selecting on the summed row
    rng = np.random.default_rng(4)
    s = (rng.integers(0, 64, (4, 700)) / 1024.0).astype(np.float32)
    summed = s.sum(axis=0, dtype=np.float64).astype(np.float32)[None]
    assert np.array_equal(summed[0].astype(np.float64), s.astype(np.float64).sum(axis=0))
    for lam, prune, mode in [(0.4, 0.9, 0), (0.5, 0.8, 1), (1.0, 0.0, 0)]:
        idx, cnt, cr = oracle.select_topp(s, 2, 16, lam, prune, pooled=True, fill_mode=mode)
        ref_i, ref_c, ref_r = oracle.select_topp(summed, 2, 16, lam, prune, fill_mode=mode)
        for h in range(4):
            assert cnt[h] == ref_c[0] and cr[h] == ref_r[0]
            assert np.array_equal(idx[h, :cnt[h]], ref_i[0, :ref_c[0]])


def test_rejects_negative_or_non_finite_scores():
    s = np.ones((1, 10), np.float32)
    s[0, 3] = -1.0
    with pytest.raises(ValueError):
        oracle.select_topp(s, 0, 0, 0.5, 0.5)
    s[0, 3] = np.inf
    with pytest.raises(ValueError):
        oracle.select_topp(s, 0, 0, 0.5, 0.5)
