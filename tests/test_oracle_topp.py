"""Pins of the oracle's SpecVLM selection (Stage I top-P retention, Stage II
uniform reduction; SpecVLM blog, "The SpecVLM Method").

These checks use exact rational arithmetic on the fp32 scores themselves
(fractions.Fraction), closed forms of the special cases and invariants of the
two stages, so a wrong order, a wrong threshold comparison, an off-by-one in
the prefix, a truncated mass or a wrong walk through the leftovers fails one of
them.  Scores spanning far more than 64 bits of dynamic range (down to fp32
subnormals) pin that every positive mass counts exactly."""
from fractions import Fraction

import numpy as np
import pytest

import oracle


def _budget(prune, n_cand):
    """(1 - r) n_cand, product in double, rounded half away from zero (exactly)."""
    return int(Fraction((1.0 - prune) * n_cand) + Fraction(1, 2)) if n_cand else 0


def _pooled_row(rows):
    """The pooled score of every token: the rows added in double, in ascending
    row order, rounded to the nearest fp32 (saturating at the largest fp32)."""
    acc = np.zeros(rows.shape[1], np.float64)
    for r in rows:
        acc = acc + r.astype(np.float64)
    with np.errstate(over="ignore"):
        out = acc.astype(np.float32)
    out[np.isinf(out)] = np.finfo(np.float32).max
    return out


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


def _check(s, n_sink, n_recent, lam, prune, fill_mode=0, pooled=False):
    idx, cnt, cr = oracle.select_topp(s, n_sink, n_recent, lam, prune, fill_mode=fill_mode,
                                      pooled=pooled)
    pooled_want = _brute(_pooled_row(s), n_sink, n_recent, lam, prune, fill_mode) if pooled else None
    for h in range(s.shape[0]):
        want, c = pooled_want or _brute(s[h], n_sink, n_recent, lam, prune, fill_mode)
        assert cr[h] == c
        assert idx[h, :cnt[h]].tolist() == want
    return idx, cnt, cr


def _wide(rng, shape, zeros=0.1):
    """Scores whose binary exponents span about 2^-149 .. 2^20: subnormals,
    tiny normals and ordinary magnitudes in one row."""
    e = rng.integers(-150, 21, shape).astype(np.float64)
    x = rng.random(shape) * np.exp2(e)
    x[rng.random(shape) < zeros] = 0.0
    return x.astype(np.float32)


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


@pytest.mark.parametrize("seed", range(10))
def test_brute_force_wide_dynamic_range(seed):
    """Masses over ~170 binary orders of magnitude: any fixed-point or
    floating-point accumulation that drops low bits picks a different c."""
    rng = np.random.default_rng(100 + seed)
    h, n = 3, int(rng.integers(2, 60))
    s = _wide(rng, (h, n))
    S, R = int(rng.integers(0, 3)), int(rng.integers(0, 4))
    for lam in (float(rng.random()), 0.5, 1.0, 1e-300):
        for mode in (0, 1):
            _check(s, S, R, lam, 0.7, mode)
            _check(s, S, R, lam, 0.7, mode, pooled=True)


def test_lambda_one_keeps_every_positive_mass_down_to_subnormals():
    # one dominant score and masses 2^-70 .. 2^-149 below it: with lambda = 1
    # the prefix reaches the total only once every positive candidate is in
    tiny = [2.0 ** -70, 2.0 ** -100, 2.0 ** -126, 2.0 ** -140, 2.0 ** -149, 0.0, 3 * 2.0 ** -149]
    s = np.array([[1.0] + tiny, tiny + [1.0]], np.float32)
    idx, cnt, cr = oracle.select_topp(s, 0, 0, 1.0, 1.0)
    for h in range(2):
        assert idx[h, :cnt[h]].tolist() == np.flatnonzero(s[h] > 0).tolist()
        assert cr[h] == 7


def test_threshold_just_past_a_prefix_by_a_tiny_mass():
    # masses 1, 1, 2^-90: half the total is 1 + 2^-91, so the first 1.0 alone is
    # short by 2^-91 and Stage I needs both (a 64-bit fixed point at this scale
    # drops 2^-90 and keeps one)
    s = np.array([[1.0, 1.0, 2.0 ** -90]], np.float32)
    _, _, cr = oracle.select_topp(s, 0, 0, 0.5, 1.0)
    assert cr[0] == 2
    # without the tiny mass half the total is exactly the first prefix
    _, _, cr = oracle.select_topp(np.array([[1.0, 1.0, 0.0]], np.float32), 0, 0, 0.5, 1.0)
    assert cr[0] == 1
    # lambda one ulp above 1/2 with total exactly 2: 1 + 2^-52 is not reached by one
    _, _, cr = oracle.select_topp(np.array([[1.0, 1.0]], np.float32), 0, 0, np.nextafter(0.5, 1.0), 1.0)
    assert cr[0] == 2


def test_order_is_by_the_score_not_a_rounded_mass():
    # two masses below 2^-100 that differ by one ulp, behind a mass of 1: the
    # larger (later index) must come first, so lambda just above 1 / (1 + a + b)
    # of the way keeps index 2, not index 1
    a = np.float32(2.0 ** -110)
    b = np.nextafter(a, np.float32(1.0))
    s = np.array([[1.0, a, b]], np.float32)
    total = Fraction(1) + Fraction(float(a)) + Fraction(float(b))
    lam = float((Fraction(1) + Fraction(float(b))) / total)  # rounds near the two-entry prefix
    idx, cnt, cr = oracle.select_topp(s, 0, 0, lam, 1.0)
    want, c = _brute(s[0], 0, 0, lam, 1.0, 0)
    assert cr[0] == c and idx[0, :cnt[0]].tolist() == want
    assert c >= 2 and 2 in idx[0, :cnt[0]].tolist()


def test_pooled_row_is_the_rounded_double_sum():
    # the rows' double sum rounds to fp32 before the rule: 1 + 2^-30 collapses
    # to 1 and ties the next token, which wins by its lower index
    s = np.array([[1.0, 2.0 ** -30, 1.0], [2.0 ** -30, 1.0, 0.0]], np.float32)
    assert _pooled_row(s).tolist() == [1.0, 1.0, 1.0]
    idx, cnt, cr = oracle.select_topp(s, 0, 0, 0.3, 1.0, pooled=True)
    assert cr.tolist() == [1, 1] and idx[0, :cnt[0]].tolist() == [0]
    # saturation at the largest fp32
    big = np.full((2, 3), np.finfo(np.float32).max, np.float32)
    _check(big, 0, 0, 0.5, 0.0, pooled=True)


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


@pytest.mark.parametrize("seed", range(4))
def test_pooled_brute_force(seed):
    rng = np.random.default_rng(200 + seed)
    s = rng.exponential(1.0, (4, int(rng.integers(5, 50)))).astype(np.float32)
    s[rng.random(s.shape) < 0.2] = 0.0
    for lam in (0.3, 0.5, 1.0):
        _check(s, 1, 2, lam, 0.8, 0, pooled=True)


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
