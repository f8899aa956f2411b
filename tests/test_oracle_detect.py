"""Pins for the oracle vertical-line detector (CPU only).

Pinned against: exact rational arithmetic (Python Fractions) on tiny grid
inputs; the linearity identity colsum(Q K^T) == (sum of Q rows) K^T computed
by a different route; a top-k written with Python's sorted(); the defining
property of the selected set; the planted vertical lines of the synthetic
workloads (a check of the data, not of the oracle).
"""
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import detect


def _grid(rng, shape, scale=2.0):
    return np.rint(rng.standard_normal(shape) * scale * 16) / 16


def test_brute_force_fractions():
    rng = np.random.default_rng(1)
    Q = _grid(rng, (6, 8))
    K = _grid(rng, (11, 8))
    units = detect.to_units(detect.column_scores(Q, K))
    for j in range(11):
        c = sum(Fraction(float(Q[r, d])) * Fraction(float(K[j, d]))
                for r in range(6) for d in range(8))
        assert Fraction(int(units[j]), 1 << 16) == c


def test_linearity_identity_exact():
    w = synth.WORKLOADS["glm32k"]
    rng = np.random.default_rng(2)
    Q = synth.round_dtype(rng.standard_normal((1024, 128)) * 1.5 + 0.3, "bf16", grid=True)
    K = synth.keys(w, 0, 0, 4096)
    assert detect.on_grid(Q) and detect.on_grid(K) and detect.exact_bound_ok(Q, K)
    via_matmul = detect.to_units(detect.column_scores(Q, K))
    # different route: sum the query rows first (exact integers), then a GEMV in int64
    qs = np.rint(np.asarray(Q, np.float64) * 16).astype(np.int64).sum(axis=0)
    ki = np.rint(np.asarray(K, np.float64) * 16).astype(np.int64)
    via_gemv = (ki @ qs) << 8            # units of 2**-8 -> 2**-16
    assert np.array_equal(via_matmul, via_gemv)


def _topk_sorted(scores, k):
    order = sorted(range(len(scores)), key=lambda j: (-int(scores[j]), j))
    return sorted(order[:k])


@pytest.mark.parametrize("seed", range(5))
def test_top_k_against_sorted_with_ties(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 3000))
    scores = rng.integers(-20, 20, n).astype(np.int64) * (1 << 12)   # heavy ties
    k = int(rng.integers(0, n + 1))
    got = detect.top_k(scores, k)
    assert got.tolist() == _topk_sorted(scores, k)
    # defining property: nothing outside beats anything inside, ties go low
    sel = np.zeros(n, bool)
    sel[got] = True
    if 0 < k < n:
        lo_in = scores[sel].min()
        assert scores[~sel].max() <= lo_in
        tied_out = np.nonzero(~sel & (scores == lo_in))[0]
        tied_in = np.nonzero(sel & (scores == lo_in))[0]
        if len(tied_out) and len(tied_in):
            assert tied_in.max() < tied_out.min()


def test_top_k_edge_cases():
    assert detect.top_k(np.array([5, 5, 5], np.int64), 0).tolist() == []
    assert detect.top_k(np.array([5, 5, 5], np.int64), 2).tolist() == [0, 1]
    assert detect.top_k(np.array([1, 9, 9, 3], np.int64), 2).tolist() == [1, 2]
    assert detect.top_k(np.array([-1, -2], np.int64), 2).tolist() == [0, 1]
    with pytest.raises(ValueError):
        detect.top_k(np.array([1], np.int64), 2)


def test_units_rounding():
    assert detect.to_units(np.array([1.0, -0.5, 2.0 ** -16, 1.5 * 2.0 ** -16])).tolist() == \
        [65536, -32768, 1, 2]


def test_detect_on_glm_workload_finds_planted_lines():
    """Data check on a slice of the GLM-shaped detector workload: nearly all
    planted positions are selected (alpha = beta = 7 puts a planted score about
    3.5 noise deviations above the rest, so a few percent fall below the top-5 %
    cut), and equal scores occur (so the tie rule is exercised)."""
    wn = synth.WORKLOADS["glm32k"]
    K = synth.all_keys(wn)
    q = synth.all_query_histories(wn)
    idx, sc = detect.detect(q, K, wn.T - wn.W, wn.k)
    planted = synth.planted_positions(wn, 0)
    for h in range(wn.Hkv):
        recall = len(set(planted.tolist()) & set(idx[0, h].tolist())) / len(planted)
        assert recall >= 0.85
        assert np.all(np.diff(idx[0, h]) > 0)
    vals, counts = np.unique(sc[0, 0], return_counts=True)
    assert counts.max() > 1


def test_rejects_non_grid_in_exact_mode():
    q = np.full((1, 2, 1, 4), 0.1)
    K = np.ones((1, 1, 8, 4))
    with pytest.raises(ValueError):
        detect.detect(q, K, 8, 2)
    idx, _ = detect.detect(q, K, 8, 2, require_exact=False)
    assert idx.tolist() == [[[0, 1]]]


def test_cache_scores_brute_force_fractions():
    """The INT4-cache scores against exact rationals: sum over rows and
    channels of q * (c * s + z), rounded to units of 2**-16 half to even."""
    from oracle import quant
    rng = np.random.default_rng(31)
    Q = _grid(rng, (5, 64))
    K = rng.standard_normal((9, 64)).astype(np.float32) * 3
    kp, ks = quant.quantize_rows(K)
    units, ok = detect.cache_scores(Q, kp, ks)
    assert ok
    codes = quant.unpack_nibbles(kp)
    s, z = quant.split_scale_zero(ks)
    for j in range(9):
        c = Fraction(0)
        for d in range(64):
            kh = Fraction(int(codes[j, d])) * Fraction(float(s[j, d // 32])) + Fraction(float(z[j, d // 32]))
            c += sum(Fraction(float(Q[r, d])) for r in range(5)) * kh
        x = c * (1 << 16)
        fl = x.numerator // x.denominator
        rem = x - fl
        want = fl + (1 if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1) else 0)
        assert int(units[j]) == want


def test_cache_scores_equal_fp64_scores_of_dequantized_keys():
    """On grid queries the exact cache scores equal the float64 column scores
    of the dequantized rows (a different route: matmul then column sums)."""
    from oracle import quant
    rng = np.random.default_rng(32)
    Q = _grid(rng, (64, 128), scale=1.0)
    K = (rng.standard_normal((500, 128)) * np.where(rng.random(128) < 0.03, 10, 1)).astype(np.float32)
    kp, ks = quant.quantize_rows(K)
    units, ok = detect.cache_scores(Q, kp, ks)
    assert ok
    ref = detect.to_units(detect.column_scores(Q, quant.dequantize_rows(kp, ks)))
    assert np.array_equal(units, ref)
    idx, _ = detect.detect_cache(Q[None, None], kp[None, None], ks[None, None], 500, 25)
    assert np.array_equal(idx[0, 0], detect.top_k(ref, 25))
    with pytest.raises(ValueError):
        detect.cache_scores(Q + 1e-3, kp, ks)


def test_cache_scores_float_rounds_to_the_exact_scores_and_tracks_fractions_off_grid():
    """The float64 cache scores: on grid queries they round (half to even) to
    the exact integer scores; off the grid (plain draws) they stay within
    1e-6 units of 2**-16 of the exact rational value (scalar brute force on a
    few keys), far below the one-unit rounding of the device's int64 scores."""
    from oracle import quant
    rng = np.random.default_rng(33)
    Qg = _grid(rng, (64, 128), scale=1.0)
    K = (rng.standard_normal((300, 128)) * np.where(rng.random(128) < 0.03, 10, 1)).astype(np.float32)
    kp, ks = quant.quantize_rows(K)
    exact, ok = detect.cache_scores(Qg, kp, ks)
    assert ok
    assert np.array_equal(np.rint(detect.cache_scores_float(Qg, kp, ks)).astype(np.int64), exact)
    Q = rng.standard_normal((6, 64)).astype(np.float32).astype(np.float64)
    kp2, ks2 = quant.quantize_rows(K[:5, :64])
    f = detect.cache_scores_float(Q, kp2, ks2)
    codes = quant.unpack_nibbles(kp2)
    s, z = quant.split_scale_zero(ks2)
    for j in range(5):
        c = Fraction(0)
        for d in range(64):
            kh = Fraction(int(codes[j, d])) * Fraction(float(s[j, d // 32])) + Fraction(float(z[j, d // 32]))
            c += sum(Fraction(float(Q[r, d])) for r in range(6)) * kh
        assert abs(Fraction(float(f[j])) - c * (1 << 16)) < Fraction(1, 10 ** 6)


def test_mass_scores_closed_forms_and_brute_force():
    """Attention-mass scores: every row's probabilities sum to one, so over
    all keys the scores sum to the number of rows; a single key gets every
    row's whole mass; a key shift common to all keys leaves the masses
    unchanged (softmax shift invariance); scalar brute force on a tiny case."""
    import math
    rng = np.random.default_rng(41)
    Q = rng.standard_normal((12, 16))
    K = rng.standard_normal((30, 16))
    c = detect.mass_scores(Q, K, 30)
    assert abs(c.sum() - 12) < 1e-12
    assert abs(detect.mass_scores(Q, K[:1], 1)[0] - 12) < 1e-12
    shift = rng.standard_normal(16)
    # a common shift of the keys moves every logit of a row by the same amount
    c2 = detect.mass_scores(Q, K + shift, 30)
    assert np.max(np.abs(c2 - c)) < 1e-12
    scale = 1 / math.sqrt(16)
    for j in range(0, 30, 7):
        tot = 0.0
        for r in range(12):
            lg = [scale * sum(Q[r, d] * K[i, d] for d in range(16)) for i in range(30)]
            m = max(lg)
            den = sum(math.exp(x - m) for x in lg)
            tot += math.exp(lg[j] - m) / den
        assert abs(c[j] - tot) < 1e-12
    idx, sc = detect.detect_mass(Q[None, None], K[None, None], 25, 5)
    assert np.array_equal(idx[0, 0], detect.top_k(sc[0, 0], 5))
    assert np.max(np.abs(sc[0, 0] - c[:25])) < 1e-15
