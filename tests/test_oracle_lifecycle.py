"""Pins of the oracle's rolling-cache lifecycle (oracle/lifecycle.py):
the update rule against a brute-force selection written with plain loops and
exact fractions, its invariants, the special case in which every position
still has a 16-bit row (then it is the detector's plain top-k), and a
scalar step-by-step re-simulation of a tiny lifecycle."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import attention, detect, lifecycle, quant


def _brute_select(scores, old_vl, p0, cand_end, k):
    """Sort (score, position) pairs by hand: larger score first, then lower
    position; keep k; return ascending."""
    cand = [int(x) for x in old_vl] + list(range(p0, cand_end))
    pairs = [(int(scores[c]), c) for c in cand]
    for i in range(len(pairs)):                  # selection sort, no library sort
        best = i
        for j in range(i + 1, len(pairs)):
            sj, pj = pairs[j]
            sb, pb = pairs[best]
            if sj > sb or (sj == sb and pj < pb):
                best = j
        pairs[i], pairs[best] = pairs[best], pairs[i]
    return sorted(p for _, p in pairs[:k])


@pytest.mark.parametrize("seed", range(8))
def test_select_matches_brute_force_with_ties(seed):
    rng = np.random.default_rng(seed)
    n = 200
    scores = rng.integers(-5, 6, n)                         # many equal scores
    p0 = 150
    old = np.sort(rng.choice(p0, 20, replace=False))
    cand_end = 180
    for k in (0, 1, 7, 20, 35, 50):
        got = lifecycle.select(scores, old, p0, cand_end, k)
        assert list(got) == _brute_select(scores, old, p0, cand_end, k)


def test_select_invariants():
    rng = np.random.default_rng(3)
    scores = rng.integers(-1000, 1000, 5000)
    old = np.sort(rng.choice(4000, 250, replace=False))
    got = lifecycle.select(scores, old, 4000, 4064, 250)
    cand = np.concatenate([old, np.arange(4000, 4064)])
    assert len(got) == 250 and np.all(np.diff(got) > 0)
    assert set(got) <= set(cand)                            # nothing without a 16-bit row is promoted
    out = np.setdiff1d(cand, got)
    worst_in = min((scores[j], -j) for j in got)
    best_out = max((scores[j], -j) for j in out)
    assert worst_in > best_out                              # no candidate beats a selected one


def test_select_with_every_row_available_is_the_plain_top_k():
    """When all positions still have 16-bit rows (p0 = 0, no earlier set),
    the update is the detector's top-k over every candidate."""
    rng = np.random.default_rng(11)
    scores = rng.integers(-50, 50, 3000)
    for k in (1, 150, 3000):
        got = lifecycle.select(scores, np.zeros(0, np.int64), 0, 3000, k)
        assert np.array_equal(got, detect.top_k(scores, k))
        assert list(got) == _brute_select(scores, [], 0, 3000, k)


def test_select_rejects_bad_inputs():
    s = np.zeros(100, np.int64)
    with pytest.raises(ValueError):
        lifecycle.select(s, np.array([5, 3]), 50, 60, 2)      # not ascending
    with pytest.raises(ValueError):
        lifecycle.select(s, np.array([55]), 50, 60, 1)        # old position not below p0
    with pytest.raises(ValueError):
        lifecycle.select(s, np.array([1, 2]), 50, 60, 13)     # k > candidates


def _grid(rng, shape, scale=1.0):
    return np.rint(rng.standard_normal(shape) * scale * 16) / 16


def test_tiny_lifecycle_against_a_scalar_re_simulation():
    """B 1, 2 query heads on 1 KV head, D 32 (one group), T0 40, W 4, R 4,
    k 3, 11 steps (two updates). The scalar re-simulation recomputes every
    score as an exact fraction from the dequantized codes, applies the
    update rule by hand and checks the oracle's sets; each step's output is
    the decode oracle with the set in force (checked against it)."""
    rng = np.random.default_rng(5)
    B, Hq, Hkv, D, T0, W, R, k, n = 1, 2, 1, 32, 40, 4, 4, 3, 11
    K = _grid(rng, (B, Hkv, T0 + n, D)).astype(np.float32)
    V = _grid(rng, (B, Hkv, T0 + n, D)).astype(np.float32)
    q = _grid(rng, (n, B, Hq, D)).astype(np.float32)
    vl0 = np.array([[[2, 17, 30]]], dtype=np.int32)
    outs, lses, sets, final = lifecycle.simulate(K, V, q, T0, W, R, k, vl0)
    assert [s for s, _ in sets] == [3, 7]

    # scalar re-simulation of the sets
    codes, s16, z16 = quant.quantize_groups(K[0, 0], 32)
    khat = [[Fraction(int(codes[j, d])) * Fraction(float(s16[j, 0])) + Fraction(float(z16[j, 0]))
             for d in range(D)] for j in range(T0 + n)]
    vl = [2, 17, 30]
    p0 = T0 - W
    ring = {}
    expect_sets = []
    for s in range(n):
        T = T0 + s
        for i in range(Hq):
            ring[(i, s % R)] = [Fraction(float(x)) for x in q[s, 0, i]]
        if s % R == R - 1:
            cand_end = T + 1 - W
            cand = vl + list(range(p0, cand_end))
            sc = {}
            for j in cand:
                sc[j] = sum(sum(row[d] * khat[j][d] for d in range(D)) for row in ring.values())
            ranked = sorted(cand, key=lambda j: (-sc[j], j))
            vl = sorted(ranked[:k])
            p0 = cand_end
            expect_sets.append((s, vl))
    for (s_got, got), (s_want, want) in zip(sets, expect_sets):
        assert s_got == s_want and list(got[0, 0]) == want
    assert list(final[0, 0]) == vl

    # each step's output is the decode oracle over the set in force
    kp, ks = quant.quantize_rows(K[:, :, :T0 + n - W])
    vp, vs = quant.quantize_rows(V[:, :, :T0 + n - W])
    cur = vl0
    upd = dict(sets)
    for s in range(n):
        T = T0 + s
        o, l = attention.decode(q[s], K[:, :, :T], V[:, :, :T], kp[:, :, :T - W], ks[:, :, :T - W],
                                vp[:, :, :T - W], vs[:, :, :T - W], cur, W)
        assert np.allclose(o, outs[s], rtol=0, atol=1e-12) and np.allclose(l, lses[s], rtol=0, atol=1e-12)
        if s in upd:
            cur = upd[s]


def test_lifecycle_promotes_only_rows_that_still_exist():
    """A position that left the window before the previous update and was not
    chosen then can never come back, however large its score becomes."""
    rng = np.random.default_rng(8)
    B, Hq, Hkv, D, T0, W, R, k, n = 1, 1, 1, 32, 30, 2, 2, 2, 6
    K = _grid(rng, (B, Hkv, T0 + n, D), 0.25).astype(np.float32)
    V = _grid(rng, (B, Hkv, T0 + n, D)).astype(np.float32)
    u = np.zeros(D, np.float32)
    u[0] = 1.0
    K[0, 0, 5] = 8.0 * u          # a strong line at position 5, not in the initial set
    q = np.broadcast_to(u, (n, B, Hq, D)).astype(np.float32).copy()
    vl0 = np.array([[[10, 20]]], dtype=np.int32)
    _, _, sets, final = lifecycle.simulate(K, V, q, T0, W, R, k, vl0)
    for _, st in sets:
        assert 5 not in st[0, 0]
    # with every row still 16-bit (the set chosen at the end of prefill), it is found
    kp, ks = quant.quantize_rows(K[0, 0, :T0 - W])
    units, ok = detect.cache_scores(q[0, 0], kp, ks)
    assert ok and 5 in detect.top_k(units, k)
