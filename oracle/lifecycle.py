"""Oracle of the rolling hybrid cache over many decode steps. Test
infrastructure only.

[WPN] body paragraph 4: the detector accumulates the decode queries and runs
every 64 tokens. [AFS] "How It Works", items 1-2: the vertical-line tokens
and a recent window (the last W tokens) stay 16-bit, everything older is
4-bit.

Reading (the pages say nothing about what becomes of the 16-bit copies
between detections): a decode-time cache keeps 16-bit rows only for its VL
set and for its window; a window ring with C >= W rows also keeps the rows of
the C - W positions that left the window last. At an update the candidates
are the current VL set and the positions [p0, T - W) that left the window
since the previous update (p0 = T - W of that update); the new set is the k
candidates with the largest column scores, equal scores to the lower
position. Other positions cannot be promoted (their 16-bit rows no longer
exist); dropped VL positions fall back to their INT4 rows, which exist for
every position.

Decode-time scores: the detector's column score of every candidate j,
c_j = sum over the R accumulated queries of every query head of the group of
q . k_j, with k_j the key as the cache holds it for scoring: the INT4 round
trip k_hat_j (``detect.cache_scores``, exact integers). Cadence: step s
appends its query to ring slot s mod R and, when s mod R == R - 1, the update
runs after the step's attention; its set is used from step s + 1 on.

The oracle keeps every 16-bit row (it is the oracle); what the cache holds is
decided by the sets alone.
"""
from __future__ import annotations

import numpy as np

from . import attention, detect, quant


def select(scores: np.ndarray, old_vl: np.ndarray, p0: int, cand_end: int, k: int) -> np.ndarray:
    """The new VL set of one (sequence, KV head): the k best candidates of
    old_vl (ascending, all < p0) and [p0, cand_end) by score (larger first,
    equal scores to the lower position). Returns int32, ascending."""
    old_vl = np.asarray(old_vl, dtype=np.int64)
    if len(old_vl) and (np.any(np.diff(old_vl) <= 0) or old_vl[-1] >= p0):
        raise ValueError("the old VL list must be ascending and below p0")
    cand = np.concatenate([old_vl, np.arange(p0, cand_end, dtype=np.int64)])
    if k > len(cand):
        raise ValueError("k exceeds the number of candidates")
    s = np.asarray(scores)[cand]
    order = np.lexsort((cand, -s))          # primary: score descending; then position ascending
    return np.sort(cand[order[:k]]).astype(np.int32)


def simulate(K: np.ndarray, V: np.ndarray, queries: np.ndarray, T0: int, W: int, R: int, k: int,
             vl0: np.ndarray, group: int = 32):
    """Decode steps s = 0 .. n - 1 of a rolling cache.

    K, V: [B][Hkv][>= T0 + n - 1][D] float32 (exact in the 16-bit dtype): the
    16-bit rows of every position; queries: [n][B][Hq][D] (on the 2**-4 grid,
    for exact scores); T0: context length at step 0 (current token
    included); vl0: [B][Hkv][k] ascending, the set at step 0 (chosen at the
    end of prefill, all below T0 - W).

    Step s has T = T0 + s positions: attention of queries[s] over [0, T)
    with the current set (``attention.decode``), then, when s mod R == R - 1,
    the update over candidates current set + [p0, T + 1 - W).

    Returns (outs [n][B][Hq][D], lses [n][B][Hq], sets: list of (step, set
    [B][Hkv][k]) for each update, final set).
    """
    n = queries.shape[0]
    B, Hkv, _, D = K.shape
    Hq = queries.shape[2]
    G = Hq // Hkv
    T_end = T0 + n
    # the INT4 rows every position gets when it leaves the window (per row,
    # so quantizing all rows at once gives the same codes)
    kp, ks = quant.quantize_rows(K[:, :, :T_end - W], group)
    vp, vs = quant.quantize_rows(V[:, :, :T_end - W], group)
    vl = np.array(vl0, dtype=np.int32)
    p0 = T0 - W
    ring = np.zeros((B, Hq, R, D), dtype=np.float64)
    outs = np.zeros((n, B, Hq, D))
    lses = np.zeros((n, B, Hq))
    sets = []
    for s in range(n):
        T = T0 + s
        nq = T - W
        outs[s], lses[s] = attention.decode(queries[s], K[:, :, :T], V[:, :, :T], kp[:, :, :nq], ks[:, :, :nq],
                                            vp[:, :, :nq], vs[:, :, :nq], vl, W)
        ring[:, :, s % R] = queries[s]
        if s % R == R - 1:
            cand_end = T + 1 - W
            new = np.empty_like(vl)
            for b in range(B):
                for h in range(Hkv):
                    rows = ring[b, h * G:(h + 1) * G].reshape(G * R, D)
                    units, ok = detect.cache_scores(rows, kp[b, h, :cand_end], ks[b, h, :cand_end], group)
                    if not ok:
                        raise ValueError("cache scores outside the exact range")
                    new[b, h] = select(units, vl[b, h], p0, cand_end, k)
            vl = new
            p0 = cand_end
            sets.append((s, vl.copy()))
    return outs, lses, sets, vl
