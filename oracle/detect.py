"""Oracle vertical-line detector. Test infrastructure only.

[WPN] body paragraph 4: the detector accumulates query vectors, runs one
matrix multiplication every 64 tokens and sums the columns of the product.
[HP] technical-approach list: vertical-line tokens are chosen from a
column-wise attention score and make up under 5 % of the tokens.
[AFS] "What to Watch For": the paper keeps the top 5 %.

Reading (the pages give no formula): for one sequence b and KV head h the
rows are the R accumulated decode queries of every query head of the group
(R * G rows); S = Q_acc K^T over the candidate positions [0, cand_end); the
score of position j is the column sum c_j = sum_rows S[row, j] of the raw
logits (a uniform 1/sqrt(D) factor cannot change the ranking); the k positions
with the largest scores are kept, equal scores going to the lower position;
the set is returned in ascending position order.

Scores are reported as int64 in units of 2**-16. When every q and k is a
multiple of 2**-4 (the "grid" inputs of the synthetic workloads) the products
are multiples of 2**-8 and the float64 matmul and column sums are exact as long
as the magnitudes stay below 2**45, which ``column_scores`` asserts; the
conversion to units is then exact too.
"""
from __future__ import annotations

import numpy as np

from . import quant

SCORE_FRAC_BITS = 16


def on_grid(x: np.ndarray, bits: int = 4) -> bool:
    """True when every value is an integer multiple of 2**-bits."""
    y = np.asarray(x, dtype=np.float64) * float(1 << bits)
    return bool(np.all(y == np.rint(y)))


def column_scores(q_rows: np.ndarray, K: np.ndarray) -> np.ndarray:
    """c_j = sum_rows (Q K^T)[row, j], float64 [n]. q_rows [rows][D], K [n][D]."""
    Q = np.asarray(q_rows, dtype=np.float64)
    Kf = np.asarray(K, dtype=np.float64)
    S = Q @ Kf.T                         # the matrix multiplication
    return S.sum(axis=0)                 # the column sums


def exact_bound_ok(q_rows: np.ndarray, K: np.ndarray) -> bool:
    """Sufficient condition for the float64 scores of grid inputs to be exact:
    every partial sum is bounded by sum_rows sum_d |q||k| < 2**45."""
    Qa = np.abs(np.asarray(q_rows, dtype=np.float64)).sum(axis=0)
    Ka = np.abs(np.asarray(K, dtype=np.float64))
    return bool((Ka @ Qa).max(initial=0.0) < 2.0 ** 45)


def to_units(c: np.ndarray) -> np.ndarray:
    """Scores in int64 units of 2**-16, rounded half to even."""
    return np.rint(np.asarray(c, dtype=np.float64) * float(1 << SCORE_FRAC_BITS)).astype(np.int64)


def top_k(scores: np.ndarray, k: int) -> np.ndarray:
    """Positions of the k largest scores, equal scores to the lower position,
    returned ascending (int32)."""
    scores = np.asarray(scores)
    n = len(scores)
    if k > n:
        raise ValueError("k exceeds the number of candidates")
    order = np.lexsort((np.arange(n), -scores))     # primary: score desc; then index asc
    return np.sort(order[:k]).astype(np.int32)


def detect_head(q_rows: np.ndarray, K: np.ndarray, cand_end: int, k: int):
    """One (b, KV head). Returns (idx int32 [k] ascending, scores int64 [cand_end])."""
    c = column_scores(q_rows, K[:cand_end])
    units = to_units(c)
    return top_k(units, k), units


def detect(q_acc: np.ndarray, K: np.ndarray, cand_end: int, k: int, require_exact: bool = True):
    """q_acc [B][Hq][R][D], K [B][Hkv][>=cand_end][D].
    Returns (idx int32 [B][Hkv][k], scores int64 [B][Hkv][cand_end])."""
    B, Hq, R, D = q_acc.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    idx = np.empty((B, Hkv, k), dtype=np.int32)
    sc = np.empty((B, Hkv, cand_end), dtype=np.int64)
    for b in range(B):
        for h in range(Hkv):
            rows = q_acc[b, h * G:(h + 1) * G].reshape(G * R, D)
            Kh = K[b, h, :cand_end]
            if require_exact:
                if not (on_grid(rows) and on_grid(Kh) and exact_bound_ok(rows, Kh)):
                    raise ValueError("exact scores need grid inputs within the magnitude bound")
            idx[b, h], sc[b, h] = detect_head(rows, Kh, cand_end, k)
    return idx, sc


def cache_scores(q_rows: np.ndarray, k_packed: np.ndarray, k_sz: np.ndarray, group: int = 32):
    """Detector variant scored from the INT4 key cache: c_j = (sum_rows q) .
    k_hat_j, k_hat = c * s + z. Exact integer arithmetic: the summed query in
    units of 2**-4 (every q must be a multiple of 2**-4) and k_hat in units of
    2**-24 (fp16 s and z are multiples of 2**-24), so c_j is an integer in
    units of 2**-28. Returns (int64 units of 2**-16 rounded half to even,
    ok) where ok says every |partial sum| stays below 2**53 units, the
    condition under which a float64 evaluation in any order is exact."""
    Q = np.asarray(q_rows, dtype=np.float64)
    if not on_grid(Q):
        raise ValueError("exact cache scores need queries on the 2**-4 grid")
    qs = np.rint(Q * 16.0).astype(np.int64).sum(axis=0)                 # [D], units 2**-4
    codes = quant.unpack_nibbles(k_packed).astype(np.int64)              # [n][D]
    s, z = quant.split_scale_zero(k_sz)                                  # [n][D/group] fp16
    s24 = np.rint(s.astype(np.float64) * 2.0 ** 24).astype(np.int64)
    z24 = np.rint(z.astype(np.float64) * 2.0 ** 24).astype(np.int64)
    kh = codes * np.repeat(s24, group, axis=1) + np.repeat(z24, group, axis=1)   # units 2**-24
    terms_abs = np.abs(kh) @ np.abs(qs)
    ok = bool(terms_abs.max(initial=0) < 2 ** 53)
    x = kh @ qs                                                          # units 2**-28
    # to units of 2**-16: divide by 2**12, round half to even
    qd, r = np.divmod(x, 4096)
    up = (r > 2048) | ((r == 2048) & (qd % 2 == 1))
    return (qd + up).astype(np.int64), ok


def cache_scores_float(q_rows: np.ndarray, k_packed: np.ndarray, k_sz: np.ndarray, group: int = 32):
    """The same column scores for queries off the 2**-4 grid: c_j = (sum_rows
    q) . k_hat_j in float64 (the summed query, the INT4 round trip
    k_hat = c * s + z, one matrix-vector product), in units of 2**-16 and
    not rounded. On the grid it rounds (half to even) to cache_scores."""
    qs = np.asarray(q_rows, dtype=np.float64).sum(axis=0)
    kh = quant.dequantize_rows(k_packed, k_sz, group).astype(np.float64)
    return (kh @ qs) * 65536.0


def detect_cache(q_acc: np.ndarray, k_packed: np.ndarray, k_sz: np.ndarray, cand_end: int, k: int,
                 require_exact: bool = True):
    """The detector scored from the INT4 key cache. q_acc [B][Hq][R][D];
    k_packed [B][Hkv][>=cand_end][D/2]; k_sz [B][Hkv][>=cand_end][D/32][2].
    Returns (idx int32 [B][Hkv][k], scores int64 [B][Hkv][cand_end])."""
    B, Hq, R, D = q_acc.shape
    Hkv = k_packed.shape[1]
    G = Hq // Hkv
    idx = np.empty((B, Hkv, k), dtype=np.int32)
    sc = np.empty((B, Hkv, cand_end), dtype=np.int64)
    for b in range(B):
        for h in range(Hkv):
            rows = q_acc[b, h * G:(h + 1) * G].reshape(G * R, D)
            units, ok = cache_scores(rows, k_packed[b, h, :cand_end], k_sz[b, h, :cand_end])
            if require_exact and not ok:
                raise ValueError("cache scores exceed the exact float64 range")
            sc[b, h] = units
            idx[b, h] = top_k(units, k)
    return idx, sc


def mass_scores(q_rows: np.ndarray, K: np.ndarray, cand_end: int, sm_scale: float | None = None) -> np.ndarray:
    """Detector variant scored by attention mass ([AFS] "What to Watch For":
    the vertical lines are the few tokens holding most of the attention
    mass): p_rho = softmax over all rows of K of sm_scale * q_rho . K^T, and
    c_j = sum over rho of p_rho,j for j in [0, cand_end). float64 [cand_end]."""
    Q = np.asarray(q_rows, dtype=np.float64)
    Kf = np.asarray(K, dtype=np.float64)
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(Q.shape[1])
    L = sm_scale * (Q @ Kf.T)                            # [rows][n]
    P = np.exp(L - L.max(axis=1, keepdims=True))
    P /= P.sum(axis=1, keepdims=True)
    return P[:, :cand_end].sum(axis=0)


def detect_mass(q_acc: np.ndarray, K: np.ndarray, cand_end: int, k: int, sm_scale: float | None = None):
    """q_acc [B][Hq][R][D], K [B][Hkv][k_rows][D] (the softmax runs over all
    k_rows keys). Returns (idx int32 [B][Hkv][k], scores float64 [B][Hkv][cand_end])."""
    B, Hq, R, D = q_acc.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    idx = np.empty((B, Hkv, k), dtype=np.int32)
    sc = np.empty((B, Hkv, cand_end), dtype=np.float64)
    for b in range(B):
        for h in range(Hkv):
            rows = q_acc[b, h * G:(h + 1) * G].reshape(G * R, D)
            sc[b, h] = mass_scores(rows, K[b, h], cand_end, sm_scale)
            idx[b, h] = top_k(sc[b, h], k)
    return idx, sc
