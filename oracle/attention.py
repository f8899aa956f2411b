"""Oracle hybrid-precision decode attention. Test infrastructure only.

What one decode step computes for one sequence b and query head i of KV
head h = i // G ([AFS] "How It Works" and "The Technical Mechanics",
Decode Stage; [KQ] "The abstract", decode sentence):

* three disjoint token sets over positions [0, T):
  Win = [T - W, T), the local window, current token included;
  VL  = the vertical-line positions vl_idx[b, h], all inside [0, T - W);
  Qs  = every other position, held as INT4 codes;
* key/value used at position j: the 16-bit row if j is in VL or Win,
  otherwise the dequantized INT4 row c * s + z (decompressed on the fly);
* one softmax over all T positions with scale sm_scale = 1/sqrt(D) (the
  pages say the 16-bit sets are overlaid into the result; a single softmax
  over the union is the reading that keeps attention well defined);
* output o = sum_j p_j v_j / sum_j p_j and lse = m + ln(sum_j exp(l_j - m)).

Everything is float64. The LSE merge combines partial softmax states of
disjoint chunks of positions; splitting the positions differently must not
change the result beyond float64 rounding.
"""
from __future__ import annotations

import numpy as np

from . import quant


def hybrid_sets(T: int, W: int, vl_idx: np.ndarray):
    """Boolean masks (vl, win, quantized) over positions [0, T)."""
    vl_idx = np.asarray(vl_idx, dtype=np.int64)
    if W < 0 or W > T:
        raise ValueError("window must satisfy 0 <= W <= T")
    if len(vl_idx):
        if np.any(np.diff(vl_idx) <= 0):
            raise ValueError("vl_idx must be strictly ascending")
        if vl_idx[0] < 0 or vl_idx[-1] >= T - W:
            raise ValueError("vl_idx must lie in [0, T - W)")
    vl = np.zeros(T, dtype=bool)
    vl[vl_idx] = True
    win = np.zeros(T, dtype=bool)
    win[T - W:] = True
    qs = ~(vl | win)
    return vl, win, qs


def hybrid_rows(X_hp: np.ndarray, packed: np.ndarray, sz: np.ndarray,
                vl_idx: np.ndarray, W: int, group: int = 32) -> np.ndarray:
    """Rows actually attended to, float64 [T][D]: 16-bit rows on VL and Win,
    dequantized INT4 rows elsewhere. ``packed``/``sz`` cover at least the
    positions [0, T - W)."""
    T, D = X_hp.shape
    vl, win, qs = hybrid_sets(T, W, vl_idx)
    out = np.empty((T, D), dtype=np.float64)
    hp = vl | win
    out[hp] = np.asarray(X_hp, dtype=np.float64)[hp]
    nq = T - W
    deq = quant.dequantize_rows(packed[:nq], sz[:nq], group)
    sel = qs[:nq]
    out[:nq][sel] = deq[sel]
    return out


def softmax_state(logits: np.ndarray, V: np.ndarray):
    """Partial softmax state of one chunk: (m, L, o) with o normalised,
    for logits [H][n] and values [n][D]. An empty chunk gives m = -inf."""
    H = logits.shape[0]
    if logits.shape[1] == 0:
        return np.full(H, -np.inf), np.zeros(H), np.zeros((H, V.shape[1]))
    m = logits.max(axis=1)
    p = np.exp(logits - m[:, None])
    L = p.sum(axis=1)
    o = (p @ V) / L[:, None]
    return m, L, o


def lse_merge(states):
    """Merge partial states (m_c, L_c, o_c) of disjoint chunks:
    m* = max m_c, L* = sum exp(m_c - m*) L_c, o* = sum exp(m_c - m*) L_c o_c / L*."""
    ms = np.stack([s[0] for s in states])          # [C][H]
    Ls = np.stack([s[1] for s in states])
    os_ = np.stack([s[2] for s in states])         # [C][H][D]
    m = ms.max(axis=0)
    with np.errstate(invalid="ignore"):
        wgt = np.where(np.isfinite(ms), np.exp(ms - m[None]), 0.0) * Ls
    L = wgt.sum(axis=0)
    o = (wgt[..., None] * os_).sum(axis=0) / L[:, None]
    return m, L, o


def attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, sm_scale: float | None = None):
    """Textbook softmax attention in float64: q [H][D], K, V [T][D].
    Returns (o [H][D], lse [H])."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(q.shape[-1])
    logits = sm_scale * (q @ K.T)
    m, L, o = softmax_state(logits, V)
    return o, m + np.log(L)


def decode_head(q: np.ndarray, K_hp: np.ndarray, V_hp: np.ndarray,
                k_packed: np.ndarray, k_sz: np.ndarray,
                v_packed: np.ndarray, v_sz: np.ndarray,
                vl_idx: np.ndarray, W: int, sm_scale: float | None = None,
                group: int = 32):
    """One (b, KV head): q [G][D] query heads of the group; K_hp, V_hp [T][D]
    the 16-bit rows; INT4 planes for positions [0, T - W). Returns
    (o [G][D], lse [G])."""
    Kt = hybrid_rows(K_hp, k_packed, k_sz, vl_idx, W, group)
    Vt = hybrid_rows(V_hp, v_packed, v_sz, vl_idx, W, group)
    return attention(q, Kt, Vt, sm_scale)


def decode_sparse_head(q: np.ndarray, K_hp: np.ndarray, V_hp: np.ndarray,
                       vl_idx: np.ndarray, W: int, sm_scale: float | None = None):
    """The sparse baseline of the ablation ([MR] "Improvements and Ablation
    Studies", Table 12: dropping the long tail that the hybrid cache keeps in
    low precision): one softmax over the VL and window positions only, the
    quantized set Qs left out. q [G][D], K_hp, V_hp [T][D]. Returns
    (o [G][D], lse [G])."""
    T = K_hp.shape[0]
    vl, win, _ = hybrid_sets(T, W, vl_idx)
    keep = vl | win
    return attention(q, np.asarray(K_hp)[keep], np.asarray(V_hp)[keep], sm_scale)


def decode(q: np.ndarray, K_hp: np.ndarray, V_hp: np.ndarray,
           k_packed: np.ndarray, k_sz: np.ndarray,
           v_packed: np.ndarray, v_sz: np.ndarray,
           vl_idx: np.ndarray, W: int, sm_scale: float | None = None,
           group: int = 32, units=None):
    """Batched decode step.

    q [B][Hq][D]; K_hp, V_hp [B][Hkv][T][D]; packed codes [B][Hkv][>=T-W][D/2];
    sz [B][Hkv][>=T-W][D/group][2]; vl_idx [B][Hkv][k].
    ``units``: optional list of (b, h) to compute (others are left NaN).
    Returns (o [B][Hq][D], lse [B][Hq]) in float64.
    """
    B, Hq, D = q.shape
    Hkv = K_hp.shape[1]
    G = Hq // Hkv
    o = np.full((B, Hq, D), np.nan)
    lse = np.full((B, Hq), np.nan)
    if units is None:
        units = [(b, h) for b in range(B) for h in range(Hkv)]
    for b, h in units:
        sl = slice(h * G, (h + 1) * G)
        o[b, sl], lse[b, sl] = decode_head(
            q[b, sl], K_hp[b, h], V_hp[b, h], k_packed[b, h], k_sz[b, h],
            v_packed[b, h], v_sz[b, h], vl_idx[b, h], W, sm_scale, group)
    return o, lse
