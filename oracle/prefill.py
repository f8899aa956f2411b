"""Oracle hybrid-precision prefill attention. Test infrastructure only.

[AFS] "The Technical Mechanics", Prefill Stage: the fused operator handles the
quantized majority first and then overlays the high-precision vertical lines
and the local window into the result. [WPN] summary: queries are quantized as
well as keys and values. [KQ] "The abstract": the prefill operator keeps the
vertical-line tokens and a local sliding window in full precision and
quantizes the rest of the context.

Reading used (causal prompt of T tokens, one KV head h with G query heads):
* q_hat, k_hat = INT4 round trip of every query and key row (same quantizer
  as the KV cache: per token, 32-channel groups, fp16 scale and zero);
* logit of query position i and key position j <= i:
    q_i . k_j          if j is a vertical-line position or i - W < j,
    q_hat_i . k_hat_j  otherwise (the quantized majority);
  the overlay replaces the quantized logit by the 16-bit one;
* one causal softmax with scale 1/sqrt(D); values stay 16-bit (P V in the
  input precision).
Everything is float64 after the INT4 round trip.
"""
from __future__ import annotations

import numpy as np

from . import quant


def prefill_rows(q: np.ndarray, K: np.ndarray, V: np.ndarray, vl_idx: np.ndarray,
                 W: int, rows: np.ndarray, sm_scale: float | None = None,
                 group: int = 32):
    """q [Gq][T][D] queries of the group; K, V [T][D]; rows: query positions to
    evaluate. Returns (o [Gq][len(rows)][D], lse [Gq][len(rows)])."""
    Gq, T, D = q.shape
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(D)
    rows = np.asarray(rows, dtype=np.int64)
    kc, ks, kz = quant.quantize_groups(K, group)
    k_hat = quant.dequantize_groups(kc, ks, kz, group)
    Kf = np.asarray(K, dtype=np.float64)
    Vf = np.asarray(V, dtype=np.float64)
    is_vl = np.zeros(T, dtype=bool)
    is_vl[np.asarray(vl_idx, dtype=np.int64)] = True
    o = np.empty((Gq, len(rows), D))
    lse = np.empty((Gq, len(rows)))
    for g in range(Gq):
        qc, qs_, qz = quant.quantize_groups(q[g, rows], group)
        q_hat = quant.dequantize_groups(qc, qs_, qz, group)      # [n][D]
        qf = np.asarray(q[g, rows], dtype=np.float64)
        lq = q_hat @ k_hat.T                                     # quantized majority
        lh = qf @ Kf.T                                           # 16-bit logits
        j = np.arange(T)[None, :]
        i = rows[:, None]
        hp = is_vl[None, :] | (j > i - W)
        logit = np.where(hp, lh, lq) * sm_scale
        logit = np.where(j <= i, logit, -np.inf)                # causal
        m = logit.max(axis=1)
        p = np.exp(logit - m[:, None])
        L = p.sum(axis=1)
        o[g] = (p @ Vf) / L[:, None]
        lse[g] = m + np.log(L)
    return o, lse
