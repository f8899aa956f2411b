"""Pins for the oracle hybrid prefill operator (CPU only): a window covering
the whole prefix reduces it to causal attention (checked against torch's
float64 SDPA); scalar brute force on tiny prompts; the overlay of a
vertical-line column replaces exactly that column's logits."""
import math

import numpy as np
import torch

from oracle import prefill, quant


def _qkv(rng, G, T, D):
    q = rng.standard_normal((G, T, D)).astype(np.float32)
    K = rng.standard_normal((T, D)).astype(np.float32)
    V = rng.standard_normal((T, D)).astype(np.float32)
    return q, K, V


def test_full_window_is_causal_attention():
    rng = np.random.default_rng(0)
    G, T, D = 2, 60, 64
    q, K, V = _qkv(rng, G, T, D)
    rows = np.arange(T)
    o, lse = prefill.prefill_rows(q, K, V, np.zeros(0, np.int64), W=T, rows=rows)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q.astype(np.float64))[None],
        torch.from_numpy(K.astype(np.float64))[None, None].expand(1, G, T, D),
        torch.from_numpy(V.astype(np.float64))[None, None].expand(1, G, T, D), is_causal=True)
    assert np.max(np.abs(o - ref[0].numpy())) < 1e-12


def test_brute_force_tiny():
    rng = np.random.default_rng(1)
    G, T, D, W = 1, 12, 32, 3
    q, K, V = _qkv(rng, G, T, D)
    vl = np.array([1, 4])
    o, lse = prefill.prefill_rows(q, K, V, vl, W=W, rows=np.arange(T))

    def rt(x):   # INT4 round trip written out per element
        mn, mx = float(np.min(x)), float(np.max(x))
        s = float(np.float16(np.float32(np.float32(mx) - np.float32(mn)) / np.float32(15)))
        z = float(np.float16(np.float32(mn)))
        out = []
        for v in x:
            c = 0 if s == 0 else min(15, max(0, int(np.rint(np.float32(np.float32(v) - np.float32(z)) / np.float32(s)))))
            out.append(c * s + z)
        return out
    for i in range(T):
        qh = rt(q[0, i])
        lg = []
        for j in range(i + 1):
            if j in (1, 4) or j > i - W:
                lg.append(sum(float(q[0, i, d]) * float(K[j, d]) for d in range(D)))
            else:
                kh = rt(K[j])
                lg.append(sum(qh[d] * kh[d] for d in range(D)))
        lg = [x / math.sqrt(D) for x in lg]
        m = max(lg)
        w = [math.exp(x - m) for x in lg]
        ref = [sum(w[j] * float(V[j, d]) for j in range(i + 1)) / sum(w) for d in range(D)]
        assert np.max(np.abs(o[0, i] - np.array(ref))) < 1e-12


def test_overlay_touches_only_vl_columns():
    rng = np.random.default_rng(2)
    G, T, D, W = 2, 80, 64, 4
    q, K, V = _qkv(rng, G, T, D)
    rows = np.array([40, 79])
    o0, _ = prefill.prefill_rows(q, K, V, np.zeros(0, np.int64), W, rows)
    o1, _ = prefill.prefill_rows(q, K, V, np.array([10]), W, rows)
    assert np.max(np.abs(o1 - o0)) > 1e-9
    # a VL column after the query row is masked anyway
    o2, _ = prefill.prefill_rows(q, K, V, np.array([60]), W, np.array([40]))
    o3, _ = prefill.prefill_rows(q, K, V, np.zeros(0, np.int64), W, np.array([40]))
    assert np.array_equal(o2, o3)
