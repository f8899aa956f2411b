"""Pins for the oracle hybrid decode attention (CPU only).

Pinned against: textbook attention and torch's scaled_dot_product_attention
in float64 when no position is quantized; plain attention over dequantized
rows when no position is 16-bit; scalar brute force on tiny inputs; LSE-merge
invariance under random splits; insensitivity to the INT4 rows of VL
positions; GQA as repeated-KV multi-head attention.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention, quant


def _case(rng, T, D=64, G=4, W=8, k=3, scale=1.0):
    q = rng.standard_normal((G, D)).astype(np.float32)
    K = (rng.standard_normal((T, D)) * scale).astype(np.float32)
    V = rng.standard_normal((T, D)).astype(np.float32)
    kp, ks = quant.quantize_rows(K[:T - W])
    vp, vs = quant.quantize_rows(V[:T - W])
    vl = np.sort(rng.choice(T - W, size=k, replace=False)).astype(np.int32) if k else np.zeros(0, np.int32)
    return q, K, V, kp, ks, vp, vs, vl


def test_all_window_equals_exact_attention():
    rng = np.random.default_rng(1)
    T, D = 200, 64
    q, K, V, _, _, _, _, _ = _case(rng, T, D, W=T, k=0)
    empty_p = np.zeros((0, D // 2), np.uint8)
    empty_s = np.zeros((0, D // 32, 2), np.uint16)
    o, lse = attention.decode_head(q, K, V, empty_p, empty_s, empty_p, empty_s,
                                   np.zeros(0, np.int32), W=T)
    # textbook
    lg = (q.astype(np.float64) @ K.astype(np.float64).T) / math.sqrt(D)
    p = np.exp(lg - lg.max(1, keepdims=True))
    ref = (p / p.sum(1, keepdims=True)) @ V.astype(np.float64)
    assert np.max(np.abs(o - ref)) < 1e-12
    # library routine
    t = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q.astype(np.float64))[None, :, None, :],
        torch.from_numpy(K.astype(np.float64))[None, None].expand(1, q.shape[0], T, D),
        torch.from_numpy(V.astype(np.float64))[None, None].expand(1, q.shape[0], T, D))
    assert np.max(np.abs(o - t[0, :, 0].numpy())) < 1e-12
    ref_lse = np.log(np.exp(lg).sum(1))
    assert np.max(np.abs(lse - ref_lse)) < 1e-12


def test_no_hp_rows_equals_attention_over_dequantized():
    rng = np.random.default_rng(2)
    T, D = 150, 64
    q, K, V, kp, ks, vp, vs, _ = _case(rng, T, D, W=0, k=0)
    o, _ = attention.decode_head(q, K, V, kp, ks, vp, vs, np.zeros(0, np.int32), W=0)
    # dequantize independently from the packed bytes
    def deq(packed, sz):
        out = np.empty((T, D))
        for t in range(T):
            for d in range(D):
                byte = int(packed[t, d // 2])
                c = (byte >> 4) if d % 2 else (byte & 15)
                s = float(np.uint16(sz[t, d // 32, 0]).view(np.float16))
                z = float(np.uint16(sz[t, d // 32, 1]).view(np.float16))
                out[t, d] = c * s + z
        return out
    Kh, Vh = deq(kp, ks), deq(vp, vs)
    t = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q.astype(np.float64))[None, :, None, :],
        torch.from_numpy(Kh)[None, None].expand(1, q.shape[0], T, D),
        torch.from_numpy(Vh)[None, None].expand(1, q.shape[0], T, D))
    assert np.max(np.abs(o - t[0, :, 0].numpy())) < 1e-12


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_tiny(seed):
    rng = np.random.default_rng(100 + seed)
    T = int(rng.integers(4, 17))
    W = int(rng.integers(0, T + 1))
    k = int(rng.integers(0, T - W + 1))
    D = 32
    q, K, V, kp, ks, vp, vs, vl = _case(rng, T, D, G=2, W=W, k=k)
    o, lse = attention.decode_head(q, K, V, kp, ks, vp, vs, vl, W)
    vls = set(int(v) for v in vl)
    for g in range(2):
        logits, rows = [], []
        for j in range(T):
            if j in vls or j >= T - W:
                kr = [float(v) for v in K[j]]
                vr = [float(v) for v in V[j]]
            else:
                kr, vr = [], []
                for d in range(D):
                    sh = 4 if d % 2 else 0
                    s_k = float(np.uint16(ks[j, 0, 0]).view(np.float16))
                    z_k = float(np.uint16(ks[j, 0, 1]).view(np.float16))
                    s_v = float(np.uint16(vs[j, 0, 0]).view(np.float16))
                    z_v = float(np.uint16(vs[j, 0, 1]).view(np.float16))
                    kr.append(((int(kp[j, d // 2]) >> sh) & 15) * s_k + z_k)
                    vr.append(((int(vp[j, d // 2]) >> sh) & 15) * s_v + z_v)
            logits.append(sum(float(q[g, d]) * kr[d] for d in range(D)) / math.sqrt(D))
            rows.append(vr)
        m = max(logits)
        w = [math.exp(x - m) for x in logits]
        L = sum(w)
        ref = [sum(w[j] * rows[j][d] for j in range(T)) / L for d in range(D)]
        assert np.max(np.abs(o[g] - np.array(ref))) < 1e-12
        assert abs(lse[g] - (m + math.log(L))) < 1e-12


def test_lse_merge_invariance():
    rng = np.random.default_rng(3)
    T, D, W = 700, 64, 40
    q, K, V, kp, ks, vp, vs, vl = _case(rng, T, D, W=W, k=20, scale=3.0)
    o_ref, lse_ref = attention.decode_head(q, K, V, kp, ks, vp, vs, vl, W)
    Kt = attention.hybrid_rows(K, kp, ks, vl, W)
    Vt = attention.hybrid_rows(V, vp, vs, vl, W)
    lg = (q.astype(np.float64) @ Kt.T) / math.sqrt(D)
    for trial in range(20):
        n_cut = int(rng.integers(1, 30))
        cuts = np.sort(rng.choice(np.arange(0, T + 1), size=n_cut, replace=True))
        edges = np.concatenate([[0], cuts, [T]])
        states = [attention.softmax_state(lg[:, a:b], Vt[a:b]) for a, b in zip(edges[:-1], edges[1:])]
        perm = rng.permutation(len(states))            # merge order must not matter
        m, L, o = attention.lse_merge([states[i] for i in perm])
        assert np.max(np.abs(o - o_ref)) <= 1e-12 * max(1.0, np.abs(o_ref).max())
        assert np.max(np.abs(m + np.log(L) - lse_ref)) < 1e-12


def test_poisoned_vl_codes_do_not_matter():
    rng = np.random.default_rng(4)
    T, D, W = 300, 64, 16
    q, K, V, kp, ks, vp, vs, vl = _case(rng, T, D, W=W, k=12)
    o1, _ = attention.decode_head(q, K, V, kp, ks, vp, vs, vl, W)
    kp2, vp2, ks2, vs2 = kp.copy(), vp.copy(), ks.copy(), vs.copy()
    kp2[vl] = rng.integers(0, 256, kp2[vl].shape, dtype=np.uint8)
    vp2[vl] = rng.integers(0, 256, vp2[vl].shape, dtype=np.uint8)
    ks2[vl] = np.float16(7.0).view(np.uint16)
    vs2[vl] = np.float16(-3.0).view(np.uint16)
    o2, _ = attention.decode_head(q, K, V, kp2, ks2, vp2, vs2, vl, W)
    assert np.array_equal(o1, o2)
    # ... while the same garbage at a quantized position does change the output
    j = next(i for i in range(T - W) if i not in set(vl.tolist()))
    kp2, vp2 = kp.copy(), vp.copy()
    vp2[j] ^= 0xFF
    kp2[j] ^= 0xFF
    o3, _ = attention.decode_head(q, K, V, kp2, ks, vp2, vs, vl, W)
    assert np.max(np.abs(o3 - o1)) > 1e-6


def test_window_uses_16bit_rows_including_current_token():
    rng = np.random.default_rng(9)
    T, D, W = 100, 64, 10
    q, K, V, kp, ks, vp, vs, vl = _case(rng, T, D, W=W, k=5)
    o1, _ = attention.decode_head(q, K, V, kp, ks, vp, vs, vl, W)
    V2 = V.copy()
    V2[T - 1] += 1.0                                   # the current token's value
    o2, _ = attention.decode_head(q, K, V2, kp, ks, vp, vs, vl, W)
    assert np.max(np.abs(o2 - o1)) > 1e-6
    V3 = V.copy()
    V3[[j for j in range(T - W) if j not in set(vl.tolist())][:5]] += 1.0   # hp rows not used there
    o3, _ = attention.decode_head(q, K, V3, kp, ks, vp, vs, vl, W)
    assert np.array_equal(o1, o3)


def test_permutation_invariance():
    rng = np.random.default_rng(10)
    T, D = 120, 64
    q = rng.standard_normal((3, D))
    K = rng.standard_normal((T, D))
    V = rng.standard_normal((T, D))
    o, lse = attention.attention(q, K, V)
    perm = rng.permutation(T)
    o2, lse2 = attention.attention(q, K[perm], V[perm])
    assert np.max(np.abs(o - o2)) < 1e-13 and np.max(np.abs(lse - lse2)) < 1e-13


def test_gqa_is_repeated_kv():
    rng = np.random.default_rng(11)
    B, Hkv, G, T, D, W, k = 2, 2, 3, 90, 64, 9, 4
    q = rng.standard_normal((B, Hkv * G, D)).astype(np.float32)
    K = rng.standard_normal((B, Hkv, T, D)).astype(np.float32)
    V = rng.standard_normal((B, Hkv, T, D)).astype(np.float32)
    kp, ks = quant.quantize_rows(K[:, :, :T - W])
    vp, vs = quant.quantize_rows(V[:, :, :T - W])
    vl = np.stack([np.stack([np.sort(rng.choice(T - W, k, replace=False)) for _ in range(Hkv)])
                   for _ in range(B)]).astype(np.int32)
    o, lse = attention.decode(q, K, V, kp, ks, vp, vs, vl, W)
    for b in range(B):
        for i in range(Hkv * G):
            h = i // G
            oi, li = attention.decode_head(q[b, i:i + 1], K[b, h], V[b, h], kp[b, h], ks[b, h],
                                           vp[b, h], vs[b, h], vl[b, h], W)
            assert np.array_equal(oi[0], o[b, i]) or np.max(np.abs(oi[0] - o[b, i])) < 1e-14


def test_set_validation():
    with pytest.raises(ValueError):
        attention.hybrid_sets(10, 3, np.array([2, 2]))
    with pytest.raises(ValueError):
        attention.hybrid_sets(10, 3, np.array([7]))       # inside the window
    vl, win, qs = attention.hybrid_sets(10, 3, np.array([0, 4]))
    assert vl.sum() == 2 and win.sum() == 3 and qs.sum() == 5
    assert not np.any(vl & win) and not np.any(vl & qs) and not np.any(win & qs)


def test_sparse_baseline_window_only_is_sdpa_over_the_window():
    """k = 0: the sparse baseline is attention over the last W rows (a
    library routine, float64)."""
    rng = np.random.default_rng(21)
    T, D, W = 150, 64, 24
    q, K, V, _, _, _, _, _ = _case(rng, T, D, W=W, k=0)
    o, lse = attention.decode_sparse_head(q, K, V, np.zeros(0, np.int32), W)
    t = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q.astype(np.float64))[None, :, None, :],
        torch.from_numpy(K[T - W:].astype(np.float64))[None, None].expand(1, q.shape[0], W, D),
        torch.from_numpy(V[T - W:].astype(np.float64))[None, None].expand(1, q.shape[0], W, D))
    assert np.max(np.abs(o - t[0, :, 0].numpy())) < 1e-12
    lg = (q.astype(np.float64) @ K[T - W:].astype(np.float64).T) / math.sqrt(D)
    assert np.max(np.abs(lse - np.log(np.exp(lg).sum(1)))) < 1e-12


def test_sparse_baseline_brute_force_and_merge_identity():
    """Scalar brute force over the VL and window positions; and merging the
    sparse state with the state of the quantized set alone gives the hybrid
    step (the sets are disjoint and cover [0, T))."""
    rng = np.random.default_rng(22)
    T, D, W, k = 40, 32, 6, 5
    q, K, V, kp, ks, vp, vs, vl = _case(rng, T, D, G=2, W=W, k=k)
    o, lse = attention.decode_sparse_head(q, K, V, vl, W)
    keep = sorted(set(int(j) for j in vl) | set(range(T - W, T)))
    for g in range(q.shape[0]):
        lg = [sum(float(q[g, d]) * float(K[j, d]) for d in range(D)) / math.sqrt(D) for j in keep]
        m = max(lg)
        e = [math.exp(x - m) for x in lg]
        L = sum(e)
        for d in range(D):
            ref = sum(e[i] * float(V[j, d]) for i, j in enumerate(keep)) / L
            assert abs(o[g, d] - ref) < 1e-12
        assert abs(lse[g] - (m + math.log(L))) < 1e-12
    # merge identity with the quantized set
    _, _, qs = attention.hybrid_sets(T, W, vl)
    Kq = quant.dequantize_rows(kp, ks)[qs[:T - W]]
    Vq = quant.dequantize_rows(vp, vs)[qs[:T - W]]
    scale = 1.0 / math.sqrt(D)
    sk = K[np.array(keep)].astype(np.float64)
    sv = V[np.array(keep)].astype(np.float64)
    oh, lh = attention.decode_head(q, K, V, kp, ks, vp, vs, vl, W)
    for g in range(q.shape[0]):
        st_s = attention.softmax_state(scale * (sk @ q[g].astype(np.float64))[None], sv)
        st_q = attention.softmax_state(scale * (Kq @ q[g].astype(np.float64))[None], Vq)
        m, L, om = attention.lse_merge([st_s, st_q])
        assert np.max(np.abs(om[0] - oh[g])) < 1e-12
        assert abs(m[0] + math.log(L[0]) - lh[g]) < 1e-12
