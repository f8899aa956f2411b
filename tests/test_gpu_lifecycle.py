"""GPU parity of the rolling hybrid cache over many decode steps against the
oracle's lifecycle simulation (oracle/lifecycle.py): 130 decode steps
crossing two re-detections, through the fused re-detection (hq_vl_redetect)
and through the detector's scores then hq_vl_update. Each step's attention
output within the decode bar; every re-detected VL set bit-exact; at the end
the INT4 planes written by the per-step eviction, the VL rows and the VL
bitmap bit-exact. hq_vl_update alone on constructed scores, and
hq_vl_redetect against the two-call path bit for bit."""
import numpy as np
import pytest
import torch

import hybrid_precision_quantized_amd as hq
import synth
from oracle import detect, lifecycle, quant
from tests.gpu_util import TORCH_DT, rel_err, say, tile16_codes, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("B,Hq,Hkv,D,T0,W,k,R,n,dtype", [
    (1, 8, 2, 128, 700, 32, 35, 64, 130, "bf16"),     # G = 4: the matrix-core INT4 pass
    (2, 4, 2, 64, 500, 16, 25, 16, 40, "f16"),        # D = 64, G = 2, a short ring (R = 16)
])
def test_rolling_cache_matches_oracle_lifecycle(B, Hq, Hkv, D, T0, W, k, R, n, dtype, fused):
    w = synth.Workload(f"life{T0}", 9100 + T0, B=B, Hq=Hq, Hkv=Hkv, D=D, T=T0 + n, W=W, k=k, dtype=dtype,
                       R=R, n_plant=max(2, int(0.02 * (T0 + n))))
    say(f"lifecycle B={B} Hq={Hq} Hkv={Hkv} D={D} T0={T0} W={W} k={k} R={R} steps={n} {dtype} fused={fused}")
    K, V = synth.all_keys(w), synth.all_values(w)                   # every position's 16-bit rows
    queries = np.stack([synth.all_queries(w.replace(seed=w.seed + 101 * (s + 1))) for s in range(n)])
    assert detect.on_grid(queries)                                   # exact detector scores
    # the set chosen at the end of prefill: the detector over the last R prompt queries
    qh = synth.all_query_histories(w)
    vl0, _ = detect.detect(qh, K[:, :, :T0], T0 - W, k)
    say("  oracle lifecycle ...")
    outs, lses, sets, final = lifecycle.simulate(K, V, queries, T0, W, R, k, vl0)
    changed = sum(len(np.setxor1d(a[1][0, 0], b[0, 0])) for a, b in zip(sets, [vl0] + [s[1] for s in sets]))
    say(f"  oracle: {len(sets)} updates, {changed} set changes in unit (0, 0)")

    dt = TORCH_DT[dtype]
    Kd, Vd = to_dev(K, dtype), to_dev(V, dtype)
    t_cap = ((T0 + n - W + 1) + 31) // 32 * 32
    rc = hq.RollingCache(B, Hkv, D, T0, W, k, dt, Hq, R=R, t_cap=t_cap)
    rc.build(Kd[:, :, :T0].contiguous(), Vd[:, :, :T0].contiguous(), torch.from_numpy(vl0).cuda())
    ws = torch.full((hq.hq_decode_workspace_size(rc.descriptor(), Hq, 0) * 2,), 0xFF, dtype=torch.uint8,
                    device="cuda")
    out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    worst = 0.0
    got_sets = []
    for s in range(n):
        rc.decode_step(to_dev(queries[s], dtype), out, lse, ws)
        o, l = out.cpu().numpy(), lse.cpu().numpy()
        e = rel_err(o, outs[s])
        worst = max(worst, e)
        assert e <= 2e-3 and np.max(np.abs(l - lses[s])) <= 1e-3, (s, e)
        rc.advance(Kd[:, :, T0 + s], Vd[:, :, T0 + s])
        if rc.due():
            rc.redetect(fused=fused)
            got_sets.append((s, np.sort(rc.vl_idx[..., :k].cpu().numpy(), axis=-1)))
    torch.cuda.synchronize()
    say(f"  worst step max|err|/rms = {worst:.3e}")
    assert [s for s, _ in got_sets] == [s for s, _ in sets]
    for (s, got), (_, want) in zip(got_sets, sets):
        assert np.array_equal(got, want), s
    # the cache as the steps left it
    nq = rc.T - W
    kp, ks = quant.quantize_rows(K[:, :, :nq])
    vp, vs = quant.quantize_rows(V[:, :, :nq])
    assert np.array_equal(rc.k_codes[:, :, :nq].cpu().numpy(), kp)
    assert np.array_equal(rc.k_sz[:, :, :nq].cpu().numpy().view(np.uint16), ks)
    assert np.array_equal(rc.v_sz[:, :, :nq].cpu().numpy().view(np.uint16), vs)
    for b in range(B):
        for h in range(Hkv):
            assert np.array_equal(tile16_codes(rc.v_codes[b, h])[:nq], vp[b, h])
            # the rows keep their slots across updates: slot i holds position vl_idx[i]
            slots = rc.vl_idx[b, h, :k].cpu().numpy()
            assert np.array_equal(np.sort(slots), final[b, h])
            rows_k = rc.vl_k[b, h, :k].float().cpu().numpy()
            rows_v = rc.vl_v[b, h, :k].float().cpu().numpy()
            assert np.array_equal(rows_k, K[b, h, slots]) and np.array_equal(rows_v, V[b, h, slots])
            bits = rc.vl_bits[b, h].cpu().numpy().view(np.uint32)
            want = np.zeros_like(bits)
            for p in final[b, h]:
                want[p >> 5] |= np.uint32(1) << np.uint32(p & 31)
            assert np.array_equal(bits, want)
    say(f"  resident bytes of the rolling cache: {rc.resident_bytes()}")


@pytest.mark.parametrize("k,n_st,spread,seed", [
    (35, 64, 3, 1),          # many equal scores: the position decides
    (5, 64, 1000, 2),        # more recent candidates than VL slots
    (1638, 64, 1 << 40, 3),  # the Llama-shaped budget, scores over a wide range (negative too)
    (8000, 64, 7, 4),        # close to the candidate limit, heavy ties
    (300, 1, 2, 5),          # one position left the window
    (20, 30, 3, 6),          # at most 64 candidates: ranked directly
    (100, 64, 0, 7),         # every score equal: the positions decide alone
])
def test_vl_update_ties_and_sizes(k, n_st, spread, seed):
    """hq_vl_update alone on constructed scores, against the oracle's update
    rule: the new set (compared as a set), the rows of every slot (kept
    slots untouched, freed ones holding the promoted ring rows) and the
    bitmap, bit for bit."""
    B, Hkv, D, W, R = 1, 2, 128, 32, 64
    C = W + R
    T = k + 3 * R + W + 200
    nq = T - W
    p0 = nq - n_st
    say(f"vl_update k={k} n_st={n_st} spread={spread}")
    rng = np.random.default_rng(seed)
    cache = hq.HybridCache(B, Hkv, D, T, W, k, torch.bfloat16, win_cap=C)
    # VL slots in no particular order, all below p0; rows and ring rows random
    old = np.stack([rng.permutation(rng.choice(p0, k, replace=False)) for _ in range(Hkv)])[None].astype(np.int32)
    cache.vl_idx.copy_(torch.from_numpy(old))
    cache.vl_k.copy_(torch.randn(cache.vl_k.shape, device="cuda").to(torch.bfloat16))
    cache.vl_v.copy_(torch.randn(cache.vl_v.shape, device="cuda").to(torch.bfloat16))
    cache.win_k.copy_(torch.randn(cache.win_k.shape, device="cuda").to(torch.bfloat16))
    cache.win_v.copy_(torch.randn(cache.win_v.shape, device="cuda").to(torch.bfloat16))
    cache.win_offset = int(rng.integers(C))
    hq.hq_vl_bitmap(cache.vl_idx, Hkv, k, cache.t_cap, cache.vl_bits)
    scores = rng.integers(-spread, spread + 1, (B, Hkv, nq), dtype=np.int64)
    sc = torch.from_numpy(scores).cuda()
    vl_k0, vl_v0 = cache.vl_k.float().cpu().numpy(), cache.vl_v.float().cpu().numpy()
    ring_k, ring_v = cache.win_k.float().cpu().numpy(), cache.win_v.float().cpu().numpy()
    hq.hq_vl_update(cache.descriptor(), cache.vl_idx, p0, sc, nq)
    torch.cuda.synchronize()
    got = cache.vl_idx.cpu().numpy()
    gk, gv = cache.vl_k.float().cpu().numpy(), cache.vl_v.float().cpu().numpy()
    bits = cache.vl_bits.cpu().numpy().view(np.uint32)
    for h in range(Hkv):
        want = lifecycle.select(scores[0, h], np.sort(old[0, h]), p0, nq, k)
        assert np.array_equal(np.sort(got[0, h]), want), h
        for slot in range(k):
            p = got[0, h, slot]
            if p == old[0, h, slot]:
                src_k, src_v = vl_k0[0, h, slot], vl_v0[0, h, slot]          # kept: untouched
            else:
                assert p0 <= p < nq                                          # promoted from the ring
                row = (cache.win_offset + (p - nq)) % C
                src_k, src_v = ring_k[0, h, row], ring_v[0, h, row]
            assert np.array_equal(gk[0, h, slot], src_k) and np.array_equal(gv[0, h, slot], src_v)
        wb = np.zeros_like(bits[0, h])
        for p in want:
            wb[p >> 5] |= np.uint32(1) << np.uint32(p & 31)
        assert np.array_equal(bits[0, h], wb)


@pytest.mark.parametrize("B,Hq,Hkv,D,T,W,k,R,n_st,dtype", [
    (1, 8, 2, 128, 3000, 32, 100, 64, 64, "bf16"),
    (2, 32, 2, 128, 5000, 128, 250, 64, 64, "bf16"),   # G = 16, the GLM-4-9B head grouping
    (1, 4, 4, 64, 2000, 16, 90, 16, 16, "f16"),        # D = 64, G = 1
    (1, 4, 2, 64, 1500, 16, 50, 8, 5, "f32"),          # fp32 rows, fewer new positions than ring slots
    (4, 32, 8, 128, 6300, 32, 5000, 64, 64, "bf16"),   # 32 heads x 5064 candidates: two rounds per scoring block
])
def test_vl_redetect_matches_detector_then_update(B, Hq, Hkv, D, T, W, k, R, n_st, dtype):
    """hq_vl_redetect (summed ring and candidate scores, then the update)
    against hq_detect_vlines_cache over every position then hq_vl_update, on
    two copies of the same cache: the index lists, the VL rows and the bitmap
    bit for bit; and the new set against the oracle's update rule over the
    oracle's INT4-key scores (queries on the 2^-4 grid: exact scores)."""
    say(f"vl_redetect B={B} Hq={Hq} Hkv={Hkv} D={D} T={T} W={W} k={k} R={R} n_st={n_st} {dtype}")
    rng = np.random.default_rng(T + k)
    nq = T - W
    p0 = nq - n_st
    grid = lambda shape, sc=1.0: np.rint(rng.standard_normal(shape) * sc * 16) / 16
    K = grid((B, Hkv, T, D)).astype(np.float32)
    V = grid((B, Hkv, T, D)).astype(np.float32)
    qring = grid((B, Hq, R, D)).astype(np.float32)
    vl = np.stack([np.stack([np.sort(rng.choice(p0, k, replace=False)) for _ in range(Hkv)])
                   for _ in range(B)]).astype(np.int32)
    dt = TORCH_DT[dtype]
    Kd, Vd, qd = to_dev(K, dtype), to_dev(V, dtype), to_dev(qring, dtype)
    caches = []
    for _ in range(2):
        c = hq.HybridCache(B, Hkv, D, T, W, k, dt, win_cap=W + R)
        c.build(Kd, Vd, torch.from_numpy(vl).cuda())
        caches.append(c)
    a, b = caches
    scores = torch.zeros((B, Hkv, nq), dtype=torch.int64, device="cuda")
    ws = torch.zeros(hq.hq_detect_workspace_size(B, Hkv, nq, 0), dtype=torch.uint8, device="cuda")
    hq.hq_detect_vlines_cache(None, qd, Hq, R, R - 1, True, a.descriptor(), nq, 0, None, scores.view(-1), ws)
    hq.hq_vl_update(a.descriptor(), a.vl_idx, p0, scores, nq)
    rws = torch.full((hq.hq_vl_redetect_workspace_size(b.descriptor()),), 0xFF, dtype=torch.uint8, device="cuda")
    hq.hq_vl_redetect(b.descriptor(), b.vl_idx, p0, qd, Hq, R, rws)
    torch.cuda.synchronize()
    for name in ("vl_idx", "vl_bits", "vl_k", "vl_v"):
        x, y = getattr(a, name), getattr(b, name)
        assert torch.equal(x, y), name
    # the oracle's rule over the oracle's scores
    G = Hq // Hkv
    kp, ks = quant.quantize_rows(K[:, :, :nq])
    got = b.vl_idx.cpu().numpy()
    for bb in range(B):
        for h in range(Hkv):
            rows = qring[bb, h * G:(h + 1) * G].reshape(G * R, D)
            units, ok = detect.cache_scores(rows, kp[bb, h], ks[bb, h])
            assert ok
            want = lifecycle.select(units, vl[bb, h], p0, nq, k)
            assert np.array_equal(np.sort(got[bb, h]), want), (bb, h)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_vl_redetect_off_grid(dtype):
    """hq_vl_redetect on plain data (no 2^-4 grid: queries N(0, 1) + 7 u, keys
    with outlier channels and planted lines, as the Llama-shaped workload
    draws them): the new set against the oracle's update rule over the
    float64 scores of the INT4 keys. The device rounds each score once to
    int64 units of 2^-16 after an fp64 evaluation, so it is within one unit
    of the oracle's; the sets may differ only among candidates whose oracle
    score lies within one unit of the k-th chosen score, and the VL rows and
    bitmap must match the device's own set."""
    w = synth.Workload(f"redet_off_{dtype}", 8800, B=1, Hq=8, Hkv=2, D=128, T=3000, W=32, k=100,
                       dtype=dtype, grid=False, n_plant=60)
    R = w.R
    nq = w.T - w.W
    p0 = nq - R
    say(f"vl_redetect off-grid {dtype}")
    K, V = synth.all_keys(w), synth.all_values(w)
    qh = synth.all_query_histories(w)
    assert not detect.on_grid(qh)
    rng = np.random.default_rng(5)
    vl = np.stack([np.sort(rng.choice(p0, w.k, replace=False)) for _ in range(w.Hkv)])[None].astype(np.int32)
    dt = TORCH_DT[dtype]
    c = hq.HybridCache(1, w.Hkv, w.D, w.T, w.W, w.k, dt, win_cap=w.W + R)
    c.build(to_dev(K, dtype), to_dev(V, dtype), torch.from_numpy(vl).cuda())
    rws = torch.zeros(hq.hq_vl_redetect_workspace_size(c.descriptor()), dtype=torch.uint8, device="cuda")
    hq.hq_vl_redetect(c.descriptor(), c.vl_idx, p0, to_dev(qh, dtype), w.Hq, R, rws)
    torch.cuda.synchronize()
    got_idx = c.vl_idx.cpu().numpy()
    kp, ks = quant.quantize_rows(K[:, :, :nq])
    G = w.Hq // w.Hkv
    changed = 0
    for h in range(w.Hkv):
        f = detect.cache_scores_float(qh[0, h * G:(h + 1) * G].reshape(G * R, w.D), kp[0, h], ks[0, h])
        want = lifecycle.select(f, vl[0, h], p0, nq, w.k)
        got = np.sort(got_idx[0, h])
        cand = np.concatenate([vl[0, h], np.arange(p0, nq)])
        assert set(got) <= set(cand.tolist()) and len(set(got)) == w.k
        kth = np.sort(f[want])[0]                   # the k-th best score among the oracle's choice
        for p in np.setxor1d(got, want):
            assert abs(f[p] - kth) <= 1.0, (h, int(p), float(f[p]), float(kth))
        changed += len(np.setdiff1d(want, vl[0, h]))
        # the rows and bitmap follow the device's set
        rows = c.vl_k[0, h].float().cpu().numpy()
        for slot, p in enumerate(got_idx[0, h]):
            assert np.array_equal(rows[slot], K[0, h, p].astype(np.float32)), (h, slot)
        bits = c.vl_bits[0, h].cpu().numpy().view(np.uint32)
        wb = np.zeros_like(bits)
        for p in got:
            wb[p >> 5] |= np.uint32(1) << np.uint32(p & 31)
        assert np.array_equal(bits, wb)
    say(f"  promoted by the oracle's rule: {changed} positions")


@pytest.mark.parametrize("name", ["llama32k", "glm32k"])
def test_rolling_cache_full_size_steps(name):
    """The configuration the benchmark times, at its full size: the rolling
    cache of a Llama-shaped layer (B 1, 32 query / 8 KV heads, D 128, context
    32768 at step 0, window 128, VL budget 1638, ring of W + 64 rows), or of
    the GLM-4-9B head grouping (32 / 2), built from the prefill-end detection,
    then three decode steps (hq_decode_step: the step's queries into the
    ring, the window's oldest row packed into its INT4 row, the automatic 64
    splits), the cache advanced after each. Every query head's output and
    log-sum-exp against the oracle's lifecycle, and the three packed INT4
    rows of every KV head bit for bit."""
    base = synth.WORKLOADS[name]
    n = 3
    w = base.replace(name=f"{name}+3", T=base.T + n)
    B, Hq, Hkv, D, W, k, R = w.B, w.Hq, w.Hkv, w.D, w.W, w.k, 64
    T0 = base.T
    say(f"rolling cache, {name}: inputs and the oracle's three steps ...")
    K, V = synth.all_keys(w), synth.all_values(w)
    queries = np.stack([synth.all_queries(w.replace(seed=w.seed + 101 * (s + 1))) for s in range(n)])
    vl0, _ = detect.detect(synth.all_query_histories(w), K[:, :, :T0], T0 - W, k)
    outs, lses, sets, _ = lifecycle.simulate(K, V, queries, T0, W, R, k, vl0)
    assert not sets                                                   # no update within three steps
    dt = TORCH_DT[w.dtype]
    Kd, Vd = to_dev(K, w.dtype), to_dev(V, w.dtype)
    t_cap = ((T0 + n - W + 1) + 31) // 32 * 32
    rc = hq.RollingCache(B, Hkv, D, T0, W, k, dt, Hq, R=R, t_cap=t_cap)
    rc.build(Kd[:, :, :T0].contiguous(), Vd[:, :, :T0].contiguous(), torch.from_numpy(vl0).cuda())
    assert hq.hq_decode_auto_splits(rc.descriptor(), Hq) == 64
    ws = torch.full((hq.hq_decode_workspace_size(rc.descriptor(), Hq, 0),), 0xFF, dtype=torch.uint8,
                    device="cuda")
    out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    for s in range(n):
        say(f"  step {s}")
        rc.decode_step(to_dev(queries[s], w.dtype), out, lse, ws)
        o, l = out.cpu().numpy(), lse.cpu().numpy()
        e = rel_err(o, outs[s])
        assert e <= 2e-3 and np.max(np.abs(l - lses[s])) <= 1e-3, (s, e)
        rc.advance(Kd[:, :, T0 + s], Vd[:, :, T0 + s])
    torch.cuda.synchronize()
    # the rows the three steps packed: positions T0 - W .. T0 - W + 2
    r0, r1 = T0 - W, T0 - W + n
    kp, ks = quant.quantize_rows(K[:, :, r0:r1])
    vp, vs = quant.quantize_rows(V[:, :, r0:r1])
    assert np.array_equal(rc.k_codes[:, :, r0:r1].cpu().numpy(), kp)
    assert np.array_equal(rc.k_sz[:, :, r0:r1].cpu().numpy().view(np.uint16), ks)
    assert np.array_equal(rc.v_sz[:, :, r0:r1].cpu().numpy().view(np.uint16), vs)
    for b in range(B):
        for h in range(Hkv):
            assert np.array_equal(tile16_codes(rc.v_codes[b, h])[r0:r1], vp[b, h])
