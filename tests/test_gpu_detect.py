"""GPU parity of hq_detect_vlines against the oracle detector: query ring
accumulation, exact int64 column scores and bit-exact index sets (both the
MFMA matmul form and the summed-query form), on tie-heavy small cases and
on the full GLM-4-9B-shaped (32 q / 2 kv heads, 32K) and
Llama-3.1-8B-shaped (32 q / 8 kv heads, 32K) workloads."""
import zlib

import numpy as np
import pytest
import torch

import hybrid_precision_quantized_amd as hq
import synth
from oracle import detect, quant
from tests.gpu_util import (TORCH_DT, matmul_exact_precondition, matmul_score_bound_units, say,
                            to_dev)

pytestmark = pytest.mark.gpu

METHODS = [hq.HQ_DETECT_MATMUL, hq.HQ_DETECT_QSUM]


def _run(q_acc, K, cand_end, k_top, method, dtype, exact=True):
    B, Hq, R, D = q_acc.shape
    if exact and method == hq.HQ_DETECT_MATMUL:
        # the matrix-core form is exact on grid inputs only while every
        # residue's absolute sum stays below 2^16 (its fp32 partials exact)
        worst = matmul_exact_precondition(q_acc, K, cand_end)
        assert worst < 2.0 ** 16, f"inputs outside the exact range of the MFMA form: {worst}"

    Hkv, k_rows = K.shape[1], K.shape[2]
    qd = to_dev(q_acc, dtype)
    kd = to_dev(K, dtype)
    idx = torch.full((B, Hkv, max(k_top, 1)), -1, dtype=torch.int32, device="cuda")
    sc = torch.zeros((B, Hkv, max(cand_end, 1)), dtype=torch.int64, device="cuda")
    ws = torch.zeros(hq.hq_detect_workspace_size(B, Hkv, cand_end, k_top), dtype=torch.uint8, device="cuda")
    ran = hq.hq_detect_vlines(None, qd, B, Hq, Hkv, D, R, 0, True, kd, k_rows, cand_end, k_top,
                              method, idx, sc, ws)
    torch.cuda.synchronize()
    assert ran
    return idx.cpu().numpy()[..., :k_top], sc.cpu().numpy()[..., :cand_end]


@pytest.mark.parametrize("method", METHODS)
@pytest.mark.parametrize("B,Hq,Hkv,D,R,n,ce,k_top,dtype,spread", [
    (2, 8, 2, 128, 64, 3000, 2900, 145, "bf16", 3.0),
    (1, 4, 4, 128, 5, 1000, 999, 50, "bf16", 0.25),     # many equal scores
    (1, 6, 2, 64, 33, 777, 700, 35, "bf16", 1.0),
    (1, 8, 1, 128, 64, 2048, 1920, 1920, "f16", 1.0),   # k_top == cand_end
    (1, 8, 2, 128, 64, 2048, 1920, 0, "bf16", 1.0),     # k_top == 0 (scores only)
    (1, 8, 2, 128, 64, 1000, 1, 1, "bf16", 1.0),        # single candidate
    (1, 8, 2, 128, 16, 40000, 39900, 1995, "bf16", 2.0),  # keys beyond the LDS-resident size
    (1, 4, 1, 128, 2, 5000, 4900, 4000, "bf16", 0.0625),  # nearly all scores tied
    (2, 8, 2, 128, 8, 20000, 16411, 700, "bf16", 2.0),    # 4 units, narrow score range
    # beyond 32768 candidates: the keys, select and write launches
    (1, 8, 2, 128, 8, 34000, 32769, 1, "bf16", 1.0),      # one above the one-launch size, k = 1
    (2, 8, 2, 128, 4, 50000, 49999, 2500, "bf16", 0.5),   # ragged last chunk, 4 units
    (1, 8, 1, 128, 16, 33300, 33000, 33000, "f16", 1.0),  # k_top == cand_end
    (1, 8, 2, 128, 8, 34000, 33000, 0, "bf16", 1.0),      # k_top == 0
    (1, 4, 1, 128, 2, 36000, 35900, 20000, "bf16", 0.0625),  # crowded first digit: the radix path
    (1, 4, 1, 128, 2, 140100, 140000, 7000, "bf16", 1.0),  # chunks over 4096 keys: two runs per write thread
    # the eight-wave column-sum blocks at D = 64: 512 staged rows in 256-column
    # blocks, and 256 resident rows in 512-column blocks (16 units x 32 blocks)
    (1, 8, 1, 64, 64, 5000, 4900, 245, "bf16", 1.0),
    (2, 32, 8, 64, 64, 16500, 16384, 819, "f16", 0.5),
])
def test_detect_small_exact(method, B, Hq, Hkv, D, R, n, ce, k_top, dtype, spread):
    say(f"detect method={method} B={B} Hq={Hq} Hkv={Hkv} D={D} R={R} n={n} ce={ce} k={k_top} {dtype}")
    rng = np.random.default_rng(n + R)
    q = np.rint(rng.standard_normal((B, Hq, R, D)) * spread * 16) / 16
    K = np.rint(rng.standard_normal((B, Hkv, n, D)) * spread * 16) / 16
    if dtype == "bf16":
        q, K = synth.round_dtype(q, "bf16"), synth.round_dtype(K, "bf16")
    else:
        q = q.astype(np.float16).astype(np.float32)
        K = K.astype(np.float16).astype(np.float32)
    want_idx, want_sc = detect.detect(q, K, ce, k_top)
    got_idx, got_sc = _run(q, K, ce, k_top, method, dtype)
    assert np.array_equal(got_sc, want_sc)
    assert np.array_equal(got_idx, want_idx)


@pytest.mark.parametrize("method", METHODS)
@pytest.mark.parametrize("n,ce,k_top", [(3000, 2900, 100), (34000, 33900, 1700)])
def test_detect_wide_range(method, n, ce, k_top):
    """A few planted columns far above the rest: the score range exceeds 31
    bits, so the keys drop low bits and the bulk shares a handful of first
    digits (the radix path with its refinement on the dropped bits), in the
    one-launch and the three-launch top-k."""
    B, Hq, Hkv, D, R = 1, 8, 2, 128, 8
    say(f"detect wide range method={method} n={n} ce={ce} k={k_top}")
    rng = np.random.default_rng(n + 7)
    q = synth.round_dtype(np.rint(rng.standard_normal((B, Hq, R, D)) * 16) / 16, "bf16")
    K = synth.round_dtype(np.rint(rng.standard_normal((B, Hkv, n, D)) * 16) / 16, "bf16")
    G = Hq // Hkv
    for h in range(Hkv):
        qs = q[0, h * G:(h + 1) * G].sum(axis=(0, 1))
        K[0, h, rng.choice(ce, 30, replace=False)] = 64.0 * np.where(qs >= 0, 1.0, -1.0)
    want_idx, want_sc = detect.detect(q, K, ce, k_top)
    span = int((want_sc.max(axis=-1) - want_sc.min(axis=-1)).min())
    assert span >= 2 ** 31, span                       # wider than the keys: low bits dropped
    got_idx, got_sc = _run(q, K, ce, k_top, method, "bf16")
    assert np.array_equal(got_sc, want_sc)
    assert np.array_equal(got_idx, want_idx)


@pytest.mark.parametrize("n", [3000, 34000])
def test_detect_refine_on_dropped_bits(n):
    """Scores wider than the 32-bit keys by about 10 bits (QSUM form, exact
    in fp64), with k_top placed where the k-th and the (k+1)-th largest
    scores share a key: the top-k must refine on the bits the keys dropped,
    in the one-launch and the three-launch paths."""
    B, Hq, Hkv, D, R = 1, 4, 1, 128, 8
    say(f"detect refine n={n}")
    rng = np.random.default_rng(n + 11)
    q = synth.round_dtype(np.rint(rng.standard_normal((B, Hq, R, D)) * 16) / 16, "bf16")
    K = synth.round_dtype(np.rint(rng.standard_normal((B, Hkv, n, D)) * 16) / 16, "bf16")
    ce = n - 50
    qs = q[0].sum(axis=(0, 1))
    K[0, 0, rng.choice(ce, 20, replace=False)] = 32768.0 * np.where(qs >= 0, 1.0, -1.0)
    _, sc = detect.detect(q, K, ce, 0)
    v = sc[0, 0].astype(object)
    lo, hi = min(v), max(v)
    nbits = int(hi - lo).bit_length()
    assert nbits > 38, nbits                            # keys drop nbits - 31 low bits
    shift = nbits - 31
    order = sorted(range(ce), key=lambda j: (-v[j], j))
    keys = [(v[j] - lo) >> shift for j in order]
    cut = next(i for i in range(30, ce - 1) if keys[i] == keys[i + 1] and v[order[i]] != v[order[i + 1]])
    k_top = cut + 1                                     # the k-th and (k+1)-th share a key, scores differ
    want_idx, want_sc = detect.detect(q, K, ce, k_top)
    got_idx, got_sc = _run(q, K, ce, k_top, hq.HQ_DETECT_QSUM, "bf16")
    assert np.array_equal(got_sc, want_sc)
    assert np.array_equal(got_idx, want_idx)


def _random_detect_cases(n, seed):
    """n detector configurations drawn from a fixed seed: batch 1-2, 1-4 KV
    heads, group 1-8, D 64 or 128, 1-64 ring slots, 1-36000 candidates
    (both sides of the one-launch top-k limit), k from 0 to all, score
    spreads from heavy ties to wide ranges, bf16 or fp16."""
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        Hkv = int(rng.choice([1, 2, 4]))
        G = int(rng.choice([1, 2, 4, 8]))
        D = int(rng.choice([64, 128]))
        R = int(rng.choice([1, 5, 16, 64]))
        ce = int(rng.choice([int(rng.integers(1, 3000)), int(rng.integers(3000, 36000))]))
        n_rows = ce + int(rng.integers(0, 200))
        k = int(rng.choice([0, 1, ce, int(rng.integers(0, ce + 1)), max(1, ce // 20)]))
        spread = float(rng.choice([0.0625, 0.25, 1.0, 2.0]))
        dtype = str(rng.choice(["bf16", "f16"]))
        cases.append((int(rng.integers(1, 3)), Hkv * G, Hkv, D, R, n_rows, ce, k, dtype, spread))
    return cases


RANDOM_DETECT = _random_detect_cases(12, 77)


@pytest.mark.parametrize("method", METHODS)
@pytest.mark.parametrize("case", RANDOM_DETECT, ids=[str(c) for c in RANDOM_DETECT])
def test_detect_random_shapes(method, case):
    """Seeded random shapes on the 2^-4 grid: int64 scores and index sets
    bit for bit against the oracle."""
    B, Hq, Hkv, D, R, n, ce, k_top, dtype, spread = case
    say(f"detect random method={method} {case}")
    rng = np.random.default_rng(zlib.crc32(str(case).encode()))
    q = np.rint(rng.standard_normal((B, Hq, R, D)) * spread * 16) / 16
    K = np.rint(rng.standard_normal((B, Hkv, n, D)) * spread * 16) / 16
    if dtype == "bf16":
        q, K = synth.round_dtype(q, "bf16"), synth.round_dtype(K, "bf16")
    else:
        q = q.astype(np.float16).astype(np.float32)
        K = K.astype(np.float16).astype(np.float32)
    want_idx, want_sc = detect.detect(q, K, ce, k_top)
    got_idx, got_sc = _run(q, K, ce, k_top, method, dtype)
    assert np.array_equal(got_sc, want_sc)
    assert np.array_equal(got_idx, want_idx)


def test_accumulate_ring_and_cadence():
    say("detect accumulate ring")
    B, Hq, Hkv, D, R, n, ce, kt = 1, 4, 2, 128, 8, 300, 280, 14
    rng = np.random.default_rng(9)
    steps = synth.round_dtype(np.rint(rng.standard_normal((2 * R, B, Hq, D)) * 16) / 16, "bf16")
    K = synth.round_dtype(np.rint(rng.standard_normal((B, Hkv, n, D)) * 16) / 16, "bf16")
    q_acc = torch.zeros((B, Hq, R, D), dtype=torch.bfloat16, device="cuda")
    kd = to_dev(K, "bf16")
    idx = torch.zeros((B, Hkv, kt), dtype=torch.int32, device="cuda")
    ws = torch.zeros(hq.hq_detect_workspace_size(B, Hkv, ce, kt), dtype=torch.uint8, device="cuda")
    ran_at = []
    for s in range(2 * R):
        if hq.hq_detect_vlines(to_dev(steps[s], "bf16"), q_acc, B, Hq, Hkv, D, R, s, False, kd, n, ce, kt,
                               hq.HQ_DETECT_MATMUL, idx, None, ws):
            ran_at.append(s)
    torch.cuda.synchronize()
    assert ran_at == [R - 1, 2 * R - 1]
    ring = q_acc.float().cpu().numpy()
    want_ring = np.moveaxis(steps[R:], 0, 2)              # [B][Hq][R][D], slot = step mod R
    assert np.array_equal(ring, want_ring)
    want_idx, _ = detect.detect(want_ring, K, ce, kt)
    assert np.array_equal(idx.cpu().numpy(), want_idx)


@pytest.mark.parametrize("name", ["glm32k", "llama32k"])
@pytest.mark.parametrize("method", METHODS)
def test_detect_full_workload(name, method):
    w = synth.WORKLOADS[name]
    say(f"detect full workload {name} method={method}")
    K = synth.all_keys(w)
    q = synth.all_query_histories(w)
    ce = w.T - w.W
    want_idx, want_sc = detect.detect(q, K, ce, w.k)
    got_idx, got_sc = _run(q, K, ce, w.k, method, w.dtype)
    assert np.array_equal(got_sc, want_sc)
    assert np.array_equal(got_idx, want_idx)


def test_detect_qwen128k_sampled():
    """Batch 16 x 128K context, MATMUL form: the GPU scores and selects for
    every (b, KV head) (the resident column-sum kernel and the keys, select
    and write launches of the top-k); the oracle checks KV heads 0 and 7 of
    sequence 0 and KV head 3 of sequence 15 (int64 scores and index sets,
    exact)."""
    w = synth.WORKLOADS["qwen128k"]
    say("detect qwen128k (upload)")
    dt = TORCH_DT[w.dtype]
    Kd = torch.empty((w.B, w.Hkv, w.T, w.D), dtype=dt, device="cuda")
    for b in range(w.B):
        kb = np.stack(synth._parallel(lambda h: synth.keys(w, b, h), [(h,) for h in range(w.Hkv)]))
        Kd[b].copy_(to_dev(kb, w.dtype))
    q = synth.all_query_histories(w)
    ce = w.T - w.W
    idx = torch.full((w.B, w.Hkv, w.k), -1, dtype=torch.int32, device="cuda")
    sc = torch.zeros((w.B, w.Hkv, ce), dtype=torch.int64, device="cuda")
    ws = torch.zeros(hq.hq_detect_workspace_size(w.B, w.Hkv, ce, w.k), dtype=torch.uint8, device="cuda")
    say("detect qwen128k (run)")
    ran = hq.hq_detect_vlines(None, to_dev(q, w.dtype), w.B, w.Hq, w.Hkv, w.D, w.R, 0, True, Kd, w.T, ce, w.k,
                              hq.HQ_DETECT_MATMUL, idx, sc, ws)
    torch.cuda.synchronize()
    assert ran
    del Kd
    got_idx, got_sc = idx.cpu().numpy(), sc.cpu().numpy()
    for b, h in [(0, 0), (0, 7), (15, 3)]:
        say(f"detect qwen128k (oracle b={b} h={h})")
        qh = q[b:b + 1, h * w.G:(h + 1) * w.G]
        Kh = synth.keys(w, b, h)[None, None]
        worst = matmul_exact_precondition(qh, Kh, ce)
        assert worst < 2.0 ** 16, f"inputs outside the exact range of the MFMA form: {worst}"
        want_idx, want_sc = detect.detect(qh, Kh, ce, w.k)
        assert np.array_equal(got_sc[b, h], want_sc[0, 0]), (b, h)
        assert np.array_equal(got_idx[b, h], want_idx[0, 0]), (b, h)


def _run_cache(q_acc, K, cand_end, k_top, dtype, T, W):
    """hq_detect_vlines_cache over a cache whose INT4 planes were written by
    hq_quantize_kv from K (positions [0, T - W))."""
    B, Hq, R, D = q_acc.shape
    Hkv = K.shape[1]
    dt = TORCH_DT[dtype]
    kd = to_dev(K, dtype)
    cache = hq.HybridCache(B, Hkv, D, T, W, 0, dt)
    cache.quantize(kd, kd)
    kv = cache.descriptor()
    qd = to_dev(q_acc, dtype)
    idx = torch.full((B, Hkv, max(k_top, 1)), -1, dtype=torch.int32, device="cuda")
    sc = torch.zeros((B, Hkv, max(cand_end, 1)), dtype=torch.int64, device="cuda")
    ws = torch.zeros(hq.hq_detect_workspace_size(B, Hkv, cand_end, k_top), dtype=torch.uint8, device="cuda")
    ran = hq.hq_detect_vlines_cache(None, qd, Hq, R, 0, True, kv, cand_end, k_top, idx, sc, ws)
    torch.cuda.synchronize()
    assert ran
    return idx.cpu().numpy()[..., :k_top], sc.cpu().numpy()[..., :cand_end]


@pytest.mark.parametrize("B,Hq,Hkv,D,R,T,W,k_top,dtype,spread", [
    (2, 8, 2, 128, 64, 3000, 100, 145, "bf16", 3.0),
    (1, 6, 2, 64, 33, 777, 77, 35, "bf16", 1.0),
    (1, 8, 1, 128, 64, 2048, 128, 1920, "f16", 1.0),     # k_top == cand_end
    (1, 8, 2, 128, 16, 40128, 128, 2000, "bf16", 2.0),   # keys beyond the LDS-resident size
    (1, 4, 1, 128, 2, 5000, 100, 3000, "bf16", 0.0625),  # many equal scores
])
def test_detect_cache_small(B, Hq, Hkv, D, R, T, W, k_top, dtype, spread):
    """Scores from the INT4 key cache: bit-exact int64 scores and index sets
    against the oracle's exact integer evaluation."""
    say(f"detect cache B={B} Hq={Hq} Hkv={Hkv} D={D} R={R} T={T} W={W} k={k_top} {dtype}")
    rng = np.random.default_rng(T + R)
    q = np.rint(rng.standard_normal((B, Hq, R, D)) * spread * 16) / 16
    K = rng.standard_normal((B, Hkv, T, D)) * spread
    if dtype == "bf16":
        q, K = synth.round_dtype(q, "bf16"), synth.round_dtype(K, "bf16")
    else:
        q = q.astype(np.float16).astype(np.float32)
        K = K.astype(np.float16).astype(np.float32)
    ce = T - W
    kp, ks = quant.quantize_rows(K[:, :, :ce])
    want_idx, want_sc = detect.detect_cache(q, kp, ks, ce, k_top)
    got_idx, got_sc = _run_cache(q, K, ce, k_top, dtype, T, W)
    assert np.array_equal(got_sc, want_sc)
    assert np.array_equal(got_idx, want_idx)


@pytest.mark.parametrize("name", ["glm32k", "llama32k"])
def test_detect_cache_full_workload(name):
    w = synth.WORKLOADS[name]
    say(f"detect cache full workload {name}")
    K = synth.all_keys(w)
    q = synth.all_query_histories(w)
    ce = w.T - w.W
    kp, ks = quant.quantize_rows(K[:, :, :ce])
    want_idx, want_sc = detect.detect_cache(q, kp, ks, ce, w.k)
    got_idx, got_sc = _run_cache(q, K, ce, w.k, w.dtype, w.T, w.W)
    assert np.array_equal(got_sc, want_sc)
    assert np.array_equal(got_idx, want_idx)
    # how many of the 16-bit detector's lines the cache form keeps
    idx16, _ = detect.detect(q, K, ce, w.k)
    overlap = np.mean([len(np.intersect1d(got_idx[0, h], idx16[0, h])) / w.k for h in range(w.Hkv)])
    say(f"   overlap with the 16-bit detector's set: {overlap:.3f}")


def _run_mass(q_acc, K, cand_end, k_top, dtype):
    B, Hq, R, D = q_acc.shape
    Hkv, k_rows = K.shape[1], K.shape[2]
    qd = to_dev(q_acc, dtype)
    kd = to_dev(K, dtype)
    idx = torch.full((B, Hkv, max(k_top, 1)), -1, dtype=torch.int32, device="cuda")
    sc = torch.zeros((B, Hkv, max(cand_end, 1)), dtype=torch.int64, device="cuda")
    ws = torch.full((hq.hq_detect_mass_workspace_size(B, Hq, Hkv, R, k_rows, cand_end),), 0xFF,
                    dtype=torch.uint8, device="cuda")
    ran = hq.hq_detect_vlines_mass(None, qd, B, Hq, Hkv, D, R, 0, True, kd, k_rows, cand_end, k_top,
                                   idx, sc, ws)
    torch.cuda.synchronize()
    assert ran
    return idx.cpu().numpy()[..., :k_top], sc.cpu().numpy()[..., :cand_end]


def _check_mass(got_idx, got_units, want_idx, want_sc, k_top, rel=1e-4):
    """Scores within rel of the unit's largest oracle score; index sets equal
    except for positions whose oracle score lies within that tolerance of the
    k-th largest (near ties the fp32 evaluation may order either way)."""
    got_sc = got_units.astype(np.float64) / float(1 << 22)
    B, Hkv, _ = want_sc.shape
    for b in range(B):
        for h in range(Hkv):
            tol = rel * max(float(want_sc[b, h].max()), 1e-30)
            err = float(np.max(np.abs(got_sc[b, h] - want_sc[b, h])))
            assert err <= tol, (b, h, err, tol)
            if k_top == 0:
                continue
            tau = np.sort(want_sc[b, h])[::-1][k_top - 1]
            diff = np.setxor1d(got_idx[b, h], want_idx[b, h])
            assert np.all(np.abs(want_sc[b, h][diff] - tau) <= 2 * tol), (b, h, diff)
            assert np.all(np.diff(got_idx[b, h]) > 0)


@pytest.mark.parametrize("B,Hq,Hkv,D,R,n,ce,k_top,dtype", [
    (2, 8, 2, 128, 64, 3000, 2900, 145, "bf16"),
    (1, 6, 2, 64, 33, 777, 700, 35, "bf16"),
    (1, 8, 1, 128, 64, 2048, 1920, 1920, "f16"),    # k_top == cand_end
    (1, 4, 2, 128, 5, 300, 1, 1, "bf16"),           # single candidate, few rows
])
def test_detect_mass_small(B, Hq, Hkv, D, R, n, ce, k_top, dtype):
    """Attention-mass scores against the oracle's float64 softmax masses."""
    say(f"detect mass B={B} Hq={Hq} Hkv={Hkv} D={D} R={R} n={n} ce={ce} k={k_top} {dtype}")
    rng = np.random.default_rng(n + 3 * R)
    q = rng.standard_normal((B, Hq, R, D)) * 2
    K = rng.standard_normal((B, Hkv, n, D))
    if dtype == "bf16":
        q, K = synth.round_dtype(q, "bf16"), synth.round_dtype(K, "bf16")
    else:
        q = q.astype(np.float16).astype(np.float32)
        K = K.astype(np.float16).astype(np.float32)
    want_idx, want_sc = detect.detect_mass(q, K, ce, k_top)
    got_idx, got_units = _run_mass(q, K, ce, k_top, dtype)
    _check_mass(got_idx, got_units, want_idx, want_sc, k_top)
    again_idx, again_units = _run_mass(q, K, ce, k_top, dtype)
    assert np.array_equal(again_units, got_units) and np.array_equal(again_idx, got_idx)


@pytest.mark.parametrize("name", ["glm32k", "llama32k"])
def test_detect_mass_full_workload(name):
    w = synth.WORKLOADS[name]
    say(f"detect mass full workload {name}")
    K = synth.all_keys(w)
    q = synth.all_query_histories(w)
    ce = w.T - w.W
    want_idx, want_sc = detect.detect_mass(q, K, ce, w.k)
    got_idx, got_units = _run_mass(q, K, ce, w.k, w.dtype)
    _check_mass(got_idx, got_units, want_idx, want_sc, w.k)
    # the mass the chosen set covers, and how it compares with the logit-sum set
    G = w.Hq // w.Hkv
    idx16, _ = detect.detect(q, K, ce, w.k)
    cover = np.mean([want_sc[0, h][got_idx[0, h]].sum() / (G * w.R) for h in range(w.Hkv)])
    cover16 = np.mean([want_sc[0, h][idx16[0, h]].sum() / (G * w.R) for h in range(w.Hkv)])
    say(f"   attention mass covered: mass set {cover:.3f}, logit-sum set {cover16:.3f}")


def _pattern_case(values, k_top, method):
    """Scores equal to (rows) * values[j] exactly: every query row is the
    first unit vector and key j carries values[j] in channel 0, so the score
    pattern (ties, skew, bucket sizes) is set by `values` alone."""
    n = len(values)
    B, Hq, Hkv, D, R = 1, 4, 1, 64, 2
    q = np.zeros((B, Hq, R, D), np.float32)
    q[..., 0] = 1.0
    K = np.zeros((B, Hkv, n, D), np.float32)
    K[0, 0, :, 0] = values
    # the other channels meet zero query entries; on the 2^-4 grid so the
    # oracle's exactness check holds
    K[0, 0, :, 1:] = np.rint(np.random.default_rng(n).standard_normal((n, D - 1)) * 16) / 16
    want_idx, want_sc = detect.detect(q, K, n, k_top)
    got_idx, got_sc = _run(q, K, n, k_top, method, "bf16")
    assert np.array_equal(got_sc, want_sc)
    assert np.array_equal(got_idx, want_idx)


def _grid_values(rng, n, lo, hi):
    return np.rint(rng.uniform(lo, hi, n) * 16).astype(np.float32) / 16


@pytest.mark.parametrize("method", METHODS)
@pytest.mark.parametrize("case", ["ties_small_bucket", "ties_large_bucket", "k_is_n", "k_is_1",
                                  "all_equal", "threshold_in_lowest_bin", "threshold_in_top_bin"])
def test_topk_score_patterns(method, case):
    """Edge cases of the top-k's two paths: a boundary bucket of at most 1024
    keys is ranked directly, a larger one goes through the remaining radix
    digits; ties at the threshold go to the lower positions either way."""
    rng = np.random.default_rng(zlib.crc32(case.encode()))
    n = 6000
    v = _grid_values(rng, n, -8.0, 8.0)
    k_top = 300
    if case == "ties_small_bucket":       # 700 equal scores straddle the cut
        tie = rng.choice(n, 700, replace=False)
        v[v > 6.0] = 5.0
        v[tie] = 6.0
        k_top = 350
    elif case == "ties_large_bucket":     # 2000 equal scores straddle the cut
        tie = rng.choice(n, 2000, replace=False)
        v[v > 6.0] = 5.0
        v[tie] = 6.0
        k_top = 1500
    elif case == "k_is_n":
        k_top = n
    elif case == "k_is_1":
        k_top = 1
    elif case == "all_equal":
        v[:] = 2.5
        k_top = 37
    elif case == "threshold_in_lowest_bin":   # almost everything selected
        k_top = n - 3
    elif case == "threshold_in_top_bin":      # only the largest few
        v[rng.choice(n, 5, replace=False)] = 7.9375
        k_top = 3
    say(f"top-k pattern {case} method={method} n={n} k={k_top}")
    _pattern_case(v, k_top, method)


@pytest.mark.parametrize("method", METHODS)
def test_detect_many_units_long_rows(method):
    """Enough (unit, 256-column group) pairs that the matmul form walks 4
    groups per block with the query rows resident in LDS (the long-context
    layout): 8 sequences x 8 KV heads, 32 query heads, 64 steps, 8064
    candidates. Scores and sets bit-exact against the oracle."""
    B, Hq, Hkv, D, R, n, ce, k_top = 8, 32, 8, 128, 64, 8192, 8064, 403
    rng = np.random.default_rng(77)
    q = synth.round_dtype(np.rint(rng.standard_normal((B, Hq, R, D)) * 16) / 16, "bf16")
    K = synth.round_dtype(np.rint(rng.standard_normal((B, Hkv, n, D)) * 16) / 16, "bf16")
    say(f"detect method={method} B={B} Hq={Hq} Hkv={Hkv} n={n} ce={ce} k={k_top} (resident rows)")
    want_idx, want_sc = detect.detect(q, K, ce, k_top)
    got_idx, got_sc = _run(q, K, ce, k_top, method, "bf16")
    assert np.array_equal(got_sc, want_sc)
    assert np.array_equal(got_idx, want_idx)


def _check_near_ties(got_idx, got_sc, want_idx, want_sc, bound, k_top):
    """Scores within their bound of the exact ones; the index sets equal
    except for positions whose exact score lies within twice the bound of the
    k-th largest exact score (there the fp32 rounding may order either way);
    every returned set ascending and of the right size."""
    B, Hkv, _ = want_sc.shape
    worst = 0.0
    n_swapped = 0
    for b in range(B):
        for h in range(Hkv):
            err = np.abs(got_sc[b, h] - want_sc[b, h]).astype(np.float64)
            assert np.all(err <= bound[b, h]), (b, h, float((err - bound[b, h]).max()))
            worst = max(worst, float((err / bound[b, h]).max()))
            if k_top == 0:
                continue
            assert len(got_idx[b, h]) == k_top and np.all(np.diff(got_idx[b, h]) > 0)
            tau = np.sort(want_sc[b, h])[::-1][k_top - 1]
            diff = np.setxor1d(got_idx[b, h], want_idx[b, h])
            n_swapped += len(diff)
            assert np.all(np.abs(want_sc[b, h][diff] - tau) <= 2 * bound[b, h][diff]), (b, h, diff)
    say(f"   max |err| / bound = {worst:.2e}; positions swapped at the cut: {n_swapped}")


@pytest.mark.parametrize("case", ["glm32k", "llama32k", "small_f16", "small_g1"])
def test_detect_matmul_off_grid(case):
    """The MFMA form on plain bf16/fp16 inputs (no 2^-4 grid): queries
    N(0, 1) + 7 u and keys with outlier channels and planted lines, as the
    GLM-4-9B-shaped detector workload draws them. The exact scores are the
    oracle's float64 ones; the GPU's differ by the fp32 rounding of each
    residue chain, bounded from the inputs, and the sets may differ only at
    near ties of the k-th score."""
    if case in ("glm32k", "llama32k"):
        w = synth.WORKLOADS[case].replace(grid=False)
    elif case == "small_f16":
        w = synth.Workload("offgrid_f16", 4711, B=2, Hq=8, Hkv=2, D=128, T=3000, W=100, k=150,
                           dtype="f16", grid=False)
    else:
        w = synth.Workload("offgrid_g1", 4712, B=1, Hq=4, Hkv=4, D=64, T=2000, W=64, k=90,
                           dtype="bf16", grid=False, R=33)
    say(f"detect matmul off-grid {case}")
    K = synth.all_keys(w)
    q = synth.all_query_histories(w)
    assert not detect.on_grid(q) and not detect.on_grid(K)
    ce = w.T - w.W
    want_idx, want_sc = detect.detect(q, K, ce, w.k, require_exact=False)
    got_idx, got_sc = _run(q, K, ce, w.k, hq.HQ_DETECT_MATMUL, w.dtype, exact=False)
    bound = matmul_score_bound_units(q, K, ce)
    _check_near_ties(got_idx, got_sc, want_idx, want_sc, bound, w.k)
    # and run to run the same bits
    again_idx, again_sc = _run(q, K, ce, w.k, hq.HQ_DETECT_MATMUL, w.dtype, exact=False)
    assert np.array_equal(again_sc, got_sc) and np.array_equal(again_idx, got_idx)
