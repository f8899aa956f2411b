"""GPU parity of hq_decode_attn (with hq_quantize_kv, hq_gather_rows and
hq_vl_bitmap building the cache) against the oracle decode step.

Bar: max |O_gpu - O_oracle| <= 2e-3 * RMS(O_oracle) over the output tensor,
fp32 outputs; lse within 1e-3. The GPU chain (quantize -> bitmap/gather ->
decode) and the oracle chain (quantize -> decode) share only the seeded
inputs."""
import math
import zlib

import numpy as np
import pytest
import torch

import hybrid_precision_quantized_amd as hq
import synth
from oracle import attention, detect, quant
from tests.gpu_util import TORCH_DT, rel_err, say, tile16_codes, tile16_slot, to_dev, upload_kv

pytestmark = pytest.mark.gpu

TOL = 2e-3


def _workload(B, Hq, Hkv, D, T, W, k, dtype, seed):
    return synth.Workload(f"case{seed}", seed, B=B, Hq=Hq, Hkv=Hkv, D=D, T=T, W=W, k=k,
                          dtype=dtype, grid=(dtype != "f32"),
                          n_plant=max(1, min(int(0.02 * T), max(T - W - 1, 1))))


def _vl_random(w):
    if w.k == 0:
        return np.zeros((w.B, w.Hkv, 0), np.int32)
    return np.stack([np.stack([synth.random_vl_index(w, b, h) for h in range(w.Hkv)])
                     for b in range(w.B)]).astype(np.int32)


def _gpu_decode(w, K, V, q, vl, n_splits=0, win_offset=0, poison=False, repeat=1):
    dt = TORCH_DT[w.dtype]
    Kd, Vd, qd = to_dev(K, w.dtype), to_dev(V, w.dtype), to_dev(q, w.dtype)
    cache = hq.HybridCache(w.B, w.Hkv, w.D, w.T, w.W, w.k, dt)
    cache.build(Kd, Vd, torch.from_numpy(vl).cuda() if w.k else None)
    if win_offset and w.W:
        cache.win_k.copy_(torch.roll(cache.win_k, win_offset, dims=2))
        cache.win_v.copy_(torch.roll(cache.win_v, win_offset, dims=2))
        cache.win_offset = win_offset
    if poison and w.k:
        g = torch.Generator(device="cpu").manual_seed(5)
        for b in range(w.B):
            for h in range(w.Hkv):
                rows = torch.from_numpy(vl[b, h].astype(np.int64)).cuda()
                cache.k_codes[b, h, rows] = torch.randint(0, 256, (w.k, w.D // 2), generator=g,
                                                          dtype=torch.uint8).cuda()
                cache.k_sz[b, h, rows] = torch.full((w.k, w.D // 32, 2), 0x7E00, dtype=torch.int16).cuda()
                cache.v_sz[b, h, rows] = torch.full((w.k, w.D // 32, 2), -1, dtype=torch.int16).cuda()
                vt = cache.v_codes[b, h].view(-1, w.D // 2, 16)
                for t in vl[b, h]:
                    vt[t // 16, :, tile16_slot(t)] = 0xFF
    kv = cache.descriptor()
    # the workspace needs no initialisation: start from garbage
    ws = torch.full((hq.hq_decode_workspace_size(kv, w.Hq, n_splits),), 0xFF, dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(repeat):
        out = torch.full((w.B, w.Hq, w.D), float("nan"), dtype=torch.float32, device="cuda")
        lse = torch.full((w.B, w.Hq), float("nan"), dtype=torch.float32, device="cuda")
        hq.hq_decode_attn(qd, w.Hq, kv, 0.0, n_splits, out, lse, ws)
        torch.cuda.synchronize()
        outs.append((out.cpu().numpy(), lse.cpu().numpy()))
    return outs if repeat > 1 else outs[0]


def _oracle(w, K, V, q, vl, units=None):
    nq = w.T - w.W
    kp, ks = quant.quantize_rows(K[:, :, :nq], 32)
    vp, vs = quant.quantize_rows(V[:, :, :nq], 32)
    return attention.decode(q, K, V, kp, ks, vp, vs, vl, w.W, units=units)


def _check(got, ref, units=None, G=1):
    o, l = got
    ro, rl = ref
    if units is not None:
        sel = [(b, i) for (b, h) in units for i in range(h * G, (h + 1) * G)]
        o = np.stack([o[b, i] for b, i in sel])
        l = np.array([l[b, i] for b, i in sel])
        ro = np.stack([ro[b, i] for b, i in sel])
        rl = np.array([rl[b, i] for b, i in sel])
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l))
    e = rel_err(o, ro)
    say(f"  max|err|/rms = {e:.3e}   lse max err = {np.max(np.abs(l - rl)):.2e}")
    assert e <= TOL
    assert np.max(np.abs(l - rl)) <= 1e-3


CASES = [
    # B, Hq, Hkv, D, T, W, k, dtype
    (1, 4, 1, 64, 512, 32, 8, "f32"),          # the tiny fp32 workload's shape
    (2, 8, 2, 128, 1000, 64, 30, "bf16"),
    (1, 8, 8, 128, 777, 16, 5, "bf16"),        # G = 1
    (2, 16, 8, 64, 1500, 32, 40, "bf16"),      # G = 2, D = 64
    (1, 32, 4, 128, 2049, 128, 90, "bf16"),    # G = 8
    (1, 32, 2, 128, 3000, 128, 100, "bf16"),   # G = 16
    (1, 8, 2, 128, 1234, 128, 61, "f16"),
    (1, 8, 2, 64, 999, 33, 17, "f32"),
    (1, 4, 1, 128, 100, 100, 0, "bf16"),       # everything in the window
    (1, 4, 1, 128, 700, 0, 0, "bf16"),         # everything INT4
    (1, 4, 2, 128, 300, 10, 290, "bf16"),      # every non-window position VL
    (1, 4, 1, 128, 1, 1, 0, "bf16"),           # one token
    (1, 4, 1, 64, 33, 0, 1, "bf16"),
    (1, 3, 3, 64, 500, 16, 10, "bf16"),        # G = 1, D = 64: 6 merge blocks, a ragged XCD grid
    (1, 2, 1, 64, 257, 8, 3, "f16"),           # G = 2: 4 merge blocks
]


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_decode_small(case):
    B, Hq, Hkv, D, T, W, k, dtype = case
    w = _workload(B, Hq, Hkv, D, T, W, k, dtype, seed=zlib.crc32(str(case).encode()) % 10000 + 10)
    say(f"decode {case}")
    K, V, q = synth.all_keys(w), synth.all_values(w), synth.all_queries(w)
    vl = _vl_random(w)
    got = _gpu_decode(w, K, V, q, vl)
    _check(got, _oracle(w, K, V, q, vl))


def _random_cases(n, seed):
    """n decode configurations drawn from a fixed seed: batch 1-3, 1-8 KV
    heads, GQA group 1-16, D 64 or 128, contexts 1-2600 with every window
    and VL budget from 0 up, fp32 / bf16 / fp16, automatic or forced split
    counts."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        Hkv = int(rng.choice([1, 2, 4, 8]))
        G = int(rng.choice([1, 2, 4, 8, 16]))
        if Hkv * G > 64:
            continue
        D = int(rng.choice([64, 128]))
        T = int(rng.integers(1, 2600))
        W = int(rng.choice([0, 1, 16, 128, T, int(rng.integers(0, T + 1))]))
        W = min(W, T)
        k = int(rng.integers(0, min(T - W, 200) + 1))
        dtype = str(rng.choice(["f32", "bf16", "f16"]))
        splits = int(rng.choice([0, 0, 1, 3, 17]))
        cases.append((int(rng.integers(1, 4)), Hkv * G, Hkv, D, T, W, k, dtype, splits))
    return cases


RANDOM_CASES = _random_cases(14, 2024)


@pytest.mark.parametrize("case", RANDOM_CASES, ids=[str(c) for c in RANDOM_CASES])
def test_decode_random_shapes(case):
    """Seeded random shapes (including empty windows and VL sets, windows
    covering the whole context and forced split counts) against the
    oracle."""
    B, Hq, Hkv, D, T, W, k, dtype, splits = case
    w = _workload(B, Hq, Hkv, D, T, W, k, dtype, seed=zlib.crc32(str(case).encode()) % 10000 + 20000)
    say(f"decode random {case}")
    K, V, q = synth.all_keys(w), synth.all_values(w), synth.all_queries(w)
    vl = _vl_random(w)
    got = _gpu_decode(w, K, V, q, vl, n_splits=splits)
    _check(got, _oracle(w, K, V, q, vl))


def test_decode_tiny_workload_with_detected_lines():
    w = synth.WORKLOADS["tiny"]
    say("decode tiny workload")
    K, V, q = synth.all_keys(w), synth.all_values(w), synth.all_queries(w)
    vl, _ = detect.detect(q[:, :, None, :], K, w.T - w.W, w.k, require_exact=False)
    got = _gpu_decode(w, K, V, q, vl)
    _check(got, _oracle(w, K, V, q, vl))
    # with W = T and k = 0 the path is plain attention: the oracle there is exact attention
    w2 = w.replace(W=w.T, k=0)
    got2 = _gpu_decode(w2, K, V, q, np.zeros((1, 1, 0), np.int32))
    ref = attention.attention(q[0], K[0, 0], V[0, 0])
    assert rel_err(got2[0][0], ref[0]) <= TOL


@pytest.mark.parametrize("n_splits", [1, 2, 7, 33, 0])
def test_decode_split_invariance(n_splits):
    w = _workload(1, 8, 2, 128, 4000, 128, 200, "bf16", seed=77)
    say(f"decode splits={n_splits}")
    K, V, q = synth.all_keys(w), synth.all_values(w), synth.all_queries(w)
    vl = _vl_random(w)
    got = _gpu_decode(w, K, V, q, vl, n_splits=n_splits)
    _check(got, _oracle(w, K, V, q, vl))


def test_decode_deterministic_and_ring_window_and_poison():
    w = _workload(2, 8, 2, 128, 3333, 128, 150, "bf16", seed=78)
    say("decode determinism / ring / poison")
    K, V, q = synth.all_keys(w), synth.all_values(w), synth.all_queries(w)
    vl = _vl_random(w)
    runs = _gpu_decode(w, K, V, q, vl, repeat=3)
    for o, l in runs[1:]:
        assert np.array_equal(o, runs[0][0]) and np.array_equal(l, runs[0][1])
    ring = _gpu_decode(w, K, V, q, vl, win_offset=37)
    assert np.array_equal(ring[0], runs[0][0])
    poisoned = _gpu_decode(w, K, V, q, vl, poison=True)
    assert np.array_equal(poisoned[0], runs[0][0])
    _check(runs[0], _oracle(w, K, V, q, vl))


def _vl_detected(w):
    """The VL set fed to decode: the oracle detector over the workload's
    64-step query history (exact on the grid inputs)."""
    K = synth.all_keys(w)
    qh = synth.all_query_histories(w)
    vl, _ = detect.detect(qh, K, w.T - w.W, w.k)
    return K, vl


def _check_planes(cache, kp, ks, vp, vs, units, nq):
    """INT4 planes written by hq_quantize_kv against the oracle quantizer,
    bit for bit: key codes (rows), value codes (TILE16, compared as logical
    rows) and both fp16 {scale, zero} planes, for the listed (b, h) units."""
    kc = cache.k_codes
    ksz = cache.k_sz
    vsz = cache.v_sz
    for i, (b, h) in enumerate(units):
        assert np.array_equal(kc[b, h, :nq].cpu().numpy(), kp[i]), ("k codes", b, h)
        assert np.array_equal(ksz[b, h, :nq].cpu().numpy().view(np.uint16), ks[i]), ("k s/z", b, h)
        assert np.array_equal(vsz[b, h, :nq].cpu().numpy().view(np.uint16), vs[i]), ("v s/z", b, h)
        vrows = tile16_codes(cache.v_codes[b, h])[:nq]
        assert np.array_equal(vrows, vp[i]), ("v codes", b, h)


def test_quantize_full_llama32k_planes():
    """Every INT4 code and fp16 scale/zero of the Llama-shaped 32K layer
    (8 KV heads x 32640 rows, K and V) bit-exact against the oracle."""
    w = synth.WORKLOADS["llama32k"]
    say("quantize full llama32k planes")
    K, V = synth.all_keys(w), synth.all_values(w)
    nq = w.T - w.W
    cache = hq.HybridCache(w.B, w.Hkv, w.D, w.T, w.W, w.k, TORCH_DT[w.dtype])
    cache.quantize(to_dev(K, w.dtype), to_dev(V, w.dtype))
    torch.cuda.synchronize()
    kp, ks = quant.quantize_rows(K[0, :, :nq])
    vp, vs = quant.quantize_rows(V[0, :, :nq])
    _check_planes(cache, kp, ks, vp, vs, [(0, h) for h in range(w.Hkv)], nq)


@pytest.mark.parametrize("name", ["llama32k", "glm32k"])
def test_decode_full_workload(name):
    w = synth.WORKLOADS[name]
    say(f"decode full workload {name}")
    K, vl = _vl_detected(w)
    V, q = synth.all_values(w), synth.all_queries(w)
    got = _gpu_decode(w, K, V, q, vl)
    _check(got, _oracle(w, K, V, q, vl))


def test_decode_qwen128k_sampled():
    """Batch 16 x 128K context: the GPU computes every (b, h); the oracle checks
    KV heads 0, 3 and 7 of sequences 0 and 15 (its inputs regenerated per slice)."""
    w = synth.WORKLOADS["qwen128k"]
    say("decode qwen128k (upload)")
    Kd, Vd = upload_kv(w)
    q = synth.all_queries(w)
    units = [(b, h) for b in (0, 15) for h in (0, 3, 7)]
    vl = np.zeros((w.B, w.Hkv, w.k), np.int32)
    for b in range(w.B):
        for h in range(w.Hkv):
            vl[b, h] = synth.random_vl_index(w, b, h)
    dt = TORCH_DT[w.dtype]
    cache = hq.HybridCache(w.B, w.Hkv, w.D, w.T, w.W, w.k, dt).build(Kd, Vd, torch.from_numpy(vl).cuda())
    del Kd, Vd
    kv = cache.descriptor()
    ws = torch.zeros(hq.hq_decode_workspace_size(kv, w.Hq, 0), dtype=torch.uint8, device="cuda")
    out = torch.empty((w.B, w.Hq, w.D), dtype=torch.float32, device="cuda")
    lse = torch.empty((w.B, w.Hq), dtype=torch.float32, device="cuda")
    say("decode qwen128k (run)")
    hq.hq_decode_attn(to_dev(q, w.dtype), w.Hq, kv, 0.0, 0, out, lse, ws)
    torch.cuda.synchronize()
    got = (out.cpu().numpy(), lse.cpu().numpy())
    say("decode qwen128k (oracle)")
    ro = np.full((w.B, w.Hq, w.D), np.nan)
    rl = np.full((w.B, w.Hq), np.nan)
    planes = ([], [], [], [])
    for b, h in units:
        Kh = synth.keys(w, b, h)
        Vh = synth.values(w, b, h)
        kp, ks = quant.quantize_rows(Kh[:w.T - w.W])
        vp, vs = quant.quantize_rows(Vh[:w.T - w.W])
        for lst, x in zip(planes, (kp, ks, vp, vs)):
            lst.append(x)
        sl = slice(h * w.G, (h + 1) * w.G)
        ro[b, sl], rl[b, sl] = attention.decode_head(q[b, sl], Kh, Vh, kp, ks, vp, vs, vl[b, h], w.W)
    _check(got, (ro, rl), units=units, G=w.G)
    say("decode qwen128k (INT4 planes of the sampled units, bit for bit)")
    _check_planes(cache, *planes, units, w.T - w.W)


@pytest.mark.parametrize("B,Hq,Hkv,D,T,W,k,dtype", [
    (2, 8, 2, 128, 1000, 64, 30, "bf16"),
    (1, 8, 2, 128, 1000, 64, 0, "bf16"),          # window only
    (1, 8, 2, 64, 999, 33, 17, "f32"),
    (1, 32, 8, 128, 32768, 128, 1638, "bf16"),    # the Llama-shaped workload (two units checked)
])
def test_decode_drop_int4(B, Hq, Hkv, D, T, W, k, dtype):
    """HQ_KV_DROP_INT4: attention over the VL and window rows only, against the
    oracle's sparse baseline."""
    say(f"drop-int4 B={B} Hq={Hq} Hkv={Hkv} D={D} T={T} W={W} k={k} {dtype}")
    w = _workload(B, Hq, Hkv, D, T, W, k, dtype, 7000 + T + k)
    K, V = synth.all_keys(w), synth.all_values(w)
    q = synth.all_queries(w)
    vl = _vl_random(w)
    dt = TORCH_DT[dtype]
    cache = hq.HybridCache(B, Hkv, D, T, W, k, dt)
    cache.build(to_dev(K, dtype), to_dev(V, dtype), torch.from_numpy(vl).cuda() if k else None)
    cache.flags = hq.HQ_KV_DROP_INT4
    kv = cache.descriptor()
    ws = torch.full((hq.hq_decode_workspace_size(kv, Hq, 0),), 0xFF, dtype=torch.uint8, device="cuda")
    out = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda")
    hq.hq_decode_attn(to_dev(q, dtype), Hq, kv, 0.0, 0, out, lse, ws)
    torch.cuda.synchronize()
    G = Hq // Hkv
    units = [(b, h) for b in range(B) for h in range(Hkv)]
    if T > 10000:
        units = [(0, 0), (0, Hkv - 1)]
    ro = np.full((B, Hq, D), np.nan)
    rl = np.full((B, Hq), np.nan)
    for b, h in units:
        sl = slice(h * G, (h + 1) * G)
        ro[b, sl], rl[b, sl] = attention.decode_sparse_head(q[b, sl], K[b, h], V[b, h], vl[b, h], W)
    _check((out.cpu().numpy(), lse.cpu().numpy()), (ro, rl), units=units, G=G)


OFF_GRID = [
    # B, Hq, Hkv, D, T, W, k, dtype, what
    (1, 8, 2, 128, 3000, 128, 100, "bf16", "plain"),    # G = 4, D = 128: the matrix-core INT4 pass
    (1, 8, 2, 128, 2500, 64, 70, "f16", "plain"),
    (1, 32, 2, 128, 2049, 128, 90, "bf16", "plain"),    # G = 16
    (2, 16, 8, 64, 1500, 32, 40, "bf16", "plain"),      # G = 2, D = 64
    (1, 8, 8, 128, 777, 16, 5, "f16", "plain"),         # G = 1
    (1, 8, 2, 128, 3000, 128, 100, "bf16", "tiny_q"),   # half the channels of q below 2^-17
    (1, 8, 2, 128, 3000, 128, 100, "f16", "tiny_q"),
    (1, 8, 2, 128, 3000, 128, 100, "bf16", "huge_q"),   # |q| up to ~6.5e4, keys scaled by 2^-14
    (1, 8, 2, 128, 3000, 128, 100, "f16", "huge_q"),
]


@pytest.mark.parametrize("case", OFF_GRID, ids=[str(c) for c in OFF_GRID])
def test_decode_off_grid(case):
    """Plain bf16 / fp16 draws (no 2^-4 grid) for K and q, and queries at
    the ends of the fp16 range the D = 128 INT4 pass converts them to: tiny
    magnitudes (the fp16 subnormal grid, absolute error below 2^-25) and
    magnitudes near 6.5e4 (the largest the fast path admits) with keys
    scaled so that the logits stay of order one."""
    B, Hq, Hkv, D, T, W, k, dtype, what = case
    seed = zlib.crc32(str(case).encode()) % 10000 + 20000
    w = synth.Workload(f"offgrid{seed}", seed, B=B, Hq=Hq, Hkv=Hkv, D=D, T=T, W=W, k=k, dtype=dtype,
                       grid=False, n_plant=max(1, int(0.02 * T)))
    say(f"decode off-grid {case}")
    K, V, q = synth.all_keys(w), synth.all_values(w), synth.all_queries(w)
    assert not detect.on_grid(K) and not detect.on_grid(q)
    if what == "tiny_q":
        q = q.copy()
        q[..., 1::2] = synth.round_dtype(q[..., 1::2].astype(np.float64) * 2.0 ** -20, dtype)
        assert np.all(np.abs(q[..., 1::2]) < 2.0 ** -17)
    elif what == "huge_q":
        q = np.clip(q.astype(np.float64) * 15000.0, -65000.0, 65000.0)
        q[..., 5] = 65000.0 * np.where(np.arange(Hq) % 2, 1.0, -1.0)   # one channel at the top of the range
        q = synth.round_dtype(q, dtype)
        K = synth.round_dtype(K.astype(np.float64) * 2.0 ** -14, dtype)
        assert 6.0e4 < np.abs(q).max() < 65504.0
    vl = _vl_random(w)
    got = _gpu_decode(w, K, V, q, vl)
    _check(got, _oracle(w, K, V, q, vl))
