"""GPU parity of hq_prefill_attn (split fp16 planes) and hq_prefill_attn_i8
(int8 MFMA over the codes) against the oracle hybrid prefill operator
(oracle/prefill.py): every output row on small prompts (ragged tails,
windows of 0 / inside / beyond the prompt, with and without vertical lines,
bf16 and fp16), and sampled rows of the full 32K-token causal prompt with
32 query / 8 KV heads and the vertical-line set the oracle detector picks
from the last 64 query rows. Bar: max |out - ref| <= 2e-3 * RMS(ref), lse
within 2e-3."""
import numpy as np
import pytest
import torch

import hybrid_precision_quantized_amd as hq
import synth
from oracle import detect, prefill
from tests.gpu_util import rel_err, say, to_dev

pytestmark = pytest.mark.gpu

TOL = 2e-3


def _inputs(w):
    q = np.stack([np.stack(synth._parallel(lambda i: synth.prefill_queries(w, b, i), [(i,) for i in range(w.Hq)]))
                  for b in range(w.B)])
    K = synth.all_keys(w)
    V = synth.all_values(w)
    return q, K, V


def _run(w, q, K, V, vl, form="split"):
    B, Hq, Hkv, T, D = w.B, w.Hq, w.Hkv, w.T, w.D
    k = vl.shape[2]
    qd, kd, vd = to_dev(q, w.dtype), to_dev(K, w.dtype), to_dev(V, w.dtype)
    vld = torch.from_numpy(np.ascontiguousarray(vl, dtype=np.int32)).cuda() if k else None
    out = torch.full((B, Hq, T, D), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, Hq, T), float("nan"), dtype=torch.float32, device="cuda")
    # the workspace needs no initialisation: start from garbage
    ws = torch.full((hq.hq_prefill_workspace_size(B, Hq, Hkv, T, D, k),), 0xFF, dtype=torch.uint8, device="cuda")
    hq.hq_prefill_attn(qd, kd, vd, B, Hq, Hkv, T, D, w.W, vld, k, 0.0, out, lse, ws, form=form)
    torch.cuda.synchronize()
    return out, lse


def _oracle(w, q, K, V, vl, rows, kv_heads=None):
    G = w.G
    kv_heads = range(w.Hkv) if kv_heads is None else kv_heads
    o = {}
    for b in range(w.B):
        for h in kv_heads:
            ro, rl = prefill.prefill_rows(q[b, h * G:(h + 1) * G], K[b, h], V[b, h], vl[b, h], w.W, rows)
            for g in range(G):
                o[(b, h * G + g)] = (ro[g], rl[g])
    return o


def _compare(got, ref, rows):
    out, lse = got
    o_got = np.stack([out[b, i, rows].cpu().numpy() for (b, i) in ref])
    o_ref = np.stack([ref[key][0] for key in ref])
    l_got = np.stack([lse[b, i, rows].cpu().numpy() for (b, i) in ref])
    l_ref = np.stack([ref[key][1] for key in ref])
    assert np.all(np.isfinite(o_got)) and np.all(np.isfinite(l_got))
    e = rel_err(o_got, o_ref)
    el = float(np.max(np.abs(l_got - l_ref)))
    say(f"   max|err|/rms = {e:.2e}, lse max|err| = {el:.2e}")
    assert e <= TOL
    assert el <= TOL


def _vl_random(w, k):
    out = np.zeros((w.B, w.Hkv, k), np.int32)
    for b in range(w.B):
        for h in range(w.Hkv):
            out[b, h] = synth.random_vl_index(w, b, h, k=k, cand_end=w.T)
    return out


FORMS = ("split", "i8")


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("B,Hq,Hkv,T,W,k,dtype", [
    (1, 4, 1, 200, 16, 10, "bf16"),
    (1, 8, 2, 333, 64, 20, "bf16"),
    (2, 4, 2, 130, 0, 0, "f16"),          # no window, no vertical lines: all quantized
    (1, 4, 1, 1, 128, 0, "bf16"),         # one token
    (1, 4, 4, 513, 600, 25, "bf16"),      # window beyond the prompt: all 16-bit
    (1, 8, 2, 1000, 128, 50, "bf16"),
    (1, 4, 1, 290, 3, 40, "f16"),
])
def test_prefill_small(B, Hq, Hkv, T, W, k, dtype, form):
    w = synth.Workload("pf", 3000 + T + W + k, B=B, Hq=Hq, Hkv=Hkv, D=128, T=T, W=W, k=k, dtype=dtype,
                       n_plant=max(1, T // 50))
    say(f"prefill small B={B} Hq={Hq} Hkv={Hkv} T={T} W={W} k={k} {dtype} {form}")
    q, K, V = _inputs(w)
    vl = _vl_random(w, k)
    rows = np.arange(T)
    _compare(_run(w, q, K, V, vl, form), _oracle(w, q, K, V, vl, rows), rows)


def _random_prefill_cases(n, seed):
    """n prompts drawn from a fixed seed: batch 1-2, 1-4 KV heads, group 1-8,
    1-1200 tokens (ragged against the 32-key and 128-query tiles), windows
    from 0 to beyond the prompt, 0-60 vertical lines, bf16 or fp16."""
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        Hkv = int(rng.choice([1, 2, 4]))
        G = int(rng.choice([1, 2, 4, 8]))
        T = int(rng.integers(1, 1200))
        W = int(rng.choice([0, 1, 31, 32, 33, 128, int(rng.integers(0, T + 2))]))
        k = int(rng.integers(0, min(T, 60) + 1))
        cases.append((int(rng.integers(1, 3)), Hkv * G, Hkv, T, W, k, str(rng.choice(["bf16", "f16"]))))
    return cases


RANDOM_PREFILL = _random_prefill_cases(8, 31)


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("case", RANDOM_PREFILL, ids=[str(c) for c in RANDOM_PREFILL])
def test_prefill_random_shapes(case, form):
    """Seeded random prompts, every output row against the oracle."""
    B, Hq, Hkv, T, W, k, dtype = case
    w = synth.Workload("pfr", 5000 + T + 7 * W + 13 * k, B=B, Hq=Hq, Hkv=Hkv, D=128, T=T, W=W, k=k,
                       dtype=dtype, n_plant=max(1, T // 50))
    say(f"prefill random {case} {form}")
    q, K, V = _inputs(w)
    vl = _vl_random(w, k)
    rows = np.arange(T)
    _compare(_run(w, q, K, V, vl, form), _oracle(w, q, K, V, vl, rows), rows)


@pytest.mark.parametrize("form", FORMS)
def test_prefill_extremes(form):
    """Plain (off-grid) rows with groups near the fp16 limit (|x| up to 6e4),
    groups below 2^-14 and constant groups, bf16: the integer form's zero-point
    operands (sums over a group, divided by 64) stay in range and the small
    groups of either form lose nothing that shows. The softmax here is peaked,
    so the bar is per element and follows from the one rounding the two forms
    share, P to fp16 for P . V (relative 2^-11 per probability): |out - ref| <=
    2^-10 sum_j p_j |v_j| + 1e-6, the sum being the oracle's output with |V|
    for V; lse within 2e-3."""
    rng = np.random.default_rng(77)
    B, Hq, Hkv, T, D, W, k = 1, 4, 1, 300, 128, 16, 6
    q = rng.standard_normal((B, Hq, T, D))
    K = rng.standard_normal((B, Hkv, T, D))
    V = rng.standard_normal((B, Hkv, T, D))
    K[:, :, ::7, 0:32] *= 3e4 / 4                     # groups reaching ~ 3e4
    K[:, :, 3::11, 32:64] = 6.0e4                     # constant groups at the top of the range
    q[:, :, ::5, 64:96] *= 1e-5                       # groups far below 2^-14
    q[:, :, 2::9, 96:128] = -2.5                      # constant query groups
    q *= 1.0 / 3e4                                    # keep the logits O(1)
    w = synth.Workload("pfx", 1, B=B, Hq=Hq, Hkv=Hkv, D=D, T=T, W=W, k=k, dtype="bf16", n_plant=1)
    qb, Kb, Vb = (synth.round_dtype(x, "bf16") for x in (q, K, V))
    vl = np.sort(rng.choice(T, (B, Hkv, k), replace=False), axis=-1).astype(np.int32)
    rows = np.arange(T)
    say(f"prefill extremes {form}")
    out, lse = _run(w, qb, Kb, Vb, vl, form)
    ref = _oracle(w, qb, Kb, Vb, vl, rows)
    mag = _oracle(w, qb, Kb, np.abs(Vb), vl, rows)
    for key in ref:
        b, i = key
        o = out[b, i].cpu().numpy()
        err = np.abs(o - ref[key][0])
        bound = 2.0 ** -10 * mag[key][0] + 1e-6
        say(f"   head {i}: max err/bound = {float(np.max(err / bound)):.3f}")
        assert np.all(np.isfinite(o)) and np.all(err <= bound)
        assert float(np.max(np.abs(lse[b, i].cpu().numpy() - ref[key][1]))) <= TOL


@pytest.mark.parametrize("form", FORMS)
def test_prefill_32k_sampled(form):
    """32K-token causal prompt, 32 query / 8 KV heads; the GPU computes every
    row of every head; the oracle checks sampled rows of KV heads 0 and 5."""
    w = synth.WORKLOADS["prefill32k"]
    say("prefill 32K (inputs)")
    q, K, V = _inputs(w)
    # the VL set: the oracle detector over the last 64 query rows
    qh = q[:, :, w.T - 64:]
    vl, _ = detect.detect(qh, K, w.T - w.W, w.k)
    say(f"prefill 32K (run, {form})")
    got = _run(w, q, K, V, vl, form)
    rows = np.array([0, 1, 2, 127, 128, 129, 255, 4095, 4096, 20011, w.T - 129, w.T - 128, w.T - 1])
    say("prefill 32K (oracle)")
    _compare(got, _oracle(w, q, K, V, vl, rows, kv_heads=(0, 5)), rows)
