"""GPU checks of hq_decode_step against hq_decode_attn and the oracle packing.

* The attention outputs and lse are bitwise those of hq_decode_attn on the
  same cache (same kernels, same split plan).
* The step's queries land in slot step % R of the detector's query ring and
  no other ring byte changes.
* With eviction, INT4 row T - W holds the oracle packing (codes, fp16 scale
  and zero: bit-exact) of the window's oldest row, read from ring row
  win_offset; no other byte of the four INT4 planes changes. Without
  eviction, or with W = 0, the planes are untouched."""
import numpy as np
import pytest
import torch

import hybrid_precision_quantized_amd as hq
import synth
from oracle import quant
from tests.gpu_util import TORCH_DT, say, sz_bits, tile16_codes, to_dev

pytestmark = pytest.mark.gpu


def _round_up(x, m):
    return (x + m - 1) // m * m


def _planes(cache):
    return [cache.k_codes.clone(), cache.k_sz.clone(), cache.v_codes.clone(), cache.v_sz.clone()]


@pytest.mark.parametrize("B,Hq,Hkv,D,T,W,k,dtype,win_offset,step,R,evict", [
    (1, 8, 2, 128, 700, 64, 20, "bf16", 0, 70, 64, True),
    (2, 16, 4, 128, 1000, 128, 30, "bf16", 37, 63, 64, True),
    (1, 32, 8, 128, 4096, 128, 204, "bf16", 100, 127, 64, True),
    (1, 4, 1, 64, 300, 32, 8, "f32", 5, 3, 8, True),
    (1, 8, 8, 128, 517, 16, 10, "f16", 15, 0, 64, True),      # row T - W = 501: mid-tile, odd slot
    (1, 8, 2, 128, 200, 0, 5, "bf16", 0, 5, 64, True),       # W = 0: nothing to evict
    (1, 8, 2, 128, 700, 64, 20, "bf16", 9, 11, 16, False),   # ring only
    (1, 3, 3, 64, 400, 16, 6, "bf16", 3, 63, 64, True),      # 6 merge blocks, upkeep after a ragged XCD grid
])
def test_decode_step(B, Hq, Hkv, D, T, W, k, dtype, win_offset, step, R, evict):
    say(f"decode_step B={B} Hq={Hq} Hkv={Hkv} D={D} T={T} W={W} k={k} {dtype} off={win_offset} "
        f"step={step} R={R} evict={evict}")
    w = synth.Workload(f"step{T}", 4100 + T + W, B=B, Hq=Hq, Hkv=Hkv, D=D, T=T, W=W, k=k, dtype=dtype,
                       grid=(dtype != "f32"), n_plant=max(1, T // 50))
    K = synth.all_keys(w)
    V = synth.all_values(w)
    q = synth.all_queries(w)
    Kd, Vd, qd = to_dev(K, dtype), to_dev(V, dtype), to_dev(q, dtype)
    vl = np.stack([np.stack([synth.random_vl_index(w, b, h) for h in range(Hkv)]) for b in range(B)])
    cache = hq.HybridCache(B, Hkv, D, T, W, k, TORCH_DT[dtype], t_cap=_round_up(T - W + 1, 32))
    cache.build(Kd, Vd, torch.from_numpy(vl.astype(np.int32)).cuda() if k else None)
    if win_offset and W:
        cache.win_k.copy_(torch.roll(cache.win_k, win_offset, dims=2))
        cache.win_v.copy_(torch.roll(cache.win_v, win_offset, dims=2))
        cache.win_offset = win_offset
    kv = cache.descriptor()
    ws = torch.full((hq.hq_decode_workspace_size(kv, Hq, 0),), 0xFF, dtype=torch.uint8, device="cuda")
    out_a = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
    lse_a = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda")
    hq.hq_decode_attn(qd, Hq, kv, 0.0, 0, out_a, lse_a, ws)
    torch.cuda.synchronize()
    before = _planes(cache)

    g = torch.Generator(device="cpu").manual_seed(T)
    ring0 = torch.randint(-30000, 30000, (B, Hq, R, D * qd.element_size() // 2), generator=g,
                          dtype=torch.int16).cuda()
    ring = ring0.clone()
    out_b = torch.full_like(out_a, float("nan"))
    lse_b = torch.full_like(lse_a, float("nan"))
    hq.hq_decode_step(qd, Hq, kv, 0.0, 0, out_b, lse_b, ws, q_acc=ring, R=R, step=step, evict=evict)
    torch.cuda.synchronize()

    assert torch.equal(out_a, out_b) and torch.equal(lse_a, lse_b)
    slot = step % R
    qbits = qd.contiguous().view(torch.int16).view(B, Hq, -1)
    assert torch.equal(ring[:, :, slot], qbits)
    others = [r for r in range(R) if r != slot]
    assert torch.equal(ring[:, :, others], ring0[:, :, others])

    after = _planes(cache)
    row = T - W
    if not (evict and W > 0):
        for x, y in zip(before, after):
            assert torch.equal(x, y)
        return
    kp, kz = quant.quantize_rows(K[:, :, row:row + 1], 32)
    vp, vz = quant.quantize_rows(V[:, :, row:row + 1], 32)
    kc, ks, vc, vs = after
    assert np.array_equal(kc.cpu().numpy()[:, :, row], kp[:, :, 0])
    assert np.array_equal(sz_bits(ks)[:, :, row], kz[:, :, 0])
    assert np.array_equal(tile16_codes(vc)[:, :, row], vp[:, :, 0])
    assert np.array_equal(sz_bits(vs)[:, :, row], vz[:, :, 0])
    # nothing else changed
    keep = [r for r in range(cache.t_cap) if r != row]
    assert np.array_equal(kc.cpu().numpy()[:, :, keep], before[0].cpu().numpy()[:, :, keep])
    assert np.array_equal(sz_bits(ks)[:, :, keep], sz_bits(before[1])[:, :, keep])
    assert np.array_equal(tile16_codes(vc)[:, :, keep], tile16_codes(before[2])[:, :, keep])
    assert np.array_equal(sz_bits(vs)[:, :, keep], sz_bits(before[3])[:, :, keep])


def test_decode_step_then_next_step_reads_the_packed_row():
    """After a step with eviction, advancing the window (T + 1, the new token
    in the freed ring row) gives the same attention as a cache built from
    scratch for T + 1: the packed row is what hq_quantize_kv would write."""
    B, Hq, Hkv, D, T, W, k = 1, 8, 2, 128, 900, 64, 16
    w = synth.Workload("step_next", 4999, B=B, Hq=Hq, Hkv=Hkv, D=D, T=T + 1, W=W, k=k, dtype="bf16",
                       grid=True, n_plant=18)
    K = synth.all_keys(w)                 # T + 1 positions
    V = synth.all_values(w)
    q = synth.all_queries(w)
    Kd, Vd, qd = to_dev(K, "bf16"), to_dev(V, "bf16"), to_dev(q, "bf16")
    vl = np.stack([np.stack([synth.random_vl_index(w.replace(T=T), 0, h, k=k) for h in range(Hkv)])])
    vld = torch.from_numpy(vl.astype(np.int32)).cuda()
    cap = _round_up(T + 1 - W, 32)
    # rolling cache at T, stepped once
    c1 = hq.HybridCache(B, Hkv, D, T, W, k, torch.bfloat16, t_cap=cap).build(
        Kd[:, :, :T].contiguous(), Vd[:, :, :T].contiguous(), vld)
    kv = c1.descriptor()
    ws = torch.empty((hq.hq_decode_workspace_size(kv, Hq, 0) * 2,), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    hq.hq_decode_step(qd, Hq, kv, 0.0, 0, out, lse, ws, evict=True)
    c1.T = T + 1
    c1.win_k[:, :, c1.win_offset] = Kd[:, :, T]
    c1.win_v[:, :, c1.win_offset] = Vd[:, :, T]
    c1.win_offset = (c1.win_offset + 1) % W
    out1 = torch.empty_like(out)
    lse1 = torch.empty_like(lse)
    hq.hq_decode_attn(qd, Hq, c1.descriptor(), 0.0, 0, out1, lse1, ws)
    # built from scratch at T + 1
    c2 = hq.HybridCache(B, Hkv, D, T + 1, W, k, torch.bfloat16, t_cap=cap).build(Kd, Vd, vld)
    out2 = torch.empty_like(out)
    lse2 = torch.empty_like(lse)
    hq.hq_decode_attn(qd, Hq, c2.descriptor(), 0.0, 0, out2, lse2, ws)
    torch.cuda.synchronize()
    # same INT4 planes over [0, T + 1 - W), and the same window contents in ring order
    n = T + 1 - W
    assert torch.equal(c1.k_codes[:, :, :n], c2.k_codes[:, :, :n])
    assert torch.equal(c1.k_sz[:, :, :n], c2.k_sz[:, :, :n])
    assert np.array_equal(tile16_codes(c1.v_codes)[:, :, :n], tile16_codes(c2.v_codes)[:, :, :n])
    assert torch.equal(c1.v_sz[:, :, :n], c2.v_sz[:, :, :n])
    # window rows agree position by position; the split plan is the same, so
    # only the window's ring order differs: the outputs agree to rounding
    assert torch.allclose(out1, out2, rtol=0, atol=1e-5)
    assert torch.allclose(lse1, lse2, rtol=0, atol=1e-5)
