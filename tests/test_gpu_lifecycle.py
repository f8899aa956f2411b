"""GPU parity of the rolling hybrid cache over many decode steps against the
oracle's lifecycle simulation (oracle/lifecycle.py): 130 decode steps
crossing two re-detections. Each step's attention output within the decode
bar; every re-detected VL set bit-exact; at the end the INT4 planes written
by the per-step eviction, the VL rows and the VL bitmap bit-exact."""
import numpy as np
import pytest
import torch

import hybrid_precision_quantized_amd as hq
import synth
from oracle import detect, lifecycle, quant
from tests.gpu_util import TORCH_DT, rel_err, say, tile16_codes, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("B,Hq,Hkv,D,T0,W,k,R,n,dtype", [
    (1, 8, 2, 128, 700, 32, 35, 64, 130, "bf16"),     # G = 4: the matrix-core INT4 pass
    (2, 4, 2, 64, 500, 16, 25, 16, 40, "f16"),        # D = 64, G = 2, a short ring (R = 16)
])
def test_rolling_cache_matches_oracle_lifecycle(B, Hq, Hkv, D, T0, W, k, R, n, dtype):
    w = synth.Workload(f"life{T0}", 9100 + T0, B=B, Hq=Hq, Hkv=Hkv, D=D, T=T0 + n, W=W, k=k, dtype=dtype,
                       R=R, n_plant=max(2, int(0.02 * (T0 + n))))
    say(f"lifecycle B={B} Hq={Hq} Hkv={Hkv} D={D} T0={T0} W={W} k={k} R={R} steps={n} {dtype}")
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
            rc.redetect()
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
