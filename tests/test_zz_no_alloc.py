"""hq_decode_attn_noalloc (split partials in the library's fixed device
array, for callers that cannot allocate) against hq_decode_attn with a
workspace: two calls in a row, the second with smaller inputs, each bitwise
equal to the workspace entry point's output and within the decode bar of the
oracle."""
import numpy as np
import pytest
import torch

import hybrid_precision_quantized_amd as hq
import synth
from oracle import attention, quant
from tests.gpu_util import TORCH_DT, rel_err, say, to_dev

pytestmark = pytest.mark.gpu


def _case(B, Hq, Hkv, D, T, W, k, dtype, seed):
    w = synth.Workload(f"noalloc{seed}", seed, B=B, Hq=Hq, Hkv=Hkv, D=D, T=T, W=W, k=k, dtype=dtype,
                       grid=False, n_plant=max(1, int(0.02 * T)))
    K, V, q = synth.all_keys(w), synth.all_values(w), synth.all_queries(w)
    vl = np.stack([np.stack([synth.random_vl_index(w, b, h) for h in range(Hkv)]) for b in range(B)])
    cache = hq.HybridCache(B, Hkv, D, T, W, k, TORCH_DT[dtype])
    cache.build(to_dev(K, dtype), to_dev(V, dtype), torch.from_numpy(vl.astype(np.int32)).cuda())
    return w, K, V, q, vl, cache


def _outs(w, qd, kv, noalloc):
    out = torch.full((w.B, w.Hq, w.D), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((w.B, w.Hq), float("nan"), dtype=torch.float32, device="cuda")
    if noalloc:
        hq.hq_decode_attn_noalloc(qd, w.Hq, kv, 0.0, 0, out, lse)
    else:
        ws = torch.full((hq.hq_decode_workspace_size(kv, w.Hq, 0),), 0xFF, dtype=torch.uint8, device="cuda")
        hq.hq_decode_attn(qd, w.Hq, kv, 0.0, 0, out, lse, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def test_noalloc_matches_workspace_entry_point_twice():
    cases = [(2, 32, 8, 128, 20000, 128, 1000, "bf16", 31),    # first call: larger
             (1, 8, 2, 128, 1500, 64, 40, "bf16", 32)]         # second call: smaller
    for c in cases:
        say(f"noalloc decode {c}")
        w, K, V, q, vl, cache = _case(*c)
        kv = cache.descriptor()
        assert hq.hq_decode_workspace_size(kv, w.Hq, 0) <= hq.HQ_DECODE_SCRATCH_BYTES
        qd = to_dev(q, w.dtype)
        got = _outs(w, qd, kv, noalloc=True)
        ref = _outs(w, qd, kv, noalloc=False)
        assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1])
        nq = w.T - w.W
        kp, ks = quant.quantize_rows(K[:, :, :nq])
        vp, vs = quant.quantize_rows(V[:, :, :nq])
        ro, rl = attention.decode(q, K, V, kp, ks, vp, vs, vl, w.W)
        e = rel_err(got[0], ro)
        say(f"  max|err|/rms = {e:.3e}")
        assert e <= 2e-3 and np.max(np.abs(got[1] - rl)) <= 1e-3


def test_noalloc_rejects_sizes_beyond_the_array():
    kv = hq.HybridCache(16, 8, 128, 4096, 128, 100, torch.bfloat16).descriptor()
    assert hq.hq_decode_workspace_size(kv, 32, 256) > hq.HQ_DECODE_SCRATCH_BYTES
    out = torch.empty((16, 32, 128), dtype=torch.float32, device="cuda")
    q = torch.zeros((16, 32, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(hq.HQError) as ei:
        hq.hq_decode_attn_noalloc(q, 32, kv, 0.0, 256, out, None)
    assert ei.value.status == hq.HQ_ERR_WORKSPACE
