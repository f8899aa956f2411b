"""The decode step and the detector under HIP graph capture.

No entry point allocates, frees, clears memory or synchronises: each call
only enqueues kernels on the given stream, so a caller can capture a run of
decode steps (with their query-ring and eviction upkeep) and a detection in
one graph and replay it. The test captures four hq_decode_step calls and a
forced hq_detect_vlines, replays the graph three times with other eager work
and synchronisations in between, and checks every replay bit for bit against
the same calls run eagerly (same kernels, same inputs, same split plan)."""
import numpy as np
import pytest
import torch

import hybrid_precision_quantized_amd as hq
import synth
from tests.gpu_util import TORCH_DT, say, to_dev

pytestmark = pytest.mark.gpu


def test_decode_steps_and_detection_replay_in_a_graph():
    B, Hq, Hkv, D, T, W, k, R, dtype = 1, 8, 2, 128, 1500, 64, 40, 64, "bf16"
    say(f"graph: 4 decode steps + detection, B={B} Hq={Hq} Hkv={Hkv} T={T} W={W} k={k}")
    w = synth.Workload("graph", 5150, B=B, Hq=Hq, Hkv=Hkv, D=D, T=T, W=W, k=k, dtype=dtype, grid=True,
                       n_plant=20)
    K, V = synth.all_keys(w), synth.all_values(w)
    Kd, Vd = to_dev(K, dtype), to_dev(V, dtype)
    vl = np.stack([np.stack([synth.random_vl_index(w, b, h) for h in range(Hkv)]) for b in range(B)])
    cache = hq.HybridCache(B, Hkv, D, T, W, k, TORCH_DT[dtype], t_cap=(T - W + 1 + 31) // 32 * 32)
    cache.build(Kd, Vd, torch.from_numpy(vl.astype(np.int32)).cuda())
    kv = cache.descriptor()
    qs = [to_dev(synth.all_queries(w.replace(seed=w.seed + 11 * s)), dtype) for s in range(4)]
    ring = to_dev(synth.all_query_histories(w, R), dtype)
    ws = torch.zeros((hq.hq_decode_workspace_size(kv, Hq, 0),), dtype=torch.uint8, device="cuda")
    det_ws = torch.zeros((hq.hq_detect_workspace_size(B, Hkv, T - W, k),), dtype=torch.uint8, device="cuda")

    def run(outs, lses, idx, stream=None):
        for s in range(4):
            hq.hq_decode_step(qs[s], Hq, kv, 0.0, 0, outs[s], lses[s], ws, q_acc=ring, R=R, step=60 + s,
                              evict=True, stream=stream)
        hq.hq_detect_vlines(None, ring, B, Hq, Hkv, D, R, 63, True, Kd, T, T - W, k, hq.HQ_DETECT_MATMUL,
                            idx, None, det_ws, stream=stream)

    def bufs():
        return ([torch.full((B, Hq, D), float("nan"), device="cuda") for _ in range(4)],
                [torch.full((B, Hq), float("nan"), device="cuda") for _ in range(4)],
                torch.full((B, Hkv, k), -1, dtype=torch.int32, device="cuda"))

    # eager reference (the ring, the INT4 row T - W and the workspaces end in
    # the same state after every run of these calls)
    eo, el, ei = bufs()
    run(eo, el, ei)
    torch.cuda.synchronize()
    ring_after = ring.clone()

    go, gl, gi = bufs()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            run(go, gl, gi, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    scratch_o = torch.empty((B, Hq, D), device="cuda")
    scratch_l = torch.empty((B, Hq), device="cuda")
    for rep in range(3):
        for t in go + gl:
            t.fill_(float("nan"))
        gi.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        for s_ in range(4):
            assert torch.equal(go[s_], eo[s_]) and torch.equal(gl[s_], el[s_]), f"replay {rep}, step {s_}"
        assert torch.equal(gi, ei), f"replay {rep}: detector set"
        assert torch.equal(ring, ring_after)
        # eager work between replays, on the same workspace and cache
        hq.hq_decode_attn(qs[(rep + 1) % 4], Hq, kv, 0.0, 0, scratch_o, scratch_l, ws)
        torch.cuda.synchronize()
    say("   3 replays bitwise equal to the eager run")


def test_redetection_replays_in_a_graph():
    """hq_vl_redetect (candidate scores, then the in-place update) captured
    in a graph and replayed three times on one rolling cache, with eager work
    and synchronisations between the replays. The update changes the cache,
    so every replay is compared with the same call run eagerly on a twin
    cache in the same state: index list, bitmap and VL rows bit for bit."""
    B, Hq, Hkv, D, T, W, k, R, dtype = 1, 8, 2, 128, 2000, 32, 60, 64, "bf16"
    say(f"graph: re-detection, B={B} Hq={Hq} Hkv={Hkv} T={T} W={W} k={k}")
    rng = np.random.default_rng(77)
    nq = T - W
    grid = lambda shape: np.rint(rng.standard_normal(shape) * 16) / 16
    Kd, Vd = to_dev(grid((B, Hkv, T, D)).astype(np.float32), dtype), to_dev(grid((B, Hkv, T, D)).astype(np.float32), dtype)
    vl = np.stack([np.sort(rng.choice(nq - R, k, replace=False)) for _ in range(Hkv)])[None].astype(np.int32)
    caches = []
    for _ in range(2):
        c = hq.HybridCache(B, Hkv, D, T, W, k, TORCH_DT[dtype], win_cap=W + R)
        c.build(Kd, Vd, torch.from_numpy(vl).cuda())
        caches.append(c)
    eager, graphed = caches
    rings = [to_dev(grid((B, Hq, R, D)).astype(np.float32), dtype) for _ in range(3)]
    ring = rings[0].clone()
    wse = torch.zeros(hq.hq_vl_redetect_workspace_size(eager.descriptor()), dtype=torch.uint8, device="cuda")
    wsg = torch.zeros_like(wse)
    p0 = nq - R

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    kvg = graphed.descriptor()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            hq.hq_vl_redetect(kvg, graphed.vl_idx, p0, ring, Hq, R, wsg, stream=s.cuda_stream)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(3):
        ring.copy_(rings[rep])                   # a new query ring for each replay
        hq.hq_vl_redetect(eager.descriptor(), eager.vl_idx, p0, rings[rep], Hq, R, wse)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name in ("vl_idx", "vl_bits", "vl_k", "vl_v"):
            assert torch.equal(getattr(graphed, name), getattr(eager, name)), f"replay {rep}: {name}"
        # eager work between replays
        wsg.fill_(0xFF)
        torch.cuda.synchronize()
