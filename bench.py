"""Benchmark of the HyQuant decode hot path on one MI355X.

One step = one steady-state decode step of one attention layer over its
hybrid KV cache:
  1. hq_decode_step: attention over INT4 + VL + window with the split-K LSE
     merge; in the same launches the step's queries go into the detector's
     64-slot ring and the window's oldest token is packed into INT4;
  2. every 64th step (step mod 64 == 63) hq_detect_vlines scores the ring
     (Q_acc . K^T column sums, top-k) and the new VL set is installed for the
     next step (hq_vl_bitmap + hq_gather_rows of the VL keys and values).
With --separate-upkeep the upkeep runs as its own calls before the
attention (hq_detect_vlines with the new queries, hq_quantize_kv_pair, then
hq_decode_attn), four launches per step instead of two.
Steps rotate over `--copies` independent layer caches (>= 1 GB in total) so
that the 256 MB Infinity Cache cannot hold the working set: every step reads
its cache from HBM as it would in a model with many layers. All inputs are
seeded synthetic tensors already resident in HBM when timing starts.

Prints one JSON line (rank 0). `value` is the algorithmic HBM bytes of a
step divided by the measured step time (GB/s); `ms_per_step` is the step
time. `roofline` is the decode call alone (split kernel + merge kernel),
timed with HIP events on the launch stream around back-to-back calls (and,
for the spread, per call: p10 / p50 / p90), beside the HBM read
ceiling (a 2 GiB sequential read), the time of a plain read of the call's
own bytes at the same size, and the median of launches that reuse one cache
copy ("warm": what the Infinity Cache can hold may come from it).
`cpu_baseline` is the CPU oracle on a bounded sample of the same step.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode attention µs/step and achieved HBM GB/s (% of peak) at 32K/128K ctx"
PREFILL_METRIC = "hybrid prefill attention ms/step and algorithmic TFLOP/s (causal 32K prompt)"
PEAK_HBM_GBS = 8000.0
PEAK_MFMA_F16_TFLOPS = 2500.0          # dense f16 / bf16 MFMA
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--workload", default="llama32k",
                    choices=["llama32k", "qwen128k", "glm32k", "prefill32k"],
                    help="decode workloads, or prefill32k: the causal hybrid prefill of a 32K prompt")
    ap.add_argument("--copies", type=int, default=0, help="layer caches to rotate over (0 = auto, >= 1 GB)")
    ap.add_argument("--detect-method", default="matmul", choices=["matmul", "qsum", "cache", "mass"],
                    help="matmul: Q_acc K^T on MFMA; qsum: summed queries, GEMV; cache: summed "
                         "queries against the INT4 key cache (hq_detect_vlines_cache); mass: "
                         "attention-mass scores (hq_detect_vlines_mass)")
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--kernel-launches", type=int, default=200)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--ablation", action="store_true",
                    help="decode settings of the ablation (hybrid, sparse, window only, strict K4V4, "
                         "all 16-bit): bytes, time and error against exact attention")
    ap.add_argument("--graph", action="store_true",
                    help="capture the timed steps in one HIP graph and time its replay")
    ap.add_argument("--separate-upkeep", action="store_true",
                    help="queries to the ring and the eviction as separate calls (hq_decode_attn)")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="also run one plain device copy of this many MB (counter calibration)")
    return ap.parse_args()


def source_hash(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "hybrid_precision_quantized_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(decode attention shards by KV head or batch with no communication; "
              "see the design notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import hybrid_precision_quantized_amd as hq
    import synth

    hq.lib()                                   # fail loudly if the library is missing
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.workload == "prefill32k":
        return main_prefill(args)
    if args.ablation:
        return main_ablation(args)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    w = synth.WORKLOADS[args.workload]
    dt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[w.dtype]
    B, Hq, Hkv, D, T, W, k = w.B, w.Hq, w.Hkv, w.D, w.T, w.W, w.k
    R = 64
    nq = T - W
    method = hq.HQ_DETECT_MATMUL if args.detect_method == "matmul" else hq.HQ_DETECT_QSUM
    from_cache = args.detect_method == "cache"
    by_mass = args.detect_method == "mass"

    # ------------------------------------------------------------ inputs
    t_setup = time.time()

    def to_dev(x32):
        if w.dtype == "bf16":
            return torch.from_numpy(synth.f32_to_bf16_bits(x32).view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(x32)).to(dev)

    K0 = torch.empty((B, Hkv, T, D), dtype=dt, device=dev)
    V0 = torch.empty_like(K0)
    for b in range(B):
        K0[b].copy_(to_dev(np.stack([synth.keys(w, b, h) for h in range(Hkv)])))
        V0[b].copy_(to_dev(np.stack([synth.values(w, b, h) for h in range(Hkv)])))
    q_steps = to_dev(np.stack([synth.all_queries(w.replace(seed=w.seed + 17 * s)) for s in range(4)]))
    q_hist = to_dev(synth.all_query_histories(w))

    layer_bytes = (2 * K0.numel() * K0.element_size()) + 2 * B * Hkv * T * (D // 2 + D // 16)
    copies = args.copies or max(1, int(np.ceil(1.2e9 / layer_bytes)))
    caches, Ks, Vs, qaccs = [], [], [], []
    idx_new = torch.zeros((B, Hkv, k), dtype=torch.int32, device=dev)
    det_ws = torch.zeros(hq.hq_detect_mass_workspace_size(B, Hq, Hkv, R, T, nq) if by_mass
                         else hq.hq_detect_workspace_size(B, Hkv, nq, k), dtype=torch.uint8, device=dev)
    for c in range(copies):
        Kc = K0 if c == 0 else K0.clone()
        Vc = V0 if c == 0 else V0.clone()
        qa = q_hist.clone()
        # one spare INT4 row: the window's oldest token is packed into row T - W
        cache = hq.HybridCache(B, Hkv, D, T, W, k, dt, t_cap=(nq + 1 + 31) // 32 * 32)
        cache.quantize(Kc, Vc)
        if from_cache:
            hq.hq_detect_vlines_cache(None, qa, Hq, R, 0, True, cache.descriptor(), nq, k, idx_new, None, det_ws)
        elif by_mass:
            hq.hq_detect_vlines_mass(None, qa, B, Hq, Hkv, D, R, 0, True, Kc, T, nq, k, idx_new, None, det_ws)
        else:
            hq.hq_detect_vlines(None, qa, B, Hq, Hkv, D, R, 0, True, Kc, T, nq, k, method, idx_new, None,
                                det_ws)
        cache.set_vl(Kc, Vc, idx_new)
        cache.set_window(Kc, Vc)
        caches.append(cache)
        Ks.append(Kc)
        Vs.append(Vc)
        qaccs.append(qa)
    descs = [c.descriptor() for c in caches]
    dec_ws = [torch.zeros(hq.hq_decode_workspace_size(d, Hq, args.splits), dtype=torch.uint8, device=dev)
              for d in descs]
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    t_setup = time.time() - t_setup

    n_heads = B * Hkv

    def detect(s, c, force, q_new=None):
        if from_cache:
            return hq.hq_detect_vlines_cache(q_new, qaccs[c], Hq, R, s, force, descs[c], nq, k, idx_new, None,
                                             det_ws)
        if by_mass:
            return hq.hq_detect_vlines_mass(q_new, qaccs[c], B, Hq, Hkv, D, R, s, force, Ks[c], T, nq, k,
                                            idx_new, None, det_ws)
        return hq.hq_detect_vlines(q_new, qaccs[c], B, Hq, Hkv, D, R, s, force, Ks[c], T, nq, k, method,
                                   idx_new, None, det_ws)

    def install(c, cache, Kc, Vc):
        hq.hq_vl_bitmap(idx_new, n_heads, k, cache.t_cap, cache.vl_bits)
        hq.hq_gather_rows(Kc, n_heads, T, D, idx_new, k, cache.vl_k)
        hq.hq_gather_rows(Vc, n_heads, T, D, idx_new, k, cache.vl_v)

    launch_stream = stream           # the stream the step's calls go to

    def step(s: int):
        c = s % copies
        cache, Kc, Vc = caches[c], Ks[c], Vs[c]
        qn = q_steps[s % q_steps.shape[0]]
        if args.separate_upkeep:
            if detect(s, c, False, qn):
                install(c, cache, Kc, Vc)
            # the token leaving the window (position T - W) goes to INT4 row T - W
            hq.hq_quantize_kv_pair(Kc[:, :, nq:], Vc[:, :, nq:], n_heads, 1, D, T * D, D,
                                   cache.k_codes, cache.k_sz, cache.v_codes, cache.v_sz,
                                   cache.t_cap, nq)
            hq.hq_decode_attn(qn, Hq, descs[c], 0.0, args.splits, out, lse, dec_ws[c])
            return
        hq.hq_decode_step(qn, Hq, descs[c], 0.0, args.splits, out, lse, dec_ws[c],
                          q_acc=qaccs[c], R=R, step=s, evict=True, stream=launch_stream.cuda_stream)
        # the queries went into the ring with the step; the detector has work
        # only on the ring's last slot, so the loop calls it there alone
        if s % R == R - 1 and detect(s, c, False):
            install(c, cache, Kc, Vc)

    # ------------------------------------------------------------ timed steps
    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    base = args.warmup
    if args.graph:
        # the same steps captured once; the replay is the timed region (the
        # library only enqueues kernels, so every call is capturable)
        graph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        launch_stream = cap
        with torch.cuda.stream(cap):
            with torch.cuda.graph(graph, stream=cap):
                for s in range(base, base + args.steps):
                    step(s)
        launch_stream = stream
        stream.wait_stream(cap)
        torch.cuda.synchronize()
    e0.record(stream)
    h0 = time.perf_counter()
    if args.graph:
        graph.replay()
    else:
        for s in range(base, base + args.steps):
            step(s)
    h1 = time.perf_counter()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_total = e0.elapsed_time(e1)
    host_us_per_step = (h1 - h0) * 1e6 / args.steps     # enqueue cost of the timed loop
    ms_per_step = ms_total / args.steps
    n_detect = sum(1 for s in range(base, base + args.steps) if s % R == R - 1)

    # ------------------------------------------------------------ decode kernels alone
    # hq_decode_attn (split kernel + merge kernel) back to back, one event pair
    # around all the calls: the mean call time without per-call event packets
    c0 = torch.cuda.Event(enable_timing=True)
    c1 = torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for i in range(args.kernel_launches):
        hq.hq_decode_attn(q_steps[i % q_steps.shape[0]], Hq, descs[i % copies], 0.0, args.splits, out, lse,
                          dec_ws[i % copies])
    c1.record(stream)
    torch.cuda.synchronize()
    dec_us = c0.elapsed_time(c1) * 1e3 / args.kernel_launches
    # the spread: every call bracketed by its own events (which add their own time)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.kernel_launches)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.kernel_launches)]
    for i in range(args.kernel_launches):
        c = i % copies
        starts[i].record(stream)
        hq.hq_decode_attn(q_steps[i % q_steps.shape[0]], Hq, descs[c], 0.0, args.splits, out, lse, dec_ws[c])
        ends[i].record(stream)
    torch.cuda.synchronize()
    durs = np.array([s.elapsed_time(e) * 1e3 for s, e in zip(starts, ends)])   # us
    dec_pct = np.percentile(durs, [10, 50, 90])

    # ------------------------------------------------------------ detector alone (amortized share)
    d0 = torch.cuda.Event(enable_timing=True)
    d1 = torch.cuda.Event(enable_timing=True)
    n_det = 20
    d0.record(stream)
    for i in range(n_det):
        detect(0, i % copies, True)
    d1.record(stream)
    torch.cuda.synchronize()
    det_us = d0.elapsed_time(d1) * 1e3 / n_det

    # ------------------------------------------------------------ HBM read ceiling, same run
    stream_gbs = stream_read_ceiling(torch, hq, dev, stream)

    # ------------------------------------------------------------ warm launches (after the rest)
    # one copy every launch, so that a cache smaller than the 256 MB Infinity
    # Cache may be served from it (labelled, never the roofline figure)
    for i in range(args.kernel_launches):
        starts[i].record(stream)
        hq.hq_decode_attn(q_steps[i % q_steps.shape[0]], Hq, descs[0], 0.0, args.splits, out, lse, dec_ws[0])
        ends[i].record(stream)
    torch.cuda.synchronize()
    warm_us = float(np.median([s.elapsed_time(e) * 1e3 for s, e in zip(starts, ends)]))

    if args.calib_copy_mb:
        a = torch.empty(args.calib_copy_mb * (1 << 20) // 4, dtype=torch.float32, device=dev).fill_(1.0)
        b_ = torch.empty_like(a)
        b_.copy_(a)
        torch.cuda.synchronize()

    # ------------------------------------------------------------ bytes
    hp = K0.element_size()
    units = B * Hkv
    dec_bytes = (units * ((nq - k) * (D + (D // 32) * 8) + (k + W) * 2 * D * hp + (T - W + 31) // 32 * 4)
                 + B * Hq * D * hp + B * Hq * D * 4 + B * Hq * 4)
    det_bytes = units * nq * D * hp + B * Hq * R * D * hp + units * k * 4
    gather_bytes = 2 * units * k * D * hp * 2 + units * (caches[0].t_cap // 32) * 4
    evict_bytes = 2 * units * (D * hp + D // 2 + (D // 32) * 4)
    acc_bytes = 2 * B * Hq * D * hp
    step_bytes = dec_bytes + evict_bytes + acc_bytes + (det_bytes + gather_bytes) * n_detect / args.steps
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = dec_bytes / (dec_us * 1e-6) / 1e9
    # the same read at this size: a plain sequential read of dec_bytes,
    # rotated past the Infinity Cache and event-timed per launch like the call
    same_us = stream_read_same_bytes_us(torch, hq, dev, stream, dec_bytes, args.kernel_launches)

    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        try:
            tr = json.load(open(TRAFFIC_FILE))
            rec = tr.get(args.workload)
            if rec and rec.get("source_hash") == source_hash("hq_decode.hip", "hq_common.h", "hq_int4.h") \
                    and rec.get("splits", 0) == args.splits:
                traffic = rec["bytes_per_launch"]
        except (OSError, ValueError, KeyError):
            traffic = None

    # ------------------------------------------------------------ CPU oracle baseline
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args.cpu_seconds, step_bytes)

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "us_per_step": round(ms_per_step * 1e3, 3),
        "host_enqueue_us_per_step": round(host_us_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4+bf16 (fp32 accumulate)" if w.dtype == "bf16" else f"int4+{w.dtype}",
        "data": "synthetic (seeded; shapes of the named model's attention layer, random-init values)",
        "config": {
            "workload": f"{args.workload}: one decode step of one attention layer, B {B}, "
                        f"{Hq} q / {Hkv} kv heads, head_dim {D}, context {T}, window {W}, "
                        f"VL budget {k}, INT4 group 32 with fp16 scale/zero",
            "global_batch": B, "seq_len": T, "parallelism": "none (1 GPU)",
            "layer_copies_rotated": copies, "detect_method": args.detect_method,
            "decode_splits": hq.hq_decode_auto_splits(descs[0], Hq) if args.splits == 0 else args.splits,
            "detect_every": R, "detections_in_timed_steps": n_detect,
            "timed_as": "one HIP graph replay of the steps" if args.graph else "stream launches per step",
            "step_calls": ("hq_detect_vlines(q) + hq_quantize_kv_pair + hq_decode_attn" if args.separate_upkeep
                           else "hq_decode_step (+ hq_detect_vlines every 64th step)"),
        },
        "roofline": {
            "kernel": "decode_kernel (hq_decode_attn)",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "traffic_unit": "bytes per hq_decode_attn call (rocprofv3 FETCH_SIZE + WRITE_SIZE, calibrated)",
            "traffic_over_algorithmic": (round(traffic / dec_bytes, 4) if traffic else None),
            "algorithmic_bytes_per_launch": int(dec_bytes),
            "avg_launch_us": round(dec_us, 3),
            "avg_launch_us_timed_as": "one event pair around back-to-back hq_decode_attn calls "
                                      "(split kernel + merge kernel each)",
            "bracketed_call_us_p10_p50_p90": [round(float(x), 3) for x in dec_pct],
            "warm_launch_us_median": round(warm_us, 3),
            "stream_read_gbs": round(stream_gbs, 1),
            "frac_of_stream_read": round(achieved / stream_gbs, 4),
            "stream_read_same_bytes_us": round(same_us, 3),
            "frac_of_stream_read_same_bytes": round(same_us / dec_us, 4),
        },
        "detector": {"us_per_detection": round(det_us, 2), "method": args.detect_method,
                     "overhead_vs_64_decode_kernels": round(det_us / (64 * dec_us), 4)},
        "step_bytes": int(step_bytes),
        "setup_s": round(t_setup, 1),
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def main_ablation(args):
    """Decode-step ablation on one workload ([MR] "Improvements and Ablation
    Studies": Table 12, keeping the low-precision long tail against dropping
    it; Table 14, memory overhead against strict K4V4). Settings, all on the
    same synthetic layer and the same detected VL set:
      hybrid      INT4 majority + VL + window (the method);
      sparse      VL + window only (HQ_KV_DROP_INT4);
      window      the window only;
      k4v4        every position INT4 (k = W = 0);
      bf16        every position 16-bit (W = T), i.e. plain attention.
    For each: the algorithmic bytes of one hq_decode_attn call, its time
    (HIP events, caches rotated past the Infinity Cache), the bytes held in
    the cache for the layer, and the output error against exact attention
    (fp32 on the GPU over the 16-bit keys and values)."""
    import torch
    import hybrid_precision_quantized_amd as hq
    import synth

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    w = synth.WORKLOADS[args.workload]
    B, Hq, Hkv, D, T, W, k = w.B, w.Hq, w.Hkv, w.D, w.T, w.W, w.k
    G = Hq // Hkv
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float16
    hp = 2

    def to_dev(x32):
        return torch.from_numpy(synth.f32_to_bf16_bits(x32).view(np.int16)).to(dev).view(torch.bfloat16)

    K = torch.empty((B, Hkv, T, D), dtype=dt, device=dev)
    V = torch.empty_like(K)
    for b in range(B):
        K[b].copy_(to_dev(np.stack([synth.keys(w, b, h) for h in range(Hkv)])))
        V[b].copy_(to_dev(np.stack([synth.values(w, b, h) for h in range(Hkv)])))
    q = to_dev(synth.all_queries(w))
    q_hist = to_dev(synth.all_query_histories(w))
    idx = torch.zeros((B, Hkv, k), dtype=torch.int32, device=dev)
    det_ws = torch.zeros(hq.hq_detect_workspace_size(B, Hkv, T - W, k), dtype=torch.uint8, device=dev)
    hq.hq_detect_vlines(None, q_hist, B, Hq, Hkv, D, 64, 0, True, K, T, T - W, k, hq.HQ_DETECT_MATMUL,
                        idx, None, det_ws)

    # exact attention, fp32
    qf = q.float().view(B, Hkv, G, D)
    Kf = K.float()
    lg = torch.matmul(qf, Kf.transpose(-1, -2).contiguous()) / np.sqrt(D)
    exact = torch.matmul(torch.softmax(lg, dim=-1), V.float()).view(B, Hq, D)
    del Kf, lg
    rms = float(exact.pow(2).mean().sqrt())

    settings = [("hybrid", k, W, 0), ("sparse", k, W, hq.HQ_KV_DROP_INT4),
                ("window", 0, W, hq.HQ_KV_DROP_INT4), ("k4v4", 0, 0, 0), ("bf16", 0, T, 0)]
    rows = []
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    for name, kk, ww, flags in settings:
        nq = T - ww
        units = B * Hkv
        int4_pos = 0 if flags else nq - kk
        dec_bytes = (units * (int4_pos * (D + (D // 32) * 8) + (kk + ww) * 2 * D * hp
                              + (0 if flags else (nq + 31) // 32 * 4))
                     + B * Hq * D * hp + B * Hq * D * 4 + B * Hq * 4)
        held = units * ((0 if flags else nq * (D + (D // 32) * 8)) + (kk + ww) * 2 * D * hp)
        per_copy = max(held, 1)
        copies = max(1, min(24, int(np.ceil(1.2e9 / per_copy))))
        caches = []
        for _ in range(copies):
            c = hq.HybridCache(B, Hkv, D, T, ww, kk, dt)
            c.build(K, V, idx[:, :, :kk].contiguous() if kk else None)
            c.flags = flags
            caches.append(c)
        descs = [c.descriptor() for c in caches]
        ws = torch.zeros(hq.hq_decode_workspace_size(descs[0], Hq, 0), dtype=torch.uint8, device=dev)
        hq.hq_decode_attn(q, Hq, descs[0], 0.0, 0, out, lse, ws)
        torch.cuda.synchronize()
        err = (out - exact).abs()
        max_rel = float(err.max()) / rms
        l2 = float(torch.linalg.vector_norm(out - exact) / torch.linalg.vector_norm(exact))
        for i in range(10):
            hq.hq_decode_attn(q, Hq, descs[i % copies], 0.0, 0, out, lse, ws)
        n = 100
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(n):
            hq.hq_decode_attn(q, Hq, descs[i % copies], 0.0, 0, out, lse, ws)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / n
        rows.append({"setting": name, "k": kk, "W": ww, "drop_int4": bool(flags),
                     "algorithmic_bytes": int(dec_bytes), "us_per_call": round(us, 2),
                     "gbs": round(dec_bytes / (us * 1e-6) / 1e9, 1), "cache_bytes": int(held),
                     "max_abs_err_over_rms": round(max_rel, 5), "rel_l2_err": round(l2, 6)})
        del caches, descs, ws
        torch.cuda.empty_cache()
    k4 = next(r for r in rows if r["setting"] == "k4v4")["cache_bytes"]
    for r in rows:
        r["cache_vs_k4v4"] = round(r["cache_bytes"] / k4 - 1.0, 4)
    line = {
        "metric": "decode ablation: bytes, us per hq_decode_attn call and error against exact attention",
        "n_gpus": 1, "data": "synthetic (seeded; shapes of the named model's attention layer)",
        "config": {"workload": f"{args.workload}: B {B}, {Hq} q / {Hkv} kv heads, head_dim {D}, context {T}, "
                               f"window {W}, VL budget {k} (detected from a 64-step query history)"},
        "exact_reference": "fp32 softmax(q K^T / sqrt(D)) V over the bf16 keys and values",
        "rows": rows,
    }
    print(json.dumps(line), flush=True)


def stream_read_ceiling(torch, hq, dev, stream, gib: int = 2, reps: int = 10) -> float:
    """GB/s of hq_stream_read (one sequential non-temporal read) over a
    buffer of `gib` GiB, far beyond the 256 MB Infinity Cache."""
    buf = torch.ones(gib << 30, dtype=torch.uint8, device=dev)
    sink = torch.zeros(hq.hq_stream_read_sink_bytes() // 4, dtype=torch.int32, device=dev)
    for _ in range(2):
        hq.hq_stream_read(buf, sink)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        hq.hq_stream_read(buf, sink)
    e1.record(stream)
    torch.cuda.synchronize()
    gbs = reps * buf.numel() / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del buf, sink
    return gbs


def stream_read_same_bytes_us(torch, hq, dev, stream, nbytes: int, launches: int) -> float:
    """Mean duration (us) of one hq_stream_read of `nbytes` in back-to-back
    launches (one event pair around them, as the decode calls are timed),
    rotating over slices of a buffer of >= 1 GiB, so that every read comes
    from HBM: the time a plain read of that many bytes takes at that size,
    launch and ramp included."""
    nb = (int(nbytes) + 255) // 256 * 256
    n = max(2, -(-(1 << 30) // nb))
    buf = torch.ones(n * nb, dtype=torch.uint8, device=dev)
    sink = torch.zeros(hq.hq_stream_read_sink_bytes() // 4, dtype=torch.int32, device=dev)
    views = [buf[i * nb:i * nb + int(nbytes) // 16 * 16] for i in range(n)]
    for i in range(n):
        hq.hq_stream_read(views[i], sink)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(launches):
        hq.hq_stream_read(views[i % n], sink)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / launches
    del views, buf, sink
    return us


def main_prefill(args):
    """One step = the prefill of one attention layer over a causal prompt:
    the vertical lines are chosen from the prompt's last 64 queries
    (hq_detect_vlines), then hq_prefill_attn computes every row's output and
    log-sum-exp. `value` is the algorithmic flops of the attention (Q K^T
    and P V over the causal triangle, 2 flops per multiply-add) divided by
    the step time."""
    import torch
    import hybrid_precision_quantized_amd as hq
    import synth

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    w = synth.WORKLOADS[args.workload]
    B, Hq, Hkv, D, T, W, k = w.B, w.Hq, w.Hkv, w.D, w.T, w.W, w.k
    R = 64
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float16
    t_setup = time.time()

    def to_dev(x32):
        if w.dtype == "bf16":
            return torch.from_numpy(synth.f32_to_bf16_bits(x32).view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float16)).to(dev)

    q = torch.empty((B, Hq, T, D), dtype=dt, device=dev)
    for b in range(B):
        for i in range(Hq):
            q[b, i].copy_(to_dev(synth.prefill_queries(w, b, i)))
    K = to_dev(synth.all_keys(w))
    V = to_dev(synth.all_values(w))
    q_last = q[:, :, T - R:].contiguous()              # the detector's 64-query window
    idx = torch.zeros((B, Hkv, k), dtype=torch.int32, device=dev)
    det_ws = torch.zeros(hq.hq_detect_workspace_size(B, Hkv, T - W, k), dtype=torch.uint8, device=dev)
    out = torch.empty((B, Hq, T, D), dtype=torch.float32, device=dev)
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device=dev)
    ws = torch.empty(hq.hq_prefill_workspace_size(B, Hq, Hkv, T, D, k), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    t_setup = time.time() - t_setup

    def detect():
        hq.hq_detect_vlines(None, q_last, B, Hq, Hkv, D, R, 0, True, K, T, T - W, k,
                            hq.HQ_DETECT_MATMUL, idx, None, det_ws)

    def prefill():
        hq.hq_prefill_attn(q, K, V, B, Hq, Hkv, T, D, W, idx, k, 0.0, out, lse, ws)

    steps = max(1, min(args.steps, 20))
    warm = max(1, min(args.warmup, 3))
    for _ in range(warm):
        detect()
        prefill()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        detect()
        prefill()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = e0.elapsed_time(e1) / steps

    # hq_prefill_attn alone, per call (pre-pass + tiling + the attention kernel)
    n_l = max(3, min(args.kernel_launches, 10))
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(n_l)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(n_l)]
    for i in range(n_l):
        starts[i].record(stream)
        prefill()
        ends[i].record(stream)
    torch.cuda.synchronize()
    call_ms = float(np.mean([a.elapsed_time(e) for a, e in zip(starts, ends)]))

    flops = 2.0 * 2.0 * B * Hq * D * (T * (T + 1) / 2.0)
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (call_ms * 1e-3) / 1e12
    cpu = None if args.no_cpu_baseline else cpu_baseline_prefill(w, args.cpu_seconds, flops)
    line = {
        "metric": PREFILL_METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4 q/k (f16 hi+lo MFMA) + bf16 (fp32 accumulate)",
        "data": "synthetic (seeded; shapes of the named model's attention layer, random-init values)",
        "config": {
            "workload": f"prefill32k: causal prefill of one attention layer, B {B}, {Hq} q / {Hkv} kv heads, "
                        f"head_dim {D}, prompt {T}, window {W}, VL budget {k} (detected from the last "
                        f"{R} queries), INT4 group 32 for the quantized Q.K majority",
            "global_batch": B, "seq_len": T, "parallelism": "none (1 GPU)",
        },
        "roofline": {
            "kernel": "prefill_kernel (hq_prefill_attn, timed per call incl. its pre-pass)",
            "bound": "mfma",
            "achieved": round(achieved, 1),
            "peak": PEAK_MFMA_F16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_MFMA_F16_TFLOPS, 4),
            "traffic": None,
            "algorithmic_flops_per_launch": int(flops),
            "avg_launch_ms": round(call_ms, 4),
        },
        "setup_s": round(t_setup, 1),
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def cpu_baseline_prefill(w, seconds: float, flops: float):
    """The CPU oracle prefill (unchanged) on a bounded sample: blocks of query
    rows of KV head 0's group, repeated until `seconds` of work, scaled to
    every row of every head (its cost per row does not depend on the row)."""
    import synth
    from oracle import prefill
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = 1
    q = np.stack([synth.prefill_queries(w, 0, i) for i in range(w.G)])
    K = synth.keys(w, 0, 0)
    V = synth.values(w, 0, 0)
    vl = synth.random_vl_index(w, 0, 0)
    rng = np.random.default_rng(5)
    t0 = time.time()
    n_rows = 0
    while time.time() - t0 < seconds and n_rows < 4096:
        rows = np.sort(rng.choice(w.T, size=32, replace=False))
        prefill.prefill_rows(q, K, V, vl, w.W, rows)
        n_rows += len(rows)
    el = time.time() - t0
    per_row_head = el / (n_rows * w.G)
    s_total = per_row_head * w.T * w.Hq * w.B
    return {"value": round(flops / s_total / 1e12, 6), "unit": "TFLOP/s", "ms_per_step": round(s_total * 1e3, 1),
            "cores": threads, "kind": "oracle",
            "sample": f"{n_rows} random query rows x {w.G} heads of KV head 0 ({el:.1f} s), "
                      f"scaled to all {w.T} rows x {w.Hq} heads"}


def cpu_baseline(w, seconds: float, step_bytes: float):
    """The CPU oracle (unchanged) on a bounded sample of the same step: the
    decode of whole (b, KV head) units over their cache, plus the amortized
    detector share, repeated until `seconds` of work; scaled to one step."""
    import synth
    from oracle import attention, detect, quant
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = 1
    nq = w.T - w.W
    units = [(b, h) for b in range(w.B) for h in range(w.Hkv)]
    prep = []
    for (b, h) in units[:4]:
        K = synth.keys(w, b, h)
        V = synth.values(w, b, h)
        kp, ks = quant.quantize_rows(K[:nq])
        vp, vs = quant.quantize_rows(V[:nq])
        vl = synth.random_vl_index(w, b, h)
        q = np.stack([synth.query(w, b, i) for i in range(h * w.G, (h + 1) * w.G)])
        qh = np.stack([synth.query_history(w, b, i) for i in range(h * w.G, (h + 1) * w.G)]).reshape(-1, w.D)
        prep.append((q, K, V, kp, ks, vp, vs, vl, qh))
    t0 = time.time()
    n_units = 0
    n_det = 0
    while time.time() - t0 < seconds:
        q, K, V, kp, ks, vp, vs, vl, qh = prep[n_units % len(prep)]
        attention.decode_head(q, K, V, kp, ks, vp, vs, vl, w.W)
        n_units += 1
        if n_units % 16 == 0:
            detect.detect_head(qh, K, nq, w.k)
            n_det += 1
        if n_units >= 200:
            break
    el = time.time() - t0
    # per unit: decode + detect share (the detector runs once per 64 steps)
    t_det_share = 0.0
    per_unit = el / max(n_units, 1)
    if n_det:
        # separate the two: time one detection alone
        q, K, V, kp, ks, vp, vs, vl, qh = prep[0]
        t1 = time.time()
        detect.detect_head(qh, K, nq, w.k)
        t_det = time.time() - t1
        per_unit = (el - n_det * t_det) / n_units
        t_det_share = t_det / 64
    s_per_step = (per_unit + t_det_share) * len(units)
    return {"value": round(step_bytes / s_per_step / 1e9, 3), "unit": "GB/s",
            "us_per_step": round(s_per_step * 1e6, 1), "cores": threads, "kind": "oracle",
            "sample": f"{n_units} (b, kv-head) decode units of the {w.name} step over prebuilt INT4 "
                      f"caches (+{n_det} detections), {el:.1f} s, scaled to all {len(units)} units "
                      f"and the detector's 1/64 share"}


if __name__ == "__main__":
    main()
