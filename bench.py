"""Benchmark of the HyQuant decode hot path on one MI355X.

One step = one steady-state decode step of one attention layer over its
rolling hybrid KV cache (16-bit rows only for the VL set and a window ring
of W + 64 rows, everything else INT4):
  1. hq_decode_step: attention over INT4 + VL + window with the split-K LSE
     merge; in the same launches the step's queries go into the detector's
     64-slot ring and the window's oldest token is packed into INT4;
  2. every 64th step a re-detection (hq_vl_redetect, two launches): the 64
     accumulated steps' summed queries, the column scores of the candidates
     (the current VL set and the ring rows behind the window, the only
     positions that can enter the set) from their INT4 keys, and the new VL
     set written in place. It is timed on its own and 1/64 of it is added to
     the step time, so that any --steps includes its share.
The decode steps rotate over `--copies` independent layer caches (>= 1 GB of
decode-read bytes in total) so that the 256 MB Infinity Cache cannot hold
the working set: every step reads its cache from HBM as it would in a model
with many layers. All inputs are seeded synthetic tensors already resident
in HBM when timing starts; the 16-bit source rows a prefill would leave are
freed once the caches are built.

Prints one JSON line (rank 0). `value` is the algorithmic HBM bytes of a
step divided by the step time (GB/s); `ms_per_step` is the step time.
`roofline` is the decode call alone (split kernel + merge kernel), timed
with HIP events on the launch stream around back-to-back calls (and, for the
spread, per call: p10 / p50 / p90), beside the HBM read ceiling (a 2 GiB
sequential read), the time of a plain read of the call's own bytes at the
same size, and the median of launches that reuse one cache copy ("warm").
`long_context` (default workload only) is the 16 x 128K workload in the
same run. `cpu_baseline` is the CPU oracle on a bounded sample of the same
step, in a process pool.
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
    ap.add_argument("--detect-method", default="matmul", choices=["matmul", "qsum", "mass"],
                    help="the detector over the full 16-bit keys reported beside the re-detection "
                         "(matmul: Q_acc K^T on MFMA; qsum: summed queries, GEMV; mass: attention-mass "
                         "scores)")
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--kernel-launches", type=int, default=200)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=30.0,
                    help="budget of the CPU baseline; its 128K sample is skipped beyond it")
    ap.add_argument("--ablation", action="store_true",
                    help="decode settings of the ablation (hybrid, sparse, window only, strict K4V4, "
                         "all 16-bit): bytes, time and error against exact attention")
    ap.add_argument("--no-graph", dest="graph", action="store_false",
                    help="time the steps as stream launches instead of one HIP graph replay (the default "
                         "captures exactly `steps` steps in one graph and times its replay, so that the "
                         "host's enqueue rate cannot set the pace)")
    ap.add_argument("--prefill-form", default="split", choices=["split", "i8"],
                    help="prefill32k: the quantized Q.K form the step uses (split fp16 planes, or int8 MFMA "
                         "over the codes); both are timed per call")
    ap.add_argument("--no-long-context", action="store_true",
                    help="skip the 16 x 128K entry of the default workload's line")
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
        print("bench.py measures one GPU only: there is no multi-GPU path here (decode attention "
              "would shard by KV head or by sequence with no communication, one GPU's share being "
              "this same kernel at its own shape). Run with --gpus 1.", file=sys.stderr)
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
    return main_decode(args, torch, hq, synth)


def build_rolling_caches(torch, hq, synth, w, copies, dev):
    """`copies` independent rolling caches of one layer at context T, in the
    state a prefill leaves them: INT4 planes for [0, T - W), the VL set from
    the pages' detector (Q_acc K^T column sums, top-k) over the prompt's last
    R queries and the 16-bit keys, the VL rows, and a ring of W + R rows
    holding positions [T - W - R, T). The 16-bit source rows are freed
    afterwards: the caches hold nothing else. Returns (caches, K source kept
    for the detector measurement or None, q_steps, idx)."""
    dt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[w.dtype]
    B, Hq, Hkv, D, T, W, k = w.B, w.Hq, w.Hkv, w.D, w.T, w.W, w.k
    R = 64
    nq = T - W

    def to_dev(x32):
        if w.dtype == "bf16":
            return torch.from_numpy(synth.f32_to_bf16_bits(x32).view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(x32)).to(dev)

    K0 = torch.empty((B, Hkv, T, D), dtype=dt, device=dev)
    V0 = torch.empty_like(K0)
    for b in range(B):
        K0[b].copy_(to_dev(np.stack(synth._parallel(lambda h: synth.keys(w, b, h), [(h,) for h in range(Hkv)]))))
        V0[b].copy_(to_dev(np.stack(synth._parallel(lambda h: synth.values(w, b, h), [(h,) for h in range(Hkv)]))))
    q_steps = to_dev(np.stack([synth.all_queries(w.replace(seed=w.seed + 17 * s)) for s in range(4)]))
    q_hist = to_dev(synth.all_query_histories(w))
    # the set at the end of prefill: the pages' detector over the full 16-bit keys
    idx = torch.zeros((B, Hkv, k), dtype=torch.int32, device=dev)
    ws = torch.zeros(hq.hq_detect_workspace_size(B, Hkv, nq, k), dtype=torch.uint8, device=dev)
    hq.hq_detect_vlines(None, q_hist, B, Hq, Hkv, D, R, 0, True, K0, T, nq, k, hq.HQ_DETECT_MATMUL, idx, None, ws)
    caches = []
    t_cap = (nq + 1 + 31) // 32 * 32              # one spare row: the step packs position T - W
    for c in range(copies):
        rc = hq.RollingCache(B, Hkv, D, T, W, k, dt, Hq, R=R, t_cap=t_cap, device=dev)
        rc.build(K0, V0, idx)
        rc.q_acc.copy_(q_hist)
        # the context is held at T: every update treats the R ring rows behind
        # the window as the positions that left it since the previous one
        rc.p0 = nq - R
        caches.append(rc)
    torch.cuda.synchronize()
    del V0
    return caches, K0, q_steps, idx


def main_decode(args, torch, hq, synth):
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    w = synth.WORKLOADS[args.workload]
    B, Hq, Hkv, D, T, W, k = w.B, w.Hq, w.Hkv, w.D, w.T, w.W, w.k
    R = 64
    nq = T - W
    hp = 2 if w.dtype in ("bf16", "f16") else 4
    units = B * Hkv

    # ------------------------------------------------------------ bytes
    # one decode call: INT4 codes and scales of the non-VL quantized
    # positions, 16-bit VL and window rows, the VL bitmap, q in, O and lse out
    dec_bytes = (units * ((nq - k) * (D + (D // 32) * 8) + (k + W) * 2 * D * hp + (nq + 31) // 32 * 4)
                 + B * Hq * D * hp + B * Hq * D * 4 + B * Hq * 4)
    # the step's upkeep: the window's oldest row read and packed, q into the ring
    evict_bytes = 2 * units * (D * hp + D // 2 + (D // 32) * 4)
    acc_bytes = 2 * B * Hq * D * hp
    # a re-detection (hq_vl_redetect): the query ring, the INT4 key codes
    # and scales of the k + R candidates, the VL index list read, and at most
    # R promoted rows per head copied from the ring into freed slots (K and V
    # read and written) with their index entries
    det_bytes = (B * Hq * R * D * hp + units * (k + R) * (D // 2 + (D // 32) * 4) + units * k * 4
                 + units * R * 2 * 2 * D * hp + units * R * 4)

    t_setup = time.time()
    copies = args.copies or max(1, int(np.ceil(1.05e9 / dec_bytes)))
    caches, K0, q_steps, idx0 = build_rolling_caches(torch, hq, synth, w, copies, dev)
    descs = [c.descriptor() for c in caches]
    ws_bytes = max(hq.hq_decode_workspace_size(d, Hq, args.splits) for d in descs)
    dec_ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    resident = caches[0].resident_bytes()
    torch.cuda.synchronize()
    t_setup = time.time() - t_setup

    launch_stream_box = [stream]             # the stream the step's calls go to
    nqs = q_steps.shape[0]

    def step(s: int):
        c = s % copies
        hq.hq_decode_step(q_steps[s % nqs], Hq, descs[c], 0.0, args.splits, out, lse, dec_ws,
                          q_acc=caches[c].q_acc, R=R, step=s, evict=True,
                          stream=launch_stream_box[0].cuda_stream)

    def redetect(c: int):
        rc = caches[c]
        rc.p0 = nq - R
        rc.redetect()
        descs[c] = rc.descriptor()

    # ------------------------------------------------------------ timed decode steps
    # the host-side setup left the device idle: untimed steps for about 0.25 s
    # bring it back to its working clocks before the warm-up steps proper
    t_end = time.time() + 0.25
    while time.time() < t_end:
        for s in range(64):
            step(s)
        torch.cuda.synchronize()
    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    base = args.warmup
    if args.graph:
        graph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        launch_stream_box[0] = cap
        with torch.cuda.stream(cap):
            with torch.cuda.graph(graph, stream=cap):
                for s in range(base, base + args.steps):
                    step(s)
        launch_stream_box[0] = stream
        stream.wait_stream(cap)
        graph.replay()                       # the first replay uploads the graph: untimed
        torch.cuda.synchronize()
    # the host's enqueue cost of the same steps launched one by one
    h0 = time.perf_counter()
    for s in range(base, base + args.steps):
        step(s)
    host_us_per_step = (time.perf_counter() - h0) * 1e6 / args.steps
    torch.cuda.synchronize()
    e0.record(stream)
    if args.graph:
        graph.replay()
    else:
        for s in range(base, base + args.steps):
            step(s)
    e1.record(stream)
    torch.cuda.synchronize()
    step_us = e0.elapsed_time(e1) * 1e3 / args.steps

    # ------------------------------------------------------------ re-detection (every R steps)
    n_det = max(8, min(2 * copies, 40))
    for c in range(min(copies, 4)):
        redetect(c)
    torch.cuda.synchronize()
    d0 = torch.cuda.Event(enable_timing=True)
    d1 = torch.cuda.Event(enable_timing=True)
    d0.record(stream)
    for i in range(n_det):
        redetect(i % copies)
    d1.record(stream)
    torch.cuda.synchronize()
    det_us_launched = d0.elapsed_time(d1) * 1e3 / n_det
    det_us = det_us_launched
    det_us_in_cycle = None
    if args.graph:
        # the same re-detections as one graph replay: the GPU's time, not the
        # host's pace of enqueueing them
        dgraph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        with torch.cuda.stream(cap):
            with torch.cuda.graph(dgraph, stream=cap):
                for i in range(n_det):
                    redetect(i % copies)
        stream.wait_stream(cap)
        dgraph.replay()
        torch.cuda.synchronize()
        best = None
        for _ in range(3):
            d0.record(stream)
            dgraph.replay()
            d1.record(stream)
            torch.cuda.synchronize()
            t = d0.elapsed_time(d1) * 1e3 / n_det
            best = t if best is None else min(best, t)
        det_us = best
        del dgraph
        # in context: one whole 64-step cycle with and without its re-detection
        # (the re-detection then runs where it does in decoding, right after a
        # step, with the clocks and caches of a busy chip)
        def cycle_us(with_det):
            g = torch.cuda.CUDAGraph()
            cs = torch.cuda.Stream()
            cs.wait_stream(stream)
            launch_stream_box[0] = cs
            with torch.cuda.stream(cs):
                with torch.cuda.graph(g, stream=cs):
                    for s_ in range(R):
                        step(s_)
                    if with_det:
                        redetect((R - 1) % copies)
            launch_stream_box[0] = stream
            stream.wait_stream(cs)
            g.replay()
            torch.cuda.synchronize()
            t_best = None
            for _ in range(3):
                d0.record(stream)
                g.replay()
                d1.record(stream)
                torch.cuda.synchronize()
                t = d0.elapsed_time(d1) * 1e3
                t_best = t if t_best is None else min(t_best, t)
            del g
            return t_best
        cyc0 = cycle_us(False)
        cyc1 = cycle_us(True)
        det_us_in_cycle = max(cyc1 - cyc0, 0.0)
    # the pages' matrix-multiplication detector on the full 16-bit keys (the
    # prefill-end detection; the detector workload of the GLM-4-9B shape)
    mm_us = detector_matmul_us(torch, hq, w, K0, caches[0].q_acc, args.detect_method, dev, stream)
    del K0

    # the share charged to a step: the re-detection timed alone (a graph of
    # back-to-back re-detections); the in-cycle difference of two ~1 ms
    # replays is reported beside it but is too noisy to charge
    det_share_us = det_us / R
    us_per_step = step_us + det_share_us
    step_bytes = dec_bytes + evict_bytes + acc_bytes + det_bytes / R
    value = step_bytes / (us_per_step * 1e-6) / 1e9

    # ------------------------------------------------------------ decode call alone
    dec_us_launched, dec_pct, warm_us = time_decode_calls(torch, hq, caches, descs, q_steps, Hq, out, lse, dec_ws,
                                                          args.splits, args.kernel_launches, stream)
    dec_us = dec_us_launched
    dec_us_graph = (graph_decode_calls_us(torch, hq, caches, descs, q_steps, Hq, out, lse, dec_ws, args.splits,
                                          args.kernel_launches, stream, launch_stream_box) if args.graph else None)
    achieved = dec_bytes / (dec_us * 1e-6) / 1e9
    if args.calib_copy_mb:
        # a plain device copy of known size: the counters' calibration
        a = torch.empty(args.calib_copy_mb * (1 << 20) // 4, dtype=torch.float32, device=dev).fill_(1.0)
        b_ = torch.empty_like(a)
        b_.copy_(a)
        torch.cuda.synchronize()
        del a, b_
    stream_gbs = stream_read_ceiling(torch, hq, dev, stream)
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
    auto_s = hq.hq_decode_auto_splits(descs[0], Hq) if args.splits == 0 else args.splits
    del caches, descs, dec_ws
    torch.cuda.empty_cache()

    # ------------------------------------------------------------ the 128K workload, same line
    long_ctx = None
    if args.workload == "llama32k" and not args.no_long_context:
        long_ctx = long_context_entry(torch, hq, synth, dev, stream, args)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args.cpu_seconds, step_bytes, us_per_step)

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us_per_step * 1e-3, 6),
        "us_per_step": round(us_per_step, 3),
        "us_per_step_parts": {"decode_step": round(step_us, 3), "redetection_share": round(det_share_us, 3),
                              "redetection_share_from": "the re-detection timed alone (graph replay), over 64"},
        "host_enqueue_us_per_step": round(host_us_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("int4 k/v (codes as fp16) + bf16 rows; q fp16 in the int4 pass, p*s fp16, fp32 accumulate"
                  if w.dtype == "bf16" else f"int4 k/v + {w.dtype} rows, fp32 accumulate"),
        "data": "synthetic (seeded; shapes of the named model's attention layer, random-init values)",
        "config": {
            "workload": f"{args.workload}: one decode step of one attention layer, B {B}, "
                        f"{Hq} q / {Hkv} kv heads, head_dim {D}, context {T}, window {W}, "
                        f"VL budget {k}, INT4 group 32 with fp16 scale/zero; rolling cache (16-bit rows: "
                        f"VL set + a ring of W + {R}), re-detection every {R} steps",
            "global_batch": B, "seq_len": T, "parallelism": "none (1 GPU)",
            "layer_copies_rotated": copies,
            "decode_read_bytes_rotated": int(copies * dec_bytes),
            "decode_splits": auto_s,
            "timed_as": (("exactly `steps` decode steps (hq_decode_step: attention + the step's upkeep) "
                          "captured in one HIP graph, its replay timed with HIP events" if args.graph else
                          "exactly `steps` decode steps (hq_decode_step: attention + the step's upkeep) "
                          "launched on the stream") +
                         ", plus 1/64 of a re-detection timed separately (hq_vl_redetect)"),
            "layer_resident_bytes": int(resident),
            "layer_resident_vs_k4v4": round(resident / (units * nq * 2 * (D // 2 + (D // 32) * 4)) - 1.0, 4),
        },
        "roofline": {
            "kernel": "decode_kernel + merge_kernel (hq_decode_attn)",
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
            "avg_launch_us_timed_as": ("one HIP event pair on the launch stream around back-to-back "
                                       "hq_decode_attn calls (split kernel + merge kernel each), caches rotated"),
            "avg_launch_us_graph_replay": (round(dec_us_graph, 3) if dec_us_graph is not None else None),
            "bracketed_call_us_p10_p50_p90": [round(float(x), 3) for x in dec_pct],
            "warm_launch_us_median": round(warm_us, 3),
            "stream_read_gbs": round(stream_gbs, 1),
            "frac_of_stream_read": round(achieved / stream_gbs, 4),
            "stream_read_same_bytes_us": round(same_us, 3),
            "frac_of_stream_read_same_bytes": round(same_us / dec_us, 4),
        },
        "detector": {
            "us_per_redetection": round(det_us, 2),
            "us_per_redetection_timed_as": ("one HIP graph replay of back-to-back re-detections (best of 3)"
                                            if args.graph else "stream launches"),
            "us_per_redetection_stream_launched": round(det_us_launched, 2),
            "us_per_redetection_in_64_step_cycle": (round(det_us_in_cycle, 2) if det_us_in_cycle is not None
                                                    else None),
            "redetection": ("hq_vl_redetect: summed ring queries and the candidates' scores from their INT4 "
                            "keys (many workgroups per head), then the in-place update (one workgroup per head)"),
            "redetection_bytes": int(det_bytes),
            "overhead_vs_64_decode_steps": round(det_share_us / step_us, 4),
            "matmul_us_per_detection": round(mm_us, 2),
            "matmul_method": args.detect_method,
            "matmul_overhead_vs_64_decode_steps": round(mm_us / (R * step_us), 4),
        },
        "step_bytes": int(step_bytes),
        "setup_s": round(t_setup, 1),
    }
    if long_ctx is not None:
        line["long_context"] = long_ctx
    line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


def graph_decode_calls_us(torch, hq, caches, descs, q_steps, Hq, out, lse, ws, splits, launches, stream,
                          launch_stream_box):
    """hq_decode_attn alone, as the steps are timed: `launches` back-to-back
    calls over the rotated caches captured in one HIP graph, HIP events on
    the launch stream around each replay; the median of 5 replays, per call."""
    copies = len(caches)
    nqs = q_steps.shape[0]
    g = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    cs.wait_stream(stream)
    with torch.cuda.stream(cs):
        with torch.cuda.graph(g, stream=cs):
            for i in range(launches):
                hq.hq_decode_attn(q_steps[i % nqs], Hq, descs[i % copies], 0.0, splits, out, lse, ws,
                                  stream=cs.cuda_stream)
    stream.wait_stream(cs)
    g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    ts = []
    for _ in range(5):
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e3 / launches)
    del g
    return float(np.median(ts))


def time_decode_calls(torch, hq, caches, descs, q_steps, Hq, out, lse, ws, splits, launches, stream):
    """hq_decode_attn alone: one event pair around back-to-back calls over
    the rotated caches (mean), each call bracketed by its own events (p10,
    p50, p90: the events add their own time), and the median of calls that
    reuse one cache ("warm": what fits the Infinity Cache may come from it)."""
    copies = len(caches)
    nqs = q_steps.shape[0]
    for i in range(min(launches, 2 * copies)):
        hq.hq_decode_attn(q_steps[i % nqs], Hq, descs[i % copies], 0.0, splits, out, lse, ws)
    torch.cuda.synchronize()
    c0 = torch.cuda.Event(enable_timing=True)
    c1 = torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for i in range(launches):
        hq.hq_decode_attn(q_steps[i % nqs], Hq, descs[i % copies], 0.0, splits, out, lse, ws)
    c1.record(stream)
    torch.cuda.synchronize()
    mean_us = c0.elapsed_time(c1) * 1e3 / launches
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(launches)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(launches)]
    for i in range(launches):
        starts[i].record(stream)
        hq.hq_decode_attn(q_steps[i % nqs], Hq, descs[i % copies], 0.0, splits, out, lse, ws)
        ends[i].record(stream)
    torch.cuda.synchronize()
    pct = np.percentile([a.elapsed_time(b) * 1e3 for a, b in zip(starts, ends)], [10, 50, 90])
    for i in range(launches):
        starts[i].record(stream)
        hq.hq_decode_attn(q_steps[i % nqs], Hq, descs[0], 0.0, splits, out, lse, ws)
        ends[i].record(stream)
    torch.cuda.synchronize()
    warm = float(np.median([a.elapsed_time(b) * 1e3 for a, b in zip(starts, ends)]))
    return mean_us, pct, warm


def detector_matmul_us(torch, hq, w, K0, q_acc, method_name, dev, stream):
    """The detector over the full 16-bit keys (what runs at the end of
    prefill, and the GLM-4-9B-shaped detector workload): mean of repeated
    detections, the keys rotated over copies past the Infinity Cache when
    they are smaller than 1 GB."""
    B, Hq, Hkv, D, T, W, k = w.B, w.Hq, w.Hkv, w.D, w.T, w.W, w.k
    R = 64
    nq = T - W
    kb = K0.numel() * K0.element_size()
    n_k = max(1, min(16, int(np.ceil(1.05e9 / kb))))
    Ks = [K0] + [K0.clone() for _ in range(n_k - 1)]
    idx = torch.zeros((B, Hkv, k), dtype=torch.int32, device=dev)
    if method_name == "mass":
        ws = torch.zeros(hq.hq_detect_mass_workspace_size(B, Hq, Hkv, R, T, nq), dtype=torch.uint8, device=dev)
        fn = lambda Kc: hq.hq_detect_vlines_mass(None, q_acc, B, Hq, Hkv, D, R, 0, True, Kc, T, nq, k, idx,
                                                 None, ws)
    else:
        method = hq.HQ_DETECT_QSUM if method_name == "qsum" else hq.HQ_DETECT_MATMUL
        ws = torch.zeros(hq.hq_detect_workspace_size(B, Hkv, nq, k), dtype=torch.uint8, device=dev)
        fn = lambda Kc: hq.hq_detect_vlines(None, q_acc, B, Hq, Hkv, D, R, 0, True, Kc, T, nq, k, method,
                                            idx, None, ws)
    for Kc in Ks:
        fn(Kc)
    torch.cuda.synchronize()
    n = 20
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(n):
        fn(Ks[i % n_k])
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / n
    del Ks
    return us


def long_context_entry(torch, hq, synth, dev, stream, args):
    """The 16 x 128K workload (Qwen3-8B-style GQA) in the same run: one
    rolling cache (3 GB of decode-read bytes, beyond the Infinity Cache by
    itself), the decode call and step time, and one re-detection."""
    w = synth.WORKLOADS["qwen128k"]
    B, Hq, Hkv, D, T, W, k = w.B, w.Hq, w.Hkv, w.D, w.T, w.W, w.k
    R = 64
    nq = T - W
    units = B * Hkv
    t0 = time.time()
    caches, K0, q_steps, _ = build_rolling_caches(torch, hq, synth, w, 1, dev)
    del K0
    torch.cuda.empty_cache()
    rc = caches[0]
    desc = rc.descriptor()
    dec_bytes = (units * ((nq - k) * (D + (D // 32) * 8) + (k + W) * 2 * D * 2 + (nq + 31) // 32 * 4)
                 + B * Hq * D * 2 + B * Hq * D * 4 + B * Hq * 4)
    ws = torch.zeros(hq.hq_decode_workspace_size(desc, Hq, 0), dtype=torch.uint8, device=dev)
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    setup_s = time.time() - t0
    n = 100
    # the device idled through the setup on the host: 400 warm-up steps
    # (about 0.2 s of load) bring it back to its working clocks, as the
    # warm-up steps of the main workload do (10 steps measured ~5 % slower)
    for i in range(400):
        hq.hq_decode_step(q_steps[i % 4], Hq, desc, 0.0, 0, out, lse, ws, q_acc=rc.q_acc, R=R, step=i, evict=True)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(n):
        hq.hq_decode_step(q_steps[i % 4], Hq, desc, 0.0, 0, out, lse, ws, q_acc=rc.q_acc, R=R, step=i, evict=True)
    e1.record(stream)
    torch.cuda.synchronize()
    step_us = e0.elapsed_time(e1) * 1e3 / n
    e0.record(stream)
    for i in range(n):
        hq.hq_decode_attn(q_steps[i % 4], Hq, desc, 0.0, 0, out, lse, ws)
    e1.record(stream)
    torch.cuda.synchronize()
    call_us = e0.elapsed_time(e1) * 1e3 / n
    rc.p0 = nq - R
    rc.redetect()
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(3):
        rc.p0 = nq - R
        rc.redetect()
    e1.record(stream)
    torch.cuda.synchronize()
    det_us = e0.elapsed_time(e1) * 1e3 / 3
    achieved = dec_bytes / (call_us * 1e-6) / 1e9
    return {"workload": f"qwen128k: B {B}, {Hq} q / {Hkv} kv heads, head_dim {D}, context {T}, window {W}, "
                        f"VL budget {k}",
            "us_per_step": round(step_us + det_us / R, 2),
            "decode_call_us": round(call_us, 2), "decode_step_us": round(step_us, 2),
            "us_per_redetection": round(det_us, 1),
            "achieved_gbs": round(achieved, 1), "frac": round(achieved / PEAK_HBM_GBS, 4),
            "algorithmic_bytes_per_launch": int(dec_bytes),
            "decode_splits": hq.hq_decode_auto_splits(desc, Hq), "setup_s": round(setup_s, 1),
            "timed_as": "one HIP event pair around 100 back-to-back calls after 400 warm-up steps; 3 GB per "
                        "call, no rotation needed"}


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
    (HIP events around 100 calls replayed from a HIP graph, caches rotated
    past the Infinity Cache; the same calls launched one by one are
    reported beside it), the bytes held in
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
        # what the layer holds in a rolling cache: the INT4 planes, the VL
        # rows with their index list and bitmap, and the window ring, which
        # keeps 64 more rows (the positions that left the window since the
        # last re-detection) whenever there is a VL set to maintain
        ring = ww + (64 if kk > 0 and ww > 0 else 0)
        held = units * ((0 if flags else nq * (D + (D // 32) * 8) + (nq + 31) // 32 * 4)
                        + (kk + ring) * 2 * D * hp + kk * 4)
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
        us_stream = e0.elapsed_time(e1) * 1e3 / n
        # the same calls replayed from a HIP graph: the GPU's time per call
        # without the host's launch cost (which bounds the small settings when
        # the calls are launched one by one)
        us = graph_decode_calls_us(torch, hq, caches, descs, q[None], Hq, out, lse, ws, 0, n, stream, None)
        rows.append({"setting": name, "k": kk, "W": ww, "drop_int4": bool(flags),
                     "algorithmic_bytes": int(dec_bytes), "us_per_call": round(us, 2),
                     "us_per_call_stream_launched": round(us_stream, 2),
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

    form = args.prefill_form

    def prefill(f=form):
        hq.hq_prefill_attn(q, K, V, B, Hq, Hkv, T, D, W, idx, k, 0.0, out, lse, ws, form=f)

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

    # one prefill call alone (pre-pass + tiling + the attention kernel), both
    # forms of the quantized Q.K
    n_l = max(3, min(args.kernel_launches, 10))

    def time_calls(f):
        prefill(f)
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(n_l)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(n_l)]
        for i in range(n_l):
            starts[i].record(stream)
            prefill(f)
            ends[i].record(stream)
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(e) for a, e in zip(starts, ends)]))

    flops = 2.0 * 2.0 * B * Hq * D * (T * (T + 1) / 2.0)
    form_ms = {f: time_calls(f) for f in ("split", "i8")}
    call_ms = form_ms[form]
    forms = {f: {"entry": "hq_prefill_attn" if f == "split" else "hq_prefill_attn_i8",
                 "avg_launch_ms": round(ms, 4), "achieved_tflops": round(flops / (ms * 1e-3) / 1e12, 1)}
             for f, ms in form_ms.items()}
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
        "dtype": ("int4 q/k (f16 hi+lo MFMA) + bf16 (fp32 accumulate)" if form == "split" else
                  "int4 q/k (int8 MFMA over the codes, fp32 scale epilogue) + bf16 (fp32 accumulate)"),
        "data": "synthetic (seeded; shapes of the named model's attention layer, random-init values)",
        "config": {
            "workload": f"prefill32k: causal prefill of one attention layer, B {B}, {Hq} q / {Hkv} kv heads, "
                        f"head_dim {D}, prompt {T}, window {W}, VL budget {k} (detected from the last "
                        f"{R} queries), INT4 group 32 for the quantized Q.K majority",
            "global_batch": B, "seq_len": T, "parallelism": "none (1 GPU)",
        },
        "roofline": {
            "kernel": (f"prefill_kernel ({forms[form]['entry']}, timed per call incl. its pre-pass)"),
            "bound": "mfma",
            "achieved": round(achieved, 1),
            "peak": PEAK_MFMA_F16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_MFMA_F16_TFLOPS, 4),
            "traffic": None,
            "algorithmic_flops_per_launch": int(flops),
            "avg_launch_ms": round(call_ms, 4),
        },
        "qk_forms": forms,
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


def _cpu_worker_init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass


def _cpu_decode_unit(task):
    """One (b, KV head) unit of a decode step on one core: its inputs
    regenerated from the seeded streams and quantized (not timed), then the
    oracle decode of the unit's query heads (timed)."""
    name, T_over, b, h = task
    import synth
    from oracle import attention, quant
    w = synth.WORKLOADS[name]
    if T_over:
        w = w.replace(T=T_over, k=int(0.05 * T_over))
    nq = w.T - w.W
    K = synth.keys(w, b, h)
    V = synth.values(w, b, h)
    kp, ks = quant.quantize_rows(K[:nq])
    vp, vs = quant.quantize_rows(V[:nq])
    vl = synth.random_vl_index(w, b, h)
    q = np.stack([synth.query(w, b, i) for i in range(h * w.G, (h + 1) * w.G)])
    t0 = time.perf_counter()
    attention.decode_head(q, K, V, kp, ks, vp, vs, vl, w.W)
    return time.perf_counter() - t0


def _cpu_detect_unit(task):
    """One (b, KV head) unit of the detector (the pages' matmul + column
    sums + top-k over the 16-bit keys, exact grid inputs) on one core."""
    name, b, h = task
    import synth
    from oracle import detect
    w = synth.WORKLOADS[name]
    K = synth.keys(w, b, h)
    rows = np.stack([synth.query_history(w, b, i) for i in range(h * w.G, (h + 1) * w.G)]).reshape(-1, w.D)
    t0 = time.perf_counter()
    detect.detect_head(rows, K, w.T - w.W, w.k)
    return time.perf_counter() - t0


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, seconds: float, step_bytes: float, gpu_us_per_step: float):
    """The CPU oracle (unchanged) on bounded samples, in a process pool of
    single-threaded workers (one (b, KV head) unit per task, BLAS limited to
    one thread per worker; at most 15 workers):
      * the benchmarked step: all its decode units at once, plus 1/64 of the
        detector over one unit per worker; the wall time is the step time;
      * the same units one after another on one core (the single-core time);
      * the tiny fp32 step, the GLM-4-9B-shaped detection, and a 16 x 128K
        step extrapolated from a sample of its units (stated)."""
    from concurrent.futures import ProcessPoolExecutor
    import multiprocessing as mp
    # fresh interpreters (spawn): the workers hold no GPU state; 15 of them
    # plus this process stay within the host share of one GPU
    workers = max(1, min(15, os.cpu_count() or 1))
    units = [(b, h) for b in range(w.B) for h in range(w.Hkv)]
    t_all = time.time()
    ctx = mp.get_context("spawn")
    with ProcessPoolExecutor(workers, mp_context=ctx, initializer=_cpu_worker_init) as ex:
        # warm the workers' imports
        list(ex.map(_cpu_decode_unit, [("tiny", 0, 0, 0)] * workers))
        t0 = time.perf_counter()
        dec = list(ex.map(_cpu_decode_unit, [(w.name, 0, b, h) for b, h in units]))
        wall_dec = time.perf_counter() - t0
        det_units = units[:max(1, min(len(units), workers))]
        t0 = time.perf_counter()
        det = list(ex.map(_cpu_detect_unit, [(w.name, b, h) for b, h in det_units]))
        wall_det = time.perf_counter() - t0
        tiny = list(ex.map(_cpu_decode_unit, [("tiny", 0, 0, 0)]))[0]
        glm = list(ex.map(_cpu_detect_unit, [("glm32k", 0, h) for h in range(2)]))
        extra = {"tiny_step_s": round(tiny, 4), "glm32k_detection_s": round(max(glm), 3)}
        if time.time() - t_all < seconds and w.name != "qwen128k":
            synth_units = [(b, h) for b in (0, 15) for h in (0, 7)][:max(1, min(4, workers))]
            qs = list(ex.map(_cpu_decode_unit, [("qwen128k", 0, b, h) for b, h in synth_units]))
            per_unit = float(np.mean(qs))
            n_units = 16 * 8
            extra["qwen128k_step_s_extrapolated"] = round(per_unit * n_units / workers, 3)
            extra["qwen128k_sample"] = (f"{len(qs)} of {n_units} units timed ({per_unit:.3f} s each on one "
                                        f"core), x {n_units} / {workers} workers")
    # step time with the pool: the units' timed oracle work spread over the
    # workers (never below the longest unit), plus 1/64 of one detection of
    # every unit spread the same way
    det_all = float(np.mean(det)) * len(units)
    s_per_step = max(sum(dec) / workers, max(dec)) + max(det_all / workers, max(det)) / 64
    single = sum(dec) + det_all / 64
    return {"value": round(step_bytes / s_per_step / 1e9, 4), "unit": "GB/s",
            "us_per_step": round(s_per_step * 1e6, 1),
            "single_core_us_per_step": round(single * 1e6, 1),
            "gpu_over_cpu": round(s_per_step * 1e6 / gpu_us_per_step, 1),
            "cores": workers, "kind": "oracle",
            "cpu_model": _cpu_model(),
            "sample": f"the {w.name} step's {len(units)} (b, kv-head) decode units in a pool of {workers} "
                      f"single-threaded processes (oracle time per unit {min(dec):.3f}-{max(dec):.3f} s; "
                      f"pool wall {wall_dec:.2f} s incl. regenerating inputs), the detector over "
                      f"{len(det_units)} units ({float(np.mean(det)):.3f} s each) x 1/64 per step; inputs "
                      f"regenerated and quantized outside the timed part",
            **extra}


if __name__ == "__main__":
    main()
