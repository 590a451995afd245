#!/usr/bin/env python3
"""Forward-pass throughput of Lightning attention on one MI355X.

Workload: B=4, H=Hkv=32, dk=dv=128, N=32768 tokens per row, bf16 q/k/v, fp32 o and
final state, decay schedule of layer 0 of 12, no initial state, forward direction.
A step is one lattn_fwd call over the whole batch with inputs already in HBM.

Order: host-side inputs (numpy) first, then the forward with a bf16 o (the same kernel;
its calls bring the clocks up), then the headline (exactly --warmup untimed and --steps
timed calls), then the other GPU legs back to back, then the CPU oracle baselines.
Timing the headline right after a short stretch of the same work keeps it clear of the
clock ramp that the first calls after an idle period show, and of the heat of the
minute of other legs.  Every leg reports the mean, median, minimum and maximum of its
per-call HIP-event times.

Prints one JSON line:  value = B*N / (seconds per step)  [tokens/s], plus
  roofline      achieved HBM GB/s of the forward kernel (algorithmic bytes / mean
                kernel time from HIP events on the launch stream) against 8 TB/s, the
                same against the dense bf16 MFMA peak on the recurrence's flops, and
                `bound` = the roofline with the larger fraction,
  cpu_baseline  the fp64 CPU oracle timed on a bounded sample of the same workload
                (with the CPU model and thread count); the sweep entries carry one
                oracle run each over the whole workload at their N,
  backward      the same for lattn_bwd on the same inputs (bf16 d_o), with its own
                roofline and oracle baseline (skipped with --no-bwd),
  decode        one decoding step (lattn_decode) over --decode-batch sequences of the
                same head shape, state updated in place,
  split         the forward at B1 H8 (same head dims and N), where the rows are split
                along the sequence, against the same call unsplit,
  gated         the gated (GLA) forward on the same inputs plus a per-key-channel gate g,
                against HBM (its binding roofline at bf16 MFMA rates), with the bf16
                matrix figure beside it,
  bf16_out      the same forward with o in bf16 (skipped with --no-bf16-out),
  configs       the other parity workloads (tiny fp32, B2 H8 d64, B2 H12 d192, packed GQA
                in both directions), forward only (skipped with --no-configs); the packed
                ones also without the split planner,
  packed_split  a skewed packed batch (one long sequence among short ones) with the
                device-planned split against the same call unsplit,
  sweep         the forward at N = 512 .. 16384 (same B, H, head dims), each N rotating
                over enough input sets that about 1 GB is touched between repeats, with
                the Lightning-2 forward time the pages print for that N beside it
                (skipped with --no-sweep).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fwd tokens/s at B4 H32 d128 bf16 N=32K; % of MFMA/HBM roofline"
HBM_PEAK_GBS = 8000.0
FP32_MFMA_PEAK_TFS = 157.3  # dense fp32 matrix peak of MI355X
BF16_MFMA_PEAK_TFS = 2500.0  # dense bf16 matrix peak of MI355X
# Lightning2 forward at B4 H32 d128 bf16 n=32768 from the OpenNLPLab lightning-attention
# README benchmark table (hardware unstated, time read as milliseconds): 17.661427 ms.
PAGE_LIGHTNING2_MS = 17.661427
# the same README table (Lightning2 column, read as ms) at B4 H32 d128, by n
PAGE_LIGHTNING2_SWEEP_MS = {512: 0.351540, 1024: 0.585876, 2048: 1.134238, 4096: 2.240815, 8192: 4.414397,
                            16384: 8.832678, 32768: 17.661427}
SWEEP_N = (512, 1024, 2048, 4096, 8192, 16384)
PAGE_LIGHTNING2_BWD_MS = 74.594788  # same table's backward row at n = 32768
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_fwd_bf16_b4_h32_d128_n32768.json")
# the forward kernel's translation unit: its source and the two headers it includes
KERNEL_SRCS = [os.path.join(ROOT, "decayed_recurrent_attention_amd", "csrc", n)
               for n in ("lattn_kernels.hip", "lattn_device.h", "lattn_launch.h")]


def algorithmic_bytes(B, T, H, Hkv, dk, dv, in_bytes, with_init=False, o_bytes=4):
    """Bytes the forward must move at least once: q, k, v in, o (fp32, or bf16 with
    o_bytes=2) out, final state out."""
    qkv = B * T * (H * dk + Hkv * dk + Hkv * dv) * in_bytes
    o = B * T * H * dv * o_bytes
    state = B * H * dk * dv * 4 * (2 if with_init else 1)
    return qkv + o + state


def kernel_sha() -> str:
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch from committed counter runs, if they match this kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_sha") != kernel_sha():
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(w, data, target_s=15.0):
    """Time the oracle on the workload's (batch row, head) pairs, about target_s of CPU work.

    The sample grows until it takes about target_s: more (batch row, head) pairs, or the
    whole workload repeated once every pair is in.  Only the last pass is reported.
    """
    import oracle

    orc = oracle.load()
    threads = orc.set_threads(0)
    all_pairs = [(b, h) for h in range(w.num_heads) for b in range(w.batch)]
    g = orc.lightning_g_gamma(w.num_heads, w.layer_idx, w.num_layers)

    def timed(pairs, reps=1):
        t0 = time.perf_counter()
        for _ in range(reps):
            orc.recurrent_fwd(data["q"], data["k"], data["v"], g, w.scale, pairs=pairs)
        return time.perf_counter() - t0

    # Grow the sample fourfold until it takes a quarter of target_s, then size it to
    # about target_s: more pairs, or whole-workload repeats once every pair is in.
    n, reps = min(len(all_pairs), threads), 1
    timed(all_pairs[:1])  # untimed: first-touch of the output buffers, thread start-up
    dt = timed(all_pairs[:n])
    while dt < target_s / 4 and n < len(all_pairs):
        n = min(len(all_pairs), 4 * n)
        dt = timed(all_pairs[:n])
    if dt < target_s:
        if n < len(all_pairs):
            n = min(len(all_pairs), int(n * target_s / dt))
        else:
            reps = max(1, min(20, round(target_s / dt)))
        dt = timed(all_pairs[:n], reps)
    frac = n * reps / len(all_pairs)
    what = (f"all {len(all_pairs)} (batch row, head) pairs x {reps}" if n == len(all_pairs)
            else f"{n} of {len(all_pairs)} (batch row, head) pairs")
    return {
        "value": w.batch * w.seqlen * frac / dt,
        "unit": "tokens/s",
        "cores": min(threads, n),
        "kind": "oracle",
        "sample": f"{what} over all {w.seqlen} tokens, fp64, {dt:.1f} s wall; "
                  f"tokens/s = whole-workload tokens x {frac:.3g} / wall",
    }


def device_bandwidth(torch, dev, gib=2, reps=5):
    """Best-of-reps GB/s of a device copy (read + write bytes) and a fill (write bytes)."""
    n = gib * (1 << 30) // 4
    src = torch.ones(n, device=dev, dtype=torch.float32)
    dst = torch.empty_like(src)
    res = {}
    for name, fn, moved in (("copy", lambda: dst.copy_(src), 2 * 4 * n), ("fill", lambda: dst.fill_(2.0), 4 * n)):
        best = float("inf")
        for _ in range(reps + 1):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1))
        res[name] = moved / (best * 1e-3) / 1e9
    del src, dst
    return f"device copy {gib} GiB: {res['copy']:.0f} GB/s (read + write), fill: {res['fill']:.0f} GB/s"


def time_calls(torch, fn, stream, warmup, steps, settle_s=0.0):
    """Run fn warmup times (and, with settle_s > 0, on until that many seconds of calls
    have passed), then time `steps` calls; returns (wall ms per call, event ms list).
    The events bracket each call on the launch stream."""
    t_end = time.perf_counter() + settle_s
    n = 0
    while n < warmup or time.perf_counter() < t_end:
        fn()
        n += 1
        if n % 64 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1 in ev:
        e0.record(stream)
        fn()
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return 1000.0 * wall / steps, [e0.elapsed_time(e1) for e0, e1 in ev]


def ms_stats(ms):
    """Mean, median, minimum and maximum of per-call event times (ms)."""
    srt = sorted(ms)
    mid = len(srt) // 2
    med = srt[mid] if len(srt) % 2 else 0.5 * (srt[mid - 1] + srt[mid])
    return {"mean": sum(ms) / len(ms), "median": med, "min": srt[0], "max": srt[-1], "calls": len(ms)}


def cpu_model() -> str:
    """The host CPU's model name from /proc/cpuinfo, with its family, model and stepping
    numbers (a virtual machine may shorten the name), or platform's guess."""
    fields = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if not line.strip():
                    break  # the first processor's block is enough
                key, _, val = line.partition(":")
                fields[key.strip()] = val.strip()
    except OSError:
        pass
    name = fields.get("model name")
    if name:
        ids = [f"{k} {fields[k]}" for k in ("cpu family", "model", "stepping") if fields.get(k)]
        return f"{name} ({', '.join(ids)})" if ids else name
    import platform

    return platform.processor() or "unknown"


def roofline_pair(alg_bytes, alg_flops, kernel_ms, flop_peak_tfs=None):
    """HBM and MFMA roofline figures for one kernel; `bound` names the larger fraction."""
    flop_peak_tfs = BF16_MFMA_PEAK_TFS if flop_peak_tfs is None else flop_peak_tfs
    gbs = alg_bytes / (kernel_ms * 1e-3) / 1e9
    tfs = alg_flops / (kernel_ms * 1e-3) / 1e12
    hbm = {"achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
           "algorithmic_bytes": alg_bytes}
    mfma = {"achieved": tfs, "peak": flop_peak_tfs, "unit": "TFLOP/s", "frac": tfs / flop_peak_tfs,
            "algorithmic_flops": alg_flops}
    bound = "hbm" if hbm["frac"] >= mfma["frac"] else "mfma"
    return bound, hbm, mfma


def fwd_algorithmic_flops(tokens, H, dk, dv):
    """The recurrence's flops: a rank-1 state update (2 dk dv) and the readout q S (2 dk dv)
    per query head and token."""
    return 4 * tokens * H * dk * dv


def bwd_algorithmic_bytes(B, T, H, Hkv, dk, dv, in_bytes):
    """Bytes the backward must move at least once: q, k, v and dO in (input dtype); dq, dk,
    dv (fp32) and d_initial_state (fp32) out."""
    ins = B * T * (H * dk + Hkv * dk + Hkv * dv + H * dv) * in_bytes
    outs = B * T * (H * dk + Hkv * dk + Hkv * dv) * 4
    return ins + outs + B * H * dk * dv * 4


def cpu_baseline_bwd(w, data, grads, target_s=10.0):
    """Time the oracle's backward on the first (batch row, head) pairs of the workload
    (row-major), about target_s of CPU work; heads of one row run as one call."""
    import numpy as np

    import oracle

    orc = oracle.load()
    threads = orc.set_threads(0)
    B, H = w.batch, w.num_heads
    assert w.num_kv_heads == H, "the sample slices heads, which needs one kv head per head"
    g = orc.lightning_g_gamma(H, w.layer_idx, w.num_layers)
    rows = {}

    def sliced(b):
        if b not in rows:
            rows[b] = [np.ascontiguousarray(a[b:b + 1]) for a in (data["q"], data["k"], data["v"], grads["d_o"])]
        return rows[b]

    def timed(n):
        dt = 0.0
        for b in range(B):
            nh = min(H, n - b * H)
            if nh <= 0:
                break
            q, k, v, do = (np.ascontiguousarray(a[:, :, :nh]) for a in sliced(b))
            t0 = time.perf_counter()
            orc.recurrent_bwd(q, k, v, g[:nh], w.scale, do, want_d_init=True)
            dt += time.perf_counter() - t0
        return dt

    total = B * H
    n = min(total, threads)
    timed(1)  # untimed warm-up
    dt = timed(n)
    while dt < target_s / 4 and n < total:
        n = min(total, 4 * n)
        dt = timed(n)
    if dt < target_s and n < total:
        n = min(total, int(n * target_s / dt))
        dt = timed(n)
    return {
        "value": B * w.seqlen * (n / total) / dt,
        "unit": "tokens/s",
        "cores": min(threads, n),
        "kind": "oracle",
        "sample": f"backward of {n} of {total} (batch row, head) pairs over all {w.seqlen} tokens, "
                  f"fp64, {dt:.1f} s in the oracle; tokens/s scaled by the pair fraction",
    }


def cpu_baseline_decode(w, data, target_s=5.0):
    """Time the oracle on the decoding step (the recurrence at seqlen 1 from the state),
    repeated until about target_s."""
    import oracle

    orc = oracle.load()
    threads = orc.set_threads(0)
    g = orc.lightning_g_gamma(w.num_heads, w.layer_idx, w.num_layers)
    args = (data["q"], data["k"], data["v"], g, w.scale)
    orc.recurrent_fwd(*args, initial_state=data["initial_state"])  # untimed warm-up
    t0 = time.perf_counter()
    reps = 0
    while time.perf_counter() - t0 < target_s and reps < 1000:
        orc.recurrent_fwd(*args, initial_state=data["initial_state"])
        reps += 1
    dt = time.perf_counter() - t0
    return {"value": w.batch * reps / dt, "unit": "tokens/s", "cores": min(threads, w.batch * w.num_heads),
            "kind": "oracle",
            "sample": f"the whole decoding step ({w.batch} sequences) x {reps}, fp64, {dt:.1f} s wall"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50,
                    help="untimed steps first: the clocks take some 20-50 forward calls to settle")
    ap.add_argument("--seqlen", type=int, default=32768)
    ap.add_argument("--settle", type=float, default=0.3,
                    help="seconds of untimed calls before each secondary leg (besides --warmup)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-bwd", action="store_true", help="skip the backward measurement")
    ap.add_argument("--no-gated", action="store_true",
                    help="skip the gated (GLA, per-token log-decay gate g) forward measurement")
    ap.add_argument("--no-split", action="store_true",
                    help="skip the intra-sequence split measurement (B1 H8, same head dims and N)")
    ap.add_argument("--decode-batch", type=int, default=128,
                    help="sequences per decoding step in the decode measurement (0 skips it)")
    ap.add_argument("--no-bf16-out", action="store_true",
                    help="skip the forward with a bf16 o (same inputs)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip timing the other parity workloads (tiny fp32, d64, d192, packed GQA)")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the forward sweep over N = 512 .. 16384 (same B, H, head dims)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a 1 GiB device copy (counter calibration for traffic)")
    ap.add_argument("--bandwidth", action="store_true",
                    help="also time a 2 GiB device copy (read + write) and fill (write) for reference")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the forward pass has no multi-GPU path "
              "(pass --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from decayed_recurrent_attention_amd import inputs, lattn

    def log(msg):
        print("[bench] " + msg, file=sys.stderr, flush=True)

    # -- host-side inputs first (numpy), so that the GPU legs below run back to back --------
    w = inputs.long_d128(seqlen=args.seqlen)
    B, T, H, Hkv, dk, dv = w.batch, w.seqlen, w.num_heads, w.num_kv_heads, w.dk, w.dv
    log(f"generating {w.name}")
    data = w.make()
    grads = None if args.no_bwd else w.make_grads(final_std=None)
    gates = None if args.no_gated else w.make_gates(("g",), 0.1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    to_dev = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    q, k, v = to_dev(data["q"]), to_dev(data["k"]), to_dev(data["v"])
    g = torch.from_numpy(lattn.lattn_lightning_g_gamma(H, w.layer_idx, w.num_layers)).to(dev)
    o = torch.empty((B, T, H, dv), device=dev, dtype=torch.float32)
    fs = torch.empty((B, H, dk, dv), device=dev, dtype=torch.float32)
    prob = lattn.LattnProblem(B, T, H, Hkv, dk, dv, 0, lattn.LATTN_BF16, lattn.LATTN_F32)
    stream = torch.cuda.current_stream(dev)
    settle = args.settle

    def step():
        rc = lattn.lattn_fwd(prob, q, k, v, g, w.scale, None, False, None, o, fs,
                             stream=stream.cuda_stream)
        if rc != lattn.LATTN_OK:
            raise lattn.LattnError(rc)

    # -- the forward with a bf16 o first (the same kernel): it brings the clocks up, so
    # that the headline right after it is not timed on the ramp that follows an idle GPU;
    # the other legs run after the headline -------------------------------------------------
    bf16_out = None
    if not args.no_bf16_out:
        # The same forward with o in bf16 (each element the round-to-nearest-even of the
        # fp32 result): 20 % fewer bytes per call.
        log("forward with a bf16 o")
        ob = torch.empty((B, T, H, dv), device=dev, dtype=torch.bfloat16)
        prob_b = lattn.LattnProblem(B, T, H, Hkv, dk, dv, 0, lattn.LATTN_BF16, lattn.LATTN_BF16)

        def step_b():
            rc = lattn.lattn_fwd(prob_b, q, k, v, g, w.scale, None, False, None, ob, fs,
                                 stream=stream.cuda_stream)
            if rc != lattn.LATTN_OK:
                raise lattn.LattnError(rc)

        b_wall, b_ms = time_calls(torch, step_b, stream, args.warmup, args.steps, settle)
        st = ms_stats(b_ms)
        b_alg = algorithmic_bytes(B, T, H, Hkv, dk, dv, 2, o_bytes=2)
        b_gbs = b_alg / (st["mean"] * 1e-3) / 1e9
        bf16_out = {"ms_per_step": b_wall, "tokens_per_s": B * T / (b_wall * 1e-3), "kernel_ms": st,
                    "roofline": {"bound": "hbm", "achieved": b_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                 "frac": b_gbs / HBM_PEAK_GBS, "algorithmic_bytes": b_alg,
                                 "call_ms": st["mean"]},
                    "inputs": "the forward's; o bf16 (round to nearest even of the fp32 result), "
                              "fp32 final state"}
        log(f"bf16 o {args.steps} steps: {b_wall:.4f} ms/step wall, mean {st['mean']:.4f} ms, "
            f"median {st['median']:.4f} ms, {b_gbs:.0f} GB/s")
        del ob

    # -- the headline: exactly --warmup untimed and --steps timed forward calls ---------------
    log("forward (headline)")
    ms_per_step, kernel_ms = time_calls(torch, step, stream, args.warmup, args.steps)
    kst = ms_stats(kernel_ms)
    log(f"{args.steps} steps: {ms_per_step:.4f} ms/step wall, kernel mean {kst['mean']:.4f} ms median "
        f"{kst['median']:.4f} ms min {kst['min']:.4f} max {kst['max']:.4f}")

    bwd = None
    if not args.no_bwd:
        d_o = to_dev(grads["d_o"])
        dq = torch.empty((B, T, H, dk), device=dev, dtype=torch.float32)
        dkk = torch.empty((B, T, Hkv, dk), device=dev, dtype=torch.float32)
        dvv = torch.empty((B, T, Hkv, dv), device=dev, dtype=torch.float32)
        dinit = torch.empty((B, H, dk, dv), device=dev, dtype=torch.float32)
        ws_bytes = lattn.lattn_bwd_workspace_size(prob)
        ws = torch.empty(ws_bytes, device=dev, dtype=torch.uint8) if ws_bytes else None

        def bstep():
            rc = lattn.lattn_bwd(prob, q, k, v, g, w.scale, None, False, None, d_o, None, dq, dkk, dvv,
                                 dinit, ws, stream=stream.cuda_stream)
            if rc != lattn.LATTN_OK:
                raise lattn.LattnError(rc)

        log("backward")
        b_wall, b_ms = time_calls(torch, bstep, stream, args.warmup, args.steps, settle)
        st = ms_stats(b_ms)
        b_alg = bwd_algorithmic_bytes(B, T, H, Hkv, dk, dv, 2)
        bound, hbm, mfma = roofline_pair(b_alg, 2 * fwd_algorithmic_flops(B * T, H, dk, dv) + 2 * B * T * H * dk * dv,
                                         st["mean"])
        log(f"backward {args.steps} steps: {b_wall:.4f} ms/step wall, mean {st['mean']:.4f} ms, "
            f"median {st['median']:.4f} ms")
        bwd = {"ms_per_step": b_wall, "tokens_per_s": B * T / (b_wall * 1e-3), "kernel_ms": st,
               "roofline": dict(bound=bound, **hbm, call_ms=st["mean"]), "mfma": mfma,
               "inputs": "q, k, v, d_o bf16; no initial state, no final-state gradient; "
                         "d_initial_state computed",
               "page_lightning2_bwd_ms": PAGE_LIGHTNING2_BWD_MS if T == 32768 else None}
        del dq, dkk, dvv, d_o

    gated = None
    if not args.no_gated:
        gdev = to_dev(gates["g"])
        go = torch.empty((B, T, H, dv), device=dev, dtype=torch.float32)
        gfs = torch.empty((B, H, dk, dv), device=dev, dtype=torch.float32)

        def gstep():
            rc = lattn.lattn_fwd_gated(prob, q, k, v, gdev, None, None, None, w.scale, None, False, None, go,
                                       gfs, stream=stream.cuda_stream)
            if rc != lattn.LATTN_OK:
                raise lattn.LattnError(rc)

        log("gated forward")
        g_wall, g_ms = time_calls(torch, gstep, stream, args.warmup, args.steps, settle)
        st = ms_stats(g_ms)
        g_bytes = algorithmic_bytes(B, T, H, Hkv, dk, dv, 2) + B * T * H * dk * 2
        # the recurrence: decay (1), rank-1 update (2) and readout (2) flops per state element per token
        g_flops = 5 * B * T * H * dk * dv
        log(f"gated {args.steps} steps: {g_wall:.4f} ms/step wall, mean {st['mean']:.4f} ms, "
            f"median {st['median']:.4f} ms")
        # bf16 inputs run on bf16 MFMA (hi/lo operand splits): at bf16 rates the
        # algorithm's bytes bind (6.45 GB at 8 TB/s vs 0.34 TFLOP at 2.5 PFLOP/s)
        bound, hbm, mfma = roofline_pair(g_bytes, g_flops, st["mean"])
        gated = {"workload": f"GLA gate g ~ U[-0.1, 0) per key channel, B{B} H{H} d{dk} N{T} bf16, "
                             "bf16 MFMA with hi/lo splits, fp32 accumulation",
                 "ms_per_step": g_wall, "tokens_per_s": B * T / (g_wall * 1e-3), "kernel_ms": st,
                 "roofline": dict(bound=bound, **hbm, call_ms=st["mean"]), "mfma": mfma}
        del gdev, go, gfs

    split = None
    if not args.no_split:
        # One batch row and 8 heads: 32 workgroups unsplit, so the forward cuts each row
        # into segments chained through their states.
        Hs = 8
        ws_ = inputs.Workload("split", 1, T, Hs, Hs, dk, dv, "bf16", w.layer_idx, w.num_layers, seed=5)
        sd = ws_.make()
        sq, sk, sv = (to_dev(sd[n]) for n in ("q", "k", "v"))
        gs = torch.from_numpy(lattn.lattn_lightning_g_gamma(Hs, w.layer_idx, w.num_layers)).to(dev)
        so = torch.empty((1, T, Hs, dv), device=dev, dtype=torch.float32)
        sfs = torch.empty((1, Hs, dk, dv), device=dev, dtype=torch.float32)
        sprob = lattn.LattnProblem(1, T, Hs, Hs, dk, dv, 0, lattn.LATTN_BF16, lattn.LATTN_F32)
        res = {}
        for mode in ("split", "unsplit"):
            with lattn.knob(lattn.LATTN_KNOB_SPLIT, 0 if mode == "unsplit" else lattn.LATTN_KNOB_AUTO):
                nbytes = lattn.lattn_fwd_workspace_size(sprob)
                sws = torch.empty(nbytes, device=dev, dtype=torch.uint8) if nbytes else None

                def sstep():
                    rc = lattn.lattn_fwd(sprob, sq, sk, sv, gs, ws_.scale, None, False, None, so, sfs, sws,
                                         stream=stream.cuda_stream)
                    if rc != lattn.LATTN_OK:
                        raise lattn.LattnError(rc)

                wall_ms, ev_ms = time_calls(torch, sstep, stream, args.warmup, args.steps, settle)
            res[mode] = (wall_ms, ms_stats(ev_ms), nbytes)
        s_alg = algorithmic_bytes(1, T, Hs, Hs, dk, dv, 2)
        s_mean = res["split"][1]["mean"]
        s_ach = s_alg / (s_mean * 1e-3) / 1e9
        log(f"split B1 H{Hs}: {s_mean:.4f} ms split, {res['unsplit'][1]['mean']:.4f} ms unsplit")
        split = {"workload": f"B1 H{Hs} d{dk} N{T} bf16, no initial state",
                 "ms_per_step": res["split"][0], "tokens_per_s": T / (res["split"][0] * 1e-3),
                 "kernel_ms": res["split"][1],
                 "unsplit_ms_per_step": res["unsplit"][0], "unsplit_kernel_ms": res["unsplit"][1],
                 "speedup": res["unsplit"][1]["mean"] / s_mean,
                 "workspace_bytes": res["split"][2],
                 "roofline": {"bound": "hbm", "achieved": s_ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                              "frac": s_ach / HBM_PEAK_GBS, "algorithmic_bytes": s_alg, "call_ms": s_mean}}
        del sq, sk, sv, so

    dec = None
    if args.decode_batch > 0:
        Bd = args.decode_batch
        wd = inputs.Workload("decode", Bd, 1, H, Hkv, dk, dv, "bf16", w.layer_idx, w.num_layers,
                             init_std=0.5, seed=3)
        dd = wd.make()
        dq_, dk_, dv_ = (to_dev(dd[n])[:, 0].contiguous() for n in ("q", "k", "v"))
        state = torch.from_numpy(dd["initial_state"]).to(dev)
        o_dec = torch.empty((Bd, H, dv), device=dev, dtype=torch.float32)
        dprob = lattn.LattnProblem(Bd, 1, H, Hkv, dk, dv, 0, lattn.LATTN_BF16, lattn.LATTN_F32)

        def dstep():
            rc = lattn.lattn_decode(dprob, dq_, dk_, dv_, g, w.scale, state, state, o_dec,
                                    stream=stream.cuda_stream)
            if rc != lattn.LATTN_OK:
                raise lattn.LattnError(rc)

        log("decode")
        d_wall, d_ms = time_calls(torch, dstep, stream, args.warmup, args.steps, settle)
        st = ms_stats(d_ms)
        d_alg = 2 * Bd * H * dk * dv * 4 + Bd * (H * dk + Hkv * dk + Hkv * dv) * 2 + Bd * H * dv * 4
        d_ach = d_alg / (st["mean"] * 1e-3) / 1e9
        log(f"decode {args.steps} steps: {d_wall:.4f} ms/step wall, mean {st['mean']:.4f} ms")
        dec = {"batch": Bd, "ms_per_step": d_wall, "tokens_per_s": Bd / (d_wall * 1e-3), "kernel_ms": st,
               "roofline": {"bound": "hbm", "achieved": d_ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": d_ach / HBM_PEAK_GBS, "algorithmic_bytes": d_alg, "call_ms": st["mean"]},
               "inputs": f"{Bd} sequences x H{H} d{dk}: q, k, v bf16, fp32 state updated in place"}
        del o_dec

    configs = None
    if not args.no_configs:
        # The other workloads of the parity suite, forward only, same timing: ms per call
        # (HIP events over every kernel of the call), tokens/s and the HBM fraction on each
        # one's algorithmic bytes.
        log("other workloads")
        configs = []
        for cw in (inputs.tiny_fp32(), inputs.bf16_d64(), inputs.d192(), inputs.varlen_gqa(False),
                   inputs.varlen_gqa(True)):
            cd = cw.make()
            f32in = cw.dtype == "f32"
            dev_in = (lambda a: torch.from_numpy(a).to(dev)) if f32in else to_dev
            cq, ck, cv = (dev_in(cd[n]) for n in ("q", "k", "v"))
            cinit = None if cd["initial_state"] is None else torch.from_numpy(cd["initial_state"]).to(dev)
            cu = None if cd["cu_seqlens"] is None else torch.from_numpy(cd["cu_seqlens"]).to(dev, torch.int32)
            cg = torch.from_numpy(lattn.lattn_lightning_g_gamma(cw.num_heads, cw.layer_idx, cw.num_layers)).to(dev)
            nseq = cw.num_seqs
            co = torch.empty((cw.batch, cw.seqlen, cw.num_heads, cw.dv), device=dev, dtype=torch.float32)
            cfs = torch.empty((nseq, cw.num_heads, cw.dk, cw.dv), device=dev, dtype=torch.float32)
            cprob = lattn.LattnProblem(cw.batch, cw.seqlen, cw.num_heads, cw.num_kv_heads, cw.dk, cw.dv,
                                       nseq if cu is not None else 0,
                                       lattn.LATTN_F32 if f32in else lattn.LATTN_BF16, lattn.LATTN_F32)
            cws_n = lattn.lattn_fwd_workspace_size(cprob)
            cws = torch.empty(cws_n, device=dev, dtype=torch.uint8) if cws_n else None

            def cstep():
                rc = lattn.lattn_fwd(cprob, cq, ck, cv, cg, cw.scale, cinit, cw.reverse, cu, co, cfs, cws,
                                     stream=stream.cuda_stream)
                if rc != lattn.LATTN_OK:
                    raise lattn.LattnError(rc)

            c_wall, c_ms = time_calls(torch, cstep, stream, args.warmup, args.steps, settle)
            st = ms_stats(c_ms)
            unplanned = None
            if cu is not None:
                # the same call without the split planner (the longest-first order only)
                with lattn.knob(lattn.LATTN_KNOB_SPLIT, 0):
                    n0 = lattn.lattn_fwd_workspace_size(cprob)
                    cws0 = torch.empty(n0, device=dev, dtype=torch.uint8) if n0 else None

                    def cstep0():
                        rc = lattn.lattn_fwd(cprob, cq, ck, cv, cg, cw.scale, cinit, cw.reverse, cu, co, cfs, cws0,
                                             stream=stream.cuda_stream)
                        if rc != lattn.LATTN_OK:
                            raise lattn.LattnError(rc)

                    unplanned = ms_stats(time_calls(torch, cstep0, stream, args.warmup, args.steps, settle)[1])
            ntok = cw.batch * cw.seqlen
            c_alg = (ntok * (cw.num_heads * cw.dk + cw.num_kv_heads * (cw.dk + cw.dv)) * (4 if f32in else 2)
                     + ntok * cw.num_heads * cw.dv * 4
                     + nseq * cw.num_heads * cw.dk * cw.dv * 4 * (2 if cinit is not None else 1))
            c_gbs = c_alg / (st["mean"] * 1e-3) / 1e9
            configs.append({"workload": cw.name, "batch": cw.batch, "tokens": ntok, "num_seqs": nseq,
                            "num_heads": cw.num_heads, "num_kv_heads": cw.num_kv_heads, "head_dim_qk": cw.dk,
                            "head_dim_v": cw.dv, "dtype": cw.dtype, "reverse": bool(cw.reverse),
                            "initial_state": cinit is not None, "ms_per_step": c_wall, "kernel_ms": st,
                            "tokens_per_s": ntok / (c_wall * 1e-3), "algorithmic_bytes": c_alg,
                            "hbm_gbs": c_gbs, "hbm_frac": c_gbs / HBM_PEAK_GBS})
            if unplanned is not None:
                configs[-1]["kernel_ms_without_planner"] = unplanned
            log(f"{cw.name}: {c_wall:.4f} ms/step wall, mean {st['mean']:.4f} ms, median {st['median']:.4f} ms, "
                f"{c_gbs:.0f} GB/s")
            del cq, ck, cv, co, cfs, cws

    packed_split = None
    if not args.no_configs:
        # A skewed packed batch: one sequence of 49152 tokens among 31 of 64 .. 1024 tokens
        # (H16 / kv 4, d128, initial states).  Unsplit, the long sequence sets the call's
        # length; the planner cuts it into segments.
        lens = [49152] + [int(x) for x in inputs.lengths(31, 64, 1024, 9)]
        pw = inputs.Workload("packed_skewed", 1, sum(lens), 16, 4, dk, dv, "bf16", 6, 12, seq_lens=lens,
                             init_std=0.1, seed=9)
        log(f"skewed packed batch ({sum(lens)} tokens)")
        pd = pw.make()
        pq, pk, pv = (to_dev(pd[n]) for n in ("q", "k", "v"))
        pinit = torch.from_numpy(pd["initial_state"]).to(dev)
        pcu = torch.from_numpy(pd["cu_seqlens"]).to(dev, torch.int32)
        pg = torch.from_numpy(lattn.lattn_lightning_g_gamma(16, 6, 12)).to(dev)
        po = torch.empty((1, pw.seqlen, 16, dv), device=dev, dtype=torch.float32)
        pfs = torch.empty((len(lens), 16, dk, dv), device=dev, dtype=torch.float32)
        pprob = lattn.LattnProblem(1, pw.seqlen, 16, 4, dk, dv, len(lens), lattn.LATTN_BF16, lattn.LATTN_F32)
        res = {}
        for mode, kv in (("planned", lattn.LATTN_KNOB_AUTO), ("unsplit", 0)):
            with lattn.knob(lattn.LATTN_KNOB_SPLIT, kv):
                nb = lattn.lattn_fwd_workspace_size(pprob)
                pws = torch.empty(nb, device=dev, dtype=torch.uint8) if nb else None

                def pstep():
                    rc = lattn.lattn_fwd(pprob, pq, pk, pv, pg, pw.scale, pinit, False, pcu, po, pfs, pws,
                                         stream=stream.cuda_stream)
                    if rc != lattn.LATTN_OK:
                        raise lattn.LattnError(rc)

                wall_ms, ev_ms = time_calls(torch, pstep, stream, args.warmup, args.steps, settle)
            res[mode] = (wall_ms, ms_stats(ev_ms), nb)
        p_alg = (pw.seqlen * (16 * dk + 4 * (dk + dv)) * 2 + pw.seqlen * 16 * dv * 4 + 2 * len(lens) * 16 * dk * dv * 4)
        p_mean = res["planned"][1]["mean"]
        p_gbs = p_alg / (p_mean * 1e-3) / 1e9
        packed_split = {"workload": f"packed: 1 x 49152 + 31 x U[64, 1024] tokens ({pw.seqlen}), H16 kv4 d{dk} bf16, "
                                    "initial states, forward",
                        "ms_per_step": res["planned"][0], "kernel_ms": res["planned"][1],
                        "unsplit_kernel_ms": res["unsplit"][1],
                        "speedup": res["unsplit"][1]["mean"] / p_mean, "workspace_bytes": res["planned"][2],
                        "tokens_per_s": pw.seqlen / (res["planned"][0] * 1e-3),
                        "roofline": {"bound": "hbm", "achieved": p_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                     "frac": p_gbs / HBM_PEAK_GBS, "algorithmic_bytes": p_alg, "call_ms": p_mean}}
        log(f"skewed packed: {p_mean:.4f} ms planned, {res['unsplit'][1]['mean']:.4f} ms unsplit")
        del pq, pk, pv, po

    sweep = None
    if not args.no_sweep:
        # The forward at smaller N on device-drawn inputs of the same shape.  Below 1 GB per
        # call, calls rotate over enough buffer sets (about 1 GB in all) that the working
        # set cannot stay in the 256 MB Infinity Cache.
        log("sweep over N")
        sweep = []
        for n in SWEEP_N:
            nbytes = algorithmic_bytes(B, n, H, Hkv, dk, dv, 2)
            nsets = max(1, min(16, -(-(1 << 30) // nbytes)))
            sets = []
            for _ in range(nsets):
                qs = torch.randn((B, n, H, dk), device=dev, dtype=torch.bfloat16)
                ks = torch.randn((B, n, Hkv, dk), device=dev, dtype=torch.bfloat16)
                vs = torch.randn((B, n, Hkv, dv), device=dev, dtype=torch.bfloat16)
                os_ = torch.empty((B, n, H, dv), device=dev, dtype=torch.float32)
                fss = torch.empty((B, H, dk, dv), device=dev, dtype=torch.float32)
                sets.append((qs, ks, vs, os_, fss))
            sprob = lattn.LattnProblem(B, n, H, Hkv, dk, dv, 0, lattn.LATTN_BF16, lattn.LATTN_F32)
            it = [0]

            def sweep_step():
                qs, ks, vs, os_, fss = sets[it[0] % nsets]
                it[0] += 1
                rc = lattn.lattn_fwd(sprob, qs, ks, vs, g, w.scale, None, False, None, os_, fss,
                                     stream=stream.cuda_stream)
                if rc != lattn.LATTN_OK:
                    raise lattn.LattnError(rc)

            n_wall, n_ms = time_calls(torch, sweep_step, stream, args.warmup, args.steps, settle)
            st = ms_stats(n_ms)
            gbs = nbytes / (st["mean"] * 1e-3) / 1e9
            sweep.append({"seq_len": n, "ms_per_step": n_wall, "kernel_ms": st,
                          "tokens_per_s": B * n / (n_wall * 1e-3), "hbm_gbs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
                          "buffer_sets": nsets, "page_lightning2_ms": PAGE_LIGHTNING2_SWEEP_MS[n]})
            log(f"sweep N={n}: {n_wall:.4f} ms/step wall, kernel mean {st['mean']:.4f} ms, median "
                f"{st['median']:.4f} ms, {gbs:.0f} GB/s ({nsets} buffer sets)")
            del sets

    if args.copy_probe:
        src = torch.empty(1 << 28, device=dev, dtype=torch.float32)  # 1 GiB
        dst = torch.empty_like(src)
        src.fill_(1.0)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if args.bandwidth:
        log(device_bandwidth(torch, dev))

    if sweep is not None:
        full_gbs = algorithmic_bytes(B, T, H, Hkv, dk, dv, 2) / (kst["mean"] * 1e-3) / 1e9
        sweep.append({"seq_len": T, "ms_per_step": ms_per_step, "kernel_ms": kst,
                      "tokens_per_s": B * T / (ms_per_step * 1e-3), "hbm_gbs": full_gbs,
                      "hbm_frac": full_gbs / HBM_PEAK_GBS, "buffer_sets": 1,
                      "page_lightning2_ms": PAGE_LIGHTNING2_SWEEP_MS.get(T)})

    alg = algorithmic_bytes(B, T, H, Hkv, dk, dv, 2)
    bound, hbm, mfma = roofline_pair(alg, fwd_algorithmic_flops(B * T, H, dk, dv), kst["mean"])
    value = B * T / (ms_per_step * 1e-3)
    page_tok_s = 4 * 32768 / (PAGE_LIGHTNING2_MS * 1e-3)
    line = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": (value / page_tok_s) if T == 32768 else None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"lightning_attn_fwd_b{B}_h{H}_d{dk}_n{T}_bf16", "batch": B,
                   "seq_len": T, "num_heads": H, "num_kv_heads": Hkv, "head_dim_qk": dk,
                   "head_dim_v": dv, "layer_idx": w.layer_idx, "num_layers": w.num_layers,
                   "out_dtype": "f32", "reverse": False, "initial_state": False},
        "roofline": {"bound": bound, "achieved": hbm["achieved"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": hbm["frac"], "traffic": measured_traffic(), "algorithmic_bytes": alg,
                     "kernel_ms": kst["mean"], "kernel_ms_median": kst["median"], "kernel_ms_min": kst["min"],
                     "kernel_ms_max": kst["max"], "mfma": mfma},
    }

    # -- CPU baselines last (the oracle on the host cores) ------------------------------------
    if not args.no_cpu_baseline:
        import oracle

        log("cpu baseline (oracle)")
        cb = cpu_baseline(w, data)
        cb["cpu_model"] = cpu_model()
        cb["threads"] = oracle.load().set_threads(0)
        line["cpu_baseline"] = cb
        if sweep is not None:
            # One oracle run per sweep N over the whole workload (all rows and heads) on the
            # first N tokens of the headline inputs, timed on the wall clock.
            orc = oracle.load()
            g_np = orc.lightning_g_gamma(H, w.layer_idx, w.num_layers)
            for ent in sweep:
                n = ent["seq_len"]
                cut = [np.ascontiguousarray(data[x][:, :n]) for x in ("q", "k", "v")]
                t0 = time.perf_counter()
                orc.recurrent_fwd(*cut, g_np, w.scale)
                dt = time.perf_counter() - t0
                ent["cpu_oracle_s"] = dt
                ent["cpu_tokens_per_s"] = B * n / dt
                del cut
            log("sweep cpu: " + ", ".join(f"N={e['seq_len']} {e['cpu_oracle_s']:.2f} s" for e in sweep))
        if bwd is not None:
            log("cpu baseline of the backward (oracle)")
            bwd["cpu_baseline"] = cpu_baseline_bwd(w, data, grads)
        if dec is not None:
            dec["cpu_baseline"] = cpu_baseline_decode(wd, dd)
    if bwd is not None:
        line["backward"] = bwd
    if dec is not None:
        line["decode"] = dec
    if split is not None:
        line["split"] = split
    if gated is not None:
        line["gated"] = gated
    if bf16_out is not None:
        line["bf16_out"] = bf16_out
    if sweep is not None:
        line["sweep"] = sweep
    if configs is not None:
        line["configs"] = configs
    if packed_split is not None:
        line["packed_split"] = packed_split
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
