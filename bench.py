"""Throughput of the streaming code2wav decoder on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--precision f32|f16|split] [--weights float|int8] [--graph] [--no-cpu-baseline] [--split-line] [--peaks-only] [--barrier-probe] [--library-gemm]

A step decodes one 25-frame chunk (2 s of audio) for each of 64 independent
streams whose states were first warmed (untimed) to different positions: the
whole decoder (RVQ gather-sum, causal conv, 8-layer windowed transformer, 2x2
upsampling, BigVGAN Snake/AMP stack, tanh) over 128 s of audio.  Inputs are
resident in device memory before timing starts; successive steps continue the
same streams (states ping-pong).  Prints one JSON line.
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

FP32_MFMA_PEAK_TFLOPS = 157.3  # MI355X dense fp32 matrix peak
FP16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 matrix peak (no sparsity)
HBM_PEAK_GBS = 8000.0
FRAME_SECONDS = 0.08  # 12.5 Hz frames


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="qwen3_b64_chunk25")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--split-line", action="store_true",
                    help="fp32 batched run: also time the split-fp16 precision on the same workload")
    ap.add_argument("--cpu-streams", type=int, default=4,
                    help="streams of the timed step whose chunks the CPU oracle decodes for cpu_baseline")
    ap.add_argument("--profile-chunk", type=int, default=0,
                    help="chunk-schedule workloads: add per-kernel device times of the chunks of this length")
    ap.add_argument("--weights", choices=["float", "int8"], default="float",
                    help="matrix weights stored as float, or int8 with one fp16 scale per 32 values")
    ap.add_argument("--graph", action="store_true",
                    help="chunk-schedule workloads: replay each call from a HIP graph")
    ap.add_argument("--precision", choices=["f32", "f16", "split"], default="f32",
                    help="matrix-product operands: f32; fp16 with fp32 sums (the half-precision decoder); or "
                         "split (fp32 values, each product as three fp16 MFMA products of hi/lo halves)")
    # measurement helpers (each replaces the timed run)
    ap.add_argument("--peaks-only", action="store_true",
                    help="run only the roofline microbenchmarks (fp32/fp16 MFMA loops, HBM read and copy)")
    ap.add_argument("--barrier-probe", action="store_true",
                    help="run only the ordering-point microbenchmarks (a grid-wide barrier inside one kernel "
                         "against a dependent launch)")
    ap.add_argument("--library-gemm", action="store_true",
                    help="time the vendor GEMM (torch.matmul) on the BigVGAN conv shapes, inputs expanded per tap")
    ap.add_argument("--counters", action="store_true",
                    help="decode exactly one batched step from fresh states, for rocprofv3 --pmc runs")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="run one device-to-device copy of this many bytes (counter calibration)")
    ap.add_argument("--trace-summary", default=None,
                    help="summarise a rocprofv3 --kernel-trace CSV over the last --steps decode calls")
    ap.add_argument("--traffic-summary", nargs=4, default=None,
                    metavar=("GEMM_FETCH", "GEMM_WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="turn rocprofv3 --pmc CSVs into profiles/traffic.json")
    return ap.parse_args()


# the arithmetic the matrix products run in: split = three fp16 products per pair, fp32 sums
DTYPES = {"f32": "f32", "f16": "f16", "split": "f16x3"}


def _kernel_family(name):
    import re
    # direct-to-LDS fp16 GEMM: TileCfgD<BM, BN, waves_m, waves_n, stages>, split-K, fp16 rows[, split fp16[,
    # slab windows]]
    m = re.search(r"TileCfgD<(\d+), (\d+), \d+, \d+, \d+>, (true|false), (?:true|false)(?:, (true|false))?"
                  r"(?:, (true|false))?", name)
    if m:
        split = "_splitk" if m.group(3) == "true" else ""
        kind = "x3" if m.group(4) == "true" else "f16_dma"
        win = "_win" if m.group(5) == "true" else ""
        return f"conv_gemm_{kind}_{m.group(1)}x{m.group(2)}_bk32{split}{win}"
    m = re.search(r"TileCfg(H?)<(\d+), (\d+), \d+, \d+, (\d+)(?:, -?\d+)*\s*>(?:, (true|false))?"
                  r"(?:, (true|false))?", name)
    if m:
        half = "f16_" if m.group(1) else ""
        q8 = "q8_" if m.group(6) == "true" else ""
        split = "_splitk" if m.group(5) == "true" else ""
        return f"conv_gemm_{half}{q8}{m.group(2)}x{m.group(3)}_bk{m.group(4)}{split}"
    m = re.search(r"(\w+)(?:<[^<>]*>)?\(", name.replace("(anonymous namespace)::", ""))
    return m.group(1) if m else name[:40]


def trace_summary(path, steps):
    """Per-kernel launches and mean duration over the last `steps` decode calls
    of a kernel-trace CSV (each decode call starts with begin_kernel)."""
    import csv

    rows = sorted(csv.DictReader(open(path)), key=lambda r: int(r["Start_Timestamp"]))
    starts = [i for i, r in enumerate(rows) if "begin_kernel" in r["Kernel_Name"]]
    first = starts[-steps]
    agg = {}
    for r in rows[first:]:
        k = _kernel_family(r["Kernel_Name"])
        d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e6
        a = agg.setdefault(k, [0, 0.0])
        a[0] += 1
        a[1] += d
    print(f"last {steps} decode calls of {path}")
    print(f"{'kernel':36s} {'launches':>9s} {'total ms':>10s} {'avg ms':>9s}")
    for k, (n, t) in sorted(agg.items(), key=lambda kv: -kv[1][1]):
        print(f"{k:36s} {n:9d} {t:10.3f} {t / n:9.4f}")


def traffic_summary(gemm_fetch, gemm_write, copy_fetch, copy_write, copy_bytes):
    """HBM bytes per launch of every conv GEMM family, from FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch), each scaled so that a plain copy of
    `copy_bytes` reads and writes exactly that many bytes."""
    import csv

    def per_kernel(paths, counter):
        # paths: one CSV, or several joined by commas (e.g. an fp32 and an fp16 run)
        out = {}
        for path in paths.split(","):
            for r in csv.DictReader(open(path)):
                if r["Counter_Name"] != counter:
                    continue
                k = _kernel_family(r["Kernel_Name"])
                out.setdefault(k, []).append(float(r["Counter_Value"]) * 1024.0)
        return out

    cf = per_kernel(copy_fetch, "FETCH_SIZE")
    cw = per_kernel(copy_write, "WRITE_SIZE")
    ck = max(cf, key=lambda k: max(cf[k]))
    f_scale = copy_bytes / max(cf[ck])
    w_scale = copy_bytes / max(cw[ck])
    gf = per_kernel(gemm_fetch, "FETCH_SIZE")
    gw = per_kernel(gemm_write, "WRITE_SIZE")
    src = os.path.join(ROOT, "vocoder_rvq_codebook_amd", "csrc", "conv_gemm.hip")
    rec = {"conv_gemm_sha256": hashlib.sha256(open(src, "rb").read()).hexdigest(),
           "copy_kernel": ck, "copy_bytes": copy_bytes, "fetch_scale": f_scale, "write_scale": w_scale,
           "kernels": {}}
    for k in gf:
        fb = sum(gf[k]) / len(gf[k]) * f_scale
        wb = sum(gw.get(k, [0.0])) / max(1, len(gw.get(k, []))) * w_scale
        rec["kernels"][k] = {"launches": len(gf[k]), "fetch_bytes_per_launch": fb, "write_bytes_per_launch": wb,
                             "hbm_bytes_per_launch": fb + wb}
    print(json.dumps(rec, indent=1))
    with open(os.path.join(ROOT, "profiles", "traffic.json"), "w") as f:
        json.dump(rec, f, indent=1)


def measure_peaks(torch, vb, reps=5):
    """The roofline denominators measured on this GPU by the library's
    microbenchmark kernels (HIP events on the current stream, best of `reps`
    after a warm-up): dense fp32 and fp16 MFMA rates from register-only MFMA
    loops, and HBM rates of a streaming read (2 GiB) and a copy (1 GiB each
    way)."""
    stream = torch.cuda.current_stream()

    def best(fn):
        fn()
        torch.cuda.synchronize()
        out = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            out.append(e0.elapsed_time(e1) / 1e3)
        return min(out)

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks, iters = 4 * cus, 16384
    sink = torch.empty(blocks * 256, device="cuda")
    res = {}
    for dtype, key in ((0, "mfma_f32_tflops"), (1, "mfma_f16_tflops")):
        def run(dtype=dtype):
            if vb.vocoder_peak_mfma(dtype, sink, blocks, iters) != vb.VOCODER_OK:
                raise SystemExit("vocoder_peak_mfma failed")
        res[key] = round(vb.vocoder_peak_mfma_flops(dtype, blocks, iters) / best(run) / 1e12, 2)
    n_read = (2 << 30) // 4
    src = torch.ones(n_read, device="cuda")
    rblocks = 8 * cus
    rsink = torch.empty(rblocks * 256, device="cuda")

    def read():
        if vb.vocoder_stream_read(src, n_read, rsink, rblocks) != vb.VOCODER_OK:
            raise SystemExit("vocoder_stream_read failed")
    res["hbm_read_gbs"] = round(4.0 * n_read / best(read) / 1e9, 1)
    n_copy = (1 << 30) // 4
    a, b = src[:n_copy], src[n_copy:2 * n_copy]

    def copy():
        if vb.vocoder_stream_copy(a, b, n_copy, rblocks) != vb.VOCODER_OK:
            raise SystemExit("vocoder_stream_copy failed")
    res["hbm_copy_gbs"] = round(8.0 * n_copy / best(copy) / 1e9, 1)
    del src, sink, rsink
    torch.cuda.empty_cache()
    res["method"] = (f"register-only MFMA loops ({blocks} workgroups x 4 waves x 4 independent chains), "
                     f"stream read of 2 GiB and copy of 1 GiB (16-byte grid-stride, {rblocks} workgroups); "
                     f"best of {reps} after a warm-up, HIP events")
    return res


def measure_barrier(torch, vb, rounds=500, launches=1000, reps=3):
    """The price of one ordering point between dependent steps, measured by
    the library's microbenchmarks (HIP events on the current stream, best of
    `reps` after a warm-up): a grid-wide barrier crossed inside one
    cooperative kernel (2 * rounds barriers per launch, each round checking
    data written by another block before the barrier), and a dependent launch
    of an empty kernel."""
    stream = torch.cuda.current_stream()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    res = {"barrier_us": {}, "method": ""}
    for blocks in (cus // 4, cus, 2 * cus):
        flags = torch.zeros(blocks + 1, dtype=torch.int32, device="cuda")
        slots = torch.empty(blocks * 64, device="cuda")
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        best = None
        for rep in range(reps + 1):
            flags.zero_()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            rc = vb.vocoder_grid_barrier(flags, slots, err, blocks, rounds)
            e1.record(stream)
            torch.cuda.synchronize()
            if rc != vb.VOCODER_OK or int(err.item()) != 0:
                raise SystemExit(f"vocoder_grid_barrier failed: rc {rc}, err {int(err.item())}")
            us = 1e3 * e0.elapsed_time(e1) / (2 * rounds)
            if rep:
                best = us if best is None else min(best, us)
        res["barrier_us"][str(blocks)] = round(best, 3)
    scratch = torch.zeros(2, dtype=torch.int32, device="cuda")
    best = None
    for rep in range(reps + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        if vb.vocoder_empty_launches(scratch, cus, launches) != vb.VOCODER_OK:
            raise SystemExit("vocoder_empty_launches failed")
        e1.record(stream)
        torch.cuda.synchronize()
        us = 1e3 * e0.elapsed_time(e1) / launches
        if rep:
            best = us if best is None else min(best, us)
    res["dependent_launch_us"] = round(best, 3)
    res["method"] = (f"cooperative grids of {cus // 4}, {cus} and {2 * cus} workgroups x 256 threads, "
                     f"{2 * rounds} barriers each (a flag per block gathered by block 0, flags and checked data "
                     f"past the caches); {launches} back-to-back launches of an empty {cus}-workgroup kernel; "
                     f"best of {reps} after a warm-up, HIP events")
    return res


def library_gemm(torch, model, batch, frames, reps=5):
    """For scale: the vendor GEMM (torch.matmul, hipBLASLt on ROCm) on the
    GEMM shapes of the BigVGAN AMP convs of the batched step (rows = the
    stage's output rows over the batch, K = channels x taps, N = channels),
    with the input already expanded per tap (k times the bytes of the conv's
    input rows) and no epilogue.  HIP events, best of `reps` after a warm-up."""
    rows = batch * frames * int(np.prod(model["up_strides"]))
    out = []
    for si, rate in enumerate(model["rates"]):
        rows *= rate
        c = model["stage_channels"][si + 1]
        for k in model["res_kernels"]:
            for dt, name in ((torch.float16, "f16"), (torch.float32, "f32")):
                a = torch.randn(rows, c * k, device="cuda", dtype=dt)
                w = torch.randn(c * k, c, device="cuda", dtype=dt)
                y = torch.empty(rows, c, device="cuda", dtype=dt)
                torch.matmul(a, w, out=y)
                torch.cuda.synchronize()
                best = None
                for _ in range(reps):
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record()
                    torch.matmul(a, w, out=y)
                    e1.record()
                    torch.cuda.synchronize()
                    ms = e0.elapsed_time(e1)
                    best = ms if best is None else min(best, ms)
                out.append({"stage": si, "channels": c, "k": k, "rows": rows, "dtype": name, "ms": round(best, 4),
                            "tflops": round(2.0 * rows * c * k * c / best / 1e9, 1)})
                del a, w, y
                torch.cuda.empty_cache()
    return out


def warm_states(dec, codes, batch, torch):
    """Bring stream b to position batched_warmup_frames(b) (untimed)."""
    import synthetic as S

    warm = [S.batched_warmup_frames(b) for b in range(batch)]
    common = min(warm)
    st_a, st_b = dec.new_state(batch), dec.new_state(batch)
    sched = [1] + [25] * ((common - 1) // 25)
    t0 = 0
    for n in sched:
        c = torch.from_numpy(np.ascontiguousarray(codes[:, t0:t0 + n])).cuda()
        dec.decode(c, st_a, st_b)
        st_a, st_b = st_b, st_a
        t0 += n
    tmp = dec.new_state(1)
    for b in range(batch):
        tb = t0
        while tb < warm[b]:
            c = torch.from_numpy(np.ascontiguousarray(codes[b:b + 1, tb:tb + 25])).cuda()
            dec.decode(c, st_a[b:b + 1], tmp)
            st_a[b:b + 1].copy_(tmp)
            tb += 25
    torch.cuda.synchronize()
    return st_a, st_b, warm


def cpu_baseline(model, W, chunks, warm):
    """The float32 oracle on the host cores, on a bounded sample of the timed
    step: the 25-frame chunks of its first len(chunks) streams (the same codes
    the GPU decodes), each decoded from a fresh state rather than after its
    untimed warm-up (which sets only the attention window's fill and the
    conv histories; the convolutions are 99 % of the work either way)."""
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import decoder as O

    cores = len(os.sched_getaffinity(0))
    with threadpool_limits(limits=cores):
        used = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        Wf = O.cast_weights(W, np.float32)
        t0 = time.perf_counter()
        for c in chunks:
            O.decode_whole(model, Wf, c, dtype=np.float32)
        el = time.perf_counter() - t0
    frames = sum(c.shape[0] for c in chunks)
    audio = frames * FRAME_SECONDS
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), cpu)
    except OSError:
        pass
    return {"value": audio / el, "unit": "audio-s/s", "cores": int(used), "kind": "oracle", "cpu_model": cpu,
            "sample": f"the timed 25-frame chunks of streams 0-{len(chunks) - 1} of the 64-stream step "
                      f"({frames} frames, {audio:g} s of audio; the GPU decodes them after warm-ups to positions "
                      f"{', '.join(str(w) for w in warm[:len(chunks)])}, the oracle from fresh states), "
                      f"float32 numpy oracle, {el:.1f} s wall"}


def stream_latency(args, wl, torch, S, Decoder, vb):
    """Streaming latency: decode the workload's chunk schedule for its streams
    (warm-up passes untimed), timing every chunk call with HIP events on the
    caller's stream.  Prints one JSON line (not the headline metric)."""
    model = dict(wl["model"], precision=args.precision, weights=args.weights)
    sched = [wl["frames"]] if wl["schedule"] == "whole" else wl["schedule"]
    B = wl["batch"]
    W = S.make_weights(model, wl["weight_seed"])
    codes = S.workload_codes(args.workload)
    dec = Decoder(model, torch.from_numpy(S.flatten_weights(model, W)), B, max(sched))
    prefix = wl.get("prefix", 0)
    pre_chunks, t0 = [], 0
    while t0 < prefix:
        n = min(max(sched), prefix - t0)
        pre_chunks.append(torch.from_numpy(np.ascontiguousarray(codes[:, t0:t0 + n])).cuda())
        t0 += n
    chunks = []
    for n in sched:
        chunks.append(torch.from_numpy(np.ascontiguousarray(codes[:, t0:t0 + n])).cuda())
        t0 += n
    pcm = [torch.empty((B, n * dec.hop), device="cuda") for n in sched]
    states = (dec.new_state(B), dec.new_state(B))
    stream = torch.cuda.current_stream()
    times, host_times, pre_times, pre_dec_times = [], [], [], []

    def run_prefix(st_a, st_b, decode):
        # the reference prefix into the state: prefill (no audio), or, for
        # comparison, ordinary decode calls whose audio is discarded
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        ev[0].record(stream)
        for c in pre_chunks:
            if decode:
                dec.decode(c, st_a, st_b)
            else:
                dec.prefill(c, st_a, st_b)
            st_a, st_b = st_b, st_a
        ev[1].record(stream)
        torch.cuda.synchronize()
        return st_a, st_b, ev[0].elapsed_time(ev[1])

    for rep in range(args.warmup + args.steps):
        # the same buffers in the same roles every repetition: with --graph the
        # warm-up repetitions record one graph per chunk, the timed ones replay
        st_a, st_b = states
        dec.reset(st_a)
        if pre_chunks:
            _, _, ms = run_prefix(st_a, st_b, True)
            dec.reset(st_a)
            st_a, st_b, ms_pre = run_prefix(st_a, st_b, False)
            if rep >= args.warmup:
                pre_dec_times.append(ms)
                pre_times.append(ms_pre)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(sched) + 1)]
        host = []
        torch.cuda.synchronize()
        ev[0].record(stream)
        for i, n in enumerate(sched):
            h0 = time.perf_counter()
            dec.decode(chunks[i], st_a, st_b, pcm[i], graph=args.graph)
            host.append((time.perf_counter() - h0) * 1e3)
            st_a, st_b = st_b, st_a
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        if rep >= args.warmup:
            times.append([ev[i].elapsed_time(ev[i + 1]) for i in range(len(sched))])
            host_times.append(host)
    if dec.status() != vb.VOCODER_OK:
        raise SystemExit("device reported an error")
    kernels = None
    if args.profile_chunk:
        # one more eager pass, recording kernel events around the chosen chunks only
        st_a, st_b = states
        dec.reset(st_a)
        agg, calls = {}, 0
        for i, n in enumerate(sched):
            if n == args.profile_chunk:
                vb.vocoder_profile_begin(dec.handle)
            dec.decode(chunks[i], st_a, st_b, pcm[i])
            if n == args.profile_chunk:
                calls += 1
                for k, v in vb.vocoder_profile_end(dec.handle).items():
                    a = agg.setdefault(k, [0, 0.0])
                    a[0] += v["launches"]
                    a[1] += v["total_ms"]
            st_a, st_b = st_b, st_a
        torch.cuda.synchronize()
        if calls:
            kernels = {"chunk_frames": args.profile_chunk,
                       "sum_ms_per_call": round(sum(a[1] for a in agg.values()) / calls, 4),
                       "launches_per_call": sum(a[0] for a in agg.values()) / calls,
                       "by_kernel": {k: {"launches": a[0] / calls, "ms": round(a[1] / calls, 4)}
                                     for k, a in sorted(agg.items(), key=lambda kv: -kv[1][1])}}
    t = np.array(times)  # [reps][chunks] ms
    per_chunk = np.median(t, axis=0)
    total = t.sum(axis=1)
    audio = sum(sched) * FRAME_SECONDS * B
    out = {"metric": "streaming chunk latency (ms) and audio-seconds/sec", "workload": args.workload,
           "streams": B, "schedule": sched, "reps": args.steps, "graph": args.graph, "weights": args.weights,
           "first_chunk_ms": round(float(per_chunk[0]), 3),
           "chunk_ms_median_by_length": {str(n): round(float(np.median(t[:, [i for i, m in enumerate(sched) if m == n]])), 3)
                                         for n in sorted(set(sched))},
           "total_ms_median": round(float(np.median(total)), 3),
           # host time to enqueue one call (its launches), per chunk length: the
           # device times above hold while it stays below them
           "host_enqueue_ms_median_by_length": {
               str(n): round(float(np.median(np.array(host_times)[:, [i for i, m in enumerate(sched) if m == n]])), 3)
               for n in sorted(set(sched))},
           "audio_s_per_s": round(audio / (float(np.median(total)) / 1e3), 2),
           "dtype": DTYPES[args.precision], "data": "synthetic"}
    if pre_chunks:
        out["prefix_frames"] = prefix
        out["prefill_ms_median"] = round(float(np.median(pre_times)), 3)
        out["prefix_as_decode_ms_median"] = round(float(np.median(pre_dec_times)), 3)
    if kernels:
        out["kernels"] = kernels
    print(json.dumps(out), flush=True)


def roofline(name, k, ms, tflops, gbs, mfma_peak, peaks, precision):
    """Roofline of the dominant kernel family: its bound is the roof with the
    longer lower-bound time for the family's algorithmic work, its FLOPs at the
    MFMA peak against its algorithmic bytes at the HBM peak (the bound is
    "hbm" when the family's FLOPs per byte fall below the ridge point, peak
    FLOP/s over peak bytes/s); `achieved` and `frac` are that roof's, and the
    other roof's fraction is reported beside it.  (The split mode's MFMAs run
    three products per counted one, so its MFMA time is three times its FLOPs
    at the peak.)"""
    intensity = k["flops"] / k["bytes"] if k["bytes"] else float("inf")
    ridge = mfma_peak * 1e12 / (HBM_PEAK_GBS * 1e9)
    mfma_meas = peaks["mfma_f32_tflops" if precision == "f32" else "mfma_f16_tflops"]
    if intensity * (3 if precision == "split" else 1) < ridge:
        r = {"kernel": name, "bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
             "frac": round(gbs / HBM_PEAK_GBS, 4), "peak_measured": peaks["hbm_read_gbs"],
             "frac_of_measured": round(gbs / peaks["hbm_read_gbs"], 4),
             "mfma": {"achieved": round(tflops, 3), "peak": mfma_peak, "unit": "TFLOP/s",
                      "frac": round(tflops / mfma_peak, 4)}}
    else:
        r = {"kernel": name, "bound": "mfma", "achieved": round(tflops, 3), "peak": mfma_peak, "unit": "TFLOP/s",
             "frac": round(tflops / mfma_peak, 4), "peak_measured": mfma_meas,
             "frac_of_measured": round(tflops / mfma_meas, 4),
             "hbm": {"achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4)}}
    r.update({"flop_per_byte": round(intensity, 1), "ridge_flop_per_byte": round(ridge, 1),
              "avg_launch_ms": round(ms, 4), "traffic": traffic_for(name)})
    return r


def traffic_for(kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except Exception:
        return None
    src = os.path.join(ROOT, "vocoder_rvq_codebook_amd", "csrc", "conv_gemm.hip")
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    k = rec.get("kernels", {}).get(kernel)
    if not k or rec.get("conv_gemm_sha256") != sha:
        return None
    return k.get("hbm_bytes_per_launch")


def main():
    args = parse()
    if args.trace_summary:
        trace_summary(args.trace_summary, args.steps)
        return
    if args.traffic_summary:
        traffic_summary(*args.traffic_summary, copy_bytes=args.copy_bytes or (1 << 30))
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this decoder runs on one GPU: streams are independent and shard across GPUs "
                                   "with no collectives, but only the single-GPU path is built; run with --gpus 1"}))
        sys.exit(2)
    import torch

    import synthetic as S
    from vocoder_rvq_codebook_amd import Decoder, binding as vb

    if args.peaks_only:
        torch.cuda.set_device(0)
        print(json.dumps({"peaks_measured": measure_peaks(torch, vb)}), flush=True)
        return
    if args.library_gemm:
        torch.cuda.set_device(0)
        wl = S.workload(args.workload)
        for r in library_gemm(torch, wl["model"], wl["batch"], wl["frames"]):
            print(json.dumps({"library_gemm": r}), flush=True)
        return
    if args.barrier_probe:
        torch.cuda.set_device(0)
        print(json.dumps({"ordering_point": measure_barrier(torch, vb)}), flush=True)
        return

    if args.copy_bytes:
        src = torch.ones(args.copy_bytes // 4, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"copied {args.copy_bytes} bytes", flush=True)
        return

    wl = S.workload(args.workload)
    model = dict(wl["model"], precision=args.precision, weights=args.weights)
    peak = FP32_MFMA_PEAK_TFLOPS if args.precision == "f32" else FP16_MFMA_PEAK_TFLOPS
    if isinstance(wl["schedule"], list) or wl["schedule"] == "whole":
        stream_latency(args, wl, torch, S, Decoder, vb)
        return
    if wl["schedule"] != "warm_then_25":
        raise SystemExit("bench.py times the batched 25-frame workload or a chunk schedule")
    B, T = wl["batch"], wl["frames"]
    W = S.make_weights(model, wl["weight_seed"])
    codes = S.workload_codes(args.workload)
    torch.cuda.set_device(0)
    peaks = None if args.counters else measure_peaks(torch, vb)
    dec = Decoder(model, torch.from_numpy(S.flatten_weights(model, W)), B, T)
    if args.counters:
        st_a, st_b = dec.new_state(B), dec.new_state(B)
        dec.decode(torch.from_numpy(np.ascontiguousarray(codes[:, :T])).cuda(), st_a, st_b)
        torch.cuda.synchronize()
        print("decoded one batched step", flush=True)
        return
    st_a, st_b, warm = warm_states(dec, codes, B, torch)
    chunk = torch.from_numpy(np.stack([codes[b, warm[b]:warm[b] + T] for b in range(B)])).cuda()
    pcm = torch.empty((B, T * dec.hop), device="cuda")
    stream = torch.cuda.current_stream()

    for _ in range(args.warmup):
        dec.decode(chunk, st_a, st_b, pcm)
        st_a, st_b = st_b, st_a
    torch.cuda.synchronize()

    vb.vocoder_profile_begin(dec.handle)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    # an event after every call as well: per-call durations for the median and quartiles
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        dec.decode(chunk, st_a, st_b, pcm)
        st_a, st_b = st_b, st_a
        evs[i].record(stream)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    call_ms = np.array([ev0.elapsed_time(evs[0])] + [evs[i - 1].elapsed_time(evs[i]) for i in range(1, args.steps)])
    prof = vb.vocoder_profile_end(dec.handle)
    if dec.status() != vb.VOCODER_OK:
        raise SystemExit("device reported an error during the timed steps")
    gpu_s = ev0.elapsed_time(ev1) / 1e3
    elapsed = max(wall, gpu_s)
    audio_per_step = B * T * FRAME_SECONDS
    value = audio_per_step * args.steps / elapsed

    flops_step = sum(k["flops"] for k in prof.values()) / args.steps
    dom_name, dom = max(prof.items(), key=lambda kv: kv[1]["total_ms"])
    dom_ms = dom["total_ms"] / dom["launches"]
    dom_tflops = dom["flops"] / dom["launches"] / (dom_ms * 1e-3) / 1e12
    dom_gbs = dom["bytes"] / dom["launches"] / (dom_ms * 1e-3) / 1e9
    roof = roofline(dom_name, dom, dom_ms, dom_tflops, dom_gbs, peak, peaks, args.precision)
    kernels = {k: {"launches_per_step": v["launches"] / args.steps, "ms_per_step": v["total_ms"] / args.steps,
                   "tflops": (v["flops"] / (v["total_ms"] * 1e-3) / 1e12) if v["flops"] else None,
                   "gbs": v["bytes"] / (v["total_ms"] * 1e-3) / 1e9}
               for k, v in sorted(prof.items(), key=lambda kv: -kv[1]["total_ms"])}

    out = {
        "metric": {"f32": "audio-seconds/sec (\u00d7real-time) for 64\u00d725-frame chunks; % fp32 MFMA peak",
                   "f16": "audio-seconds/sec (\u00d7real-time) for 64\u00d725-frame chunks, fp16 operands; "
                          "% fp16 MFMA peak",
                   "split": "audio-seconds/sec (\u00d7real-time) for 64\u00d725-frame chunks, fp32 values on "
                            "split-fp16 MFMA (3 products per pair); % fp16 MFMA peak"}[args.precision],
        "value": round(value, 3),
        "unit": "audio-s/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 3),
        "call_ms": {"median": round(float(np.median(call_ms)), 3), "p25": round(float(np.percentile(call_ms, 25)), 3),
                    "p75": round(float(np.percentile(call_ms, 75)), 3)},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPES[args.precision],
        "data": "synthetic (seeded random-init weights, uniform random codes)",
        "config": {"workload": args.workload, "streams": B, "frames_per_chunk": T, "weights": args.weights,
                   "samples_per_frame": dec.hop, "warm_positions": sorted(set(warm))},
        "tflops": round(flops_step / (elapsed / args.steps) / 1e12, 3),
        "mfma_frac": round(flops_step / (elapsed / args.steps) / 1e12 / peak, 4),
        "roofline": roof,
        "peaks_measured": peaks,
        "kernels": kernels,
    }
    if args.precision == "f32" and args.weights == "float" and args.split_line:
        # the same workload with fp32-accurate products on the fp16 MFMA, timed
        # the same way in a child process (its own device memory); `value` above
        # stays the fp32 MFMA path's
        del dec, st_a, st_b, pcm, chunk
        torch.cuda.empty_cache()
        out["split16"] = split_line(args)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(model, W, [codes[b, warm[b]:warm[b] + T] for b in range(args.cpu_streams)],
                                           warm)
    print(json.dumps(out), flush=True)


def split_line(args):
    """Run `bench.py --precision split` on the same workload as a child process
    and keep the essentials of its JSON line."""
    import subprocess
    cmd = [sys.executable, os.path.abspath(__file__), "--precision", "split", "--workload", args.workload,
           "--steps", str(args.steps), "--warmup", str(args.warmup), "--no-cpu-baseline"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    if r.returncode != 0 or not lines:
        return {"error": f"exit {r.returncode}", "stderr": r.stderr[-500:]}
    d = json.loads(lines[-1])
    ro = d["roofline"]
    return {"what": "same workload, fp32 values with every matrix product as three fp16 MFMA products per pair "
                    "(meets the same float64-oracle bar; --precision split)",
            "value": d["value"], "unit": d["unit"], "ms_per_step": d["ms_per_step"], "dtype": d["dtype"],
            "roofline": {"kernel": ro["kernel"], "achieved": ro["achieved"], "peak": ro["peak"], "unit": ro["unit"],
                         "frac": ro["frac"], "traffic": ro["traffic"]}}


if __name__ == "__main__":
    main()
