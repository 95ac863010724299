"""Throughput of per-frame float_ssim at 3840x2160 on one MI355X.

One step = one pass of the whole scoring path (upload-free: decimate, SSIM
map, fixed-tree reduction, 8-byte result, one host wait per frame) over the
workload's 50 distinct device-resident frame pairs (1.66 GB, larger than the
256 MB last-level cache, so every frame comes from HBM).  The K timed steps
run as one continuous stream of 50*K frames through the C ABI's pipelined
loop (vqm_score_frames): batches of frames per launch, each frame collected
with one wait once `lag` later frames are submitted.

Prints one JSON line (see the keys below).  ``--workload`` picks another of
the five synthetic workloads; the default is the 2160p 10-bit float_ssim one.
"""

from __future__ import annotations

import argparse
import collections
import dataclasses
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0                    # MI355X HBM3E, GB/s
# The published fp32 vector peak: 256 CUs x 4 SIMD x 32 lane-FMAs per clock x
# 2 flops x 2.4 GHz.  The library's kernels use ordinary (non-packed) FMA
# instructions, and those reach it too: --valu-probe measures about 127
# TFLOP/s with plain v_fma_f32 chains at eight waves per SIMD, above the
# 78.6 that 16 lanes per clock would allow.
FP32_VALU_PEAK_TFLOPS = 256 * 4 * 32 * 2 * 2.4e9 / 1e12   # 157.3

# Kernel sources whose counters profiles/ssim_step_2160p10_traffic.json holds.
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "ssim_step_2160p10_traffic.json")
KERNEL_SOURCES = ["ssim_step.hip", "decimate_device.h", "ssim_common.h", "vqm_kernels.h"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def covered_extent(n: int, s: int) -> int:
    """Raw samples along one side that some decimation window reads."""
    dn = -(-n // s)
    return min(n, s * (dn - 1) + s - s // 2)


def algorithmic_bytes(wl, s: int) -> int:
    """Raw bytes the method must read once per frame pair (both planes)."""
    bps = 1 if wl.bpc == 8 else 2
    if wl.metric == "ms_ssim":
        return 2 * wl.w * wl.h * bps
    return 2 * covered_extent(wl.w, s) * covered_extent(wl.h, s) * bps


def kernel_sources_sha256() -> str:
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "full_reference_video_amd", "csrc", name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def recorded_traffic(workload_name: str, frames_per_launch: float):
    """HBM bytes per launch from the committed FETCH_SIZE/WRITE_SIZE record
    (taken on full launches), scaled to this run's average frames per launch
    like the algorithmic bytes; None when there is no record for this workload
    or the kernel sources changed since it was taken."""
    try:
        with open(TRAFFIC_RECORD) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("workload") != workload_name or rec.get("kernel_sources_sha256") != kernel_sources_sha256():
        return None
    per_launch = rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]
    return int(round(per_launch * frames_per_launch / rec["frames_per_launch"]))


def ms_flops_per_frame(w: int, h: int) -> float:
    """Algorithmic fp32 flops of one MS-SSIM frame: per level and per valid
    map pixel, the separable 11-tap moments (5 planes x 11 FMA horizontally
    and vertically = 220 flops) and the three products of its input sample
    (3), plus the l/c/s terms (20: two square roots, three reciprocals and
    the arithmetic around them, counted one each)."""
    total = 0.0
    lw, lh = w, h
    for _ in range(5):
        total += (lw - 10) * (lh - 10) * (220 + 3 + 20)
        lw, lh = lw // 2, lh // 2
    return total


def ssim_map_flops_per_frame(w: int, h: int, s: int) -> float:
    """Algorithmic fp32 flops of one float_ssim frame's SSIM map: per valid map
    pixel of the decimated plane, the separable 11-tap moments of the four
    planes the map needs (x, y, x^2 + y^2, xy: 4 x 11 FMA horizontally and
    vertically = 176 flops), the three products of its input sample (3) and
    the per-pixel term (20, the reciprocal counted once)."""
    dw, dh = -(-w // s), -(-h // s)
    return float((dw - 10) * (dh - 10) * (176 + 3 + 20))


def run_pass(ctxs, frameset, metric, batch, lag):
    """Score every frame pair of `frameset` once, as one continuous stream,
    through the C ABI's pipelined loop (batches rotate over the contexts; one
    wait per frame)."""
    from full_reference_video_amd import vqm
    m = vqm.VQM_METRIC_MS_SSIM if metric == "ms_ssim" else vqm.VQM_METRIC_FLOAT_SSIM
    return vqm.vqm_score_frames(ctxs, m, frameset, batch, lag).tolist()


def default_streams(metric: str, scale: int) -> int:
    """Contexts (each on its own stream) the timed stream rotates its batches
    over.  float_ssim with decimation: one; a second one overlapping
    consecutive launches measured slower (the steps contend for HBM and for
    the per-XCD layout: 2160p 164k -> 149k, 1080p 675k -> 634k, 853x481
    919k -> 843k frames/s).  The scale-1 map takes two: its launches' last
    tiles leave SIMDs idle, which the other context's batch fills (576x324
    1.03M -> 1.15M).  MS-SSIM takes one: a context on its own stream already
    alternates its batches over two streams, which fills the small levels'
    idle SIMDs the same way (2160p 19.8k -> 21.8k; two such contexts 21.3k)."""
    return 2 if scale == 1 and metric != "ms_ssim" else 1


def cpu_model() -> str:
    """The host CPU's model name, as /proc/cpuinfo gives it."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def cpu_baseline(host, wl, budget_s: float):
    """The oracle as it stands, one thread, over the workload's frames in order
    (cycling), until about ``budget_s`` seconds of oracle time are spent."""
    import oracle
    fn = oracle.msssim if wl.metric == "ms_ssim" else oracle.ssim
    n = 0
    t0 = time.perf_counter()
    while True:
        r, d = host[n % len(host)]
        fn(r, d, wl.bpc)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or n >= 40 * len(host):
            break
    return {"value": round(n / el, 3), "unit": "frames/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} frame pairs of {wl.name} (frames 0..{min(n, len(host)) - 1}, cycling), "
                      f"one thread, {el:.1f} s, {cpu_model()}"}


# Frames the all-cores baseline's worker processes read (inherited through
# fork, never pickled).
_ORACLE_TIMING_FRAMES = None


def _oracle_worker(args):
    """One process of the all-cores baseline: the unchanged oracle over
    frames i, i + P, ... (cycling) for about `budget_s` seconds."""
    metric, bpc, i, p, budget_s = args
    import oracle
    host = _ORACLE_TIMING_FRAMES
    fn = oracle.msssim if metric == "ms_ssim" else oracle.ssim
    n, k = 0, i
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        r, d = host[k % len(host)]
        fn(r, d, bpc)
        n += 1
        k += p
    return n, time.perf_counter() - t0


def cpu_baseline_all_cores(host, wl, budget_s: float, cores: int):
    """The same oracle, one single-threaded process per core, each on its own
    frames; frames/s summed over the processes.  Forks: call it before the
    GPU is touched."""
    import multiprocessing as mp
    global _ORACLE_TIMING_FRAMES
    _ORACLE_TIMING_FRAMES = host
    try:
        with mp.get_context("fork").Pool(cores) as pool:
            res = pool.map(_oracle_worker, [(wl.metric, wl.bpc, i, cores, budget_s) for i in range(cores)])
    finally:
        _ORACLE_TIMING_FRAMES = None
    n = sum(r[0] for r in res)
    el = max(r[1] for r in res)
    return {"value": round(n / el, 3), "unit": "frames/s", "cores": cores, "kind": "oracle",
            "sample": f"{n} frame pairs of {wl.name}, {cores} processes of the single-threaded oracle "
                      f"on disjoint frames, {el:.1f} s, {cpu_model()}"}


def copy_bandwidth(torch, mib: int = 1024, reps: int = 10) -> float:
    """Bytes read plus written per second by torch's device-to-device copy of
    `mib` MiB: a measured ceiling on this machine, reported beside the roofline's
    published peak."""
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    del src, dst
    return round(2.0 * n * reps / el / 1e9, 1)


def ss2_chain_work(w: int, h: int, nscales: int = 6, nch: int = 3):
    """Per frame: the recursions' fp32 operations (five planes per channel,
    a causal and an anticausal walk along every row and every column, 7
    rounded operations a step), the pixels of every scale, and the bytes the
    chain must move at the least (the two pictures' planes read once)."""
    ops, px, sw, sh = 0, 0, w, h
    for _ in range(nscales):
        n = sw * sh
        px += n
        ops += nch * 5 * n * 2 * 2 * 7
        sw, sh = (sw + 1) // 2, (sh + 1) // 2
    return ops, px, 2 * nch * 4 * w * h


def run_ss2_chain(args):
    import numpy as np
    import torch

    from full_reference_video_amd import synth, vqm
    sw, sh = (int(v) for v in args.ss2_chain.lower().split("x"))
    nscales, nch = 6, 3
    coef = vqm.vqm_ss2_cascade_coefficients(1.5)
    # distinct frames, more bytes than the 256 MB last-level cache
    sets = max(2, -(-(300 << 20) // (2 * nch * 4 * sw * sh)))
    host = [synth.ss2_images(20 + k, sw, sh, nch) for k in range(sets)]
    cpu = None
    if args.cpu_budget > 0:  # the oracle's chain, one thread, before the GPU is touched
        import oracle
        log("oracle timing on the host")
        ocoef = oracle.ss2_cascade_coefficients(1.5)
        n_cpu, t0 = 0, time.perf_counter()
        while True:
            oracle.ss2_chain(*host[n_cpu % sets], nscales, ocoef)
            n_cpu += 1
            el_cpu = time.perf_counter() - t0
            if el_cpu >= args.cpu_budget or n_cpu >= 40 * sets:
                break
        cpu = {"value": round(n_cpu / el_cpu, 4), "unit": "frames/s", "cores": 1, "kind": "oracle",
               "sample": f"{n_cpu} frames of the chain ({nch} channels of {sw}x{sh}, {nscales} scales), one thread, "
                         f"{el_cpu:.1f} s, {cpu_model()}"}
    frames = [([torch.from_numpy(p).cuda() for p in ref], [torch.from_numpy(p).cuda() for p in dis])
              for ref, dis in host]
    torch.cuda.synchronize()
    first = vqm.vqm_ss2_scale_sums(*frames[0], nscales, coef)
    for f in frames:
        vqm.vqm_ss2_scale_sums(*f, nscales, coef)  # warm-up (grows the workspace once)
    n = max(1, args.steps)
    callers = max(1, args.ss2_callers)

    pipelined = args.ss2_pipelined
    if pipelined and callers != 1:
        raise SystemExit("--ss2-pipelined is one caller's submit/collect loop: drop --ss2-callers")
    ctx = vqm.Context(0) if pipelined else None
    depth = args.ss2_depth or vqm.VQM_SS2_MAX_IN_FLIGHT
    if not 1 <= depth <= vqm.VQM_SS2_MAX_IN_FLIGHT:
        raise SystemExit(f"--ss2-depth outside 1..{vqm.VQM_SS2_MAX_IN_FLIGHT}")

    def caller(k, out):
        # ctypes releases the GIL for the call, so the callers' frames overlap on the GPU
        for i in range(k, n, callers):
            got = vqm.vqm_ss2_scale_sums(*frames[i % sets], nscales, coef)
            if i % sets == 0:
                out.append(got)

    def pipeline(out):
        # one caller, VQM_SS2_MAX_IN_FLIGHT frames in flight on one context
        order = collections.deque()
        for i in range(n):
            if ctx.vqm_ss2_in_flight() == depth:
                got = ctx.vqm_ss2_collect()
                if order.popleft() == 0:
                    out.append(got)
            ctx.vqm_ss2_submit(*frames[i % sets], nscales, coef)
            order.append(i % sets)
        while order:
            got = ctx.vqm_ss2_collect()
            if order.popleft() == 0:
                out.append(got)

    if pipelined:
        pipeline([])  # warm-up: every slot's workspace and stream

    runs = []
    for _ in range(max(1, args.reps)):
        outs = [[] for _ in range(callers)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        if pipelined:
            pipeline(outs[0])
        elif callers == 1:
            caller(0, outs[0])
        else:
            import threading
            th = [threading.Thread(target=caller, args=(k, outs[k])) for k in range(callers)]
            for x in th:
                x.start()
            for x in th:
                x.join()
        torch.cuda.synchronize()
        runs.append((time.perf_counter() - t0) / n)
        for o in outs:
            for got in o:
                if not np.array_equal(got, first):
                    raise RuntimeError("ssimulacra2 chain sums changed between calls")
    el = sorted(runs)[len(runs) // 2]
    ops, px, minbytes = ss2_chain_work(sw, sh, nscales, nch)
    if pipelined:
        how = f"one caller, {depth} frames in flight on one context"
        ctx.close()
    else:
        how = "one blocking call per frame" if callers == 1 else f"blocking calls from {callers} host threads"
    print(json.dumps({"metric": f"ssimulacra2 per-scale chain, {nch} channels of {sw}x{sh}, {nscales} scales, {how}",
                      "value": round(1.0 / el, 1), "unit": "frames/s", "ms_per_frame": round(el * 1e3, 4),
                      "recursion_ops_per_frame": ops, "recursion_Gops": round(ops / el / 1e9, 1),
                      "pixels_all_scales": px, "min_bytes_per_frame": minbytes,
                      "frames": sets, "reps": len(runs), "cpu_baseline": cpu}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--reps", type=int, default=7,
                    help="timed runs of K steps each; value is the median run's rate")
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", type=int, default=4, help="workload number 1..5")
    ap.add_argument("--streams", type=int, default=0,
                    help="contexts batches rotate over (0: the metric's best: 1, or 2 for float_ssim at scale 1)")
    ap.add_argument("--batch", type=int, default=32, help="frames per submit (and per kernel launch)")
    ap.add_argument("--ctx-streams", choices=("own", "torch"), default="own",
                    help="contexts on library-owned streams (default) or on torch streams")
    ap.add_argument("--lag", type=int, default=0,
                    help="frames submitted after a frame before it is collected (0: 3*batch)")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle timing (0: skip)")
    ap.add_argument("--cpu-cores", type=int, default=0,
                    help="processes of the all-cores oracle baseline (0: the host's CPUs, at most 16; -1: skip)")
    ap.add_argument("--host-input", choices=("none", "pinned", "pageable"), default="none",
                    help="score frames from host memory (pinned tensors or pageable arrays) instead of HBM: the "
                         "end-to-end rate with one upload per frame, reported under its own metric name")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of a recorded pass (vqm_graph_*) over the workload's device frames, one "
                         "replay and one wait per step, reported under its own metric name")
    ap.add_argument("--frame", default="", metavar="WxHxBPC",
                    help="score frames of this size and depth instead (the 2160p workload's recipe, 16 frames; for "
                         "sizes outside the workloads, e.g. 1280x720x8, 2560x1440x10 or 7680x4320x10)")
    ap.add_argument("--blocking", action="store_true",
                    help="score the stream one blocking call per frame (vqm_ssim_frame / vqm_msssim_frame on the "
                         "device frames: one submit, one wait, one 8-byte read-back each), reported under its own "
                         "metric name")
    ap.add_argument("--ss2", default="", metavar="WxH",
                    help="only time the ssimulacra2 per-scale statistics (vqm_ss2_channel_sums) of three channels of "
                         "WxH seeded planes, against the HBM roofline of its seven fp32 planes per channel, and exit")
    ap.add_argument("--ss2-chain", default="", metavar="WxH",
                    help="only time the ssimulacra2 per-scale chain (vqm_ss2_scale_sums: six scales of multiplies, "
                         "recursive blur, statistics and downsample) on three channels of WxH seeded planes, one "
                         "blocking call per frame, and exit")
    ap.add_argument("--ss2-pipelined", action="store_true",
                    help="with --ss2-chain: one caller submitting to one context and collecting in order")
    ap.add_argument("--ss2-depth", type=int, default=0, metavar="D",
                    help="with --ss2-pipelined: frames kept in flight (0: VQM_SS2_MAX_IN_FLIGHT)")
    ap.add_argument("--ss2-callers", type=int, default=1, metavar="N",
                    help="with --ss2-chain: N host threads each make the blocking calls, so N frames are in flight "
                         "on N pooled contexts (streams)")
    ap.add_argument("--valu-probe", type=int, default=0, metavar="ITERS",
                    help="time plain fp32 FMA chains (ITERS steps of 16 per lane) at 1-16 waves per SIMD and exit")
    ap.add_argument("--read-probe", type=int, default=0, metavar="MIB",
                    help="only time the library's streaming 16-byte non-temporal read over MIB MiB of device memory "
                         "(the HBM read ceiling of the decimation's loads) and exit")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run torch's device-to-device copy of MIB MiB 20 times (a kernel of known "
                         "traffic, to calibrate the FETCH_SIZE/WRITE_SIZE counters) and exit")
    args = ap.parse_args()

    if args.copy_probe:
        import torch
        n = args.copy_probe << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(20):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "launches": 20}), flush=True)
        return

    if args.ss2:
        import numpy as np
        import torch

        from full_reference_video_amd import synth, vqm
        sw, sh = (int(v) for v in args.ss2.lower().split("x"))
        # Distinct plane sets, more bytes than the 256 MB last-level cache.
        sets = max(2, -(-(300 << 20) // (3 * 7 * 4 * sw * sh)))
        host = synth.ss2_planes(11, sw, sh, 3)
        dev = []
        for k in range(sets):
            dev.append([[torch.from_numpy(p).cuda().add_(0.0) for p in ch] for ch in host])
        torch.cuda.synchronize()
        ref = vqm.vqm_ss2_channel_sums(dev[0])
        for d in dev:
            vqm.vqm_ss2_channel_sums(d)  # warm-up
        n = max(1, args.steps)
        runs = []
        for _ in range(max(1, args.reps)):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in range(n):
                got = vqm.vqm_ss2_channel_sums(dev[i % sets])
            torch.cuda.synchronize()
            runs.append((time.perf_counter() - t0) / n)
        if not np.array_equal(vqm.vqm_ss2_channel_sums(dev[0]), ref):
            raise RuntimeError("ssimulacra2 sums changed between calls")
        el = sorted(runs)[len(runs) // 2]
        alg = 3 * 7 * 4 * sw * sh
        gbps = alg / el / 1e9
        print(json.dumps({"metric": f"ssimulacra2 per-scale statistics, 3 channels of {sw}x{sh}, one blocking call",
                          "value": round(1.0 / el, 1), "unit": "calls/s", "us_per_call": round(el * 1e6, 2),
                          "algorithmic_bytes": alg, "GBps": round(gbps, 1),
                          "hbm_frac": round(gbps / HBM_PEAK_GBS, 4), "plane_sets": sets}), flush=True)
        return

    if args.ss2_chain:
        run_ss2_chain(args)
        return

    if args.valu_probe:
        from full_reference_video_amd import vqm
        for w in (1, 2, 4, 8, 16):
            t = vqm.vqm_debug_valu_probe(waves_per_simd=w, iters=args.valu_probe, reps=5)
            print(json.dumps({"valu_probe_waves_per_simd": w, "iters": args.valu_probe, "TFLOPs": round(t, 1),
                              "frac_of_peak": round(t / FP32_VALU_PEAK_TFLOPS, 4)}), flush=True)
        return

    if args.read_probe:
        import torch

        from full_reference_video_amd import vqm
        n = args.read_probe << 20
        buf = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        torch.cuda.synchronize()
        ms = vqm.vqm_debug_read_probe(buf, reps=20)
        gbps = n / (ms * 1e-3) / 1e9
        print(json.dumps({"read_probe_bytes": n, "kernel_ms": round(ms, 4), "GBps": round(gbps, 1),
                          "frac_of_peak": round(gbps / HBM_PEAK_GBS, 4)}), flush=True)
        return

    if args.gpus != 1:
        print(f"bench.py: this build scores on one GPU; --gpus {args.gpus} is not supported "
              "(frames shard across GPUs with no collective; see the design notes)", file=sys.stderr)
        sys.exit(2)

    import numpy as np

    from full_reference_video_amd import synth

    wl = synth.WORKLOADS[args.workload]
    src = synth.FrameSource(args.workload)
    if args.frame:
        fw, fh, fb = (int(v) for v in args.frame.lower().split("x"))
        base = synth.WORKLOADS[4] if wl.metric == "float_ssim" else wl
        wl = dataclasses.replace(base, name=f"{base.metric}_{fw}x{fh}_{fb}bit", w=fw, h=fh, bpc=fb, frames=16)
        src = synth.FrameSource(base.index, w=fw, h=fh, bpc=fb)
    log(f"generating {wl.frames} frame pairs of {wl.name}")
    host = [src.pair(t) for t in range(wl.frames)]

    # The oracle baselines run first, before anything touches the GPU (the
    # all-cores one forks worker processes).
    cpu = cpu_all = None
    if args.cpu_budget > 0:
        log("oracle timing on the host")
        cpu = cpu_baseline(host, wl, args.cpu_budget)
        if args.cpu_cores >= 0:
            cores = args.cpu_cores or min(16, len(os.sched_getaffinity(0)))
            log(f"oracle timing on {cores} host processes")
            cpu_all = cpu_baseline_all_cores(host, wl, args.cpu_budget, cores)

    import torch

    from full_reference_video_amd import vqm

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    s = vqm.vqm_ssim_scale(wl.w, wl.h) if wl.metric == "float_ssim" else 1
    dev = []
    for r, d in host:
        tr = torch.from_numpy(r.view(np.int16) if r.dtype == np.uint16 else r)
        td = torch.from_numpy(d.view(np.int16) if d.dtype == np.uint16 else d)
        if args.host_input == "none":
            tr, td = tr.cuda(), td.cuda()
        elif args.host_input == "pinned":
            tr, td = tr.pin_memory(), td.pin_memory()
        else:
            tr, td = r, d
        dev.append((tr, td))
    torch.cuda.synchronize()

    if args.streams <= 0:
        args.streams = default_streams(wl.metric, s)
    streams = [torch.cuda.Stream() for _ in range(args.streams)]
    # Contexts on library-owned streams by default: such a context alternates
    # its MS-SSIM batches over two streams of its own (on a caller's stream
    # every batch stays there); float_ssim measures the same on either.
    ctxs = [vqm.Context(0, st) if args.ctx_streams == "torch" else vqm.Context(0) for st in streams]
    lag = args.lag if args.lag > 0 else 3 * args.batch
    # The timed run streams the workload's frames K times over without a
    # break, as a video is scored (the pipeline fills once and drains once).
    stream_set_r = [r for _ in range(args.steps) for r, _ in dev]
    stream_set_d = [d for _ in range(args.steps) for _, d in dev]
    stream_set = vqm.FrameSet(stream_set_r, stream_set_d, wl.bpc)

    # Each warm-up pass streams the workload's frames, repeated to at least
    # twice the in-flight limit: a context's in-flight slots allocate their
    # buffers on first use, and the timed stream must find them all ready.
    reps = max(1, -(-2 * vqm.VQM_MAX_IN_FLIGHT // wl.frames))
    warm_set = vqm.FrameSet([r for _ in range(reps) for r, _ in dev],
                            [d for _ in range(reps) for _, d in dev], wl.bpc)
    log(f"warmup {args.warmup} passes of {reps * wl.frames} frames")
    ref_scores = None
    for _ in range(args.warmup):
        sc = run_pass(ctxs, warm_set, wl.metric, args.batch, lag)
        if ref_scores is None:
            ref_scores = sc[:wl.frames]
        if sc != ref_scores * reps:
            raise RuntimeError("scores changed between passes")
    torch.cuda.synchronize()

    frames = args.steps * wl.frames
    runs = []
    if args.graph:
        if args.host_input != "none":
            raise SystemExit("--graph replays device-resident frames only")
        # One recorded pass over the workload's frames; a step is one replay
        # and its one wait.
        graph = vqm.Graph(0, streams[0], vqm.VQM_METRIC_MS_SSIM if wl.metric == "ms_ssim"
                          else vqm.VQM_METRIC_FLOAT_SSIM, vqm.FrameSet([r for r, _ in dev], [d for _, d in dev],
                                                                        wl.bpc), args.batch)
        for _ in range(max(1, args.warmup)):
            graph.vqm_graph_launch()
            got = graph.vqm_graph_collect().tolist()
            if ref_scores is None:
                ref_scores = got
            elif got != ref_scores:
                raise RuntimeError("a replay differs from the eager pass")
        log(f"timed {args.reps} x {args.steps} graph replays over {wl.frames} frames, batch {args.batch}")
        for _ in range(args.reps):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(args.steps):
                graph.vqm_graph_launch()
                sc = graph.vqm_graph_collect()
            torch.cuda.synchronize()
            runs.append(time.perf_counter() - t0)
            if sc.tolist() != ref_scores:
                raise RuntimeError("a replay differs from the eager pass")
        graph.close()
    elif args.blocking:
        fn = vqm.vqm_msssim_frame if wl.metric == "ms_ssim" else vqm.vqm_ssim_frame
        # the blocking calls' pooled context allocates its slot on first use
        for r, d in dev:
            fn(r, d, wl.bpc)
        log(f"timed {args.reps} x {args.steps} passes over {wl.frames} frames, one blocking call per frame")
        for _ in range(args.reps):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            sc = [fn(r, d, wl.bpc) for r, d in zip(stream_set_r, stream_set_d)]
            torch.cuda.synchronize()
            runs.append(time.perf_counter() - t0)
            if ref_scores is not None and sc != ref_scores * args.steps:
                raise RuntimeError("scores changed between passes")
    else:
        log(f"timed {args.reps} x {args.steps} passes over {wl.frames} frames, batch {args.batch}, "
            f"{args.streams} streams, lag {lag}")
        for _ in range(args.reps):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            sc = run_pass(ctxs, stream_set, wl.metric, args.batch, lag)
            torch.cuda.synchronize()
            runs.append(time.perf_counter() - t0)
            if ref_scores is not None and sc != ref_scores * args.steps:
                raise RuntimeError("scores changed between passes")
    el = sorted(runs)[len(runs) // 2]  # the median run
    fps = frames / el
    marginal_us = None
    if not args.graph and not args.blocking and frames > 2:
        # The pages' per-frame figure, (t(N) - t(2)) / (N - 2): the same
        # stream over its first two frames, timed as often, takes out the
        # pipeline's fill and drain and the loop's start.
        two = vqm.FrameSet([stream_set_r[0], stream_set_r[1]], [stream_set_d[0], stream_set_d[1]], wl.bpc)
        t2 = []
        for _ in range(args.reps):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            run_pass(ctxs, two, wl.metric, args.batch, lag)
            torch.cuda.synchronize()
            t2.append(time.perf_counter() - t0)
        marginal_us = round(1e6 * (el - sorted(t2)[len(t2) // 2]) / (frames - 2), 3)

    # Per-kernel durations from HIP events on the launch stream, in a pass on
    # one context: with several, concurrent batches share the GPU and each
    # launch's own duration would no longer be one kernel's.
    log("kernel timing pass")
    tctx = ctxs[:1]
    for c in tctx:
        c.vqm_ctx_set_timing(True)
    run_pass(tctx, stream_set, wl.metric, args.batch, lag)
    kt = {}
    for cls, name in ((vqm.VQM_KERNEL_SSIM_STEP, "ssim_step"), (vqm.VQM_KERNEL_SSIM_DRAIN, "ssim_drain"),
                      (vqm.VQM_KERNEL_MSSSIM_LEVEL1, "ms_level1"),
                      (vqm.VQM_KERNEL_MSSSIM_COARSE, "ms_levels2_5")):
        ms = n = nf = 0
        for c in tctx:
            a, b, fr = c.vqm_ctx_kernel_time(cls)
            ms += a
            n += b
            nf += fr
        if n:
            kt[name] = {"avg_us": 1000.0 * ms / n, "launches": n, "frames_per_launch": nf / n}
    for c in tctx:
        c.vqm_ctx_set_timing(False)
    # After the kernel timing: a burst of copies changes the clocks that a
    # compute-bound kernel timed right after it would see.
    copy_gbps = copy_bandwidth(torch)

    alg = algorithmic_bytes(wl, s)
    if wl.metric == "float_ssim":
        # The step kernel streams the raw samples (HBM) and computes the SSIM
        # map (VALU).  Both rooflines are computed; the one the kernel comes
        # closer to binds (HBM at 2160p, the map's VALU work at the smaller
        # frames, where there is little to decimate) and the other is listed
        # under "other".
        name = "ssim_step" if "ssim_step" in kt else "ssim_drain"
        per_launch = alg * kt[name]["frames_per_launch"]
        avg_s = kt[name]["avg_us"] * 1e-6
        achieved = per_launch / avg_s / 1e9
        hbm = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
               "frac": round(achieved / HBM_PEAK_GBS, 4),
               "traffic": recorded_traffic(wl.name, kt[name]["frames_per_launch"]),
               "kernel": "ssim_step", "bytes_per_launch": int(per_launch)}
        map_flops = ssim_map_flops_per_frame(wl.w, wl.h, s) * kt[name]["frames_per_launch"]
        alu_tflops = map_flops / avg_s / 1e12
        alu = {"bound": "alu", "achieved": round(alu_tflops, 2), "peak": round(FP32_VALU_PEAK_TFLOPS, 1),
               "unit": "TFLOP/s", "frac": round(alu_tflops / FP32_VALU_PEAK_TFLOPS, 4), "traffic": hbm["traffic"],
               "kernel": "ssim_step", "flops_per_launch": int(map_flops)}
        roof, other = (hbm, alu) if hbm["frac"] >= alu["frac"] else (alu, hbm)
        roof["other"] = {k: other[k] for k in ("bound", "achieved", "peak", "unit", "frac")}
    else:
        # MS-SSIM is VALU-bound; every level kernel counts, with its share of
        # the frame's algorithmic flops.
        ms = sum(kt[k]["avg_us"] * kt[k]["launches"] for k in ("ms_level1", "ms_levels2_5") if k in kt)
        frames_timed = kt["ms_level1"]["launches"] * kt["ms_level1"]["frames_per_launch"]
        flops = ms_flops_per_frame(wl.w, wl.h) * frames_timed
        achieved = flops / (ms * 1e-6) / 1e12
        roof = {"bound": "alu", "achieved": round(achieved, 2), "peak": round(FP32_VALU_PEAK_TFLOPS, 1),
                "unit": "TFLOP/s", "frac": round(achieved / FP32_VALU_PEAK_TFLOPS, 4), "traffic": None,
                "kernel": "ms_level (all five levels)",
                "flops_per_frame": ms_flops_per_frame(wl.w, wl.h)}


    out = {
        "metric": ("frames/sec and achieved HBM GB/s (% of peak), float_ssim at 3840x2160"
                   if wl.index == 4 and not args.frame else f"frames/sec, {wl.name}")
                  + ("" if args.host_input == "none" else f", end to end from {args.host_input} host frames")
                  + (", recorded-pass replays" if args.graph else "")
                  + (", one blocking call per frame" if args.blocking else ""),
        "value": round(fps, 1),
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(1000.0 * el / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "input": "hbm" if args.host_input == "none" else args.host_input + " host",
                   "w": wl.w, "h": wl.h, "bpc": wl.bpc, "frames_per_step": wl.frames,
                   "scale": s, "batch": args.batch, "streams": args.streams, "lag": lag,
                   "mode": "graph replay" if args.graph else ("blocking calls" if args.blocking else "stream"),
                   "path_GBps": round(alg * fps / 1e9, 1)},
        "runs": {"n": len(runs), "frames_per_s_min": round(frames / max(runs), 1),
                 "frames_per_s_max": round(frames / min(runs), 1),
                 "us_per_frame": round(1e6 * el / frames, 3), "us_per_frame_marginal": marginal_us},
        "copy_GBps": copy_gbps,
        "kernels": kt,
        "roofline": roof,
        "cpu_baseline": cpu,
        "cpu_baseline_all_cores": cpu_all,
    }
    print(json.dumps(out), flush=True)
    for c in ctxs:
        c.close()


if __name__ == "__main__":
    main()
