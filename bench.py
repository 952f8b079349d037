"""Benchmark of the block-quantized matmul hot path on one MI355X.

Headline workload (one "step"): the matrix-vector regime -- Q4_K, Q6_K and Q8_0 weights of
4096 x 4096, each times N = 1, 2, 5 and 8 columns of N(0,1) fp32 activations, i.e. 12 calls of
quantize-to-q8_1 + matmul.  value = effective GB/s of the whole step:
    algorithmic bytes = weight blocks + q8_1 activation blocks + fp32 outputs, per call,
divided by the step time.  Weights rotate over several distinct copies (> 512 MB in all) so the
256 MB Infinity Cache cannot serve them; the cache-warm rate is reported separately.

Also in the same JSON line:
  roofline      for the dominant kernel (the matrix-vector kernel): per case, the weights rotate over
                copies totalling > 512 MB, a HIP graph holds one launch per copy, and every replay
                is timed by HIP events on the launch stream (median / p10 / p90 per launch);
                peak = 8 TB/s HBM.  probe: the loads-only streaming read (libqmm_probe) of the same
                rotated weight bytes, and at the 66 MB fused gate/up decode size; frac_of_probe =
                probe time / kernel time.  traffic comes from the committed rocprofv3
                FETCH_SIZE/WRITE_SIZE summary when it matches the current kernel sources.
  cpu_baseline  the oracle (plain C, all host threads) on whole steps of the same workload; the
                host CPU model; one-thread figures on the small dense workload and one step.
  f16act_matvec  per-call timing (encoder + kernel) of the fp16-activation mode on the step's shapes
  extra_types_matvec  per-launch timing of the same matrix-vector shapes in Q5_K, Q4_0, Q3_K and IQ4_XS (not
                part of the step).
  panel_layout  the step's shapes read from the panel layout (qmm_repack / qmm_matmul_packed), and
                the repack's first-call versus steady-state cost at 8192 x 4096 Q4_K, one column.
  secondary     for the prefill and MoE shapes and the gate/up products fused with SwiGLU: per-call
                median / p10 / p90, int8 TOPS as a fraction of the 5.0 POP/s datasheet peak and of
                the int8 MFMA probe, % of roofline (max of bytes / 8 TB/s and ops / 5 POP/s over
                the time); weights rotated over > 512 MB, MoE also with resident weights (warm).

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu] [--no-secondary]
       python bench.py --secondary-only [--calib-copy]   only the prefill / MoE shapes (profiling)

Profile summaries (no GPU; read the SQLite databases rocprofv3 writes under -d DIR):
  python bench.py --summarize-trace DIR          per-kernel durations of a --kernel-trace run
  python bench.py --summarize-counters DIR       per-kernel, per-launch-shape averages of the
                 counters of a --pmc run, with rocprofv3's derived MfmaUtil and VALUBusy and the
                 int8 MFMA ops (MOPS_I8 * 512)
  python bench.py --summarize-pmc FDIR WDIR [--write-traffic]
                 per-kernel FETCH_SIZE / WRITE_SIZE of two --pmc runs of `bench.py --calib-copy`,
                 scaled to bytes by the 256 MiB device copy (tiled and grouping kernels get one
                 line per launch shape); --write-traffic stores the matrix-vector kernels'
                 average in profiles/mmvq_traffic.json (with a hash of the kernel sources, so
                 the figure is dropped once they change).
"""
import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
INT8_PEAK_TOPS = 5000.0
STEP_ROWS = 4096   # weight rows of every matrix-vector call of the step (synth.MMVQ_CASES)


# Sources of the matrix-vector kernels themselves: a change to any of them drops the stored counter
# traffic; changes elsewhere (tiled kernels, planner, shared headers of declarations) do not
# change those kernels' memory traffic.
MV_SOURCES = ["q8_1.hpp", "mv_cols.hpp", "mmvq.hip", "mmvq_stream.hip", "mmvq_dot4.hip"]


def probe_lib():
    """The measurement probes (include/qmm_probe.h), loaded after torch like libqmm."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "block_quantized_matmul_quantize_amd", "libqmm_probe.so"))
    lib.qmm_probe_read.restype = ctypes.c_int
    lib.qmm_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                   ctypes.c_void_p]
    lib.qmm_probe_mfma_i8.restype = ctypes.c_int
    lib.qmm_probe_mfma_i8.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    return lib


PROBE_WGS, PROBE_THREADS = 2048, 256   # the read probe's launch shape (the fastest of those measured)


def pct(vals, q):
    import numpy as np
    return round(float(np.percentile(np.asarray(vals), q)), 3)


def source_hash():
    h = hashlib.sha256()
    for name in MV_SOURCES:
        with open(os.path.join(ROOT, "block_quantized_matmul_quantize_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algo_bytes(qtype, rows, k, n, block_bytes, block_values):
    """Bytes one call must move: weight blocks + q8_1 activation blocks + fp32 outputs."""
    return rows * (k // block_values[qtype]) * block_bytes[qtype] + n * (k // 32) * 36 + n * rows * 4


def launch_bytes(qtype, rows, k, n, block_bytes, block_values, fp32_in):
    """Bytes one matrix-vector launch must move: as algo_bytes, with fp32 activations (4 B per
    value) in place of q8_1 blocks when the kernel quantizes its input itself."""
    if not fp32_in:
        return algo_bytes(qtype, rows, k, n, block_bytes, block_values)
    return rows * (k // block_values[qtype]) * block_bytes[qtype] + n * k * 4 + n * rows * 4


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--rotations", type=int, default=4)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--secondary-only", action="store_true",
                    help="time only the prefill and MoE shapes (for profiling them); prints their JSON")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run one 256 MiB device copy (known bytes) to scale profiler counters")
    ap.add_argument("--summarize-trace", metavar="DIR")
    ap.add_argument("--summarize-counters", metavar="DIR")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--write-traffic", action="store_true")
    ap.add_argument("--cpu-single", action="store_true", help=argparse.SUPPRESS)
    args = ap.parse_args()
    if args.cpu_single:
        cpu_single_thread()
        return
    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters)
        return
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc, write=args.write_traffic)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the sharded "
              "design is described in DESIGN.md, not built)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import block_quantized_matmul_quantize_amd as qmm
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calib_copy:
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    BB, BV = qmm.BLOCK_BYTES, qmm.BLOCK_VALUES
    cases = synth.MMVQ_CASES
    log = lambda *a: print(*a, file=sys.stderr, flush=True)
    if args.secondary_only:
        print(json.dumps({"secondary": run_secondary(torch, np, qmm, synth, dev, log)}), flush=True)
        return

    # ---------------------------------------------------------------- inputs (resident in HBM)
    R = max(1, args.rotations)
    W = [[None] * len(cases) for _ in range(R)]
    X, XQ, Y = [], [], []
    for i, c in enumerate(cases):
        for r in range(R):
            g = synth.rngs(1000 * r + i, 1)[0]
            W[r][i] = torch.from_numpy(synth.gen_weights(c["qtype"], c["rows"], c["k"], g)).to(dev)
        x = torch.from_numpy(synth.gen_activations(c["n"], c["k"], synth.rngs(7 + i, 1)[0])).to(dev)
        X.append(x)
        XQ.append(qmm.quantize_q8_1(x))
        Y.append(torch.empty((c["n"], c["rows"]), dtype=torch.float32, device=dev))
    WS = [qmm._workspace(qmm.matmul_workspace(c["qtype"], c["rows"], c["k"], c["n"]), dev) for c in cases]
    step_bytes = sum(algo_bytes(c["qtype"], c["rows"], c["k"], c["n"], BB, BV) for c in cases)
    weight_total = sum(w.numel() for row in W for w in row)
    log(f"[bench] {len(cases)} calls per step, {step_bytes / 1e6:.1f} MB algorithmic per step, "
        f"{R} weight rotations ({weight_total / 1e6:.0f} MB of weights)")

    def step(r):
        for i, c in enumerate(cases):
            qmm.matmul(W[r][i], c["qtype"], c["rows"], c["k"], X[i], out=Y[i], ws=WS[i])

    def capture(fn):
        """One HIP graph of fn() (kernel launches only; every buffer is preallocated)."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        torch.cuda.synchronize()
        return g

    # One graph per weight rotation: a step is 12 x (quantize + matmul) = 24 kernels, replayed
    # without host launch overhead (the eager rate is reported as well).
    graphs = [capture(lambda r=r: step(r)) for r in range(R)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)

    def run(nsteps, fn):
        torch.cuda.synchronize()
        t0.record()
        for s in range(nsteps):
            fn(s)
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / nsteps

    # ---------------------------------------------------------------- timed region
    for s in range(args.warmup):
        graphs[s % R].replay()
    wall0 = time.perf_counter()
    ms_per_step = run(args.steps, lambda s: graphs[s % R].replay())
    wall = time.perf_counter() - wall0
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    log(f"[bench] timed {args.steps} steps (graph replay): {ms_per_step:.4f} ms/step, {value:.1f} GB/s "
        f"(wall {wall:.2f} s)")
    eager_ms = run(args.steps, lambda s: step(s % R))
    eager_gbps = step_bytes / (eager_ms * 1e-3) / 1e9
    log(f"[bench] eager launches: {eager_ms:.4f} ms/step, {eager_gbps:.1f} GB/s")
    # cache-warm rate (same weights every step), reported separately
    warm_ms = run(args.steps, lambda s: graphs[0].replay())
    warm_gbps = step_bytes / (warm_ms * 1e-3) / 1e9

    # ---------------------------------------------------------------- per-launch kernel timing
    # The matrix-vector kernel as the step launches it.  qmm.matvec_kernel names it per case and
    # says whether it quantizes the fp32 input itself: then qmm.matmul is exactly one launch of it
    # (reading fp32 activations); otherwise qmm.matmul_q8_1 on the pre-quantized activations is
    # one launch of it (the step adds one quantize launch).  Per case, the weights rotate over
    # copies totalling > 512 MB (whole rows rolled on the device), a HIP graph holds one launch per
    # copy back to back, and each of `reps` replays is timed by two HIP events on the stream the
    # graph runs on: duration per launch = replay time / copies; median, p10 and p90 over replays.
    # The loads-only probe (libqmm_probe) reads the same rotated weight bytes in the same way.
    plib = probe_lib()
    sink = torch.zeros(1 << 16, dtype=torch.int32, device=dev)

    def replay_samples(g, per, reps):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        g.replay()
        torch.cuda.synchronize()
        for a, b in ev:
            a.record()
            g.replay()
            b.record()
        torch.cuda.synchronize()
        return [a.elapsed_time(b) * 1e3 / per for a, b in ev]

    def rotations(w0, row_bytes, target=600e6):
        n = max(2, int(np.ceil(target / w0.numel())))
        flat = w0.reshape(-1)
        return [torch.roll(flat, r * row_bytes) for r in range(n)]

    def probe_us(bufs, reps):
        def launch():
            st = torch.cuda.current_stream().cuda_stream
            for wb in bufs:
                assert plib.qmm_probe_read(wb.data_ptr(), wb.numel(), sink.data_ptr(), PROBE_WGS, PROBE_THREADS, st) == 0
        return replay_samples(capture(launch), len(bufs), reps)

    per_case = []
    tot_bytes = tot_us = tot_probe_us = 0.0
    reps = max(20, args.steps)
    for i, c in enumerate(cases):
        kid, fused = qmm.matvec_kernel(c["qtype"], W[0][i], c["rows"], c["k"], X[i], c["n"], x_fp32=True)
        rot = rotations(W[0][i], (c["k"] // BV[c["qtype"]]) * BB[c["qtype"]])
        if fused:
            call = lambda r, i=i, c=c: qmm.matmul(rot[r], c["qtype"], c["rows"], c["k"], X[i], out=Y[i], ws=WS[i])
        else:
            call = lambda r, i=i, c=c: qmm.matmul_q8_1(rot[r], c["qtype"], c["rows"], c["k"], XQ[i], c["n"],
                                                       out=Y[i])
        g = capture(lambda: [call(r) for r in range(len(rot))])
        smp = replay_samples(g, len(rot), reps)
        us = pct(smp, 50)
        pus = pct(probe_us(rot, reps), 50)
        b = launch_bytes(c["qtype"], c["rows"], c["k"], c["n"], BB, BV, fused)
        wb = rot[0].numel()
        per_case.append({"case": c["name"], "kernel": qmm.MV_KERNEL_NAMES.get(kid, "?") + (" (fp32 in)" if fused else ""),
                         "us": us, "us_p10": pct(smp, 10), "us_p90": pct(smp, 90), "bytes": b,
                         "GBps": round(b / us / 1e3, 1), "frac": round(b / us / 1e3 / HBM_PEAK_GBPS, 4),
                         "probe_us": pus, "probe_GBps": round(wb / pus / 1e3, 1),
                         "frac_of_probe": round(pus / us, 4), "weight_copies": len(rot)})
        tot_bytes += b
        tot_us += us
        tot_probe_us += pus
        del g, rot
    achieved = tot_bytes / tot_us / 1e3
    for pc in per_case:
        log(f"[bench]   {pc['case']:24s} {pc['kernel']:30s} {pc['us']:8.3f} us (p10 {pc['us_p10']:.3f} p90 "
            f"{pc['us_p90']:.3f})  {pc['GBps']:8.1f} GB/s; loads-only probe {pc['probe_us']:.3f} us")
    # the probe at the fused gate/up decode size: two Q4_K 14336 x 4096 matrices (66 MB)
    big = torch.zeros(2 * 14336 * 16 * 144, dtype=torch.uint8, device=dev)
    big_rot = rotations(big, 16 * 144)
    probe_66 = pct(probe_us(big_rot, max(10, reps // 4)), 50)
    del big, big_rot
    probe = {"kernel": "qmm_probe_read (streaming 16-byte loads, %d x %d threads)" % (PROBE_WGS, PROBE_THREADS),
             "avg_launch_us": round(tot_probe_us / len(cases), 3),
             "GBps_at_step_sizes": round(sum(pc["probe_GBps"] * pc["probe_us"] for pc in per_case) / tot_probe_us, 1),
             "us_66MB": probe_66, "GBps_66MB": round(2 * 14336 * 16 * 144 / probe_66 / 1e3, 1)}
    log(f"[bench] loads-only probe: {probe}")

    # Q5_K and Q4_0, types beyond the headline workload: the same per-launch timing (not in the step)
    q5_cases = []
    for i, c in enumerate(synth.EXTRA_MMVQ_CASES):
        w5 = rotations(torch.from_numpy(synth.gen_weights(c["qtype"], c["rows"], c["k"], synth.rngs(3000 + i, 1)[0])).to(dev),
                       (c["k"] // BV[c["qtype"]]) * BB[c["qtype"]])
        x5 = torch.from_numpy(synth.gen_activations(c["n"], c["k"], synth.rngs(70 + i, 1)[0])).to(dev)
        y5 = torch.empty((c["n"], c["rows"]), dtype=torch.float32, device=dev)
        ws5 = qmm._workspace(qmm.matmul_workspace(c["qtype"], c["rows"], c["k"], c["n"]), dev)
        kid, fused = qmm.matvec_kernel(c["qtype"], w5[0], c["rows"], c["k"], x5, c["n"], x_fp32=True)
        g = capture(lambda: [qmm.matmul(w5[r], c["qtype"], c["rows"], c["k"], x5, out=y5, ws=ws5)
                             for r in range(len(w5))])
        us = pct(replay_samples(g, len(w5), max(10, reps // 4)), 50)
        b = launch_bytes(c["qtype"], c["rows"], c["k"], c["n"], BB, BV, fused)
        # one call = one launch where the kernel quantizes x itself, else quantize + kernel
        q5_cases.append({"case": c["name"], "launches_per_call": 1 if fused else 2,
                         "kernel": qmm.MV_KERNEL_NAMES.get(kid, "?") + (" (fp32 in)" if fused else ""),
                         "us": round(us, 3), "GBps": round(b / us / 1e3, 1), "frac": round(b / us / 1e3 / HBM_PEAK_GBPS, 4)})
        log(f"[bench]   {c['name']:24s} {q5_cases[-1]['kernel']:30s} {us:8.3f} us  {b / us / 1e3:8.1f} GB/s")
        del w5

    # fp16-activation mode (encoder + wave-per-row kernel: two launches per call) on the step's shapes
    f16_cases = []
    for i, c in enumerate(synth.MMVQ_CASES):
        wf = rotations(torch.from_numpy(synth.gen_weights(c["qtype"], c["rows"], c["k"], synth.rngs(5000 + i, 1)[0])).to(dev),
                       (c["k"] // BV[c["qtype"]]) * BB[c["qtype"]])
        xf = torch.from_numpy(synth.gen_activations(c["n"], c["k"], synth.rngs(90 + i, 1)[0])).to(dev)
        yf = torch.empty((c["n"], c["rows"]), dtype=torch.float32, device=dev)
        wsf = qmm._workspace(qmm.matmul_f16act_workspace(c["k"], c["n"]), dev)
        g = capture(lambda: [qmm.matmul_f16act(wf[r], c["qtype"], c["rows"], c["k"], xf, out=yf, ws=wsf)
                             for r in range(len(wf))])
        us = pct(replay_samples(g, len(wf), max(10, reps // 4)), 50)
        b = launch_bytes(c["qtype"], c["rows"], c["k"], c["n"], BB, BV, True)
        f16_cases.append({"case": c["name"], "launches_per_call": 2, "us": round(us, 3),
                          "GBps": round(b / us / 1e3, 1), "frac": round(b / us / 1e3 / HBM_PEAK_GBPS, 4)})
        log(f"[bench]   f16act {c['name']:24s} {us:8.3f} us  {b / us / 1e3:8.1f} GB/s")
        del wf

    # Panel layout (one-time repack, qmm_repack): the step's shapes from panels, timed like the
    # per-case figures above (weights rotated by whole row groups over > 512 MB, graph-replayed),
    # and the first-call versus steady-state cost at 8192 x 4096 Q4_K, one column.
    panel_cases = []
    for i, c in enumerate(cases):
        wp0 = qmm.repack(W[0][i], c["qtype"], c["rows"], c["k"])
        rotp = rotations(wp0, wp0.numel() // ((c["rows"] + 15) // 16))
        wsp = qmm._workspace(qmm.matmul_packed_workspace(c["qtype"], c["rows"], c["k"], c["n"]), dev)
        g = capture(lambda: [qmm.matmul_packed(rotp[r], c["qtype"], c["rows"], c["k"], X[i], out=Y[i], ws=wsp)
                             for r in range(len(rotp))])
        us = pct(replay_samples(g, len(rotp), max(10, reps // 4)), 50)
        b = launch_bytes(c["qtype"], c["rows"], c["k"], c["n"], BB, BV, True)
        panel_cases.append({"case": c["name"], "us": round(us, 3), "GBps": round(b / us / 1e3, 1),
                            "frac": round(b / us / 1e3 / HBM_PEAK_GBPS, 4), "original_layout_us": per_case[i]["us"]})
        log(f"[bench]   panels {c['name']:24s} {us:8.3f} us  {b / us / 1e3:8.1f} GB/s "
            f"(original layout {per_case[i]['us']:.3f} us)")
        del g, rotp, wp0
    fc = dict(qtype=qmm.Q4_K, rows=8192, k=4096, n=1)
    wfc = rotations(torch.from_numpy(synth.gen_weights(fc["qtype"], fc["rows"], fc["k"], synth.rngs(6000, 1)[0])).to(dev),
                    (fc["k"] // 256) * 144)
    xfc = torch.from_numpy(synth.gen_activations(1, fc["k"], synth.rngs(6001, 1)[0])).to(dev)
    yfc = torch.empty((1, fc["rows"]), dtype=torch.float32, device=dev)
    nbp = qmm.repack_bytes(fc["qtype"], fc["rows"], fc["k"])
    wpfc = [torch.empty(nbp, dtype=torch.uint8, device=dev) for _ in wfc]
    wsfc = qmm._workspace(qmm.matmul_workspace(fc["qtype"], fc["rows"], fc["k"], 1), dev)
    wspfc = qmm._workspace(qmm.matmul_packed_workspace(fc["qtype"], fc["rows"], fc["k"], 1), dev)
    rep = lambda r: qmm.repack(wfc[r], fc["qtype"], fc["rows"], fc["k"], out=wpfc[r])
    prod = lambda r: qmm.matmul_packed(wpfc[r], fc["qtype"], fc["rows"], fc["k"], xfc, out=yfc, ws=wspfc)
    nfc = len(wfc)
    t_rep = pct(replay_samples(capture(lambda: [rep(r) for r in range(nfc)]), nfc, 10), 50)
    t_first = pct(replay_samples(capture(lambda: [(rep(r), prod(r)) for r in range(nfc)]), nfc, 10), 50)
    t_steady = pct(replay_samples(capture(lambda: [prod(r) for r in range(nfc)]), nfc, 10), 50)
    t_orig = pct(replay_samples(capture(lambda: [qmm.matmul(wfc[r], fc["qtype"], fc["rows"], fc["k"], xfc, out=yfc,
                                                            ws=wsfc) for r in range(nfc)]), nfc, 10), 50)
    first_call = {"case": "q4_K 8192x4096 N=1", "repack_us": round(t_rep, 3), "first_call_us": round(t_first, 3),
                  "steady_us": round(t_steady, 3), "original_layout_us": round(t_orig, 3),
                  "repacked_bytes": nbp, "original_bytes": wfc[0].numel()}
    log(f"[bench] panel layout first call vs steady state: {first_call}")
    del wfc, wpfc
    panel_layout = {"matvec": panel_cases, "first_call": first_call}

    traffic = None
    tpath = os.path.join(ROOT, "profiles", "mmvq_traffic.json")
    if os.path.exists(tpath):
        with open(tpath) as f:
            tj = json.load(f)
        if tj.get("source_hash") == source_hash():
            traffic = tj.get("bytes_per_launch_avg")

    roofline = {"kernel": "matrix-vector kernels as the step launches them (mmvq_dot4_kernel, "
                          "mmvq_stream_kernel), 12 cases", "bound": "hbm",
                "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                "algorithmic_bytes_per_launch_avg": round(tot_bytes / len(cases), 1),
                "avg_launch_us": round(tot_us / len(cases), 3),
                "probe": probe, "frac_of_probe": round(tot_probe_us / tot_us, 4), "per_case": per_case}

    # ---------------------------------------------------------------- secondary: prefill / MoE
    secondary = None
    if not args.no_secondary:
        secondary = run_secondary(torch, np, qmm, synth, dev, log)

    # ---------------------------------------------------------------- CPU baseline (oracle)
    cpu = None
    if not args.no_cpu:
        cpu = run_cpu_baseline(np, synth, cases, BB, BV, args.cpu_seconds, log)

    out = {
        "metric": "Q4_K x q8_1 qmatmul effective GB/s (N<=8) & int8 TOPS (prefill/MoE), % roofline",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int8 (q8_1 x Q4_K/Q6_K/Q8_0 codes), fp32 fixups", "data": "synthetic",
        "config": {"workload": "matrix-vector regime: Q4_K, Q6_K, Q8_0 4096x4096 x N in {1,2,5,8} "
                               "N(0,1) fp32 activations (12 quantize+matmul calls per step, replayed "
                               "as one HIP graph per weight rotation)",
                   "weight_rotations": R, "algorithmic_bytes_per_step": step_bytes},
        "warm_cache_GBps": round(warm_gbps, 1),
        "eager_launch_GBps": round(eager_gbps, 1),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "secondary": secondary,
        "extra_types_matvec": q5_cases,
        "panel_layout": panel_layout,
        "f16act_matvec": f16_cases,
    }
    print(json.dumps(out), flush=True)


# -------------------------------------------------------------------- profile summaries (host only)
COPY_BYTES = 256 << 20   # the --calib-copy device copy


def _rocpd(d):
    import sqlite3
    dbs = sorted(glob.glob(os.path.join(d, "**", "*.db"), recursive=True))
    if not dbs:
        raise SystemExit(f"no rocprofv3 database under {d}")
    return sqlite3.connect(dbs[0])


def _short(name):
    import re
    name = name.replace("(anonymous namespace)::", "")
    return re.sub(r"^void ", "", name.split("(")[0])


def summarize_trace(d):
    import statistics
    con = _rocpd(d)
    by = {}
    for name, start, end in con.execute("select name, start, end from kernels"):
        by.setdefault(_short(name), []).append((end - start) / 1000.0)
    print(f"{'kernel':66s} {'count':>6s} {'avg_us':>9s} {'med_us':>9s} {'min_us':>9s} {'max_us':>9s} {'total_ms':>9s}")
    for n, ds in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        print(f"{n[:66]:66s} {len(ds):6d} {sum(ds) / len(ds):9.3f} {statistics.median(ds):9.3f} "
              f"{min(ds):9.3f} {max(ds):9.3f} {sum(ds) / 1e3:9.3f}")


def summarize_counters(d, cus=256, simds=1024, xcds=8, clock_ghz=2.4):
    """Per kernel and launch shape: the average of each counter over the dispatches, and rocprofv3's
    derived metrics MfmaUtil = sum(SQ_VALU_MFMA_BUSY_CYCLES) / (max(GRBM_GUI_ACTIVE) * SIMDs) and
    VALUBusy = sum(SQ_ACTIVE_INST_VALU) / CUs / max(GRBM_GUI_ACTIVE).  The database holds counters
    summed over their instances; GRBM_GUI_ACTIVE is counted once per XCD, so its max over the 8 XCDs
    (all busy for the whole dispatch) is the stored sum / 8."""
    import statistics
    con = _rocpd(d)
    rows = con.execute("select kernel_name, grid_size, counter_name, value from counters_collection").fetchall()
    by = {}
    for name, grid, cname, value in rows:
        by.setdefault((_short(name), grid), {}).setdefault(cname, []).append(value)
    names = sorted({c for v in by.values() for c in v})
    print("| kernel | grid (threads) | dispatches | " + " | ".join(names) +
          " | busy us | MfmaUtil | VALUBusy | int8 ops |")
    print("|---|---|---|" + "---|" * len(names) + "---|---|---|---|")
    for (k, grid), cs in sorted(by.items()):
        avg = {c: statistics.mean(v) for c, v in cs.items()}
        disp = max(len(v) for v in cs.values())
        gui = avg.get("GRBM_GUI_ACTIVE", 0) / xcds
        mfma = avg["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui * simds) if gui and "SQ_VALU_MFMA_BUSY_CYCLES" in avg else None
        valu = avg["SQ_ACTIVE_INST_VALU"] / cus / gui if gui and "SQ_ACTIVE_INST_VALU" in avg else None
        ops = avg.get("SQ_INSTS_VALU_MFMA_MOPS_I8", 0) * 512
        fmt = lambda v: "-" if v is None else f"{100 * v:.1f} %"
        busy = f"{gui / (clock_ghz * 1e3):.1f}" if gui else "-"
        print(f"| `{k[:60]}` | {grid} | {disp} | " + " | ".join(f"{avg.get(c, 0):.4g}" for c in names) +
              f" | {busy} | {fmt(mfma)} | {fmt(valu)} | {ops:.4g} |")


def summarize_pmc(fdir, wdir, write=False):
    import re
    import statistics

    def load(d):
        by = {}
        for name, value in _rocpd(d).execute("select kernel_name, value from counters_collection"):
            by.setdefault(_short(name), []).append(value)
        return by

    def by_grid(d):
        out = {}
        for name, value, grid, wg in _rocpd(d).execute(
                "select kernel_name, value, grid_size, workgroup_size from counters_collection"):
            out.setdefault((_short(name), grid, wg), []).append(value)
        return out

    F, Wr = load(fdir), load(wdir)
    copy = [k for k in F if "copyBuffer" in k or "copy" in k.lower()]
    if not copy:
        raise SystemExit("no device-copy dispatch found: run bench.py with --calib-copy")
    fs = COPY_BYTES / (max(max(F[k]) for k in copy) * 1024)
    ws = COPY_BYTES / (max(max(Wr[k]) for k in copy if k in Wr) * 1024)
    print(f"calibration: {COPY_BYTES >> 20} MiB device copy -> FETCH_SIZE x{fs:.3f}, WRITE_SIZE x{ws:.3f}")
    print("| kernel | dispatches | FETCH_SIZE KiB/dispatch (raw) | WRITE_SIZE KiB/dispatch (raw) | HBM bytes/dispatch (scaled) |")
    print("|---|---|---|---|---|")
    for k in sorted(F, key=lambda k: -statistics.mean(F[k])):
        f = statistics.mean(F[k])
        w = statistics.mean(Wr.get(k, [0.0]))
        b = f * 1024 * fs + w * 1024 * ws
        print(f"| `{k}` | {len(F[k])} | {f:.1f} | {w:.1f} | {b / 1e6:.3f} MB |")
    FG, WG = by_grid(fdir), by_grid(wdir)
    # The step's launches: the headline types (8, 12, 14) in the forms the step takes (fp32 input,
    # no fusion, original layout) at its 4096 rows, i.e. 256 workgroups of 16 rows (dot4 picks its
    # workgroup size per launch, so the workgroup count, not the grid, identifies the shape); not
    # the extra types, the fp16-activation mode, the panel layout or the larger-row comparisons.
    step_kernel = re.compile(r"^qmm::mmvq_(stream_kernel<(8|12|14), false, false, true, false, false>"
                             r"|dot4_kernel<(8|12|14), \d, false, false, true, false>)$")
    # Each case of a type runs the same number of launches, so a kernel's share of its type's
    # dispatches counts the cases it served; the figure is the mean over the step's cases, as the
    # algorithmic bytes per launch are.
    groups = {}
    for (k, grid, wg), fv in FG.items():
        m = step_kernel.match(k)
        if m and wg and grid // wg == STEP_ROWS // 16:
            b = statistics.mean(fv) * 1024 * fs + statistics.mean(WG.get((k, grid, wg), [0.0])) * 1024 * ws
            groups[k] = (int(m.group(2) or m.group(3)), len(fv), b)
    import synth
    ncases = {t: sum(c["qtype"] == t for c in synth.MMVQ_CASES) for t in {c["qtype"] for c in synth.MMVQ_CASES}}
    per_type = {}
    for t, cnt, _ in groups.values():
        per_type[t] = per_type.get(t, 0) + cnt
    mv_tot = mv_cnt = 0.0
    for t, cnt, b in groups.values():
        cases = ncases[t] * cnt / per_type[t]
        mv_tot += b * cases
        mv_cnt += cases
    # tiled and grouping kernels: one line per launch shape (grid size), as the shapes differ
    tiled = sorted(k for k in FG if "mmq" in k[0] or "moe_group" in k[0] or "fixup" in k[0])
    if tiled:
        print()
        print("| kernel | grid (threads) | dispatches | HBM bytes/dispatch fetched | written |")
        print("|---|---|---|---|---|")
        for k in tiled:
            f = statistics.mean(FG[k]) * 1024 * fs
            w = statistics.mean(WG.get(k, [0.0])) * 1024 * ws
            print(f"| `{k[0]}` | {k[1]} | {len(FG[k])} | {f / 1e6:.1f} MB | {w / 1e6:.1f} MB |")
    if not mv_cnt:
        if write:
            raise SystemExit("no matrix-vector kernel dispatches in the counter runs")
        return
    avg = mv_tot / mv_cnt
    print(f"matrix-vector kernels of the step: {sum(g[1] for g in groups.values())} dispatches, "
          f"{mv_cnt:.0f} cases, mean over the cases of HBM bytes per launch {avg / 1e6:.3f} MB")
    if write:
        with open(os.path.join(ROOT, "profiles", "mmvq_traffic.json"), "w") as f:
            json.dump({"kernel": "matrix-vector kernels as the step launches them (12 cases)",
                       "bytes_per_launch_avg": round(avg), "fetch_scale": fs, "write_scale": ws,
                       "source_hash": source_hash(),
                       "command": "rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) -- python3 bench.py --no-cpu "
                                  "--no-secondary --calib-copy --steps 20 --warmup 2"}, f, indent=1)
            f.write("\n")


def mfma_probe_tops(torch, dev, log):
    """Attainable int8 matrix-core rate: the MFMA probe on 4 / 8 / 16 waves per compute unit, best of
    the three (TOPS)."""
    plib = probe_lib()
    sink = torch.zeros(16, dtype=torch.int32, device=dev)
    ncu = torch.cuda.get_device_properties(dev).multi_processor_count
    best = 0.0
    iters = 2000
    for wpc in (4, 8, 16):
        wgs = ncu * wpc // 4
        st = torch.cuda.current_stream().cuda_stream
        assert plib.qmm_probe_mfma_i8(iters, wgs, sink.data_ptr(), st) == 0
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(3):
            assert plib.qmm_probe_mfma_i8(iters, wgs, sink.data_ptr(), st) == 0
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / 3
        tops = 2.0 * 32 * 32 * 32 * 4 * iters * wgs * 4 / us / 1e6
        best = max(best, tops)
    log(f"[bench] int8 MFMA probe: {best:.1f} TOPS")
    return best


def run_secondary(torch, np, qmm, synth, dev, log):
    """Prefill and MoE shapes: int8 TOPS = 2*rows*k*columns / call time, as a fraction of the 5.0
    POP/s datasheet peak and of the MFMA probe; % of roofline = max(bytes / 8 TB/s, ops / 5 POP/s) /
    time with bytes = weights + q8_1 activations + fp32 outputs.  Each call is timed by two HIP
    events (median, p10, p90 over the calls); weights rotate over copies totalling > 512 MB so
    the 256 MB Infinity Cache cannot hold them (the MoE shapes also with one resident copy,
    labelled warm)."""
    res = []
    mfma_tops = mfma_probe_tops(torch, dev, log)

    def timed(fn, ncopies, calls):
        # every rotated weight copy is touched before timing (first touches of a fresh buffer run
        # ~10 % slower), so the timed calls see weights streamed from HBM at steady state
        for r in range(ncopies):
            fn(r)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
        for r, (a, b) in enumerate(ev):
            a.record()
            fn(r)
            b.record()
        torch.cuda.synchronize()
        return [a.elapsed_time(b) * 1e3 for a, b in ev]   # us

    def entry(name, smp, ops, nbytes, **extra):
        us = pct(smp, 50)
        tops = ops / us / 1e6
        roof = max(nbytes / (HBM_PEAK_GBPS * 1e3), ops / (INT8_PEAK_TOPS * 1e6)) / us
        e = {"case": name, "us": us, "us_p10": pct(smp, 10), "us_p90": pct(smp, 90), "TOPS": round(tops, 1),
             "frac_int8_peak": round(tops / INT8_PEAK_TOPS, 4), "frac_of_mfma_probe": round(tops / mfma_tops, 4),
             "frac_roofline": round(roof, 4), "bytes": int(nbytes)}
        e.update(extra)
        log(f"[bench] {name:40s} {us:9.1f} us {tops:8.1f} TOPS  {100 * roof:5.1f} % of roofline "
            f"{' '.join(f'{k}={v}' for k, v in extra.items())}")
        res.append(e)

    def copies(w, target=600e6):
        n = max(1, int(np.ceil(target / w.nbytes)))
        base = torch.from_numpy(w).to(dev).reshape(-1)
        rb = w.shape[-1] if w.ndim == 2 else 1
        return [torch.roll(base, r * rb) for r in range(n)]

    for c in synth.PREFILL_CASES + synth.EXTRA_PREFILL_CASES:
        w, x = synth.make_dense(c)
        ws_ = copies(w)
        xd = torch.from_numpy(x).to(dev)
        y = torch.empty((c["n"], c["rows"]), dtype=torch.float32, device=dev)
        wsb = qmm._workspace(qmm.matmul_workspace(c["qtype"], c["rows"], c["k"], c["n"]), dev)
        smp = timed(lambda r: qmm.matmul(ws_[r % len(ws_)], c["qtype"], c["rows"], c["k"], xd, out=y, ws=wsb),
                    len(ws_), max(20, 2 * len(ws_)))
        ops = 2.0 * c["rows"] * c["k"] * c["n"]
        nbytes = w.nbytes + c["n"] * (c["k"] // 32) * 36 + c["n"] * c["rows"] * 4
        entry(c["name"], smp, ops, nbytes, weight_copies=len(ws_))
        del ws_
    for c in synth.MOE_CASES[:3]:
        w, x, ids = synth.make_moe(c)
        xd, idd = torch.from_numpy(x).to(dev), torch.from_numpy(ids).to(dev)
        out = torch.empty((c["n_tok"], c["top_k"], c["rows"]), dtype=torch.float32, device=dev)
        wsb = qmm._workspace(qmm.matmul_id_workspace(c["qtype"], c["n_exp"], c["rows"], c["k"], c["n_tok"],
                                                     c["top_k"], c["x_per_tok"]), dev)
        ops = 2.0 * c["rows"] * c["k"] * c["n_tok"] * c["top_k"]
        nx = c["n_tok"] * c["x_per_tok"]
        nbytes = w.nbytes + nx * (c["k"] // 32) * 36 + c["n_tok"] * c["top_k"] * c["rows"] * 4
        for cache in ("cold", "warm"):
            wd = copies(w) if cache == "cold" else [torch.from_numpy(w).to(dev).reshape(-1)]
            smp = timed(lambda r: qmm.matmul_id(wd[r % len(wd)], c["qtype"], c["n_exp"], c["rows"], c["k"], xd, idd,
                                                x_per_tok=c["x_per_tok"], out=out, ws=wsb), max(8, len(wd)),
                        max(20, 2 * len(wd)))
            entry(c["name"], smp, ops, nbytes, cache="weights rotated over %d copies (%.0f MB)" % (
                len(wd), len(wd) * w.nbytes / 1e6) if cache == "cold" else "weights resident (warm)")
            del wd
    # gate/up products fused with SwiGLU (one call for both matrices)
    for c in synth.GLU_CASES:
        wg, wu, x, ids = synth.make_glu(c)
        xd = torch.from_numpy(x).to(dev)
        if c["kind"] == "dense":
            gs, us_ = copies(wg, 300e6), copies(wu, 300e6)
            nrot = len(gs)
            y = torch.empty((c["n"], c["rows"]), dtype=torch.float32, device=dev)
            wsb = qmm._workspace(qmm.matmul_glu_workspace(c["qtype"], c["rows"], c["k"], c["n"]), dev)
            smp = timed(lambda r: qmm.matmul_glu(gs[r % nrot], us_[r % nrot], c["qtype"], c["rows"], c["k"], xd,
                                                 out=y, ws=wsb), nrot, max(20, 2 * nrot))
            cols = c["n"]
            del gs, us_
            extra = {}
            if c["n"] <= 8:
                gbs = 2.0 * wg.nbytes / pct(smp, 50) / 1e3
                extra = {"GBps_weights": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBPS, 4)}
            nbytes = 2 * wg.nbytes + cols * (c["k"] // 32) * 36 + cols * c["rows"] * 4
        else:
            wgd, wud = torch.from_numpy(wg).to(dev), torch.from_numpy(wu).to(dev)
            idd = torch.from_numpy(ids).to(dev)
            out = torch.empty((c["n_tok"], c["top_k"], c["rows"]), dtype=torch.float32, device=dev)
            wsb = qmm._workspace(qmm.matmul_id_glu_workspace(c["qtype"], c["n_exp"], c["rows"], c["k"], c["n_tok"],
                                                             c["top_k"]), dev)
            smp = timed(lambda r: qmm.matmul_id_glu(wgd, wud, c["qtype"], c["n_exp"], c["rows"], c["k"], xd, idd,
                                                    out=out, ws=wsb), 8, 20)
            cols = c["n_tok"] * c["top_k"]
            del wgd, wud
            extra = {"cache": "weights resident (warm)"}
            nbytes = 2 * wg.nbytes + c["n_tok"] * (c["k"] // 32) * 36 + cols * c["rows"] * 4
        entry(c["name"], smp, 2.0 * 2 * c["rows"] * c["k"] * cols, nbytes, **extra)
    return {"mfma_probe_TOPS": round(mfma_tops, 1), "cases": res}


def run_cpu_baseline(np, synth, cases, BB, BV, seconds, log):
    import oracle
    data = []
    for i, c in enumerate(cases):
        g = synth.rngs(1000 * 0 + i, 1)[0]
        w = synth.gen_weights(c["qtype"], c["rows"], c["k"], g)
        x = synth.gen_activations(c["n"], c["k"], synth.rngs(7 + i, 1)[0])
        data.append((c, w, x))
    step_bytes = sum(algo_bytes(c["qtype"], c["rows"], c["k"], c["n"], BB, BV) for c in cases)
    t0 = time.perf_counter()
    nsteps = 0
    while True:
        for c, w, x in data:
            oracle.matmul(c["qtype"], w, c["rows"], c["k"], x)
        nsteps += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    gbps = step_bytes * nsteps / dt / 1e9
    log(f"[bench] cpu oracle: {nsteps} steps in {dt:.2f} s -> {gbps:.3f} GB/s on {cores} threads")
    # one thread, in a child process (the OpenMP thread count is fixed when the oracle loads)
    import subprocess
    single = None
    r = subprocess.run([sys.executable, os.path.abspath(__file__), "--cpu-single"], capture_output=True, text=True,
                       env=dict(os.environ, OMP_NUM_THREADS="1"), timeout=600)
    if r.returncode == 0 and r.stdout.strip():
        single = json.loads(r.stdout.strip().splitlines()[-1])
        log(f"[bench] cpu oracle, one thread: {single}")
    return {"value": round(gbps, 3), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"{nsteps} whole steps of the same 12-call workload ({dt:.1f} s), weights from rotation 0",
            "ms_per_step": round(dt / nsteps * 1e3, 2), "cpu_model": cpu_model(), "host_threads": os.cpu_count(),
            "single_thread": single}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_single_thread():
    """The oracle on one thread (OMP_NUM_THREADS=1 set by the parent): the small dense workload
    (Q4_K 512 x 1024 x 16 tokens) and one whole matrix-vector step (the 12 calls); ms and GB/s."""
    import numpy as np  # noqa: F401
    import oracle
    import synth
    BB = {2: 18, 8: 34, 12: 144, 13: 176, 14: 210}
    BV = {2: 32, 8: 32, 12: 256, 13: 256, 14: 256}
    c = synth.DENSE_SMALL
    w, x = synth.make_dense(c)
    t0 = time.perf_counter()
    reps = 20
    for _ in range(reps):
        oracle.matmul(c["qtype"], w, c["rows"], c["k"], x)
    small_ms = (time.perf_counter() - t0) * 1e3 / reps
    small_b = algo_bytes(c["qtype"], c["rows"], c["k"], c["n"], BB, BV)
    data = []
    for i, cc in enumerate(synth.MMVQ_CASES):
        data.append((cc, synth.gen_weights(cc["qtype"], cc["rows"], cc["k"], synth.rngs(i, 1)[0]),
                     synth.gen_activations(cc["n"], cc["k"], synth.rngs(7 + i, 1)[0])))
    t0 = time.perf_counter()
    for cc, ww, xx in data:
        oracle.matmul(cc["qtype"], ww, cc["rows"], cc["k"], xx)
    step_ms = (time.perf_counter() - t0) * 1e3
    step_b = sum(algo_bytes(cc["qtype"], cc["rows"], cc["k"], cc["n"], BB, BV) for cc, _, _ in data)
    print(json.dumps({"threads": 1, "dense_small_ms": round(small_ms, 3),
                      "dense_small_GBps": round(small_b / small_ms / 1e6, 4),
                      "matvec_step_ms": round(step_ms, 1), "matvec_step_GBps": round(step_b / step_ms / 1e6, 4)}))


if __name__ == "__main__":
    main()
