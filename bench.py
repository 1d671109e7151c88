"""Benchmark of the direct sliding-window correlation hot path on one MI355X.

Headline (``value``): u8 normalized correlation of a 1920x1080 image with a
64x64 template cut from it (valid-mode output 1857x1017, all four outputs:
SumI, SumISq, SumIT and the coefficient), in nominal Gdot4/s:
3 * (t_width/4) * t_height packed-byte dot products per output, through the
packed-byte (DP4A-style) kernel the method describes.  One step is one
ncc_u8_run_variant(..., XC_NCC_DOT4_ILP) call on that image with inputs
resident in HBM.  The other kernel variants (the page's ablation points and
the matrix-core recast, which ncc_u8_run picks for this template) are timed
on the same workload under "ncc_variants"; every variant returns identical
outputs.

The generalizations (best-match search, a 63 x 63 template) are timed on the
same image under "ncc_ext"; one-to-one pairs of 512 and 1024 rows under
"xcorr_large".

The fp32 cross-correlation form is timed in the same run (its own loops,
reported under "xcorr"): one-to-one 256x256, one-to-many 1x64 of 64x64 and
n-to-m 8x16 of 32x32, in GFLOP/s counted as 2*rows^2*cols^2 per pair.

Kernel durations come from two HIP events recorded on the stream the kernels
run on, around the back-to-back launches of the timed region.  The CPU oracle is timed on a
bounded sample of the same workload on this host ("cpu_baseline").

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "u8 NCC Gdot4/s & fp32 xcorr GFLOP/s, % of gfx950 peak, 1 GPU"

# MI355X figures (spec sheet): 256 CUs at 2.4 GHz, 64 lanes per CU per clock.
CUS, CLOCK_HZ, LANES = 256, 2.4e9, 64
DOT4_PEAK = CUS * LANES * CLOCK_HZ  # one v_dot4_u32_u8 per lane per clock: 39.32 T/s
FP32_PEAK = 157.3e12                # spec FP32 vector peak (2 FMA per lane per clock)
I8_MFMA_PEAK = 5.0e15               # spec dense int8 matrix-core peak (ops/s)

PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "cross_correlation_amd", "csrc")


def source_digest(names) -> str:
    """First 16 hex digits of the sha256 of the named kernel sources, in order."""
    import hashlib
    h = hashlib.sha256()
    for name in ([names] if isinstance(names, str) else names):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def profiled_traffic(profile: str, source):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or None
    when the kernel source changed since the counters were taken."""
    path = os.path.join(PROFILES, profile)
    if not os.path.exists(path):
        return None
    fig = {}
    with open(path) as f:
        for line in f:
            if line.startswith("figure "):
                k, v = line[len("figure "):].split("=", 1)
                fig[k.strip()] = v.strip()
    if fig.get("source_sha256_16") != source_digest(source):
        return None
    return int(fig["hbm_bytes_per_launch"])


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target length of the CPU sample")
    ap.add_argument("--only", choices=["ncc", "xcorr", "all"], default="all")
    ap.add_argument("--json-out", default=None)
    ap.add_argument("--no-peak-probe", action="store_true", help="skip the measured issue-rate ceilings")
    ap.add_argument("--no-ext", action="store_true",
                    help="skip the ncc_ext timings (profiling runs: each kernel then sees one workload)")
    ap.add_argument("--trial-ms", type=float, default=100.0,
                    help="minimum length of each timed trial of the headline and the workloads (ms)")
    ap.add_argument("--trials", type=int, default=5, help="timed trials per workload (the median is reported)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB (a known-size kernel that "
                         "calibrates the FETCH_SIZE / WRITE_SIZE counters), then exit")
    return ap.parse_args()


def copy_probe(mib: int, torch) -> None:
    """A plain copy kernel of known size: reads and writes exactly `mib` MiB."""
    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n * 4, "copy_probe_bytes_written": n * 4, "launches": 3}),
          flush=True)


def timed_loop(launch, steps, warmup, torch):
    """Run `launch` warmup + steps times; return (wall ms per step, event ms per launch).

    The timed launches run back to back on the current stream between two HIP
    events recorded on that stream; the event time divided by the number of
    launches is the mean launch duration (it includes the gaps between
    dispatches but no per-launch event overhead, so it agrees with a
    rocprofv3 kernel trace of back-to-back launches)."""
    for _ in range(warmup):
        launch()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        launch()
    end.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    per = start.elapsed_time(end) / steps
    return wall, per


def trial_stats(launch, torch, min_ms=100.0, n_trials=5):
    """Kernel time per launch as the median of `n_trials` trials, each a run
    of back-to-back launches on the current stream lasting at least `min_ms`,
    bracketed by two HIP events recorded on that stream (divided by the
    launch count).  Returns the median, the spread and the trial size."""
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(3):
        launch()
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(3):
        launch()
    e1.record(stream)
    torch.cuda.synchronize()
    est = e0.elapsed_time(e1) / 3
    reps = max(1, int(-(-min_ms // max(est, 1e-4))))
    times = []
    for _ in range(n_trials):
        e0.record(stream)
        for _ in range(reps):
            launch()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) / reps)
    times.sort()
    return {"median_ms": times[len(times) // 2], "min_ms": times[0], "max_ms": times[-1], "trials": n_trials,
            "launches_per_trial": reps}


def peak_probes():
    """Measured issue-rate ceilings of v_dot4_u32_u8, v_fmac_f32 (32
    independent chains per lane; with a literal and one fixed register as the
    factors, and with both factors drawn from two 4-register vectors, the
    operand form of the fp32 walks) and the two signed-byte MFMA shapes (8 or
    4 independent accumulators per wave), 2..16 waves per SIMD; the best rate
    is the measured ceiling."""
    import ctypes
    from cross_correlation_amd import build as b

    lib = ctypes.CDLL(b.PEAK_LIB)
    lib.xc_peak_probe.restype = ctypes.c_int
    lib.xc_peak_probe.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                  ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]
    res = {}
    for kind, name, per_op in ((0, "dot4_T_per_s", 1.0), (1, "fp32_TFLOP_per_s", 2.0),
                               (4, "fp32_register_operands_TFLOP_per_s", 2.0),
                               (2, "mfma_i8_16x16x64_TOP_per_s", 1.0), (3, "mfma_i8_32x32x32_TOP_per_s", 1.0)):
        rates = {}
        for w in (2, 4, 8, 16):
            ms, ops = ctypes.c_double(), ctypes.c_double()
            if lib.xc_peak_probe(kind, w, 2048, 3, ctypes.byref(ms), ctypes.byref(ops)) != 0:
                raise RuntimeError("peak probe failed")
            rates[w] = per_op * ops.value / (ms.value * 1e-3) / 1e12
        res[name] = {f"waves_per_simd_{w}": round(r, 2) for w, r in rates.items()}
        res[name]["max"] = round(max(rates.values()), 2)
    return res


def bench_ncc(args, torch, lib, inputs, variant=0, steps=None, warmup=None, workload="ncc_1920x1080_t64",
              min_ms=None, n_trials=None):
    steps = args.steps if steps is None else steps
    warmup = args.warmup if warmup is None else warmup
    min_ms = args.trial_ms if min_ms is None else min(min_ms, args.trial_ms)
    n_trials = args.trials if n_trials is None else min(n_trials, args.trials)
    case = inputs.workload(workload)
    dev = torch.device("cuda:0")
    img = torch.from_numpy(case.image).to(dev)
    tm = torch.from_numpy(case.tmpl).to(dev)
    oh, ow = case.out_shape
    outs = [torch.empty((oh, ow), dtype=torch.int32, device=dev) for _ in range(3)]
    coef = torch.empty((oh, ow), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    p = [img.data_ptr(), case.width, case.height, case.pitch, tm.data_ptr(), case.t_width, case.t_height,
         outs[0].data_ptr(), outs[1].data_ptr(), outs[2].data_ptr(), coef.data_ptr()]

    def launch():
        st = lib.ncc_u8_run(*p, stream=stream, variant=variant)
        if st != 0:
            raise RuntimeError(lib.status_str(st))

    wall, per = timed_loop(launch, steps, warmup, torch)
    tr = trial_stats(launch, torch, min_ms=min_ms, n_trials=n_trials)
    dot4 = 3 * (case.t_width // 4) * case.t_height * oh * ow
    bytes_alg = case.height * case.width + case.t_width * case.t_height + 16 * oh * ow
    return case, dict(wall_ms=wall, loop_kernel_ms=per, kernel_ms=tr["median_ms"], trials=tr, dot4=dot4,
                      outputs=oh * ow, bytes=bytes_alg)


def bench_ncc_ext(args, torch, lib, inputs):
    """The generalizations on the headline image: the best-match search
    (ncc_u8_peak, with and without the coefficient map), a template width
    that is not a multiple of four (63 x 63, the last packed word of each
    template row masked), a 16 x 16 template (the matrix-core kernel's two
    tile widths), the same and full output modes (ncc_u8_run_mode: the
    zero-padded copy, then the automatic variant; all four outputs), and
    small images (each variant against the automatic choice)."""
    from cross_correlation_amd.inputs import ncc_case
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    res = {}
    steps, warmup = min(args.steps, 50), min(args.warmup, 5)
    case = inputs.workload("ncc_1920x1080_t64")
    img = torch.from_numpy(case.image).to(dev)
    tm = torch.from_numpy(case.tmpl).to(dev)
    oh, ow = case.out_shape
    coef = torch.empty((oh, ow), dtype=torch.float32, device=dev)
    peak = torch.empty(lib.PEAK_BYTES // 8, dtype=torch.int64, device=dev)
    for name, cptr in (("peak_only", 0), ("peak_and_coef", coef.data_ptr())):
        def launch():
            st = lib.ncc_u8_peak(img.data_ptr(), case.width, case.height, case.pitch, tm.data_ptr(), case.t_width,
                                 case.t_height, 0, 0, 0, cptr, peak.data_ptr(), stream=stream)
            if st != 0:
                raise RuntimeError(lib.status_str(st))
        wall, per = timed_loop(launch, steps, warmup, torch)
        res[name] = {"ms_per_step": round(wall, 5), "launches_ms": round(per, 5),
                     "outputs_per_s": round(oh * ow / (per * 1e-3), 1)}
    # A template width that is not a multiple of four (63 x 63), and a small
    # template (16 x 16: 536 matrix-core tiles of 256 columns, two rounds of
    # two workgroups per CU, against 1,005 of 128 columns, one round of four).
    for tname, t, vlist in (("t63x63", 63, (("dot4_ilp", lib.XC_NCC_DOT4_ILP), ("auto", lib.XC_NCC_AUTO))),
                            ("t16x16", 16, (("dot4_ilp", lib.XC_NCC_DOT4_ILP), ("mfma_w4", lib.XC_NCC_MFMA_W4),
                                            ("auto", lib.XC_NCC_AUTO)))):
        sc = ncc_case(f"ncc_1920x1080_{tname}", 2, 1080, 1920, t, t, image_kind="gradient", cut=True)
        img_s = torch.from_numpy(sc.image).to(dev)
        tm_s = torch.from_numpy(sc.tmpl).to(dev)
        oh_s, ow_s = sc.out_shape
        outs = [torch.empty((oh_s, ow_s), dtype=torch.int32, device=dev) for _ in range(3)]
        coef_s = torch.empty((oh_s, ow_s), dtype=torch.float32, device=dev)
        for vname, v in vlist:
            def launch():
                st = lib.ncc_u8_run(img_s.data_ptr(), sc.width, sc.height, sc.pitch, tm_s.data_ptr(), sc.t_width,
                                    sc.t_height, outs[0].data_ptr(), outs[1].data_ptr(), outs[2].data_ptr(),
                                    coef_s.data_ptr(), stream=stream, variant=v)
                if st != 0:
                    raise RuntimeError(lib.status_str(st))
            wall, per = timed_loop(launch, steps, warmup, torch)
            # packed-byte work: 3 dot4 per packed word (the last one masked when t % 4 != 0) per output
            dot4 = 3 * ((sc.t_width + 3) // 4) * sc.t_height * oh_s * ow_s
            res[f"{tname}_{vname}"] = {"kernel_ms": round(per, 5), "outputs_per_s": round(oh_s * ow_s / (per * 1e-3), 1),
                                       "issued_Gdot4_per_s": round(dot4 / (per * 1e-3) / 1e9, 2)}
    for mname, mode in (("same_mode", lib.XC_NCC_MODE_SAME), ("full_mode", lib.XC_NCC_MODE_FULL)):
        st, nbytes = lib.ncc_u8_mode_workspace(case.width, case.height, case.t_width, case.t_height, mode)
        if st != 0:
            raise RuntimeError(lib.status_str(st))
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        moh, mow = lib.ncc_mode_shape(case.width, case.height, case.t_width, case.t_height, mode)
        mouts = [torch.empty((moh, mow), dtype=torch.int32, device=dev) for _ in range(3)]
        mcoef = torch.empty((moh, mow), dtype=torch.float32, device=dev)

        def launch():
            st = lib.ncc_u8_run_mode(img.data_ptr(), case.width, case.height, case.pitch, tm.data_ptr(),
                                     case.t_width, case.t_height, mode, ws.data_ptr(), nbytes, mouts[0].data_ptr(),
                                     mouts[1].data_ptr(), mouts[2].data_ptr(), mcoef.data_ptr(), stream=stream)
            if st != 0:
                raise RuntimeError(lib.status_str(st))
        wall, per = timed_loop(launch, steps, warmup, torch)
        res[mname] = {"launches_ms": round(per, 5), "out_shape": [moh, mow],
                      "outputs_per_s": round(moh * mow / (per * 1e-3), 1)}
    # Small images, where the packed-byte kernel's 256 x 16 tiles would not
    # fill the chip: HIP-event microseconds per launch of each variant and of
    # the automatic choice (uniform pixels, template cut from the image).
    small = {}
    vlist = (("dot4_ilp", lib.XC_NCC_DOT4_ILP), ("dot4_c1", lib.XC_NCC_DOT4_C1), ("mfma_w2", lib.XC_NCC_MFMA_W2),
             ("auto", lib.XC_NCC_AUTO))
    for (h, w, t) in ((256, 256, 16), (480, 640, 8), (480, 640, 16), (600, 800, 8)):
        sc = ncc_case(f"ncc_{w}x{h}_t{t}", 3, h, w, t, t)
        img_s = torch.from_numpy(sc.image).to(dev)
        tm_s = torch.from_numpy(sc.tmpl).to(dev)
        oh_s, ow_s = sc.out_shape
        outs = [torch.empty((oh_s, ow_s), dtype=torch.int32, device=dev) for _ in range(3)]
        coef_s = torch.empty((oh_s, ow_s), dtype=torch.float32, device=dev)
        row = {}
        for vname, v in vlist:
            def launch():
                st = lib.ncc_u8_run(img_s.data_ptr(), sc.width, sc.height, sc.pitch, tm_s.data_ptr(), sc.t_width,
                                    sc.t_height, outs[0].data_ptr(), outs[1].data_ptr(), outs[2].data_ptr(),
                                    coef_s.data_ptr(), stream=stream, variant=v)
                if st != 0:
                    raise RuntimeError(lib.status_str(st))
            wall, per = timed_loop(launch, steps, warmup, torch)
            row[vname + "_us"] = round(per * 1e3, 2)
        st, av = lib.ncc_u8_auto_variant(sc.width, sc.height, sc.t_width, sc.t_height)
        row["auto_picks"] = {lib.XC_NCC_MFMA: "mfma", lib.XC_NCC_DOT4_C1: "dot4_c1",
                             lib.XC_NCC_DOT4_ILP: "dot4_ilp"}.get(av, str(av)) if st == 0 else None
        small[f"{w}x{h}_t{t}x{t}"] = row
    res["small_images"] = small
    return res


def bench_xcorr_large(args, torch, lib, inputs):
    """One-to-one pairs beyond 256 rows (the block-diagonal kernel in passes of
    64 row blocks), with the overlap-wise baseline on the smaller one."""
    from cross_correlation_amd.inputs import xcorr_case
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    res = {}
    names = {"auto": lib.XC_XCORR_AUTO, "overlap": lib.XC_XCORR_OVERLAP, "wave": lib.XC_XCORR_WAVE}
    for n, seed, algos in ((512, 6, ("auto", "overlap", "wave")), (1024, 7, ("auto", "wave"))):
        c = xcorr_case(f"xcorr_1to1_{n}", seed, 1, 1, n, n)
        L = torch.from_numpy(c.left).to(dev)
        R = torch.from_numpy(c.right).to(dev)
        out = torch.empty(c.out_shape, dtype=torch.float32, device=dev)
        flop = 2.0 * n ** 4
        for an in algos:
            algo = names[an]

            def launch():
                st = lib.xcorr_f32_run(L.data_ptr(), 1, R.data_ptr(), 1, n, n, out.data_ptr(), stream=stream, algo=algo)
                if st != 0:
                    raise RuntimeError(lib.status_str(st))

            tr = trial_stats(launch, torch, min_ms=args.trial_ms, n_trials=min(args.trials, 5 if an == "auto" else 3))
            per = tr["median_ms"]
            res[f"xcorr_1to1_{n}_{an}"] = {"kernel_ms": round(per, 4), "gflops": round(flop / (per * 1e-3) / 1e9, 1),
                                           "frac_of_157.3T": round(flop / (per * 1e-3) / FP32_PEAK, 4),
                                           "trials": f"median of {tr['trials']} x {tr['launches_per_trial']} launches"}
    return res


def bench_xcorr_small(args, torch, lib, inputs):
    """Groupings of small matrices (rows <= 12, below the block-diagonal
    kernel's 13): the small-matrix kernel (what the automatic choice runs)
    against the overlap-wise baseline."""
    from cross_correlation_amd.inputs import xcorr_case
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    res = {}
    for nl, nr, rows, cols in ((64, 64, 8, 8), (1, 512, 4, 4), (16, 16, 12, 12), (4, 4, 6, 200)):
        c = xcorr_case("small", 8, nl, nr, rows, cols)
        L = torch.from_numpy(c.left).to(dev)
        R = torch.from_numpy(c.right).to(dev)
        out = torch.empty(c.out_shape, dtype=torch.float32, device=dev)
        flop = 2.0 * nl * nr * (rows * cols) ** 2
        row = {}
        for an, algo in (("small", lib.XC_XCORR_SMALL), ("overlap", lib.XC_XCORR_OVERLAP)):
            def launch():
                st = lib.xcorr_f32_run(L.data_ptr(), nl, R.data_ptr(), nr, rows, cols, out.data_ptr(), stream=stream,
                                       algo=algo)
                if st != 0:
                    raise RuntimeError(lib.status_str(st))
            tr = trial_stats(launch, torch, min_ms=min(40.0, args.trial_ms), n_trials=min(3, args.trials))
            row[f"{an}_us"] = round(tr["median_ms"] * 1e3, 2)
            row[f"{an}_gflops"] = round(flop / (tr["median_ms"] * 1e-3) / 1e9, 1)
        row["speedup"] = round(row["overlap_us"] / row["small_us"], 2)
        res[f"{nl}x{nr}_of_{rows}x{cols}"] = row
    return res


def bench_xcorr(args, torch, lib, inputs, oracle_mod=None):
    dev = torch.device("cuda:0")
    res = {}
    for name in ("xcorr_1to1_256", "xcorr_1to64_64", "xcorr_8to16_32"):
        c = inputs.workload(name)
        L = torch.from_numpy(c.left).to(dev)
        R = torch.from_numpy(c.right).to(dev)
        out = torch.empty(c.out_shape, dtype=torch.float32, device=dev)
        stream = torch.cuda.current_stream().cuda_stream
        nl, nr = c.left.shape[0], c.right.shape[0]
        p = [L.data_ptr(), nl, R.data_ptr(), nr, c.rows, c.cols, out.data_ptr()]

        def launch():
            st = lib.xcorr_f32_run(*p, stream=stream)
            if st != 0:
                raise RuntimeError(lib.status_str(st))

        wall, _ = timed_loop(launch, args.steps, args.warmup, torch)
        tr = trial_stats(launch, torch, min_ms=args.trial_ms, n_trials=args.trials)
        per = tr["median_ms"]
        flop = 2.0 * nl * nr * (c.rows * c.cols) ** 2
        res[name] = {
            "ms_per_step": round(wall, 5),
            "kernel_ms": round(per, 5),
            "kernel_ms_min_max": [round(tr["min_ms"], 5), round(tr["max_ms"], 5)],
            "trials": f"median of {tr['trials']} x {tr['launches_per_trial']} launches",
            "gflops": round(flop / (wall * 1e-3) / 1e9, 1),
            "kernel_gflops": round(flop / (per * 1e-3) / 1e9, 1),
            "frac_of_157.3T": round(flop / (per * 1e-3) / FP32_PEAK, 4),
            "flop_per_step": flop,
        }
        # the same workload through each algorithm that takes it
        algos = {"blockdiag": lib.XC_XCORR_BLOCKDIAG, "mfma": lib.XC_XCORR_MFMA}
        res[name]["algos"] = {}
        for an, av in algos.items():
            def launch_a(av=av):
                st = lib.xcorr_f32_run(*p, stream=stream, algo=av)
                if st != 0:
                    raise RuntimeError(lib.status_str(st))
            if lib.xcorr_f32_run(*p, stream=stream, algo=av) != 0:
                continue
            tra = trial_stats(launch_a, torch, min_ms=min(args.trial_ms, 40.0), n_trials=3)
            res[name]["algos"][an] = {"kernel_ms": round(tra["median_ms"], 5),
                                      "frac_of_157.3T": round(flop / (tra["median_ms"] * 1e-3) / FP32_PEAK, 4)}
        if oracle_mod is not None:
            res[name]["cpu_baseline"] = cpu_baseline_xcorr(args, c, oracle_mod)
    return res


def cpu_baseline(args, inputs, oracle_mod):
    """The oracle on a bounded sample of the headline workload.

    The sample is a band of leading output rows, or the whole image repeated,
    sized to about ``--cpu-seconds`` of host time from a short probe."""
    case = inputs.workload("ncc_1920x1080_t64")
    oh, ow = case.out_shape
    per_out = 3 * (case.t_width // 4) * case.t_height
    # probe: 16 output rows, then the whole image once if that is still short
    t0 = time.perf_counter()
    oracle_mod.ncc_u8(case.image, case.width, case.height, case.tmpl, y_begin=0, y_end=16)
    t_row = (time.perf_counter() - t0) / 16
    if t_row * oh < args.cpu_seconds:
        t0 = time.perf_counter()
        oracle_mod.ncc_u8(case.image, case.width, case.height, case.tmpl)
        t_row = (time.perf_counter() - t0) / oh
    want_rows = args.cpu_seconds / max(t_row, 1e-9)
    if want_rows < oh:
        rows, reps = int(max(16, want_rows)), 1
    else:
        rows, reps = oh, int(max(1, round(want_rows / oh)))
    t0 = time.perf_counter()
    for _ in range(reps):
        oracle_mod.ncc_u8(case.image, case.width, case.height, case.tmpl, y_begin=0, y_end=rows)
    dt = time.perf_counter() - t0
    what = (f"output rows 0..{rows - 1} of {oh}" if reps == 1 else f"the full {oh}x{ow} output, {reps} times")
    return {
        "value": round(per_out * rows * ow * reps / dt / 1e9, 3),
        "unit": "Gdot4/s",
        "cores": oracle_mod.max_threads(),
        "kind": "oracle",
        "sample": f"{what} of the 1920x1080 image / 64x64 template workload ({dt:.1f} s)",
        "host": host_info(),
    }


def cpu_baseline_xcorr(args, case, oracle_mod):
    """The fp32 cross-correlation oracle (fp64 accumulation, the plain output
    without the tolerance sums) on the whole workload, repeated to about
    ``--cpu-seconds`` / 4 of host time; GFLOP/s at 2 * rows^2 * cols^2 per pair."""
    nl, nr = case.left.shape[0], case.right.shape[0]
    flop = 2.0 * nl * nr * (case.rows * case.cols) ** 2
    t0 = time.perf_counter()
    oracle_mod.xcorr_f32(case.left, case.right, with_abs=False)
    dt1 = time.perf_counter() - t0
    reps = max(1, int(round(args.cpu_seconds / 4 / max(dt1, 1e-6))))
    t0 = time.perf_counter()
    for _ in range(reps):
        oracle_mod.xcorr_f32(case.left, case.right, with_abs=False)
    dt = time.perf_counter() - t0
    return {"value": round(flop * reps / dt / 1e9, 3), "unit": "GFLOP/s", "cores": oracle_mod.max_threads(),
            "kind": "oracle", "sample": f"the whole {case.name} workload, {reps} times ({dt:.1f} s)"}


def cpu_baseline_ncc_small(args, case, oracle_mod):
    """The u8 correlation oracle on the whole of a small workload, repeated to
    about ``--cpu-seconds`` / 4 of host time."""
    oh, ow = case.out_shape
    per_out = 3 * ((case.t_width + 3) // 4) * case.t_height
    t0 = time.perf_counter()
    oracle_mod.ncc_u8(case.image, case.width, case.height, case.tmpl)
    dt1 = time.perf_counter() - t0
    reps = max(1, int(round(args.cpu_seconds / 4 / max(dt1, 1e-6))))
    t0 = time.perf_counter()
    for _ in range(reps):
        oracle_mod.ncc_u8(case.image, case.width, case.height, case.tmpl)
    dt = time.perf_counter() - t0
    return {"value": round(per_out * oh * ow * reps / dt / 1e9, 3), "unit": "Gdot4/s",
            "cores": oracle_mod.max_threads(), "kind": "oracle",
            "sample": f"the whole {case.name} workload ({oh}x{ow} outputs), {reps} times ({dt:.1f} s)"}


def host_info() -> dict:
    """The host the oracle ran on: CPU model, CPUs this process may use, and
    OMP_NUM_THREADS as set."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count()
    return {"cpu_model": model, "usable_cpus": usable, "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the hot path runs on a single MI355X)", file=sys.stderr)
        sys.exit(2)
    import torch

    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib, torch)
        return
    from cross_correlation_amd import _lib, inputs

    _lib.load()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    props = torch.cuda.get_device_properties(0)
    out = {
        "metric": METRIC,
        "value": None,
        "unit": "Gdot4/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u8",
        "data": "synthetic",
        "config": {"workload": "ncc_1920x1080_t64", "image": "1920x1080 u8 (uniform + gradient)",
                   "template": "64x64 cut from the image", "outputs": "sum_i,sum_isq,sum_it,coef (1857x1017)"},
        "device": {"name": props.name, "cus": props.multi_processor_count},
    }
    if args.only in ("ncc", "all"):
        case, r = bench_ncc(args, torch, _lib, inputs, variant=_lib.XC_NCC_DOT4_ILP)
        out["value"] = round(r["dot4"] / (r["wall_ms"] * 1e-3) / 1e9, 2)
        out["ms_per_step"] = round(r["wall_ms"], 5)
        achieved = r["dot4"] / (r["kernel_ms"] * 1e-3)
        out["roofline"] = {
            "bound": "alu",
            "achieved": round(achieved / 1e12, 4),
            "peak": round(DOT4_PEAK / 1e12, 4),
            "unit": "Tdot4/s",
            "frac": round(achieved / DOT4_PEAK, 4),
            "traffic": profiled_traffic("ncc_u8_1080p_t64.md", ["ncc_u8.hip", "ncc_common.h"]),
            "kernel": "ncc_u8_ilp_kernel",
            "kernel_ms": round(r["kernel_ms"], 5),
            "kernel_ms_min_max": [round(r["trials"]["min_ms"], 5), round(r["trials"]["max_ms"], 5)],
            "trials": f"median of {r['trials']['trials']} trials x {r['trials']['launches_per_trial']} "
                      f"back-to-back launches (HIP events on the kernel's stream)",
            "outputs_per_s": round(r["outputs"] / (r["kernel_ms"] * 1e-3), 1),
        }
        # The small u8 workload (256x256 image, 16x16 template): launch-bound,
        # reported beside the headline with the oracle on the same input.
        c1, r1 = bench_ncc(args, torch, _lib, inputs, variant=_lib.XC_NCC_AUTO, workload="ncc_256x256_t16")
        out["ncc_256x256_t16"] = {
            "kernel_ms": round(r1["kernel_ms"], 5),
            "kernel_ms_min_max": [round(r1["trials"]["min_ms"], 5), round(r1["trials"]["max_ms"], 5)],
            "nominal_Gdot4_per_s": round(r1["dot4"] / (r1["kernel_ms"] * 1e-3) / 1e9, 2),
            "frac_of_dot4_peak": round(r1["dot4"] / (r1["kernel_ms"] * 1e-3) / DOT4_PEAK, 4),
            "outputs_per_s": round(r1["outputs"] / (r1["kernel_ms"] * 1e-3), 1),
            "auto_picks": {_lib.XC_NCC_MFMA: "mfma", _lib.XC_NCC_DOT4_C1: "dot4_c1", _lib.XC_NCC_DOT4_ILP: "dot4_ilp"}.get(
                _lib.ncc_u8_auto_variant(c1.width, c1.height, c1.t_width, c1.t_height)[1]),
        }
        if not args.no_cpu_baseline:
            import oracle
            out["ncc_256x256_t16"]["cpu_baseline"] = cpu_baseline_ncc_small(args, c1, oracle)
        # The same workload through the other kernel variants (every variant
        # returns identical outputs): the page's ablation points (one output
        # per lane, byte-wise or packed-byte), the ILP series (4 columns x Q
        # rows per lane, no template-row split) and the matrix-core recast of
        # SumIT.
        variants = {"dot4_c1": _lib.XC_NCC_DOT4_C1, "scalar_c1": _lib.XC_NCC_SCALAR_C1,
                    "dot4_ilp_q1": _lib.XC_NCC_DOT4_ILP_Q1, "dot4_ilp_q2": _lib.XC_NCC_DOT4_ILP_Q2,
                    "dot4_ilp_q4": _lib.XC_NCC_DOT4_ILP_Q4,
                    "dot4_cols1": _lib.XC_NCC_DOT4_COLS1, "dot4_cols2": _lib.XC_NCC_DOT4_COLS2,
                    "dot4_cols4": _lib.XC_NCC_DOT4_COLS4, "dot4_cols8": _lib.XC_NCC_DOT4_COLS8,
                    "mfma": _lib.XC_NCC_MFMA, "mfma32": _lib.XC_NCC_MFMA32, "auto": _lib.XC_NCC_AUTO}
        out["ncc_variants"] = {"dot4_ilp": {"kernel_ms": round(r["kernel_ms"], 5), "speedup_vs_dot4_ilp": 1.0}}
        for name, v in variants.items():
            full = name in ("mfma", "mfma32", "auto")
            k = args.steps if full else min(args.steps, 10)
            _, rv = bench_ncc(args, torch, _lib, inputs, variant=v, steps=k, warmup=min(args.warmup, 3),
                              min_ms=100.0 if full else 40.0, n_trials=5 if full else 3)
            out["ncc_variants"][name] = {
                "kernel_ms": round(rv["kernel_ms"], 5),
                "nominal_Gdot4_per_s": round(rv["dot4"] / (rv["kernel_ms"] * 1e-3) / 1e9, 2),
                "outputs_per_s": round(rv["outputs"] / (rv["kernel_ms"] * 1e-3), 1),
                "speedup_vs_dot4_ilp": round(r["kernel_ms"] / rv["kernel_ms"], 3),
            }
        m = out["ncc_variants"]["mfma"]
        # Matrix-core accounting: the SumIT products the method defines (2
        # int8 ops per template pixel per output) over the kernel time.
        ops = 2 * case.t_width * case.t_height * r["outputs"]
        mf_achieved = ops / (m["kernel_ms"] * 1e-3)
        m["roofline"] = {"bound": "mfma", "achieved": round(mf_achieved / 1e12, 2), "peak": I8_MFMA_PEAK / 1e12,
                         "unit": "TOP/s", "frac": round(mf_achieved / I8_MFMA_PEAK, 4),
                         "kernel": "ncc_u8_mfma_kernel",
                         "note": "the column-sum waves' vector work does not hide under the products "
                                 "of its SIMD and lengthens the walk; staging before and the SumIT and "
                                 "coefficient writes after it do not overlap the walk"}
        if not args.no_ext:
            out["ncc_ext"] = bench_ncc_ext(args, torch, _lib, inputs)
    if args.only in ("xcorr", "all"):
        orc = None
        if not args.no_cpu_baseline:
            import oracle as orc
        out["xcorr"] = bench_xcorr(args, torch, _lib, inputs, orc)
        if not args.no_ext:
            out["xcorr_large"] = bench_xcorr_large(args, torch, _lib, inputs)
            out["xcorr_small"] = bench_xcorr_small(args, torch, _lib, inputs)
    if not args.no_peak_probe:
        out["measured_ceilings"] = peak_probes()
        if "ncc_variants" in out:
            ceil = out["measured_ceilings"]["mfma_i8_16x16x64_TOP_per_s"]["max"]
            mr = out["ncc_variants"]["mfma"]["roofline"]
            mr["frac_of_measured_ceiling"] = round(mr["achieved"] / ceil, 4)
        if "roofline" in out:
            ceil = out["measured_ceilings"]["dot4_T_per_s"]["max"]
            out["roofline"]["frac_of_measured_ceiling"] = round(out["roofline"]["achieved"] / ceil, 4)
        if "xcorr" in out:
            ceil = out["measured_ceilings"]["fp32_TFLOP_per_s"]["max"]
            ceil_r = out["measured_ceilings"]["fp32_register_operands_TFLOP_per_s"]["max"]
            for v in out["xcorr"].values():
                v["frac_of_measured_ceiling"] = round(v["kernel_gflops"] / 1e3 / ceil, 4)
                v["frac_of_register_operand_ceiling"] = round(v["kernel_gflops"] / 1e3 / ceil_r, 4)
    if not args.no_cpu_baseline and args.only in ("ncc", "all"):
        import oracle

        out["cpu_baseline"] = cpu_baseline(args, inputs, oracle)
    line = json.dumps(out)
    print(line, flush=True)
    if args.json_out:
        # the folder may not exist yet (a profiler creates its output folder
        # only when the program ends)
        os.makedirs(os.path.dirname(os.path.abspath(args.json_out)), exist_ok=True)
        with open(args.json_out, "w") as f:
            f.write(line + "\n")


if __name__ == "__main__":
    main()
