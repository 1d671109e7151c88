"""Benchmark of the direct sliding-window correlation hot path on one MI355X.

Headline (``value``): u8 normalized correlation of a 1920x1080 image with a
64x64 template cut from it (valid-mode output 1857x1017, all four outputs:
SumI, SumISq, SumIT and the coefficient), in nominal Gdot4/s:
3 * (t_width/4) * t_height packed-byte dot products per output.  One step is
one ncc_u8_run call on that image with inputs resident in HBM.

The fp32 cross-correlation form is timed in the same run (its own loops,
reported under "xcorr"): one-to-one 256x256, one-to-many 1x64 of 64x64 and
n-to-m 8x16 of 32x32, in GFLOP/s counted as 2*rows^2*cols^2 per pair.

Kernel durations come from HIP events recorded on the stream the kernels run
on, around every launch of the timed region.  The CPU oracle is timed on a
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
DOT4_PEAK = CUS * LANES * CLOCK_HZ          # one v_dot4_u32_u8 per lane per clock
FP32_PEAK = 157.3e12                        # spec vector peak (packed FMA)
FP32_NONPACKED = CUS * LANES * 2 * CLOCK_HZ  # v_fma_f32: 78.6 TFLOP/s


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target length of the CPU sample")
    ap.add_argument("--only", choices=["ncc", "xcorr", "all"], default="all")
    ap.add_argument("--json-out", default=None)
    return ap.parse_args()


def timed_loop(launch, steps, warmup, torch):
    """Run `launch` warmup + steps times; return (wall ms per step, mean event ms per launch)."""
    for _ in range(warmup):
        launch()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s, e in ev:
        s.record(stream)
        launch()
        e.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    per = sum(s.elapsed_time(e) for s, e in ev) / steps
    return wall, per


def bench_ncc(args, torch, lib, inputs):
    case = inputs.workload("ncc_1920x1080_t64")
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
        st = lib.ncc_u8_run(*p, stream=stream)
        if st != 0:
            raise RuntimeError(lib.status_str(st))

    wall, per = timed_loop(launch, args.steps, args.warmup, torch)
    dot4 = 3 * (case.t_width // 4) * case.t_height * oh * ow
    bytes_alg = case.height * case.width + case.t_width * case.t_height + 16 * oh * ow
    return case, dict(wall_ms=wall, kernel_ms=per, dot4=dot4, outputs=oh * ow, bytes=bytes_alg)


def bench_xcorr(args, torch, lib, inputs):
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

        wall, per = timed_loop(launch, args.steps, args.warmup, torch)
        flop = 2.0 * nl * nr * (c.rows * c.cols) ** 2
        res[name] = {
            "ms_per_step": round(wall, 5),
            "kernel_ms": round(per, 5),
            "gflops": round(flop / (wall * 1e-3) / 1e9, 1),
            "kernel_gflops": round(flop / (per * 1e-3) / 1e9, 1),
            "frac_of_157.3T": round(flop / (per * 1e-3) / FP32_PEAK, 4),
            "frac_of_nonpacked_78.6T": round(flop / (per * 1e-3) / FP32_NONPACKED, 4),
            "flop_per_step": flop,
        }
    return res


def cpu_baseline(args, inputs, oracle_mod):
    """The oracle on a bounded sample of the headline workload.

    The sample is a band of leading output rows, or the whole image repeated,
    sized to about ``--cpu-seconds`` of host time from a short probe."""
    case = inputs.workload("ncc_1920x1080_t64")
    oh, ow = case.out_shape
    per_out = 3 * (case.t_width // 4) * case.t_height
    t0 = time.perf_counter()
    oracle_mod.ncc_u8(case.image, case.width, case.height, case.tmpl, y_begin=0, y_end=8)
    t_row = (time.perf_counter() - t0) / 8
    want_rows = args.cpu_seconds / max(t_row, 1e-9)
    if want_rows < oh:
        rows, reps = int(max(8, want_rows)), 1
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
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the hot path runs on a single MI355X)", file=sys.stderr)
        sys.exit(2)
    import torch

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
        case, r = bench_ncc(args, torch, _lib, inputs)
        out["value"] = round(r["dot4"] / (r["wall_ms"] * 1e-3) / 1e9, 2)
        out["ms_per_step"] = round(r["wall_ms"], 5)
        achieved = r["dot4"] / (r["kernel_ms"] * 1e-3)
        out["roofline"] = {
            "bound": "alu",
            "achieved": round(achieved / 1e12, 4),
            "peak": round(DOT4_PEAK / 1e12, 4),
            "unit": "Tdot4/s",
            "frac": round(achieved / DOT4_PEAK, 4),
            "traffic": None,
            "kernel": "ncc_u8_ilp_kernel",
            "kernel_ms": round(r["kernel_ms"], 5),
            "outputs_per_s": round(r["outputs"] / (r["kernel_ms"] * 1e-3), 1),
        }
    if args.only in ("xcorr", "all"):
        out["xcorr"] = bench_xcorr(args, torch, _lib, inputs)
    if not args.no_cpu_baseline and args.only in ("ncc", "all"):
        import oracle

        out["cpu_baseline"] = cpu_baseline(args, inputs, oracle)
    line = json.dumps(out)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(line + "\n")
    print(line, flush=True)


if __name__ == "__main__":
    main()
