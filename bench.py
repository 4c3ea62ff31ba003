"""Benchmark: all-pairs angular-separation histograms (DD + DR + RR) on one MI355X.

Workload (default): 100,000 clustered D galaxies + 100,000 uniform R galaxies (fp32
arcmin, seeds 1 and 2), 720 bins of 0.25 deg -- the shape of the 100k + 100k problem of
"CUDA Deep Dive: 10B Galaxy Pairs on an RTX 5080", section "The problem", on synthetic
catalogs.  One step = the whole path on device-resident inputs: prepare D and R (unit
vectors), the histogram call (the tables launch, then the pair kernel: DD, DR, RR), the totals
reduction and omega.

Prints one JSON line.  value = ordered pairs per second (N_D^2 + N_D N_R + N_R^2 per step).
roofline: the pair kernel's algorithmic FP32 work (25 flops per evaluated pair, where the
symmetric families evaluate N(N+1)/2 pairs) over its event-timed duration, against the
MI355X FP32 vector peak.  ceilings: measured VALU and LDS-atomic rates of this GPU, and the
pair kernel's time expressed in those units.  cpu_baseline: the fp64 oracle on a bounded
sample of the same workload (rows of D against all of R), on the host's cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

FLOPS_PER_PAIR = 25.0          # algorithmic FP32 flops per evaluated pair (FMA = 2)
FP32_PEAK_TFLOPS = 157.3       # MI355X FP32 vector peak (published)
NOMINAL_LANE_OPS = 256 * 64 * 2.4e9  # non-packed VALU lane operations per second at 2.4 GHz
DEVICE_SOURCES = ("two_point_angular_amd/csrc/gc_kernels.hip", "two_point_angular_amd/csrc/gc_internal.h",
                  "two_point_angular_amd/csrc/gc_acos_poly.h", "two_point_angular_amd/csrc/gc_api.cpp")


def measured_traffic(workload):
    """HBM bytes per pair-kernel launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    summary of this workload, or None when there is none or the device sources changed since."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"pairs_kernel_{workload}.md")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        parts = line.strip().split(": ")
        if len(parts) == 2 and parts[0] in ("traffic_bytes_per_launch", "device_source_sha256"):
            vals[parts[0]] = parts[1]
    h = hashlib.sha256()
    for f in DEVICE_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    if vals.get("device_source_sha256") != h.hexdigest() or "traffic_bytes_per_launch" not in vals:
        return None
    return float(vals["traffic_bytes_per_launch"])


def cpu_baseline(D, R, nbins, w, target_s=16.0):
    import numpy as np
    from oracle import oracle

    threads = oracle.max_threads()
    rows = 200
    t0 = time.perf_counter()
    oracle.family_rows(D.ra, D.dec, R.ra, R.dec, nbins, w, row0=0, row1=rows)
    dt = time.perf_counter() - t0
    rows2 = int(min(len(D), max(rows, rows * target_s / max(dt, 1e-3))))
    t0 = time.perf_counter()
    fam = oracle.family_rows(D.ra, D.dec, R.ra, R.dec, nbins, w, row0=0, row1=rows2)
    dt2 = time.perf_counter() - t0
    pairs = rows2 * len(R)
    assert int(fam.hist.sum()) == pairs
    return {"value": pairs / dt2, "unit": "pairs/s", "cores": threads, "kind": "oracle",
            "sample": f"DR rows D[0:{rows2}] x R[0:{len(R)}] ({pairs:.3e} ordered pairs, fp64, "
                      f"{dt2:.1f} s on {threads} threads)", "cpu": _cpu_model()}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


LADDER_VARIANTS = [
    # label, rung, arccos, tile, bin stride (0: nbins)
    ("L0 one thread per pair, per-pair sin/cos, acosf", 0, "rung", 0, 0),
    ("L1 + DD/RR symmetry", 1, "rung", 0, 0),
    ("L2 + per-galaxy sin/cos prepass", 2, "rung", 0, 0),
    ("L3 + LDS j-tile (512)", 3, "rung", 512, 0),
    ("L4 + handbook polynomial acos", 4, "rung", 512, 0),
    ("L5 + unroll 8, launch bounds, diagonal skip", 5, "rung", 512, 0),
    ("L5 with acosf", 5, "libm", 512, 0),
    ("L5 with the degree-6 fit (no guard)", 5, "fit6", 512, 0),
    ("L5 tile 64", 5, "rung", 64, 0),
    ("L5 tile 128", 5, "rung", 128, 0),
    ("L5 tile 256", 5, "rung", 256, 0),
    ("L5 tile 1024", 5, "rung", 1024, 0),
    ("L5 bins padded to a multiple of 64", 5, "rung", 512, -64),
    ("L5 bin stride nbins + 1", 5, "rung", 512, -1),
]


def run_ladder(gc, wl, D, R, ra_d, dec_d, ra_r, dec_r, pd, pr, out, ws, reps, warmup):
    """Time each ladder variant (HIP events around the call, median of `reps`) and compare its
    counts with the certified path's: moved pairs = sum over edges of |net flow|, the number of
    bins that differ, and the largest omega change where RR >= 1000."""
    import numpy as np
    import torch

    n_d, n_r, nbins, w = len(D), len(R), wl.nbins, wl.bin_width_deg
    ordered = float(n_d * n_d + n_d * n_r + n_r * n_r)

    def timed(fn):
        for _ in range(warmup):
            fn()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts)), float(np.min(ts))

    def omega(h):
        dd, dr, rr = (x.astype(np.float64) for x in h)
        with np.errstate(divide="ignore", invalid="ignore"):
            return (dd / n_d**2 - 2 * dr / (n_d * n_r) + rr / n_r**2) / (rr / n_r**2)

    gc.prepare(ra_d, dec_d, out=pd)
    gc.prepare(ra_r, dec_r, out=pr)
    ms, mn = timed(lambda: gc.histogram_dd_dr_rr(pd, n_d, pr, n_r, nbins, w, out=out, workspace=ws))
    ref = [x.cpu().numpy().astype(np.int64) for x in out]
    ref_om = omega(ref)
    rows = [{"variant": "certified path (gc.h pair kernel)", "ms": ms, "min_ms": mn, "moved_pairs": 0,
             "bins_differing": 0, "max_abs_domega": 0.0}]
    lws = torch.empty(gc.ladder_workspace_bytes(n_d, n_r), dtype=torch.uint8, device=out.device)
    lout = torch.empty_like(out)
    for label, rung, acos, tile, stride in LADDER_VARIANTS:
        st = stride if stride >= 0 else (((nbins + 63) // 64) * 64 if stride == -64 else nbins + 1)

        def call():
            gc.ladder_histogram(rung, ra_d, dec_d, ra_r, dec_r, nbins, w, acos=acos, tile=tile, bin_stride=st,
                                out=lout, workspace=lws)
        ms, mn = timed(call)
        h = [x.cpu().numpy().astype(np.int64) for x in lout]
        for x, want in zip(h, (n_d * n_d, n_d * n_r, n_r * n_r)):
            if int(x.sum()) != want:
                print(f"{label}: total {int(x.sum())} != {want}", file=sys.stderr)
                sys.exit(1)
        moved = int(sum(np.abs(np.cumsum(a - b)[:-1]).sum() for a, b in zip(h, ref)))
        differing = int(np.any(np.stack([a != b for a, b in zip(h, ref)]), axis=0).sum())
        ok = ref[2] >= 1000
        dom = float(np.max(np.abs(omega(h)[ok] - ref_om[ok]))) if ok.any() else 0.0
        rows.append({"variant": label, "rung": rung, "acos": acos, "tile": tile, "bin_stride": st, "ms": ms,
                     "min_ms": mn, "moved_pairs": moved, "bins_differing": differing, "max_abs_domega": dom})
    for r in rows:
        print(f"# {r['variant']:50s} {r['ms']:10.3f} ms  {ordered / (r['ms'] / 1e3):.3e} pairs/s  "
              f"moved {r['moved_pairs']:9d}  bins differing {r['bins_differing']:4d}  "
              f"max|d omega| {r['max_abs_domega']:.2e}", flush=True)
    print(json.dumps({"ladder": rows, "workload": wl.name, "ordered_pairs": ordered, "reps": reps,
                      "what": "median of HIP-event-timed calls; counts compared with the certified path"}),
          flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="clustered100k_720")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--all", action="store_true",
                    help="one JSON line for each workload (10k, 100k at 720 and 3600 bins, 1M + 1M, the patch), "
                         "each with its CPU baseline; the 1M + 1M run takes a tenth of --steps")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the VALU / LDS ceiling microbenchmarks")
    ap.add_argument("--dot", type=int, default=0, help="tuning: dot-product precision (0 auto, 32, 64)")
    ap.add_argument("--k", type=int, default=0, help="tuning: i galaxies per lane (0 auto, 4, 8)")
    ap.add_argument("--blocks-per-cu", type=int, default=0)
    ap.add_argument("--tune", default="",
                    help="launch-plan overrides as name=value[,name=value...] (fields of gc_tuning, include/gc.h)")
    ap.add_argument("--parts", type=int, default=1,
                    help="run each step's histogram job as this many additive parts (gc_histogram_part)")
    ap.add_argument("--ladder", action="store_true",
                    help="instead of the bench line: time every rung of the page's ablation ladder "
                         "(include/gc_ladder.h) on the workload and compare its counts with the exact path")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="after timing, copy this many bytes device-to-device with a plain copy kernel "
                         "(reference dispatch for scaling FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: the histogram path has no multi-GPU mode "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import two_point_angular_amd as gc
    from two_point_angular_amd import catalogs

    tuning = None
    fields = dict(dot_precision=args.dot, i_per_lane=args.k, blocks_per_cu=args.blocks_per_cu)
    fields.update((kv.split("=")[0], int(kv.split("=")[1])) for kv in args.tune.split(",") if kv)
    if any(fields.values()):
        tuning = gc.Tuning(**fields)
    gc.load()
    if args.all:
        ceilings = None if args.no_ceilings else measure_ceilings(gc)
        for name in ALL_WORKLOADS:
            steps = max(2, args.steps // 10) if name == "clustered1m_720" else args.steps
            line = measure(gc, catalogs.WORKLOADS[name], args, tuning, steps, args.warmup)
            if ceilings:
                line["ceilings"] = ceilings
            print(json.dumps(line), flush=True)
        return
    wl = catalogs.WORKLOADS[args.workload]
    if args.ladder:
        D, R = wl.catalogs()
        dev = torch.device("cuda:0")
        ra_d, dec_d = torch.from_numpy(D.ra).to(dev), torch.from_numpy(D.dec).to(dev)
        ra_r, dec_r = torch.from_numpy(R.ra).to(dev), torch.from_numpy(R.dec).to(dev)
        pd = torch.empty(gc.prepared_bytes(len(D)), dtype=torch.uint8, device=dev)
        pr = torch.empty(gc.prepared_bytes(len(R)), dtype=torch.uint8, device=dev)
        out = torch.empty((3, wl.nbins), dtype=torch.int64, device=dev)
        ws = torch.empty(gc.workspace_bytes(wl.nbins), dtype=torch.uint8, device=dev)
        run_ladder(gc, wl, D, R, ra_d, dec_d, ra_r, dec_r, pd, pr, out, ws, max(args.steps, 1), args.warmup)
        return
    line = measure(gc, wl, args, tuning, args.steps, args.warmup)
    if not args.no_ceilings:
        line["ceilings"] = measure_ceilings(gc)
    print(json.dumps(line), flush=True)


# The workloads of one --all run, in order: the small case, the headline, its 3600-bin and 1M + 1M
# variants, the small-angle patch.
ALL_WORKLOADS = ("uniform10k_720", "clustered100k_720", "clustered100k_3600", "clustered1m_720", "patch100k_1500")


def measure(gc, wl, args, tuning, steps, warmup):
    """One workload: the whole path (prepare D and R, histograms, totals, omega) on resident
    inputs, `warmup` untimed steps then `steps` timed ones.  Every step's histogram call is also
    timed with HIP events on the launch stream; the first step is the cold run (first launch of
    the code), reported apart, and steps 2-9 give the page's median and minimum."""
    import numpy as np
    import torch

    D, R = wl.catalogs()
    n_d, n_r, nbins, w = len(D), len(R), wl.nbins, wl.bin_width_deg
    dev = torch.device("cuda:0")
    ra_d, dec_d = torch.from_numpy(D.ra).to(dev), torch.from_numpy(D.dec).to(dev)
    ra_r, dec_r = torch.from_numpy(R.ra).to(dev), torch.from_numpy(R.dec).to(dev)
    pd = torch.empty(gc.prepared_bytes(n_d), dtype=torch.uint8, device=dev)
    pr = torch.empty(gc.prepared_bytes(n_r), dtype=torch.uint8, device=dev)
    out = torch.empty((3, nbins), dtype=torch.int64, device=dev)
    ws = torch.empty(gc.workspace_bytes(nbins), dtype=torch.uint8, device=dev)
    om = torch.empty(nbins, dtype=torch.float64, device=dev)
    totals = torch.empty((steps + warmup, 3), dtype=torch.int64, device=dev)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps + warmup)]

    def step(idx):
        gc.prepare(ra_d, dec_d, out=pd)
        gc.prepare(ra_r, dec_r, out=pr)
        evs[idx][0].record()
        if args.parts == 1:
            dd, dr, rr = gc.histogram_dd_dr_rr(pd, n_d, pr, n_r, nbins, w, out=out, workspace=ws, tuning=tuning)
        else:
            out.zero_()
            for p in range(args.parts):
                gc.histogram_part(pd, n_d, pr, n_r, nbins, w, p, args.parts, out, workspace=ws, tuning=tuning)
            dd, dr, rr = out[0], out[1], out[2]
        evs[idx][1].record()
        gc.histogram_totals(dd, dr, rr, out=totals[idx])
        gc.omega(dd, dr, rr, n_d, n_r, out=om)

    torch.cuda.synchronize()
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(warmup + i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    if args.copy_bytes:
        src = torch.ones(args.copy_bytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    tot = totals.cpu().numpy().view(np.uint64)
    want = np.array([n_d * n_d, n_d * n_r, n_r * n_r], dtype=np.uint64)
    if not np.all(tot == want[None, :]):
        print(f"{wl.name}: totals mismatch: {tot[:3]} vs {want}", file=sys.stderr)
        sys.exit(1)
    all_ms = np.array([a.elapsed_time(b) for a, b in evs])
    kern_ms = all_ms[warmup:]
    ms_per_step = elapsed * 1e3 / steps
    ordered = float(n_d * n_d + n_d * n_r + n_r * n_r)
    evaluated = float(n_d * n_r + n_d * (n_d + 1) // 2 + n_r * (n_r + 1) // 2)
    kernel_s = float(np.mean(kern_ms)) / 1e3
    achieved = evaluated * FLOPS_PER_PAIR / kernel_s / 1e12
    runs_2_9 = all_ms[1:9]

    line = {
        "metric": "galaxy pairs/sec (DD+DR+RR, 100k×100k, 720 bins); % FP32 VALU peak",
        "value": ordered / (ms_per_step / 1e3),
        "unit": "pairs/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "n_d": n_d, "n_r": n_r, "nbins": nbins, "bin_width_deg": w,
                   "catalogs": f"D {wl.kind} seed 1, R uniform seed 2" if wl.kind == "clustered" else
                   f"D {wl.kind} seed 1, R {wl.kind} seed 2",
                   "ordered_pairs_per_step": ordered, "evaluated_pairs_per_step": evaluated,
                   "parallelism": "1 GPU", **({"parts": args.parts} if args.parts != 1 else {})},
        "kernel_ms": {"mean": float(np.mean(kern_ms)), "median": float(np.median(kern_ms)),
                      "min": float(np.min(kern_ms)),
                      "what": "the histogram call (tables launch + pair kernel), HIP events over the "
                              "timed steps" +
                              (f" ({args.parts} parts)" if args.parts != 1 else "")},
        "protocol": {"cold_ms": float(all_ms[0]),
                     "runs_2_9_median_ms": float(np.median(runs_2_9)) if len(runs_2_9) else None,
                     "runs_2_9_min_ms": float(np.min(runs_2_9)) if len(runs_2_9) else None,
                     "what": "the histogram call's HIP-event time: run 1 cold (first launch in the process), "
                             "median and minimum of runs 2-9 (warm-up steps included)"},
        "roofline": {"bound": "alu", "achieved": achieved, "peak": FP32_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / FP32_PEAK_TFLOPS,
                     # the profile's counters hold for the default plan of one call only
                     "traffic": measured_traffic(wl.name) if tuning is None and args.parts == 1 else None,
                     "note": f"{FLOPS_PER_PAIR:.0f} algorithmic FP32 flops per evaluated pair; achieved over the "
                             "mean event time of the timed steps"},
        "cpu_baseline": None,
        "launch_plan": gc.launch_plan(n_d, n_r, nbins, w, tuning),
    }
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(D, R, nbins, w)
    return line


# The LDS and L1 ceiling probes: (name, probe kind, LDS or table words (a multiple of 128), threads,
# histogram columns).  11520 words: about the sixteen-column histogram of 720 bins; 3712 words:
# about the bin table of 0.25-degree bins.
LDS_CEILINGS = (("lds_atomic_random", "add", 11520, 1024, 0),
                ("lds_atomic_16_columns", "add", 11520, 1024, 16),
                ("lds_read64_random", "read64", 3712, 256, 0))
L1_CEILING = ("l1_read64_random", 3712, 256)


def measure_ceilings(gc):
    """This GPU's measured rates for the resources the pair kernel uses: VALU (independent fp32 and
    fp64 FMA chains, fp32 square roots) and LDS (random ds_add_u32 into one histogram, into a
    sixteen-column one, onto one word; random 8-byte reads) and random 8-byte reads through the
    vector L1 (a 14.8 KiB table).  LDS and L1 rates are 64-lane instructions per second."""
    fma = gc.ceiling_valu(0)
    return {
        "what": "measured in this run; LDS and L1 entries in 64-lane instructions per second and CU cycles "
                "per instruction at 2.4 GHz",
        "fp32_fma_lane_ops_per_s": fma,
        "fp32_fma_frac_of_nominal_2p4ghz": fma / NOMINAL_LANE_OPS,
        "fp32_sqrt_lane_ops_per_s": gc.ceiling_valu(1, iters=2048),
        "fp64_fma_lane_ops_per_s": gc.ceiling_valu(2),
        **{name: {"instr_per_s": r, "cu_cycles_per_instr": 256 * 2.4e9 / r}
           for name, r in ([(n, gc.ceiling_lds(kind, words, threads, cols=cols))
                            for n, kind, words, threads, cols in LDS_CEILINGS] +
                           [("lds_atomic_one_word", gc.ceiling_lds_atomic(720, same_bin=True, iters=256) / 64),
                            (L1_CEILING[0], gc.ceiling_l1(L1_CEILING[1], L1_CEILING[2]))])},
    }


if __name__ == "__main__":
    main()
