#!/usr/bin/env python3
"""Absorbed MLA verify step on one MI355X: microseconds per call and
latent-cache bandwidth, with the roofline of the dominant kernel and the
float64 CPU oracle timed beside it.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
    python bench.py --crossover        # forced-path sweep over L (GLM-4.7-Flash-like geometry)
    python bench.py --verify-curve     # verify cost at L = 1..16 and the derived draft cap
    python bench.py --sparse 2048      # attention over 2048 selected positions vs dense
    python bench.py --indexer          # pooled top-k indexer step: incremental tail vs full pooling

A step is one whole absorbed verify call over one batch of synthetic inputs
already resident in device memory: mla_fold_query (q_lat = q_nope . W_UK),
then mla_absorbed_attention: the split-KV latent attention pass and the merge
(log-sum-exp combine and W_UV up-projection).  The split pass and the merge
are also timed alone (mla_absorbed_splits / mla_absorbed_merge, launches back
to back).  Default workload: DeepSeek-V3
MLA geometry (r 512, n 128, v 128, rope 64), 128 heads, one sequence with a
cache of 8192 positions, L = 8 query rows, bf16 storage, fp32 accumulation.

Input sets are cloned on the device and rotated step by step so that the
data of a step has been evicted from L2 and the 256 MB Infinity Cache before
it is reused (cold); a warm variant reuses one set.  Prints one JSON line.

Other workloads (``--workload``, e.g. the 16-head share of the benchmark
workload, where HBM rather than MFMA bounds the split kernel) print the same
line with their own metric name.  ``--crossover`` times the absorbed call
(fold + attention) against the materialised call (expand + attention) at each
L of the sweep, arms interleaved sample by sample, and prints one line per L.
"""

from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "absorbed MLA verify µs/call + latent-cache HBM GB/s (L=8, Kv=8192, H=128)"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
HEADLINE = "dsv3_h128_kv8192_l8_bf16"

# HBM traffic of the split kernel per launch comes from a committed counter
# summary (rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE, each scaled by the same
# counter on a plain device copy of known size), written by --write-counters
# and keyed to a hash of the kernel's sources: when the kernel has changed since
# the counters were taken the field is reported as null.
COUNTERS_FILE = os.path.join(ROOT, "profiles", "absorbed_split_dsv3_h128_kv8192_l8_counters.md")
KERNEL_SOURCES = ("mla_speculative_decode_amd/csrc/split_absorbed.hip", "mla_speculative_decode_amd/csrc/mla_device.h",
                  "mla_speculative_decode_amd/csrc/internal.h")
SPLIT_KERNEL = "absorbed_split_kernel"


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def read_counter_summary(path=COUNTERS_FILE):
    """The key: value lines of the fenced 'traffic' block of a counter summary, or None."""
    if not os.path.exists(path):
        return None
    out, inside = {}, False
    with open(path) as f:
        for line in f:
            if line.strip() == "```traffic":
                inside = True
            elif inside and line.strip() == "```":
                break
            elif inside and ":" in line:
                k, v = line.split(":", 1)
                out[k.strip()] = v.strip()
    return out or None


def split_traffic_bytes():
    """HBM bytes per split-kernel launch from the counter summary, if it was taken
    on the kernel source that is built now; else None."""
    t = read_counter_summary()
    if not t or t.get("source_sha256") != kernel_source_hash():
        return None
    return round(1024 * (float(t["fetch_kib"]) * float(t["fetch_factor"]) +
                         float(t["write_kib"]) * float(t["write_factor"])))


def write_counter_summary(fetch_csv, write_csv, cal_fetch_csv, cal_write_csv, cal_mib, out_path, commands):
    """Mean FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of every kernel in the
    rocprofv3 counter CSVs, the calibration factors from the plain-copy runs
    (--copy-calibration MIB: MIB read and written per copy), and the fenced
    block bench.py reads, keyed to the hash of the kernel sources built now."""
    import csv
    from collections import defaultdict

    def means(path, counter):
        acc = defaultdict(list)
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    acc[r["Kernel_Name"]].append(float(r["Counter_Value"]))
        return {k: (sum(v) / len(v), len(v)) for k, v in acc.items()}

    fetch, write = means(fetch_csv, "FETCH_SIZE"), means(write_csv, "WRITE_SIZE")
    nbytes = cal_mib * 1048576.0
    cf = max(v[0] for v in means(cal_fetch_csv, "FETCH_SIZE").values())
    cw = max(v[0] for v in means(cal_write_csv, "WRITE_SIZE").values())
    f_fac, w_fac = nbytes / (cf * 1024), nbytes / (cw * 1024)
    split = [k for k in fetch if SPLIT_KERNEL in k]
    if not split:
        raise SystemExit(f"no {SPLIT_KERNEL} dispatch in {fetch_csv}")
    k = split[0]
    lines = ["# Counters: absorbed verify step, DeepSeek-V3 geometry, 128 heads, Kv 8192, L 8, bf16", "",
             "Commands (repository root, on the GPU; one counter per run):", ""]
    lines += ["    " + c for c in commands]
    lines += ["", f"Calibration: the largest kernel of a plain {cal_mib} MiB device copy reads FETCH_SIZE x "
                  f"{f_fac:.3f} and WRITE_SIZE x {w_fac:.3f} of the bytes it moves.", "",
              "| kernel | dispatches | FETCH_SIZE KiB | fetched (scaled) | WRITE_SIZE KiB | written (scaled) |",
              "|---|---:|---:|---:|---:|---:|"]
    for name in sorted(fetch, key=lambda n: -fetch[n][0]):
        if name not in write:
            continue
        fk, n = fetch[name]
        wk = write[name][0]
        short = name.split("(")[0][:70]
        lines.append(f"| {short} | {n} | {fk:,.1f} | {fk * 1024 * f_fac / 1e6:.2f} MB | {wk:,.1f} | "
                     f"{wk * 1024 * w_fac / 1e6:.2f} MB |")
    fk, wk = fetch[k][0], write[k][0]
    lines += ["", "Machine-readable summary of the split kernel (read by bench.py; valid only while the",
              "kernel sources hash to source_sha256):", "", "```traffic",
              f"source_sha256: {kernel_source_hash()}", f"kernel: {k.split('(')[0]}",
              f"fetch_kib: {fk:.1f}", f"write_kib: {wk:.1f}", f"fetch_factor: {f_fac:.4f}",
              f"write_factor: {w_fac:.4f}", "```", ""]
    with open(out_path, "w") as f:
        f.write("\n".join(lines))
    print(f"wrote {out_path}: {SPLIT_KERNEL} fetch {fk:.1f} KiB x {f_fac:.3f}, write {wk:.1f} KiB x {w_fac:.3f}")


def host_info():
    """CPU model and software versions of the machine the line was measured on."""
    import platform
    import torch
    cpu = platform.processor() or ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    rocm = None
    for path in ("/opt/rocm/.info/version", "/opt/rocm/.info/version-dev"):
        if os.path.exists(path):
            with open(path) as f:
                rocm = f.read().strip()
            break
    gpu = torch.cuda.get_device_name(0) if torch.cuda.is_available() else None
    return {"cpu_model": cpu, "host_cpus": os.cpu_count(), "rocm": rocm, "torch": torch.__version__,
            "hip": getattr(torch.version, "hip", None), "gpu": gpu}


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="dsv3_h128_kv8192_l8_bf16")
    ap.add_argument("--cache", choices=("bf16", "fp8"), default="bf16",
                    help="latent cache form: bf16, or fp8 (E4M3 codes + power-of-two scale per position)")
    ap.add_argument("--cold-bytes", type=float, default=768e6,
                    help="total bytes of rotated input sets (cold protocol); 0 = warm only")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--crossover", action="store_true",
                    help="forced-path sweep: absorbed vs materialised call at each L of the sweep")
    ap.add_argument("--samples", type=int, default=15, help="samples per arm and L (--crossover)")
    ap.add_argument("--verify-curve", action="store_true",
                    help="time the verify call at L = 1..max-width and derive the draft cap from the curve")
    ap.add_argument("--max-width", type=int, default=16, help="largest L of --verify-curve")
    ap.add_argument("--sparse", type=int, default=0, metavar="BUDGET",
                    help="time attention over BUDGET selected positions against dense attention, GLM-5.3-like "
                         "geometry, caches of 2048..32768")
    ap.add_argument("--indexer", action="store_true",
                    help="time the pooled top-k indexer step (tail vs full pooling, scores, selection) and the "
                         "sparse attention it feeds, caches of 8192 and 131072")
    ap.add_argument("--lds-probe", action="store_true",
                    help="LDS lane groups of ds_read_b128 / ds_read_b64_tr_b16 and the split kernel's read layouts")
    ap.add_argument("--write-counters", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "CAL_FETCH_CSV", "CAL_WRITE_CSV"),
                    help="write the split kernel's counter summary from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE "
                         "CSVs of the benchmark and of --copy-calibration runs (no GPU needed)")
    ap.add_argument("--calibration-mib", type=int, default=256, help="MiB copied by the calibration runs")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (counter calibration) and exit")
    return ap.parse_args()


def main():
    args = parse()
    if args.lds_probe:
        lds_probe()
        return
    if args.write_counters:
        cmds = ["rocprofv3 --pmc FETCH_SIZE --output-format csv -d <out> -o fetch -- python bench.py --steps 20 "
                "--warmup 5 --no-cpu-baseline",
                "rocprofv3 --pmc WRITE_SIZE --output-format csv -d <out> -o write -- python bench.py --steps 20 "
                "--warmup 5 --no-cpu-baseline",
                f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d <out> -o cfetch -- python bench.py "
                f"--copy-calibration {args.calibration_mib}",
                f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d <out> -o cwrite -- python bench.py "
                f"--copy-calibration {args.calibration_mib}",
                "python bench.py --write-counters <out>/fetch_counter_collection.csv "
                "<out>/write_counter_collection.csv <out>/cfetch_counter_collection.csv "
                "<out>/cwrite_counter_collection.csv"]
        write_counter_summary(*args.write_counters, args.calibration_mib, COUNTERS_FILE, cmds)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path (asked for {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import mla_speculative_decode_amd as mla
    from mla_speculative_decode_amd import synth, _lib

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": 3}))
        return
    if args.crossover:
        crossover(args)
        return
    if args.verify_curve:
        verify_curve(args)
        return
    if args.sparse:
        sparse_sweep(args)
        return
    if args.indexer:
        indexer_sweep(args)
        return
    w = synth.WORKLOADS[args.workload]
    if w.dtype != "bf16":
        raise SystemExit("bench.py times the bf16 path")
    x = synth.make_inputs(w)
    B, L, H = w.batch, x.L, w.heads
    t0 = time.perf_counter()
    fp8 = args.cache == "fp8"
    cold, warm, nsets = absorbed_timing(w, x, args.cold_bytes, args.steps, args.warmup, fp8=fp8)
    wall = time.perf_counter() - t0

    peaks = measured_peaks()

    # algorithmic work of one call
    lens = np.diff(x.offsets)
    vis = sum(int(H * (kv * L - L * (L - 1) // 2)) for kv in lens)          # sum over rows of visible positions
    attn_flop = 2.0 * (2 * w.r + w.rope) * vis                            # scores (r+rope) + latent PV (r)
    # bf16 cache: 2 bytes per value; fp8 cache: 1 byte per value + a float32 scale per position
    cache_bytes = float(lens.sum() * ((w.r + w.rope) + 4)) if fp8 else float(lens.sum() * (w.r + w.rope) * 2)
    q_bytes = float(B * L * H * (w.r + w.rope) * 2)                       # q_lat + q_pe read by the split kernel
    weight_bytes = float(2 * H * w.n * w.r * 2)                            # W_UK + W_UV, bf16
    # split partials written by the split pass and read back by the merge (bf16 sums + (max, sum) floats)
    geom = mla.Geom(w.r, w.n, w.v, w.rope, H)
    ws_bytes = mla.absorbed_workspace_size(geom, _lib.MLA_BF16, L, mla.Offsets(x.offsets.astype(np.int32), "cpu"))
    partial_bytes = float(ws_bytes)
    us_step, us_fold, us_attn, _, us_evented, us_split_b2b, us_merge_b2b, us_fold_b2b = cold
    # roofline of the split kernel: its launches back to back (per-launch duration
    # without the dispatch gap that an event pair around one launch also measures)
    intensity = attn_flop / cache_bytes
    # fp8 cache: the scores run on fp8 MFMA, PV on bf16, so the contraction's peak
    # is the rate at which both halves would finish at their own peaks
    score_flop = 2.0 * (w.r + w.rope) * vis
    mfma_peak = (attn_flop / (score_flop / PEAK_FP8_TFLOPS + (attn_flop - score_flop) / PEAK_BF16_TFLOPS)
                 if fp8 else PEAK_BF16_TFLOPS)
    if intensity >= mfma_peak * 1e12 / (PEAK_HBM_GBPS * 1e9):
        achieved = attn_flop / (us_split_b2b * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": round(mfma_peak, 1), "unit": "TFLOP/s",
                "frac": round(achieved / mfma_peak, 4)}
    else:
        achieved = (cache_bytes + q_bytes) / (us_split_b2b * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBPS, 4)}
    measured = (peaks["mfma_bf16_TFLOPs"] * mfma_peak / PEAK_BF16_TFLOPS if roof["bound"] == "mfma"
                else peaks["hbm_read_GBps"])
    traffic = split_traffic_bytes() if (w.name == HEADLINE and not fp8) else None
    alg_bytes = cache_bytes + q_bytes + partial_bytes
    roof = {"kernel": ("absorbed_split_f8_kernel (mla_absorbed_splits_fp8q)" if fp8 else
                       "absorbed_split_kernel (mla_absorbed_splits)"), **roof, "duration_us": round(us_split_b2b, 3),
            "traffic": traffic,
            "traffic_over_algorithmic": round(traffic / alg_bytes, 3) if traffic else None,
            "algorithmic_bytes": round(alg_bytes),
            "measured_peak": round(measured, 1), "frac_measured": round(roof["achieved"] / measured, 4)}

    line = {
        "metric": METRIC if (w.name == HEADLINE and not fp8) else
                  f"absorbed MLA verify µs/call + latent-cache HBM GB/s ({w.name}{', fp8 cache' if fp8 else ''})",
        "value": round(us_step, 3),
        "unit": "us/call",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us_step / 1e3, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations, N(0,1/r) weights)",
        "config": {"workload": w.name, "r": w.r, "n": w.n, "v": w.v, "rope": w.rope, "heads": H, "batch": B,
                   "kv": int(lens.max()), "kv_total": int(lens.sum()), "L": L, "cache": args.cache,
                   "cache_state": f"cold ({nsets} rotated input sets)"},
        "latent_cache_GBps": round(cache_bytes / (us_split_b2b * 1e-6) / 1e9, 1),
        "latent_cache_GBps_split_merge": round(cache_bytes / ((us_split_b2b + us_merge_b2b) * 1e-6) / 1e9, 1),
        "step_GBps": round((cache_bytes + weight_bytes) / (us_step * 1e-6) / 1e9, 1),
        "flop_per_cache_byte": round(intensity, 1),
        "per_launch_us": {"fold": round(us_fold, 3), "attention": round(us_attn, 3),
                          "splits_back_to_back": round(us_split_b2b, 3),
                          "merge_back_to_back": round(us_merge_b2b, 3), "fold_back_to_back": round(us_fold_b2b, 3)},
        "warm_us_per_call": round(warm[0], 3),
        "warm_per_launch_us": {"fold": round(warm[1], 3), "attention": round(warm[2], 3),
                               "splits_back_to_back": round(warm[5], 3)},
        "partial_sum_bytes_per_step": round(partial_bytes),
        "roofline": roof,
        "host": host_info(),
        "peaks_measured": {k: round(v, 1) for k, v in peaks.items()},
        "wall_s": round(wall, 3),
    }

    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(x, args.cpu_seconds)
    print(json.dumps(line), flush=True)


def lds_probe():
    """Which lanes of one LDS read the hardware serves in the same cycle (a pair
    of lanes on one bank set slows the read only then), and the cycles per read
    of the bf16 split kernel's score-fragment and transposed V reads under the
    row layouts it was measured with.  Prints one JSON line."""
    import torch
    blib = ctypes.CDLL(os.path.join(ROOT, "mla_speculative_decode_amd", "libmla_bench.so"))
    scratch = torch.zeros(256 * 8, dtype=torch.int64, device="cuda:0")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda:0")
    stream = torch.cuda.current_stream()
    clk = ctypes.c_double()
    args = (ctypes.c_void_p(scratch.data_ptr()), ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(stream.cuda_stream),
            ctypes.byref(clk))
    blib.mlab_lds_pair.restype = ctypes.c_int
    blib.mlab_lds_layout.restype = ctypes.c_int

    def pair(op, li, lj, same):
        if blib.mlab_lds_pair(op, li, lj, same, 200, *args) != 0:
            raise RuntimeError("LDS probe failed")
        return clk.value

    def layout(pat, lrb, swz):
        if blib.mlab_lds_layout(pat, lrb, swz, 400, *args) != 0:
            raise RuntimeError("LDS probe failed")
        return round(clk.value, 2)

    groups = {}
    for op, name in ((0, "ds_read_b128"), (1, "ds_read_b64_tr_b16")):
        groups[name] = {}
        for li in (0, 4, 32):
            same_cycle = [lj for lj in range(64) if lj == li or pair(op, li, lj, 1) > 1.06 * pair(op, li, lj, 0)]
            groups[name]["lane %d" % li] = same_cycle
    layouts = {}
    for lrb, swz in ((1072, 0), (1056, 0), (1088, 0), (1088, 1)):
        key = "%d-byte rows%s" % (lrb, ", chunk swizzle" if swz else "")
        layouts[key] = {"score fragments (ds_read_b128)": layout(0, lrb, swz),
                        "transposed V (ds_read_b64_tr_b16)": layout(1, lrb, swz)}
    print(json.dumps({"lds_lanes_served_together": groups, "lds_clk_per_read": layouts}), flush=True)


def measured_peaks():
    """Achievable peaks on this GPU (libmla_bench.so): a streaming read of 1 GiB
    and a dense stream of independent bf16 32x32x16 MFMAs."""
    import torch
    blib = ctypes.CDLL(os.path.join(ROOT, "mla_speculative_decode_amd", "libmla_bench.so"))
    buf = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0")
    sink = torch.zeros(16, dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream()
    gbps, tflops = ctypes.c_double(), ctypes.c_double()
    for fn, args in ((blib.mlab_stream_read, (ctypes.c_void_p(buf.data_ptr()), ctypes.c_size_t(buf.numel()),
                                               ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(stream.cuda_stream),
                                               5, ctypes.byref(gbps))),
                     (blib.mlab_mfma_peak, (ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(stream.cuda_stream),
                                            4096, ctypes.byref(tflops)))):
        fn.restype = ctypes.c_int
        if fn(*args) != 0:
            raise RuntimeError("peak measurement failed")
    torch.cuda.synchronize()
    del buf
    return {"hbm_read_GBps": gbps.value, "mfma_bf16_TFLOPs": tflops.value}


def absorbed_timing(w, x, cold_bytes, steps, warmup, fp8=False):
    """Time the absorbed verify call on inputs x through the native loop: the
    cold rotation of cloned input sets, then one warm set.  Returns the result
    arrays of both runs (see bench_driver.cpp) and the number of sets."""
    import torch
    import mla_speculative_decode_amd as mla
    from mla_speculative_decode_amd import _lib

    lib = _lib.load()
    blib = ctypes.CDLL(os.path.join(ROOT, "mla_speculative_decode_amd", "libmla_bench.so"))
    blib.mlab_absorbed_run.restype = ctypes.c_int
    B, L, H = w.batch, x.L, w.heads
    dev = torch.device("cuda:0")

    def up(a):
        return torch.from_numpy(a).to(torch.bfloat16).to(dev).contiguous()

    base = {k: up(getattr(x, k)) for k in ("q_nope", "q_pe", "c_kv", "k_pe", "w_uk", "w_uv")}
    if fp8:   # the cache in its fp8 form (quantised once, outside the timed region)
        base["codes"], base["scales"] = mla.quantize_latent_fp8(base["c_kv"], base["k_pe"])
        del base["c_kv"], base["k_pe"]
        base["c_kv"], base["k_pe"] = base["codes"], base["codes"]   # placeholders, not read
    set_bytes = sum(t.numel() * t.element_size() for k, t in base.items() if k not in ("c_kv", "k_pe") or not fp8)
    nsets = max(1, int(math.ceil(cold_bytes / set_bytes))) if cold_bytes > 0 else 1
    sets = [base] + [{k: t.clone() for k, t in base.items()} for _ in range(nsets - 1)]
    if fp8:
        for st in sets:
            st["c_kv"], st["k_pe"] = st["codes"], st["codes"]
    geom = mla.Geom(w.r, w.n, w.v, w.rope, H)
    for st in sets:
        st["q_lat"] = torch.empty((B, L, H, w.r), dtype=torch.bfloat16, device=dev)
        st["out"] = torch.empty((B, L, H, w.v), dtype=torch.float32, device=dev)
        if fp8:   # the fold's E4M3 query block (mla_fold_query_fp8 -> mla_absorbed_attention_fp8q)
            st["q8"] = torch.empty(mla.query_fp8_bytes(geom, B, L), dtype=torch.uint8, device=dev)
    offs = mla.Offsets(x.offsets.astype(np.int32), dev)
    ws_bytes = mla.absorbed_workspace_size(geom, _lib.MLA_BF16, L, offs)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.Stream()

    def ptrs(key, idx):
        return (ctypes.c_void_p * len(idx))(*[sets[i][key].data_ptr() for i in idx])

    def run(idx):
        res = (ctypes.c_double * 8)()
        torch.cuda.synchronize()
        rc = blib.mlab_absorbed_run(
            ctypes.byref(geom), B, L, len(idx), ptrs("q_nope", idx), ptrs("q_pe", idx), ptrs("c_kv", idx),
            ptrs("k_pe", idx), ptrs("w_uk", idx), ptrs("w_uv", idx), ptrs("q_lat", idx), ptrs("out", idx),
            offs.host_ptr(), offs.dev_ptr(), ctypes.c_float(x.scale), ctypes.c_void_p(ws.data_ptr()),
            ctypes.c_size_t(ws_bytes), ctypes.c_void_p(stream.cuda_stream), warmup, steps, res,
            ptrs("codes", idx) if fp8 else None, ptrs("scales", idx) if fp8 else None,
            ptrs("q8", idx) if fp8 else None)
        torch.cuda.synchronize()
        if rc != 0:
            raise RuntimeError(f"bench step failed: {lib.mla_status_string(rc).decode()}")
        return list(res)

    # timed region: W untimed steps, then K steps between synchronisations
    cold = run(list(range(nsets)))
    warm = run([0])
    return cold, warm, nsets


def verify_curve(args):
    """Verify-width cost curve of the benchmark geometry (DeepSeek-V3 MLA, 128
    heads, one cache of 8192 positions): the absorbed verify call timed at
    L = 1..16 rows, cold, and the draft cap a speculative decoder would derive
    from it (mla_draft_cap) for a few survival rates p and drafter costs.  The
    curve covers the attention of the verify step only."""
    import mla_speculative_decode_amd as mla
    from mla_speculative_decode_amd import synth

    w = synth.WORKLOADS[HEADLINE]
    us = []
    for L in range(1, args.max_width + 1):
        x = synth.make_inputs(w, L=L)
        cold, warm, nsets = absorbed_timing(w, x, args.cold_bytes, args.steps, args.warmup)
        us.append(cold[0])
        print(json.dumps({"verify_curve": w.name, "L": L, "us_per_call": round(cold[0], 3),
                          "splits_us": round(cold[5], 3), "merge_us": round(cold[6], 3), "fold_us": round(cold[7], 3),
                          "relative": round(cold[0] / us[0], 4), "cache_state": f"cold ({nsets} rotated input sets)"}),
              flush=True)
    caps = []
    for drafter in (0.05, 0.2):
        for p in (0.5, 0.6, 0.7, 0.8, 0.9):
            cap, sp, by_cap = mla.draft_cap(us, p, drafter)
            caps.append({"p": p, "drafter": drafter, "cap": cap, "speedup": round(sp, 4)})
    print(json.dumps({"verify_curve_summary": w.name, "relative_cost": [round(u / us[0], 4) for u in us],
                      "derived_caps": caps}), flush=True)


class ReadScrub:
    """Evicts the caches between samples by reading 512 MiB (a sum into one float).
    A read leaves clean lines behind; a scrub by writing would leave dirty lines
    whose write-back the next sample's reads pay for (measured: a cold 67 MB read
    at 2.8 TB/s after a write scrub against 5.3 TB/s after this one)."""

    def __init__(self, dev):
        import torch
        self.buf = torch.zeros(128 << 20, dtype=torch.float32, device=dev)
        self.sink = torch.empty((), dtype=torch.float32, device=dev)

    def __call__(self):
        import torch
        torch.sum(self.buf, dim=0, out=self.sink)


def sparse_sweep(args):
    """Absorbed attention (after the fold) over a selection of `budget` cached
    positions against dense attention over the whole cache: GLM-5.3-Flash-like
    geometry (r 512, n 256, v 256, rope 64), 64 heads, L = 16, one sequence, caches
    of 2048, 8192 and 32768 positions.  The selection is seeded random positions
    plus the newest L (an indexer's top-k stands in; its scoring is not part of
    this path).  Cold: a 512 MiB read scrub (ReadScrub) before every sample; events around
    the call, median of `samples`."""
    import torch
    import mla_speculative_decode_amd as mla
    from mla_speculative_decode_amd import synth

    budget = args.sparse
    dev = torch.device("cuda:0")
    scrub = ReadScrub(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(1000)
    e0.record()
    torch.cuda._sleep(1_000_000)
    e1.record()
    torch.cuda.synchronize()
    spin = int(1_000_000 * 2.0 / max(e0.elapsed_time(e1), 1e-3))
    for kv in (2048, 8192, 32768):
        w = synth.custom(512, 256, 256, 64, 64, 1, 16, kv=kv, dtype="bf16", seed=9, name=f"glm53_h64_kv{kv}_l16")
        x = synth.make_inputs(w)
        rng = np.random.default_rng(kv)
        k = min(budget, kv)
        sel = np.sort(np.concatenate([rng.choice(kv - w.L, size=k - w.L, replace=False),
                                      np.arange(kv - w.L, kv)])).astype(np.int32)
        d = {n: torch.from_numpy(getattr(x, n)).to(torch.bfloat16).to(dev).contiguous()
             for n in ("q_nope", "q_pe", "c_kv", "k_pe", "w_uk", "w_uv")}
        q_lat = mla.fold_query(d["q_nope"], d["w_uk"])
        offs = mla.Offsets(x.offsets.astype(np.int32), dev)
        soffs = mla.Offsets(np.array([0, k], dtype=np.int32), dev)
        sel_d = torch.from_numpy(sel).to(dev)
        out = torch.empty((1, w.L, w.heads, w.v), dtype=torch.float32, device=dev)
        arms = {
            "sparse": lambda: mla.absorbed_attention_sparse(q_lat, d["q_pe"], d["c_kv"], d["k_pe"], d["w_uv"], offs,
                                                            sel_d, soffs, scale=x.scale, out=out),
            "dense": lambda: mla.absorbed_attention(q_lat, d["q_pe"], d["c_kv"], d["k_pe"], d["w_uv"], offs,
                                                    scale=x.scale, out=out),
        }
        if args.cache == "fp8":   # the same two calls over the fp8 form of the cache
            codes, scales = mla.quantize_latent_fp8(d["c_kv"], d["k_pe"])
            arms = {
                "sparse": lambda: mla.absorbed_attention_sparse_fp8(q_lat, d["q_pe"], codes, scales, d["w_uv"], offs,
                                                                    sel_d, soffs, scale=x.scale, out=out),
                "dense": lambda: mla.absorbed_attention_fp8(q_lat, d["q_pe"], codes, scales, d["w_uv"], offs,
                                                            scale=x.scale, out=out),
            }
        for f in arms.values():
            f()
        times = {a: [] for a in arms}
        for i in range(args.samples):
            for a in (("sparse", "dense") if i % 2 == 0 else ("dense", "sparse")):
                scrub()
                torch.cuda._sleep(spin)
                e0.record()
                arms[a]()
                e1.record()
                torch.cuda.synchronize()
                times[a].append(e0.elapsed_time(e1) * 1e3)
        print(json.dumps({"sparse_attention": w.name, "kv": kv, "budget": k, "cache": args.cache,
                          "sparse_us": round(float(np.median(times["sparse"])), 2),
                          "dense_us": round(float(np.median(times["dense"])), 2),
                          "samples": args.samples, "cache_state": "cold (512 MiB read scrub before each sample)"}),
              flush=True)
        del d, q_lat, out, sel_d
        torch.cuda.empty_cache()


def indexer_sweep(args):
    """The pooled top-k indexer of a sparse layer, one sequence, a verify step
    of S = 8 new positions, keys = the bf16 latent rows (width 512), budget 2048:
    the whole indexer step (pooling, scores, selection) with the incremental
    tail (guards hold; separately, or pooled by the scoring launch itself)
    against pooling the whole cache, each kernel on its own,
    and the absorbed attention over the selected positions that follows
    (GLM-5.3-Flash-like geometry, 64 heads, the step's 8 rows).  Cold: a 512 MiB
    read scrub (ReadScrub) before every sample; the host queues a sample's launches behind
    a 2 ms device spin, so they run back to back.  Each sample runs twice: with
    events around each piece (an event between kernels adds a dispatch gap of
    about 6 us), and with events only around the step, which gives the step
    figures.  Median of `samples`, arms interleaved."""
    import torch
    import mla_speculative_decode_amd as mla
    from mla_speculative_decode_amd import synth

    wl = synth.INDEXER_WORKLOAD
    S, d, budget = wl["S"], wl["d"], wl["budget"]
    dev = torch.device("cuda:0")
    scrub = ReadScrub(dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(8)]
    torch.cuda._sleep(1000)
    ev[0].record()
    torch.cuda._sleep(1_000_000)
    ev[1].record()
    torch.cuda.synchronize()
    spin = int(1_000_000 * 2.0 / max(ev[0].elapsed_time(ev[1]), 1e-3))
    for T in (8192, wl["kv"]):
        x = synth.indexer_inputs([T], d, seed=wl["seed"])
        keys = torch.from_numpy(x.keys).to(torch.bfloat16).to(dev)   # also the attention's c_kv
        q = torch.from_numpy(x.q).to(dev)
        offs = mla.Offsets(x.offsets.astype(np.int32), dev)
        cap = (T + 3) // 4
        pool = mla.IndexerPool(capacity=cap, batch_max=1, d=d, device=dev)
        assert not pool.step(keys[:T - S], [0, T - S], S=T - S)
        assert pool.step(keys, offs, S=S)
        scores = torch.empty((1, cap), dtype=torch.float32, device=dev)
        soffs = mla.selection_offsets(offs, budget, dev)
        k = int(soffs.host[-1])
        sel = torch.empty(k, dtype=torch.int32, device=dev)
        # attention that follows: GLM-5.3-Flash-like heads over the same latent rows
        H, L, n, v, rope = 64, S, 256, 256, 64
        aw = synth.custom(512, n, v, rope, H, 1, L, kv=T, seed=wl["seed"] + 1)
        q_nope = torch.from_numpy(synth.draw_like((1, L, H, n), 1.0, "bf16", 71)).to(torch.bfloat16).to(dev)
        q_pe = torch.from_numpy(synth.draw_like((1, L, H, rope), 1.0, "bf16", 72)).to(torch.bfloat16).to(dev)
        k_pe = torch.from_numpy(synth.draw_like((T, rope), 1.0, "bf16", 73)).to(torch.bfloat16).to(dev)
        w_uk = torch.from_numpy(synth.draw_like((H, n, 512), 1 / math.sqrt(512), "bf16", 74)).to(torch.bfloat16).to(dev)
        w_uv = torch.from_numpy(synth.draw_like((H, 512, v), 1 / math.sqrt(512), "bf16", 75)).to(torch.bfloat16).to(dev)
        q_lat = torch.empty((1, L, H, 512), dtype=torch.bfloat16, device=dev)
        out = torch.empty((1, L, H, v), dtype=torch.float32, device=dev)

        def pool_tail():
            pool.trim([T - S])   # host only: the pool again covers T - S positions
            assert pool.step(keys, offs, S=S)

        def pool_full():
            pool.state.valid = 0   # host only: no pool, so every window is pooled
            assert not pool.step(keys, offs, S=S)

        def score():
            pool.scores(q, offs, out=scores)

        def select():
            mla.indexer_select(scores, offs, budget, sel_offsets=soffs, out=sel)

        def attend():
            mla.fold_query(q_nope, w_uk, out=q_lat)
            mla.absorbed_attention_sparse(q_lat, q_pe, keys, k_pe, w_uv, offs, sel, soffs, scale=aw.scale, out=out)

        def fused():   # the tail pooled by the scoring launch itself
            pool.trim([T - S])
            assert pool.step_scores(keys, offs, S=S, q=q, out=scores)[1]

        def nothing():
            pass

        arms = {"incremental": (pool_tail, score, select, attend), "full": (pool_full, score, select, attend),
                "fused": (fused, nothing, select, attend)}
        for parts in arms.values():
            for f in parts:
                f()
        times = {a: [[] for _ in range(4)] for a in arms}
        whole = {a: [[], []] for a in arms}
        for i in range(args.samples):
            for a in (("incremental", "full", "fused") if i % 2 == 0 else ("fused", "full", "incremental")):
                # pieces: an event after every piece (each event adds a dispatch gap)
                scrub()
                torch.cuda._sleep(spin)
                ev[0].record()
                for j, f in enumerate(arms[a]):
                    f()
                    ev[j + 1].record()
                torch.cuda.synchronize()
                for j in range(4):
                    times[a][j].append(ev[j].elapsed_time(ev[j + 1]) * 1e3)
                # whole: events only before the step, after the selection and after the attention
                scrub()
                torch.cuda._sleep(spin)
                ev[5].record()
                for f in arms[a][:3]:
                    f()
                ev[6].record()
                arms[a][3]()
                ev[7].record()
                torch.cuda.synchronize()
                whole[a][0].append(ev[5].elapsed_time(ev[6]) * 1e3)
                whole[a][1].append(ev[5].elapsed_time(ev[7]) * 1e3)
        med = {a: [float(np.median(t)) for t in times[a]] for a in arms}
        wmed = {a: [float(np.median(t)) for t in whole[a]] for a in arms}
        inc, full = med["incremental"], med["full"]
        W = cap
        print(json.dumps({
            "indexer": wl["name"] if T == wl["kv"] else f"indexer_kv{T}_s{S}_d{d}_top{budget}", "kv": T, "S": S,
            "d": d, "budget": budget, "windows": W,
            "indexer_step_us": {"incremental": round(wmed["incremental"][0], 2), "full": round(wmed["full"][0], 2),
                                "incremental_fused": round(wmed["fused"][0], 2)},
            "layer_step_us": {"incremental": round(wmed["incremental"][1], 2), "full": round(wmed["full"][1], 2),
                              "incremental_fused": round(wmed["fused"][1], 2)},
            "pieces_us (each with one dispatch gap)": {
                "pool_tail": round(inc[0], 2), "pool_full": round(full[0], 2), "scores": round(inc[1], 2),
                "pool_tail_and_scores_fused": round(med["fused"][0], 2),
                "select": round(inc[2], 2), "sparse_attention": round(inc[3], 2)},
            "attention_geometry": "r 512, n 256, v 256, rope 64, 64 heads, L 8 (GLM-5.3-Flash-like)",
            "samples": args.samples, "cache_state": "cold (512 MiB read scrub before each sample)"}), flush=True)
        del pool, keys, k_pe, scores, sel, q_lat, out
        torch.cuda.empty_cache()


def crossover(args):
    """Forced-path sweep on the GLM-4.7-Flash-like workload (r 512, n 192, v 256,
    rope 64, 32 heads, one sequence of 8192 positions): at each L, the absorbed
    call (fold + attention) and the materialised call (expand K/V + attention),
    interleaved sample by sample.  Each sample starts after a 512 MiB scrub write
    (inputs evicted from L2 and the Infinity Cache) and a device-side delay, so
    that the host has enqueued the whole call before the first event is passed:
    the event pair then measures device time only."""
    import torch
    import mla_speculative_decode_amd as mla
    from mla_speculative_decode_amd import synth

    w = synth.WORKLOADS["glm47_h32_kv8192_bf16"]
    dev = torch.device("cuda:0")
    scrub = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # device delay of about 2 ms (torch's spin kernel, calibrated here)
    torch.cuda._sleep(1000)
    e0.record()
    torch.cuda._sleep(1_000_000)
    e1.record()
    torch.cuda.synchronize()
    spin = int(1_000_000 * 2.0 / max(e0.elapsed_time(e1), 1e-3))
    geom = mla.Geom(w.r, w.n, w.v, w.rope, w.heads)
    rows = []
    for L in synth.SWEEP_L:
        x = synth.make_inputs(w, L=L)
        d = {k: torch.from_numpy(getattr(x, k)).to(torch.bfloat16).to(dev).contiguous()
             for k in ("q_nope", "q_pe", "c_kv", "k_pe", "w_uk", "w_uv")}
        offs = mla.Offsets(x.offsets.astype(np.int32), dev)
        T = int(x.offsets[-1])
        q_lat = torch.empty((1, L, w.heads, w.r), dtype=torch.bfloat16, device=dev)
        out_a = torch.empty((1, L, w.heads, w.v), dtype=torch.float32, device=dev)
        out_m = torch.empty_like(out_a)
        ws_a = torch.empty(max(256, mla.absorbed_workspace_size(geom, 1, L, offs)), dtype=torch.uint8, device=dev)
        gm = mla.Geom(1, w.n, w.v, w.rope, w.heads)
        ws_m = torch.empty(max(256, mla.materialized_workspace_size(gm, 1, L, offs)), dtype=torch.uint8, device=dev)
        K = torch.empty((T, w.heads, w.n + w.rope), dtype=torch.bfloat16, device=dev)
        V = torch.empty((T, w.heads, w.v), dtype=torch.bfloat16, device=dev)

        def absorbed():
            mla.fold_query(d["q_nope"], d["w_uk"], out=q_lat)
            mla.absorbed_attention(q_lat, d["q_pe"], d["c_kv"], d["k_pe"], d["w_uv"], offs, scale=x.scale,
                                   out=out_a, workspace=ws_a)

        def materialized():
            mla.materialize_kv(d["c_kv"], d["k_pe"], d["w_uk"], d["w_uv"], k=K, v=V)
            mla.materialized_attention(d["q_nope"], d["q_pe"], K, V, offs, scale=x.scale, out=out_m, workspace=ws_m)

        arms = {"absorbed": absorbed, "materialized": materialized}
        for f in arms.values():
            f()
            f()
        times = {a: [] for a in arms}
        for i in range(args.samples):
            order = ("absorbed", "materialized") if i % 2 == 0 else ("materialized", "absorbed")
            for a in order:
                scrub.fill_(i & 255)
                torch.cuda._sleep(spin)
                e0.record()
                arms[a]()
                e1.record()
                torch.cuda.synchronize()
                times[a].append(e0.elapsed_time(e1) * 1e3)
        diff = float(torch.max(torch.abs(out_a - out_m)))
        path, max_abs = mla.select_path(geom, L, T)
        med = {a: float(np.median(t)) for a, t in times.items()}
        row = {"crossover": w.name, "L": L, "T": T,
               "absorbed_us": round(med["absorbed"], 2), "materialized_us": round(med["materialized"], 2),
               "absorbed_us_min": round(min(times["absorbed"]), 2),
               "materialized_us_min": round(min(times["materialized"]), 2),
               "faster": min(med, key=med.get), "ratio_mat_over_abs": round(med["materialized"] / med["absorbed"], 3),
               "formula_path": "absorbed" if path == mla.MLA_ABSORBED else "materialized",
               "formula_max_absorbed": max_abs, "max_abs_diff_paths": diff, "samples": args.samples,
               "cache_state": "cold (512 MiB scrub before each sample)"}
        rows.append(row)
        print(json.dumps(row), flush=True)
        del d, q_lat, out_a, out_m, ws_a, ws_m, K, V
        torch.cuda.empty_cache()
    # measured crossover: between the last L where absorbed is faster and the first where it is not
    last_abs = max([r["L"] for r in rows if r["faster"] == "absorbed"], default=None)
    first_mat = min([r["L"] for r in rows if r["faster"] == "materialized"], default=None)
    print(json.dumps({"crossover_summary": w.name, "absorbed_faster_up_to_L": last_abs,
                      "materialized_faster_from_L": first_mat, "formula_max_absorbed": rows[0]["formula_max_absorbed"]}),
          flush=True)


def cpu_baseline(x, target_s: float):
    """The float64 oracle on the host cores, on a sample of the (row, head) pairs
    of the same workload, scaled to microseconds per whole call."""
    import oracle
    B, L, H = x.w.batch, x.L, x.w.heads
    total = B * L * H
    rng = np.random.default_rng(0)
    probe = np.sort(rng.choice(total, size=min(16, total), replace=False))
    t0 = time.perf_counter()
    oracle.absorbed(x.q_nope, x.q_pe, x.c_kv, x.k_pe, x.w_uk, x.w_uv, x.offsets, L, x.scale, sel=probe)
    per_row = (time.perf_counter() - t0) / probe.size
    k = int(min(total, max(probe.size, target_s / max(per_row, 1e-9))))
    sel = np.sort(rng.choice(total, size=k, replace=False))
    t0 = time.perf_counter()
    oracle.absorbed(x.q_nope, x.q_pe, x.c_kv, x.k_pe, x.w_uk, x.w_uv, x.offsets, L, x.scale, sel=sel)
    dt = time.perf_counter() - t0
    return {"value": round(dt / k * total * 1e6, 1), "unit": "us/call", "cores": oracle.max_threads(),
            "kind": "oracle",
            "sample": f"{k} of {total} (row, head) pairs of the same workload, timed {dt:.2f} s, "
                      f"scaled by {total / k:.2f}"}


if __name__ == "__main__":
    main()
