#!/usr/bin/env python3
"""Absorbed MLA verify step on one MI355X: microseconds per call and
latent-cache bandwidth, with the roofline of the dominant kernel and the
float64 CPU oracle timed beside it.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one whole absorbed verify call over one batch of synthetic inputs
already resident in device memory: mla_fold_query (q_lat = q_nope . W_UK),
mla_absorbed_splits (split-KV latent attention) and mla_absorbed_merge
(log-sum-exp merge and W_UV up-projection).  Default workload: DeepSeek-V3
MLA geometry (r 512, n 128, v 128, rope 64), 128 heads, one sequence with a
cache of 8192 positions, L = 8 query rows, bf16 storage, fp32 accumulation.

Input sets are cloned on the device and rotated step by step so that the
data of a step has been evicted from L2 and the 256 MB Infinity Cache before
it is reused (cold); a warm variant reuses one set.  Prints one JSON line.
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
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E

# HBM traffic of the split kernel per launch, from rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE
# (KiB per dispatch) scaled by what the same counters read for a plain 256 MiB device copy
# (FETCH x2.00, WRITE x1.00); valid only for the kernel source it was measured on.
SPLIT_TRAFFIC = {"source_sha256": "6db54ddfce32115cc3071eea063749ffa152369664d5846d13d1b8befac0d50e",
                 "fetch_kib": 9360.2, "write_kib": 16512.0, "fetch_factor": 2.0, "write_factor": 1.0}
KERNEL_SOURCES = ("mla_speculative_decode_amd/csrc/attn.hip", "mla_speculative_decode_amd/csrc/mla_device.h")


def split_traffic_bytes():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    t = SPLIT_TRAFFIC
    if h.hexdigest() != t["source_sha256"]:
        return None   # the kernel changed since the counters were taken
    return round(1024 * (t["fetch_kib"] * t["fetch_factor"] + t["write_kib"] * t["write_factor"]))


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="dsv3_h128_kv8192_l8_bf16")
    ap.add_argument("--cold-bytes", type=float, default=768e6,
                    help="total bytes of rotated input sets (cold protocol); 0 = warm only")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (counter calibration) and exit")
    return ap.parse_args()


def main():
    args = parse()
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
    lib = _lib.load()
    blib = ctypes.CDLL(os.path.join(ROOT, "mla_speculative_decode_amd", "libmla_bench.so"))
    blib.mlab_absorbed_run.restype = ctypes.c_int

    w = synth.WORKLOADS[args.workload]
    if w.dtype != "bf16":
        raise SystemExit("bench.py times the bf16 path")
    x = synth.make_inputs(w)
    B, L, H = w.batch, x.L, w.heads
    dev = torch.device("cuda:0")

    def up(a):
        return torch.from_numpy(a).to(torch.bfloat16).to(dev).contiguous()

    base = {k: up(getattr(x, k)) for k in ("q_nope", "q_pe", "c_kv", "k_pe", "w_uk", "w_uv")}
    set_bytes = sum(t.numel() * t.element_size() for t in base.values())
    nsets = max(1, int(math.ceil(args.cold_bytes / set_bytes))) if args.cold_bytes > 0 else 1
    sets = [base] + [{k: t.clone() for k, t in base.items()} for _ in range(nsets - 1)]
    for s in sets:
        s["q_lat"] = torch.empty((B, L, H, w.r), dtype=torch.bfloat16, device=dev)
        s["out"] = torch.empty((B, L, H, w.v), dtype=torch.float32, device=dev)
    offs = mla.Offsets(x.offsets.astype(np.int32), dev)
    geom = mla.Geom(w.r, w.n, w.v, w.rope, H)
    ws_bytes = mla.absorbed_workspace_size(geom, _lib.MLA_BF16, L, offs)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.Stream()

    def ptrs(key, idx):
        arr = (ctypes.c_void_p * len(idx))(*[sets[i][key].data_ptr() for i in idx])
        return arr

    def run(idx, steps, warmup):
        res = (ctypes.c_double * 6)()
        torch.cuda.synchronize()
        rc = blib.mlab_absorbed_run(
            ctypes.byref(geom), B, L, len(idx), ptrs("q_nope", idx), ptrs("q_pe", idx), ptrs("c_kv", idx),
            ptrs("k_pe", idx), ptrs("w_uk", idx), ptrs("w_uv", idx), ptrs("q_lat", idx), ptrs("out", idx),
            offs.host_ptr(), offs.dev_ptr(), ctypes.c_float(x.scale), ctypes.c_void_p(ws.data_ptr()),
            ctypes.c_size_t(ws_bytes), ctypes.c_void_p(stream.cuda_stream), warmup, steps, res)
        torch.cuda.synchronize()
        if rc != 0:
            raise RuntimeError(f"bench step failed: {lib.mla_status_string(rc).decode()}")
        return list(res)

    # timed region: W untimed steps, then K steps between synchronisations
    t0 = time.perf_counter()
    cold = run(list(range(nsets)), args.steps, args.warmup)
    wall = time.perf_counter() - t0
    warm = run([0], args.steps, args.warmup)

    # algorithmic work of one call
    lens = np.diff(x.offsets)
    vis = sum(int(H * (kv * L - L * (L - 1) // 2)) for kv in lens)          # sum over rows of visible positions
    attn_flop = 2.0 * (2 * w.r + w.rope) * vis                            # scores (r+rope) + latent PV (r)
    cache_bytes = float(lens.sum() * (w.r + w.rope) * 2)
    weight_bytes = float(2 * H * w.n * w.r * 2)                            # W_UK + W_UV, bf16
    us_step, us_fold, us_split, us_merge, us_evented, us_split_b2b = cold
    # roofline of the split kernel: its launches back to back (per-launch duration
    # without the dispatch gap that an event pair around one launch also measures)
    achieved_tflops = attn_flop / (us_split_b2b * 1e-6) / 1e12

    line = {
        "metric": METRIC,
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
                   "kv": int(lens.max()), "L": L, "cache_state": f"cold ({nsets} rotated input sets)"},
        "latent_cache_GBps": round(cache_bytes / (us_split_b2b * 1e-6) / 1e9, 1),
        "step_GBps": round((cache_bytes + weight_bytes) / (us_step * 1e-6) / 1e9, 1),
        "per_launch_us": {"fold": round(us_fold, 3), "splits": round(us_split, 3), "merge": round(us_merge, 3),
                          "splits_back_to_back": round(us_split_b2b, 3)},
        "warm_us_per_call": round(warm[0], 3),
        "warm_per_launch_us": {"fold": round(warm[1], 3), "splits": round(warm[2], 3), "merge": round(warm[3], 3)},
        "roofline": {"kernel": "attn_bf16_kernel (mla_absorbed_splits)", "bound": "mfma",
                     "duration_us": round(us_split_b2b, 3),
                     "achieved": round(achieved_tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved_tflops / PEAK_BF16_TFLOPS, 4), "traffic": split_traffic_bytes()},
        "wall_s": round(wall, 3),
    }

    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(x, args.cpu_seconds)
    print(json.dumps(line), flush=True)


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
