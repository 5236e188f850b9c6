#!/usr/bin/env python3
"""Benchmark of one decode step of paged low-rank-compressed attention on
one MI355X (q projection, split-K latent attention, combine, W_h
up-projection), the workload being batch 16 x 2048 cached tokens, 32 heads,
d = 128, r_k = 64 per head, joint r_v = 512, 16-token pages, fp16 storage.

    python bench.py [--steps K] [--warmup W] [--workload decode_b16] [--no-cpu]

Prints ONE JSON line.  Timing: every step is preceded (outside the timed
events) by a 512 MiB fill that evicts the 256 MB Infinity Cache, so each step
reads its latents from HBM; each step is bracketed by HIP events on the
stream the library launches on, and the split-K kernel alone by events the
library records around its launch.  `value` is latent-KV bytes per step /
mean step time.  The CPU leg times the fp64 oracle on a bounded sample of
the same workload on the host cores.

Other modes:
    --profile-run             a few steps plus a 256 MiB copy, for rocprofv3
    --summarize-pmc F W OUT   turn FETCH_SIZE / WRITE_SIZE counter CSVs into
                              the traffic summary the benchmark reads back
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-step attn ms + latent-KV HBM GB/s (% peak), 32h d128 r_k64 r_v512 fp16"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, AMD public specification
FLUSH_BYTES = 512 << 20        # > 2x the 256 MB Infinity Cache
COPY_BYTES = 256 << 20         # plain copy used to calibrate the HBM counters
DECODE_KERNEL = "decode_split_kernel"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_split_kernel_decode_b16_traffic.txt")
KERNEL_SOURCES = ["rank_compressed_paged_amd/csrc/decode.hip", "rank_compressed_paged_amd/csrc/common.h"]


def kernel_source_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(per_launch_algorithmic_bytes):
    """HBM bytes per launch from the committed counter summary, or None when
    the summary is missing or was taken on another version of the kernel."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.strip().split("=", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha") != kernel_source_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def parse_args(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode_b16",
                    choices=["decode_b16", "decode_b64", "long_b20", "tiny"])
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="CPU sample budget")
    ap.add_argument("--flush", choices=["read", "write"], default="read",
                    help="evict the Infinity Cache by reading (default) or writing 512 MiB")
    ap.add_argument("--profile-run", action="store_true")
    ap.add_argument("--summarize-pmc", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "OUT"))
    return ap.parse_args(argv)


def make_inputs(name):
    import numpy as np
    import torch
    from rank_compressed_paged_amd import workloads as wl
    case = wl.make_config(name)
    c = case.cache
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    t = dict(q=dev(case.q), k_cache=dev(c.k_cache), v_cache=dev(c.v_cache), U=dev(case.U),
             W=dev(case.W), block_tables=dev(c.block_tables), seq_lens=dev(c.seq_lens))
    return case, t


def cpu_baseline(case, budget_s):
    """The fp64 oracle, as it stands, on the first sequences of the same
    workload until about budget_s seconds of CPU work are spent."""
    import numpy as np
    import oracle
    from rank_compressed_paged_amd import metrics
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()
                       if p.get("user_api") == "blas"] or [1])
    except Exception:
        threads = int(os.environ.get("OMP_NUM_THREADS", "1"))
    c = case.cache
    sh = case.shape
    done, spent, tokens = 0, 0.0, 0
    while done < case.B and spent < budget_s:
        t0 = time.perf_counter()
        oracle.decode(case.q, c.k_cache, c.v_cache, case.U, case.W, c.block_tables,
                      c.seq_lens, case.scale, batch_indices=[done])
        spent += time.perf_counter() - t0
        tokens += int(c.seq_lens[done])
        done += 1
    lat = tokens * metrics.latent_bytes_per_token(sh.H, sh.r_k, sh.r_v)
    return {"value": round(lat / spent / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{done} of {case.B} sequences of one {case.name} step "
                      f"({tokens} cached tokens), {spent:.1f} s, fp64 numpy rebuild-then-attend",
            "ms_per_step_extrapolated": round(spent / done * case.B * 1e3, 1)}


def run_bench(args):
    import numpy as np
    import torch
    from rank_compressed_paged_amd import metrics
    from rank_compressed_paged_amd import starkv as sk

    case, t = make_inputs(args.workload)
    sh = case.shape
    B = case.B
    msl = int(case.cache.seq_lens.max())
    dims = sk.dims_of(t["k_cache"], t["v_cache"], t["U"], t["W"])
    ws = sk.alloc_workspace(sk.decode_workspace_size(dims, B, msl), "cuda")
    out = torch.empty((B, sh.H, sh.d), dtype=torch.float16, device="cuda")
    flush = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    flush_sink = torch.empty((), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def do_flush(i):
        # a read-only sweep leaves clean lines behind; a write sweep leaves
        # dirty ones whose write-back competes with the next step's reads
        if args.flush == "read":
            torch.sum(flush, dim=0, out=flush_sink)
        else:
            flush.fill_(float(i & 0xFF))
    lat_bytes = metrics.decode_latent_bytes(case.cache.seq_lens, sh.H, sh.r_k, sh.r_v)
    pps, ns = sk.decode_plan(dims, B, msl)

    def step():
        sk.decode_attn(t["q"], t["k_cache"], t["v_cache"], t["U"], t["W"], t["block_tables"],
                       t["seq_lens"], msl, case.scale, out=out, workspace=ws)

    # append of the step's B new tokens (second row, reported beside the headline)
    rng = np.random.default_rng(123)
    k_new = torch.from_numpy(rng.standard_normal((B, sh.H, sh.d), dtype=np.float32)
                             .astype(np.float16)).cuda()
    v_new = torch.from_numpy(rng.standard_normal((B, sh.H, sh.d), dtype=np.float32)
                             .astype(np.float16)).cuda()
    nb_app = (B + sh.bs - 1) // sh.bs    # a separate cache: the timed appends leave the step's input alone
    kc_app = torch.zeros((nb_app, sh.H, sh.bs, sh.r_k), dtype=torch.float16, device="cuda")
    vc_app = torch.zeros((nb_app, sh.r_v, sh.bs), dtype=torch.float16, device="cuda")
    slots = torch.arange(B, dtype=torch.int64, device="cuda")

    def append_step():
        sk.append(k_new, v_new, t["U"], t["W"], slots, kc_app, vc_app)

    def timed(fn, n, flushed, kernel_sel=sk.TIME_NONE):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(n)]
        kev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n)]
        for a, b in kev:   # materialise the HIP events before handing them over
            a.record()
            b.record()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(n):
            if flushed:
                do_flush(i)
            if kernel_sel:
                sk.set_timing_events(kev[i][0], kev[i][1], kernel_sel)
            ev[i][0].record(stream)
            fn()
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        sk.set_timing_events(None, None, sk.TIME_NONE)
        steps_ms = [a.elapsed_time(b) for a, b in ev]
        kern_ms = [a.elapsed_time(b) for a, b in kev] if kernel_sel else []
        return steps_ms, kern_ms, wall

    # warmup (untimed)
    for i in range(args.warmup):
        do_flush(i)
        step()
    torch.cuda.synchronize()

    # headline: whole steps, cache flushed before each, no events inside the step
    step_ms, _, wall = timed(step, args.steps, True)
    # the split-K kernel alone (events recorded around its launch), flushed
    _, kern_ms, _ = timed(step, args.steps, True, sk.TIME_DECODE_SPLIT)
    # warm (latents left in the Infinity Cache), for reference only
    warm_ms, _, _ = timed(step, args.steps, False)
    _, warm_kern_ms, _ = timed(step, args.steps, False, sk.TIME_DECODE_SPLIT)
    app_ms, _, _ = timed(append_step, max(args.steps, 10), True)
    _, app_kern_ms, _ = timed(append_step, max(args.steps, 10), True, sk.TIME_APPEND)

    # measured streaming-read ceiling on this machine: the library's plain
    # 16-byte streaming read over as many bytes as one step's latents, after
    # the same flush
    ceil_buf = torch.ones(lat_bytes, dtype=torch.uint8, device="cuda")
    ceil_sink = torch.zeros(1024, dtype=torch.int32, device="cuda")
    ceil_ms, _, _ = timed(lambda: sk.stream_read(ceil_buf, ceil_sink), max(args.steps, 10), True)
    ceiling_gbs = lat_bytes / (statistics.fmean(ceil_ms) * 1e-3) / 1e9
    del ceil_buf

    ms = statistics.fmean(step_ms)
    kern = statistics.fmean(kern_ms)
    value = lat_bytes / (ms * 1e-3) / 1e9
    achieved = lat_bytes / (kern * 1e-3) / 1e9
    traffic = read_traffic(lat_bytes)
    q = lambda xs, p: sorted(xs)[min(len(xs) - 1, int(round(p * (len(xs) - 1))))]
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": case.name, "batch": B, "seq_len": msl, "heads": sh.H,
                   "head_dim": sh.d, "rank_k": sh.r_k, "rank_v": sh.r_v,
                   "block_size": sh.bs, "parallelism": "none"},
        "pct_peak_hbm": round(100.0 * value / HBM_PEAK_GBS, 2),
        "latent_bytes_per_step": int(lat_bytes),
        "step_ms_median": round(statistics.median(step_ms), 5),
        "step_ms_p10": round(q(step_ms, 0.1), 5),
        "step_ms_p90": round(q(step_ms, 0.9), 5),
        "warm_step_ms": round(statistics.fmean(warm_ms), 5),
        "warm_split_kernel_ms": round(statistics.fmean(warm_kern_ms), 5),
        "append_step_ms": round(statistics.fmean(app_ms), 5),
        "append_kernel_ms": round(statistics.fmean(app_kern_ms), 5),
        "wall_s_timed_loop_incl_flush": round(wall, 4),
        "split_plan": {"pages_per_split": pps, "num_splits": ns},
        "flush": args.flush,
        "stream_read_ceiling_gbs": round(ceiling_gbs, 1),
        "roofline": {
            "kernel": DECODE_KERNEL,
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel_ms": round(kern, 5),
            "algorithmic_bytes_per_launch": int(lat_bytes),
        },
    }
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


def profile_run(args):
    """A short run for rocprofv3: warm steps of the workload, then a plain
    COPY_BYTES device copy used to calibrate FETCH_SIZE / WRITE_SIZE."""
    import torch
    from rank_compressed_paged_amd import starkv as sk
    case, t = make_inputs(args.workload)
    msl = int(case.cache.seq_lens.max())
    dims = sk.dims_of(t["k_cache"], t["v_cache"], t["U"], t["W"])
    ws = sk.alloc_workspace(sk.decode_workspace_size(dims, case.B, msl), "cuda")
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
    for _ in range(max(args.steps, 1)):
        flush.fill_(1)
        sk.decode_attn(t["q"], t["k_cache"], t["v_cache"], t["U"], t["W"], t["block_tables"],
                       t["seq_lens"], msl, case.scale, workspace=ws)
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(3)
    dst = torch.empty_like(src)
    for _ in range(3):
        flush.fill_(2)
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"profile-run done: {args.steps} steps of {case.name}, 3 copies of {COPY_BYTES} B",
          flush=True)


def _pmc_rows(path):
    with open(path) as f:
        return list(csv.DictReader(f))


def summarize_pmc(fetch_csv, write_csv, out_path):
    """Average FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the split-K
    kernel and of the plain copy; scale each by the copy's bytes-per-KiB."""
    from rank_compressed_paged_amd import metrics, workloads as wl
    def avg(rows, counter, match):
        vals = [float(r["Counter_Value"]) for r in rows
                if match(r["Kernel_Name"]) and r["Counter_Name"] == counter]
        return sum(vals) / len(vals) if vals else float("nan"), len(vals)
    is_split = lambda n: DECODE_KERNEL in n
    is_copy = lambda n: ("copy" in n.lower() or "elementwise" in n.lower()) and "fill" not in n.lower()
    fr, wr = _pmc_rows(fetch_csv), _pmc_rows(write_csv)
    f_split, nf = avg(fr, "FETCH_SIZE", is_split)
    w_split, nw = avg(wr, "WRITE_SIZE", is_split)
    f_copy, _ = avg(fr, "FETCH_SIZE", is_copy)
    w_copy, _ = avg(wr, "WRITE_SIZE", is_copy)
    f_scale = COPY_BYTES / f_copy          # bytes per counted KiB, reads
    w_scale = COPY_BYTES / w_copy          # bytes per counted KiB, writes
    case = wl.CONFIGS["decode_b16"]
    lat = 16 * 2048 * metrics.latent_bytes_per_token(32, 64, 512)
    hbm = f_split * f_scale + w_split * w_scale
    with open(out_path, "w") as f:
        f.write("# HBM traffic of the split-K decode kernel, decode_b16 (batch 16 x 2048, H32 d128 r_k64 r_v512)\n")
        f.write("# FETCH_SIZE and WRITE_SIZE from two rocprofv3 --pmc runs of `bench.py --profile-run`,\n")
        f.write("# each scaled by the same counter on a plain copy of COPY_BYTES bytes.\n")
        f.write(f"kernel_source_sha={kernel_source_hash()}\n")
        f.write(f"dispatches_fetch={nf}\ndispatches_write={nw}\n")
        f.write(f"fetch_kib_per_dispatch={f_split:.1f}\nwrite_kib_per_dispatch={w_split:.1f}\n")
        f.write(f"copy_bytes={COPY_BYTES}\ncopy_fetch_kib={f_copy:.1f}\ncopy_write_kib={w_copy:.1f}\n")
        f.write(f"fetch_scale_bytes_per_kib={f_scale:.2f}\nwrite_scale_bytes_per_kib={w_scale:.2f}\n")
        f.write(f"hbm_bytes_per_launch={hbm:.0f}\nalgorithmic_bytes_per_launch={lat}\n")
        f.write(f"traffic_over_algorithmic={hbm / lat:.3f}\n")
    print(open(out_path).read())


def main():
    args = parse_args()
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return 0
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU: the decode path has "
                                   "no cross-GPU step (sequences shard with zero exchange); run "
                                   "with --gpus 1"}), flush=True)
        return 2
    if args.profile_run:
        profile_run(args)
        return 0
    run_bench(args)
    return 0


if __name__ == "__main__":
    sys.exit(main())
