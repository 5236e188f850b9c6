#!/usr/bin/env python3
"""Benchmark of one decode step of paged low-rank-compressed attention on
one MI355X (q projection, split-K latent attention, the merge of the
splits with the W_h up-projection), the workload being batch 16 x 2048 cached tokens, 32 heads,
d = 128, r_k = 64 per head, joint r_v = 512, 16-token pages, fp16 storage.

    python bench.py [--steps K] [--warmup W] [--workload decode_b16] [--no-cpu]

Prints ONE JSON line.  By default 20 untimed warm-up steps, then 200 timed
ones (the median, p10 and p90 are reported beside the mean).  Timing: every
step is preceded (outside the timed
events) by a 512 MiB read sweep that evicts the 256 MB Infinity Cache, so
each step reads its latents from HBM; each step is bracketed by HIP events on
the stream the library launches on.  The split-K kernel alone is timed by
events that take its dispatch's own begin and end timestamps.  `value` is
latent-KV bytes per step / mean step time.  Beside the headline the line
carries the step with its append, a streaming-read ceiling, the chunked
prefill workload (16 requests x 4096 cached + 256 new tokens: attention and
append, as TFLOP/s against the fp16 MFMA peak; also over FP8 caches, and at
the conservative ranks r_k 128, r_v 1024 on the generic kernels), the append at 16 to 4096
tokens, the other fp16 decode
configurations of the same shape (decode_b64, long_b20, tiny), decode at other
layouts (gqa8_b16: 32 query heads on 8 key/value heads; lowrank_b16: r_k
32, r_v 256; decode_b16_fp8 and decode_b64_fp8: FP8 E4M3 latents), low-batch
decode latency (batch 1-4: eager calls against a captured HIP graph), the bases
fit from 16384
K/V samples (its Gram kernel against the same peak), and the CPU leg, which
times the fp64 oracle on a bounded sample of the decode workload on the host
cores.

Other modes:
    --profile-run             a few steps plus a 256 MiB copy, for rocprofv3
    --summarize-pmc F W OUT   turn FETCH_SIZE / WRITE_SIZE counter CSVs into
                              the traffic summary the benchmark reads back
    --plan-sweep              decode step and split kernel at forced split
                              plans (pages per split, and with --sweep-merge
                              finish-kernel tiles) beside the planner's own,
                              one JSON line per plan
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
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 MFMA, AMD public specification
FLUSH_BYTES = 512 << 20        # > 2x the 256 MB Infinity Cache
COPY_BYTES = 256 << 20         # plain copy used to calibrate the HBM counters
DECODE_KERNEL = "decode_split_kernel"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_split_kernel_decode_b16_traffic.txt")
TRAFFIC_WORKLOAD = "decode_b16"
SPLIT_SECTION = ("// 2. split-K latent attention", "// 3. finish")
LAUNCH_DECODE = "hipError_t launch_decode("


def kernel_source_hash():
    """Hash of the split-K kernel's device code (its section of decode.hip),
    of the launcher that picks its instance, and of the shared device
    helpers: the traffic summary is only used while this matches the code
    the counters were taken on."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "rank_compressed_paged_amd", "csrc")
    with open(os.path.join(csrc, "decode.hip")) as f:
        text = f.read()
    a, b = text.index(SPLIT_SECTION[0]), text.index(SPLIT_SECTION[1])
    h.update(text[a:b].encode())
    h.update(text[text.index(LAUNCH_DECODE):].encode())
    with open(os.path.join(csrc, "common.h"), "rb") as f:
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
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode_b16",
                    choices=["decode_b16", "decode_b64", "long_b20", "tiny"])
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill_b16 leg")
    ap.add_argument("--no-fit", action="store_true", help="skip the bases-fit leg")
    ap.add_argument("--no-low-batch", action="store_true", help="skip the low-batch latency leg")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the decode_b64, long_b20 and tiny legs")
    ap.add_argument("--no-layouts", action="store_true",
                    help="skip the grouped-query and low-rank decode legs")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="CPU sample budget")
    ap.add_argument("--cpu-prefill-seconds", type=float, default=5.0,
                    help="CPU sample budget of the prefill leg's oracle baseline")
    ap.add_argument("--flush", choices=["read", "write"], default="read",
                    help="evict the Infinity Cache by reading (default) or writing 512 MiB")
    ap.add_argument("--profile-run", action="store_true")
    ap.add_argument("--profile-fit", action="store_true",
                    help="a few bases fits (fit_n16384, 8 iterations), for rocprofv3")
    ap.add_argument("--summarize-pmc", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "OUT"))
    ap.add_argument("--plan-sweep", action="store_true",
                    help="decode steps at forced pages_per_split values (JSON line per plan)")
    ap.add_argument("--sweep-workloads", default="decode_b16,decode_b64,long_b20",
                    help="workloads of --plan-sweep")
    ap.add_argument("--sweep-pps", default="4,6,8,9,12,16,32,64,128",
                    help="pages_per_split values of --plan-sweep (0 = the planner's)")
    ap.add_argument("--sweep-merge", default="",
                    help="merge_seqs values of --plan-sweep, each at the planner's split plan "
                         "(0 = the planner's)")
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


def host_cpu_info():
    """The host the CPU oracle runs on: the cores this process may use, the
    CPU model, and numpy's BLAS library with its thread count (the oracle's
    matrix products run there)."""
    info = {"affinity_cores": len(os.sched_getaffinity(0)), "cpu_model": None,
            "blas": None, "blas_threads": int(os.environ.get("OMP_NUM_THREADS", "1"))}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    info["cpu_model"] = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if blas:
            info["blas"] = f"{blas[0].get('internal_api')} {blas[0].get('version')}"
            info["blas_threads"] = int(max(p.get("num_threads", 1) for p in blas))
    except Exception:
        pass
    return info


def cpu_baseline(case, budget_s):
    """The fp64 oracle, as it stands, on the first sequences of the same
    workload until about budget_s seconds of CPU work are spent."""
    import numpy as np
    import oracle
    from rank_compressed_paged_amd import metrics
    host = host_cpu_info()
    threads = host["blas_threads"]
    c = case.cache
    sh = case.shape
    done, spent, tokens = 0, 0.0, 0
    # whole sequences, cycling over the batch, until the budget is spent
    while spent < budget_s or done < 1:
        b = done % case.B
        t0 = time.perf_counter()
        oracle.decode(case.q, c.k_cache, c.v_cache, case.U, case.W, c.block_tables,
                      c.seq_lens, case.scale, batch_indices=[b])
        spent += time.perf_counter() - t0
        tokens += int(c.seq_lens[b])
        done += 1
    lat = tokens * metrics.latent_bytes_per_token(sh.H, sh.r_k, sh.r_v)
    return {"value": round(lat / spent / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle", "host": host,
            "sample": f"{done} sequence decodes cycling over the {case.B} sequences of one "
                      f"{case.name} step ({tokens} cached tokens, {done / case.B:.1f} steps' "
                      f"worth), {spent:.1f} s, fp64 numpy rebuild-then-attend",
            "ms_per_step_extrapolated": round(spent / tokens * int(c.seq_lens.sum()) * 1e3, 1)}


def settle(fn, flush_fn=None, seconds=0.2):
    """Run fn (each call after flush_fn) for about `seconds` of GPU time.
    Matrix-core-heavy kernels start up to about 30% slower and take some tens
    of milliseconds of sustained load to reach their steady clock (the
    prefill kernel's per-dispatch durations in a kernel trace fall from about
    0.85 ms to 0.65 ms over its first ~50 calls); timing starts after that.
    Memory-bound kernels show no such ramp."""
    import torch
    t0 = time.perf_counter()
    i = 0
    while True:
        for _ in range(8):
            if flush_fn is not None:
                flush_fn(i)
            fn()
            i += 1
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return i


# GPU work enqueued ahead of every timed loop (set by run_bench): the host
# then enqueues the loop's calls while the GPU is still busy with it, so no
# call's events ever wait for the host to launch its kernels.  Without it a
# short call (the few-token append: about 9 us of kernels after a 75 us
# flush) read 35-48 us, the host's Python launch path included.
HEAD_START = {"fn": None}


def timed(fn, n, flush_fn=None, kernel_sel=0):
    """Run fn n times, each optionally after flush_fn (outside the events).
    Returns per-call ms from events around the call on the current stream,
    per-call ms of one kernel through the library's timing hook (when
    kernel_sel selects one: the library's timing events, bound to that
    dispatch and recorded without a system-scope fence), and the wall time of
    the loop (which includes the head start)."""
    import torch
    from rank_compressed_paged_amd import starkv as sk
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    kev = [(sk.TimingEvent(), sk.TimingEvent()) for _ in range(n)] if kernel_sel else []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if HEAD_START["fn"] is not None:
        HEAD_START["fn"](n)
    for i in range(n):
        if flush_fn is not None:
            flush_fn(i)
        if kernel_sel:
            sk.set_timing_events(kev[i][0], kev[i][1], kernel_sel)
        ev[i][0].record(stream)
        fn()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    sk.set_timing_events(None, None, sk.TIME_NONE)
    steps_ms = [a.elapsed_time(b) for a, b in ev]
    kern_ms = [a.elapsed_ms(b) for a, b in kev]
    return steps_ms, kern_ms, wall


def stream_ceiling_gbs(nbytes, flush_fn, steps):
    """The streaming-read ceiling at nbytes: a plain read (16-byte
    non-temporal loads, 16 in flight per thread) of that many bytes after the
    same flush, timed like the split kernel (the library's events, from the
    end of the dispatch before it to the end of its own)."""
    import torch
    from rank_compressed_paged_amd import starkv as sk
    buf = torch.ones(int(nbytes) // 16 * 16, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1024, dtype=torch.int32, device="cuda")
    for i in range(3):
        flush_fn(i)
        sk.stream_read(buf, sink)
    torch.cuda.synchronize()
    _, kern_ms, _ = timed(lambda: sk.stream_read(buf, sink), steps, flush_fn, sk.TIME_STREAM_READ)
    gbs = buf.numel() / (statistics.fmean(kern_ms) * 1e-3) / 1e9
    del buf
    return gbs


def rocminfo_gpu():
    """Marketing name, maximum engine clock and compute units of the first
    GPU agent as rocminfo prints them (empty when rocminfo is unavailable)."""
    import subprocess
    try:
        txt = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=60).stdout
    except Exception:
        return {}
    for agent in txt.split("*******")[1:]:
        if "Device Type:             GPU" not in agent and "Device Type: GPU" not in " ".join(agent.split()):
            continue
        info = {}
        for line in agent.splitlines():
            key, _, val = line.strip().partition(":")
            val = val.strip()
            if key == "Marketing Name" and val:
                info["marketing_name"] = val
            elif key == "Max Clock Freq. (MHz)" and val.isdigit():
                info["max_clock_mhz"] = int(val)
            elif key == "Compute Unit" and val.isdigit():
                info["rocminfo_compute_units"] = int(val)
        if info:
            return info
    return {}


def device_info():
    import torch
    p = torch.cuda.get_device_properties(0)
    d = {"name": p.name, "arch": getattr(p, "gcnArchName", ""),
         "compute_units": p.multi_processor_count,
         "hbm_gib": round(p.total_memory / 2**30, 1)}
    d.update(rocminfo_gpu())
    return d


def cpu_prefill_baseline(pc, budget_s):
    """The fp64 oracle, as it stands, on whole requests of the same prefill
    workload (each request's chunk appended by the oracle first, untimed)
    until about budget_s seconds of prefill attention are spent; algorithmic
    TFLOP/s, the unit of the GPU prefill figures."""
    import numpy as np
    import oracle
    from rank_compressed_paged_amd import metrics
    host = host_cpu_info()
    threads = host["blas_threads"]
    sh, c = pc.shape, pc.cache
    qsl = pc.query_start_loc
    B = len(qsl) - 1
    done, spent, flops = 0, 0.0, 0
    kc, vc = c.k_cache, c.v_cache
    while spent < budget_s or done < 1:
        b = done % B
        rows = slice(int(qsl[b]), int(qsl[b + 1]))
        kc, vc = oracle.append(pc.k_new[rows], pc.v_new[rows], pc.U, pc.W, pc.slot_mapping[rows],
                               kc, vc)
        t0 = time.perf_counter()
        oracle.prefill(pc.q, qsl, kc, vc, pc.U, pc.W, c.block_tables, c.seq_lens, pc.scale,
                       request_indices=[b])
        spent += time.perf_counter() - t0
        flops += metrics.prefill_flops(pc.cached_lens[b:b + 1], np.diff(qsl)[b:b + 1], sh.H, sh.d,
                                       sh.r_k, sh.r_v)
        done += 1
    total = metrics.prefill_flops(pc.cached_lens, np.diff(qsl), sh.H, sh.d, sh.r_k, sh.r_v)
    return {"value": round(flops / spent / 1e12, 5), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "host": host,
            "sample": f"{done} whole requests of the {B} of one {pc.name} call "
                      f"({done / B:.2f} calls' worth), {spent:.1f} s, fp64 numpy "
                      f"rebuild-then-attend",
            "ms_per_call_extrapolated": round(spent / flops * total * 1e3, 1)}


def prefill_leg(flush_fn, steps, name="prefill_b16", cpu_budget_s=0.0, upproj_in_kernel=True):
    """Chunked prefill at 16 requests x (4096 cached + 256 new) tokens: the
    chunk's append (4096 tokens), then causal attention for the 4096 chunk
    queries (prefill_b16; prefill_b16_fp8 the same over FP8 caches;
    conservative_prefill_b16 at r_k 128, r_v 1024 on the generic kernels).
    upproj_in_kernel: the attention kernel applies the up-projection in its
    epilogue, so its algorithmic flops include it.  Reports time, algorithmic
    TFLOP/s and the fraction of the dense fp16 MFMA peak for the attention
    kernel and for the append."""
    import numpy as np
    import torch
    from rank_compressed_paged_amd import metrics
    from rank_compressed_paged_amd import starkv as sk
    from rank_compressed_paged_amd import workloads as wl
    pc = wl.make_config(name)
    sh, c = pc.shape, pc.cache
    fp8 = c.k_cache.dtype == np.uint8
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    q, k_new, v_new = dev(pc.q), dev(pc.k_new), dev(pc.v_new)
    U, W = dev(pc.U), dev(pc.W)
    kc, vc = dev(c.k_cache), dev(c.v_cache)
    bt, sl = dev(c.block_tables), dev(c.seq_lens)
    qsl, slots = dev(pc.query_start_loc), dev(pc.slot_mapping)
    chunk = np.diff(pc.query_start_loc)
    T, B = int(chunk.sum()), len(chunk)
    mql, msl = int(chunk.max()), int(c.seq_lens.max())
    dims = sk.dims_of(kc, vc, U, W)
    ws = sk.alloc_workspace(sk.prefill_workspace_size(dims, B, T, msl), "cuda")
    out = torch.empty((T, sh.H, sh.d), dtype=torch.float16, device="cuda")

    ws_app = sk.alloc_workspace(sk.append_workspace_size(dims, T), "cuda")

    def app():   # same slots each time: idempotent
        if fp8:
            sk.append_fp8(k_new, v_new, U, W, slots, pc.k_scale, pc.v_scale, kc, vc,
                          workspace=ws_app)
        else:
            sk.append(k_new, v_new, U, W, slots, kc, vc, workspace=ws_app)

    def attn():
        if fp8:
            sk.prefill_attn_fp8(q, qsl, mql, kc, vc, U, W, bt, sl, msl, pc.k_scale, pc.v_scale,
                                pc.scale, out=out, workspace=ws)
        else:
            sk.prefill_attn(q, qsl, mql, kc, vc, U, W, bt, sl, msl, pc.scale, out=out,
                            workspace=ws)

    app()
    settle(attn, flush_fn, 0.25)
    n = max(steps // 2, 10)
    attn_ms, _, _ = timed(attn, n, flush_fn)
    _, attn_kern_ms, _ = timed(attn, n, flush_fn, sk.TIME_PREFILL_ATTN)
    app_ms, _, _ = timed(app, n, flush_fn)
    _, app_kern_ms, _ = timed(app, n, flush_fn, sk.TIME_APPEND)
    flops = metrics.prefill_flops(pc.cached_lens, chunk, sh.H, sh.d, sh.r_k, sh.r_v)
    pairs = metrics.prefill_pairs(pc.cached_lens, chunk)
    # the kernel's share: scores + P.c_v, and the up-projection when the
    # kernel applies it in its epilogue (the main-shape instances)
    kern_flops = 2 * sh.H * pairs * (sh.r_k + sh.r_v)
    if upproj_in_kernel:
        kern_flops += 2 * sh.H * T * sh.r_v * sh.d
    app_flops = metrics.append_flops(T, sh.H, sh.d, sh.r_k, sh.r_v)
    app_bytes = (2 * T * sh.H * sh.d * 2 + T * 8 + metrics.basis_bytes(sh.H, sh.d, sh.r_k, sh.r_v)
                 + T * metrics.latent_bytes_per_token(sh.H, sh.r_k, sh.r_v))
    m = statistics.fmean
    tf = lambda f, ms: f / (ms * 1e-3) / 1e12
    return {
        "workload": name, "requests": B, "cached": int(pc.cached_lens[0]),
        "chunk": int(chunk[0]), "steps": n,
        "attn_call_ms": round(m(attn_ms), 4),
        "attn_call_tflops": round(tf(flops, m(attn_ms)), 1),
        "attn_call_mfma_frac": round(tf(flops, m(attn_ms)) / MFMA_F16_PEAK_TFLOPS, 4),
        "attn_kernel_ms": round(m(attn_kern_ms), 4),
        "attn_kernel_tflops": round(tf(kern_flops, m(attn_kern_ms)), 1),
        "attn_kernel_mfma_frac": round(tf(kern_flops, m(attn_kern_ms)) / MFMA_F16_PEAK_TFLOPS, 4),
        "algorithmic_gflop_call": round(flops / 1e9, 1),
        "algorithmic_gflop_kernel": round(kern_flops / 1e9, 1),
        "kernel_includes_upprojection": bool(upproj_in_kernel),
        "append_tokens": T,
        "append_call_ms": round(m(app_ms), 4),
        "append_kernel_ms": round(m(app_kern_ms), 4),
        "append_kernel_tflops": round(tf(app_flops, m(app_kern_ms)), 1),
        "append_kernel_mfma_frac": round(tf(app_flops, m(app_kern_ms)) / MFMA_F16_PEAK_TFLOPS, 4),
        "append_kernel_gbs": round(app_bytes / (m(app_kern_ms) * 1e-3) / 1e9, 1),
        "cpu_baseline": cpu_prefill_baseline(pc, cpu_budget_s) if cpu_budget_s > 0 else None,
    }


def decode_leg(name, flush_fn, steps):
    """Decode on another workload: the other fp16 configurations of the main
    shape (decode_b64: 64 x U{4096..8192} tokens; long_b20: 20 x 32768; tiny:
    the small parity shape), or another layout of 16 x 2048 tokens: gqa8_b16
    (32 query heads on 8 key/value heads, r_k 64, r_v 512: 2048 latent bytes
    per token), lowrank_b16 (r_k 32, r_v 256: 2560 bytes per token) and the
    FP8 caches.  Flushed steps (events around the call) and the split-K
    kernel (the library's timing events), as latent GB/s against the 8 TB/s
    peak."""
    import numpy as np
    import torch
    from rank_compressed_paged_amd import metrics
    from rank_compressed_paged_amd import starkv as sk
    from rank_compressed_paged_amd import workloads as wl
    case = wl.make_config(name)
    sh, c = case.shape, case.cache
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    q, kc, vc, U, W = dev(case.q), dev(c.k_cache), dev(c.v_cache), dev(case.U), dev(case.W)
    bt, sl = dev(c.block_tables), dev(c.seq_lens)
    B, msl = case.B, int(c.seq_lens.max())
    dims = sk.dims_of(kc, vc, U, W, num_heads=sh.H)
    ws = sk.alloc_workspace(sk.decode_workspace_size(dims, B, msl), "cuda")
    out = torch.empty((B, sh.H, sh.d), dtype=torch.float16, device="cuda")
    fp8 = c.k_cache.dtype == np.uint8

    def step():
        if fp8:
            sk.decode_attn_fp8(q, kc, vc, U, W, bt, sl, msl, case.k_scale, case.v_scale,
                               case.scale, out=out, workspace=ws)
        else:
            sk.decode_attn(q, kc, vc, U, W, bt, sl, msl, case.scale, out=out, workspace=ws)

    for i in range(5):
        flush_fn(i)
        step()
    torch.cuda.synchronize()
    step_ms, _, _ = timed(step, steps, flush_fn)
    _, kern_ms, _ = timed(step, steps, flush_fn, sk.TIME_DECODE_SPLIT)
    lat = metrics.decode_latent_bytes(c.seq_lens, sh.kv, sh.r_k, sh.r_v) // (2 if fp8 else 1)
    m = statistics.fmean
    gbs = lambda ms: lat / (ms * 1e-3) / 1e9
    del q, kc, vc, ws
    ceiling = stream_ceiling_gbs(lat, flush_fn, steps)
    return {
        "workload": name, "batch": B, "seq_len": msl, "heads": sh.H, "kv_heads": sh.kv,
        "rank_k": sh.r_k, "rank_v": sh.r_v, "latent_dtype": "e4m3" if fp8 else "f16",
        "latent_bytes_per_step": int(lat), "steps": steps,
        "step_ms": round(m(step_ms), 5), "step_gbs": round(gbs(m(step_ms)), 1),
        "split_kernel_ms": round(m(kern_ms), 5),
        "split_kernel_gbs": round(gbs(m(kern_ms)), 1),
        "split_kernel_hbm_frac": round(gbs(m(kern_ms)) / HBM_PEAK_GBS, 4),
        "stream_read_ceiling_gbs": round(ceiling, 1),
        "split_kernel_over_ceiling": round(gbs(m(kern_ms)) / ceiling, 4),
    }


def low_batch_leg(flush_fn, steps):
    """Low-batch decode latency (batch 1, 2, 4 x 2048 tokens, main shape):
    per step, after the Infinity-Cache flush and a device synchronisation,
    host wall time from the call to its completion (synchronise), once with
    the decode call made eagerly (three kernel launches from the host) and
    once replaying a HIP graph that captured it; plus the GPU time of the
    step from events on the stream."""
    import numpy as np
    import torch
    from rank_compressed_paged_amd import starkv as sk
    from rank_compressed_paged_amd import workloads as wl
    rows = []
    n = max(steps, 20)
    for B in (1, 2, 4):
        case = wl.make_decode_case(wl.MAIN, seq_lens=[2048] * B, seed=93)
        c = case.cache
        dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
        q, kc, vc, U, W = dev(case.q), dev(c.k_cache), dev(c.v_cache), dev(case.U), dev(case.W)
        bt, sl = dev(c.block_tables), dev(c.seq_lens)
        dims = sk.dims_of(kc, vc, U, W)
        ws = sk.alloc_workspace(sk.decode_workspace_size(dims, B, 2048), "cuda")
        out = torch.empty((B, 32, 128), dtype=torch.float16, device="cuda")

        def step():
            sk.decode_attn(q, kc, vc, U, W, bt, sl, 2048, case.scale, out=out, workspace=ws)

        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        torch.cuda.synchronize()

        def wall(fn):
            ts = []
            for i in range(n):
                flush_fn(i)
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                fn()
                torch.cuda.synchronize()
                ts.append((time.perf_counter() - t0) * 1e6)
            return statistics.median(ts)
        eager_us = wall(step)
        graph_us = wall(g.replay)
        gpu_ms, _, _ = timed(step, n, flush_fn)
        ws2 = sk.alloc_workspace(sk.decode_workspace_size(dims, B, 2048, launches=2), "cuda")
        fused_ms, _, _ = timed(lambda: sk.decode_attn(q, kc, vc, U, W, bt, sl, 2048, case.scale,
                                                      out=out, workspace=ws2, launches=2),
                               n, flush_fn)
        pps, ns = sk.decode_plan(dims, B, 2048)
        rows.append({"batch": B, "seq_len": 2048, "plan": [pps, ns],
                     "gpu_step_us": round(statistics.fmean(gpu_ms) * 1e3, 2),
                     "fused_gpu_step_us": round(statistics.fmean(fused_ms) * 1e3, 2),
                     "eager_latency_us": round(eager_us, 2),
                     "graph_latency_us": round(graph_us, 2)})
        del g
    return rows


def append_sizes_leg(flush_fn, steps):
    """The append at the main shape over a range of token counts (a decode
    step's 16 tokens up to a prefill chunk's 4096), flushed: events around the
    call and the library's timing events around its kernels, with the
    workspace the call needs (few-token path up to 64 tokens, the tiled
    kernel with its contraction split in four or two parts up to 2816, the
    unsplit tiled kernel above)."""
    import numpy as np
    import torch
    from rank_compressed_paged_amd import metrics
    from rank_compressed_paged_amd import starkv as sk
    from rank_compressed_paged_amd import workloads as wl
    sh = wl.MAIN
    rng = np.random.default_rng(321)
    U, W = wl.draw_bases(rng, sh)
    U, W = torch.from_numpy(U).cuda(), torch.from_numpy(W).cuda()
    out = []
    for n in (16, 64, 128, 512, 1024, 2048, 4096):
        k = torch.from_numpy(rng.standard_normal((n, sh.H, sh.d), dtype=np.float32)
                             .astype(np.float16)).cuda()
        v = torch.from_numpy(rng.standard_normal((n, sh.H, sh.d), dtype=np.float32)
                             .astype(np.float16)).cuda()
        nb = (n + sh.bs - 1) // sh.bs
        kc = torch.zeros((nb, sh.H, sh.bs, sh.r_k), dtype=torch.float16, device="cuda")
        vc = torch.zeros((nb, sh.r_v, sh.bs), dtype=torch.float16, device="cuda")
        slots = torch.arange(n, dtype=torch.int64, device="cuda")
        dims = sk.dims_of(kc, vc, U, W)
        need = sk.append_workspace_size(dims, n)
        ws = sk.alloc_workspace(need, "cuda") if need else None

        def app():   # same slots each time: idempotent
            sk.append(k, v, U, W, slots, kc, vc, workspace=ws)
        for i in range(3):
            flush_fn(i)
            app()
        torch.cuda.synchronize()
        call_ms, _, _ = timed(app, steps, flush_fn)
        _, kern_ms, _ = timed(app, steps, flush_fn, sk.TIME_APPEND)
        kern = statistics.fmean(kern_ms)
        flops = metrics.append_flops(n, sh.H, sh.d, sh.r_k, sh.r_v)
        out.append({"tokens": n, "call_us": round(statistics.fmean(call_ms) * 1e3, 2),
                    "kernel_us": round(kern * 1e3, 2), "workspace_bytes": int(need),
                    "kernel_tflops": round(flops / (kern * 1e-3) / 1e12, 1)})
    return out


def fit_leg(steps):
    """The bases fit at 16384 K/V samples of the main shape, 8 iterations:
    the whole call, and its Gram-matrix kernel (algorithmic TFLOP/s of the
    distinct second-moment entries against the fp16 MFMA peak)."""
    import numpy as np
    import torch
    from rank_compressed_paged_amd import metrics
    from rank_compressed_paged_amd import starkv as sk
    from rank_compressed_paged_amd import workloads as wl
    iters = 8
    fc = wl.make_config("fit_n16384")
    sh = fc.shape
    N = fc.k.shape[0]
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    k, v, u0, w0 = dev(fc.k), dev(fc.v), dev(fc.u0), dev(fc.w0)
    U = torch.empty((sh.H, sh.d, sh.r_k), dtype=torch.float16, device="cuda")
    W = torch.empty((sh.H * sh.d, sh.r_v), dtype=torch.float16, device="cuda")
    ws = sk.alloc_workspace(sk.fit_workspace_size(sk.make_dims(sh.H, sh.d, sh.r_k, sh.r_v, 1)),
                            "cuda")

    def fit():
        sk.fit_bases(k, v, sh.r_k, sh.r_v, u0, w0, iters, U=U, W=W, workspace=ws)

    settle(fit, None, 0.25)
    n = max(min(steps // 5, 10), 3)
    call_ms, _, _ = timed(fit, n)
    _, gram_ms, _ = timed(fit, n, None, sk.TIME_FIT_GRAM)
    m = statistics.fmean
    gf = metrics.gram_flops(N, sh.H, sh.d)
    itf = metrics.fit_iteration_flops(sh.H, sh.d, sh.r_k, sh.r_v)
    gram_tf = gf / (m(gram_ms) * 1e-3) / 1e12
    sample_bytes = 2 * N * sh.H * sh.d * 2
    return {
        "workload": "fit_n16384", "samples": N, "iters": iters, "steps": n,
        "call_ms": round(m(call_ms), 4),
        "gram_kernel_ms": round(m(gram_ms), 4),
        "gram_kernel_tflops": round(gram_tf, 1),
        "gram_kernel_mfma_frac": round(gram_tf / MFMA_F16_PEAK_TFLOPS, 4),
        "gram_algorithmic_gflop": round(gf / 1e9, 1),
        "gram_sample_bytes": int(sample_bytes),
        "after_gram_ms": round(m(call_ms) - m(gram_ms), 4),
        "iteration_algorithmic_gflop": round(itf / 1e9, 2),
    }


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

    def head_start(n):
        # about 150 us of GPU work per call to be timed (two 512 MiB reads)
        for _ in range(2 * n):
            torch.sum(flush, dim=0, out=flush_sink)
    HEAD_START["fn"] = head_start

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
    ws_app = sk.alloc_workspace(sk.append_workspace_size(sk.dims_of(kc_app, vc_app, t["U"], t["W"]), B),
                                "cuda")

    def append_step():
        sk.append(k_new, v_new, t["U"], t["W"], slots, kc_app, vc_app, workspace=ws_app)

    # warmup (untimed)
    for i in range(args.warmup):
        do_flush(i)
        step()
    torch.cuda.synchronize()

    # headline: whole steps, cache flushed before each, no events inside the step
    step_ms, _, wall = timed(step, args.steps, do_flush)
    # the split-K kernel alone (the dispatch's own timestamps), flushed
    _, kern_ms, _ = timed(step, args.steps, do_flush, sk.TIME_DECODE_SPLIT)
    # warm (latents left in the Infinity Cache), for reference only
    warm_ms, _, _ = timed(step, args.steps)
    _, warm_kern_ms, _ = timed(step, args.steps, None, sk.TIME_DECODE_SPLIT)
    app_ms, _, _ = timed(append_step, max(args.steps, 10), do_flush)
    _, app_kern_ms, _ = timed(append_step, max(args.steps, 10), do_flush, sk.TIME_APPEND)
    # the step with its append in front (second row)
    both_ms, _, _ = timed(lambda: (append_step(), step()), args.steps, do_flush)
    # the same step with the split pass and the merge fused into one kernel
    # (the q projection, then that kernel) instead of three kernels
    ws2 = sk.alloc_workspace(sk.decode_workspace_size(dims, B, msl, launches=2), "cuda")

    def step2():
        sk.decode_attn(t["q"], t["k_cache"], t["v_cache"], t["U"], t["W"], t["block_tables"],
                       t["seq_lens"], msl, case.scale, out=out, workspace=ws2, launches=2)
    fused_ms, _, _ = timed(step2, args.steps, do_flush)
    _, fused_kern_ms, _ = timed(step2, args.steps, do_flush, sk.TIME_DECODE_SPLIT)
    del ws2

    # the streaming-read ceiling measured on this machine at this step's size
    ceiling_gbs = stream_ceiling_gbs(lat_bytes, do_flush, max(args.steps, 10))

    ms = statistics.fmean(step_ms)
    kern = statistics.fmean(kern_ms)
    value = lat_bytes / (ms * 1e-3) / 1e9
    achieved = lat_bytes / (kern * 1e-3) / 1e9
    # the counter summary covers the decode_b16 launch only
    traffic = read_traffic(lat_bytes) if case.name == TRAFFIC_WORKLOAD else None
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
        "step_with_append_ms": round(statistics.fmean(both_ms), 5),
        "fused_step_ms": round(statistics.fmean(fused_ms), 5),
        "fused_kernel_ms": round(statistics.fmean(fused_kern_ms), 5),
        "wall_s_timed_loop_incl_flush": round(wall, 4),
        "split_plan": {"pages_per_split": pps, "num_splits": ns},
        "flush": args.flush,
        "stream_read_ceiling_gbs": round(ceiling_gbs, 1),
        "split_kernel_over_ceiling": round(achieved / ceiling_gbs, 4),
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
    if not args.no_prefill:
        res["prefill"] = prefill_leg(do_flush, args.steps,
                                     cpu_budget_s=0.0 if args.no_cpu else args.cpu_prefill_seconds)
        res["prefill_fp8"] = prefill_leg(do_flush, args.steps, "prefill_b16_fp8")
        res["prefill_generic"] = prefill_leg(do_flush, args.steps, "conservative_prefill_b16")
        res["append_sizes"] = append_sizes_leg(do_flush, args.steps)
    if not args.no_low_batch:
        res["low_batch"] = low_batch_leg(do_flush, args.steps)
    if not args.no_configs:
        # the other fp16 configurations of the metric's shape
        res["decode_configs"] = [decode_leg(n, do_flush, args.steps)
                                 for n in ("decode_b64", "long_b20", "tiny")]
    if not args.no_layouts:
        res["layouts"] = [decode_leg(n, do_flush, args.steps)
                          for n in ("gqa8_b16", "lowrank_b16", "decode_b16_fp8", "decode_b64_fp8",
                                    "conservative_b16", "odd_h28_b16")]
    if not args.no_fit:
        res["fit"] = fit_leg(args.steps)
    res["device"] = device_info()
    if case.name == "decode_b16":
        # the pages' own decode-step figures for this shape (NVIDIA L4, other
        # hardware): context only, not a target
        res["context_l4"] = {"source": "Proxima README, Per-decode-step attention table",
                             "seq_len": 2048, "batch": 16, "star_kv_ms": 1.735,
                             "flash_attn2_ms": 2.314, "hardware": "NVIDIA L4"}
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


def profile_fit(args):
    """A short run for rocprofv3: bases fits of the fit_n16384 workload."""
    import numpy as np
    import torch
    from rank_compressed_paged_amd import starkv as sk
    from rank_compressed_paged_amd import workloads as wl
    fc = wl.make_config("fit_n16384")
    sh = fc.shape
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    k, v, u0, w0 = dev(fc.k), dev(fc.v), dev(fc.u0), dev(fc.w0)
    ws = sk.alloc_workspace(sk.fit_workspace_size(sk.make_dims(sh.H, sh.d, sh.r_k, sh.r_v, 1)),
                            "cuda")
    for _ in range(max(args.steps, 1)):
        sk.fit_bases(k, v, sh.r_k, sh.r_v, u0, w0, 8, workspace=ws)
    torch.cuda.synchronize()
    print(f"profile-fit done: {args.steps} fits of fit_n16384", flush=True)


def profile_run(args):
    """A short run for rocprofv3: warm steps of the workload, then a plain
    COPY_BYTES device copy used to calibrate FETCH_SIZE / WRITE_SIZE."""
    import torch
    from rank_compressed_paged_amd import starkv as sk
    case, t = make_inputs(args.workload)
    msl = int(case.cache.seq_lens.max())
    dims = sk.dims_of(t["k_cache"], t["v_cache"], t["U"], t["W"])
    ws = sk.alloc_workspace(sk.decode_workspace_size(dims, case.B, msl), "cuda")
    flush = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    sink = torch.empty((), dtype=torch.float32, device="cuda")
    for _ in range(max(args.steps, 1)):
        torch.sum(flush, dim=0, out=sink)   # the benchmark's read flush
        sk.decode_attn(t["q"], t["k_cache"], t["v_cache"], t["U"], t["W"], t["block_tables"],
                       t["seq_lens"], msl, case.scale, workspace=ws)
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(3)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.sum(flush, dim=0, out=sink)
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"profile-run done: {args.steps} steps of {case.name}, 3 copies of {COPY_BYTES} B",
          flush=True)


def plan_sweep(args):
    """Decode steps and the split-K kernel (flushed, as in the benchmark) at
    the planner's split plan, at forced pages_per_split values and at forced
    finish-kernel tiles (merge_seqs, rows per work group): the evidence for
    the planner's choices, one JSON line per (workload, plan)."""
    import numpy as np
    import torch
    from rank_compressed_paged_amd import metrics
    from rank_compressed_paged_amd import starkv as sk
    from rank_compressed_paged_amd import workloads as wl
    flush = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    sink = torch.empty((), dtype=torch.float32, device="cuda")
    fl = lambda i: torch.sum(flush, dim=0, out=sink)
    HEAD_START["fn"] = lambda n: [torch.sum(flush, dim=0, out=sink) for _ in range(2 * n)]
    for name in args.sweep_workloads.split(","):
        case = wl.make_config(name)
        sh, c = case.shape, case.cache
        dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
        q, kc, vc, U, W = dev(case.q), dev(c.k_cache), dev(c.v_cache), dev(case.U), dev(case.W)
        bt, sl = dev(c.block_tables), dev(c.seq_lens)
        B, msl = case.B, int(c.seq_lens.max())
        dims = sk.dims_of(kc, vc, U, W, num_heads=sh.H)
        lat = metrics.decode_latent_bytes(c.seq_lens, sh.kv, sh.r_k, sh.r_v)
        out = torch.empty((B, sh.H, sh.d), dtype=torch.float16, device="cuda")
        pages = (msl + sh.bs - 1) // sh.bs
        plans = [(pps, 0) for pps in [0] + [int(x) for x in args.sweep_pps.split(",") if x]]
        plans += [(0, m) for m in [int(x) for x in args.sweep_merge.split(",") if x]]
        for pps, merge in plans:
            if pps > pages:
                continue
            ws = sk.alloc_workspace(sk.decode_workspace_size(dims, B, msl, pages_per_split=pps,
                                                             merge_seqs=merge), "cuda")

            def step():
                sk.decode_attn(q, kc, vc, U, W, bt, sl, msl, case.scale, out=out, workspace=ws,
                               pages_per_split=pps, merge_seqs=merge)
            for i in range(5):
                fl(i)
                step()
            torch.cuda.synchronize()
            s_ms, _, _ = timed(step, args.steps, fl)
            _, k_ms, _ = timed(step, args.steps, fl, sk.TIME_DECODE_SPLIT)
            sm, km = statistics.fmean(s_ms), statistics.fmean(k_ms)
            plan = sk.decode_plan(dims, B, msl) if pps == 0 else (pps, (pages + pps - 1) // pps)
            print(json.dumps({"workload": name, "pages_per_split": plan[0], "num_splits": plan[1],
                              "merge_seqs": merge or "planner",
                              "planner": pps == 0 and merge == 0, "work_groups": B * plan[1],
                              "step_us": round(sm * 1e3, 2), "split_kernel_us": round(km * 1e3, 2),
                              "split_kernel_hbm_frac": round(lat / (km * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                              "step_hbm_frac": round(lat / (sm * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}),
                  flush=True)
            del ws


def _pmc_rows(path):
    with open(path) as f:
        return list(csv.DictReader(f))


def summarize_pmc(fetch_csv, write_csv, out_path):
    """Average FETCH_SIZE / WRITE_SIZE per dispatch of the split-K kernel and
    of the COPY_BYTES device copies, and scale the kernel's counts by the
    bytes each counted unit represents on the copy."""
    from rank_compressed_paged_amd import metrics

    def per_dispatch(rows, counter, match):
        vals = [float(r["Counter_Value"]) for r in rows
                if match(r["Kernel_Name"]) and r["Counter_Name"] == counter]
        return vals

    def big_copy(rows, counter):
        vals = per_dispatch(rows, counter, lambda n: "copyBuffer" in n)
        top = max(vals)
        big = [v for v in vals if v > 0.5 * top]      # the COPY_BYTES copies
        return sum(big) / len(big), len(big)

    is_split = lambda n: DECODE_KERNEL in n
    fr, wr = _pmc_rows(fetch_csv), _pmc_rows(write_csv)
    fv = per_dispatch(fr, "FETCH_SIZE", is_split)
    wv = per_dispatch(wr, "WRITE_SIZE", is_split)
    f_split, w_split = sum(fv) / len(fv), sum(wv) / len(wv)
    f_copy, nfc = big_copy(fr, "FETCH_SIZE")
    w_copy, nwc = big_copy(wr, "WRITE_SIZE")
    f_scale = COPY_BYTES / f_copy          # bytes per counted unit, reads
    w_scale = COPY_BYTES / w_copy          # bytes per counted unit, writes
    lat = 16 * 2048 * metrics.latent_bytes_per_token(32, 64, 512)
    rd, wb = f_split * f_scale, w_split * w_scale
    with open(out_path, "w") as f:
        f.write("# HBM traffic of the split-K decode kernel, decode_b16 "
                "(batch 16 x 2048 tokens, H32 d128 r_k64 r_v512, 16-token pages)\n")
        f.write("# FETCH_SIZE and WRITE_SIZE from two rocprofv3 --pmc passes over\n")
        f.write("#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir> -o fetch -- "
                "python3 bench.py --profile-run --steps 5\n")
        f.write("#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir> -o write -- "
                "python3 bench.py --profile-run --steps 5\n")
        f.write("# each kernel count is scaled by the bytes per counted unit measured on a\n")
        f.write("# plain device copy of copy_bytes bytes in the same run; written with\n")
        f.write("#   python3 bench.py --summarize-pmc <fetch csv> <write csv> <this file>\n")
        f.write(f"kernel_source_sha={kernel_source_hash()}\n")
        f.write(f"dispatches_fetch={len(fv)}\ndispatches_write={len(wv)}\n")
        f.write(f"fetch_units_per_dispatch={f_split:.1f}\nwrite_units_per_dispatch={w_split:.1f}\n")
        f.write(f"copy_bytes={COPY_BYTES}\ncopy_fetch_units={f_copy:.1f} (over {nfc} copies)\n")
        f.write(f"copy_write_units={w_copy:.1f} (over {nwc} copies)\n")
        f.write(f"fetch_bytes_per_unit={f_scale:.2f}\nwrite_bytes_per_unit={w_scale:.2f}\n")
        f.write(f"hbm_read_bytes_per_launch={rd:.0f}\nhbm_write_bytes_per_launch={wb:.0f}\n")
        f.write(f"hbm_bytes_per_launch={rd + wb:.0f}\nalgorithmic_bytes_per_launch={lat}\n")
        f.write(f"read_over_algorithmic={rd / lat:.4f}\n")
        f.write(f"traffic_over_algorithmic={(rd + wb) / lat:.4f}\n")
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
    if args.profile_fit:
        profile_fit(args)
        return 0
    if args.plan_sweep:
        plan_sweep(args)
        return 0
    run_bench(args)
    return 0


if __name__ == "__main__":
    sys.exit(main())
