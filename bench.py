"""Benchmark of tree-masked MLA verify attention on one MI355X.

Workload (one step = one verify call = split partials, each workgroup planning
from the raw metadata, + merge):
1 request, 91,136-token prefix scattered over a 1,048,576-slot page_size=1 pool,
32-node random draft tree, H = 8 heads, 576-wide bf16 latent (V = first 512
dims), 1% of prefix rows scaled by 8, fp32 output + LSE.  Inputs are seeded
synthetic data resident in HBM before the timed region.

Prints one JSON line: value = effective KV bandwidth (bytes of the gathered
latent rows / time per call) in GB/s; us_per_call beside it; the roofline of the
split-partial kernel (MFMA-bound at 256 query rows: algorithmic flops / its
average duration from HIP events on the launch stream); and the CPU oracle
timed on this host on the same call.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs/call + effective KV GB/s & %roofline, 91k-prefix 32-node tree verify"
WORKLOAD = "p91136_t32"
PEAK_MFMA_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0              # MI355X HBM3E
KERNEL_SRC = os.path.join(ROOT, "speculative_decoding_mla_page_amd", "csrc", "mla_verify_kernels.hip")
DESCRIPTIONS = {
    "p91136_t32": "1 request, 91,136-token prefix, 32-node random tree, H=8, 576-d bf16 latent "
                  "(V = first 512), 1% outlier rows x8, page_size=1 pool of 1,048,576 slots, fp32 out + LSE",
    "decode_b32_h16": "decode: 32 requests x 1 query token, prefixes U[512, 8192] (142,576 keys), H=16, "
                      "576-d bf16 latent, page_size=1 pool of 262,144 slots, fp32 out + LSE",
    "decode_b64_h128": "decode: 64 requests x 1 query token, prefixes U[512, 8192] (292,951 keys), H=128, "
                       "576-d bf16 latent, page_size=1 pool of 524,288 slots, fp32 out + LSE",
    "p91136_t32_h64": "1 request, 91,136-token prefix, 32-node random tree, H=64 (2,048 query rows), 576-d bf16 "
                      "latent (V = first 512), 1% outlier rows x8, page_size=1 pool of 1,048,576 slots, "
                      "fp32 out + LSE",
    "p23040_t32": "1 request, 23,040-token prefix, 32-node random tree, H=8, 576-d bf16 latent (V = first 512), "
                  "page_size=1 pool of 262,144 slots, fp32 out + LSE",
    "p5632_t16": "1 request, 5,632-token prefix, 16-node random tree, H=8, 576-d bf16 latent (V = first 512), "
                 "page_size=1 pool of 65,536 slots, fp32 out + LSE",
}
GRAPH_WORKLOAD = "segmented_b8_graph"
DESCRIPTIONS[GRAPH_WORKLOAD] = (
    "segmented batch: 8 requests, prefixes U[1000, 185000], trees U[8, 64] (random parents), H=8, 576-d bf16 "
    "latent, fully populated 2,097,152-slot pool; one hipGraph capture, replayed with the indptrs, kv_indices, "
    "out_cache_loc, masks and queries rewritten in place before each replay (fresh draws, seeds 2000 + r)")


def traffic_file(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"mla_verify_partial_{workload}_traffic.txt")


def kernel_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def algorithmic(inst, kv_index_bytes=4, ocl_bytes=8):
    """Algorithmic work of one call.  flops: every query row (node x head)
    takes 576 + 512 multiply-adds per visible-or-not key of its request.
    kv_bytes: the gathered latent rows (1,152 B per key).  bytes: everything
    the call must move once - latent rows, prefix indices, tree slots, the
    tree mask block, queries (1,152 B per row), out (2,048 B) and lse (4 B)
    per row."""
    flops = 0
    kv_bytes = 0
    all_bytes = 0
    h = inst.num_heads
    for p, t in zip(inst.prefix_lens, inst.tree_sizes):
        n = p + t
        rows = t * h
        flops += 2 * rows * n * (576 + 512)
        kv_bytes += n * 1152
        all_bytes += n * 1152 + p * kv_index_bytes + t * ocl_bytes + t * t + rows * 1152 + rows * (2048 + 4)
    return flops, kv_bytes, all_bytes


def read_traffic(workload: str):
    """HBM bytes per partial-kernel launch from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source."""
    path = traffic_file(workload)
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_hash = re.search(r"kernel_source_sha256_16:\s*(\w+)", txt)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_hash():
        return None
    return float(m_bytes.group(1))


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor()


def cpu_baseline(inst, kv_bytes, workload: str, min_s: float = 10.0, budget_s: float = 30.0):
    """The oracle, as it stands, on the same call: repeated until about min_s
    seconds of CPU work (at least 3 runs, at most budget_s), median reported."""
    import numpy as np
    from oracle import mla_verify_ref as R
    try:
        import threadpoolctl
        np.ones((4, 4)) @ np.ones((4, 4))
        info = threadpoolctl.threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    view = inst.pool_view()
    times = []
    t_start = time.perf_counter()
    while len(times) < 3 or (time.perf_counter() - t_start) < min_s:
        if len(times) >= 1 and time.perf_counter() - t_start >= budget_s:
            break
        t0 = time.perf_counter()
        R.mla_verify_reference(inst.q, view, inst.qo_indptr, inst.kv_indptr, inst.kv_indices,
                               inst.out_cache_loc, inst.custom_mask, inst.mask_indptr,
                               inst.num_heads, inst.sm_scale)
        times.append(time.perf_counter() - t0)
    t = float(np.median(times))
    return {"value": kv_bytes / t / 1e9, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"whole {workload} call ({inst.total_q} query tokens x {inst.num_heads} heads over "
                      f"{inst.total_kv + inst.total_q:,} keys), median of {len(times)} runs, numpy fp64 "
                      f"with {threads} BLAS threads on {cpu_model()}",
            "us_per_call": t * 1e6}


def achievable_peaks(torch, B):
    """Rates this GPU reaches, as a second reference beside the datasheet peaks:
    the library's HBM read stream over 1 GiB and its dense bf16 MFMA loop (16
    waves per compute unit, four independent accumulator chains each), plus a
    1 GiB device-to-device copy (read + write bytes); each timed with events,
    median of 10 runs after 3 untimed ones."""
    import numpy as np
    stream = torch.cuda.current_stream()
    sp = int(stream.cuda_stream)

    def timed(fn, reps=10, warm=3):
        for _ in range(warm):
            fn()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return float(np.median(ts))

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks = 4 * cus
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    n = 1 << 28                                       # float32 elements: 1 GiB
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    t_read = timed(lambda: B.calibrate_read(src, blocks, out, sp))
    dst = torch.empty_like(src)
    t_copy = timed(lambda: dst.copy_(src))
    del src, dst
    iters = 8192
    t_mfma = timed(lambda: B.calibrate_mfma(iters, blocks, out, sp))
    return {"hbm_read_GBps": n * 4 / t_read / 1e9,
            "hbm_copy_GBps": 2 * n * 4 / t_copy / 1e9,
            "mfma_bf16_TFLOPs": blocks * 4 * iters * 65536 / t_mfma / 1e12,
            "how": f"library read stream over 1 GiB ({blocks} workgroups of 256 threads); 1 GiB device copy, "
                   f"read + write bytes; bf16 16x16x32 MFMA loop, {blocks} workgroups x 4 waves x {iters} "
                   f"rounds of 4 chains; median of 10 after 3 untimed runs; fractions use the read stream"}


def with_achievable(peaks, bound, achieved, t_roof_s, call_s):
    """The fractions of the measured peaks beside the datasheet ones."""
    ref = peaks["mfma_bf16_TFLOPs"] if bound == "mfma" else peaks["hbm_read_GBps"]
    return dict(peaks, roofline_frac=achieved / ref, call_frac=t_roof_s / call_s)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # back-to-back calls settle within 20-40 ms (the first few hundred
    # headline calls run 5-15 % slower while clocks and address translation
    # warm up), so the default warm-up spans that before the timed region
    ap.add_argument("--warmup", type=int, default=400)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", default=WORKLOAD, choices=sorted(DESCRIPTIONS),
                    help="the headline workload by default; the decode shapes are extra measurements")
    ap.add_argument("--cold-calls", type=int, default=20,
                    help="extra calls each preceded by a 1 GiB cache scrub (reported, not the value)")
    ap.add_argument("--fused-save-calls", type=int, default=50,
                    help="extra calls that also store the draft rows into the pool (reported, not the value)")
    ap.add_argument("--compact-calls", type=int, default=5,
                    help="prefix compactions onto fresh slots, then the call again (reported, not the value)")
    ap.add_argument("--no-achievable", action="store_true",
                    help="skip the measured copy and MFMA-loop peaks (reported beside the datasheet ones)")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="also run one device-to-device copy of this many MiB (a known-size "
                         "kernel for scaling hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "the bench runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import numpy as np
    import torch
    from speculative_decoding_mla_page_amd import binding as B
    from speculative_decoding_mla_page_amd.device import DeviceInputs, Verifier
    from workloads import gen

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU"}), flush=True)
        sys.exit(1)
    torch.cuda.set_device(0)
    workload = args.workload
    if workload == GRAPH_WORKLOAD:
        bench_graph(args)
        return
    inst = gen.config(workload)
    flops, kv_bytes, alg_bytes = algorithmic(inst)
    di = DeviceInputs(inst)
    # the plan's tree-size bound is the largest draft tree the caller runs
    ver = Verifier.for_inputs(di, max_tree_nodes=max(1, max(int(t) for t in inst.tree_sizes)))
    out, lse = di.alloc_outputs()
    a = ver.args(di, out, lse)
    stream = torch.cuda.current_stream()
    sp = int(stream.cuda_stream)

    def step(evs=None):
        if evs is None:
            B.run(ver.plan, a, ver.workspace, sp)
            return
        evs[0].record(stream)
        B.run_phase(ver.plan, a, ver.workspace, B.PHASE_PARTIAL, sp)
        evs[1].record(stream)
        B.run_phase(ver.plan, a, ver.workspace, B.PHASE_MERGE, sp)
        evs[2].record(stream)

    if args.calibration_copy_mib > 0:
        n = args.calibration_copy_mib << 18          # float32 elements
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if ver.error_word() != 0:
        raise RuntimeError(f"device error word {ver.error_word():#x}")

    # timed region: K whole calls (mla_verify_run, two launches each) back to
    # back on the stream, bracketed by one event pair and the host clock
    span = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    span[0].record(stream)
    for _ in range(args.steps):
        step()
    span[1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    span_ms = span[0].elapsed_time(span[1])

    # per-kernel times: the same K calls again, launched phase by phase with
    # events between the launches (the events add gaps, so this loop is not
    # the value; the partial kernel's mean here gives the roofline figure)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    part_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    merge_ms = np.array([e[1].elapsed_time(e[2]) for e in evs])
    call_ms = np.array([e[0].elapsed_time(e[2]) for e in evs])
    ms_per_step = wall * 1e3 / args.steps

    # cold calls: before each, push the call's data out of the 256 MB Infinity
    # Cache and the L2s with a 1 GiB scrub, either read (clean lines: the call
    # pays only for its misses; the basis of the whole-call roofline fraction)
    # or written (the call also pays for writing back the scrub's dirty lines
    # it evicts); per-phase events give the partial kernel's cold duration
    cold_us = cold_dirty_us = cold_part_us = None
    if args.cold_calls > 0:
        scrub = torch.zeros(1 << 28, dtype=torch.float32, device="cuda")
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        sums = torch.empty(4 * cus * 256, dtype=torch.float32, device="cuda")

        def cold(scrub_fn, phases=False):
            ce = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.cold_calls)]
            for i in range(args.cold_calls):
                scrub_fn(i)
                if phases:
                    step(ce[i])
                else:
                    ce[i][0].record(stream)
                    step()
                    ce[i][2].record(stream)
            torch.cuda.synchronize()
            call = float(np.median([e[0].elapsed_time(e[2]) for e in ce]) * 1e3)
            part = float(np.median([e[0].elapsed_time(e[1]) for e in ce]) * 1e3) if phases else None
            return call, part

        read_scrub = lambda i: B.calibrate_read(scrub, 4 * cus, sums, sp)  # noqa: E731
        cold_us, _ = cold(read_scrub)
        _, cold_part_us = cold(read_scrub, phases=True)
        cold_dirty_us, _ = cold(lambda i: scrub.fill_(float(i)))
        del scrub, sums

    # the same call with the fused KV save: the draft rows are handed over and
    # stored at out_cache_loc by the split-partial launch (same values, so the
    # pool is unchanged); timed over its own loop, not the value
    fused = None
    if args.fused_save_calls > 0:
        ocl = di.out_cache_loc[:di.total_q].to(torch.int64)
        kv_new = di.pool[ocl][:, :576].contiguous()
        a2 = B.make_args(di.batch, di.sm_scale, di.q, di.pool, di.qo_indptr, di.kv_indptr,
                         di.kv_indices, di.out_cache_loc, di.custom_mask, di.mask_indptr,
                         out, lse, num_slots=di.num_slots, kv_new=kv_new)
        for _ in range(args.warmup):   # after the cache scrubs above: back to steady state
            B.run(ver.plan, a2, ver.workspace, sp)
        fe = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.fused_save_calls)]
        for e in fe:
            e[0].record(stream)
            B.run_phase(ver.plan, a2, ver.workspace, B.PHASE_PARTIAL, sp)
            e[1].record(stream)
            B.run_phase(ver.plan, a2, ver.workspace, B.PHASE_MERGE, sp)
        fe_all = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        fe_all[0].record(stream)
        for _ in range(args.fused_save_calls):
            B.run(ver.plan, a2, ver.workspace, sp)
        fe_all[1].record(stream)
        torch.cuda.synchronize()
        fused = {"us_per_call": fe_all[0].elapsed_time(fe_all[1]) * 1e3 / args.fused_save_calls,
                 "partial_us": float(np.median([e[0].elapsed_time(e[1]) for e in fe]) * 1e3),
                 "rows_saved": int(di.total_q), "calls": args.fused_save_calls}

    # prefix compaction (KV defragmentation) onto fresh contiguous slots, then
    # the same call on the compacted pool; last, since it rewrites the inputs
    compaction = None
    if args.compact_calls > 0:
        if ver.error_word() != 0:
            raise RuntimeError(f"device error word {ver.error_word():#x}")
        base = di.num_slots
        di.pool = torch.cat([di.pool, torch.empty((di.total_kv, di.pool.shape[1]), dtype=di.pool.dtype,
                                                  device=di.pool.device)])
        di.num_slots = di.pool.shape[0]
        a = ver.args(di, out, lse)
        dst = torch.tensor([base + int(x) for x in np.asarray(inst.kv_indptr)[:-1]], dtype=torch.int64,
                           device=di.pool.device)
        err = torch.zeros(1, dtype=torch.int32, device=di.pool.device)
        ce2 = [torch.cuda.Event(enable_timing=True) for _ in range(args.compact_calls + 1)]
        ce2[0].record(stream)
        for k in range(args.compact_calls):
            B.compact(ver.plan, a, dst, err, sp)   # the first call moves, the rest copy in place
            ce2[k + 1].record(stream)
        for _ in range(args.warmup):   # after the cache scrubs above: back to steady state
            B.run(ver.plan, a, ver.workspace, sp)
        ve = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ve[0].record(stream)
        for _ in range(args.steps):
            B.run(ver.plan, a, ver.workspace, sp)
        ve[1].record(stream)
        # the same calls through the contiguous-prefix fast path
        ver_c = Verifier.for_inputs(di, max_tree_nodes=max(1, max(int(t) for t in inst.tree_sizes)),
                                    flags=B.FLAG_CONTIGUOUS_PREFIX)
        a_c = ver_c.args(di, out, lse)
        for _ in range(args.warmup):   # after the cache scrubs above: back to steady state
            B.run(ver_c.plan, a_c, ver_c.workspace, sp)
        vc = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        vc[0].record(stream)
        for _ in range(args.steps):
            B.run(ver_c.plan, a_c, ver_c.workspace, sp)
        vc[1].record(stream)
        torch.cuda.synchronize()
        if int(err.item()) != 0 or ver.error_word() != 0 or ver_c.error_word() != 0:
            raise RuntimeError("compaction reported an error")
        compaction = {"first_call_us": ce2[0].elapsed_time(ce2[1]) * 1e3,
                      "us_per_call": float(np.median([ce2[k].elapsed_time(ce2[k + 1])
                                                      for k in range(args.compact_calls)]) * 1e3),
                      "rows": int(di.total_kv), "bytes_moved": int(di.total_kv) * 1152 * 2,
                      "verify_us_per_call_after": ve[0].elapsed_time(ve[1]) * 1e3 / args.steps,
                      "verify_us_per_call_contiguous_prefix": vc[0].elapsed_time(vc[1]) * 1e3 / args.steps}

    # reference numbers: the same call checked for the device error word
    if ver.error_word() != 0:
        raise RuntimeError(f"device error word {ver.error_word():#x}")

    # throughput of the timed region: first event to last over the K calls
    us_call = float(span_ms * 1e3 / args.steps)
    part_us = float(np.mean(part_ms) * 1e3)
    traffic = read_traffic(workload)
    # the split-partial kernel's own algorithmic bytes: the call's less out and lse
    rows_all = inst.total_q * inst.num_heads
    part_bytes = alg_bytes - rows_all * (2048 + 4)
    # the bound of the partial kernel on this workload: MFMA when its flops take
    # longer at peak than its bytes
    t_mfma = flops / (PEAK_MFMA_BF16_TFLOPS * 1e12)
    if flops / (PEAK_MFMA_BF16_TFLOPS * 1e12) >= part_bytes / (PEAK_HBM_GBS * 1e9):
        work, scale, peak, unit, bound = flops, 1e12, PEAK_MFMA_BF16_TFLOPS, "TFLOP/s", "mfma"
    else:
        work, scale, peak, unit, bound = part_bytes, 1e9, PEAK_HBM_GBS, "GB/s", "hbm"
    achieved = work / (part_us * 1e-6) / scale
    roof = {"bound": bound, "achieved": achieved, "peak": peak, "unit": unit, "frac": achieved / peak,
            "traffic": traffic, "kernel": "partial_kernel", "kernel_source_sha256_16": kernel_hash(),
            "algorithmic_per_launch": work, "launch_us_warm": part_us}
    if cold_part_us:
        roof["launch_us_cold"] = cold_part_us
        roof["frac_cold"] = work / (cold_part_us * 1e-6) / scale / peak
    if bound == "mfma":
        # the split P (hi + lo) runs 2 x (576 + 512 + 512) = 3,200 MFMA flops per
        # (row, key) for 2,176 algorithmic ones: the design's ceiling on frac
        roof["design_ceiling_frac"] = 2176.0 / 3200.0
    # the whole call against its roofline: all algorithmic bytes vs flops, over
    # the cold (read-scrubbed) call; the warm and write-scrubbed calls beside
    t_hbm = alg_bytes / (PEAK_HBM_GBS * 1e9)
    t_roof = max(t_hbm, t_mfma)
    call_basis = cold_us if cold_us else us_call
    roof_call = {"t_roof_us": t_roof * 1e6, "basis": "cold (read-scrubbed) call" if cold_us else "warm call",
                 "frac": t_roof / (call_basis * 1e-6), "frac_hbm": t_hbm / (call_basis * 1e-6),
                 "frac_mfma": t_mfma / (call_basis * 1e-6), "frac_warm": t_roof / (us_call * 1e-6)}
    if cold_dirty_us:
        roof_call["frac_after_write_scrub"] = t_roof / (cold_dirty_us * 1e-6)
    achievable = None
    if not args.no_achievable:
        peaks = achievable_peaks(torch, B)
        t_roof_a = max(alg_bytes / (peaks["hbm_read_GBps"] * 1e9), flops / (peaks["mfma_bf16_TFLOPs"] * 1e12))
        achievable = with_achievable(peaks, bound, achieved, t_roof_a, call_basis * 1e-6)
    metric = METRIC if workload == WORKLOAD else f"µs/call + effective KV GB/s & %roofline, {workload}"
    result = {
        "metric": metric,
        "value": kv_bytes / (us_call * 1e-6) / 1e9,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": DESCRIPTIONS[workload], "name": workload, "batch": inst.batch,
                   "prefix_tokens": inst.total_kv, "tree_nodes": inst.total_q,
                   "heads": inst.num_heads, "query_rows": inst.total_q * inst.num_heads,
                   "keys": inst.total_kv + inst.total_q},
        "us_per_call": us_call,
        "us_per_call_each_p10_p50_p90": [float(np.percentile(call_ms, q) * 1e3) for q in (10, 50, 90)],
        "us_per_call_cold": cold_us,
        "us_per_call_cold_after_write_scrub": cold_dirty_us,
        "kernel_us": {"partial": part_us, "merge": float(np.mean(merge_ms) * 1e3)},
        "tflops_per_call": flops / (us_call * 1e-6) / 1e12,
        "algorithmic": {"flops": flops, "kv_bytes": kv_bytes, "bytes": alg_bytes},
        "roofline": roof,
        "roofline_call": roof_call,
        "achievable": achievable,
        "fused_kv_save": fused,
        "compaction": compaction,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(inst, kv_bytes, workload)
    print(json.dumps(result), flush=True)


def bench_graph(args):
    """The segmented batch under hipGraph replay.  The call is captured twice,
    on two sets of buffers sized to the plan bounds.  Replay i uses set i % 2;
    draw i (one of R fresh draws) is copied into that set on a side stream,
    after replay i - 2 has finished with it and while replay i - 1 still runs.
    The replay is then queued behind replay i - 1, so the events around it
    bracket the graph alone (no copy, no host submission gap)."""
    import numpy as np
    import torch
    from speculative_decoding_mla_page_amd import binding as B
    from speculative_decoding_mla_page_amd.device import Verifier
    from workloads import gen

    dev = torch.device("cuda")
    bounds = gen.SEGMENTED_BOUNDS
    h = gen.SEGMENTED["num_heads"]
    pool = torch.from_numpy(gen.segmented_pool().view(np.int16)).to(dev)
    mq = bounds["max_q_tokens"]
    ver = Verifier(h, bounds["max_batch"], mq, bounds["max_kv_tokens"], max_tree_nodes=bounds["max_tree_nodes"])

    def buffers():
        st = {
            "q": torch.zeros((mq, h, 576), dtype=torch.int16, device=dev),
            "qo_indptr": torch.zeros(bounds["max_batch"] + 1, dtype=torch.int32, device=dev),
            "kv_indptr": torch.zeros(bounds["max_batch"] + 1, dtype=torch.int32, device=dev),
            "mask_indptr": torch.zeros(bounds["max_batch"] + 1, dtype=torch.int32, device=dev),
            "kv_indices": torch.zeros(bounds["max_kv_tokens"], dtype=torch.int32, device=dev),
            "out_cache_loc": torch.zeros(mq, dtype=torch.int64, device=dev),
            "custom_mask": torch.zeros(mq * bounds["max_tree_nodes"], dtype=torch.uint8, device=dev),
            "out": torch.zeros((mq, h, 512), dtype=torch.float32, device=dev),
            "lse": torch.zeros((mq, h), dtype=torch.float32, device=dev),
        }
        st["args"] = B.make_args(gen.SEGMENTED["batch"], float(gen.SM_SCALE), st["q"], pool, st["qo_indptr"],
                                 st["kv_indptr"], st["kv_indices"], st["out_cache_loc"], st["custom_mask"],
                                 st["mask_indptr"], st["out"], st["lse"])
        return st

    sets = [buffers(), buffers()]

    n_draws = max(1, min(args.steps, 25))
    draws = []
    for r in range(n_draws):
        rep = gen.segmented_replay(r)
        host = {k: torch.from_numpy(np.ascontiguousarray(v)).reshape(-1)
                for k, v in (("qo_indptr", rep.qo_indptr), ("kv_indptr", rep.kv_indptr),
                             ("mask_indptr", rep.mask_indptr), ("kv_indices", rep.kv_indices),
                             ("out_cache_loc", rep.out_cache_loc), ("custom_mask", rep.custom_mask))}
        host["q"] = torch.from_numpy(rep.q.view(np.int16))
        flops, kv_bytes, all_bytes = algorithmic(rep)
        draws.append((host, flops, kv_bytes, all_bytes))

    def fill(st, host):
        for k, t in host.items():
            if k == "q":
                st["q"][:t.shape[0]].copy_(t)
            else:
                st[k][:t.numel()].copy_(t.view(st[k].dtype))

    main = torch.cuda.current_stream()
    graphs = []
    for st in sets:
        fill(st, draws[0][0])
        torch.cuda.synchronize()
        B.run(ver.plan, st["args"], ver.workspace)     # loads the code objects before capture
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(main)
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                B.run(ver.plan, st["args"], ver.workspace)
        main.wait_stream(side)
        torch.cuda.synchronize()
        graphs.append(g)

    copy_stream = torch.cuda.Stream()
    done = [torch.cuda.Event(), torch.cuda.Event()]
    for d in done:
        d.record(main)

    def replay(i, evs=None):
        k = i % 2
        host = draws[i % n_draws][0]
        with torch.cuda.stream(copy_stream):
            copy_stream.wait_event(done[k])       # replay i - 2 has finished with set k
            fill(sets[k], host)                   # returns once the copies are done
        main.wait_stream(copy_stream)
        if evs is not None:
            evs[0].record(main)
        graphs[k].replay()
        if evs is not None:
            evs[1].record(main)
        done[k].record(main)

    for w in range(args.warmup):
        replay(w)
    torch.cuda.synchronize()
    if ver.error_word() != 0:
        raise RuntimeError(f"device error word {ver.error_word():#x}")
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    flops_all = bytes_all = alg_all = 0
    t0 = time.perf_counter()
    for i in range(args.steps):
        replay(args.warmup + i, evs[i])
        _, fl, kb, ab = draws[(args.warmup + i) % n_draws]
        flops_all += fl
        bytes_all += kb
        alg_all += ab
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if ver.error_word() != 0:
        raise RuntimeError(f"device error word {ver.error_word():#x}")
    rep_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    total_s = float(rep_ms.sum()) * 1e-3
    t_hbm = alg_all / (PEAK_HBM_GBS * 1e9)
    t_mfma = flops_all / (PEAK_MFMA_BF16_TFLOPS * 1e12)
    bound = "mfma" if t_mfma >= t_hbm else "hbm"
    achieved = (flops_all / total_s / 1e12) if bound == "mfma" else (alg_all / total_s / 1e9)
    peak = PEAK_MFMA_BF16_TFLOPS if bound == "mfma" else PEAK_HBM_GBS
    achievable = None
    if not args.no_achievable:
        peaks = achievable_peaks(torch, B)
        t_roof_a = max(alg_all / (peaks["hbm_read_GBps"] * 1e9), flops_all / (peaks["mfma_bf16_TFLOPs"] * 1e12))
        achievable = with_achievable(peaks, bound, achieved, t_roof_a, total_s)
    result = {
        "metric": f"µs/call + effective KV GB/s & %roofline, {GRAPH_WORKLOAD}",
        "value": bytes_all / total_s / 1e9,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": DESCRIPTIONS[GRAPH_WORKLOAD], "name": GRAPH_WORKLOAD,
                   "batch": gen.SEGMENTED["batch"], "heads": h, "distinct_draws": n_draws,
                   "mean_keys_per_replay": bytes_all / 1152 / args.steps},
        "us_per_call": float(rep_ms.mean() * 1e3),
        "us_per_call_each_p10_p50_p90": [float(np.percentile(rep_ms, q) * 1e3) for q in (10, 50, 90)],
        "tflops_per_call": flops_all / total_s / 1e12,
        "algorithmic": {"flops_per_call": flops_all / args.steps, "kv_bytes_per_call": bytes_all / args.steps,
                        "bytes_per_call": alg_all / args.steps},
        "roofline": {"bound": bound, "achieved": achieved, "peak": peak,
                     "unit": "TFLOP/s" if bound == "mfma" else "GB/s", "frac": achieved / peak,
                     "traffic": None, "kernel": "whole call (graph replay: split partials with the device-side plan, merge)"},
        "roofline_call": {"frac": max(t_hbm, t_mfma) / total_s, "frac_hbm": t_hbm / total_s,
                          "frac_mfma": t_mfma / total_s},
        "achievable": achievable,
        "cpu_baseline": None,
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
