"""Benchmark: MLA decode over a paged bf16 latent cache on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload mixed]

One step is one pass of the whole decode path over one synthetic batch:
mla_get_metadata (split-KV plan) then mla_decode_fwd (decode kernel + split
combine). Each step reads a different replica of (kcache, block_table, q), and
the replicas together exceed twice the 256 MB Infinity Cache, so the cache is
read from HBM. After W untimed steps, K steps captured in one HIP graph are replayed
between two events on the launch stream. Prints one JSON line.

The default workload is mixed (B=128, s_q=2, h_q=128), the largest one-GPU
configuration; it sits above the ridge of the roofline, so value is TFLOP/s
(the QK^T + PV MAC flops per step / step time) and gbs beside it the
algorithmic bytes per step / step time (each cached row counted once, plus q,
out, lse, the used block-table entries and cache_seqlens). Below the ridge
(memory_bound, long, tiny) value is GB/s. The plan alone (plan_ms) and the
decode call alone (decode_fwd_ms) are timed the same way. The roofline entry
is for the decode kernel alone: K launches (graphs holding only
mla_decode_fwd_splits) run back to back over the replicas between two events
on the same stream, and achieved = algorithmic flops (or bytes) per launch / the
average launch time.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads as wl  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2516.6      # MI355X dense bf16 MFMA, published (256 CU x 4096 flop/clk x 2.4 GHz)
MALL_BYTES = 256 * 2 ** 20
CSRC = os.path.join(ROOT, "mla_paged_latent_amd", "csrc")
# the sources that decide each benchmark case's dominant kernel and its traffic: the kernel's own file, the
# shared headers and, for the decode kernels, the plan and its sizing (they set the split partials it writes)
PLAN_SRCS = ("mla_plan.hip", "mla_api.hip")
KERNEL_SRCS = {
    "decode_wide_kernel": ("mla_decode_wide.hip", "mla_device.h", "mla_common.h") + PLAN_SRCS,
    "decode_wide_fp8_kernel": ("mla_decode_wide_fp8.hip", "mla_device.h", "mla_common.h") + PLAN_SRCS,
    "stream": ("mla_decode.hip", "mla_device.h", "mla_common.h") + PLAN_SRCS,
    "append": ("mla_append.hip", "mla_device.h", "mla_common.h"),
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def traffic_key(op: str, workload: str) -> str:
    """Name of a benchmark case in profiles/traffic.json."""
    if op == "decode":
        return workload
    if op == "fp8":
        return "fp8_" + workload
    return op


def traffic_kernel(key: str) -> str:
    """The dominant kernel of a case (a substring of its name in rocprofv3 output)."""
    if key in ("compute_bound", "mixed"):
        return "decode_wide_kernel"
    if key in ("fp8_compute_bound", "fp8_mixed"):
        return "decode_wide_fp8_kernel"
    if key.startswith("fp8_"):
        return "decode_stream_fp8_kernel"
    if key == "sparse":
        return "decode_stream_kernel<1, true>"
    if key in ("append", "append_fp8"):
        return key + "_kernel"
    return "decode_stream_kernel<1, false>"


def kernel_source_digest(key: str = "memory_bound") -> str:
    """Digest of the sources of a case's dominant kernel: its traffic counters stay valid
    while these files are unchanged."""
    kname = traffic_kernel(key)
    files = KERNEL_SRCS.get(kname) or KERNEL_SRCS["append" if key.startswith("append") else "stream"]
    h = hashlib.sha256()
    for name in files:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(key: str):
    """HBM bytes per launch of the case's dominant kernel from committed rocprofv3
    counter runs, if they were taken on the current source of that kernel; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            doc = json.load(f)
    except (OSError, ValueError):
        return None
    ent = doc.get(key)
    if not ent or ent.get("kernel_source_sha") != kernel_source_digest(key):
        return None
    return ent.get("hbm_bytes_per_launch")


def cpu_model() -> str:
    """The host CPU's model name (first 'model name' line of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def spread_sample(batch: int, k: int):
    """k sequence indices spread evenly over [0, batch) (so a sample keeps the batch's length mix)."""
    k = max(1, min(int(k), batch))
    return sorted(set(int(round(x)) for x in np.linspace(0, batch - 1, k)))


def median_rate(seconds, nbytes, flops):
    """(median seconds, GB/s, TFLOP/s) of repeated passes over a sample of nbytes / flops."""
    med = float(np.median(np.asarray(seconds, dtype=np.float64)))
    return med, nbytes / med / 1e9, flops / med / 1e12


def cpu_baseline(inp, bound: str, budget_s: float = 20.0, one_thread: bool = False):
    """The oracle, as it is, on the host cores: a sample of the batch's sequences (spread
    over the batch) sized so that one pass takes about budget_s / 5 seconds, timed three
    times; the median pass gives the rates. With one_thread, the same on one thread."""
    import oracle
    oracle.load()
    threads = oracle.default_threads()

    def passes(sub, nth, n=3):
        out = []
        for _ in range(n):
            t0 = time.perf_counter()
            oracle.decode_inputs(sub, nthreads=nth)
            out.append(time.perf_counter() - t0)
        return out

    def sized_sample(nth, target):
        # calibrate on one sequence, then grow the sample to about `target` seconds per pass
        k = 1
        while True:
            idx = spread_sample(inp.batch, k)
            sub = wl.subset(inp, idx)
            t0 = time.perf_counter()
            oracle.decode_inputs(sub, nthreads=nth)
            el = time.perf_counter() - t0
            if el >= target / 4 or len(idx) == inp.batch:
                break
            k = min(inp.batch, max(k + 1, int(k * min(8.0, target / max(el, 1e-4)))))
        if el < target and len(idx) < inp.batch:
            idx = spread_sample(inp.batch, min(inp.batch, max(len(idx), int(len(idx) * target / max(el, 1e-4)))))
        return idx

    def leg(nth, target):
        idx = sized_sample(nth, target)
        sub = wl.subset(inp, idx)
        nb, fl = wl.algorithmic_counts(sub.cache_seqlens, sub.s_q, sub.h_q, sub.causal)
        secs = passes(sub, nth)
        med, gbs, tf = median_rate(secs, nb, fl)
        return idx, secs, med, gbs, tf

    idx, secs, med, gbs, tf = leg(threads, budget_s / 5)
    res = {"value": round(tf, 6) if bound == "mfma" else round(gbs, 4),
           "unit": "TFLOP/s" if bound == "mfma" else "GB/s",
           "cores": threads, "kind": "oracle", "gbs": round(gbs, 4), "tflops": round(tf, 6),
           "cpu_model": cpu_model(), "nproc": os.cpu_count(),
           "sample": "%d of the %d sequences of the %s batch (evenly spread), float64 oracle on %d threads, "
                     "median of 3 passes (%s s)" % (len(idx), inp.batch, inp.name, threads,
                                                   ", ".join("%.2f" % x for x in secs))}
    if one_thread:
        idx1, secs1, med1, gbs1, tf1 = leg(1, budget_s / 5)
        res["one_thread"] = {"gbs": round(gbs1, 4), "tflops": round(tf1, 6),
                             "sample": "%d of the %d sequences, 1 thread, median of 3 passes (%s s)"
                                       % (len(idx1), inp.batch, ", ".join("%.2f" % x for x in secs1))}
    return res


def context_ceilings(torch, dev):
    """Measured ceilings of this GPU, for context beside the spec peaks: a 1 GiB device copy
    (torch's copy kernel; read + write bytes / time) and an 8192^3 bf16 GEMM (torch.matmul)."""
    n = 2 ** 30
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    a = torch.randn(8192, 8192, device=dev).to(torch.bfloat16)
    b = torch.randn(8192, 8192, device=dev).to(torch.bfloat16)
    torch.cuda.synchronize()

    def best(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        t = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            t.append(e0.elapsed_time(e1))
        return min(t)

    ms_copy = best(lambda: dst.copy_(src))
    ms_gemm = best(lambda: a @ b)
    del src, dst, a, b
    return {"copy_gbs": round(2 * n / (ms_copy * 1e-3) / 1e9, 1),
            "gemm_bf16_tflops": round(2 * 8192 ** 3 / (ms_gemm * 1e-3) / 1e12, 1),
            "how": "best of 5: 1 GiB torch copy (read + write bytes), 8192^3 bf16 torch.matmul"}


def _counter_means(csv_dir, counter, name_part):
    """Mean value of `counter` per dispatch of kernels whose name contains name_part,
    from a rocprofv3 --pmc csv output directory."""
    import csv
    import glob
    vals = []
    for path in glob.glob(os.path.join(csv_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for row in csv.DictReader(f):
                if row["Counter_Name"] == counter and name_part in row["Kernel_Name"]:
                    vals.append(float(row["Counter_Value"]))
    if not vals:
        raise SystemExit("no %s samples for kernels matching %r under %s" % (counter, name_part, csv_dir))
    return sum(vals) / len(vals), len(vals)


def pmc_summary(args):
    """Turn FETCH_SIZE / WRITE_SIZE counter runs of a case's dominant kernel, and the same
    counters over a plain device copy of known size, into HBM bytes per launch; stored in
    profiles/traffic.json under the case's name (traffic_key)."""
    fetch_dir, write_dir, cfetch_dir, cwrite_dir = args.pmc_summary
    key = traffic_key(args.op, args.workload)
    kname = traffic_kernel(key)
    copy_bytes = args.copy_bytes
    cf, _ = _counter_means(cfetch_dir, "FETCH_SIZE", "copy")
    cw, _ = _counter_means(cwrite_dir, "WRITE_SIZE", "copy")
    f_fetch = copy_bytes / (cf * 1024.0)       # counters are in KiB
    f_write = copy_bytes / (cw * 1024.0)
    kf, nf = _counter_means(fetch_dir, "FETCH_SIZE", kname)
    kw, nw = _counter_means(write_dir, "WRITE_SIZE", kname)
    ent = {
        "kernel": kname,
        "fetch_kib_per_dispatch": round(kf, 1), "write_kib_per_dispatch": round(kw, 1),
        "dispatches": [nf, nw],
        "copy_calibration_bytes": copy_bytes,
        "copy_fetch_kib": round(cf, 1), "copy_write_kib": round(cw, 1),
        "factor_fetch": round(f_fetch, 4), "factor_write": round(f_write, 4),
        "hbm_bytes_per_launch": int(kf * 1024.0 * f_fetch + kw * 1024.0 * f_write),
        "kernel_source_sha": kernel_source_digest(key),
    }
    try:
        with open(TRAFFIC_FILE) as f:
            doc = json.load(f)
    except (OSError, ValueError):
        doc = {}
    doc[key] = ent
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(doc, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps({key: ent}))
    return 0


def inp_flops(inp):
    return wl.algorithmic_counts(inp.cache_seqlens, inp.s_q, inp.h_q, inp.causal)[1]


def bench_append(args, torch, mla, dev):
    """The cache append alone: K launches of mla_append_kv (bf16 copy) or, for
    --op append_fp8, of mla_append_kv_fp8 (quantizing append), over replicas of
    (cache, new rows)."""
    fp8 = args.op == "append_fp8"
    inp = wl.make_append()
    B, s_new, width = inp.new_rows.shape
    nbytes = wl.append_bytes(inp, fp8=fp8)
    nblocks = inp.kcache.shape[0]
    cache_bytes = nblocks * wl.PAGE * (width + 4) if fp8 else inp.kcache.nbytes
    rep_bytes = cache_bytes + inp.new_rows.nbytes
    R = args.replicas or max(2, math.ceil(2 * MALL_BYTES / rep_bytes))

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    table = torch.from_numpy(inp.block_table).to(dev)
    lens = torch.from_numpy(inp.cache_seqlens).to(dev)
    if fp8:
        reps = [(torch.zeros((nblocks, wl.PAGE, width), dtype=torch.uint8, device=dev),
                 torch.zeros((nblocks, wl.PAGE), dtype=torch.float32, device=dev), bf16(inp.new_rows))
                for _ in range(R)]
    else:
        reps = [(bf16(inp.kcache), bf16(inp.new_rows)) for _ in range(R)]

    def step(k):
        if fp8:
            c, sc, rows = reps[k % R]
            mla.mla_append_kv_fp8(c, sc, table, lens, rows)
        else:
            kc, rows = reps[k % R]
            mla.mla_append_kv(kc, table, lens, rows)

    for k in range(max(args.warmup, R)):
        step(k)
    torch.cuda.synchronize()
    cap = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        for k in range(args.steps):
            step(k)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    gbs = nbytes / (ms * 1e-3) / 1e9
    kname = "append_fp8_kernel (mla_append_kv_fp8)" if fp8 else "append_kernel (mla_append_kv)"
    result = {
        "metric": "MLA cache append HBM GB/s (fraction of MI355X peak), paged %s"
                  % ("FP8 (E4M3 + per-row scale) from bf16 rows" if fp8 else "bf16"),
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 6), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 in, fp8e4m3 + f32 scale out" if fp8 else "bf16", "data": "synthetic",
        "config": {"workload": "append%s: %s, row 576, block 64, shuffled block_table"
                               % ("_fp8" if fp8 else "", wl.APPEND_DESCRIPTION),
                   "batch": int(B), "s_new": int(s_new), "replicas": R},
        "alg_bytes_per_step": nbytes,
        "roofline": {"bound": "hbm", "kernel": kname, "achieved": round(gbs, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(args.op), "kernel_ms_avg": round(ms, 6)},
    }
    if not args.no_cpu_baseline:
        from oracle import append as oracle_append
        from oracle import fp8 as oracle_fp8
        if fp8:
            c0 = np.zeros((nblocks, wl.PAGE, width), dtype=np.uint8)
            s0 = np.zeros((nblocks, wl.PAGE), dtype=np.float32)
        t0 = time.perf_counter()
        n = 0
        while True:
            if fp8:
                oracle_fp8.append_rows_fp8(c0, s0, inp.block_table, inp.cache_seqlens, inp.new_rows)
            else:
                oracle_append.append_rows(inp.kcache, inp.block_table, inp.cache_seqlens, inp.new_rows)
            n += 1
            if time.perf_counter() - t0 >= min(args.cpu_seconds, 10.0) or n >= 50:
                break
        sec = (time.perf_counter() - t0) / n
        result["cpu_baseline"] = {"value": round(nbytes / sec / 1e9, 4), "unit": "GB/s", "cores": 1,
                                  "kind": "oracle",
                                  "sample": "%d full appends of the workload (copy of the cache included)" % n}
    print(json.dumps(result), flush=True)
    return 0


def graph_ms(torch, fn, n):
    """fn(0), ..., fn(n - 1) captured in one HIP graph (on a side stream), replayed once,
    then one replay timed with events on the current stream: ms per call."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        for k in range(n):
            fn(k)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def kernel_roofline(mla, name, lens, h_q, s_q, units, nbytes, flops, kern_ms, traffic, plan_h_q=None):
    """Roofline entry of a decode kernel timed alone (a *_splits call): out/lse of the
    sequences (lists) the plan splits are the combine kernel's bytes, not the kernel's.
    plan_h_q: the head count whose geometry the plan used (sparse plans: 16-row units)."""
    _, host_splits = mla.mla_get_metadata_host(lens, plan_h_q or h_q, s_q, units)
    split_rows = int((np.diff(host_splits) > 1).sum()) * s_q * h_q
    kb = nbytes - split_rows * (2 * wl.D_V + 4)
    k_gbs = kb / (kern_ms * 1e-3) / 1e9
    k_tf = flops / (kern_ms * 1e-3) / 1e12
    r = {"bound": "hbm", "kernel": name, "achieved": round(k_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
         "frac": round(k_gbs / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel_alg_bytes": kb,
         "kernel_ms_avg": round(kern_ms, 6), "kernel_tflops": round(k_tf, 3),
         "kernel_mfma_frac": round(k_tf / BF16_PEAK_TFLOPS, 5)}
    if flops / nbytes >= BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9):
        # above the ridge (the matrix ops run in bf16): judged against the bf16 matrix peak
        r.update({"bound": "mfma", "achieved": round(k_tf, 3), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                  "frac": round(k_tf / BF16_PEAK_TFLOPS, 5), "kernel_gbs": round(k_gbs, 2),
                  "kernel_hbm_frac": round(k_gbs / HBM_PEAK_GBS, 4)})
    return r


def bench_sparse(args, torch, mla, dev):
    """Sparse decode: plan (mla_get_metadata_sparse) + mla_decode_sparse_fwd per step."""
    sp = wl.make_sparse()
    d = sp.dec
    B, s_q, h_q = d.batch, d.s_q, d.h_q
    topk = sp.indices.shape[2]
    nbytes, flops = wl.sparse_counts(sp)
    rep_bytes = d.kcache.nbytes + d.q.nbytes
    R = args.replicas or max(2, math.ceil(2 * MALL_BYTES / rep_bytes))

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    table = torch.from_numpy(d.block_table).to(dev)
    idx = torch.from_numpy(sp.indices).to(dev)
    lens = torch.from_numpy(sp.counts).to(dev)
    reps = [(bf16(d.kcache), bf16(d.q)) for _ in range(R)]
    sizes = mla.mla_sparse_plan_sizes(B, s_q, h_q, topk)
    units = sizes["num_units"]
    meta = torch.empty((units, mla.META_INTS), dtype=torch.int32, device=dev)
    splits = torch.empty((B * s_q + 1,), dtype=torch.int32, device=dev)
    out = torch.empty((B, s_q, h_q, mla.D_V), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, s_q, h_q), dtype=torch.float32, device=dev)
    ws = torch.empty((sizes["workspace_bytes"],), dtype=torch.uint8, device=dev)

    def step(k):
        kc, q = reps[k % R]
        mla.mla_get_metadata_sparse(lens, B, s_q, h_q, topk, num_units=units, tile_meta=meta, num_splits=splits)
        mla.mla_decode_sparse_fwd(q, kc, table, idx, lens, d.softmax_scale, meta, splits, out=out, lse=lse,
                                  workspace=ws)

    for k in range(max(args.warmup, R)):
        step(k)
    torch.cuda.synchronize()
    cap = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        for k in range(args.steps):
            step(k)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps

    def decode_only(k):
        kc, q = reps[k % R]
        mla.mla_decode_sparse_fwd_splits(q, kc, table, idx, lens, d.softmax_scale, meta, splits, out=out, lse=lse,
                                         workspace=ws)
    kern_ms = graph_ms(torch, decode_only, args.steps)

    def plan_only(k):
        mla.mla_get_metadata_sparse(lens, B, s_q, h_q, topk, num_units=units, tile_meta=meta, num_splits=splits)

    def decode_fwd(k):
        kc, q = reps[k % R]
        mla.mla_decode_sparse_fwd(q, kc, table, idx, lens, d.softmax_scale, meta, splits, out=out, lse=lse,
                                  workspace=ws)
    # the plan alone and the decode call alone (decode kernel + combine), K launches back to back
    plan_ms = graph_ms(torch, plan_only, args.steps)
    fwd_ms = graph_ms(torch, decode_fwd, args.steps)
    gbs = nbytes / (ms * 1e-3) / 1e9
    tf = flops / (ms * 1e-3) / 1e12
    result = {
        "metric": "MLA sparse (top-k) decode HBM GB/s + TFLOPS (fraction of MI355X peak), paged bf16",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 6), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "sparse: " + wl.SPARSE_DESCRIPTION + ", d_qk=576, d_v=512, block 64, shuffled "
                               "block_table, bf16 N(0,1), scale 1/sqrt(192)",
                   "batch": B, "s_q": s_q, "h_q": h_q, "topk": topk, "replicas": R, "num_units": units},
        "step": "mla_get_metadata_sparse + mla_decode_sparse_fwd (plan, decode kernel, split combine)",
        "tflops": round(tf, 3), "plan_ms": round(plan_ms, 6), "decode_fwd_ms": round(fwd_ms, 6),
        "alg_bytes_per_step": nbytes, "alg_flops_per_step": flops,
        "roofline": kernel_roofline(mla, "sparse decode kernel (mla_decode_sparse_fwd_splits)", sp.counts, h_q, 1,
                                    units, nbytes, flops, kern_ms, measured_traffic("sparse"), plan_h_q=16),
    }
    if not args.no_cpu_baseline:
        import oracle as orc
        nth = orc.default_threads()
        sample = [0, 1, 2, 3]
        sub = wl.subset(d, sample)
        t0 = time.perf_counter()
        n = 0
        while True:
            orc.mla_decode_sparse(sub.q, sub.kcache, sub.block_table, sp.indices[sample], sp.counts[sample],
                                  d.softmax_scale, nthreads=nth)
            n += 1
            if time.perf_counter() - t0 >= min(args.cpu_seconds, 10.0) or n >= 20:
                break
        sec = (time.perf_counter() - t0) / n * (B / len(sample))
        result["cpu_baseline"] = {"value": round(nbytes / sec / 1e9, 4), "unit": "GB/s", "cores": nth,
                                  "kind": "oracle",
                                  "sample": "%d passes over sequences %s of the batch, scaled to all %d" % (n, sample, B)}
    print(json.dumps(result), flush=True)
    return 0


def bench_fp8(args, torch, mla, dev):
    """Decode over the FP8 cache: plan (mla_get_metadata_fp8) + mla_decode_fp8_fwd per step.
    The cache is the named workload's bf16 cache, quantized on the GPU by mla_append_kv_fp8
    (each sequence appended whole), then copied into R replicas."""
    inp = wl.make_workload(args.workload, poison=False)
    B, s_q, h_q = inp.batch, inp.s_q, inp.h_q
    nbytes, flops = wl.fp8_counts(inp.cache_seqlens, s_q, h_q, inp.causal)
    nblocks = inp.kcache.shape[0]

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    table = torch.from_numpy(inp.block_table).to(dev)
    lens = torch.from_numpy(inp.cache_seqlens).to(dev)
    codes0 = torch.zeros((nblocks, wl.PAGE, wl.D_QK), dtype=torch.uint8, device=dev)
    scales0 = torch.zeros((nblocks, wl.PAGE), dtype=torch.float32, device=dev)
    mla.mla_append_kv_fp8(codes0, scales0, table, lens, bf16(wl.rows_in_token_order(inp)))
    torch.cuda.synchronize()
    rep_bytes = codes0.numel() + 4 * scales0.numel() + inp.q.nbytes + inp.block_table.nbytes
    R = args.replicas or max(2, math.ceil(2 * MALL_BYTES / rep_bytes))
    q0 = bf16(inp.q)
    reps = [(codes0.clone(), scales0.clone(), q0.clone(), table.clone(), lens.clone()) for _ in range(R)]
    del codes0, scales0, q0
    sizes = mla.mla_fp8_plan_sizes(B, s_q, h_q)
    units = args.num_units or sizes["num_units"]
    sizes["workspace_bytes"] = mla.mla_workspace_bytes(B, s_q, h_q, units)
    plans = [(torch.empty((units, mla.META_INTS), dtype=torch.int32, device=dev),
              torch.empty((B + 1,), dtype=torch.int32, device=dev)) for _ in range(R)]
    out = torch.empty((B, s_q, h_q, mla.D_V), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, s_q, h_q), dtype=torch.float32, device=dev)
    ws = torch.empty((max(sizes["workspace_bytes"], 16),), dtype=torch.uint8, device=dev)

    def step(k):
        c, sc, q, tab, ln = reps[k % R]
        meta, splits = plans[k % R]
        mla.mla_get_metadata_fp8(ln, h_q, s_q, num_units=units, tile_meta=meta, num_splits=splits)
        mla.mla_decode_fp8_fwd(q, c, sc, tab, ln, inp.softmax_scale, meta, splits, causal=inp.causal, out=out,
                               lse=lse, workspace=ws)

    for k in range(max(args.warmup, R)):
        step(k)
    torch.cuda.synchronize()
    cap = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        for k in range(args.steps):
            step(k)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps

    def decode_only(k):
        c, sc, q, tab, ln = reps[k % R]
        meta, splits = plans[k % R]
        mla.mla_decode_fp8_fwd_splits(q, c, sc, tab, ln, inp.softmax_scale, meta, splits, causal=inp.causal,
                                      out=out, lse=lse, workspace=ws)
    kern_ms = graph_ms(torch, decode_only, args.steps)

    def plan_only(k):
        meta, splits = plans[k % R]
        mla.mla_get_metadata_fp8(reps[k % R][4], h_q, s_q, num_units=units, tile_meta=meta, num_splits=splits)

    def decode_fwd(k):
        c, sc, q, tab, ln = reps[k % R]
        meta, splits = plans[k % R]
        mla.mla_decode_fp8_fwd(q, c, sc, tab, ln, inp.softmax_scale, meta, splits, causal=inp.causal, out=out,
                               lse=lse, workspace=ws)
    # the plan alone and the decode call alone (decode kernel + combine), K launches back to back
    plan_ms = graph_ms(torch, plan_only, args.steps)
    fwd_ms = graph_ms(torch, decode_fwd, args.steps)
    gbs = nbytes / (ms * 1e-3) / 1e9
    tf = flops / (ms * 1e-3) / 1e12
    result = {
        "metric": "MLA decode over an FP8 (E4M3 + per-row scale) paged latent cache, HBM GB/s + TFLOPS",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 6), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8e4m3 cache, bf16 query/output, f32 accumulate", "data": "synthetic",
        "config": {"workload": "fp8 %s: %s, cache quantized per row (E4M3, f32 scale), d_qk=576, d_v=512, block 64, "
                               "shuffled block_table, scale 1/sqrt(192)"
                               % (args.workload, wl.DESCRIPTIONS[args.workload]),
                   "batch": B, "s_q": s_q, "h_q": h_q, "tokens": int(inp.cache_seqlens.sum()), "replicas": R,
                   "num_units": units},
        "step": "mla_get_metadata_fp8 + mla_decode_fp8_fwd (plan, decode kernel, split combine)",
        "tflops": round(tf, 3), "plan_ms": round(plan_ms, 6), "decode_fwd_ms": round(fwd_ms, 6),
        "alg_bytes_per_step": nbytes, "alg_flops_per_step": flops,
        "roofline": kernel_roofline(mla, "FP8 decode kernel (mla_decode_fp8_fwd_splits)", inp.cache_seqlens, h_q,
                                    s_q, units, nbytes, flops, kern_ms, measured_traffic("fp8_" + args.workload)),
    }
    if not args.no_cpu_baseline:
        import oracle as orc
        from oracle import fp8 as ofp8
        nth = orc.default_threads()
        codes, scales = ofp8.quantize_rows(inp.kcache)
        sample = [0, 1]
        sub = wl.subset(inp, sample)
        t0 = time.perf_counter()
        n = 0
        while True:
            orc.mla_decode_fp8(sub.q, codes, scales, sub.block_table, sub.cache_seqlens, inp.softmax_scale,
                               inp.causal, nthreads=nth)
            n += 1
            if time.perf_counter() - t0 >= min(args.cpu_seconds, 10.0) or n >= 20:
                break
        sec = (time.perf_counter() - t0) / n
        sub_bytes = wl.fp8_counts(sub.cache_seqlens, s_q, h_q, inp.causal)[0]
        result["cpu_baseline"] = {"value": round(sub_bytes / sec / 1e9, 4), "unit": "GB/s", "cores": nth,
                                  "kind": "oracle",
                                  "sample": "%d passes over sequences %s of the batch" % (n, sample)}
    print(json.dumps(result), flush=True)
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="mixed", choices=sorted(wl.WORKLOADS),
                    help="default: mixed, the largest single-GPU configuration")
    ap.add_argument("--replicas", type=int, default=0, help="0: enough to exceed 2x the 256 MB cache")
    ap.add_argument("--num-units", type=int, default=0,
                    help="decode / fp8: plan over this many units instead of the library's choice (0)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0, help="about the CPU-baseline leg's wall time")
    ap.add_argument("--no-context", action="store_true", help="skip the copy / GEMM ceiling measurements")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (for counter calibration) and exit")
    ap.add_argument("--pmc-summary", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="no GPU: write the HBM bytes per launch of the dominant kernel of --op/--workload to "
                         "profiles/traffic.json from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE csv outputs")
    ap.add_argument("--copy-bytes", type=int, default=256 * 2 ** 20, help="size of the calibration copy")
    ap.add_argument("--op", default="decode", choices=["decode", "append", "append_fp8", "sparse", "fp8"],
                    help="decode: the hot path (default); append / append_fp8: the cache-append kernel alone "
                         "(bf16 copy / quantizing FP8 append); sparse: top-k index decode (plan + decode + "
                         "combine); fp8: decode over the FP8 cache of --workload")
    args = ap.parse_args(argv)
    if args.pmc_summary:
        return pmc_summary(args)

    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (--gpus %d refused)" % args.gpus,
              file=sys.stderr)
        return 2

    import torch
    import mla_paged_latent_amd as mla

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_calibration:
        n = args.copy_calibration * 2 ** 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 5}))
        return 0

    mla.load_library()
    if args.op in ("append", "append_fp8"):
        return bench_append(args, torch, mla, dev)
    if args.op == "fp8":
        return bench_fp8(args, torch, mla, dev)
    if args.op == "sparse":
        return bench_sparse(args, torch, mla, dev)
    inp = wl.make_workload(args.workload, poison=False)
    B, s_q, h_q = inp.batch, inp.s_q, inp.h_q
    nbytes, flops = wl.algorithmic_counts(inp.cache_seqlens, s_q, h_q, inp.causal)
    replica_bytes = inp.kcache.nbytes + inp.q.nbytes + inp.block_table.nbytes
    R = args.replicas or max(2, math.ceil(2 * MALL_BYTES / replica_bytes))

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    base_k, base_q = bf16(inp.kcache), bf16(inp.q)
    base_t = torch.from_numpy(inp.block_table).to(dev)
    lens = torch.from_numpy(inp.cache_seqlens).to(dev)
    reps = [(base_k.clone(), base_q.clone(), base_t.clone(), lens.clone()) for _ in range(R)]
    del base_k, base_q, base_t

    sizes = mla.mla_plan_sizes(B, s_q, h_q)
    units = args.num_units or sizes["num_units"]
    sizes["workspace_bytes"] = mla.mla_workspace_bytes(B, s_q, h_q, units)
    out = torch.empty((B, s_q, h_q, mla.D_V), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, s_q, h_q), dtype=torch.float32, device=dev)
    ws = torch.empty((sizes["workspace_bytes"],), dtype=torch.uint8, device=dev)
    plans = [(torch.empty((units, mla.META_INTS), dtype=torch.int32, device=dev),
              torch.empty((B + 1,), dtype=torch.int32, device=dev)) for _ in range(R)]

    def step(k):
        # one pass of the path: the plan (mla_get_metadata), then mla_decode_fwd (decode kernel + combine)
        kc, q, tab, ln = reps[k % R]
        meta, splits = plans[k % R]
        mla.mla_get_metadata(ln, h_q, s_q, num_units=units, tile_meta=meta, num_splits=splits)
        mla.mla_decode_fwd(q, kc, tab, ln, inp.softmax_scale, meta, splits, causal=inp.causal,
                           out=out, lse=lse, workspace=ws)

    def plan_only(k):
        ln = reps[k % R][3]
        meta, splits = plans[k % R]
        mla.mla_get_metadata(ln, h_q, s_q, num_units=units, tile_meta=meta, num_splits=splits)

    def decode_fwd(k):
        kc, q, tab, ln = reps[k % R]
        meta, splits = plans[k % R]
        mla.mla_decode_fwd(q, kc, tab, ln, inp.softmax_scale, meta, splits, causal=inp.causal,
                           out=out, lse=lse, workspace=ws)

    def decode_only(k):
        kc, q, tab, ln = reps[k % R]
        meta, splits = plans[k % R]
        mla.mla_decode_fwd_splits(q, kc, tab, ln, inp.softmax_scale, meta, splits, causal=inp.causal,
                                  out=out, lse=lse, workspace=ws)

    # The timed steps are captured in one HIP graph (step k uses replica k mod R) and replayed
    # once, as a serving loop would run them: the host issues one launch for all K steps, so
    # host-side argument marshalling stays out of the device timeline. The same steps issued
    # eagerly are timed afterwards for reference (eager_ms_per_step).
    for k in range(max(args.warmup, R)):
        step(k)
    torch.cuda.synchronize()
    cap = torch.cuda.Stream()

    def capture(fn, n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            for k in range(n):
                fn(k)
        torch.cuda.synchronize()
        return g

    def timed(run, n):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        e0.record(stream)
        h0 = time.perf_counter()
        run()
        host = (time.perf_counter() - h0) * 1e3 / n
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n, host

    def graph_ms(fn):
        g = capture(fn, args.steps)
        g.replay()
        ms, host = timed(g.replay, args.steps)
        del g
        return ms, host

    steps_graph = capture(step, args.steps)
    if args.warmup:
        capture(step, args.warmup).replay()
    ms_step, host_ms = timed(steps_graph.replay, args.steps)
    del steps_graph
    # the plan alone and the decode call alone (decode kernel + combine), K launches back to back
    plan_ms, _ = graph_ms(plan_only)
    fwd_ms, _ = graph_ms(decode_fwd)
    # the decode kernel alone, K launches back to back over the replicas: the roofline figure
    kern_ms, host_kern_ms = graph_ms(decode_only)
    n_eager = min(args.steps, 50)

    def eager():
        for k in range(n_eager):
            step(k)
    eager_ms, eager_host_ms = timed(eager, n_eager)

    bound = "hbm" if flops / nbytes < BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9) else "mfma"
    gbs = nbytes / (ms_step * 1e-3) / 1e9
    tflops = flops / (ms_step * 1e-3) / 1e12
    # the decode kernel's own algorithmic bytes: out/lse of sequences the plan split are
    # written by the combine kernel, so they are not credited to it
    _, host_splits = mla.mla_get_metadata_host(inp.cache_seqlens, h_q, s_q, units)
    split_rows = int((np.diff(host_splits) > 1).sum()) * s_q * h_q
    kernel_bytes = nbytes - split_rows * (2 * wl.D_V + 4)
    k_gbs = kernel_bytes / (kern_ms * 1e-3) / 1e9
    k_tf = flops / (kern_ms * 1e-3) / 1e12
    traffic = measured_traffic(traffic_key("decode", args.workload))

    result = {
        "metric": "MLA decode TFLOPS + HBM GB/s (fraction of MI355X peak), paged bf16",
        "value": round(tflops, 3) if bound == "mfma" else round(gbs, 2),
        "unit": "TFLOP/s" if bound == "mfma" else "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "%s: %s, d_qk=576, d_v=512, block 64, shuffled block_table, bf16 N(0,1), "
                               "scale 1/sqrt(192)" % (args.workload, wl.DESCRIPTIONS[args.workload]),
                   "batch": B, "s_q": s_q, "h_q": h_q, "tokens": int(inp.cache_seqlens.sum()),
                   "replicas": R, "num_units": units},
        "step": "mla_get_metadata + mla_decode_fwd (plan, decode kernel, split combine); value and "
                "ms_per_step include the plan",
        "tflops": round(tflops, 3),
        "gbs": round(gbs, 2),
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "mfma_frac": round(tflops / BF16_PEAK_TFLOPS, 5),
        "plan_ms": round(plan_ms, 6),
        "decode_fwd_ms": round(fwd_ms, 6),
        "decode_fwd_tflops": round(flops / (fwd_ms * 1e-3) / 1e12, 3),
        "decode_fwd_gbs": round(nbytes / (fwd_ms * 1e-3) / 1e9, 2),
        "host_ms_per_step": round(host_ms, 6),
        "eager_ms_per_step": round(eager_ms, 6),
        "eager_host_ms_per_step": round(eager_host_ms, 6),
        "alg_bytes_per_step": nbytes,
        "alg_flops_per_step": flops,
        "roofline": {
            "bound": bound,
            "kernel": "decode kernel (mla_decode_fwd_splits)",
            "achieved": round(k_gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(k_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel_alg_bytes": kernel_bytes,
            "kernel_ms_avg": round(kern_ms, 6),
            "kernel_tflops": round(k_tf, 3),
            "kernel_mfma_frac": round(k_tf / BF16_PEAK_TFLOPS, 5),
            "host_ms_per_launch": round(host_kern_ms, 6),
        },
    }
    if bound == "mfma":
        r = result["roofline"]
        r.update({"achieved": round(k_tf, 3), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                  "frac": round(k_tf / BF16_PEAK_TFLOPS, 5), "kernel_gbs": round(k_gbs, 2),
                  "kernel_hbm_frac": round(k_gbs / HBM_PEAK_GBS, 4)})
    if not args.no_context:
        result["context"] = context_ceilings(torch, dev)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(inp, bound, budget_s=args.cpu_seconds,
                                              one_thread=args.workload in ("tiny", "memory_bound"))
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
