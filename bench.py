#!/usr/bin/env python3
"""Throughput of the hierarchical beam-search selection step on one MI355X.

One step = one rtopk_beam_step call over a whole [B, beam, V] logit tensor
(pass 1, pass 2, per-batch sort: the entire path, one kernel launch). The
default workload is the B=128, beam=4, k=4, V=40000 fp16 configuration with
26 of 512 beams finished. Inputs are seeded synthetic logits, resident in HBM
before the timed region; the step rotates through a pool of distinct logit
buffers larger than the 256 MB Infinity Cache so every step reads cold HBM.

Prints one JSON line: beam-steps/s (whole job), logit GB/s against the 8 TB/s
HBM peak (roofline of the one kernel), and the CPU oracle's throughput on the
host cores as a baseline.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config b128]
"""
import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_rtopk_step_b128.txt")
KERNEL_SOURCES = [os.path.join(ROOT, "beam_search_top_amd", "csrc", f)
                  for f in ("rtopk_kernels.hip", "rtopk_host.cpp", "rtopk_internal.h", "rtopk_draw.h")]


def kernel_sha():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(s):
    """Bytes the method must move once: every alive logit row, the running
    scores and finished mask, and the [B, k] outputs (ids and scores)."""
    esz = {0: 4, 1: 2, 2: 2}[s.dtype]
    alive_rows = s.B * s.beam - s.n_finished
    return alive_rows * s.V * esz + 4 * s.B * s.beam + s.B * s.beam + 12 * s.B * s.k


def read_traffic(config):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources; else None."""
    if config != "b128" or not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                vals[key.strip()] = val.strip()
    if vals.get("kernel_sha") != kernel_sha():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def read_ceiling(L, ptrs, nbytes, K, cur):
    """Practical HBM ceiling: a plain streaming read (rtopk_read_probe) of the
    step's algorithmic byte count, over the same rotating buffers, replayed
    from a captured graph like the step."""
    import torch
    n = nbytes - nbytes % 16
    out = torch.zeros(1, dtype=torch.int32, device="cuda:0")

    def probe(i, stream):
        rc = L.rtopk_read_probe(ptrs[i % len(ptrs)], n, 0x7fc00001, out.data_ptr(), stream)
        if rc != 0:
            raise RuntimeError("read probe failed")

    cur_s = cur.cuda_stream
    for i in range(20):
        probe(i, cur_s)
    graph = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    cs.wait_stream(cur)
    with torch.cuda.graph(graph, stream=cs):
        for i in range(100):
            probe(i, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    reps = max(1, K // 100)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(cur)
    for _ in range(reps):
        graph.replay()
    end.record(cur)
    torch.cuda.synchronize()
    us = start.elapsed_time(end) * 1e3 / (reps * 100)
    gbps = n / (us * 1e-6) / 1e9
    return {"us_per_launch": us, "bytes": n, "GBps": gbps, "frac_of_peak": gbps / HBM_PEAK_GBPS,
            "kernel": "rtopk_read_probe (16-byte non-temporal loads, 10 per lane, nothing else)"}


def bench_reorder(args):
    """Cache refresh after the selection (rtopk_beam_reorder): a beam-major
    cache of 6 layers x {keys, values} (12 slabs) of B*beam = 128*4 rows of
    16 heads x 32 positions x 64 dims fp16 (64 KiB per row, 384 MiB per
    cache), reordered by seeded beam ids; two caches alternate as source and
    destination, each larger than the 256 MB Infinity Cache. Algorithmic bytes
    = every destination row written once + every distinct source row read
    once (beams that continue the same old beam share its read)."""
    import numpy as np
    import torch

    from beam_search_top_amd import rtopk
    rtopk.load()
    L = rtopk.load()
    dev = torch.device("cuda:0")
    nslabs, B, beam, heads, pos, dim = 12, 128, 4, 16, 32, 64
    row_bytes = heads * pos * dim * 2
    n = nslabs * B * beam * row_bytes
    caches = [torch.empty(n, dtype=torch.uint8, device=dev) for _ in range(2)]
    for c in caches:
        c.random_(0, 256)
    rng = np.random.default_rng(1007)
    ids_h = rng.integers(0, beam, size=(B, beam)).astype(np.int32)
    ids = torch.from_numpy(ids_h).to(dev)
    distinct = sum(len(set(r.tolist())) for r in ids_h)  # source rows per slab actually needed
    cur = torch.cuda.current_stream()

    def step(i):
        src, dst = caches[i % 2], caches[(i + 1) % 2]
        rc = L.rtopk_beam_reorder(src.data_ptr(), dst.data_ptr(), nslabs, B, beam, row_bytes, ids.data_ptr(), beam,
                                  cur.cuda_stream)
        if rc != 0:
            raise RuntimeError(rtopk.rtopk_last_error())

    def timed(fn, K):
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(cur)
        for i in range(K):
            fn(i)
        end.record(cur)
        torch.cuda.synchronize()
        return start.elapsed_time(end) / K

    K = max(1, min(args.steps, 400))
    for i in range(max(2, min(args.warmup, 20))):
        step(i)
    ms = timed(step, K)
    alg = n + nslabs * distinct * row_bytes
    gbps = alg / (ms * 1e-3) / 1e9
    # practical ceiling: a plain device copy of the same bytes (torch's copy kernel)
    copy_ms = timed(lambda i: caches[(i + 1) % 2].copy_(caches[i % 2]), K)
    copy_gbps = 2 * n / (copy_ms * 1e-3) / 1e9
    line = {
        "metric": "KV-cache beam reorder (cache refresh) GB/s, read + write, 1xMI355X",
        "value": gbps, "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u8", "data": "synthetic",
        "config": {"workload": f"reorder_b128: {nslabs} slabs (6 layers x K/V) x B={B} x beam={beam} rows of "
                               f"{heads}x{pos}x{dim} fp16 ({row_bytes} B), seeded beam ids",
                   "slabs": nslabs, "B": B, "beam": beam, "row_bytes": row_bytes},
        "algorithmic_bytes_per_step": alg,
        "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": gbps / HBM_PEAK_GBPS, "traffic": None},
        "copy_ceiling": {"GBps": copy_gbps, "ms": copy_ms,
                         "kernel": "torch device copy_ of one whole cache (reads and writes every row once)"},
        "distinct_source_rows": distinct, "rows": B * beam,
        "frac_of_copy_ceiling": gbps / copy_gbps,
    }
    print(json.dumps(line), flush=True)


def bench_sample(args):
    """Top-k sampling decode (rtopk_sample_step): R = 512 rows (sequences) of
    V = 40000 fp16 logits ~ N(0, 3), k = 40, temperature 1, one Philox draw
    per row; rows rotate through a 1 GiB pool so every step reads cold HBM.
    Algorithmic bytes = every logit once + the [R] token and log-prob outputs."""
    import numpy as np
    import torch

    from beam_search_top_amd import rtopk
    L = rtopk.load()
    dev = torch.device("cuda:0")
    R, V, k = 512, 40000, 40
    rng = np.random.default_rng(1008)
    x0 = torch.from_numpy(rng.normal(0, 3.0, size=(R, V)).astype(np.float16)).to(dev)
    nbuf = max(1, math.ceil(args.pool_mib * 2**20 / (R * V * 2)))
    pool = [x0] + [torch.roll(x0, shifts=7919 * i, dims=1).contiguous() for i in range(1, nbuf)]
    tok = torch.empty(R, dtype=torch.int32, device=dev)
    lp = torch.empty(R, dtype=torch.float32, device=dev)
    cur = torch.cuda.current_stream()

    def launch(i, stream):
        rc = L.rtopk_sample_step(pool[i % nbuf].data_ptr(), 1, R, V, k, 1.0, 77, i, tok.data_ptr(), lp.data_ptr(),
                                 stream)
        if rc != 0:
            raise RuntimeError(rtopk.rtopk_last_error())

    for i in range(max(2, args.warmup)):
        launch(i, cur.cuda_stream)
    graph = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    cs.wait_stream(cur)
    launch(0, cs.cuda_stream)  # the library workspace of the capture stream exists before capture
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=cs):
        for i in range(100):
            launch(i, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    reps = max(1, args.steps // 100)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(cur)
    for _ in range(reps):
        graph.replay()
    end.record(cur)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / (reps * 100)
    alg = R * V * 2 + 8 * R
    gbps = alg / (ms * 1e-3) / 1e9
    line = {
        "metric": "top-k sampling decode steps/sec and logit GB/s (% HBM peak), 1xMI355X",
        "value": 1e3 / ms, "unit": "sample-steps/s", "n_gpus": 1, "steps": reps * 100, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": f"sample_r512: R={R} rows x V={V} fp16 N(0,3), k={k}, temperature 1, seed 1008",
                   "R": R, "V": V, "k": k, "logit_pool_buffers": nbuf},
        "algorithmic_bytes_per_step": alg,
        "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": gbps / HBM_PEAK_GBPS, "traffic": None},
    }
    print(json.dumps(line), flush=True)


MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix-core peak


def bench_lmhead(args):
    """The step fused into the LM head (rtopk_lmhead_step): hidden states
    [B*beam, H] and the [V, H] output projection in bfloat16 for B=128,
    beam=4, H=1024 (the hidden size of the LightSeq training article's
    benchmark model), V=40000, k=4, 26 of 512 beams finished; seeded synthetic
    values (hidden N(0,1), weights N(0, 3/sqrt(H)), so logits are about
    N(0,3)). The weights rotate through a pool larger than the 256 MB
    Infinity Cache so every step reads them from HBM. The roofline is the
    matrix cores' (2 M V H flops per step against the 2.5 PFLOP/s dense bf16
    peak). For reference the same step unfused is timed too: torch's GEMM
    (hipBLASLt) writing bf16 logits, then rtopk_beam_step on them."""
    import numpy as np
    import torch

    from beam_search_top_amd import rtopk, synth
    L = rtopk.load()
    dev = torch.device("cuda:0")
    B, beam, H, V, k = 128, 4, 1024, 40000, 4
    M = B * beam
    rng = np.random.default_rng(1009)
    x = torch.from_numpy(rng.normal(0, 1, (M, H)).astype(np.float32)).to(dev).to(torch.bfloat16)
    w0 = torch.from_numpy(rng.normal(0, 3.0 / np.sqrt(H), (V, H)).astype(np.float32)).to(dev).to(torch.bfloat16)
    nbuf = max(1, math.ceil(args.pool_mib * 2**20 / (V * H * 2)))
    pool = [w0] + [torch.roll(w0, shifts=7 * i, dims=1).contiguous() for i in range(1, nbuf)]
    alive = torch.from_numpy(rng.uniform(-30, 0, (B, beam)).astype(np.float32)).to(dev)
    fin_h = np.zeros(M, np.uint8)
    fin_h[rng.choice(M, 26, replace=False)] = 1
    fin = torch.from_numpy(fin_h.reshape(B, beam)).to(dev)
    ob = torch.empty((B, k), dtype=torch.int32, device=dev)
    ot = torch.empty_like(ob)
    osc = torch.empty((B, k), dtype=torch.float32, device=dev)
    cur = torch.cuda.current_stream()

    def launch(i, stream):
        rc = L.rtopk_lmhead_step(x.data_ptr(), pool[i % nbuf].data_ptr(), alive.data_ptr(), fin.data_ptr(), B, beam,
                                 H, V, k, 2, ob.data_ptr(), ot.data_ptr(), osc.data_ptr(), stream)
        if rc != 0:
            raise RuntimeError(rtopk.rtopk_last_error())

    for i in range(max(2, min(args.warmup, 20))):
        launch(i, cur.cuda_stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    cs.wait_stream(cur)
    launch(0, cs.cuda_stream)  # the library workspace of the capture stream exists before capture
    torch.cuda.synchronize()
    glen = 20
    with torch.cuda.graph(graph, stream=cs):
        for i in range(glen):
            launch(i, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    K = max(glen, (min(args.steps, 2000) // glen) * glen)

    def timed(fn, n):
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(cur)
        for i in range(n):
            fn(i)
        end.record(cur)
        torch.cuda.synchronize()
        return start.elapsed_time(end) / n

    trials = [timed(lambda i: graph.replay(), K // glen) / glen for _ in range(5)]
    ms = float(np.median(trials))
    # unfused reference: GEMM to bf16 logits, then the selection on them
    logits = torch.empty((M, V), dtype=torch.bfloat16, device=dev)

    def unfused(i):
        torch.matmul(x, pool[i % nbuf].t(), out=logits)
        rc = L.rtopk_beam_step(logits.data_ptr(), 2, alive.data_ptr(), fin.data_ptr(), B, beam, V, k, 2,
                               ob.data_ptr(), ot.data_ptr(), osc.data_ptr(), cur.cuda_stream)
        if rc != 0:
            raise RuntimeError(rtopk.rtopk_last_error())

    for i in range(5):
        unfused(i)
    ms_unfused = float(np.median([timed(unfused, 50) for _ in range(3)]))
    ms_gemm = float(np.median([timed(lambda i: torch.matmul(x, pool[i % nbuf].t(), out=logits), 50)
                               for _ in range(3)]))
    flops = 2.0 * M * V * H
    tflops = flops / (ms * 1e-3) / 1e12
    line = {
        "metric": "LM head fused with the selection step: steps/s and matrix-core TFLOP/s, 1xMI355X",
        "value": 1e3 / ms, "unit": "beam-steps/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"lmhead_b128: hidden [{M}, {H}] x weight [{V}, {H}] bf16, B={B} beam={beam} k={k}, "
                               "26/512 beams finished, seed 1009", "B": B, "beam": beam, "H": H, "V": V, "k": k,
                   "weight_pool_buffers": nbuf},
        "flops_per_step": flops,
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / MFMA_BF16_PEAK_TFLOPS, "traffic": None},
        "trials_ms": trials,
        "weight_GBps": V * H * 2 / (ms * 1e-3) / 1e9,
        "unfused_ms_per_step": ms_unfused,
        "unfused_gemm_ms": ms_gemm,
        "unfused": "torch.matmul (hipBLASLt) to bf16 logits [512, 40000], then rtopk_beam_step on them",
    }
    print(json.dumps(line), flush=True)


def usable_cpus():
    """CPUs this process may run on: its affinity set, bounded by the cgroup's
    CPU quota when one is set (a container's share of a larger host)."""
    n = len(os.sched_getaffinity(0))
    try:
        with open("/sys/fs/cgroup/cpu.max") as f:
            quota, period = f.read().split()[:2]
        if quota != "max":
            n = min(n, max(1, int(int(quota) // int(period))))
    except (OSError, ValueError):
        pass
    return n


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(s, seconds):
    """The oracle, untuned, on this host's cores: once single-threaded and once
    with every usable CPU, each repeated until it has run seconds / 2 (at
    least one step)."""
    import oracle
    threads = usable_cpus()

    def rate(nthreads):
        oracle.step_of(s, nthreads=nthreads)  # warm (page-in)
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.step_of(s, nthreads=nthreads)
            reps += 1
            el = time.perf_counter() - t0
            if el >= seconds / 2 or reps >= 1000:
                return reps, el

    r1, e1 = rate(1)
    rt, et = rate(threads)
    return {"value": rt / et, "unit": "beam-steps/s", "cores": threads, "kind": "oracle",
            "sample": f"{rt} full {s.name} steps (B={s.B} beam={s.beam} V={s.V}) in {et:.1f} s with {threads} "
                      f"threads, {r1} in {e1:.1f} s with 1; float64 log-softmax + full sort per batch element",
            "single_thread": {"value": r1 / e1, "unit": "beam-steps/s", "cores": 1},
            "affinity_cpus": len(os.sched_getaffinity(0)), "cpu_model": cpu_model()}


def read_sweep(L, cur):
    """Plain streaming reads (rtopk_read_probe_shape) of 38.88 MB (the
    algorithmic bytes of the b128 step) and of 256 MiB, for several launch
    shapes, each over a pool of distinct buffers larger than the Infinity
    Cache and replayed from a captured graph; prints one line per shape."""
    import torch
    pool_bytes = 1 << 30
    for nbytes in (38_880_000, 256 << 20):
        nbuf = max(2, -(-pool_bytes // nbytes))
        bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda:0").fill_(1) for _ in range(nbuf)]
        out = torch.zeros(1, dtype=torch.int32, device="cuda:0")
        for vecs in (1, 2, 4, 8, 10, 16):
            for threads in (256, 512, 1024):
                def probe(i, stream):
                    rc = L.rtopk_read_probe_shape(bufs[i % nbuf].data_ptr(), nbytes, vecs, threads, 0x7fc00001,
                                                  out.data_ptr(), stream)
                    if rc != 0:
                        raise RuntimeError("read probe failed")
                for i in range(10):
                    probe(i, cur.cuda_stream)
                graph = torch.cuda.CUDAGraph()
                cs = torch.cuda.Stream()
                cs.wait_stream(cur)
                n_in = 20
                with torch.cuda.graph(graph, stream=cs):
                    for i in range(n_in):
                        probe(i, torch.cuda.current_stream().cuda_stream)
                torch.cuda.synchronize()
                graph.replay()
                torch.cuda.synchronize()
                times = []
                for _ in range(5):
                    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    start.record(cur)
                    for _ in range(5):
                        graph.replay()
                    end.record(cur)
                    torch.cuda.synchronize()
                    times.append(start.elapsed_time(end) * 1e3 / (5 * n_in))
                us = sorted(times)[2]
                grid = -(-nbytes // (16 * vecs * threads))
                print(json.dumps({"bytes": nbytes, "vecs_per_lane": vecs, "threads": threads, "grid": grid,
                                  "us_per_launch": round(us, 3), "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
                                  "frac_of_peak": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}),
                      flush=True)
        del bufs


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--config", default="b128")
    ap.add_argument("--shards", type=int, default=1,
                    help="select over G vocabulary shards (rtopk_beam_step_sharded), each its own tensor")
    ap.add_argument("--path", default="select", choices=["select", "reorder", "sample", "lmhead"],
                    help="select: the selection step (the default line); reorder: the cache refresh after it; "
                         "sample: top-k sampling with the same selection; lmhead: the step fused into the "
                         "LM head GEMM")
    ap.add_argument("--launch", default="graph", choices=["graph", "eager"],
                    help="replay the K launches from a captured HIP graph, or launch each from Python")
    ap.add_argument("--pool-mib", type=int, default=1024, help="distinct logit buffers rotated through")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-read-ceiling", action="store_true", help="skip the plain-read ceiling measurement")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 256 MiB device copy (reference kernel for HBM counters)")
    ap.add_argument("--read-sweep", action="store_true",
                    help="print plain-read times for several launch shapes at 38.88 MB and 256 MiB, then exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the selection step of a batch "
              "element needs no other GPU, and the benchmark measures the one-GPU kernel.", file=sys.stderr)
        sys.exit(2)

    if args.path == "reorder":
        bench_reorder(args)
        return
    if args.path == "sample":
        bench_sample(args)
        return
    if args.path == "lmhead":
        bench_lmhead(args)
        return
    if args.read_sweep:
        import torch

        from beam_search_top_amd import rtopk
        read_sweep(rtopk.load(), torch.cuda.current_stream())
        return

    import numpy as np
    import torch

    from beam_search_top_amd import rtopk, synth

    if not os.path.exists(rtopk.LIB_PATH):
        from beam_search_top_amd import _build
        _build.build()
    rtopk.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    s = synth.make_step(args.config)
    if s.dtype == synth.BF16:
        x0 = torch.from_numpy(s.logits.view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        x0 = torch.from_numpy(s.logits).to(dev)
    alive = torch.from_numpy(s.alive).to(dev)
    fin = torch.from_numpy(s.finished).to(dev)
    nbuf = max(1, math.ceil(args.pool_mib * 2**20 / s.logit_bytes))
    pool = [x0] + [torch.roll(x0, shifts=7919 * i, dims=2).contiguous() for i in range(1, nbuf)]
    G = args.shards
    if G > 1:  # each pool entry becomes G shard tensors [B, beam, V/G]
        Vs = s.V // G
        pool = [[x[:, :, g * Vs:(g + 1) * Vs].contiguous() for g in range(G)] for x in pool]
        shard_arrays = [(ctypes.c_void_p * G)(*[t.data_ptr() for t in shards]) for shards in pool]
    ob = torch.empty((s.B, s.k), dtype=torch.int32, device=dev)
    ot = torch.empty((s.B, s.k), dtype=torch.int32, device=dev)
    osc = torch.empty((s.B, s.k), dtype=torch.float32, device=dev)
    nws = rtopk.rtopk_workspace_bytes(s.B, s.beam, s.V, s.k, s.dtype)
    ws = torch.zeros(nws, dtype=torch.uint8, device=dev)
    st, plan = rtopk.rtopk_plan(x0.data_ptr(), s.B, s.beam, s.V, s.k, s.dtype)
    assert st == 0, rtopk.rtopk_last_error()
    L = rtopk.load()
    fixed = (s.dtype, alive.data_ptr(), fin.data_ptr(), s.B, s.beam, s.V, s.k, s.eos_id,
             ob.data_ptr(), ot.data_ptr(), osc.data_ptr())
    ptrs = [p.data_ptr() for p in pool] if G == 1 else [shards[0].data_ptr() for shards in pool]
    wsp = ws.data_ptr()

    def launch(i, stream):
        if G == 1:
            rc = L.rtopk_beam_step_ws(ptrs[i % nbuf], *fixed, wsp, nws, stream)
        else:
            rc = L.rtopk_beam_step_sharded(shard_arrays[i % nbuf], G, s.dtype, alive.data_ptr(), fin.data_ptr(),
                                           s.B, s.beam, s.V // G, s.k, s.eos_id, ob.data_ptr(), ot.data_ptr(),
                                           osc.data_ptr(), stream)
        if rc != 0:
            raise RuntimeError(rtopk.rtopk_last_error())

    torch.cuda.synchronize()
    cur = torch.cuda.current_stream()
    # warmup (eager)
    for i in range(args.warmup):
        launch(i, cur.cuda_stream)
    torch.cuda.synchronize()

    K = args.steps
    graph, glen = None, 0
    if args.launch == "graph":
        glen = min(K, 100)
        graph = torch.cuda.CUDAGraph()
        cs = torch.cuda.Stream()
        cs.wait_stream(cur)
        if G > 1:  # the sharded entry point uses the library workspace of its stream: create it before capture
            launch(0, cs.cuda_stream)
            torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=cs):
            for i in range(glen):
                launch(i, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        for _ in range(3):
            graph.replay()
        torch.cuda.synchronize()

    def timed(mode, n):
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(cur)
        if mode == "graph":
            for _ in range(n // glen):
                graph.replay()
            for i in range(n % glen):
                launch(i, cur.cuda_stream)
        else:
            for i in range(n):
                launch(i, cur.cuda_stream)
        end.record(cur)
        torch.cuda.synchronize()
        return start.elapsed_time(end)

    # the GPU time: K steps in 5 trials (K / 5 steps each, the last takes the
    # remainder), each bracketed by events and synchronisation; the median trial
    ntr = min(5, K)
    sizes = [K // ntr] * (ntr - 1) + [K - (K // ntr) * (ntr - 1)]
    trials = [timed(args.launch, n) / n for n in sizes]
    ms_step = float(np.median(trials))
    other = {"trials_ms_per_step": [round(t, 6) for t in trials], "trial_steps": sizes}
    if args.launch == "graph":
        other["eager_ms_per_step"] = round(timed("eager", K) / K, 6)

    # the last step's outputs come from buffer (K-1) % nbuf; re-run buffer 0 for a sanity check
    launch(0, cur.cuda_stream)
    torch.cuda.synchronize()
    assert (ob >= -1).all() and (ob < s.beam).all(), "beam ids out of range"

    if args.copy_calibration:
        n = 256 * 2**20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    alg = algorithmic_bytes(s)
    # the probe reads alg contiguous bytes of one buffer: only an unsharded pool has them
    ceiling = None if args.no_read_ceiling or G > 1 else read_ceiling(L, ptrs, alg, K, cur)
    traffic = read_traffic(args.config)  # measured HBM bytes per launch, if taken on these sources
    achieved = alg / (ms_step * 1e-3) / 1e9
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(s, args.cpu_seconds)
    dtype_name = {0: "f32", 1: "f16", 2: "bf16"}[s.dtype]
    line = {
        "metric": "beam-steps/sec and logit GB/s (% HBM peak) at BxbeamxV, 1xMI355X",
        "value": 1e3 / ms_step,
        "unit": "beam-steps/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype_name,
        "data": "synthetic",
        "config": {
            "workload": f"{s.name}: B={s.B} beam={s.beam} k={s.k} V={s.V} {dtype_name} logits, "
                        f"{s.n_finished}/{s.B * s.beam} beams finished, seed {s.seed}",
            "B": s.B, "beam": s.beam, "k": s.k, "V": s.V, "launch": args.launch, "vocab_shards": G,
            "logit_pool_buffers": nbuf, "chunks": plan.chunks, "vecs_per_thread": plan.vecs_per_thread,
            "grid": plan.grid,
        },
        "sequences_per_s": s.B * 1e3 / ms_step,
        "logit_GBps": achieved,
        "hbm_frac": achieved / HBM_PEAK_GBPS,
        "algorithmic_bytes_per_step": alg,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": None if traffic is None else traffic / (ms_step * 1e-3) / 1e9},
        "traffic_bytes_per_launch": traffic,
        "read_ceiling": ceiling,
        "frac_of_read_ceiling": None if ceiling is None else achieved / ceiling["GBps"],
        "cpu_baseline": cpu,
        "kernel_sha": kernel_sha(),
    }
    line.update(other)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
