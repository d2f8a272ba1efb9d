#!/usr/bin/env python3
"""Decode-step benchmark of the 8-bit paged KV cache on one MI355X.

A step is one decode step of one attention layer: the append of one new token per sequence and
paged attention over the whole cache, through kvq_decode_step (append fused into the partition
kernel, then the merge kernel; `--separate-calls` times kvq_append + kvq_paged_decode_attn
instead).  Inputs are seeded synthetic tensors already resident in HBM.  The
timed loop walks over `--layers` copies of the layer's cache so consecutive steps read different
memory (the 256 MB last-level cache cannot serve a step from the previous one).

Prints one JSON line: achieved HBM GB/s of the whole step (algorithmic bytes / step time), with
tokens/s, the roofline of the dominant kernel (the attention partition kernel, timed with HIP
events on its own stream in a second pass) and the CPU oracle timed on this host as a baseline.
Besides: the spread of the per-step time over ten blocks of the timed steps, the attention alone
(kvq_paged_decode_attn without the append), and the step on one cache every time (no rotation).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FP8-KV paged decode attention: achieved HBM GB/s (% of peak), tokens/s"
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, 8 TB/s
DEFAULT_WORKLOAD = "llama2-7b-mha-e4m3"
PROFILE_DIR = os.path.join(ROOT, "profiles")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def partition_kernel(w) -> tuple[str, str]:
    """(kernel name, source file) of the partition kernel that serves the workload."""
    mha = w.num_q_heads == w.num_kv_heads
    if w.fp8_math:  # every grouping runs on the grouped-head kernel
        return f"attn_partition_mfma<{w.dtype}, fp8 math>", "kvq_attn_gqa.hip"
    if w.dtype == "int4":
        return (("attn_partition_valu4", "kvq_attn_mha4.hip") if mha
                else ("attn_partition_mfma4", "kvq_attn_gqa4.hip"))
    if mha:
        return f"attn_partition_valu<{w.dtype}>", "kvq_attn_mha.hip"
    return f"attn_partition_mfma<{w.dtype}>", "kvq_attn_gqa.hip"


def kernel_source_files(w) -> tuple:
    """The partition kernel's file and the headers it includes."""
    src = partition_kernel(w)[1]
    extra = ("kvq_int4.h", "kvq_attn4.h") if w.dtype == "int4" else ()
    if src == "kvq_attn_gqa.hip":
        extra += ("kvq_mfma.h", "kvq_fp8m.h")
    return (src, "kvq_attn.h", "kvq_device.h") + extra


def kernel_source_digest(w) -> str:
    """Digest of the partition kernel's sources (its file and the headers it includes)."""
    import hashlib
    h = hashlib.sha256()
    for f in kernel_source_files(w):
        with open(os.path.join(ROOT, "quantized_kv_cache_03_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str, digest: str):
    """HBM bytes per launch of the partition kernel from the committed rocprofv3 --pmc summary,
    only if it was taken on the current kernel source."""
    path = os.path.join(PROFILE_DIR, f"pmc_attn_partition_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_source_digest") != digest:
        return None
    return d.get("hbm_bytes_per_launch")


def read_ceiling(mib: int = 2048, waves: int = 2048, iters: int = 10):
    """The HBM read rate a plain read kernel reaches on this GPU (libkvq_probe.so): 2 KiB tiles
    streamed by `waves` waves in sequential order and in a shuffled order (as a shuffled block
    table lays the tiles out), over `mib` MiB, far past the last-level cache.  None if the probe
    library is missing."""
    import ctypes

    import numpy as np
    import torch
    path = os.path.join(ROOT, "quantized_kv_cache_03_amd", "libkvq_probe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.kvq_probe_read_tiles.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                         ctypes.c_void_p, ctypes.c_void_p]
    lib.kvq_probe_read_tiles.restype = ctypes.c_int
    n = (mib << 20) // 2048
    buf = torch.empty(n * 2048, dtype=torch.uint8, device="cuda").fill_(1)
    sink = torch.empty(waves * 64, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    res = {"kernel": "kvq_probe_read_tiles (quantized_kv_cache_03_amd/probe/read_probe.hip)",
           "bytes_per_pass": n * 2048, "waves": waves, "tile_bytes": 2048}
    orders = {"sequential": np.arange(n, dtype=np.int32),
              "shuffled": np.random.default_rng(0).permutation(n).astype(np.int32)}
    for name, order in orders.items():
        o = torch.from_numpy(order).cuda()

        def call():
            rc = lib.kvq_probe_read_tiles(buf.data_ptr(), o.data_ptr(), n, waves, sink.data_ptr(),
                                          stream.cuda_stream)
            if rc != 0:
                raise RuntimeError(f"kvq_probe_read_tiles failed ({rc})")
        for _ in range(2):
            call()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(iters):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        res[f"{name}_gbs"] = round(n * 2048 * iters / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
    del buf, sink
    torch.cuda.empty_cache()
    return res


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, threads: int, budget_s: float, scale: float):
    """The oracle as it stands (C, fp64): append + attention for a prefix of the batch, timed on
    this host; reported in the metric's unit (algorithmic GB/s of the sample)."""
    import numpy as np

    import oracle
    from quantized_kv_cache_03_amd import workloads as W

    ctx_all = W.context_lens(w)
    ch = W.outlier_channels(w)
    # a bounded sample: the first sequences of the batch, all their heads
    nseq = 0
    est = 0.0
    per_tok_head_s = 2.5e-6  # rough single-thread cost of one (token, head) of append+attention
    while nseq < len(ctx_all):
        est += ctx_all[nseq] * w.num_q_heads * per_tok_head_s / max(1, threads)
        nseq += 1
        if est > budget_s:
            break
    seqs = list(range(nseq))
    ctx = ctx_all[seqs].astype(np.int32)
    sub = w.scaled(name=w.name + "-cpu-sample", batch=len(seqs), context=("list", ctx.tolist()))
    bt, nb = W.block_tables(sub, ctx)
    rows = [W.kv_rows(w, b, int(ctx[i]), ch) for i, b in enumerate(seqs)]
    k = np.concatenate([r[0] for r in rows])
    v = np.concatenate([r[1] for r in rows])
    cu = np.zeros(len(seqs) + 1, np.int32)
    cu[1:] = np.cumsum(ctx)
    q = W.query(w)[seqs]
    dt = {"fp8_e4m3": oracle.E4M3, "fp8_e5m2": oracle.E5M2, "int8": oracle.INT8,
          "fp8_e4m3fnuz": oracle.E4M3FNUZ, "int4": oracle.INT4}[w.dtype]
    cache = oracle.Cache(dt, nb, w.num_kv_heads, scale)
    t0 = time.perf_counter()
    oracle.append(cache, k, v, bt, ctx, cu)  # the prefill of the sample's rows (single-threaded)
    t1 = time.perf_counter()
    # the timed step: the append of one token per sequence + attention over the whole sample,
    # repeated (the append rewrites the same slots) until about budget_s of CPU time has passed
    last = cu[1:] - 1
    reps = 0
    while True:
        oracle.append(cache, k[last], v[last], bt, ctx)
        oracle.decode_attn(cache, q, bt, ctx, threads=threads, fp8_math=w.fp8_math)
        reps += 1
        if time.perf_counter() - t1 >= budget_s:
            break
    t2 = time.perf_counter()
    from quantized_kv_cache_03_amd.harness import kv_bytes_per_token
    per_tok = kv_bytes_per_token(w.dtype)
    bytes_ = (int(ctx.sum()) * w.num_kv_heads * per_tok + 2 * len(seqs) * w.num_q_heads * 128 * 2
              + 4 * int(((ctx + 15) // 16).sum()) + 4 * len(seqs))
    step_s = (t2 - t1) / reps
    # the same step on one thread, for the first sequence alone (a few seconds at most)
    b0 = cu[1] - 1
    t3 = time.perf_counter()
    oracle.append(cache, k[b0:b0 + 1], v[b0:b0 + 1], bt[:1], ctx[:1])
    oracle.decode_attn(cache, q[:1], bt[:1], ctx[:1], threads=1, fp8_math=w.fp8_math)
    one_s = time.perf_counter() - t3
    one_bytes = (int(ctx[0]) * w.num_kv_heads * per_tok + 2 * w.num_q_heads * 128 * 2
                 + 4 * int((ctx[0] + 15) // 16) + 4)
    return {"value": bytes_ / step_s / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"first {len(seqs)} of {len(ctx_all)} sequences (sum ctx {int(ctx.sum())}), "
                      f"all {w.num_q_heads} heads: one append + fp64 attention, {reps} repetitions "
                      f"in {t2 - t1:.1f} s ({step_s:.3f} s each); prefill of the sample not timed "
                      f"({t1 - t0:.1f} s)",
            "tokens_per_s": len(seqs) / step_s,
            "single_thread": {"value": one_bytes / one_s / 1e9, "unit": "GB/s",
                              "sample": f"sequence 0 ({int(ctx[0])} tokens), all heads, one step"}}


PREFILL_METRIC = "prefill attention over the 8-bit paged cache: achieved TFLOP/s (% of fp16 MFMA peak)"
PEAK_MFMA_F16_TFLOPS = 2500.0  # MI355X dense fp16 matrix peak
PEAK_MFMA_F8_TFLOPS = 5000.0   # MI355X dense fp8 matrix peak
# FP8 math: QK^T (half the flops) on the fp8 peak, PV on the fp16 one -> the peak of the mix
PEAK_MFMA_F8F16_TFLOPS = 2.0 / (1.0 / PEAK_MFMA_F8_TFLOPS + 1.0 / PEAK_MFMA_F16_TFLOPS)


def run_prefill(args, w):
    """Prefill (causal) attention over whole prompts (or the last --prefill-rows tokens of each):
    kvq_paged_prefill_attn after the prompt's bulk append.  Prints one JSON line."""
    import numpy as np
    import torch

    from quantized_kv_cache_03_amd import harness, kvq

    w = w.scaled(name=w.name + f"-prefill{args.prefill_ctx}", batch=args.prefill_batch,
                 context=("fixed", args.prefill_ctx))
    case = harness.DeviceCase(w, keep_host_rows=not args.no_cpu_baseline)
    n = int(case.ctx[0])
    m = min(n, args.prefill_rows or n)
    nq = [m] * case.B
    cu_q = np.arange(case.B + 1, dtype=np.int32) * m
    q = np.random.default_rng([w.seed, 9]).standard_normal((int(cu_q[-1]), w.num_q_heads, 128),
                                                          dtype=np.float32).astype(np.float16)
    q_d, cu_d = torch.from_numpy(q).cuda(), torch.from_numpy(cu_q).cuda()
    out = torch.empty_like(q_d)
    stream = torch.cuda.current_stream()

    attn = kvq.paged_prefill_attn_fp8math if w.fp8_math else kvq.paged_prefill_attn
    peak = PEAK_MFMA_F8F16_TFLOPS if w.fp8_math else PEAK_MFMA_F16_TFLOPS

    def call():
        attn(case.cache, q_d, cu_d, case.bt_d, case.ctx_d, case.max_ctx, m, out=out, stream=stream)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    kvq.timing_begin(args.steps)
    for _ in range(args.steps):
        call()
    torch.cuda.synchronize()
    kms, kn = kvq.timing_end()
    kms /= max(1, kn)
    # algorithmic flops: QK^T and PV, 2 * 2 * 128 per (row, head, visible token); visible tokens of
    # row j of a sequence of n tokens with m query rows: n - m + j + 1
    visible = case.B * (m * (n - m) + m * (m + 1) // 2)
    flops = 4 * 128 * w.num_q_heads * visible
    per_tok = harness.kv_bytes_per_token(w.dtype)
    code_bytes = case.B * n * w.num_kv_heads * per_tok
    cpu = None
    parity = None
    if not args.no_cpu_baseline:
        # the oracle as it stands (fp64) on 8 evenly spaced query rows, all heads
        import oracle
        threads = max(1, min(len(os.sched_getaffinity(0)), 16))
        dt = {"fp8_e4m3": oracle.E4M3, "fp8_e5m2": oracle.E5M2, "int8": oracle.INT8,
          "fp8_e4m3fnuz": oracle.E4M3FNUZ, "int4": oracle.INT4}[w.dtype]
        oc = oracle.Cache(dt, case.num_blocks, w.num_kv_heads, case.kv_scale)
        oracle.append(oc, case.k_host, case.v_host, case.bt, case.ctx, case.cu)
        T = int(cu_q[-1])
        rows = sorted(set(np.linspace(0, T - 1, 8).astype(int).tolist()))
        t0 = time.perf_counter()
        ref = oracle.prefill_attn(oc, q, case.bt, case.ctx, cu_q, rows=rows, threads=threads,
                                  fp8_math=w.fp8_math)
        sec = time.perf_counter() - t0
        fl = sum(4 * 128 * w.num_q_heads * (n - m + (r % m) + 1) for r in rows)
        cpu = {"value": fl / sec / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
               "cpu_model": cpu_model(),
               "sample": f"{len(rows)} of {T} query rows, all {w.num_q_heads} heads, fp64 ({sec:.2f} s)"}
        g = out.cpu().numpy()[rows].astype(np.float64)
        err = np.abs(g - ref[rows])
        parity = {"rows": len(rows), "max_abs": float(err.max()),
                  "within_gate": bool((err <= 1e-3 + 1e-2 * np.abs(ref[rows])).all())}
    res = {
        "metric": PREFILL_METRIC,
        "value": round(flops / (ms * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f8+f16" if w.fp8_math else "f16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "num_q_heads": w.num_q_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim": 128, "block_size": 16,
                   "context": n, "query_rows_per_sequence": m, "kv_cache_dtype": w.dtype,
                   "entry_points": ("kvq_paged_prefill_attn_fp8math" if w.fp8_math
                                    else "kvq_paged_prefill_attn")},
        "flops": flops,
        "kv_code_bytes": code_bytes,
        "roofline": {"kernel": ("attn_prefill_mfma4" if w.dtype == "int4" else
                                f"attn_prefill_mfma<{w.dtype}{', fp8 math' if w.fp8_math else ''}>"),
                     "bound": "mfma",
                     "achieved": round(flops / (kms * 1e-3) / 1e12, 2), "peak": round(peak, 1),
                     "unit": "TFLOP/s", "frac": round(flops / (kms * 1e-3) / 1e12 / peak, 4),
                     "traffic": None, "kernel_ms": round(kms, 5)},
        "parity_sampled_rows": parity,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--layers", type=int, default=4, help="cache copies the steps rotate over")
    ap.add_argument("--partition", type=int, default=None, help="override the split-K partition size")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=15.0)
    ap.add_argument("--separate-calls", action="store_true",
                    help="time kvq_append + kvq_paged_decode_attn instead of the fused kvq_decode_step")
    ap.add_argument("--prefill", action="store_true",
                    help="measure prefill attention (kvq_paged_prefill_attn) instead of the decode step")
    ap.add_argument("--prefill-ctx", type=int, default=4096, help="prompt length (prefill mode)")
    ap.add_argument("--prefill-batch", type=int, default=4, help="prompts (prefill mode)")
    ap.add_argument("--prefill-rows", type=int, default=0,
                    help="query rows per prompt, its last tokens (0: the whole prompt)")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="before warmup, run one plain device-to-device copy of this many MiB (a known "
                         "amount of HBM traffic, used to calibrate memory counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the decode kernels run on a single MI355X and the library "
              "has no multi-GPU path (the design notes describe how it would shard). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from quantized_kv_cache_03_amd import harness, kvq, workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    w = W.WORKLOADS[args.workload]
    if args.prefill:
        run_prefill(args, w)
        return
    if args.partition is not None:
        w = w.scaled(name=w.name, partition_size=args.partition)
    log(f"[bench] workload {w.name}: B={w.batch} Hq={w.num_q_heads} Hkv={w.num_kv_heads} {w.dtype} "
        f"partition={w.partition_size}")
    t0 = time.time()
    case = harness.DeviceCase(w, verbose=False)
    log(f"[bench] cache filled in {time.time() - t0:.1f} s: {case.num_blocks} blocks, "
        f"sum ctx {int(case.ctx.sum())}")
    # layer copies: same codes, distinct memory
    layers = [case.cache]
    for _ in range(args.layers - 1):
        layers.append(case.cache.clone())
    stream = torch.cuda.current_stream()
    if args.calibration_copy_mib > 0:
        nbytes = args.calibration_copy_mib << 20
        src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy: {nbytes} bytes read and {nbytes} bytes written")
        del src, dst

    # The fused step of each cache copy, its arguments checked once (kvq.PreparedCall): the timed
    # loops then spend no host time on the binding's checks, which would bound a small step.
    prepared = [case.prepared_step(layer, stream) for layer in layers]

    def step(i):
        if args.separate_calls:
            case.cache = layers[i % len(layers)]
            case.step(stream=stream, fused=False)
        else:
            prepared[i % len(prepared)]()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    def timed(fn, n: int, blocks: int = 1):
        """Run fn(i) for i < n with an event at each of `blocks` block boundaries only (no event
        between the launches inside a block); -> (total ms, per-step ms of each block)."""
        bounds = [n * k // blocks for k in range(blocks + 1)]
        evs = [torch.cuda.Event(enable_timing=True) for _ in bounds]
        torch.cuda.synchronize()
        evs[0].record(stream)
        for k in range(blocks):
            for i in range(bounds[k], bounds[k + 1]):
                fn(i)
            evs[k + 1].record(stream)
        torch.cuda.synchronize()
        per = [evs[k].elapsed_time(evs[k + 1]) / max(1, bounds[k + 1] - bounds[k]) for k in range(blocks)
               if bounds[k + 1] > bounds[k]]
        return evs[0].elapsed_time(evs[-1]), per

    # Region 1: the step throughput, with nothing between the launches but ten block boundaries
    # (for the spread of the per-step time across blocks).
    wall0 = time.perf_counter()
    ms_total, block_ms = timed(step, args.steps, blocks=min(10, args.steps))
    wall = time.perf_counter() - wall0
    ms_step = ms_total / args.steps
    # Region 2: the same steps again with a HIP event pair in every partition-kernel dispatch (the
    # library's timing hook launches it through hipExtLaunchKernel), on the stream it is launched
    # on.  This region gives the kernel's own duration; the step time comes from region 1 alone.
    kvq.timing_begin(args.steps)
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    main_ms, main_n = kvq.timing_end()

    # Region 3: attention alone (kvq_paged_decode_attn, no append), over the rotated caches.
    def attend(i):
        case.cache = layers[i % len(layers)]
        case.attention(stream=stream)
    attn_ms = timed(attend, args.steps)[0] / args.steps
    # Region 4: the step on one cache every time (the last-level cache keeps what it can).
    def step_same(i):
        if args.separate_calls:
            case.cache = layers[0]
            case.step(stream=stream, fused=False)
        else:
            prepared[0]()
    same_ms = timed(step_same, args.steps)[0] / args.steps
    step_bytes = case.algorithmic_bytes()
    attn_bytes = case.attention_bytes()
    gbs = step_bytes / (ms_step * 1e-3) / 1e9
    main_avg_ms = main_ms / max(1, main_n)
    achieved = attn_bytes / (main_avg_ms * 1e-3) / 1e9
    digest = kernel_source_digest(w)
    traffic = load_traffic(w.name, digest)
    ceiling = read_ceiling()

    cpu = None
    if not args.no_cpu_baseline:
        threads = len(os.sched_getaffinity(0))
        threads = max(1, min(threads, 16))
        log(f"[bench] cpu baseline: oracle on {threads} threads")
        cpu = cpu_baseline(w, threads, args.cpu_budget_s, case.kv_scale)

    res = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f8+f16" if w.fp8_math else "f16",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "batch": w.batch,
            "num_q_heads": w.num_q_heads,
            "num_kv_heads": w.num_kv_heads,
            "head_dim": 128,
            "block_size": 16,
            "context": list(w.context),
            "sum_context": int(case.ctx.sum()),
            "block_table": w.table,
            "kv_cache_dtype": w.dtype,
            "kv_scale": case.kv_scale,
            "partition_size": w.partition_size,
            "layers_rotated": args.layers,
            "entry_points": ("kvq_append+kvq_paged_decode_attn" if args.separate_calls
                             else "kvq_decode_step") + ("_fp8math" if w.fp8_math else ""),
        },
        "pct_of_peak_hbm": round(100.0 * gbs / PEAK_HBM_GBS, 2),
        "tokens_per_s": round(w.batch / (ms_step * 1e-3), 1),
        "kv_tokens_per_s": round(int(case.ctx.sum()) / (ms_step * 1e-3), 1),
        "step_bytes": step_bytes,
        "wall_s_timed_region": round(wall, 4),
        "kernel_timing": "partition kernel timed with HIP events in a second pass over the same steps",
        "kernels_ms": {"attn_partition_avg": round(main_avg_ms, 5)},
        "step_ms_blocks": {"blocks": len(block_ms), "p10": round(float(np.percentile(block_ms, 10)), 5),
                           "median": round(float(np.median(block_ms)), 5),
                           "p90": round(float(np.percentile(block_ms, 90)), 5)},
        "attention_only": {"ms": round(attn_ms, 5),
                           "gbs": round(attn_bytes / (attn_ms * 1e-3) / 1e9, 2)},
        "step_ms_same_cache": round(same_ms, 5),
        "roofline": {
            "kernel": partition_kernel(w)[0],
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": attn_bytes,
            "kernel_source_digest": digest,
        },
        # a plain read kernel's rate on this GPU, beside the nominal peak (the kernel's achieved
        # rate as a fraction of it: the table order matching the workload's)
        "read_ceiling": ceiling,
        "frac_of_read_ceiling": (None if not ceiling else round(
            achieved / ceiling["shuffled_gbs" if w.table == "shuffled" else "sequential_gbs"], 4)),
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
