"""Benchmark: one attention layer-step over a paged KV cache on one MI355X.

A step is the whole hot path for one layer: append this step's new K/V
(reshape_and_cache), then paged decode attention (partition kernel plus the
split-K reduction) and, for workloads with a prefill chunk, the MFMA
prefill-chunk kernel. Inputs are seeded synthetic tensors of the workload's
shapes, resident in HBM before timing starts. Steps rotate over R copies of the
pool (one library "layer" each, >= 2 GiB in total) so the 256 MB Infinity
Cache cannot serve repeated reads.

Prints ONE JSON line on stdout; progress goes to stderr.
  python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 3|4|5|6] [--kv-dtype bf16|fp8]
                  [--block-size 16|32] [--queries-per-seq T] [--shared] [--graph]

--kv-dtype fp8 keeps the same bf16 step (queries, new K/V rows, outputs) but
stores the cache as e4m3 codes with per-layer scales: the append quantizes,
attention reads one byte per cached element.

--queries-per-seq T (T > 1) gives every decoding sequence T query rows (a
speculative-verification step: the last T tokens of each sequence are this
step's, appended first) and runs paged_attention_decode_multi.

--config 6 is a parallel-sampling step (32 prompts of 2000 tokens, 8 samples
each, every sample sharing its prompt's blocks). --shared runs it through
paged_attention_decode_shared, which reads each prompt's blocks once for its
8 samples; without it the same step runs through paged_attention_decode.
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
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, AMD's published figure
BF16_MFMA_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak (no sparsity)
COUNTERS_FILES = {
    "bf16": os.path.join(ROOT, "profiles", "decode_partition_llama8b_b256_counters.txt"),
    "fp8": os.path.join(ROOT, "profiles", "decode_partition_llama8b_b256_fp8_counters.txt"),
}
FP8_SCALE = 1.0 / 80     # K and V scale of every layer of an e4m3 pool (N(0,1) inputs)
KERNEL_SOURCES = ["decode.hip", "device_common.h", "kernels.h"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "paged_kv_decode_reshape_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def make_step(config: int, block_size: int = 16, qwen=(16, 512)):
    from paged_kv_decode_reshape_amd import workloads as W
    if block_size != 16 and config != 3:
        raise SystemExit("--block-size other than 16 is benchmarked on config 3")
    if config == 2:
        if tuple(qwen) not in W.QWEN_GRID:
            raise SystemExit(f"--qwen-batch/--qwen-context {qwen} is not a point of the grid {W.QWEN_GRID}")
        return W.qwen_layer(*qwen)
    if config == 3:
        return W.llama8b_continuous(block_size=block_size)
    if config == 4:
        return W.long_context()
    if config == 5:
        return W.mixed_chunked_prefill()
    if config == 6:
        return W.parallel_sampling()
    raise SystemExit(f"--config {config}: the bench runs configs 2 to 6 (1 is a parity case)")


def multi_query_inputs(step, t: int, seed: int = 11):
    """T query rows and T new K/V rows (the last T positions) per decoding
    sequence, seeded N(0, 1) rounded to bf16, and their slots."""
    from paged_kv_decode_reshape_amd import workloads as W
    rng = np.random.default_rng(seed)
    bt, cl = step.decode_inputs()
    hq, hkv, d = step.num_q_heads, step.num_kv_heads, step.head_dim
    slots = []
    for b in range(len(cl)):
        pos = np.arange(int(cl[b]) - t, int(cl[b]))
        slots.append(bt[b, pos // step.block_size].astype(np.int64) * step.block_size + pos % step.block_size)
    n = len(cl) * t
    q = W.make_values(rng.standard_normal((n, hq, d), dtype=np.float32), step.dtype)
    k = W.make_values(rng.standard_normal((n, hkv, d), dtype=np.float32), step.dtype)
    v = W.make_values(rng.standard_normal((n, hkv, d), dtype=np.float32), step.dtype)
    return q, k, v, np.concatenate(slots)


def algorithmic_bytes(step, kv_dtype: str = "bf16", q_per_seq: int = 1, shared: bool = False):
    """Bytes a perfect implementation moves (each byte once). e: bytes of a
    query/output/new-row element; ekv: bytes of a cached element. shared: a
    prefix shared by a group of sequences is counted once for the group."""
    e = 2 if step.dtype == "bf16" else 4
    ekv = 1 if kv_dtype == "fp8" else e
    hkv, hq, d = step.num_kv_heads, step.num_q_heads, step.head_dim
    _, dec_ctx = step.decode_inputs()
    b = len(dec_ctx)
    tokens = step.info["unique_tokens"] if shared else int(dec_ctx.astype(np.int64).sum())
    decode_kv = tokens * hkv * d * 2 * ekv
    decode_qo = 2 * b * q_per_seq * hq * d * e
    n_new = len(step.new_slots) if q_per_seq == 1 else b * q_per_seq
    append = 2 * n_new * hkv * d * (e + ekv)            # read new K,V + write them
    out = {"decode_kv": decode_kv, "decode_qo": decode_qo, "append": append}
    if step.cu_q_lens is not None:
        _, pctx = step.prefill_inputs()
        qlens = np.diff(step.cu_q_lens)
        kv = int(pctx.astype(np.int64).sum()) * hkv * d * 2 * ekv
        out["prefill_bytes"] = kv + 2 * int(qlens.sum()) * hq * d * e
        pairs = sum(int(np.sum(c - t + np.arange(t) + 1)) for c, t in zip(pctx, qlens))
        out["prefill_flops"] = 4 * hq * d * pairs
    return out


def read_traffic(kv_dtype: str):
    """HBM bytes per partition-kernel launch from committed rocprofv3 counters,
    if they were taken on the current kernel source; else None."""
    path = COUNTERS_FILES[kv_dtype]
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if "=" in line and not line.lstrip().startswith("#"):
            k, v = line.split("=", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha") != kernel_source_hash():
        return None
    try:
        return int(float(vals["hbm_bytes_per_dispatch"]))
    except (KeyError, ValueError):
        return None


def host_description() -> dict:
    """The host the CPU baseline runs on: CPU model, logical CPUs, the CPUs this
    process may run on, and numpy's BLAS (vendor, version, thread pool)."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.lower().startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = {}
    try:
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                blas = {"vendor": i.get("internal_api"), "version": i.get("version"),
                        "threads": i.get("num_threads")}
                break
    except Exception:
        pass
    if not blas:
        try:
            cfg = np.show_config(mode="dicts")
            b = cfg["Build Dependencies"]["blas"]
            blas = {"vendor": b.get("name"), "version": b.get("version"), "threads": None}
        except Exception:
            blas = {"vendor": "unknown"}
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = None
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(), "affinity_cpus": affinity, "blas": blas}


def percentiles(xs) -> dict:
    a = np.asarray(xs, dtype=np.float64)
    if a.size == 0:
        return {}
    return {"median": round(float(np.median(a)), 2), "p10": round(float(np.percentile(a, 10)), 2),
            "p90": round(float(np.percentile(a, 90)), 2), "mean": round(float(a.mean()), 2), "n": int(a.size)}


def cpu_baseline(step, kv_dtype: str = "bf16", multi=None, min_seconds: float = 10.0, max_reps: int = 30):
    """The oracle, as it stands, on the same workload: append (with e4m3
    quantization for an fp8 cache) + decode (+ prefill), repeated until about
    ``min_seconds`` of CPU work (at least 3 runs) and timed per run; returns the
    median seconds per step, the runs and the threads."""
    import oracle
    from oracle import fp8 as f8
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    s = step
    pk = oracle.new_pool(s.num_blocks, s.block_size, s.num_kv_heads, s.head_dim, np.float32)
    pv = oracle.new_pool(s.num_blocks, s.block_size, s.num_kv_heads, s.head_dim, np.float32)
    if kv_dtype == "fp8":
        def stored(x):
            return f8.quantize_dequantize(x, FP8_SCALE)
    else:
        def stored(x):
            return x
    oracle.append(pk, pv, stored(s.cached_key.f32), stored(s.cached_value.f32), s.cached_slots)
    nk, nv, q = s.new_key.f32, s.new_value.f32, s.decode_query.f32
    new_slots = s.new_slots
    bt, cl = s.decode_inputs()
    if multi is not None:     # (T, query, new keys, new values, their slots)
        t, mq, mk, mv, new_slots = multi
        nk, nv, q = mk.f32, mv.f32, mq.f32
        cu = np.arange(len(cl) + 1, dtype=np.int64) * t
    pq = s.prefill_query.f32 if s.prefill_query is not None else None
    times = []
    while len(times) < 3 or (sum(times) < min_seconds and len(times) < max_reps):
        t0 = time.perf_counter()
        oracle.append(pk, pv, stored(nk), stored(nv), new_slots)
        if multi is None:
            oracle.paged_decode(q, pk, pv, bt, cl, s.scale)
        else:
            oracle.paged_prefill_chunk(q, cu, pk, pv, bt, cl, s.scale)
        if pq is not None:
            pbt, pcl = s.prefill_inputs()
            oracle.paged_prefill_chunk(pq, s.cu_q_lens, pk, pv, pbt, pcl, s.scale)
        times.append(time.perf_counter() - t0)
    return float(np.median(times)), len(times), threads


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--replicas", type=int, default=0, help="pool copies to rotate (0 = auto, >= 2 GiB)")
    ap.add_argument("--partition-size", type=int, default=None)
    ap.add_argument("--kv-dtype", choices=("bf16", "fp8"), default="bf16",
                    help="cache storage: bf16 (the workload's dtype) or e4m3 codes")
    ap.add_argument("--queries-per-seq", type=int, default=1,
                    help="query rows per decoding sequence (> 1: speculative-verification step)")
    ap.add_argument("--qwen-batch", type=int, default=16, help="--config 2: sequences (1, 4, 16, 64, 128)")
    ap.add_argument("--qwen-context", type=int, default=512, help="--config 2: context (128, 512, 2048)")
    ap.add_argument("--block-size", type=int, default=16, choices=(16, 32),
                    help="tokens per pool block (32: config 3 only)")
    ap.add_argument("--fused-append", action="store_true",
                    help="append and decode in one call (paged_attention_decode_append)")
    ap.add_argument("--shared", action="store_true",
                    help="decode through paged_attention_decode_shared with the step's sharing groups "
                         "(--config 6)")
    ap.add_argument("--graph", action="store_true",
                    help="capture each step in a HIP graph (torch.cuda.CUDAGraph) and time the replays")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-gather", action="store_true",
                    help="skip the gather-ceiling pass (paged_kv_gather_checksum over the same tiles)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="before warmup, copy this many MiB device-to-device once (a plain copy "
                         "of known size, to scale hardware byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the attention step "
              "has no cross-GPU part in this build.", file=sys.stderr)
        sys.exit(2)

    import torch
    import paged_kv_decode_reshape_amd as pkv
    pkv.load()
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)
    log(f"device: {props.name} ({getattr(props, 'gcnArchName', '?')}), "
        f"{props.multi_processor_count} CUs, {props.total_memory / 2**30:.0f} GiB")

    t0 = time.time()
    step = make_step(args.config, args.block_size, (args.qwen_batch, args.qwen_context))
    s = step
    log(f"workload {s.name}: generated in {time.time() - t0:.1f}s; "
        f"{len(s.decode_seqs)} decode seqs, tokens {int(s.context_lens.sum())}, info {s.info}")
    kvd = args.kv_dtype
    if kvd == "fp8" and s.dtype != "bf16":
        raise SystemExit("--kv-dtype fp8 needs a bf16 workload")
    tq = args.queries_per_seq
    if tq < 1:
        raise SystemExit("--queries-per-seq must be >= 1")
    shared = bool(args.shared)
    fused = bool(args.fused_append)
    if fused and (shared or tq != 1 or s.cu_q_lens is not None):
        raise SystemExit("--fused-append takes a decode-only step with one query row per sequence")
    if shared and ("group_starts" not in s.info or tq != 1):
        raise SystemExit("--shared needs a workload with sharing groups (--config 6) and one query per sequence")
    ab = algorithmic_bytes(s, kvd, tq, shared)
    tdt = torch.bfloat16 if s.dtype == "bf16" else torch.float32
    pool_dt = torch.uint8 if kvd == "fp8" else tdt
    pool_e = 1 if kvd == "fp8" else (2 if s.dtype == "bf16" else 4)
    dt_code = pkv.FP8_E4M3 if kvd == "fp8" else (pkv.BF16 if s.dtype == "bf16" else pkv.F32)

    def dev_vals(v):
        if v.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(v.bits).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(v.bits)).to(dev)

    def dev_int(a, dt=torch.int32):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dt).to(dev)

    # ---- pools: R replicas = R library layers ----
    kb, _ = pkv.kv_pool_bytes(s.num_blocks, s.block_size, s.num_kv_heads, s.head_dim, dt_code)
    # Enough copies that the rotation spans >= 2 GiB, capped at 64: smaller
    # pools then fit the 256 MB Infinity Cache together and the timing is warm
    # (config.cache says which).
    reps = args.replicas or min(64, max(2, math.ceil(2 * 2**30 / (2 * kb))))
    cache_state = "cold (rotation >= 2 GiB)" if reps * 2 * kb >= 2 * 2**30 else "warm (rotation fits the Infinity Cache)" \
        if reps * 2 * kb <= 256 * 2**20 else "partly warm"
    k_layers = [torch.empty(kb // pool_e, dtype=pool_dt, device=dev) for _ in range(reps)]
    v_layers = [torch.empty(kb // pool_e, dtype=pool_dt, device=dev) for _ in range(reps)]
    pool = pkv.kv_pool_create(reps, s.num_blocks, s.block_size, s.num_kv_heads, s.head_dim,
                              dt_code, k_layers, v_layers)
    if kvd == "fp8":
        pkv.kv_pool_set_fp8_scales(pool, [FP8_SCALE] * reps, [FP8_SCALE] * reps)
    stream = torch.cuda.current_stream(dev)
    pkv.reshape_and_cache(pool, 0, dev_vals(s.cached_key), dev_vals(s.cached_value),
                          dev_int(s.cached_slots, torch.int64), len(s.cached_slots), stream)
    for r in range(1, reps):
        k_layers[r].copy_(k_layers[0])
        v_layers[r].copy_(v_layers[0])
    bt, cl = s.decode_inputs()
    bt_d, cl_d = dev_int(bt), dev_int(cl)
    nseq = len(cl)
    multi = None
    if tq > 1:
        multi = (tq,) + multi_query_inputs(s, tq)
        _, mq, mk, mv, mslots = multi
        new_k, new_v, new_slots, n_new = dev_vals(mk), dev_vals(mv), dev_int(mslots, torch.int64), len(mslots)
        q_d = dev_vals(mq)
    else:
        new_k, new_v = dev_vals(s.new_key), dev_vals(s.new_value)
        new_slots = dev_int(s.new_slots, torch.int64)
        n_new = len(s.new_slots)
        q_d = dev_vals(s.decode_query)
    out = torch.empty((nseq * tq, s.num_q_heads, s.head_dim), dtype=tdt, device=dev)
    if fused:
        # the new rows are in sequence order: every decoding sequence appends one token
        assert len(s.new_slots) == nseq and (cl > 0).all()
    part = s.partition_size if args.partition_size is None else args.partition_size
    if shared:
        gs_d, pl_d = dev_int(s.info["group_starts"]), dev_int(s.info["prefix_lens"])
        n_groups = len(s.info["prefix_lens"])
        max_group = int(np.max(np.diff(s.info["group_starts"])))
        wsb = pkv.paged_attention_decode_shared_workspace_bytes(pool, nseq, s.num_q_heads, bt.shape[1], part)
    else:
        wsb = pkv.paged_attention_decode_multi_workspace_bytes(pool, nseq, tq, s.num_q_heads, bt.shape[1], part)
    ws = torch.zeros(max(wsb, 16), dtype=torch.uint8, device=dev)
    has_prefill = s.cu_q_lens is not None
    if has_prefill:
        pbt, pcl = s.prefill_inputs()
        pbt_d, pcl_d, cu_d = dev_int(pbt), dev_int(pcl), dev_int(s.cu_q_lens)
        pq_d = dev_vals(s.prefill_query)
        ptotal = int(s.cu_q_lens[-1])
        pmax = int(np.max(np.diff(s.cu_q_lens)))
        pout = torch.empty((ptotal, s.num_q_heads, s.head_dim), dtype=tdt, device=dev)
    torch.cuda.synchronize()
    log(f"pool: {reps} replicas x {2 * kb / 2**30:.2f} GiB (K+V); workspace {wsb / 2**20:.1f} MiB")

    def one_step(i):
        layer = i % reps
        stream = torch.cuda.current_stream(dev)     # the capture stream while a graph is recorded
        if fused:
            pkv.paged_attention_decode_append(pool, layer, out, q_d, new_k, new_v, bt_d, cl_d, nseq, s.num_q_heads,
                                              bt.shape[1], s.scale, part, ws, wsb, stream)
            return
        pkv.reshape_and_cache(pool, layer, new_k, new_v, new_slots, n_new, stream)
        if shared:
            pkv.paged_attention_decode_shared(pool, layer, out, q_d, bt_d, cl_d, gs_d, pl_d, nseq, n_groups,
                                              max_group, s.num_q_heads, bt.shape[1], s.scale, part, ws, wsb,
                                              stream)
        elif tq == 1:
            pkv.paged_attention_decode(pool, layer, out, q_d, bt_d, cl_d, nseq, s.num_q_heads,
                                       bt.shape[1], s.scale, part, ws, wsb, stream)
        else:
            pkv.paged_attention_decode_multi(pool, layer, out, q_d, tq, bt_d, cl_d, nseq, s.num_q_heads,
                                             bt.shape[1], s.scale, part, ws, wsb, stream)
        if has_prefill:
            pkv.paged_attention_prefill_chunk(pool, layer, pout, pq_d, cu_d, pbt_d, pcl_d,
                                              len(pcl), ptotal, pmax, s.num_q_heads,
                                              pbt.shape[1], s.scale, stream)

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty(n, dtype=torch.uint8, device=dev)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for i in range(args.warmup):
        one_step(i)
    torch.cuda.synchronize()
    # Timed region: HIP events only around the kernels the JSON's rates need
    # (the decode partition kernel, and the prefill kernel when present); each
    # event pair adds a gap to the stream.
    kinds_all = (("append", pkv.KERNEL_APPEND), ("partition", pkv.KERNEL_DECODE_PARTITION),
                 ("reduce", pkv.KERNEL_DECODE_REDUCE), ("prefill", pkv.KERNEL_PREFILL),
                 ("prefix", pkv.KERNEL_DECODE_PREFIX))
    timed_kinds = [pkv.KERNEL_DECODE_PARTITION, pkv.KERNEL_DECODE_REDUCE] + \
        ([pkv.KERNEL_PREFILL] if has_prefill else []) + ([pkv.KERNEL_DECODE_PREFIX] if shared else [])
    launches = {}
    if args.graph:
        # One captured step per pool replica; step i replays graph i % reps.
        # Kernel durations then come from the separate eager pass below.
        graphs = []
        for r in range(reps):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                one_step(r)
            graphs.append(g)
        for i in range(args.warmup):
            graphs[i % reps].replay()
        torch.cuda.synchronize()
        timed_kinds = []
        kt = {}
        t_start = time.perf_counter()
        for i in range(args.steps):
            graphs[i % reps].replay()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t_start
    else:
        pkv.pkv_timing_enable(2 * args.steps + 8, timed_kinds)
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        for i in range(args.steps):
            one_step(args.warmup + i)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t_start
        kt = {name: pkv.pkv_timing_read(kind) for name, kind in kinds_all if kind in timed_kinds}
        launches = {name: pkv.pkv_timing_read_launches(kind, 2 * args.steps + 8)
                    for name, kind in kinds_all if kind in timed_kinds}
        pkv.pkv_timing_disable()
    # The other kernels' durations, from a separate untimed pass with events on
    # every kernel.
    n_break = min(args.steps, 20)
    pkv.pkv_timing_enable(4 * n_break + 8)
    for i in range(n_break):
        one_step(args.warmup + args.steps + i)
    torch.cuda.synchronize()
    for name, kind in kinds_all:
        if kind not in timed_kinds:
            kt[name] = pkv.pkv_timing_read(kind)
    pkv.pkv_timing_disable()
    # Per-step durations: a separate pass of the same number of steps, with one
    # event pair around every step on the launch stream (no library events),
    # for the median and p10/p90.
    stream_now = torch.cuda.current_stream(dev)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        evs[i][0].record(stream_now)
        if args.graph:
            graphs[i % reps].replay()
        else:
            one_step(args.warmup + i)
        evs[i][1].record(stream_now)
    torch.cuda.synchronize()
    step_us = [a.elapsed_time(b) * 1e3 for a, b in evs]
    # Gather ceiling: the decode's K/V words read through the same tables, the
    # same pool rotation and the same split, with no attention arithmetic
    # (paged_kv_gather_checksum); its kernel's event times, in a pass of its own.
    gather_us = None
    if not args.no_gather and tq == 1 and not shared and nseq <= 8192:
        chk = torch.empty((nseq, s.num_kv_heads), dtype=torch.int32, device=dev)
        gws = torch.empty(((nseq + 1) * 4 + 15) // 16 * 16, dtype=torch.uint8, device=dev)

        def gather(i):
            pkv.paged_kv_gather_checksum(pool, i % reps, chk, bt_d, cl_d, nseq, bt.shape[1], gws, gws.numel(),
                                         torch.cuda.current_stream(dev))

        for i in range(args.warmup):
            gather(i)
        torch.cuda.synchronize()
        pkv.pkv_timing_enable(args.steps + 8, [pkv.KERNEL_GATHER])
        for i in range(args.steps):
            gather(args.warmup + i)
        torch.cuda.synchronize()
        gather_us = [x * 1e3 for x in pkv.pkv_timing_read_launches(pkv.KERNEL_GATHER, args.steps + 8)]
        pkv.pkv_timing_disable()
    ms_per_step = wall * 1e3 / args.steps
    avg_us = {k: (ms / n * 1e3 if n else 0.0) for k, (n, ms) in kt.items()}
    avg_us = {k: avg_us[k] for k, _ in kinds_all}
    log("kernel avg us: " + ", ".join(f"{k} {v:.1f}" for k, v in avg_us.items()))

    step_bytes = ab["decode_kv"] + ab["decode_qo"] + ab["append"] + ab.get("prefill_bytes", 0)
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    part_bytes = ab["decode_kv"] + ab["decode_qo"]
    # With shared prefixes the KV is read by two kernels (the groups' shared
    # partitions, then each sequence's own): the roofline covers both.
    read_us = avg_us["partition"] + avg_us["prefix"]
    decode_us = read_us + avg_us["reduce"]
    # The roofline covers the whole decode: the partition kernel(s) and, where
    # split rows are combined by a second kernel, that reduction too.
    achieved = part_bytes / (decode_us * 1e-6) / 1e9 if decode_us else 0.0
    achieved_read = part_bytes / (read_us * 1e-6) / 1e9 if read_us else 0.0
    balanced = (part == 0) and nseq <= 4096
    if shared:
        kernel_label = "decode_prefix_kernel + decode_balanced_kernel + decode_balanced_reduce_kernel"
    elif balanced and not avg_us["reduce"]:
        kernel_label = "decode_balanced_kernel (split rows combined in the launch" + \
                       (", append fused)" if fused else ")")
    elif balanced:
        kernel_label = "decode_balanced_kernel + decode_balanced_reduce(_coop)_kernel"
    else:
        kernel_label = "decode_partition_kernel" + (" + decode_reduce_kernel" if avg_us["reduce"] else "")
    result = {
        "metric": "paged decode attention: achieved HBM GB/s (% of peak) and us per layer-step",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": s.dtype,
        "data": {2: "synthetic (seeded N(0,1) values, uniform context, blocks scattered by a seeded permutation)",
                 3: "synthetic (seeded N(0,1) values, lognormal lengths, churned block tables)",
                 4: "synthetic (seeded N(0,1) values, 1% of K rows x8, blocks scattered by a seeded permutation)",
                 5: "synthetic (seeded N(0,1) values, uniform 128..4096 decode contexts, one shared scattered pool)",
                 6: "synthetic (seeded N(0,1) values, 32 prompts x 8 samples sharing prompt blocks, "
                    "uniform 1..512 generated tokens)"}[args.config],
        "config": {
            "workload": s.name if tq == 1 else f"{s.name}_q{tq}",
            "batch": nseq,
            "num_q_heads": s.num_q_heads, "num_kv_heads": s.num_kv_heads,
            "head_dim": s.head_dim, "block_size": s.block_size,
            "context_tokens": int(cl.sum()),
            "partition_size": part if part else "auto",
            "kv_cache_dtype": "fp8_e4m3" if kvd == "fp8" else s.dtype,
            "queries_per_seq": tq,
            "shared_prefix_decode": shared,
            "fused_append": fused,
            "cache": cache_state,
            "pool_replicas": reps,
            "parallelism": "single GPU",
        },
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 1),
        "us_per_layer_step": round(ms_per_step * 1e3, 2),
        "kernel_us": {k: round(v, 2) for k, v in avg_us.items()},
        "kernel_us_source": ("all kernels: a separate eager pass of " if args.graph else
                             "decode partition and reduction" + (" and prefill" if has_prefill else "") +
                             ": HIP events in the timed region; the others: a separate ") +
                            f"{n_break}-step pass with events on every kernel",
        "kernel_us_percentiles": {k: percentiles([x * 1e3 for x in v]) for k, v in launches.items() if v},
        "step_us": dict(percentiles(step_us), source=f"a separate pass of {args.steps} steps, one HIP event "
                                                     "pair around each step on the launch stream"),
        "graph": bool(args.graph),
        "decode_attention_gbs": round(part_bytes / (decode_us * 1e-6) / 1e9, 1) if decode_us else None,
        "algorithmic_bytes": ab,
        "roofline": {
            "kernel": kernel_label,
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": (read_traffic(kvd) if tq == 1 and not shared and not fused and args.config == 3 and
                        s.block_size == 16 else None),
            "algorithmic_bytes_per_launch": part_bytes,
            "decode_us": round(decode_us, 2),
            "partition_only": {"achieved": round(achieved_read, 1),
                               "frac": round(achieved_read / HBM_PEAK_GBS, 4), "us": round(read_us, 2)},
        },
    }
    if gather_us:
        g_mean = sum(gather_us) / len(gather_us)
        g_gbs = ab["decode_kv"] / (g_mean * 1e-6) / 1e9
        result["gather_ceiling"] = {
            "kernel": "gather_kernel (paged_kv_gather_checksum: the decode's K/V words, no arithmetic)",
            "us": percentiles(gather_us),
            "achieved": round(g_gbs, 1), "unit": "GB/s", "frac_of_peak": round(g_gbs / HBM_PEAK_GBS, 4),
            "bytes_per_launch": ab["decode_kv"],
            "decode_over_gather": round(decode_us / g_mean, 4) if decode_us else None,
        }
    if has_prefill and avg_us["prefill"]:
        tf = ab["prefill_flops"] / (avg_us["prefill"] * 1e-6) / 1e12
        result["prefill_mfma"] = {"tflops": round(tf, 1), "peak": BF16_MFMA_PEAK_TFLOPS,
                                  "utilisation": round(tf / BF16_MFMA_PEAK_TFLOPS, 4),
                                  "flops_per_launch": ab["prefill_flops"]}
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on the same step ...")
        t_cpu, runs, threads = cpu_baseline(s, kvd, multi)
        result["cpu_baseline"] = {
            "value": round(step_bytes / t_cpu / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "host": host_description(),
            "sample": f"the whole step ({s.name}{', e4m3 cache' if kvd == 'fp8' else ''}"
                      f"{f', {tq} query rows per sequence' if tq > 1 else ''}: append + decode of all {nseq} sequences"
                      f"{' + prefill chunk' if has_prefill else ''}), numpy float64, median of {runs} runs"
                      f" ({runs * t_cpu:.0f} s of CPU work); {t_cpu:.2f} s per step; BLAS pool of"
                      f" {threads} threads, the per-sequence loop single-threaded; {os.cpu_count()} host CPUs",
        }
    pkv.kv_pool_destroy(pool)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
