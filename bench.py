#!/usr/bin/env python3
"""Paged-decode benchmark on one MI355X.

A step is one pass of the whole hot path over one batch: the native block
manager appends one token to every sequence (slots), the step's slots,
positions and new lengths go to pinned host memory, the cache write stores
the new K/V rows and patches the device-resident block tables and lengths
from those slots, and paged decode (partition kernel + log-sum-exp merge)
attends over every context.  Contexts grow by one token per step.
Inputs are seeded synthetic values of the workload's shape, resident in HBM
before timing starts.

Prints one JSON line: whole-step KV throughput (GB/s), the roofline of the
dominant kernel (decode partitions, timed with HIP events on the launch
stream), the HBM read ceilings of a plain stream and of a random gather of
decode tiles on the same GPU, and the CPU oracle timed on a bounded sample of
the same workload.  The serving workloads (serving_bf16, serving_prefix_bf16)
instead time whole scheduler + kernel steps (steps/s).
"""

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

METRIC = "paged decode KV GB/s and % of HBM peak (seqs/s) at 1 MI355X"
# The headline: the largest single-GPU decode configuration, 16 sequences at
# 32,768 tokens, 64/8 heads, bf16, at its stated 512-token partitions.  The
# other gated decode configurations, and the headline's at the library's
# default partition, are reported in the same line (kernel figures only).
HEADLINE = "longctx_bf16"
EVENT_EVERY = 4  # timed steps per step whose decode launches are bracketed by timing events
RING_GROUP = 8  # pinned metadata slots covered by one completion event
EXTRA_CONFIGS = ["mha7b_f16", "gqa8b_bf16", "longctx_bf16"]
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16/fp16 matrix, published
ESIZE = {"f32": 4, "f16": 2, "bf16": 2}
KERNEL_SOURCES = ["paged_kv_cache_395_amd/csrc/decode_kernels.hip", "paged_kv_cache_395_amd/csrc/device_common.h",
                  "paged_kv_cache_395_amd/csrc/pa_internal.h"]


class TimingEvent:
    """A HIP event for timing only, recorded without the system-scope fence.

    torch's events release at system scope when they are recorded: the L2 is
    written back and invalidated, which costs the next kernel its cached
    inputs and adds several microseconds per record to a ~0.2 ms step.
    These events are read only after a device synchronisation, so they need
    no fence (hipEventDisableSystemFence).  They are made through the HIP
    runtime torch loaded (the library shares that runtime).  Events the host
    waits on before it rewrites pinned memory stay torch's.
    """

    _hip = None
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes

        import torch

        if TimingEvent._hip is None:
            lib = ctypes.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
            lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
            TimingEvent._hip = lib
        self._ct = ctypes
        self._h = ctypes.c_void_p()
        self._check(TimingEvent._hip.hipEventCreateWithFlags(ctypes.byref(self._h), self.DISABLE_SYSTEM_FENCE),
                    "hipEventCreateWithFlags")

    @staticmethod
    def _check(rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed with HIP error {rc}")

    def record(self, stream=None):
        import torch

        s = stream if stream is not None else torch.cuda.current_stream()
        self._check(TimingEvent._hip.hipEventRecord(self._h, self._ct.c_void_p(s.cuda_stream)), "hipEventRecord")

    def elapsed_time(self, end) -> float:
        """Milliseconds from this event to ``end`` (both recorded, the device synchronised)."""
        ms = self._ct.c_float()
        self._check(TimingEvent._hip.hipEventElapsedTime(self._ct.byref(ms), self._h, end._h), "hipEventElapsedTime")
        return ms.value

    def __del__(self):
        if TimingEvent._hip is not None and self._h:
            TimingEvent._hip.hipEventDestroy(self._h)


def appends_fit(bm, w, tokens: int) -> bool:
    """Whether the pool's free blocks hold ``tokens`` more tokens for every sequence of the batch."""
    bs = w.block_size
    need = 0
    for s in w.batch:
        n = bm.num_tokens(int(s))
        need += -(-(n + tokens) // bs) - -(-n // bs)
    return need <= bm.num_free()


def decode_bytes(ctx: np.ndarray, w) -> float:
    """Algorithmic bytes of one decode: K+V rows of every context token, q, out, table entries read."""
    e = ESIZE[w.dtype]
    kv = float(np.sum(ctx, dtype=np.int64)) * w.num_kv_heads * w.head_dim * 2 * e
    nq = w.append if w.lengths.get("mode") == "multi" else 1  # queries per sequence
    qo = 2.0 * len(ctx) * nq * w.num_q_heads * w.head_dim * e
    bs = w.block_size
    tab = float(np.sum((ctx + bs - 1) // bs, dtype=np.int64)) * 4
    return kv + qo + tab


def physical_kv_bytes(table: np.ndarray, ctx: np.ndarray, w) -> float:
    """K/V bytes of the distinct physical blocks a batch reads: each block's
    valid tokens once, however many sequences share it."""
    bs = w.block_size
    valid = {}
    for s in range(len(ctx)):
        n = int(ctx[s])
        for lb in range((n + bs - 1) // bs):
            b = int(table[s, lb])
            valid[b] = max(valid.get(b, 0), min(bs, n - lb * bs))
    return float(sum(valid.values())) * w.num_kv_heads * w.head_dim * 2 * ESIZE[w.dtype]


def prefill_flops(ctx: np.ndarray, chunk: int, w) -> float:
    """4 * D flops (QK and PV) per (query row, q head, attended key)."""
    total = 0.0
    for c in ctx:
        keys = np.arange(int(c) - chunk + 1, int(c) + 1, dtype=np.float64)
        total += float(keys.sum())
    return total * 4.0 * w.head_dim * w.num_q_heads


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str, bytes_per_launch: float):
    """(HBM bytes per launch, HBM / algorithmic bytes) from committed rocprofv3
    counter runs, if they were taken on the current kernel source; else
    (None, None).  The counter runs time a few short steps; the measured
    ratio of HBM to algorithmic bytes carries over to this run's mean launch
    (longer contexts after more steps), so the bytes are scaled by it."""
    path = os.path.join(ROOT, "profiles", f"decode_partitions_{workload}_traffic.json")
    if not os.path.exists(path):
        return None, None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha") != kernel_source_hash():
        return None, None
    ratio = rec["hbm_bytes_per_launch"] / rec["algorithmic_bytes_per_launch"]
    return ratio * bytes_per_launch, ratio


def _host_threads() -> int:
    """Host cores this process may use: the CPU share the environment
    states (OMP_NUM_THREADS), else the affinity mask."""
    env = os.environ.get("OMP_NUM_THREADS", "")
    n = int(env) if env.isdigit() and int(env) > 0 else 0
    return min(n, len(os.sched_getaffinity(0))) if n else len(os.sched_getaffinity(0))


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, budget_s: float = 15.0):
    """The oracle, as it stands, on the sequences of the same step in order,
    cycling over the batch again when a pass ends, until ~budget_s of work,
    with BLAS on every host core the process may use."""
    from threadpoolctl import threadpool_limits

    from oracle import attention as OA
    from oracle.block_manager import RefBlockManager
    from workloads import run_program

    ref = RefBlockManager(w.num_blocks, block_size=w.block_size, free_order=w.free_order)
    run_program(ref, w.program)
    slots, _ = ref.append_tokens(list(w.step_seqs))
    table, ctx = ref.block_table(list(w.batch), w.max_blocks_per_seq(), pad=0)
    table, ctx = np.array(table, np.int32), np.array(ctx, np.int32)
    k, v = w.k_pool, w.v_pool  # written in place; the benchmark has its own device copies
    done = []
    cores = _host_threads()
    with threadpool_limits(limits=cores):
        t0 = time.perf_counter()
        OA.reshape_and_cache(k, v, w.step_rows("k"), w.step_rows("v"), np.array(slots))
        multi = w.lengths.get("mode") == "multi"
        for i in range(100 * w.num_seqs):
            s = i % w.num_seqs
            if multi:  # the verification workload: each sequence's last w.append positions, causally
                OA.prefill_chunk(w.q, k, v, table, ctx, w.scale, w.dtype, seqs=[s])
            else:
                OA.decode(w.decode_q, k, v, table, ctx, w.scale, w.dtype, seqs=[s])
            done.append(s)
            if time.perf_counter() - t0 > budget_s:
                break
        dt = time.perf_counter() - t0
    sub = ctx[done]
    gbs = decode_bytes(sub, w) / dt / 1e9
    passes = len(done) / w.num_seqs
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": cores, "kind": "oracle", "cpu": _cpu_model(),
            "sample": f"the step's cache write of {w.num_seqs} tokens, then fp64 attention over its sequences "
                      f"in order, {len(done)} sequence decodes ({passes:.2f} passes over the {w.num_seqs}), all "
                      f"{w.num_q_heads} q heads; {dt:.1f} s; seqs/s {len(done) / dt:.2f}; numpy, BLAS on "
                      f"{cores} cores"}


SERVING = dict(num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16", rows=256, num_blocks=10000,
               host_blocks=8000, max_blocks=192, budget=4096, requests=1200, mean_gap=0.5, prompt_median=512,
               prompt_hi=2048, output_median=256, output_hi=1024, seed=2024)
SERVING_DESC = ("continuous batching: GQA 32/8 heads, head_dim 128, bf16, 256 rows, pool 10000 blocks (640 MiB; "
                "too small for the peak, so requests are preempted), host swap pool 8000 blocks, Poisson arrivals "
                "every 0.5 steps, prompts lognormal median 512 (<= 2048), outputs median 256 (<= 1024), "
                "4096 batched tokens per step")


def serving_cpu_baseline(c, trace, steps: int, budget_s: float = 15.0, prefix: bool = False):
    """The oracle scheduler over the same trace, plus oracle fp64 decode of a
    bounded sample of rows at the last step, scaled to one whole step."""
    from threadpoolctl import threadpool_limits

    from oracle import attention as OA
    from oracle.block_manager import RefBlockManager
    from oracle.scheduler import RefScheduler
    from workloads import to_storage

    bm = RefBlockManager(c["num_blocks"])
    if prefix:
        bm.enable_prefix_cache()
    bm.set_host_pool(c["host_blocks"])
    sched = RefScheduler(bm, c["rows"], c["max_blocks"], c["budget"])
    pending = list(trace)
    t0 = time.perf_counter()
    for step in range(steps):
        while pending and pending[0][0] <= step:
            _, i, p, t = pending.pop(0)
            if prefix:
                sched.submit(i, len(p), t, p)
            else:
                sched.submit(i, p, t)
        st = sched.step()
    t_sched = (time.perf_counter() - t0) / steps
    # attention of a sample of rows over random pools of the real shape
    rng = np.random.default_rng(5)
    Hq, Hkv, D, dt = c["num_q_heads"], c["num_kv_heads"], c["head_dim"], c["dtype"]
    rows = [r for r, s in enumerate(st["row_seq"]) if s >= 0]
    table, ctx = np.zeros((len(rows), c["max_blocks"]), np.int32), np.zeros(len(rows), np.int32)
    for j, r in enumerate(rows):
        t, n = bm.block_table([st["row_seq"][r]], c["max_blocks"], pad=0)
        table[j], ctx[j] = t[0], n[0]
    used = sorted({int(b) for j in range(len(rows)) for b in table[j, : -(-int(ctx[j]) // 16)]})
    remap = {b: i for i, b in enumerate(used)}
    table = np.vectorize(lambda b: remap.get(int(b), 0))(table).astype(np.int32)
    k = to_storage(rng.standard_normal((len(used), Hkv, 16 * D), dtype=np.float32), dt)
    v = to_storage(rng.standard_normal((len(used), Hkv, 16 * D), dtype=np.float32), dt)
    q = to_storage(rng.standard_normal((len(rows), Hq, D), dtype=np.float32), dt)
    done = []
    cores = _host_threads()
    with threadpool_limits(limits=cores):
        t1 = time.perf_counter()
        for j in range(len(rows)):
            OA.decode(q, k, v, table, ctx, D ** -0.5, dt, seqs=[j])
            done.append(j)
            if time.perf_counter() - t1 > budget_s:
                break
        t_att = time.perf_counter() - t1
    per_step = t_sched + t_att * len(rows) / len(done)
    return {"value": round(1.0 / per_step, 4), "unit": "steps/s", "cores": cores, "kind": "oracle", "cpu": _cpu_model(),
            "sample": f"oracle scheduler over the first {steps} steps of the same trace ({t_sched * 1e3:.2f} ms "
                      f"per step) + fp64 oracle decode of {len(done)} of the {len(rows)} running rows at the "
                      f"last step ({t_att:.1f} s), scaled to all rows; numpy, BLAS on {cores} cores"}


SERVING_PREFIX = dict(SERVING, prompts=8, system_len=512, tail_median=128, tail_hi=1024)
SERVING_PREFIX_DESC = ("continuous batching with automatic prefix caching: the serving_bf16 shapes, pool and "
                       "arrivals, prompts = one of 8 shared 512-token system prompts + a lognormal tail "
                       "(median 128, <= 1024), outputs median 256 (<= 1024); admission shares cached prompt blocks")


def bench_serving(args) -> None:
    """Continuous batching through the native scheduler and the driver."""
    import torch

    from paged_kv_cache_395_amd import ops
    from paged_kv_cache_395_amd.driver import Driver
    from workloads.serving import prefix_requests, request_trace

    prefix = args.workload == "serving_prefix_bf16"
    c = dict(SERVING_PREFIX if prefix else SERVING)
    if prefix:
        trace = prefix_requests(c["seed"], c["requests"], c["prompts"], c["system_len"], c["tail_median"],
                                c["tail_hi"], c["output_median"], c["output_hi"], c["mean_gap"])
        trace = [(a, i, ids, min(t, c["max_blocks"] * 16)) for a, i, ids, t in trace]
    else:
        trace = request_trace(c["seed"], c["requests"], c["mean_gap"], c["prompt_median"], c["prompt_hi"],
                              c["output_median"], c["output_hi"], lo=16)
        trace = [(a, i, p, min(t, c["max_blocks"] * 16)) for a, i, p, t in trace]
    torch.cuda.set_device(0)
    Hq, Hkv, D = c["num_q_heads"], c["num_kv_heads"], c["head_dim"]
    drv = Driver(c["num_blocks"], c["host_blocks"], Hq, Hkv, D, c["dtype"], c["rows"], c["max_blocks"],
                 c["budget"], D ** -0.5, prefix_cache=prefix)
    g = torch.Generator(device="cuda")
    g.manual_seed(c["seed"])
    for t in (drv.key, drv.value, drv.q, drv.k_pool, drv.v_pool):
        t.copy_(torch.randn(t.shape, generator=g, device="cuda", dtype=torch.float32).to(t.dtype))
    esize = ESIZE[c["dtype"]]
    block_bytes = Hkv * 16 * D * esize * 2
    pending = list(trace)
    stats = {"decode_bytes": 0.0, "tokens": 0, "prompt_tokens": 0, "cached_tokens": 0, "swap_blocks": 0, "swap_out": 0, "swap_in": 0, "recompute": 0,
             "admitted": 0, "finished": 0, "rows": 0}
    ev = []

    def one(step, timed):
        while pending and pending[0][0] <= step:
            _, i, p, t = pending.pop(0)
            if prefix:
                drv.submit(i, len(p), t, p)
            else:
                drv.submit(i, p, t)
        st = drv.schedule()
        e = (TimingEvent(), TimingEvent()) if timed else None
        drv.launch(st, decode_events=e)
        if timed:
            ev.append(e)
            ctx = st.context_lens.astype(np.float64)
            stats["decode_bytes"] += float((ctx * Hkv * D * 2 * esize).sum() + (ctx > 0).sum() * Hq * D * (esize + 4))
            generated = st.num_running - st.num_admitted  # one token each; the rest are admitted prompts
            stats["tokens"] += generated
            stats["prompt_tokens"] += len(st.slots) - generated
            stats["cached_tokens"] += st.num_cached_tokens
            stats["swap_blocks"] += len(st.swap_out) + len(st.swap_in)
            stats["swap_out"] += st.num_preempted_swap
            stats["swap_in"] += st.num_swapped_in
            stats["recompute"] += st.num_preempted_recompute
            stats["admitted"] += st.num_admitted
            stats["finished"] += len(st.finished)
            stats["rows"] += st.num_running
        return st

    for i in range(args.warmup):
        one(i, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        one(args.warmup + i, True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    dec_ms = np.array([a.elapsed_time(b) for a, b in ev])
    K = args.steps
    read_bytes = stats["decode_bytes"]
    unique = None
    if prefix:
        # rows that share cached prompt blocks read each shared block once from HBM (the rest hit in cache);
        # the roofline counts each distinct block once.  Replaying the same trace through a host-only
        # scheduler reproduces every step's tables (the block manager is deterministic).
        from paged_kv_cache_395_amd import BlockManager, Scheduler
        bm2 = BlockManager(c["num_blocks"])
        bm2.enable_prefix_cache()
        bm2.set_host_pool(c["host_blocks"])
        sc2 = Scheduler(bm2, c["rows"], c["max_blocks"], c["budget"])
        pend2 = list(trace)
        dup_tokens = 0
        for step in range(args.warmup + K):
            while pend2 and pend2[0][0] <= step:
                _, i, p, t = pend2.pop(0)
                sc2.submit(i, len(p), t, p)
            st2 = sc2.step()
            if step < args.warmup:
                continue
            live = [int(x) for x in st2.row_seq if x >= 0]
            tab, ctx2 = bm2.block_table(live, c["max_blocks"])
            refs = np.concatenate([tab[j, : -(-int(n) // 16)] for j, n in enumerate(ctx2)])
            _, counts = np.unique(refs, return_counts=True)
            dup_tokens += int((counts - 1).sum()) * 16  # only full prompt blocks are shared
        unique = read_bytes - dup_tokens * Hkv * D * 2 * esize
        read_bytes = unique
    achieved = read_bytes / (dec_ms.sum() * 1e-3) / 1e9
    rec = {
        "metric": "continuous-batching attention steps/s (decode KV GB/s) at 1 MI355X",
        "value": round(K / elapsed, 2),
        "unit": "steps/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": round(elapsed / K * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": c["dtype"], "data": "synthetic",
        "config": {"workload": (f"serving_prefix_bf16: {SERVING_PREFIX_DESC}" if prefix
                                else f"serving_bf16: {SERVING_DESC}"), **{k: c[k] for k in ("rows", "num_blocks",
                   "host_blocks", "budget", "num_q_heads", "num_kv_heads", "head_dim")}},
        "generated_tokens_per_s": round(stats["tokens"] / elapsed, 1),
        "prompt_tokens_written_per_s": round(stats["prompt_tokens"] / elapsed, 1),
        "prompt_tokens_from_prefix_cache_per_s": round(stats["cached_tokens"] / elapsed, 1),
        "mean_running_rows": round(stats["rows"] / K, 1),
        "decode_kv_gbs_whole_step": round(stats["decode_bytes"] / elapsed / 1e9, 1),
        "swap": {"blocks": stats["swap_blocks"], "gb": round(stats["swap_blocks"] * block_bytes / 1e9, 3),
                 "preempted_swap": stats["swap_out"], "swapped_in": stats["swap_in"],
                 "preempted_recompute": stats["recompute"]},
        "admitted": stats["admitted"], "finished": stats["finished"],
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None, "kernel": "decode_partition_kernel",
                     "algorithmic_bytes_per_launch": round(read_bytes / K, 1)},
    }
    if unique is not None:
        rec["roofline"]["bytes_note"] = ("distinct blocks counted once; rows read "
                                         f"{stats['decode_bytes'] / unique:.2f}x these bytes in all, the shared "
                                         "prompt blocks from cache")
        rec["roofline"]["logical_gbs"] = round(stats["decode_bytes"] / (dec_ms.sum() * 1e-3) / 1e9, 2)
    # the swap copy alone: one launch of 2048 block pairs each way
    n = min(2048, c["host_blocks"], c["num_blocks"])
    pairs_out = torch.from_numpy(np.stack([np.arange(n), np.arange(n)], axis=1).astype(np.int64)).cuda()
    a, b, d = (TimingEvent() for _ in range(3))
    ops.swap_blocks(drv.k_host, drv.v_host, drv.k_pool, drv.v_pool, pairs_out)
    a.record()
    ops.swap_blocks(drv.k_host, drv.v_host, drv.k_pool, drv.v_pool, pairs_out)
    b.record()
    ops.swap_blocks(drv.k_pool, drv.v_pool, drv.k_host, drv.v_host, pairs_out)
    d.record()
    torch.cuda.synchronize()
    rec["swap_copy_gbs"] = {"device_to_host": round(n * block_bytes / (a.elapsed_time(b) * 1e-3) / 1e9, 2),
                            "host_to_device": round(n * block_bytes / (b.elapsed_time(d) * 1e-3) / 1e9, 2),
                            "blocks": n}
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = serving_cpu_baseline(c, trace, args.warmup + args.steps, prefix=prefix)
    print(json.dumps(rec), flush=True)


COPY_KERNEL = "__amd_rocclr_copyBuffer"


def _csv_rows(directory: str, suffix: str):
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True)):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    return rows


def _per_dispatch(rows, name: str) -> tuple:
    vals = [float(r["Counter_Value"]) for r in rows if name in r["Kernel_Name"]]
    return (sum(vals) / len(vals), len(vals)) if vals else (float("nan"), 0)


def _largest_dispatch(rows, name: str) -> float:
    """The copy probe: the largest of the run's copy dispatches (the others
    are the small table / length copies of the set-up)."""
    vals = [float(r["Counter_Value"]) for r in rows if name in r["Kernel_Name"]]
    return max(vals) if vals else float("nan")


def summarize_prefill(args, rec) -> None:
    """Matrix-core utilisation of the chunked-prefill kernel from one rocprofv3
    counter pass (SQ block) and one GRBM pass of the same command."""
    wl = args.workload
    rows = _csv_rows(args.prefill_pmc_dir, "counter_collection.csv")
    grbm = _csv_rows(args.prefill_grbm_dir, "counter_collection.csv")

    def avg(rs, counter):
        v = [float(r["Counter_Value"]) for r in rs if "prefill_mfma_kernel" in r["Kernel_Name"]
             and r["Counter_Name"] == counter]
        return sum(v) / len(v) if v else float("nan"), len(v)

    busy, n = avg(rows, "SQ_VALU_MFMA_BUSY_CYCLES")
    cu, _ = avg(rows, "SQ_BUSY_CU_CYCLES")
    vact, _ = avg(rows, "SQ_ACTIVE_INST_VALU")
    mfma, _ = avg(rows, "SQ_INSTS_MFMA")
    valu, _ = avg(rows, "SQ_INSTS_VALU")
    lds, _ = avg(rows, "SQ_INSTS_LDS")
    waits, _ = avg(rows, "SQ_WAIT_INST_ANY")
    wcyc, _ = avg(rows, "SQ_WAVE_CYCLES")
    gui, _ = avg(grbm, "GRBM_GUI_ACTIVE")
    pf = rec["prefill"]
    base = ("python -u bench.py --workload %s --steps 2 --warmup 1 --cold-iters 0 --no-cpu-baseline "
            "--no-extra-configs" % wl)
    md = [f"# Matrix-core utilisation of `prefill_mfma_kernel`: {wl}", "",
          "Two counter passes of the same command (one per counter block):", "", "```",
          f"timeout -s KILL 180 rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES SQ_INSTS_MFMA SQ_INSTS_VALU "
          f"SQ_INSTS_LDS SQ_ACTIVE_INST_VALU SQ_WAVE_CYCLES SQ_WAIT_INST_ANY --output-format csv "
          f"-d {args.prefill_pmc_dir} -o pf -- {base}",
          f"timeout -s KILL 180 rocprofv3 --pmc GRBM_GUI_ACTIVE --output-format csv -d {args.prefill_grbm_dir} "
          f"-o pfg -- {base}", "```", "",
          f"Per dispatch (mean of {n}):", "",
          f"- GRBM_GUI_ACTIVE {gui:.4g} (summed over the 8 XCDs: {gui / 8:.4g} cycles of the GPU clock)",
          f"- SQ_BUSY_CU_CYCLES {cu:.4g} (summed over CUs); SQ_VALU_MFMA_BUSY_CYCLES {busy:.4g} (summed over SIMDs)",
          f"- matrix pipe busy = MFMA_BUSY / (4 x BUSY_CU) = {busy / (4 * cu):.3f} of the time each SIMD is active",
          f"- instructions: MFMA {mfma:.4g}, VALU {valu:.4g} (MFMAs included; {(valu - mfma) / mfma:.2f} others "
          f"per MFMA), LDS {lds:.4g}",
          f"- per SIMD (1024 of them): VALU {vact * 4 / 1024:.4g} cycles (SQ_ACTIVE_INST_VALU counts 4-cycle units: "
          f"x4 matches the VALU count at 4 cycles each, 16 for an exponential), matrix {busy / 1024:.4g} cycles, "
          f"busy {cu / 256:.4g} cycles; VALU hidden under matrix work = "
          f"{max(0.0, (vact * 4 + busy) / 1024 - cu / 256):.4g} cycles",
          f"- SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES = {waits / wcyc:.3f} (waves stalled on a dependency)", "",
          "Same workload, bench.py without the profiler:", "",
          f"- {pf['ms']} ms for {pf['algorithmic_tflop']} TFLOP (4 D flops per attended (query, head, key)) = "
          f"{pf['tflops']} TFLOP/s = {pf['frac_of_dense_mfma_peak']:.3f} of the 2.5 PFLOP/s dense bf16 peak",
          "- per 64-key stage a wave issues 68 products for 64 algorithmic ones (32 QK, 32 PV, 4 row sums): "
          "the matrix pipe executes 1.06x the algorithmic flops", ""]
    with open(os.path.join(ROOT, "profiles", f"prefill_{wl}_mfma.md"), "w") as f:
        f.write("\n".join(md))
    print("\n".join(md))


def summarize(args) -> None:
    """Turn rocprofv3 output (the kernel trace and the FETCH_SIZE / WRITE_SIZE
    passes of the commands below) into the summaries kept under profiles/."""
    wl = args.workload
    with open(args.bench_json) as f:
        rec = json.load(f)
    if args.prefill_pmc_dir:
        summarize_prefill(args, rec)
    if args.trace_dir is None:
        return
    alg = rec["roofline"]["algorithmic_bytes_per_launch"]
    kname = rec["roofline"]["kernel"]
    prof = os.path.join(ROOT, "profiles")
    base = "python -u bench.py --workload %s" % wl
    serving = "kernels_ms" not in rec  # the serving rows run their own step count and warm-up
    # the bench's own step count, so the trace's mean decode launch is the launch bench.py times
    run_args = "" if serving else " --cold-iters 3 --no-extra-configs"
    trace_cmd = (f"rocprofv3 --kernel-trace --stats --output-format csv -d {args.trace_dir} -o trace -- "
                 f"{base}{run_args} --no-cpu-baseline")
    pmc_cmd = (f"timeout -s KILL 120 rocprofv3 --pmc {{counter}} --output-format csv -d {{out_dir}} "
               f"-o {{tag}} -- {base} --steps 3 --warmup 1 --cold-iters 0 --no-cpu-baseline --no-extra-configs "
               f"--copy-probe-mib 1024")
    lines = [f"# Kernel trace: {wl}", "", f"{rec['config']['workload']}", "",
             "Command (from the repository root, one MI355X):", "", "```", trace_cmd, "```", "",
             "| kernel | calls | avg us | min us | max us | % time |", "|---|---|---|---|---|---|"]
    for r in _csv_rows(args.trace_dir, "kernel_stats.csv"):
        lines.append(f"| `{r['Name'][:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} |")
    lines += ["", "Same workload, bench.py without the profiler (HIP events on the launch stream):", ""]
    if serving:
        lines += [f"- decode kernel over the timed steps: {rec['roofline']['achieved']:.0f} GB/s = "
                  f"{rec['roofline']['frac']:.3f} of 8 TB/s ({rec['roofline'].get('bytes_note', 'logical bytes')})",
                  f"- {rec['value']} steps/s, {rec['ms_per_step']} ms per step, {rec['mean_running_rows']} rows "
                  f"running on average; swap: {rec['swap']}", ""]
    else:
        lines += [f"- decode kernel: {rec['kernels_ms']['decode_partitions'] * 1e3:.1f} us per launch, "
                  f"{rec['roofline']['achieved']:.0f} GB/s = {rec['roofline']['frac']:.3f} of 8 TB/s",
                  f"- kernels_ms: {rec['kernels_ms']}", f"- whole step: {rec['value']} GB/s, {rec['ms_per_step']} ms",
                  ""]
    with open(os.path.join(prof, f"decode_{wl}_kernel_trace.md"), "w") as f:
        f.write("\n".join(lines))
    if args.fetch_dir is None:
        return

    if args.counter_log:
        # the counter runs' own algorithmic bytes (their JSON line): a few short steps, not the bench's mean
        with open(args.counter_log) as f:
            alg = json.loads([l for l in f if l.startswith("{")][-1])["roofline"]["algorithmic_bytes_per_launch"]
    fetch = _csv_rows(args.fetch_dir, "counter_collection.csv")
    write = _csv_rows(args.write_dir, "counter_collection.csv")
    f_dec, n_dec = _per_dispatch(fetch, kname)
    w_dec, _ = _per_dispatch(write, kname)
    f_cp = _largest_dispatch(fetch, COPY_KERNEL)
    w_cp = _largest_dispatch(write, COPY_KERNEL)
    probe_kib = 1024 * 1024
    fs, ws = probe_kib / f_cp, probe_kib / w_cp  # each counter against a copy of known size
    hbm_f, hbm_w = f_dec * 1024 * fs, w_dec * 1024 * ws
    out = {"workload": wl, "kernel": kname, "kernel_source_sha": kernel_source_hash(),
           "fetch_kib_per_dispatch_raw": f_dec, "write_kib_per_dispatch_raw": w_dec, "dispatches": n_dec,
           "copy_probe_kib": probe_kib, "copy_fetch_kib_raw": f_cp, "copy_write_kib_raw": w_cp,
           "fetch_scale": fs, "write_scale": ws, "hbm_fetch_bytes_per_launch": hbm_f,
           "hbm_write_bytes_per_launch": hbm_w, "hbm_bytes_per_launch": hbm_f + hbm_w,
           "algorithmic_bytes_per_launch": alg,
           "commands": [pmc_cmd.format(counter="FETCH_SIZE", out_dir=args.fetch_dir, tag="fetch"),
                        pmc_cmd.format(counter="WRITE_SIZE", out_dir=args.write_dir, tag="write")]}
    with open(os.path.join(prof, f"decode_partitions_{wl}_traffic.json"), "w") as f:
        json.dump(out, f, indent=1)
    md = [f"# HBM traffic of `{kname}`: {wl}", "",
          "Two counter passes (one counter each), same command otherwise:", "", "```"] + out["commands"] + [
          "```", "",
          f"- FETCH_SIZE per dispatch (raw): {f_dec:.1f} KiB over {n_dec} dispatches",
          f"- WRITE_SIZE per dispatch (raw): {w_dec:.1f} KiB",
          f"- calibration: a plain 1 GiB device copy (`{COPY_KERNEL}`) reads FETCH_SIZE {f_cp:.1f} KiB and "
          f"WRITE_SIZE {w_cp:.1f} KiB for {probe_kib} KiB moved each way: scale x{fs:.4f} (fetch), x{ws:.4f} (write)",
          f"- HBM bytes per launch (scaled): fetch {hbm_f / 1e9:.4f} GB + write {hbm_w / 1e9:.4f} GB = "
          f"{(hbm_f + hbm_w) / 1e9:.4f} GB",
          f"- algorithmic bytes per launch of the counter runs (bench formula): {alg / 1e9:.4f} GB -> traffic / algorithmic = "
          f"{(hbm_f + hbm_w) / alg:.3f}",
          f"- kernel source sha256[:16]: {out['kernel_source_sha']} (bench.py reports `traffic` only while this "
          "matches)", ""]
    with open(os.path.join(prof, f"decode_{wl}_hbm_traffic.md"), "w") as f:
        f.write("\n".join(md))
    print("\n".join(md))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (decode: up to 200, fewer when the pool cannot hold that many appends; "
                         "serving: 200)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps first (5; 150 for serving_bf16, which fills its batch meanwhile)")
    ap.add_argument("--workload", default=HEADLINE,
                    choices=["tiny_f32", "mha7b_f16", "gqa8b_bf16", "shared_prefix_bf16", "longctx_bf16",
                             "specdec_bf16", "serving_bf16", "serving_prefix_bf16", "mha7b_f16_bs32",
                             "mha7b_f16_bs64", "gqa8b_bf16_bs32"])
    ap.add_argument("--partition", type=int, default=None,
                    help="tokens per context partition (0 = the library's choice; default: the workload's stated "
                         "partition, 512 for longctx_bf16, else the library's choice)")
    ap.add_argument("--no-extra-configs", action="store_true",
                    help="skip the other decode configurations the headline line reports")
    ap.add_argument("--append-meta", choices=["pinned", "args"], default="pinned",
                    help="where the step's slots, positions and lengths reach the cache write: pinned host memory "
                         "read by the kernel, or the kernel arguments (pa_append_step_host)")
    ap.add_argument("--cold-iters", type=int, default=20, help="decode launches timed after a 1 GiB cache flush")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (scales HBM byte counters)")
    ap.add_argument("--summarize", action="store_true",
                    help="write profiles/ summaries from rocprofv3 output (--trace-dir, --fetch-dir, --write-dir) "
                         "and a bench.py JSON line of the same workload (--bench-json); no GPU work")
    ap.add_argument("--trace-dir")
    ap.add_argument("--fetch-dir")
    ap.add_argument("--write-dir")
    ap.add_argument("--counter-log", help="output of the FETCH_SIZE counter run (its JSON line gives the "
                                          "algorithmic bytes per launch of that run)")
    ap.add_argument("--bench-json")
    ap.add_argument("--prefill-pmc-dir")
    ap.add_argument("--prefill-grbm-dir")
    args = ap.parse_args()
    serving = args.workload in ("serving_bf16", "serving_prefix_bf16")
    if serving:
        args.steps = 200 if args.steps is None else args.steps
        args.warmup = 150 if args.warmup is None else args.warmup
    if args.summarize:
        summarize(args)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        sys.stderr.write("bench.py measures one GPU only: the paged decode path runs on one GPU's share "
                         "of the work and several GPUs are not supported (run with --gpus 1).\n")
        sys.exit(2)

    if args.workload in ("serving_bf16", "serving_prefix_bf16"):
        bench_serving(args)
        return

    import torch

    from workloads import make_workload

    torch.cuda.set_device(0)
    w = make_workload(args.workload)
    partition = w.partition_size if args.partition is None else args.partition
    rec = bench_decode(w, partition, args, full=True)
    if args.workload == HEADLINE and not args.no_extra_configs:
        # the other gated decode configurations (and the headline's at the
        # library's default partition), kernel figures only, same step
        del w
        torch.cuda.empty_cache()
        extra = {}
        for name in EXTRA_CONFIGS:
            wx = make_workload(name)
            px = wx.partition_size if name != HEADLINE else 0
            r = bench_decode(wx, px, argparse.Namespace(**dict(vars(args), steps=None, warmup=None)), full=False)
            extra[name if name != HEADLINE else f"{name}_default_partition"] = r
            del wx
            torch.cuda.empty_cache()
        rec["other_configs"] = extra
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(make_workload(args.workload))
    print(json.dumps(rec), flush=True)


def bench_decode(w, partition: int, args, full: bool = True) -> dict:
    """Time the decode step of workload ``w`` at ``partition`` tokens per
    context partition (0: the library's choice).  With ``full`` the record
    is the benchmark line (ceilings, cold-cache decode, prefill); otherwise
    the kernel figures only."""
    import torch

    from paged_kv_cache_395_amd import BlockManager, ops
    from workloads import run_program

    dev = torch.device("cuda", 0)
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[w.dtype]

    def to_dev(a):
        a = np.ascontiguousarray(a)
        if w.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    S, Hq, Hkv, D = w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim
    multi = w.lengths.get("mode") == "multi"  # each step appends and verifies w.append drafted tokens per sequence
    # tokens every sequence appends in a timed step: the verification workload
    # its w.append drafted tokens, the others one.  The long-context workload
    # first writes its w.append-token chunk (untimed); its steps then decode
    # one new token per sequence like the rest.
    per_step = w.append if multi else 1
    chunk = w.append > 1 and not multi
    bm = BlockManager(w.num_blocks, block_size=w.block_size, free_order=w.free_order)
    run_program(bm, w.program)
    k_pool, v_pool = to_dev(w.k_pool), to_dev(w.v_pool)
    if chunk:
        slots0, cow0 = bm.append_tokens(np.ascontiguousarray(w.step_seqs, dtype=np.int64))
        if len(cow0):
            raise RuntimeError("copy-on-write is not expected in this workload")
        ops.reshape_and_cache(to_dev(w.step_rows("k")), to_dev(w.step_rows("v")), k_pool, v_pool,
                              torch.from_numpy(slots0).to(dev))
        torch.cuda.synchronize()
    steps, warmup = args.steps, args.warmup
    if steps is None or warmup is None:
        # the longest run (about 40-80 ms timed, so a host stall of a few ms
        # does not decide the figure) whose appends the pool can hold
        for k in (200, 100, 50, 20):
            if appends_fit(bm, w, (k + k // 10 + 2) * per_step):
                break
        steps = k if steps is None else steps
        warmup = max(5, k // 10) if warmup is None else warmup
    extra = (warmup + steps + 2) * per_step
    maxB = w.max_blocks_per_seq(extra)
    pad = w.num_blocks + 1  # never read

    if multi:
        step_k, step_v = to_dev(w.step_rows("k")), to_dev(w.step_rows("v"))
    else:  # one row per sequence: each sequence's last drawn row
        step_k = to_dev(np.ascontiguousarray(w.step_k[:, -1]))
        step_v = to_dev(np.ascontiguousarray(w.step_v[:, -1]))
    q = to_dev(w.q) if multi else to_dev(w.decode_q)
    out = torch.empty(tuple(q.shape), dtype=tdt, device=dev)

    # block tables and context lengths live on the device: copied once here,
    # then patched in place by each step's cache write from the step's slots
    n_tok = S * per_step
    table0, ctx0 = bm.block_table(np.ascontiguousarray(w.batch, dtype=np.int64), maxB, pad=pad)
    d_table = torch.from_numpy(table0).to(dev)
    d_ctx = torch.from_numpy(ctx0).to(dev)
    host_ctx = ctx0.astype(np.int64)  # the host's copy of the lengths (the block manager's counts)
    first_ctx = int(host_ctx.max())
    final_ctx = first_ctx + extra
    ws_need = max(ops.StepPlan.workspace_bytes_for(S, per_step, Hq, Hkv, D, c, partition)
                  for c in range(first_ctx, final_ctx + 1))
    ws = torch.empty(max(1, ws_need), dtype=torch.uint8, device=dev)
    seqs = np.repeat(np.ascontiguousarray(w.batch, dtype=np.int64), per_step)
    stream = torch.cuda.current_stream()
    # a step ships only its tokens' slots and positions and the new lengths:
    # either the write kernel reads them straight from pinned host memory (a
    # ring of buffers the host refills once the write that read them has run),
    # or they travel in the kernel arguments, copied at launch
    host_args = args.append_meta == "args"
    rows_np = np.repeat(np.arange(S, dtype=np.int32), per_step)
    rows = torch.from_numpy(rows_np) if host_args else torch.from_numpy(rows_np).to(dev)
    offs = np.tile(np.arange(per_step, dtype=np.int64), S)
    ring = [{"slots": torch.empty(n_tok, dtype=torch.int64, pin_memory=not host_args),
             "pos": torch.empty(n_tok, dtype=torch.int32, pin_memory=not host_args),
             "nctx": torch.empty(S, dtype=torch.int32, pin_memory=not host_args)}
            for _ in range(1 if host_args else 16)]
    plans = [ops.StepPlan(out, q, k_pool, v_pool, d_table, d_ctx, w.scale, ws, key=step_k, value=step_v,
                          slot_mapping=r["slots"], partition_size=partition,
                          append=(rows, r["pos"], r["nctx"]), host_args=host_args) for r in ring]
    # one event per group of RING_GROUP slots, recorded after the group's last
    # write: an event record carries a system-scope fence that costs the step
    # queue time, so one per step would be the step's largest overhead
    n_groups = max(1, len(ring) // RING_GROUP)
    ring_done = [torch.cuda.Event() for _ in range(n_groups)]
    ring_used = [False] * n_groups

    def ring_group(r):
        return r * n_groups // len(ring)

    def prepare_step(i, append):
        """Host part of a step: block manager -> this step's pinned metadata."""
        r = i % len(ring)
        if append:
            grp = ring_group(r)
            if ring_used[grp] and r * n_groups % len(ring) == 0:
                # first slot of a group: every write that last read the group has run
                ring_done[grp].synchronize()
            _, cow = bm.append_tokens(seqs, slots_out=ring[r]["slots"].numpy())
            if len(cow):
                raise RuntimeError("copy-on-write is not expected in this workload")
            np.add(np.repeat(host_ctx, per_step), offs, out=ring[r]["pos"].numpy(), casting="unsafe")
            host_ctx[:] += per_step
            ring[r]["nctx"].numpy()[:] = host_ctx
        return plans[r], host_ctx.copy()

    def issue_write(i, plan):
        plan.cache_write()
        if not host_args:  # copied into the launch otherwise: the host may refill at once
            r = i % len(ring)
            if ring_group(r + 1) != ring_group(r) or r + 1 == len(ring):  # the group's last slot
                grp = ring_group(r)
                ring_done[grp].record(stream)
                ring_used[grp] = True

    # decode is bracketed by events in every EVENT_EVERY-th timed step: the
    # partition kernel alone (the roofline's kernel) and with the merge.  An
    # event record costs the step ~2 us of queue time, so sampling keeps the
    # whole-step figure close to the event-free step while the roofline's
    # launch durations are still measured live in the timed region.
    ev_dec = [(TimingEvent(), TimingEvent(), TimingEvent()) for _ in range(0, steps, EVENT_EVERY)]
    ev_bytes = []

    def step(i, timed_idx=None):
        plan, ctx_np = prepare_step(i, True)
        mx = int(ctx_np.max())
        issue_write(i, plan)
        ev = ev_dec[timed_idx // EVENT_EVERY] if timed_idx is not None and timed_idx % EVENT_EVERY == 0 else None
        if ev is not None:
            ev[0].record(stream)
            ev_bytes.append(decode_bytes(ctx_np, w))
        plan.decode_partitions(mx)
        if ev is not None:
            ev[1].record(stream)
        plan.decode_reduce(mx)
        if ev is not None:
            ev[2].record(stream)
        return decode_bytes(ctx_np, w)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    total_bytes = 0.0
    host_s = 0.0  # time the host spends issuing a step (the GPU runs behind it)
    t0 = time.perf_counter()
    for i in range(steps):
        h0 = time.perf_counter()
        total_bytes += step(warmup + i, i)
        host_s += time.perf_counter() - h0
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0

    # the small kernels and the whole kernel span of a step, outside the timed region
    side = []
    # the device tables must equal the block manager's after every timed step
    t_host, c_host = bm.block_table(np.ascontiguousarray(w.batch, dtype=np.int64), maxB, pad=pad)
    if not (np.array_equal(d_table.cpu().numpy(), t_host) and np.array_equal(d_ctx.cpu().numpy(), c_host)):
        raise RuntimeError("device block tables diverged from the block manager")
    # re-issuing the last step's write is idempotent (same slots, rows and lengths)
    plan, ctx_side = prepare_step(warmup + steps - 1, False)
    mx_side = int(ctx_side.max())
    for _ in range(10):
        e = [TimingEvent() for _ in range(4)]
        e[0].record(stream)
        plan.cache_write()
        e[1].record(stream)
        plan.decode_partitions(mx_side)
        e[2].record(stream)
        plan.decode_reduce(mx_side)
        e[3].record(stream)
        side.append(e)
    torch.cuda.synchronize()

    k2_ms = np.array([a.elapsed_time(b) for a, b, _ in ev_dec])
    k23_ms = np.array([a.elapsed_time(c) for a, _, c in ev_dec])
    k1_ms = np.array([a[0].elapsed_time(a[1]) for a in side])
    k3_ms = np.array([a[2].elapsed_time(a[3]) for a in side])
    kd_side = np.array([a[1].elapsed_time(a[2]) for a in side])  # decode on the last timed step's tables
    span_ms = np.array([a[0].elapsed_time(a[3]) for a in side])  # first kernel start to last kernel end
    bytes_per_launch = total_bytes / steps
    ev_bytes_mean = float(np.mean(ev_bytes))  # the timed launches' own contexts
    achieved = ev_bytes_mean / (k2_ms.mean() * 1e-3) / 1e9
    # pa_decode_multi makes both launches in one call, so its partition-launch
    # events already cover the merge and the merge's own interval is empty
    achieved23 = achieved if multi else ev_bytes_mean / (k23_ms.mean() * 1e-3) / 1e9
    reduce_ms = None if multi else round(float(k3_ms.mean()), 5)
    value = total_bytes / elapsed / 1e9
    used_partition = ops.decode_partition_size(S, Hkv, int(host_ctx.max()), partition)
    # the launch is over sequences; a sequence's queries share its workgroups
    kernel, nwg = ops.decode_launch_shape(q.dtype, D, out.dtype, S, Hq, Hkv, int(host_ctx.max()), partition)
    grid = {"kernel": kernel, "workgroups": nwg}
    if not full:
        return {"workload": f"{w.name}: {w.description}", "partition": used_partition, "decode_grid": grid,
                "mean_context": round(float(host_ctx.mean()), 1), "steps": steps,
                "decode_partitions_us": round(float(k2_ms.mean()) * 1e3, 2),
                "decode_reduce_us": None if multi else round(float(k3_ms.mean()) * 1e3, 2),
                "frac_decode_kernel": round(achieved / HBM_PEAK_GBS, 4),
                "frac_decode_with_merge": round(achieved23 / HBM_PEAK_GBS, 4),
                "whole_step_gbs": round(value, 2), "hbm_frac_whole_step": round(value / HBM_PEAK_GBS, 4),
                "ms_per_step": round(elapsed / steps * 1e3, 4),
                "algorithmic_bytes_per_launch": round(ev_bytes_mean, 1)}

    # cold-cache decode: each launch after a 1 GiB write evicts L2 and the 256 MiB MALL
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    cold = []
    ctx_now = host_ctx.copy()
    mx = int(ctx_now.max())
    for _ in range(args.cold_iters):
        scratch.zero_()
        a, b = TimingEvent(), TimingEvent()
        a.record(stream)
        plan.decode_partitions(mx)
        b.record(stream)
        cold.append((a, b))
    torch.cuda.synchronize()
    cold_ms = np.array([a.elapsed_time(b) for a, b in cold])
    cold_gbs = decode_bytes(ctx_now, w) / (np.median(cold_ms) * 1e-3) / 1e9 if len(cold_ms) else None
    # HBM read ceiling: one streaming read of a 4 GiB buffer with decode's load style
    big = torch.empty(1 << 32, dtype=torch.uint8, device=dev)
    big.fill_(1)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    ops.probe_read_bandwidth(big, sink)
    probe = []
    for _ in range(5):
        a, b = TimingEvent(), TimingEvent()
        a.record(stream)
        ops.probe_read_bandwidth(big, sink)
        b.record(stream)
        probe.append((a, b))
    torch.cuda.synchronize()
    read_gbs = big.numel() / (np.median([a.elapsed_time(b) for a, b in probe]) * 1e-3) / 1e9
    # gather ceiling: the same buffer read as decode tiles (16 tokens of one kv head) in a random order
    tile_bytes = 16 * w.head_dim * ESIZE[w.dtype]
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    order = torch.randperm(big.numel() // tile_bytes, generator=gen, device=dev, dtype=torch.int32)
    ops.probe_gather_bandwidth(big, order, tile_bytes, sink)
    probe = []
    for _ in range(5):
        a, b = TimingEvent(), TimingEvent()
        a.record(stream)
        ops.probe_gather_bandwidth(big, order, tile_bytes, sink)
        b.record(stream)
        probe.append((a, b))
    torch.cuda.synchronize()
    gather_gbs = order.numel() * tile_bytes / (np.median([a.elapsed_time(b) for a, b in probe]) * 1e-3) / 1e9
    del big, scratch, order

    extra_fields = {}
    if args.copy_probe_mib:
        src = torch.ones(args.copy_probe_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        extra_fields["copy_probe_bytes"] = {"read": src.numel(), "write": dst.numel()}
        del src, dst
    if chunk:
        # the chunk workload also times its chunked prefill (matrix-core
        # bound): the w.append-token chunk at the end of each context as it
        # stands after the timed steps
        qc = to_dev(w.q)
        oc = torch.empty(qc.shape, dtype=tdt, device=dev)
        ops.prefill_chunk(oc, qc, k_pool, v_pool, d_table, d_ctx, w.scale, int(ctx_now.max()))
        pe = []
        for _ in range(3):
            a, b = TimingEvent(), TimingEvent()
            a.record(stream)
            ops.prefill_chunk(oc, qc, k_pool, v_pool, d_table, d_ctx, w.scale, int(ctx_now.max()))
            b.record(stream)
            pe.append((a, b))
        torch.cuda.synchronize()
        p_ms = float(np.median([a.elapsed_time(b) for a, b in pe]))
        fl = prefill_flops(ctx_now, w.append, w)
        extra_fields["prefill"] = {"ms": round(p_ms, 3), "tflops": round(fl / (p_ms * 1e-3) / 1e12, 2),
                                   "frac_of_dense_mfma_peak": round(fl / (p_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                                   "algorithmic_tflop": round(fl / 1e12, 4)}

    traffic, traffic_ratio = load_traffic(w.name, ev_bytes_mean)
    phys_bytes = physical_kv_bytes(t_host, c_host, w)
    value = total_bytes / elapsed / 1e9
    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(elapsed / steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.description}", "append_meta": args.append_meta, "num_seqs": S,
                   "num_q_heads": Hq,
                   "num_kv_heads": Hkv, "head_dim": D, "block_size": w.block_size,
                   "mean_context": round(float(ctx_now.mean()), 1),
                   "partition": used_partition, "decode_grid": grid},
        "hbm_frac_whole_step": round(value / HBM_PEAK_GBS, 4),
        # shared prefix blocks are read by many rows but come from HBM about once (the rest hit in cache)
        "kv_physical": {"bytes_per_launch": round(phys_bytes, 1),
                        "gbs": round(phys_bytes / (float(kd_side.mean()) * 1e-3) / 1e9, 2),
                        "note": "K/V of the distinct blocks the last timed step reads, each block's valid "
                                "tokens once, over the time of decode launches on that same state"},
        "seqs_per_s": round(S * steps / elapsed, 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else round(traffic, 1),
                     "traffic_over_algorithmic": None if traffic_ratio is None else round(traffic_ratio, 4),
                     "kernel": kernel,
                     "algorithmic_bytes_per_launch": round(ev_bytes_mean, 1),
                     "timed_launches": len(ev_dec),
                     **({"timed_call": "pa_decode_multi: the partition kernel and the merge in one call (a kernel "
                                       "trace gives the two apart)"} if multi else {}),
                     # the same bytes over the partition kernel plus the log-sum-exp merge launch
                     "achieved_with_merge": round(achieved23, 2),
                     "frac_with_merge": round(achieved23 / HBM_PEAK_GBS, 4)},
        "kernels_ms": {"append_step": round(float(k1_ms.mean()), 5),
                       "decode_partitions": round(float(k2_ms.mean()), 5),
                       "decode_reduce": reduce_ms,
                       "step_kernels_span": round(float(span_ms.mean()), 5)},
        "host_ms_per_step": round(host_s / steps * 1e3, 4),
        "decode_partitions_cold": None if cold_gbs is None else {
            "median_ms": round(float(np.median(cold_ms)), 5), "p10_ms": round(float(np.percentile(cold_ms, 10)), 5),
            "p90_ms": round(float(np.percentile(cold_ms, 90)), 5), "gbs": round(cold_gbs, 2)},
        "hbm_read_ceiling_gbs": round(read_gbs, 1),
        "hbm_gather_ceiling_gbs": round(gather_gbs, 1),
        **extra_fields,
    }
    return rec




if __name__ == "__main__":
    main()
