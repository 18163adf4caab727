#!/usr/bin/env python3
"""Paged-decode benchmark on one MI355X.

A step is one pass of the whole hot path over one batch: the native block
manager appends one token to every sequence (slots, block tables), one
pinned host->device copy ships slots / lengths / tables, the cache write
stores the new K/V rows, and paged decode (partition kernel + log-sum-exp
merge) attends over every context.  Contexts grow by one token per step.
Inputs are seeded synthetic values of the workload's shape, resident in HBM
before timing starts.

Prints one JSON line: whole-step KV throughput (GB/s), the roofline of the
dominant kernel (decode partitions, timed with HIP events on the launch
stream), and the CPU oracle timed on a bounded sample of the same workload.
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
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16/fp16 matrix, published
ESIZE = {"f32": 4, "f16": 2, "bf16": 2}
KERNEL_SOURCES = ["paged_kv_cache_395_amd/csrc/decode_kernels.hip", "paged_kv_cache_395_amd/csrc/device_common.h"]


def decode_bytes(ctx: np.ndarray, w) -> float:
    """Algorithmic bytes of one decode: K+V rows of every context token, q, out, table entries read."""
    e = ESIZE[w.dtype]
    kv = float(np.sum(ctx, dtype=np.int64)) * w.num_kv_heads * w.head_dim * 2 * e
    qo = 2.0 * len(ctx) * w.num_q_heads * w.head_dim * e
    tab = float(np.sum((ctx + 15) // 16, dtype=np.int64)) * 4
    return kv + qo + tab


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
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"decode_partitions_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(w, budget_s: float = 15.0):
    """The oracle, as it stands, on the first sequences of the same step until
    ~budget_s of work; BLAS limited to one thread (the oracle is a Python loop)."""
    from threadpoolctl import threadpool_limits

    from oracle import attention as OA
    from oracle.block_manager import RefBlockManager
    from workloads import run_program

    ref = RefBlockManager(w.num_blocks, free_order=w.free_order)
    run_program(ref, w.program)
    slots, _ = ref.append_tokens(list(w.step_seqs))
    table, ctx = ref.block_table(list(w.batch), w.max_blocks_per_seq(), pad=0)
    table, ctx = np.array(table, np.int32), np.array(ctx, np.int32)
    k, v = w.k_pool, w.v_pool  # written in place; the benchmark has its own device copies
    done = []
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        OA.reshape_and_cache(k, v, w.step_rows("k"), w.step_rows("v"), np.array(slots))
        for s in range(w.num_seqs):
            OA.decode(w.decode_q, k, v, table, ctx, w.scale, w.dtype, seqs=[s])
            done.append(s)
            if time.perf_counter() - t0 > budget_s:
                break
        dt = time.perf_counter() - t0
    sub = ctx[done]
    gbs = decode_bytes(sub, w) / dt / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"one decode step (cache write of {w.num_seqs} tokens + fp64 attention) for the first "
                      f"{len(done)} of {w.num_seqs} sequences, all {w.num_q_heads} q heads; "
                      f"{dt:.1f} s; seqs/s {len(done) / dt:.2f}; numpy, BLAS 1 thread"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mha7b_f16",
                    choices=["tiny_f32", "mha7b_f16", "gqa8b_bf16", "shared_prefix_bf16", "longctx_bf16"])
    ap.add_argument("--partition", type=int, default=0, help="tokens per context partition (0 = the library's choice)")
    ap.add_argument("--cold-iters", type=int, default=20, help="decode launches timed after a 1 GiB cache flush")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (scales HBM byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        sys.stderr.write("bench.py measures one GPU only: every box here has one MI355X, and the paged "
                         "decode path is built and measured on a single GPU (run with --gpus 1).\n")
        sys.exit(2)

    import torch

    from paged_kv_cache_395_amd import BlockManager, ops
    from workloads import make_workload, run_program

    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    w = make_workload(args.workload)
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[w.dtype]

    def to_dev(a):
        a = np.ascontiguousarray(a)
        if w.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    S, Hq, Hkv, D = w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim
    grows = w.append == 1  # decode workloads append one token per step; the chunk workload decodes in place
    extra = (args.warmup + args.steps + 1) if grows else 0
    maxB = w.max_blocks_per_seq(extra)
    pad = w.num_blocks + 1  # never read
    bm = BlockManager(w.num_blocks, free_order=w.free_order)
    run_program(bm, w.program)

    k_pool, v_pool = to_dev(w.k_pool), to_dev(w.v_pool)
    step_k, step_v = to_dev(w.step_rows("k")), to_dev(w.step_rows("v"))
    q = to_dev(w.decode_q)
    out = torch.empty((S, Hq, D), dtype=tdt, device=dev)

    # per-step host -> device staging: slots (int64 [n]) | ctx (int32 [S]) | table (int32 [S, maxB])
    n_tok = S * w.append
    nbytes = 8 * n_tok + 4 * S + 4 * S * maxB
    ring = [torch.empty(nbytes, dtype=torch.uint8, pin_memory=True) for _ in range(4)]
    ring_ev = [None] * len(ring)
    dbuf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    d_slots = dbuf[: 8 * n_tok].view(torch.int64)
    d_ctx = dbuf[8 * n_tok: 8 * n_tok + 4 * S].view(torch.int32)
    d_table = dbuf[8 * n_tok + 4 * S:].view(torch.int32).view(S, maxB)
    final_ctx = int(w.lengths["final_ctx"].max()) + extra
    first_ctx = int(w.lengths["final_ctx"].max())
    ws_need = max(ops.decode_workspace_bytes(S, Hq, Hkv, D, c, args.partition) for c in range(first_ctx, final_ctx + 1))
    ws = torch.empty(max(1, ws_need), dtype=torch.uint8, device=dev)
    seqs = np.ascontiguousarray(w.step_seqs, dtype=np.int64)
    batch = np.ascontiguousarray(w.batch, dtype=np.int64)
    stream = torch.cuda.current_stream()

    def views(buf):
        a = buf.numpy()
        return (a[: 8 * n_tok].view(np.int64), a[8 * n_tok: 8 * n_tok + 4 * S].view(np.int32),
                a[8 * n_tok + 4 * S:].view(np.int32).reshape(S, maxB))

    def prepare_step(i, append):
        r = i % len(ring)
        if ring_ev[r] is not None:
            ring_ev[r].synchronize()
        slots_np, ctx_np, table_np = views(ring[r])
        if append:
            _, cow = bm.append_tokens(seqs, slots_out=slots_np)
            if len(cow):
                raise RuntimeError("copy-on-write is not expected in this workload")
        bm.block_table(batch, maxB, pad=pad, table_out=table_np, ctx_out=ctx_np)
        dbuf.copy_(ring[r], non_blocking=True)
        ev = torch.cuda.Event()
        ev.record(stream)
        ring_ev[r] = ev
        return ctx_np.copy()

    if not grows:
        # the chunk workload: write the chunk once (untimed); every step then decodes in place
        prepare_step(0, True)
        ops.reshape_and_cache(step_k, step_v, k_pool, v_pool, d_slots)
        torch.cuda.synchronize()

    ev_pairs = []

    def step(i, timed):
        ctx_np = prepare_step(i, grows)
        mx = int(ctx_np.max())
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)] if timed else None
        if timed:
            e[0].record(stream)
        if grows:
            ops.reshape_and_cache(step_k, step_v, k_pool, v_pool, d_slots)
        if timed:
            e[1].record(stream)
        ops.decode_partitions(out, q, k_pool, v_pool, d_table, d_ctx, w.scale, mx, args.partition, ws)
        if timed:
            e[2].record(stream)
        ops.decode_reduce(out, d_ctx, Hkv, mx, args.partition, ws)
        if timed:
            e[3].record(stream)
            ev_pairs.append(e)
        return decode_bytes(ctx_np, w)

    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    total_bytes = 0.0
    t0 = time.perf_counter()
    for i in range(args.steps):
        total_bytes += step(args.warmup + i, True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0

    k1_ms = np.array([a[0].elapsed_time(a[1]) for a in ev_pairs])
    k2_ms = np.array([a[1].elapsed_time(a[2]) for a in ev_pairs])
    k3_ms = np.array([a[2].elapsed_time(a[3]) for a in ev_pairs])
    bytes_per_launch = total_bytes / args.steps
    achieved = bytes_per_launch / (k2_ms.mean() * 1e-3) / 1e9

    # cold-cache decode: each launch after a 1 GiB write evicts L2 and the 256 MiB MALL
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    cold = []
    ctx_now = prepare_step(10 ** 6, False)
    mx = int(ctx_now.max())
    for _ in range(args.cold_iters):
        scratch.zero_()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        ops.decode_partitions(out, q, k_pool, v_pool, d_table, d_ctx, w.scale, mx, args.partition, ws)
        b.record(stream)
        cold.append((a, b))
    torch.cuda.synchronize()
    cold_ms = np.array([a.elapsed_time(b) for a, b in cold])
    cold_gbs = decode_bytes(ctx_now, w) / (np.median(cold_ms) * 1e-3) / 1e9 if len(cold_ms) else None

    # plain streaming read of a 4 GiB buffer, for context
    big = torch.ones(1 << 31, dtype=torch.bfloat16, device=dev)
    big.sum()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(5):
        big.sum()
    b.record(stream)
    torch.cuda.synchronize()
    read_gbs = 5 * big.numel() * 2 / (a.elapsed_time(b) * 1e-3) / 1e9
    del big, scratch

    extra_fields = {}
    if args.copy_probe_mib:
        src = torch.ones(args.copy_probe_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        extra_fields["copy_probe_bytes"] = {"read": src.numel(), "write": dst.numel()}
        del src, dst
    if w.append > 1:
        # the chunk workload also times its chunked prefill (matrix-core bound)
        qc = to_dev(w.q)
        oc = torch.empty(qc.shape, dtype=tdt, device=dev)
        ops.prefill_chunk(oc, qc, k_pool, v_pool, d_table, d_ctx, w.scale, int(ctx_now.max()))
        pe = []
        for _ in range(3):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
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

    traffic = load_traffic(args.workload, bytes_per_launch)
    value = total_bytes / elapsed / 1e9
    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.description}", "num_seqs": S, "num_q_heads": Hq,
                   "num_kv_heads": Hkv, "head_dim": D, "block_size": 16,
                   "mean_context": round(float(ctx_now.mean()), 1),
                   "partition": ops.decode_partition_size(S, Hkv, int(ctx_now.max()), args.partition)},
        "hbm_frac_whole_step": round(value / HBM_PEAK_GBS, 4),
        "seqs_per_s": round(S * args.steps / elapsed, 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else round(traffic, 1),
                     "kernel": "decode_mfma_kernel" if w.dtype != "f32" else "decode_f32_kernel",
                     "algorithmic_bytes_per_launch": round(bytes_per_launch, 1)},
        "kernels_ms": {"reshape_and_cache": round(float(k1_ms.mean()), 5),
                       "decode_partitions": round(float(k2_ms.mean()), 5),
                       "decode_reduce": round(float(k3_ms.mean()), 5)},
        "decode_partitions_cold": None if cold_gbs is None else {
            "median_ms": round(float(np.median(cold_ms)), 5), "p10_ms": round(float(np.percentile(cold_ms, 10)), 5),
            "p90_ms": round(float(np.percentile(cold_ms, 90)), 5), "gbs": round(cold_gbs, 2)},
        "hbm_read_ceiling_gbs": round(read_gbs, 1),
        **extra_fields,
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
