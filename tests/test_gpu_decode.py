"""Paged decode on the GPU against the oracle.

Every workload at full size with the launch configuration the benchmark
uses (the library's default partitions), reduced sizes with ragged tails, the
output-dtype path, partition-size agreement, and the closed-form / paging
properties: single-token contexts, dominant keys, zero queries, scores growing
along the context (rescales and far-apart partition maxima), physical
relabelling, determinism, NaN poison in unread memory, zero-length
contexts and out-of-pool table entries.
"""
import functools

import numpy as np
import pytest
import torch

from oracle import attention as OA
from tests._gpu import Prepared, assert_close, out_f64, say, to_dev, to_host
from workloads import make_workload, to_storage

pytestmark = pytest.mark.gpu


@functools.lru_cache(maxsize=2)
def prepared(name, **overrides):
    say(f"[prepare] {name} {overrides}")
    return Prepared(make_workload(name, **overrides))


FULL = ["tiny_f32", "mha7b_f16", "gqa8b_bf16", "shared_prefix_bf16", "longctx_bf16"]
REDUCED = [
    ("mha7b_f16", dict(num_seqs=6, lo=1, hi=1100)),
    ("gqa8b_bf16", dict(num_seqs=12, hi=1500)),
    ("shared_prefix_bf16", dict(num_users=10, num_prompts=3, user_tail=(16, 700))),
    ("longctx_bf16", dict(num_seqs=2, ctx=3000, chunk=1)),
]


@pytest.mark.parametrize("name", FULL)
def test_decode_full_size_matches_oracle(name):
    p = prepared(name)
    say(f"[decode] {name} S={p.w.num_seqs} max_ctx={p.max_ctx}")
    d = p.device()
    p.write_step(d)
    out = p.gpu_decode(d)
    torch.cuda.synchronize()
    ref = p.oracle_decode()
    stats = assert_close(out_f64(out), ref, p.w.dtype, name)
    say(f"[decode] {name} {stats}")


def test_long_context_at_its_stated_partitions_matches_oracle():
    """16 x 32,768 tokens, 64/8 heads, at the 512-token partitions the
    workload states (64 partitions per context, merged by log-sum-exp): the
    launch the benchmark times."""
    p = prepared("longctx_bf16")
    assert p.w.partition_size == 512
    say(f"[decode] longctx_bf16 P=512 max_ctx={p.max_ctx}")
    d = p.device()
    p.write_step(d)
    out = p.gpu_decode(d, partition=p.w.partition_size)
    torch.cuda.synchronize()
    stats = assert_close(out_f64(out), p.oracle_decode(), "bf16", "longctx P=512")
    say(f"[decode] longctx_bf16 P=512 {stats}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_merge_of_more_than_256_slots_per_row(dtype):
    """One sequence of 8,192 tokens and one kv head at 16-token partitions:
    more partial slots per row than the merge weighs in one round (256)."""
    name = "longctx_bf16"
    p = Prepared(make_workload(name, num_seqs=1, ctx=8192, chunk=1, Hq=8, Hkv=1,
                               dtype=dtype, head_dim=128 if dtype == "bf16" else 64))
    d = p.device()
    p.write_step(d)
    out = p.gpu_decode(d, partition=16)
    assert_close(out_f64(out), p.oracle_decode(), dtype, f"{dtype} P=16")


def test_reduce_with_other_sizes_than_the_partition_launch_gives_nan_rows():
    """pa_decode_reduce reads the partials at the stride the partition launch
    used; a call with another partition size or length bound is detected
    from the workspace header and reported as NaN rows."""
    from paged_kv_cache_395_amd import ops
    p = prepared("gqa8b_bf16", num_seqs=12, hi=1500)
    d = p.device()
    p.write_step(d)
    S, Hq, Hkv, D = 12, 32, 8, 128
    ws = torch.empty(ops.decode_workspace_bytes(S, Hq, Hkv, D, p.max_ctx, 64), dtype=torch.uint8, device="cuda")
    out = torch.empty(S, Hq, D, dtype=torch.float32, device="cuda")
    ops.decode_partitions(out, d["q"], d["k"], d["v"], d["table"], d["ctx"], p.w.scale, p.max_ctx, 64, ws)
    ops.decode_reduce(out, d["ctx"], Hkv, p.max_ctx, 64, ws)
    assert_close(out_f64(out), p.oracle_decode(), "bf16", "matched")
    # same workspace, another partition size (a smaller stride): every row NaN
    ops.decode_reduce(out, d["ctx"], Hkv, p.max_ctx, 128, ws)
    assert torch.isnan(out).all()
    # another length bound
    ops.decode_partitions(out, d["q"], d["k"], d["v"], d["table"], d["ctx"], p.w.scale, p.max_ctx, 64, ws)
    ops.decode_reduce(out, d["ctx"], Hkv, p.max_ctx - 16, 64, ws)
    assert torch.isnan(out).all()
    # a workspace no partition launch wrote
    ws.zero_()
    ops.decode_reduce(out, d["ctx"], Hkv, p.max_ctx, 64, ws)
    assert torch.isnan(out).all()


@pytest.mark.parametrize("name,kw", REDUCED, ids=[r[0] for r in REDUCED])
def test_decode_reduced_matches_oracle(name, kw):
    p = prepared(name, **kw)
    d = p.device()
    p.write_step(d)
    out = p.gpu_decode(d)
    assert_close(out_f64(out), p.oracle_decode(), p.w.dtype, name)


@pytest.mark.parametrize("name,kw", REDUCED[:2] + [("tiny_f32", {})], ids=["f16", "bf16", "f32"])
def test_output_in_input_dtype_is_the_rounded_result(name, kw):
    p = prepared(name, **kw)
    d = p.device()
    p.write_step(d)
    out = p.gpu_decode(d, out_f32=False)
    ref = p.oracle_decode()
    dt = p.w.dtype
    got = OA.to_f64(to_host(out, dt), dt)
    want = OA.to_f64(OA.round_f64_to(ref, dt), dt)
    # the stored value is the correct rounding of a value within 1e-5 of the
    # oracle: one unit in the last place for ordinary magnitudes, more only
    # where the 16-bit spacing is finer than fp32 accumulation error (near 0)
    if dt == "f32":
        assert_close(got, ref, dt)
    else:
        g = ordered_bits(to_host(out, dt), dt)
        lo = ordered_bits(OA.round_f64_to(ref - 1e-5, dt), dt)
        hi = ordered_bits(OA.round_f64_to(ref + 1e-5, dt), dt)
        assert np.all((lo <= g) & (g <= hi))
        assert np.mean(g == ordered_bits(OA.round_f64_to(ref, dt), dt)) > 0.9
    if dt == "f16":
        assert_close(got, ref, dt)


def ordered_bits(bits: np.ndarray, dt: str) -> np.ndarray:
    """16-bit float patterns mapped to integers in the order of their values."""
    x = (bits.view(np.uint16) if dt == "f16" else bits).astype(np.int64)
    return np.where(x & 0x8000, -(x & 0x7FFF), x)


@pytest.mark.parametrize("partition", [16, 64, 256, 512, 2048, 0])
def test_partition_sizes_agree(partition):
    # up to 8 partitions of the longest context (1,500 tokens): one workgroup
    # per partition; more: the persistent grid
    p = prepared("gqa8b_bf16", num_seqs=12, hi=1500)
    d = p.device()
    p.write_step(d)
    out = p.gpu_decode(d, partition=partition)
    assert_close(out_f64(out), p.oracle_decode(), "bf16", f"P={partition}")


def test_split_and_unsplit_launches_match_single_call():
    from paged_kv_cache_395_amd import ops
    p = prepared("gqa8b_bf16", num_seqs=12, hi=1500)
    d = p.device()
    p.write_step(d)
    a = p.gpu_decode(d)
    ws = torch.empty(ops.decode_workspace_bytes(12, 32, 8, 128, p.max_ctx, 0), dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    ops.decode_partitions(b, d["q"], d["k"], d["v"], d["table"], d["ctx"], p.w.scale, p.max_ctx, 0, ws)
    ops.decode_reduce(b, d["ctx"], 8, p.max_ctx, 0, ws)
    assert torch.equal(a, b)
    # the same with an explicit split into several partitions
    a = p.gpu_decode(d, partition=256)
    ws = torch.empty(ops.decode_workspace_bytes(12, 32, 8, 128, p.max_ctx, 256), dtype=torch.uint8, device="cuda")
    ops.decode_partitions(b, d["q"], d["k"], d["v"], d["table"], d["ctx"], p.w.scale, p.max_ctx, 256, ws)
    ops.decode_reduce(b, d["ctx"], 8, p.max_ctx, 256, ws)
    assert torch.equal(a, b)


def test_repeat_runs_are_bitwise_identical():
    p = prepared("gqa8b_bf16", num_seqs=12, hi=1500)
    d = p.device()
    p.write_step(d)
    a = p.gpu_decode(d)
    for _ in range(3):
        assert torch.equal(a, p.gpu_decode(d))


@pytest.mark.parametrize("name,kw", [("gqa8b_bf16", dict(num_seqs=12, hi=1500)), ("tiny_f32", {}),
                                     ("mha7b_f16", dict(num_seqs=6, lo=1, hi=1100))], ids=["bf16", "f32", "f16"])
def test_relabelling_physical_blocks_is_bitwise_invisible(name, kw):
    p = prepared(name, **kw)
    d = p.device()
    p.write_step(d)
    a = p.gpu_decode(d)
    perm = torch.from_numpy(np.random.default_rng(5).permutation(p.w.num_blocks)).cuda()
    k2 = torch.empty_like(d["k"])
    v2 = torch.empty_like(d["v"])
    k2[perm] = d["k"]
    v2[perm] = d["v"]
    table = d["table"].long()
    live = table < p.w.num_blocks
    t2 = torch.where(live, perm[table.clamp(max=p.w.num_blocks - 1)], table).to(torch.int32)
    d2 = dict(d, k=k2, v=v2, table=t2)
    assert torch.equal(a, p.gpu_decode(d2))


def test_nan_in_unread_memory_never_reaches_the_output():
    # unused blocks and tail slots past each context are NaN; padding entries
    # of the table point outside the pool
    p = prepared("gqa8b_bf16", num_seqs=12, hi=1500)
    w = p.w
    k, v = (a.copy() for a in p.oracle_pools())
    used = np.zeros(w.num_blocks, bool)
    for s, c in enumerate(p.ctx):
        nb = -(-int(c) // 16)
        used[p.table[s, :nb]] = True
        # tail slots of the last block: write NaN tokens there through the oracle's cache write
        tail = [int(p.table[s, nb - 1]) * 16 + o for o in range(int(c) - (nb - 1) * 16, 16)]
        if tail:
            nan = np.full((len(tail), w.num_kv_heads, w.head_dim), 0x7FC0, np.uint16)
            OA.reshape_and_cache(k, v, nan, nan, np.array(tail))
    k[~used] = 0x7FC0
    v[~used] = 0x7FC0
    d = p.device()
    d["k"] = to_dev(k, "bf16")
    d["v"] = to_dev(v, "bf16")
    out = p.gpu_decode(d)
    assert_close(out_f64(out), p.oracle_decode(), "bf16", "poisoned")


def test_single_token_context_returns_its_value_exactly():
    p = prepared("tiny_f32")
    d = p.device()
    p.write_step(d)
    out = out_f64(p.gpu_decode(d))
    s = int(np.nonzero(p.ctx == 1)[0][0])
    G = p.w.group
    for h in range(p.w.num_q_heads):
        assert np.array_equal(out[s, h], p.w.step_v[s, 0, h // G].astype(np.float64))
    # bf16 on the matrix cores: same property
    w = make_workload("gqa8b_bf16", num_seqs=3, hi=40)
    w.program[0] = ("add", 0, 0)  # sequence 0 holds only the token the step writes
    w.lengths["final_ctx"][0] = 1
    q = Prepared(w)
    dq = q.device()
    q.write_step(dq)
    out = out_f64(q.gpu_decode(dq))
    want = OA.to_f64(w.step_v[0, 0], "bf16")
    for h in range(w.num_q_heads):
        assert np.array_equal(out[0, h], want[h // w.group])


def test_dominant_key_selects_its_value_and_zero_query_averages():
    p = prepared("gqa8b_bf16", num_seqs=12, hi=1500)
    w = p.w
    d = p.device()
    p.write_step(d)
    # zero query: the mean of V over the context
    q0 = torch.zeros_like(d["q"])
    out = out_f64(p.gpu_decode(d, q=q0))
    ref = p.oracle_decode(q=np.zeros_like(w.decode_q))
    assert_close(out, ref, "bf16", "q=0")
    # dominant key: make q parallel to one cached key with a huge norm
    s, t = 3, int(p.ctx[3]) // 2
    k, v = p.oracle_pools()
    K, V = OA.gather_kv(k, v, p.table[s], int(p.ctx[s]), "bf16")
    qd = w.decode_q.copy()
    G = w.group
    for h in range(w.num_q_heads):
        kt = K[h // G, t]
        from workloads import to_storage
        qd[s, h] = to_storage((kt * 64.0).astype(np.float32), "bf16")
    out = out_f64(p.gpu_decode(d, q=to_dev(qd, "bf16")))
    ref = p.oracle_decode(q=qd, seqs=[s])
    assert_close(out[s], ref[s], "bf16", "dominant")


def test_zero_length_context_gives_a_zero_row_and_bad_entries_give_nan():
    p = prepared("gqa8b_bf16", num_seqs=12, hi=1500)
    d = p.device()
    p.write_step(d)
    ctx = d["ctx"].clone()
    ctx[2] = 0
    table = d["table"].clone()
    table[5, 0] = p.w.num_blocks + 3  # outside the pool: guarded, reported as NaN
    out = out_f64(p.gpu_decode(d, ctx=ctx, table=table))
    assert np.all(out[2] == 0)
    assert np.all(np.isnan(out[5]))
    ref = p.oracle_decode()
    keep = [s for s in range(12) if s not in (2, 5)]
    assert_close(out[keep], ref[keep], "bf16", "other rows")
    # a context longer than max_context_len is reported, not read past the grid
    ctx = d["ctx"].clone()
    ctx[7] = p.max_ctx + 1
    out = out_f64(p.gpu_decode(d, ctx=ctx))
    assert np.all(np.isnan(out[7]))


def _scale_blocks_along_context(p, per=8):
    """Multiply every key block by 2^(logical block // per) (exact for these
    types), so scores grow along each context."""
    w = p.w
    if w.dtype == "bf16":
        k = (w.k_pool.astype(np.uint32) << np.uint32(16)).view(np.float32)
    else:
        k = w.k_pool.astype(np.float32)
    done = set()
    for s in range(len(p.ctx)):
        for lb in range(-(-int(p.ctx[s]) // w.block_size)):
            b = int(p.table[s, lb])
            assert b not in done, "a shared block would be scaled twice"
            done.add(b)
            k[b] *= np.float32(2.0 ** (lb // per))
    w.k_pool[...] = to_storage(k, w.dtype) if w.dtype != "f32" else k


@pytest.mark.parametrize("name,kw", [("mha7b_f16", dict(num_seqs=5, lo=300, hi=1100)),
                                     ("gqa8b_bf16", dict(num_seqs=8, hi=1500))], ids=["f16", "bf16"])
@pytest.mark.parametrize("partition", [64, 0])
def test_scores_growing_along_the_context(name, kw, partition):
    """The running max moves again and again inside a partition (lazy
    rescale) and the partitions' maxima differ by orders of magnitude (LSE
    merge)."""
    p = Prepared(make_workload(name, **kw))
    _scale_blocks_along_context(p)
    say(f"[decode] growing scores {name} P={partition}")
    d = p.device()
    p.write_step(d)
    out = p.gpu_decode(d, partition=partition)
    assert_close(out_f64(out), p.oracle_decode(), p.w.dtype, f"{name} growing scores")
