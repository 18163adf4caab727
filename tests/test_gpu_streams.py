"""Stream semantics of the device entry points.

Every device entry point runs on the stream it is given (the caller's
current torch stream by default) and waits for nothing else.

Each test first keeps a side stream busy with a spin kernel, then writes an
input of the call on that stream, then makes the call there.  A call that
went to another stream would run before the input is written and give a
wrong result.  The last test keeps the default stream busy instead and
checks that a call on a side stream finishes while the default stream is
still spinning: the library neither synchronises nor uses the default stream.
"""
import time

import numpy as np
import pytest
import torch

from oracle import attention as OA
from paged_kv_cache_395_amd import ops
from tests._gpu import Prepared, assert_close, out_f64, say, to_dev, to_host
from workloads import make_workload

pytestmark = pytest.mark.gpu

SPIN = 50_000_000  # GPU clock cycles of the spin kernel: tens of milliseconds


def _busy(stream):
    with torch.cuda.stream(stream):
        torch.cuda._sleep(SPIN)


@pytest.fixture
def prep():
    p = Prepared(make_workload("gqa8b_bf16", num_seqs=8))
    d = p.device()
    torch.cuda.synchronize()
    return p, d


@pytest.mark.parametrize("explicit", [True, False], ids=["stream_arg", "current_stream"])
def test_cache_write_and_decode_wait_for_earlier_work_on_their_stream(prep, explicit):
    p, d = prep
    say(f"[streams] cache write + decode, explicit={explicit}")
    s = torch.cuda.Stream()
    slots = torch.full_like(d["slots"], -1)  # all skipped until the copy below lands
    q = torch.zeros_like(d["q"])
    out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    _busy(s)
    with torch.cuda.stream(s):
        slots.copy_(d["slots"])
        q.copy_(d["q"])
        arg = s if explicit else None
        ops.reshape_and_cache(d["step_k"], d["step_v"], d["k"], d["v"], slots, stream=arg)
        ops.decode(out, q, d["k"], d["v"], d["table"], d["ctx"], p.w.scale, p.max_ctx, stream=arg)
    s.synchronize()
    k_ref, v_ref = p.oracle_pools()
    assert np.array_equal(to_host(d["k"], "bf16"), k_ref) and np.array_equal(to_host(d["v"], "bf16"), v_ref)
    assert_close(out_f64(out), p.oracle_decode(), "bf16", "decode on a side stream")


def test_prefill_and_multi_query_decode_run_on_their_stream():
    p = Prepared(make_workload("longctx_bf16", num_seqs=2, ctx=300, chunk=40))
    say("[streams] prefill")
    d = p.device()
    p.write_step(d)
    q_src = to_dev(p.w.q, "bf16")
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    q = torch.zeros_like(q_src)
    out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    _busy(s)
    with torch.cuda.stream(s):
        q.copy_(q_src)
    ops.prefill_chunk(out, q, d["k"], d["v"], d["table"], d["ctx"], p.w.scale, p.max_ctx, stream=s)
    s.synchronize()
    k, v = p.oracle_pools()
    ref = OA.prefill_chunk(p.w.q, k, v, p.table, p.ctx, p.w.scale, "bf16")
    assert_close(out_f64(out), ref, "bf16", "prefill on a side stream")

    m = Prepared(make_workload("specdec_bf16", num_seqs=6, hi=400))
    say("[streams] multi-query decode")
    dm = m.device()
    m.write_step(dm)
    qm_src = to_dev(m.w.q, "bf16")
    torch.cuda.synchronize()
    qm = torch.zeros_like(qm_src)
    outm = torch.empty(qm.shape, dtype=torch.float32, device="cuda")
    _busy(s)
    with torch.cuda.stream(s):
        qm.copy_(qm_src)
    ops.decode_multi(outm, qm, dm["k"], dm["v"], dm["table"], dm["ctx"], m.w.scale, m.max_ctx, stream=s)
    s.synchronize()
    km, vm = m.oracle_pools()
    refm = OA.prefill_chunk(m.w.q, km, vm, m.table, m.ctx, m.w.scale, "bf16")
    assert_close(out_f64(outm), refm, "bf16", "multi-query decode on a side stream")


def test_append_step_and_block_copies_run_on_their_stream(prep):
    p, d = prep
    say("[streams] append step, copy_blocks")
    w = p.w
    S = len(p.ctx)
    rows = np.arange(S, dtype=np.int32)
    pos = (p.ctx - 1).astype(np.int32)
    table = p.table.copy()
    table[rows, pos // 16] = w.num_blocks + 777  # the append writes this entry back
    d_table = torch.from_numpy(table).cuda()
    d_ctx = torch.from_numpy(p.ctx - 1).cuda()
    meta_src = [torch.from_numpy(a).cuda() for a in (p.slots, rows, pos, p.ctx)]
    meta = [torch.zeros_like(t) for t in meta_src]
    meta[0].fill_(-1)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    _busy(s)
    with torch.cuda.stream(s):
        for a, b in zip(meta, meta_src):
            a.copy_(b)
    ops.append_step(d["step_k"], d["step_v"], d["k"], d["v"], *meta[:3], d_table, d_ctx, meta[3], stream=s)
    s.synchronize()
    assert np.array_equal(d_table.cpu().numpy(), p.table)
    assert np.array_equal(d_ctx.cpu().numpy(), p.ctx)
    k_ref, v_ref = p.oracle_pools()
    assert np.array_equal(to_host(d["k"], "bf16"), k_ref) and np.array_equal(to_host(d["v"], "bf16"), v_ref)

    used = set(p.table[p.table < w.num_blocks].ravel().tolist())
    free = [b for b in range(w.num_blocks) if b not in used][:4]
    src = sorted(used)[:4]
    pairs_src = torch.tensor(list(zip(src, free)), dtype=torch.int64, device="cuda")
    pairs = torch.zeros_like(pairs_src)
    pairs[:, 1] = free[0]  # block 0 onto one free block until the copy below lands
    pairs[:, 0] = 0
    torch.cuda.synchronize()
    _busy(s)
    with torch.cuda.stream(s):
        pairs.copy_(pairs_src)
    ops.copy_blocks(d["k"], d["v"], pairs, stream=s)
    s.synchronize()
    k_ref, v_ref = k_ref.copy(), v_ref.copy()
    OA.copy_blocks(k_ref, v_ref, np.array(list(zip(src, free)), dtype=np.int64))
    assert np.array_equal(to_host(d["k"], "bf16"), k_ref) and np.array_equal(to_host(d["v"], "bf16"), v_ref)


def test_a_side_stream_call_does_not_wait_for_the_default_stream(prep):
    p, d = prep
    say("[streams] no wait on the default stream")
    s = torch.cuda.Stream()
    out = torch.empty(d["q"].shape, dtype=torch.float32, device="cuda")
    # every entry point used below has run once (code objects loaded)
    ops.decode(out, d["q"], d["k"], d["v"], d["table"], d["ctx"], p.w.scale, p.max_ctx, stream=s)
    s.synchronize()
    default = torch.cuda.default_stream()
    with torch.cuda.stream(default):
        torch.cuda._sleep(10 * SPIN)  # about a quarter of a second
    t0 = time.perf_counter()
    ops.decode(out, d["q"], d["k"], d["v"], d["table"], d["ctx"], p.w.scale, p.max_ctx, stream=s)
    s.synchronize()
    waited = time.perf_counter() - t0
    still_busy = not default.query()
    torch.cuda.synchronize()
    assert still_busy, f"the side-stream decode finished only after the default stream ({waited:.3f} s)"
