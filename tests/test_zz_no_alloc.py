"""The allocation-free decode (pa_decode_noalloc) against pa_decode, through
the C ABI: bitwise the same output on two calls in a row, the second on a
smaller batch (the shared scratch array keeps the first call's contents),
each also within the stated tolerance of the oracle; sizes beyond the array
are refused before any launch."""
import ctypes

import numpy as np
import pytest
import torch

from paged_kv_cache_395_amd import _lib, ops
from tests._gpu import Prepared, assert_close, out_f64, say
from workloads import make_workload

pytestmark = pytest.mark.gpu


def _call_noalloc(out, d, p, partition):
    w = p.w
    L = _lib.load()
    q = d["q"]
    NB, Hkv, D, bs = ops._pools(d["k"], d["v"], q.shape[-1])
    st = L.pa_decode_noalloc(ctypes.c_void_p(out.data_ptr()), ops._code(out), ctypes.c_void_p(q.data_ptr()),
                             ctypes.c_void_p(d["k"].data_ptr()), ctypes.c_void_p(d["v"].data_ptr()),
                             ctypes.c_void_p(d["table"].data_ptr()), d["table"].shape[1],
                             ctypes.c_void_p(d["ctx"].data_ptr()), q.shape[0], q.shape[1], Hkv, D, bs, NB,
                             float(w.scale), p.max_ctx, partition, ops._code(q),
                             ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st


@pytest.mark.parametrize("partition", [64, 0])
def test_noalloc_decode_matches_decode_on_two_calls_the_second_smaller(partition):
    # first call: 40 GQA sequences; second: 9 shorter ones (P=64 splits them
    # over many partitions, the persistent grid; 0 = the library's choice)
    for i, kw in enumerate([dict(num_seqs=40, hi=3000), dict(num_seqs=9, hi=900)]):
        p = Prepared(make_workload("gqa8b_bf16", seed=77 + i, **kw))
        say(f"[noalloc] call {i} S={p.w.num_seqs} max_ctx={p.max_ctx} P={partition}")
        d = p.device()
        p.write_step(d)
        ref = torch.empty(d["q"].shape, dtype=torch.float32, device="cuda")
        ops.decode(ref, d["q"], d["k"], d["v"], d["table"], d["ctx"], p.w.scale, p.max_ctx, partition)
        out = torch.full_like(ref, float("nan"))
        assert _call_noalloc(out, d, p, partition) == _lib.PA_OK, _lib.load().pa_last_error()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        assert_close(out_f64(out), p.oracle_decode(), "bf16", f"noalloc call {i}")


def test_noalloc_refuses_sizes_beyond_its_array():
    L = _lib.load()
    cap = L.pa_decode_noalloc_scratch_bytes()
    assert cap == 64 << 20
    # 16 sequences x 64 heads bounded by 65,536 tokens in 16-token partitions
    # need far more; every buffer has its full size and every context is 0,
    # so nothing would be read even if a launch happened
    S, Hq, Hkv, D, maxb = 16, 64, 8, 128, 4096
    need = ops.decode_workspace_bytes(S, Hq, Hkv, D, 65536, 16)
    assert need > cap
    q = torch.zeros(S, Hq, D, dtype=torch.bfloat16, device="cuda")
    out = torch.empty(S, Hq, D, dtype=torch.float32, device="cuda")
    k = torch.zeros(4, Hkv, 16 * D, dtype=torch.bfloat16, device="cuda")
    v = torch.zeros_like(k)
    table = torch.zeros(S, maxb, dtype=torch.int32, device="cuda")
    ctx = torch.zeros(S, dtype=torch.int32, device="cuda")
    p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    st = L.pa_decode_noalloc(p(out), _lib.PA_F32, p(q), p(k), p(v), p(table), maxb, p(ctx), S, Hq, Hkv, D, 16, 4,
                             0.1, 65536, 16, _lib.PA_BF16, None)
    assert st == _lib.PA_EWORKSPACE
    assert b"scratch" in L.pa_last_error()
