"""Several queries per sequence (verifying drafted tokens) on the GPU against
the oracle: the last q_len positions of each context attend causally, which
is the oracle's chunked prefill with a small chunk."""
import numpy as np
import pytest
import torch

from oracle import attention as OA
from paged_kv_cache_395_amd import PAError, ops
from tests._gpu import TORCH, Prepared, assert_close, out_f64, say, to_dev
from workloads import make_workload

pytestmark = pytest.mark.gpu


def run_multi(p, d, partition=0, out_f32=True, q=None):
    w = p.w
    q = to_dev(w.q, w.dtype) if q is None else q
    out = torch.empty(q.shape, dtype=torch.float32 if out_f32 else q.dtype, device="cuda")
    ops.decode_multi(out, q, d["k"], d["v"], d["table"], d["ctx"], w.scale, p.max_ctx, partition)
    return out


@pytest.mark.parametrize("partition", [0, 16, 64, 512])
def test_multi_query_matches_oracle_on_ragged_contexts(partition):
    # P = 16 leaves partitions that hold only keys past the early queries' positions
    p = Prepared(make_workload("specdec_bf16", num_seqs=12, hi=1500))
    say(f"[multi] specdec reduced P={partition}")
    d = p.device()
    p.write_step(d)
    out = run_multi(p, d, partition)
    k, v = p.oracle_pools()
    ref = OA.prefill_chunk(p.w.q, k, v, p.table, p.ctx, p.w.scale, "bf16")
    assert_close(out_f64(out), ref, "bf16", f"P={partition}")


def test_multi_query_with_moved_share_boundaries():
    # The longest context spans 9 partitions of 512 (the persistent grid) and
    # the shares are longer than 16 + 32 tiles, so a boundary that would
    # leave at most 16 tiles (16 rows per pair) of a pair on one side moves
    # to the pair's edge.  Every row is checked.
    p = Prepared(make_workload("specdec_bf16", num_seqs=64, hi=4600))
    w = p.w
    kernel, grid = ops.decode_launch_shape(TORCH[w.dtype], w.head_dim, torch.float32, w.num_seqs, w.num_q_heads,
                                           w.num_kv_heads, p.max_ctx)
    weight = sum(((int(c) + 15) // 16 + 12) * w.num_kv_heads for c in p.ctx if c > 0)
    assert kernel == "decode_persistent_kernel" and weight // min(grid, weight // 32) > 16 + 32, (kernel, grid, weight)
    say(f"[multi] specdec 64 sequences, moved share boundaries, grid {grid}")
    d = p.device()
    p.write_step(d)
    out = run_multi(p, d)
    k, v = p.oracle_pools()
    ref = OA.prefill_chunk(w.q, k, v, p.table, p.ctx, w.scale, "bf16")
    assert_close(out_f64(out), ref, "bf16", "64 sequences")


def test_multi_query_full_size_on_sampled_sequences():
    p = Prepared(make_workload("specdec_bf16"))
    say("[multi] specdec full size, 256 x 4 queries")
    d = p.device()
    p.write_step(d)
    out = out_f64(run_multi(p, d))
    k, v = p.oracle_pools()
    longest = int(np.argmax(p.ctx))
    seqs = sorted({0, 1, 100, 255, longest})
    ref = OA.prefill_chunk(p.w.q, k, v, p.table, p.ctx, p.w.scale, "bf16", seqs=seqs)
    assert_close(out[seqs], ref[seqs], "bf16", "sampled sequences")


def test_mha_eight_queries_fp16_and_too_many_columns():
    # group 1, fp16, 8 queries per sequence (from the long-context generator's shapes)
    w = make_workload("longctx_bf16", num_seqs=5, ctx=777, chunk=8, Hq=4, Hkv=4, dtype="f16")
    p = Prepared(w)
    d = p.device()
    p.write_step(d)
    out = run_multi(p, d)
    k, v = p.oracle_pools()
    ref = OA.prefill_chunk(w.q, k, v, p.table, p.ctx, w.scale, "f16")
    assert_close(out_f64(out), ref, "f16", "mha q_len 8")
    # 8 queries x group 4 = 32 columns: not a decode-shaped problem (the chunked-prefill kernel serves it)
    w8 = make_workload("specdec_bf16", num_seqs=3, hi=300, q_len=8)
    p8 = Prepared(w8)
    d8 = p8.device()
    with pytest.raises(PAError):
        run_multi(p8, d8)


def test_single_query_is_decode_bit_for_bit_and_last_query_matches_decode():
    p = Prepared(make_workload("specdec_bf16", num_seqs=12, hi=1500))
    d = p.device()
    p.write_step(d)
    # q_len 1 with the last position's query: the decode kernel's own result
    q1 = to_dev(np.ascontiguousarray(p.w.q[:, -1:]), "bf16")
    one = run_multi(p, d, q=q1)
    dec = p.gpu_decode(d)
    assert torch.equal(one[:, 0], dec)
    # the last of 4 queries sees the whole context: its column computes exactly decode's sums
    many = run_multi(p, d)
    assert torch.equal(many[:, -1], dec)


def test_output_in_input_dtype_and_short_context_rows():
    p = Prepared(make_workload("specdec_bf16", num_seqs=6, hi=400))
    d = p.device()
    p.write_step(d)
    outf = run_multi(p, d)
    outb = run_multi(p, d, out_f32=False)
    assert torch.equal(outb, outf.to(torch.bfloat16))
    # a context shorter than q_len violates the contract: NaN rows for that sequence only
    ctx = d["ctx"].clone()
    ctx[2] = 3
    out = torch.empty_like(outf)
    ops.decode_multi(out, to_dev(p.w.q, "bf16"), d["k"], d["v"], d["table"], ctx, p.w.scale, p.max_ctx)
    got = out_f64(out)
    assert np.all(np.isnan(got[2]))
    keep = [s for s in range(6) if s != 2]
    assert np.array_equal(got[keep], out_f64(outf)[keep])
