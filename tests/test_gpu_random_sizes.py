"""Decode and chunked prefill on seeded random batch shapes against the fp64
oracle.  Decode: GQA and MHA single-query decode and several queries per
sequence, at partition sizes from 16 to 512 tokens, so that both launch
shapes run, the persistent split's share boundaries move off short pair ends
and its odd-XCD shares are lighter, and the per-partition grid with 32 kv
heads deals its items over the XCDs.  Prefill: chunks, head groups, both
16-bit types, head sizes and block sizes drawn at random."""
import numpy as np
import pytest
import torch

from oracle import attention as OA
from paged_kv_cache_395_amd import ops
from tests._gpu import Prepared, assert_close, out_f64, say, to_dev
from workloads import make_workload

pytestmark = pytest.mark.gpu


def _cases(n, seed=20261203):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        kind = str(rng.choice(["gqa", "spec", "mha"]))
        P = int(rng.choice([16, 32, 64, 128, 512]))
        wseed = int(rng.integers(1 << 30))
        if kind == "gqa":
            kw = dict(num_seqs=int(rng.integers(4, 40)), median=int(rng.choice([64, 300, 900])),
                      hi=int(rng.choice([600, 2500])))
        elif kind == "spec":
            kw = dict(num_seqs=int(rng.integers(4, 40)), median=int(rng.choice([64, 300, 900])),
                      hi=int(rng.choice([600, 2500])), q_len=int(rng.choice([2, 4])))
        else:
            kw = dict(num_seqs=int(rng.integers(2, 24)), lo=1, hi=int(rng.choice([300, 1500])))
        out.append((kind, P, wseed, kw))
    return out


@pytest.mark.parametrize("kind, P, wseed, kw", _cases(24))
def test_decode_on_random_shapes_matches_oracle(kind, P, wseed, kw):
    name = {"gqa": "gqa8b_bf16", "spec": "specdec_bf16", "mha": "mha7b_f16"}[kind]
    w = make_workload(name, seed=wseed, **kw)
    p = Prepared(w)
    say(f"[random] {kind} P={P} seed={wseed} {kw}")
    d = p.device()
    p.write_step(d)
    k, v = p.oracle_pools()
    if kind == "spec":
        q = to_dev(w.q, w.dtype)
        out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
        ops.decode_multi(out, q, d["k"], d["v"], d["table"], d["ctx"], w.scale, p.max_ctx, P)
        ref = OA.prefill_chunk(w.q, k, v, p.table, p.ctx, w.scale, w.dtype)
    else:
        out = p.gpu_decode(d, partition=P)
        ref = p.oracle_decode()
    assert_close(out_f64(out), ref, w.dtype, f"{kind} P={P} seed={wseed}")


def _prefill_cases(n, seed=20261204):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        Hq, Hkv = [(8, 8), (16, 4), (32, 8), (32, 4), (8, 1), (16, 16)][int(rng.integers(6))]
        chunk = int(rng.choice([1, 3, 17, 64, 100, 128]))
        kw = dict(num_seqs=int(rng.integers(1, 4)), ctx=int(rng.integers(chunk, 1500)), chunk=chunk, Hq=Hq,
                  Hkv=Hkv, dtype=str(rng.choice(["bf16", "f16"])), head_dim=int(rng.choice([64, 128])),
                  block_size=int(rng.choice([16, 32, 64])))
        out.append((int(rng.integers(1 << 30)), kw))
    return out


@pytest.mark.parametrize("wseed, kw", _prefill_cases(24))
def test_prefill_on_random_shapes_matches_oracle(wseed, kw):
    # chunks of 1 to 128 queries, head groups 1 to 8, both 16-bit types,
    # head_dim 64 / 128, blocks of 16 / 32 / 64 tokens
    w = make_workload("longctx_bf16", seed=wseed, **kw)
    p = Prepared(w)
    say(f"[random prefill] seed={wseed} {kw}")
    d = p.device()
    p.write_step(d)
    q = to_dev(w.q, w.dtype)
    out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    ops.prefill_chunk(out, q, d["k"], d["v"], d["table"], d["ctx"], w.scale, p.max_ctx)
    k, v = p.oracle_pools()
    ref = OA.prefill_chunk(w.q, k, v, p.table, p.ctx, w.scale, w.dtype)
    assert_close(out_f64(out), ref, w.dtype, f"prefill seed={wseed} {kw}")
