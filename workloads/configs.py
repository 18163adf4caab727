"""Seeded workload definitions for paged decode, paged prefill and the cache write.

Every workload is a fixed recipe of shapes, length distributions and sharing
structure, drawn from ``numpy.random.default_rng(seed)`` in a fixed order:

  1. context / tail lengths
  2. the initial free-block order (a permutation of the whole pool)
  3. the K and V pools, i.i.d. N(0, 1) over every element of every block
  4. the queries of the step
  5. the K and V rows of the tokens the step appends

Floating values are drawn in fp32 and rounded to the storage type by
round-to-nearest-even on the host; bf16 is carried as its raw 16-bit pattern
(``uint16``).  The GPU never re-rounds an input.

The sequences' cached state is described by a *program* of block-manager
operations (add a sequence, add one that shares a prefix, fork, free, extend).
Applying the program to a block manager yields the block tables; the step then
appends ``append`` tokens to every sequence of ``batch`` (seq-major order) and
runs attention for the batch.  Nothing here computes a slot, a tile offset or
an attention value.

The recipes mirror the situations on the pages: scattered physical blocks
("PagedAttention: How vLLM Serves AI Like an Operating System", section
"PagedAttention: Virtual Memory for KV Cache"), a 4-sequence 20-page pool
("vLLM Architecture and PagedAttention - Interactive Visualization", Page Table
Visualization), a shared system prompt and n=4 parallel sampling (same
article, section "Copy-on-Write: Sharing KV Cache").  The pages benchmark a
served model on a chat dataset; synthetic values of the model's attention
shape stand in for it here.
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np

BLOCK_SIZE = 16

_STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}


def storage_dtype(dtype: str):
    """numpy storage type of a pool / q / out element of ``dtype``."""
    return _STORAGE[dtype]


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp32 values to the storage type by round-to-nearest-even.

    bf16 comes back as raw uint16 bit patterns (the upper half of the fp32
    pattern after rounding); NaN stays a quiet NaN.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "f16":
        return x.astype(np.float16)  # numpy's conversion rounds to nearest even
    if dtype == "bf16":
        u = x.view(np.uint32)
        lsb = (u >> np.uint32(16)) & np.uint32(1)
        r = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
        nan = np.isnan(x)
        if nan.any():
            r[nan] = np.uint16(0x7FC0)
        return r
    raise ValueError(f"unknown dtype {dtype!r}")


def _normal_storage(rng: np.random.Generator, shape, dtype: str, chunk_rows: int = 1024) -> np.ndarray:
    """i.i.d. N(0,1) fp32 draws rounded to ``dtype``.

    Rows are cut into fixed chunks; chunk i draws from the i-th generator
    spawned from ``rng``, so the values do not depend on how many threads
    fill them.
    """
    out = np.empty(shape, dtype=storage_dtype(dtype))
    rows = shape[0]
    inner = tuple(shape[1:])
    starts = list(range(0, rows, chunk_rows))
    children = rng.spawn(len(starts))

    def fill(i):
        r0 = starts[i]
        r1 = min(rows, r0 + chunk_rows)
        out[r0:r1] = to_storage(children[i].standard_normal((r1 - r0,) + inner, dtype=np.float32), dtype)

    workers = min(len(starts), _workers())
    if workers <= 1:
        for i in range(len(starts)):
            fill(i)
    else:
        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(fill, range(len(starts))))
    return out


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


@dataclass
class Workload:
    name: str
    dtype: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    num_blocks: int
    scale: float
    partition_size: int              # tokens per context partition the workload states (0: the library's choice)
    append: int                      # tokens each batch sequence appends in the step
    free_order: np.ndarray           # int32 [num_blocks], the initial free-list order
    program: List[Tuple]             # block-manager operations that build the cached state
    batch: np.ndarray                # int64 [num_seqs], sequence ids in output-row order
    k_pool: np.ndarray               # storage [num_blocks, Hkv, BLOCK_SIZE * D]
    v_pool: np.ndarray
    q: np.ndarray                    # storage [S, append, Hq, D]
    step_k: np.ndarray               # storage [S, append, Hkv, D]
    step_v: np.ndarray
    block_size: int = BLOCK_SIZE
    description: str = ""
    lengths: dict = field(default_factory=dict)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def decode_q(self) -> np.ndarray:
        """Query of each sequence's last position, [S, Hq, D]."""
        return np.ascontiguousarray(self.q[:, -1])

    @property
    def step_seqs(self) -> np.ndarray:
        """Sequence id of every appended token, seq-major: [S * append]."""
        return np.repeat(self.batch, self.append)

    def step_rows(self, which: str) -> np.ndarray:
        """The appended tokens' K or V rows flattened to [S * append, Hkv, D]."""
        a = self.step_k if which == "k" else self.step_v
        return np.ascontiguousarray(a.reshape(self.num_seqs * self.append, self.num_kv_heads, self.head_dim))

    def max_blocks_per_seq(self, extra_tokens: int = 0) -> int:
        longest = int(self.lengths["final_ctx"].max()) + extra_tokens
        return -(-longest // self.block_size)


def _blocks(n: int, bs: int = BLOCK_SIZE) -> int:
    return -(-int(n) // bs)


def run_program(bm, program) -> None:
    """Apply a workload program to a block manager (the library's or the oracle's)."""
    for op in program:
        kind = op[0]
        if kind == "add":
            bm.add_seq(op[1], op[2])
        elif kind == "add_prefix":
            bm.add_seq_with_prefix(op[1], op[2], op[3], op[4])
        elif kind == "fork":
            bm.fork(op[1], op[2])
        elif kind == "free":
            bm.free_seq(op[1])
        elif kind == "extend":
            if op[2] > 0:
                bm.append_tokens(np.full(op[2], op[1], dtype=np.int64))
        else:
            raise ValueError(f"unknown program op {kind!r}")


def _finish(rng, name, dtype, S, Hq, Hkv, D, NB, scale, P, append, program, batch,
            description, lengths, block_size=BLOCK_SIZE) -> Workload:
    free_order = rng.permutation(NB).astype(np.int32)
    k_pool = _normal_storage(rng, (NB, Hkv, block_size * D), dtype)
    v_pool = _normal_storage(rng, (NB, Hkv, block_size * D), dtype)
    q = _normal_storage(rng, (S, append, Hq, D), dtype, chunk_rows=max(1, 65536 // max(1, append)))
    step_k = _normal_storage(rng, (S, append, Hkv, D), dtype, chunk_rows=max(1, 65536 // max(1, append)))
    step_v = _normal_storage(rng, (S, append, Hkv, D), dtype, chunk_rows=max(1, 65536 // max(1, append)))
    return Workload(name=name, dtype=dtype, num_seqs=S, num_q_heads=Hq, num_kv_heads=Hkv,
                    head_dim=D, num_blocks=NB, scale=scale, partition_size=P, append=append,
                    free_order=free_order, program=program, batch=np.asarray(batch, dtype=np.int64),
                    k_pool=k_pool, v_pool=v_pool, q=q, step_k=step_k, step_v=step_v,
                    block_size=block_size, description=description, lengths=lengths)


def _decode_from_lengths(rng, name, dtype, ctx, Hq, Hkv, D, P, NB=None, description="", block_size=BLOCK_SIZE):
    """Independent sequences: sequence s caches ctx[s]-1 tokens, the step appends one."""
    ctx = np.asarray(ctx, dtype=np.int64)
    S = len(ctx)
    need = int(sum(_blocks(c, block_size) for c in ctx))
    if NB is None:
        NB = int(math.ceil(1.25 * need))
    program = [("add", s, int(ctx[s]) - 1) for s in range(S)]
    if block_size != BLOCK_SIZE:
        description += f"; {block_size}-token blocks"
    return _finish(rng, name, dtype, S, Hq, Hkv, D, NB, 1.0 / math.sqrt(D), P, 1, program,
                   np.arange(S), description, {"final_ctx": ctx, "blocks_needed": need}, block_size)


def _tiny_f32(rng, ctx=(20, 37, 16, 1), block_size=BLOCK_SIZE):
    return _decode_from_lengths(
        rng, "tiny_f32", "f32", ctx, 4, 4, 64, 0, NB=20,
        description="4 sequences, fp32, 4/4 heads, head_dim 64, 20-block pool, 1 new token each",
        block_size=block_size)


def _mha7b_f16(rng, num_seqs=64, lo=128, hi=2048, block_size=BLOCK_SIZE, name="mha7b_f16"):
    ctx = rng.integers(lo, hi + 1, size=num_seqs)
    return _decode_from_lengths(
        rng, name, "f16", ctx, 32, 32, 128, 0,
        description=f"7B-shaped decode, fp16, batch {num_seqs}, 32/32 heads, head_dim 128, "
                    f"ctx U[{lo},{hi}], pool 1.25x need", block_size=block_size)


def _gqa8b_bf16(rng, num_seqs=256, median=1024, lo=16, hi=8192, block_size=BLOCK_SIZE, name="gqa8b_bf16"):
    ctx = np.clip(np.rint(np.exp(math.log(median) + rng.standard_normal(num_seqs))), lo, hi).astype(np.int64)
    return _decode_from_lengths(
        rng, name, "bf16", ctx, 32, 8, 128, 0, block_size=block_size,
        description=f"Llama-3-8B-shaped GQA decode, bf16, batch {num_seqs}, 32/8 heads, head_dim 128, "
                    f"ctx lognormal(median {median}, sigma 1) clipped to [{lo},{hi}]")


def _shared_prefix_bf16(rng, num_users=512, num_prompts=128, n_samples=4,
                        sys_tokens=64, prompt_tokens=96, user_tail=(16, 1024), sample_tail=(17, 32)):
    if sys_tokens % BLOCK_SIZE or prompt_tokens % BLOCK_SIZE:
        raise ValueError("shared prefixes are whole blocks")
    user_tails = rng.integers(user_tail[0], user_tail[1] + 1, size=num_users)
    sample_tails = rng.integers(sample_tail[0], sample_tail[1] + 1, size=num_prompts * n_samples)
    SYS = 1_000_000
    PROMPT0 = 2_000_000
    program: List[Tuple] = [("add", SYS, sys_tokens)]
    for u in range(num_users):
        program.append(("add_prefix", u, SYS, sys_tokens, int(user_tails[u]) - 1))
    program.append(("free", SYS))
    child = num_users
    for p in range(num_prompts):
        program.append(("add", PROMPT0 + p, prompt_tokens))
        kids = list(range(child, child + n_samples))
        for c in kids:
            program.append(("fork", PROMPT0 + p, c))
        program.append(("free", PROMPT0 + p))
        for c in kids:
            program.append(("extend", c, int(sample_tails[c - num_users]) - 1))
        child += n_samples
    S = num_users + num_prompts * n_samples
    final_ctx = np.concatenate([sys_tokens + user_tails, prompt_tokens + sample_tails]).astype(np.int64)
    need = (_blocks(sys_tokens) + int(sum(_blocks(t) for t in user_tails))
            + num_prompts * _blocks(prompt_tokens) + int(sum(_blocks(t) for t in sample_tails)))
    NB = int(math.ceil(1.25 * need))
    return _finish(rng, "shared_prefix_bf16", "bf16", S, 32, 8, 128, NB, 1.0 / math.sqrt(128), 0, 1,
                   program, np.arange(S),
                   f"{num_users} sequences on a {sys_tokens}-token shared prompt plus {num_prompts} prompts "
                   f"of {prompt_tokens} tokens sampled n={n_samples}; bf16, 32/8 heads, head_dim 128",
                   {"final_ctx": final_ctx, "blocks_needed": need})


def _longctx_bf16(rng, num_seqs=16, ctx=32768, chunk=512, Hq=64, Hkv=8, NB=None, dtype="bf16", head_dim=128,
                  block_size=BLOCK_SIZE):
    if ctx < chunk:
        raise ValueError("the chunk lies inside the context")
    need = num_seqs * _blocks(ctx, block_size)
    if NB is None:
        NB = int(math.ceil(1.25 * need))
    program = [("add", s, ctx - chunk) for s in range(num_seqs)]
    D = head_dim
    return _finish(rng, "longctx_bf16", dtype, num_seqs, Hq, Hkv, D, NB, 1.0 / math.sqrt(D), 512,
                   chunk, program, np.arange(num_seqs),
                   f"{num_seqs} sequences at context {ctx} (the last {chunk} tokens appended as one chunk), "
                   f"{dtype}, {Hq}/{Hkv} heads, head_dim {D}, 512-token partitions"
                   + ("" if block_size == BLOCK_SIZE else f", {block_size}-token blocks"),
                   {"final_ctx": np.full(num_seqs, ctx, dtype=np.int64), "blocks_needed": need}, block_size)


def _specdec_bf16(rng, num_seqs=256, median=1024, lo=16, hi=8192, q_len=4, block_size=BLOCK_SIZE):
    """Speculative verification: every sequence appends q_len drafted tokens and attends each causally."""
    ctx = np.clip(np.rint(np.exp(math.log(median) + rng.standard_normal(num_seqs))), max(lo, q_len), hi)
    ctx = ctx.astype(np.int64)
    need = int(sum(_blocks(c, block_size) for c in ctx))
    NB = int(math.ceil(1.25 * need))
    program = [("add", s, int(ctx[s]) - q_len) for s in range(num_seqs)]
    return _finish(rng, "specdec_bf16", "bf16", num_seqs, 32, 8, 128, NB, 1.0 / math.sqrt(128), 0, q_len,
                   program, np.arange(num_seqs),
                   f"Llama-3-8B-shaped GQA verification of {q_len} drafted tokens per sequence, bf16, batch "
                   f"{num_seqs}, 32/8 heads, head_dim 128, ctx lognormal(median {median}, sigma 1) clipped to "
                   f"[{max(lo, q_len)},{hi}]" + ("" if block_size == BLOCK_SIZE else f", {block_size}-token blocks"),
                   {"final_ctx": ctx, "blocks_needed": need, "mode": "multi"}, block_size)


WORKLOADS = {
    "tiny_f32": (1001, _tiny_f32),
    "mha7b_f16": (1002, _mha7b_f16),
    "gqa8b_bf16": (1003, _gqa8b_bf16),
    "shared_prefix_bf16": (1004, _shared_prefix_bf16),
    "longctx_bf16": (1005, _longctx_bf16),
    "specdec_bf16": (1006, _specdec_bf16),
    # block-size variants of the 7B and GQA decode workloads (same contexts: same seeds)
    "mha7b_f16_bs32": (1002, lambda rng, **kw: _mha7b_f16(rng, block_size=32, name="mha7b_f16_bs32", **kw)),
    "mha7b_f16_bs64": (1002, lambda rng, **kw: _mha7b_f16(rng, block_size=64, name="mha7b_f16_bs64", **kw)),
    "gqa8b_bf16_bs32": (1003, lambda rng, **kw: _gqa8b_bf16(rng, block_size=32, name="gqa8b_bf16_bs32", **kw)),
}


def make_workload(name: str, seed: Optional[int] = None, **overrides) -> Workload:
    """Build a named workload.  ``overrides`` shrink it (fewer sequences, shorter contexts)."""
    default_seed, fn = WORKLOADS[name]
    rng = np.random.default_rng(default_seed if seed is None else seed)
    return fn(rng, **overrides)
