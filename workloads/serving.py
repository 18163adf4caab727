"""Seeded synthetic inputs for continuous-batching runs.

A request trace (arrival step, id, prompt length, final length) and K/V /
query rows that depend only on (seed, request, position) or (seed, request,
step), so that a request's cached tokens have the same values however often
it is preempted, moved or recomputed.  No attention or paging arithmetic
lives here.
"""

import zlib

import numpy as np

from .configs import to_storage


def request_trace(seed: int, num_requests: int, mean_gap: float, prompt_median: int, prompt_hi: int,
                  output_median: int, output_hi: int, lo: int = 1):
    """Poisson arrivals (per step) with lognormal prompt and output lengths.

    Returns a sorted list of (arrival_step, request_id, prompt_tokens, total_tokens).
    """
    rng = np.random.default_rng(seed)
    gaps = rng.exponential(mean_gap, size=num_requests)
    arrive = np.floor(np.cumsum(gaps) - gaps[0]).astype(np.int64)
    prompt = np.clip(np.round(rng.lognormal(np.log(prompt_median), 0.8, size=num_requests)), lo, prompt_hi)
    output = np.clip(np.round(rng.lognormal(np.log(output_median), 0.8, size=num_requests)), 1, output_hi)
    return [(int(a), i, int(p), int(p + o)) for i, (a, p, o) in enumerate(zip(arrive, prompt, output))]


def kv_rows(seed: int, seq: int, positions, num_kv_heads: int, head_dim: int, dtype: str):
    """K and V storage rows [len(positions), Hkv, D] of one request's tokens."""
    k = np.empty((len(positions), num_kv_heads, head_dim), dtype=np.float32)
    v = np.empty_like(k)
    for i, p in enumerate(positions):
        rng = np.random.default_rng([seed, int(seq), int(p)])
        k[i] = rng.standard_normal((num_kv_heads, head_dim), dtype=np.float32)
        v[i] = rng.standard_normal((num_kv_heads, head_dim), dtype=np.float32)
    return to_storage(k, dtype), to_storage(v, dtype)


def query_rows(seed: int, seq: int, step: int, num_q_heads: int, head_dim: int, dtype: str):
    """One request's query [Hq, D] at one step."""
    rng = np.random.default_rng([seed, 1 << 20, int(seq), int(step)])
    return to_storage(rng.standard_normal((num_q_heads, head_dim), dtype=np.float32), dtype)


def token_keys(seq: int, positions, prompt_ids=None):
    """An integer per token naming its K/V content: a prompt token is named by
    its whole prefix of ids (equal prefixes give equal K/V, as a model's would),
    any other token by (request, position)."""
    keys = []
    for p in positions:
        p = int(p)
        if prompt_ids is not None and p < len(prompt_ids):
            h = zlib.crc32(np.asarray(prompt_ids[: p + 1], dtype=np.int32).tobytes())
            keys.append((1 << 40) + (p << 32) + h)
        else:
            keys.append((2 << 40) + (int(seq) << 20) + p)
    return keys


def kv_rows_by_key(seed: int, keys, num_kv_heads: int, head_dim: int, dtype: str):
    """K and V storage rows [len(keys), Hkv, D], one per content key."""
    k = np.empty((len(keys), num_kv_heads, head_dim), dtype=np.float32)
    v = np.empty_like(k)
    for i, key in enumerate(keys):
        rng = np.random.default_rng([seed, int(key) & 0xFFFFFFFF, int(key) >> 32])
        k[i] = rng.standard_normal((num_kv_heads, head_dim), dtype=np.float32)
        v[i] = rng.standard_normal((num_kv_heads, head_dim), dtype=np.float32)
    return to_storage(k, dtype), to_storage(v, dtype)


def prefix_requests(seed: int, num_requests: int, num_prompts: int, system_len: int, tail_median: int,
                    tail_hi: int, output_median: int, output_hi: int, mean_gap: float, vocab: int = 32000):
    """Requests on a few shared system prompts: (arrival, id, prompt ids, total)."""
    rng = np.random.default_rng(seed)
    systems = [rng.integers(0, vocab, size=system_len).tolist() for _ in range(num_prompts)]
    gaps = rng.exponential(mean_gap, size=num_requests)
    arrive = np.floor(np.cumsum(gaps) - gaps[0]).astype(np.int64)
    out = []
    for i in range(num_requests):
        tail = int(np.clip(round(rng.lognormal(np.log(tail_median), 0.8)), 1, tail_hi))
        gen = int(np.clip(round(rng.lognormal(np.log(output_median), 0.8)), 1, output_hi))
        ids = systems[int(rng.integers(num_prompts))] + rng.integers(0, vocab, size=tail).tolist()
        out.append((int(arrive[i]), i, ids, len(ids) + gen))
    return out
