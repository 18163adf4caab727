"""Seeded synthetic inputs for continuous-batching runs.

A request trace (arrival step, id, prompt length, final length) and K/V /
query rows that depend only on (seed, request, position) or (seed, request,
step), so that a request's cached tokens have the same values however often
it is preempted, moved or recomputed.  No attention or paging arithmetic
lives here.
"""

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
