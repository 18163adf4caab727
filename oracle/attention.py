"""Plain fp64 reference for the cache write, block copy and paged attention.

Pages cited (by title and section):
  [OS]  "PagedAttention: How vLLM Serves AI Like an Operating System"
  [VIZ] "vLLM Architecture and PagedAttention - Interactive Visualization"

What the pages fix: the KV cache lives in fixed 16-token blocks scattered
through GPU memory, and a per-request block table maps logical block i to a
physical block ([OS] "PagedAttention: Virtual Memory for KV Cache", How It
Works and the memory-layout example).  Paging changes where values live, not
what attention computes: the article says the gains come from memory
management alone, with the model's result unchanged ([OS] "Throughput Impact:
The Numbers").  The oracle therefore gathers each sequence's K and V through
its block table into a contiguous array (the "traditional" contiguous cache of
[OS] "The KV Cache Waste Problem") and runs textbook scaled dot-product
attention on it in fp64: softmax(scale * q K^T) V.  The attention formula
itself is not printed on the pages; it is the standard one of a decoder.

Readings where the pages are silent (each is listed with its reason in the
design notes):
  * context_lens counts the token the step just wrote (it sits at ctx - 1).
  * q head h reads kv head h // (Hq / Hkv) (contiguous GQA groups).
  * a slot is physical_block * bs + offset (bs = 16, the pages' size; 32 and
    64 as variants); a negative slot is skipped.
  * a chunk of C queries occupies the last C positions of the context, and
    query i attends keys 0 .. ctx - C + i.
  * ctx == 0 yields a zero output row.

Storage arrays are numpy float32 / float16, or uint16 holding bf16 bit
patterns; the oracle widens those exact values to fp64 itself.
"""

import numpy as np

from .layout import BLOCK_SIZE, block_index


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 value of every stored element."""
    if dtype in ("f32", "f16"):
        return np.asarray(a).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def round_f64_to(a: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp64 values to ``dtype`` storage by round-to-nearest-even (for out_dtype == dtype checks)."""
    if dtype == "f32":
        return a.astype(np.float32)
    if dtype == "f16":
        return a.astype(np.float16)
    if dtype == "bf16":
        # fp64 -> fp32 first is exact for the mantissa bits bf16 keeps except in
        # double-rounding ties; resolve those by comparing against the two
        # bf16 neighbours in fp64.
        f = a.astype(np.float32)
        u = f.view(np.uint32)
        lo = (u & np.uint32(0xFFFF0000))
        hi = lo + np.uint32(0x10000)
        lo_v = lo.view(np.float32).astype(np.float64)
        hi_v = hi.view(np.float32).astype(np.float64)
        dlo = np.abs(a - lo_v)
        dhi = np.abs(hi_v - a)
        lsb_odd = ((lo >> np.uint32(16)) & np.uint32(1)).astype(bool)
        pick_hi = (dhi < dlo) | ((dhi == dlo) & lsb_odd)
        r = np.where(pick_hi, hi, lo)
        return (r >> np.uint32(16)).astype(np.uint16)
    raise ValueError(f"unknown dtype {dtype!r}")


def reshape_and_cache(k_cache: np.ndarray, v_cache: np.ndarray, key: np.ndarray, value: np.ndarray,
                      slot_mapping: np.ndarray) -> None:
    """Write each new token's K and V rows into its slot, in place, bit for bit.

    key / value are [T, Hkv, D]; slot t names physical block slot // bs and
    offset slot % bs, bs = the pool's block size (16 unless a variant pool of
    32 or 64 tokens per block is passed) (on-demand filling of blocks as
    tokens are stored: [OS] "PagedAttention: Virtual Memory for KV Cache", How
    It Works).  Negative slots are skipped.
    """
    T, Hkv, D = key.shape
    bs = k_cache.shape[2] // D
    kidx = block_index("k", D, bs)
    vidx = block_index("v", D, bs)
    for t in range(T):
        slot = int(slot_mapping[t])
        if slot < 0:
            continue
        b, o = divmod(slot, bs)
        for h in range(Hkv):
            k_cache[b, h, kidx[o]] = key[t, h]
            v_cache[b, h, vidx[o]] = value[t, h]


def copy_blocks(k_cache: np.ndarray, v_cache: np.ndarray, pairs: np.ndarray) -> None:
    """Copy whole physical blocks (all kv heads, K and V) src -> dst, in pair order.

    This is the copy a shared block gets before a sequence may modify it
    ([OS] "Copy-on-Write: Sharing KV Cache").
    """
    for src, dst in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):
        k_cache[dst] = k_cache[src]
        v_cache[dst] = v_cache[src]


def swap_blocks(dst_k: np.ndarray, dst_v: np.ndarray, src_k: np.ndarray, src_v: np.ndarray, pairs) -> None:
    """Copy block pairs[i][0] of the source pools into block pairs[i][1] of the
    destination pools (a preempted request's blocks moving to CPU memory and
    back: "PagedAttention: How vLLM Serves AI Like an Operating System",
    section "vLLM Architecture")."""
    for src, dst in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):
        dst_k[dst] = src_k[src]
        dst_v[dst] = src_v[src]


def gather_kv(k_cache, v_cache, table_row, ctx: int, dtype: str, block_size: int = BLOCK_SIZE):
    """Contiguous fp64 K and V of one sequence, [Hkv, ctx, D] each.

    Logical block j of the sequence is physical block table_row[j]; token
    position p is offset p % bs of logical block p // bs.  Only the first
    ceil(ctx / bs) table entries are read.
    """
    NB, Hkv, run = k_cache.shape
    bs = block_size
    D = run // bs
    nb = -(-ctx // bs)
    phys = np.asarray(table_row[:nb], dtype=np.int64)
    kidx = block_index("k", D, bs)
    vidx = block_index("v", D, bs)
    # [nb, Hkv, bs, D] in (logical block, head, token, dim) order
    K = to_f64(k_cache[phys][:, :, kidx], dtype)
    V = to_f64(v_cache[phys][:, :, vidx], dtype)
    K = K.transpose(1, 0, 2, 3).reshape(Hkv, nb * bs, D)[:, :ctx]
    V = V.transpose(1, 0, 2, 3).reshape(Hkv, nb * bs, D)[:, :ctx]
    return K, V


def _softmax_weighted_sum(z: np.ndarray, V: np.ndarray) -> np.ndarray:
    """sum_t softmax(z)_t * V[t], in fp64."""
    e = np.exp(z - z.max())
    return (e / e.sum()) @ V


def decode(q, k_cache, v_cache, block_tables, context_lens, scale: float, dtype: str,
           seqs=None, heads=None) -> np.ndarray:
    """Decode attention for every (sequence, q head): fp64 [S, Hq, D].

    q is [S, Hq, D] storage; output row (s, h) is softmax(scale * q K^T) V over
    the ctx_s tokens of sequence s, with K/V of kv head h // G.  ``seqs`` /
    ``heads`` restrict the rows computed (others stay 0) for sampled checks.
    """
    S, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    bs = k_cache.shape[2] // D
    G = Hq // Hkv
    out = np.zeros((S, Hq, D), dtype=np.float64)
    qf = to_f64(q, dtype)
    for s in (range(S) if seqs is None else seqs):
        n = int(context_lens[s])
        if n == 0:
            continue
        K, V = gather_kv(k_cache, v_cache, block_tables[s], n, dtype, bs)
        for h in (range(Hq) if heads is None else heads):
            g = h // G
            z = scale * (K[g] @ qf[s, h])
            out[s, h] = _softmax_weighted_sum(z, V[g])
    return out


def prefill_chunk(q, k_cache, v_cache, block_tables, context_lens, scale: float, dtype: str,
                  seqs=None, heads=None, rows=None) -> np.ndarray:
    """Causal attention of a C-query chunk over the paged cache: fp64 [S, C, Hq, D].

    q is [S, C, Hq, D]; query i of sequence s sits at position ctx_s - C + i
    and attends keys 0 .. ctx_s - C + i.  ``seqs`` / ``heads`` / ``rows``
    restrict what is computed (others stay 0).
    """
    S, C, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    bs = k_cache.shape[2] // D
    G = Hq // Hkv
    out = np.zeros((S, C, Hq, D), dtype=np.float64)
    for s in (range(S) if seqs is None else seqs):
        n = int(context_lens[s])
        if n < C:
            raise ValueError("the chunk must lie inside the context")
        K, V = gather_kv(k_cache, v_cache, block_tables[s], n, dtype, bs)
        qf = to_f64(q[s], dtype)
        for i in (range(C) if rows is None else rows):
            last = n - C + i
            for h in (range(Hq) if heads is None else heads):
                g = h // G
                z = scale * (K[g, :last + 1] @ qf[i, h])
                out[s, i, h] = _softmax_weighted_sum(z, V[g, :last + 1])
    return out
