"""Element order inside one (physical block, kv head) tile of the KV pools.

The pages fix only that the cache is cut into fixed blocks of 16 tokens that
may sit anywhere in memory ("PagedAttention: How vLLM Serves AI Like an
Operating System", section "PagedAttention: Virtual Memory for KV Cache").
How the 16 x D values of one block and head are ordered is not on the pages;
this is the reading the library's interface states, written out as index
formulas.  A pool is ``[num_blocks][num_kv_heads][16 * D]``; inside a tile:

K tile  element (token t, dim d) sits at  ((d // 8) * 16 + t) * 8 + d % 8
        i.e. [D/8][16 tokens][8 dims]

V tile  element (token t, dim d) sits at
        (((d // 32) * 4 + t // 4) * 16 + d % 16) * 8 + ((d // 16) % 2) * 4 + t % 4
        i.e. [D/32][4 token quads][16 dims][2 dim halves][4 tokens]

D must be a multiple of 32.

Blocks of 32 or 64 tokens (variants; the pages fix 16): the (block, kv head)
run of bs * D elements is bs / 16 such tiles one after another, token t of
the block in tile t // 16 at token t % 16.
"""

import numpy as np

BLOCK_SIZE = 16


def k_offset(t: int, d: int) -> int:
    """Position of K[token t][dim d] inside a K tile."""
    return ((d // 8) * 16 + t) * 8 + d % 8


def v_offset(t: int, d: int) -> int:
    """Position of V[token t][dim d] inside a V tile."""
    return (((d // 32) * 4 + t // 4) * 16 + d % 16) * 8 + ((d // 16) % 2) * 4 + t % 4


def tile_index(which: str, head_dim: int) -> np.ndarray:
    """[16, D] int64 array: tile position of every (token, dim), by the formulas above."""
    if head_dim % 32:
        raise ValueError("head_dim must be a multiple of 32")
    f = k_offset if which == "k" else v_offset
    idx = np.empty((BLOCK_SIZE, head_dim), dtype=np.int64)
    for t in range(BLOCK_SIZE):
        for d in range(head_dim):
            idx[t, d] = f(t, d)
    return idx


def block_index(which: str, head_dim: int, block_size: int = BLOCK_SIZE) -> np.ndarray:
    """[block_size, D] int64 array: position of every (token, dim) inside one
    (block, kv head) run of block_size * D elements."""
    if block_size % BLOCK_SIZE:
        raise ValueError("block_size must be a multiple of 16")
    tile = tile_index(which, head_dim)
    idx = np.empty((block_size, head_dim), dtype=np.int64)
    for t in range(block_size):
        idx[t] = (t // BLOCK_SIZE) * BLOCK_SIZE * head_dim + tile[t % BLOCK_SIZE]
    return idx
