"""Python face of the native host block manager (``pa_bm_*``).

All state lives in C++; this class only marshals arguments.  Sequence ids are
64-bit integers.
"""

import ctypes

import numpy as np

from . import _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


class BlockManager:
    """Pool of ``num_blocks`` blocks of ``block_size`` (16, 32 or 64) tokens with
    a free list, reference counts and copy-on-write (see include/pa.h for the
    exact rules)."""

    def __init__(self, num_blocks: int, block_size: int = 16, free_order=None):
        self._l = _lib.load()
        order = None
        if free_order is not None:
            order = np.ascontiguousarray(free_order, dtype=np.int32)
            if order.shape != (num_blocks,):
                raise ValueError("free_order must list every block once")
        h = self._l.pa_bm_create(int(num_blocks), int(block_size), None if order is None else _ptr(order))
        if not h:
            raise _lib.PAError(_lib.PA_EINVAL, self._l.pa_last_error().decode())
        self._h = ctypes.c_void_p(h)
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)

    def close(self) -> None:
        if getattr(self, "_h", None):
            self._l.pa_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # interpreter shutdown
            pass

    # -- updates -------------------------------------------------------------
    def add_seq(self, seq: int, num_tokens: int) -> None:
        _lib.check(self._l.pa_bm_add_seq(self._h, int(seq), int(num_tokens)))

    def add_seq_with_prefix(self, seq: int, prefix_seq: int, prefix_tokens: int, tail_tokens: int) -> None:
        _lib.check(self._l.pa_bm_add_seq_with_prefix(self._h, int(seq), int(prefix_seq), int(prefix_tokens),
                                                     int(tail_tokens)))

    def fork(self, parent: int, child: int) -> None:
        _lib.check(self._l.pa_bm_fork(self._h, int(parent), int(child)))

    def free_seq(self, seq: int) -> None:
        _lib.check(self._l.pa_bm_free_seq(self._h, int(seq)))

    def append_tokens(self, seqs, slots_out: np.ndarray = None, cow_out: np.ndarray = None):
        """One token for each listed sequence, in order.  Returns (slots int64 [n], cow pairs int64 [k, 2])."""
        seqs = np.ascontiguousarray(seqs, dtype=np.int64)
        n = seqs.shape[0]
        slots = np.empty(n, dtype=np.int64) if slots_out is None else slots_out
        cow = np.empty((max(n, 1), 2), dtype=np.int64) if cow_out is None else cow_out
        ncow = ctypes.c_int32(0)
        _lib.check(self._l.pa_bm_append_tokens(self._h, _ptr(seqs), n, _ptr(slots), _ptr(cow), ctypes.byref(ncow)))
        return slots[:n], cow[: ncow.value]

    def append_token(self, seq: int):
        slots, cow = self.append_tokens([seq])
        return int(slots[0]), (tuple(int(x) for x in cow[0]) if len(cow) else (-1, -1))

    # -- prefix cache ----------------------------------------------------------
    def enable_prefix_cache(self) -> None:
        _lib.check(self._l.pa_bm_enable_prefix_cache(self._h))

    def add_seq_tokens(self, seq: int, tokens) -> int:
        """New sequence from its token ids; returns how many leading tokens were already cached."""
        tokens = np.ascontiguousarray(tokens, dtype=np.int32)
        cached = ctypes.c_int32(0)
        _lib.check(self._l.pa_bm_add_seq_tokens(self._h, int(seq), _ptr(tokens), tokens.shape[0],
                                                ctypes.byref(cached)))
        return cached.value

    def num_cached_free(self) -> int:
        return int(self._l.pa_bm_num_cached_free(self._h))

    # -- swap pool -----------------------------------------------------------
    def set_host_pool(self, num_host_blocks: int) -> None:
        _lib.check(self._l.pa_bm_set_host_pool(self._h, int(num_host_blocks)))

    def _swap(self, fn, seqs):
        seqs = np.ascontiguousarray(seqs, dtype=np.int64)
        total = sum(-(-max(self.num_tokens(int(s)), 0) // self.block_size) for s in seqs)
        pairs = np.empty((max(total, 1), 2), dtype=np.int64)
        n = ctypes.c_int32(0)
        _lib.check(fn(self._h, _ptr(seqs), seqs.shape[0], _ptr(pairs), ctypes.byref(n)))
        return pairs[: n.value]

    def swap_out(self, seqs):
        """Move the sequences' blocks to the host pool; returns (device, host) copies int64 [k, 2]."""
        return self._swap(self._l.pa_bm_swap_out, seqs)

    def swap_in(self, seqs):
        """Bring swapped-out sequences back into fresh blocks; returns (host, device) copies int64 [k, 2]."""
        return self._swap(self._l.pa_bm_swap_in, seqs)

    def is_swapped(self, seq: int) -> bool:
        r = int(self._l.pa_bm_is_swapped(self._h, int(seq)))
        if r < 0:
            raise _lib.UnknownSequence(_lib.PA_ENOENT, f"unknown sequence {seq}")
        return bool(r)

    def num_free_host(self) -> int:
        return int(self._l.pa_bm_num_free_host(self._h))

    def host_refcount(self, block: int) -> int:
        return int(self._l.pa_bm_host_refcount(self._h, int(block)))

    # -- queries -------------------------------------------------------------
    def block_table(self, seqs, max_blocks: int, pad: int = -1, table_out: np.ndarray = None,
                    ctx_out: np.ndarray = None):
        seqs = np.ascontiguousarray(seqs, dtype=np.int64)
        n = seqs.shape[0]
        table = np.empty((n, max_blocks), dtype=np.int32) if table_out is None else table_out
        ctx = np.empty(n, dtype=np.int32) if ctx_out is None else ctx_out
        _lib.check(self._l.pa_bm_block_table(self._h, _ptr(seqs), n, int(max_blocks), int(pad), _ptr(table), _ptr(ctx)))
        return table, ctx

    def num_free(self) -> int:
        return int(self._l.pa_bm_num_free(self._h))

    def refcount(self, block: int) -> int:
        return int(self._l.pa_bm_refcount(self._h, int(block)))

    def usage(self) -> float:
        return float(self._l.pa_bm_usage(self._h))

    def num_tokens(self, seq: int) -> int:
        return int(self._l.pa_bm_num_tokens(self._h, int(seq)))

    def free_list(self) -> list:
        n = int(self._l.pa_bm_free_list(self._h, None, 0))
        out = np.empty(max(n, 1), dtype=np.int32)
        self._l.pa_bm_free_list(self._h, _ptr(out), n)
        return out[:n].tolist()

    def blocks_of(self, seq: int) -> list:
        n = self.num_tokens(seq)
        if n < 0:
            raise _lib.UnknownSequence(_lib.PA_ENOENT, f"unknown sequence {seq}")
        nb = -(-n // self.block_size)
        table, _ = self.block_table([seq], max(nb, 1))
        return table[0, :nb].tolist()
