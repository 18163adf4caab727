"""Python face of the native continuous-batching scheduler (``pa_sched_*``).

The policy lives in C++ (include/pa.h documents it); this class marshals
arguments and copies each step's outputs into numpy arrays.
"""

import ctypes
from dataclasses import dataclass

import numpy as np

from . import _lib


def _arr(ptr, n, dtype, shape=None):
    if n == 0:
        return np.zeros((0,) if shape is None else (0,) + shape[1:], dtype=dtype)
    a = np.ctypeslib.as_array(ptr, shape=(n * (1 if shape is None else int(np.prod(shape[1:]))),)).copy()
    return a.astype(dtype, copy=False) if shape is None else a.astype(dtype, copy=False).reshape((n,) + shape[1:])


@dataclass
class Step:
    slots: np.ndarray            # int64 [T]
    token_rows: np.ndarray       # int32 [T]
    token_positions: np.ndarray  # int32 [T]
    context_lens: np.ndarray     # int32 [rows]
    row_seq: np.ndarray          # int64 [rows], -1 = empty
    swap_out: np.ndarray         # int64 [k, 2] (device, host)
    swap_in: np.ndarray          # int64 [k, 2] (host, device)
    cow: np.ndarray              # int64 [k, 2] (src, dst)
    patches: np.ndarray          # int32 [k, 3] (row, logical, physical)
    finished: np.ndarray         # int64 [k]
    num_admitted: int
    num_swapped_in: int
    num_preempted_swap: int
    num_preempted_recompute: int
    num_running: int
    num_waiting: int
    num_swapped: int
    num_cached_tokens: int

    @property
    def idle(self) -> bool:
        return self.num_running == 0 and self.num_waiting == 0 and self.num_swapped == 0


class Scheduler:
    """Continuous batching over ``max_rows`` batch rows of a BlockManager."""

    def __init__(self, bm, max_rows: int, max_blocks_per_seq: int, max_batched_tokens: int):
        self._l = _lib.load()
        self.bm = bm  # kept alive: the scheduler points at it
        h = self._l.pa_sched_create(bm._h, int(max_rows), int(max_blocks_per_seq), int(max_batched_tokens))
        if not h:
            raise _lib.PAError(_lib.PA_EINVAL, self._l.pa_last_error().decode())
        self._h = ctypes.c_void_p(h)
        self.max_rows = int(max_rows)
        self._out = _lib.SchedOut()

    def close(self) -> None:
        if getattr(self, "_h", None):
            self._l.pa_sched_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # interpreter shutdown
            pass

    def submit(self, seq: int, prompt_tokens: int, total_tokens: int, prompt_ids=None) -> None:
        """Queue a request; with ``prompt_ids`` (and prefix caching on) admission reuses cached prefix blocks."""
        if prompt_ids is None:
            _lib.check(self._l.pa_sched_submit(self._h, int(seq), int(prompt_tokens), int(total_tokens)))
            return
        ids = np.ascontiguousarray(prompt_ids, dtype=np.int32)
        if ids.shape != (int(prompt_tokens),):
            raise ValueError("prompt_ids must hold prompt_tokens ids")
        _lib.check(self._l.pa_sched_submit_tokens(self._h, int(seq), ids.ctypes.data_as(ctypes.c_void_p),
                                                  int(prompt_tokens), int(total_tokens)))

    def step(self) -> Step:
        o = self._out
        _lib.check(self._l.pa_sched_step(self._h, ctypes.byref(o)))
        return Step(
            slots=_arr(o.slots, o.num_tokens, np.int64),
            token_rows=_arr(o.token_rows, o.num_tokens, np.int32),
            token_positions=_arr(o.token_positions, o.num_tokens, np.int32),
            context_lens=_arr(o.context_lens, o.num_rows, np.int32),
            row_seq=_arr(o.row_seq, o.num_rows, np.int64),
            swap_out=_arr(o.swap_out_pairs, o.num_swap_out, np.int64, (0, 2)),
            swap_in=_arr(o.swap_in_pairs, o.num_swap_in, np.int64, (0, 2)),
            cow=_arr(o.cow_pairs, o.num_cow, np.int64, (0, 2)),
            patches=_arr(o.table_patches, o.num_patches, np.int32, (0, 3)),
            finished=_arr(o.finished, o.num_finished, np.int64),
            num_admitted=o.num_admitted, num_swapped_in=o.num_swapped_in,
            num_preempted_swap=o.num_preempted_swap, num_preempted_recompute=o.num_preempted_recompute,
            num_running=o.num_running, num_waiting=o.num_waiting, num_swapped=o.num_swapped,
            num_cached_tokens=o.num_cached_tokens)
