"""Continuous-batching attention driver: the native scheduler's steps run on
the device kernels over fixed buffers.

Each step has a host half (``schedule``: the scheduler picks the batch,
allocates slots, preempts and brings back requests) and a device half
(``launch``): swap-out copies into the pinned host pool (on a second stream,
beside the previous step's decode), then on the main stream swap-in copies
back, copy-on-write, table patches, the cache write that also patches the
device-resident tables and lengths, and decode over every batch row.  Between the two halves the caller fills ``key[:T]``, ``value[:T]``
(the step's new K/V rows, in the order of ``Step.slots``) and ``q`` (one
query per row).  Every computation runs in libpa's kernels; this module only
stages metadata and marshals arguments.

Pages: "PagedAttention: How vLLM Serves AI Like an Operating System",
sections "Continuous Batching: The Other Half" and "vLLM Architecture"; the
scheduling rules are the ones include/pa.h documents for pa_sched_step.
"""

import ctypes

import numpy as np
import torch

from . import _lib
from .block_manager import BlockManager
from .ops import _code, _p
from .scheduler import Scheduler

_TORCH = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


class _DeviceEvent:
    """A HIP event that only other streams wait on, created through the HIP
    runtime torch loaded with hipEventDisableSystemFence | hipEventDisableTiming.
    torch's events release to system scope at every record (an L2 write-back
    and invalidate) so the host may read them; a stream-to-stream dependency
    does not need that."""

    _hip = None
    _FLAGS = 0x20000000 | 0x2  # hipEventDisableSystemFence | hipEventDisableTiming

    def __init__(self):
        if _DeviceEvent._hip is None:
            import os

            lib = ctypes.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
            lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            lib.hipStreamWaitEvent.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint]
            lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
            _DeviceEvent._hip = lib
        self._h = ctypes.c_void_p()
        self._check(_DeviceEvent._hip.hipEventCreateWithFlags(ctypes.byref(self._h), self._FLAGS),
                    "hipEventCreateWithFlags")

    @staticmethod
    def _check(rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed with HIP error {rc}")

    def record(self, stream: ctypes.c_void_p) -> None:
        self._check(_DeviceEvent._hip.hipEventRecord(self._h, stream), "hipEventRecord")

    def make_wait(self, stream: ctypes.c_void_p) -> None:
        """Work enqueued on ``stream`` from now on waits for the last record."""
        self._check(_DeviceEvent._hip.hipStreamWaitEvent(stream, self._h, 0), "hipStreamWaitEvent")

    def __del__(self):
        if self._h and _DeviceEvent._hip is not None:
            _DeviceEvent._hip.hipEventDestroy(self._h)


class Driver:
    def __init__(self, num_blocks, num_host_blocks, num_q_heads, num_kv_heads, head_dim, dtype, max_rows,
                 max_blocks_per_seq, max_batched_tokens, scale, free_order=None, device="cuda", ring=8,
                 partition_size=0, prefix_cache=False, block_size=16):
        self._l = _lib.load()
        self.dtype = dtype
        tdt = _TORCH[dtype]
        dev = torch.device(device)
        self.NB, self.NH = int(num_blocks), int(num_host_blocks)
        self.Hq, self.Hkv, self.D = num_q_heads, num_kv_heads, head_dim
        self.rows, self.maxB = int(max_rows), int(max_blocks_per_seq)
        self.scale = float(scale)
        self.partition = int(partition_size)
        self.bs = int(block_size)
        self.bm = BlockManager(num_blocks, block_size=block_size, free_order=free_order)
        if prefix_cache:
            self.bm.enable_prefix_cache()
        self.bm.set_host_pool(num_host_blocks)
        self.sched = Scheduler(self.bm, max_rows, max_blocks_per_seq, max_batched_tokens)
        tile = self.bs * head_dim
        self.k_pool = torch.zeros((num_blocks, num_kv_heads, tile), dtype=tdt, device=dev)
        self.v_pool = torch.zeros_like(self.k_pool)
        nh = max(self.NH, 1)
        self.k_host = torch.zeros((nh, num_kv_heads, tile), dtype=tdt).pin_memory()
        self.v_host = torch.zeros_like(self.k_host).pin_memory()
        # tables and lengths stay on the device; unused entries point outside the pool
        self.table = torch.full((max_rows, max_blocks_per_seq), num_blocks, dtype=torch.int32, device=dev)
        self.ctx = torch.zeros(max_rows, dtype=torch.int32, device=dev)
        # the first admission of a step may exceed the token budget by one whole request
        self.cap = max_rows + max_batched_tokens + max_blocks_per_seq * self.bs
        self.key = torch.zeros((self.cap, num_kv_heads, head_dim), dtype=tdt, device=dev)
        self.value = torch.zeros_like(self.key)
        self.q = torch.zeros((max_rows, num_q_heads, head_dim), dtype=tdt, device=dev)
        self.out = torch.zeros((max_rows, num_q_heads, head_dim), dtype=torch.float32, device=dev)
        max_ctx = max_blocks_per_seq * self.bs
        ws = max(int(self._l.pa_decode_workspace_bytes(max_rows, num_q_heads, num_kv_heads, head_dim, c,
                                                       self.partition)) for c in range(1, max_ctx + 1))
        self.workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=dev)
        self.stream = torch.cuda.current_stream(dev)
        self._s = ctypes.c_void_p(self.stream.cuda_stream)
        # swap-outs run on a second stream (default priority) beside the previous step's decode
        self.swap_stream = torch.cuda.Stream(dev)
        self._ss = ctypes.c_void_p(self.swap_stream.cuda_stream)
        # recorded on the main stream after every step's cache write; a swap-out waits for it
        self._after_append = _DeviceEvent()
        self._appended = False
        # pinned staging, one set per in-flight step, in two groups: one
        # host-visible completion event per group, recorded after its last
        # set's launch and waited for before its first set is refilled (each
        # record of such an event costs the step a system-scope fence)
        pair_cap = 2 * max(num_blocks, nh)
        self._groups = 2 if ring >= 4 else ring
        self._group_done = [torch.cuda.Event() for _ in range(self._groups)]
        self._group_used = [False] * self._groups
        self._ring = []
        for _ in range(ring):
            self._ring.append({
                "slots": torch.empty(self.cap, dtype=torch.int64).pin_memory(),
                "rows": torch.empty(self.cap, dtype=torch.int32).pin_memory(),
                "pos": torch.empty(self.cap, dtype=torch.int32).pin_memory(),
                "ctx": torch.empty(max_rows, dtype=torch.int32).pin_memory(),
                "out_pairs": torch.empty((pair_cap, 2), dtype=torch.int64).pin_memory(),
                "in_pairs": torch.empty((pair_cap, 2), dtype=torch.int64).pin_memory(),
                "cow": torch.empty((max_rows, 2), dtype=torch.int64).pin_memory(),
                "patches": torch.empty((max_rows * max_blocks_per_seq, 3), dtype=torch.int32).pin_memory(),
            })
        self._i = 0
        self._code = _code(self.k_pool)
        self.steps = 0

    def _group_of(self, i: int) -> int:
        return i * self._groups // len(self._ring)

    # -- host half -------------------------------------------------------------
    def submit(self, seq: int, prompt_tokens: int, total_tokens: int, prompt_ids=None) -> None:
        self.sched.submit(seq, prompt_tokens, total_tokens, prompt_ids)

    def schedule(self):
        """Run the scheduler for one step and stage its metadata; returns the Step."""
        st = self.sched.step()
        T = len(st.slots)
        if T > self.cap:
            raise RuntimeError(f"step writes {T} tokens, more than the staging capacity {self.cap}")
        i = self._i % len(self._ring)
        r = self._ring[i]
        g = self._group_of(i)
        if self._group_used[g] and i * self._groups % len(self._ring) == 0:
            self._group_done[g].synchronize()  # the launches that last read this group's sets have run
        r["slots"].numpy()[:T] = st.slots
        r["rows"].numpy()[:T] = st.token_rows
        r["pos"].numpy()[:T] = st.token_positions
        r["ctx"].numpy()[:] = st.context_lens
        r["out_pairs"].numpy()[: len(st.swap_out)] = st.swap_out
        r["in_pairs"].numpy()[: len(st.swap_in)] = st.swap_in
        r["cow"].numpy()[: len(st.cow)] = st.cow
        r["patches"].numpy()[: len(st.patches)] = st.patches
        return st

    # -- device half -----------------------------------------------------------
    def launch(self, st, decode_events=None) -> None:
        """Enqueue the step's device work on the driver's stream (``decode_events``:
        an optional pair of events recorded around the decode launch)."""
        L, s, code = self._l, self._s, self._code
        r = self._ring[self._i % len(self._ring)]
        Hkv, D, NB, NH = self.Hkv, self.D, self.NB, max(self.NH, 1)
        if len(st.swap_out):
            # A preempted request ran in the last step: its blocks are final once that step's cache
            # write is done, and the last step's decode only reads them, so the copy to host memory
            # starts there, beside that decode.  This step's work waits for it: the freed blocks may
            # take this step's writes.  Host blocks it fills were released by swap-ins of earlier
            # steps, which ran before that cache write.
            if self._appended:
                self._after_append.make_wait(self._ss)
            _lib.check(L.pa_swap_blocks(_p(self.k_host), _p(self.v_host), NH, _p(self.k_pool), _p(self.v_pool), NB,
                                        _p(r["out_pairs"]), len(st.swap_out), Hkv, D, self.bs, code, self._ss))
            swapped = torch.cuda.Event()
            swapped.record(self.swap_stream)
            self.stream.wait_event(swapped)
        if len(st.swap_in):
            _lib.check(L.pa_swap_blocks(_p(self.k_pool), _p(self.v_pool), NB, _p(self.k_host), _p(self.v_host), NH,
                                        _p(r["in_pairs"]), len(st.swap_in), Hkv, D, self.bs, code, s))
        if len(st.cow):
            _lib.check(L.pa_copy_blocks(_p(self.k_pool), _p(self.v_pool), _p(r["cow"]), len(st.cow), Hkv, D,
                                        self.bs, NB, code, s))
        if len(st.patches):
            _lib.check(L.pa_patch_tables(_p(self.table), self.maxB, self.rows, _p(r["patches"]), len(st.patches), s))
        _lib.check(L.pa_append_step(_p(self.key), _p(self.value), _p(self.k_pool), _p(self.v_pool), _p(r["slots"]),
                                    _p(r["rows"]), _p(r["pos"]), len(st.slots), _p(self.table), self.maxB,
                                    _p(self.ctx), _p(r["ctx"]), self.rows, Hkv, D, self.bs, NB, code, s))
        i = self._i % len(self._ring)
        if i + 1 == len(self._ring) or self._group_of(i + 1) != self._group_of(i):  # the group's last set
            g = self._group_of(i)
            self._group_done[g].record(self.stream)  # also after the swap-out: the stream waited for it
            self._group_used[g] = True
        self._after_append.record(self._s)
        self._appended = True
        self._i += 1
        # with every row empty the kernel still runs and writes zero rows
        max_ctx = max(int(st.context_lens.max()), 1)
        if decode_events is not None:
            decode_events[0].record(self.stream)
        _lib.check(L.pa_decode(_p(self.out), _lib.PA_F32, _p(self.q), _p(self.k_pool), _p(self.v_pool),
                               _p(self.table), self.maxB, _p(self.ctx), self.rows, self.Hq, Hkv, D, self.bs, NB,
                               self.scale, max_ctx, self.partition, _p(self.workspace), self.workspace.numel(),
                               code, s))
        if decode_events is not None:
            decode_events[1].record(self.stream)
        self.steps += 1

    def step(self):
        st = self.schedule()
        self.launch(st)
        return st
