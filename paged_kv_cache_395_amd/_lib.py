"""ctypes loader for ``libpa.so`` (the C ABI declared in include/pa.h).

The library must have been built (``python paged_kv_cache_395_amd/build.py``); there is
no fallback of any kind: importing without it raises.
"""

import ctypes
import os
import threading

# PA_LIBRARY may name another build of the same library (the host-sanitized
# build of build.py --sanitize); it must exist like the default one.
LIB_PATH = os.environ.get("PA_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libpa.so")

PA_OK, PA_EINVAL, PA_EUNSUPPORTED, PA_EWORKSPACE, PA_EHIP, PA_ENOSPC, PA_ENOENT = range(7)
PA_F32, PA_F16, PA_BF16 = 0, 1, 2
PA_DECODE_GRID_VECTOR, PA_DECODE_GRID_PARTITIONS, PA_DECODE_GRID_PERSISTENT = 0, 1, 2
STATUS_NAMES = {0: "PA_OK", 1: "PA_EINVAL", 2: "PA_EUNSUPPORTED", 3: "PA_EWORKSPACE", 4: "PA_EHIP",
                5: "PA_ENOSPC", 6: "PA_ENOENT"}


class PAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class NoSpace(PAError):
    """The block manager's pool has fewer free blocks than the operation needs."""


class UnknownSequence(PAError):
    pass


_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_f32 = ctypes.c_float
_sz = ctypes.c_size_t
_pi32 = ctypes.POINTER(ctypes.c_int32)
_pi64 = ctypes.POINTER(ctypes.c_int64)

# name -> (restype, argtypes); mirrors include/pa.h
SIGNATURES = {
    "pa_version": (ctypes.c_char_p, []),
    "pa_last_error": (ctypes.c_char_p, []),
    "pa_reshape_and_cache": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i64, ctypes.c_int, _vp]),
    "pa_append_step": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _vp, _vp, _i32, _i32, _i32,
                                      _i32, _i64, ctypes.c_int, _vp]),
    "pa_append_step_host": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _vp, _vp, _i32, _i32,
                                           _i32, _i32, _i64, ctypes.c_int, _vp]),
    "pa_copy_blocks": (ctypes.c_int, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i64, ctypes.c_int, _vp]),
    "pa_swap_blocks": (ctypes.c_int, [_vp, _vp, _i64, _vp, _vp, _i64, _vp, _i32, _i32, _i32, _i32, ctypes.c_int,
                                      _vp]),
    "pa_patch_tables": (ctypes.c_int, [_vp, _i32, _i32, _vp, _i32, _vp]),
    "pa_decode_partition_size": (_i32, [_i32, _i32, _i32, _i32]),
    "pa_decode_launch_shape": (_i32, [ctypes.c_int, _i32, ctypes.c_int, _i32, _i32, _i32, _i32, _i32, _pi64]),
    "pa_decode_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "pa_decode": (ctypes.c_int, [_vp, ctypes.c_int, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _i32,
                                 _i64, _f32, _i32, _i32, _vp, _sz, ctypes.c_int, _vp]),
    "pa_decode_noalloc_scratch_bytes": (_sz, []),
    "pa_decode_noalloc": (ctypes.c_int, [_vp, ctypes.c_int, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32,
                                         _i32, _i64, _f32, _i32, _i32, ctypes.c_int, _vp]),
    "pa_decode_multi_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "pa_decode_multi": (ctypes.c_int, [_vp, ctypes.c_int, _vp, _i32, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32,
                                       _i32, _i64, _f32, _i32, _i32, _vp, _sz, ctypes.c_int, _vp]),
    "pa_decode_partitions": (ctypes.c_int, [_vp, ctypes.c_int, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32,
                                            _i32, _i64, _f32, _i32, _i32, _vp, _sz, ctypes.c_int, _vp]),
    "pa_decode_reduce": (ctypes.c_int, [_vp, ctypes.c_int, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _sz, _vp]),
    "pa_prefill_chunk": (ctypes.c_int, [_vp, ctypes.c_int, _vp, _i32, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32,
                                        _i32, _i32, _i64, _f32, _i32, ctypes.c_int, _vp]),
    "pa_probe_read_bandwidth": (ctypes.c_int, [_vp, _i64, _vp, _i32, _vp]),
    "pa_probe_gather_bandwidth": (ctypes.c_int, [_vp, _i64, _vp, _i64, _i32, _vp, _i32, _vp]),
    "pa_bm_create": (_vp, [_i64, _i32, _vp]),
    "pa_bm_destroy": (None, [_vp]),
    "pa_bm_add_seq": (ctypes.c_int, [_vp, _i64, _i32]),
    "pa_bm_add_seq_with_prefix": (ctypes.c_int, [_vp, _i64, _i64, _i32, _i32]),
    "pa_bm_fork": (ctypes.c_int, [_vp, _i64, _i64]),
    "pa_bm_free_seq": (ctypes.c_int, [_vp, _i64]),
    "pa_bm_append_tokens": (ctypes.c_int, [_vp, _vp, _i32, _vp, _vp, _pi32]),
    "pa_bm_block_table": (ctypes.c_int, [_vp, _vp, _i32, _i32, _i32, _vp, _vp]),
    "pa_bm_num_free": (_i64, [_vp]),
    "pa_bm_refcount": (_i32, [_vp, _i64]),
    "pa_bm_usage": (ctypes.c_double, [_vp]),
    "pa_bm_num_tokens": (_i32, [_vp, _i64]),
    "pa_bm_free_list": (_i64, [_vp, _vp, _i64]),
    "pa_bm_enable_prefix_cache": (ctypes.c_int, [_vp]),
    "pa_bm_add_seq_tokens": (ctypes.c_int, [_vp, _i64, _vp, _i32, _pi32]),
    "pa_bm_num_cached_free": (_i64, [_vp]),
    "pa_bm_set_host_pool": (ctypes.c_int, [_vp, _i64]),
    "pa_bm_swap_out": (ctypes.c_int, [_vp, _vp, _i32, _vp, _pi32]),
    "pa_bm_swap_in": (ctypes.c_int, [_vp, _vp, _i32, _vp, _pi32]),
    "pa_bm_is_swapped": (_i32, [_vp, _i64]),
    "pa_bm_num_free_host": (_i64, [_vp]),
    "pa_bm_host_refcount": (_i32, [_vp, _i64]),
    "pa_sched_create": (_vp, [_vp, _i32, _i32, _i32]),
    "pa_sched_destroy": (None, [_vp]),
    "pa_sched_submit": (ctypes.c_int, [_vp, _i64, _i32, _i32]),
    "pa_sched_submit_tokens": (ctypes.c_int, [_vp, _i64, _vp, _i32, _i32]),
    "pa_sched_step": (ctypes.c_int, [_vp, _vp]),
}



class SchedOut(ctypes.Structure):
    """pa_sched_out_t."""
    _fields_ = [("num_tokens", _i32), ("slots", _pi64), ("token_rows", _pi32), ("token_positions", _pi32),
                ("num_rows", _i32), ("context_lens", _pi32), ("row_seq", _pi64),
                ("num_swap_out", _i32), ("swap_out_pairs", _pi64), ("num_swap_in", _i32), ("swap_in_pairs", _pi64),
                ("num_cow", _i32), ("cow_pairs", _pi64), ("num_patches", _i32), ("table_patches", _pi32),
                ("num_finished", _i32), ("finished", _pi64),
                ("num_admitted", _i32), ("num_swapped_in", _i32), ("num_preempted_swap", _i32),
                ("num_preempted_recompute", _i32), ("num_running", _i32), ("num_waiting", _i32),
                ("num_swapped", _i32), ("num_cached_tokens", _i32)]


_lock = threading.Lock()
_lib = None


def load() -> ctypes.CDLL:
    """Load libpa.so once; raise if it has not been built.

    A process must hold a single HIP runtime.  torch ships its own
    libamdhip64 and loads it by path; when libpa.so is loaded first it pulls
    the system copy through its run path and the two runtimes conflict (the
    second reports no device).  Importing torch first makes libpa.so bind to
    the runtime torch already loaded.
    """
    global _lib
    with _lock:
        if _lib is None:
            try:
                import torch  # noqa: F401
            except ImportError:  # host-only use (block manager) without torch
                pass
            if not os.path.exists(LIB_PATH):
                raise ImportError(f"{LIB_PATH} is missing: build it with `python paged_kv_cache_395_amd/build.py`")
            lib = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(lib, name)
                fn.restype = res
                fn.argtypes = args
            _lib = lib
    return _lib


def check(status: int) -> None:
    if status != PA_OK:
        msg = load().pa_last_error().decode(errors="replace")
        if status == PA_ENOSPC:
            raise NoSpace(status, msg)
        if status == PA_ENOENT:
            raise UnknownSequence(status, msg)
        raise PAError(status, msg)
