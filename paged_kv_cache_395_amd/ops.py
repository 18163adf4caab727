"""torch-tensor wrappers over the device entry points of libpa.so.

Argument marshalling only: each function checks shapes / dtypes / devices,
takes raw device pointers and the current HIP stream, and calls the C ABI.
All computation happens in the library's gfx950 kernels.
"""

import ctypes

import torch

from . import _lib

_DTYPE = {torch.float32: _lib.PA_F32, torch.float16: _lib.PA_F16, torch.bfloat16: _lib.PA_BF16}
BLOCK_SIZE = 16


def _code(t: torch.Tensor) -> int:
    try:
        return _DTYPE[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}") from None


def _dev(*ts):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("all tensors must live on the GPU")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")


def _stream(stream=None) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _p(t: torch.Tensor) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr())


BLOCK_SIZES = (16, 32, 64)


def _pool_dims(k_cache: torch.Tensor, head_dim: int = None):
    """(num_blocks, num_kv_heads, head_dim, block_size) of a pool
    [num_blocks, num_kv_heads, block_size * head_dim].  Without ``head_dim``
    (whole-block copies, where only the block's bytes matter) the first block
    size that leaves a supported head_dim is taken."""
    if k_cache.dim() != 3:
        raise ValueError("pools are [num_blocks, num_kv_heads, block_size * head_dim]")
    run = k_cache.shape[2]
    if head_dim is not None:
        if run % head_dim or run // head_dim not in BLOCK_SIZES:
            raise ValueError(f"pool rows of {run} elements do not hold 16, 32 or 64 tokens of head_dim {head_dim}")
        return k_cache.shape[0], k_cache.shape[1], head_dim, run // head_dim
    for bs in BLOCK_SIZES:
        if run % bs == 0 and run // bs in (64, 128):
            return k_cache.shape[0], k_cache.shape[1], run // bs, bs
    raise ValueError("pools are [num_blocks, num_kv_heads, block_size * head_dim]")


def _pools(k_cache: torch.Tensor, v_cache: torch.Tensor, head_dim: int = None):
    """Dimensions of a K / V pool pair; the two must have one shape and dtype
    (the kernels address both with the K pool's geometry)."""
    if v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype:
        raise ValueError("k_cache and v_cache must have the same shape and dtype")
    return _pool_dims(k_cache, head_dim)


def reshape_and_cache(key, value, k_cache, v_cache, slot_mapping, stream=None) -> None:
    """Write key/value [T, Hkv, D] into their slots (int64 [T]) of the pools."""
    _dev(key, value, k_cache, v_cache, slot_mapping)
    NB, Hkv, D, bs = _pools(k_cache, v_cache, key.shape[-1])
    if key.shape != value.shape or key.dim() != 3 or key.shape[1:] != (Hkv, D):
        raise ValueError("key / value must be [T, num_kv_heads, head_dim]")
    if slot_mapping.dtype != torch.int64 or slot_mapping.shape != (key.shape[0],):
        raise ValueError("slot_mapping must be int64 [T]")
    if not (key.dtype == value.dtype == k_cache.dtype == v_cache.dtype):
        raise TypeError("key, value and the pools must share one dtype")
    _lib.check(_lib.load().pa_reshape_and_cache(_p(key), _p(value), _p(k_cache), _p(v_cache), _p(slot_mapping),
                                                key.shape[0], Hkv, D, bs, NB, _code(k_cache),
                                                _stream(stream)))


def _dev_or_pinned(*ts):
    for t in ts:
        if not (t.is_cuda or t.is_pinned()):
            raise ValueError("step metadata must live on the GPU or in pinned host memory")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")


def _host(*ts):
    for t in ts:
        if t.is_cuda:
            raise ValueError("step metadata of append_step_host must live in host memory")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")


def _append_args(key, value, k_cache, v_cache, slot_mapping, token_rows, token_positions, block_tables,
                 context_lens, new_context_lens, stream, host_meta=False):
    _dev(key, value, k_cache, v_cache, block_tables, context_lens)
    (_host if host_meta else _dev_or_pinned)(slot_mapping, token_rows, token_positions, new_context_lens)
    NB, Hkv, D, bs = _pools(k_cache, v_cache, key.shape[-1])
    if key.shape != value.shape or key.dim() != 3 or key.shape[1:] != (Hkv, D):
        raise ValueError("key / value must be [T, num_kv_heads, head_dim]")
    T = key.shape[0]
    if slot_mapping.dtype != torch.int64 or slot_mapping.shape != (T,):
        raise ValueError("slot_mapping must be int64 [T]")
    for t in (token_rows, token_positions):
        if t.dtype != torch.int32 or t.shape != (T,):
            raise ValueError("token_rows / token_positions must be int32 [T]")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2:
        raise ValueError("block_tables must be int32 [num_seqs, max_blocks]")
    S = block_tables.shape[0]
    for t in (context_lens, new_context_lens):
        if t.dtype != torch.int32 or t.shape != (S,):
            raise ValueError("context_lens / new_context_lens must be int32 [num_seqs]")
    if not (key.dtype == value.dtype == k_cache.dtype == v_cache.dtype):
        raise TypeError("key, value and the pools must share one dtype")
    return (_p(key), _p(value), _p(k_cache), _p(v_cache), _p(slot_mapping), _p(token_rows), _p(token_positions), T,
            _p(block_tables), block_tables.shape[1], _p(context_lens), _p(new_context_lens), S, Hkv, D, bs,
            NB, _code(k_cache), _stream(stream))


def append_step(key, value, k_cache, v_cache, slot_mapping, token_rows, token_positions, block_tables, context_lens,
                new_context_lens, stream=None) -> None:
    """Cache write plus in-place update of device-resident tables and lengths.

    Token t goes to slot ``slot_mapping[t]``; ``block_tables[token_rows[t]]
    [token_positions[t] // block_size]`` becomes ``slot_mapping[t] // block_size``; then
    ``context_lens`` takes ``new_context_lens``.  The four step vectors may be
    device tensors or pinned host tensors.
    """
    _lib.check(_lib.load().pa_append_step(*_append_args(key, value, k_cache, v_cache, slot_mapping, token_rows,
                                                        token_positions, block_tables, context_lens,
                                                        new_context_lens, stream)))


def append_step_host(key, value, k_cache, v_cache, slot_mapping, token_rows, token_positions, block_tables,
                     context_lens, new_context_lens, stream=None) -> None:
    """append_step with the four step vectors in host memory (CPU tensors, pinned or not).

    Their values are copied into the launch's kernel arguments before the call
    returns (the caller may overwrite them at once), so the kernel reads
    nothing from host memory.
    """
    _lib.check(_lib.load().pa_append_step_host(*_append_args(key, value, k_cache, v_cache, slot_mapping, token_rows,
                                                             token_positions, block_tables, context_lens,
                                                             new_context_lens, stream, host_meta=True)))


def copy_blocks(k_cache, v_cache, pairs, stream=None) -> None:
    """Copy physical blocks src -> dst for each row (src, dst) of int64 ``pairs`` [n, 2]."""
    _dev(k_cache, v_cache, pairs)
    NB, Hkv, D, bs = _pools(k_cache, v_cache)
    if pairs.dtype != torch.int64 or pairs.dim() != 2 or pairs.shape[1] != 2:
        raise ValueError("pairs must be int64 [n, 2]")
    _lib.check(_lib.load().pa_copy_blocks(_p(k_cache), _p(v_cache), _p(pairs), pairs.shape[0], Hkv, D, bs,
                                          NB, _code(k_cache), _stream(stream)))


def swap_blocks(dst_k, dst_v, src_k, src_v, pairs, stream=None) -> None:
    """Copy block pairs[i, 0] of the source pools into block pairs[i, 1] of the
    destination pools; one side may be pinned host memory (a swap)."""
    for t in (dst_k, dst_v, src_k, src_v, pairs):
        if not (t.is_cuda or t.is_pinned()):
            raise ValueError("pools and pairs must live on the GPU or in pinned host memory")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    NBd, Hkv, D, bs = _pool_dims(dst_k)
    NBs, Hkv_s, D_s, bs_s = _pool_dims(src_k)
    if (Hkv_s, D_s, bs_s) != (Hkv, D, bs) or dst_v.shape != dst_k.shape or src_v.shape != src_k.shape:
        raise ValueError("both sides must be pools of the same geometry")
    if not (dst_k.dtype == dst_v.dtype == src_k.dtype == src_v.dtype):
        raise TypeError("the pools must share one dtype")
    if pairs.dtype != torch.int64 or pairs.dim() != 2 or pairs.shape[1] != 2:
        raise ValueError("pairs must be int64 [n, 2]")
    _lib.check(_lib.load().pa_swap_blocks(_p(dst_k), _p(dst_v), NBd, _p(src_k), _p(src_v), NBs, _p(pairs),
                                          pairs.shape[0], Hkv, D, bs, _code(dst_k), _stream(stream)))


def patch_tables(block_tables, patches, stream=None) -> None:
    """block_tables[row, idx] = block for each (row, idx, block) row of int32 ``patches``."""
    _dev(block_tables)
    _dev_or_pinned(patches)
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2:
        raise ValueError("block_tables must be int32 [num_seqs, max_blocks]")
    if patches.dtype != torch.int32 or patches.dim() != 2 or patches.shape[1] != 3:
        raise ValueError("patches must be int32 [n, 3]")
    _lib.check(_lib.load().pa_patch_tables(_p(block_tables), block_tables.shape[1], block_tables.shape[0],
                                           _p(patches), patches.shape[0], _stream(stream)))


def decode_partition_size(num_seqs: int, num_kv_heads: int, max_context_len: int, partition_size: int = 0) -> int:
    """Tokens per context partition decode uses for these sizes (0 = the library's choice)."""
    return int(_lib.load().pa_decode_partition_size(num_seqs, num_kv_heads, max_context_len, partition_size))


DECODE_KERNELS = {_lib.PA_DECODE_GRID_VECTOR: "decode_f32_kernel",
                  _lib.PA_DECODE_GRID_PARTITIONS: "decode_partition_kernel",
                  _lib.PA_DECODE_GRID_PERSISTENT: "decode_persistent_kernel"}


def decode_launch_shape(dtype: torch.dtype, head_dim: int, out_dtype: torch.dtype, num_seqs: int, num_q_heads: int,
                        num_kv_heads: int, max_context_len: int, partition_size: int = 0):
    """(kernel name, workgroups) of decode's partition launch for these sizes on the current device."""
    n = ctypes.c_int64(0)
    shape = _lib.load().pa_decode_launch_shape(_DTYPE[dtype], head_dim, _DTYPE[out_dtype], num_seqs, num_q_heads,
                                               num_kv_heads, max_context_len, partition_size, ctypes.byref(n))
    if shape < 0:
        raise ValueError("invalid decode sizes")
    return DECODE_KERNELS[shape], int(n.value)


def decode_workspace_bytes(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int, max_context_len: int,
                           partition_size: int = 0) -> int:
    return int(_lib.load().pa_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                                                     partition_size))


def _decode_args(out, q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len, partition_size,
                 workspace, allocate=True):
    _dev(out, q, k_cache, v_cache, block_tables, context_lens)
    NB, Hkv, D, bs = _pools(k_cache, v_cache, q.shape[-1])
    if q.dim() != 3 or q.shape[2] != D:
        raise ValueError("q must be [num_seqs, num_q_heads, head_dim]")
    S, Hq = q.shape[0], q.shape[1]
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.shape[0] != S:
        raise ValueError("block_tables must be int32 [num_seqs, max_blocks]")
    if context_lens.dtype != torch.int32 or context_lens.shape != (S,):
        raise ValueError("context_lens must be int32 [num_seqs]")
    if not (q.dtype == k_cache.dtype == v_cache.dtype):
        raise TypeError("q and the pools must share one dtype")
    need = decode_workspace_bytes(S, Hq, Hkv, D, max_context_len, partition_size)
    if workspace is None and need > 0 and allocate:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = _p(workspace) if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    return (_p(out), _code(out), _p(q), _p(k_cache), _p(v_cache), _p(block_tables), block_tables.shape[1],
            _p(context_lens), S, Hq, Hkv, D, bs, NB, float(scale), int(max_context_len),
            int(partition_size), ws_ptr, ws_bytes, _code(q)), workspace


def decode(out, q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len, partition_size=0,
           workspace=None, stream=None) -> None:
    """out[s, h] = softmax(scale * q[s, h] . K_s^T) V_s over the paged context of sequence s."""
    args, _ = _decode_args(out, q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len,
                           partition_size, workspace)
    _lib.check(_lib.load().pa_decode(*args, _stream(stream)))


def decode_noalloc(out, q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len, partition_size=0,
                   stream=None) -> None:
    """decode without a workspace: the split partials go to the library's fixed device array
    (pa_decode_noalloc); nothing is allocated.  Calls that overlap on one GPU race."""
    args, _ = _decode_args(out, q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len,
                           partition_size, None, allocate=False)
    _lib.check(_lib.load().pa_decode_noalloc(*args[:17], args[19], _stream(stream)))


def decode_partitions(out, q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len, partition_size,
                      workspace, stream=None) -> None:
    """First of decode's two launches (see decode_reduce)."""
    args, _ = _decode_args(out, q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len,
                           partition_size, workspace)
    _lib.check(_lib.load().pa_decode_partitions(*args, _stream(stream)))


def decode_reduce(out, context_lens, num_kv_heads, max_context_len, partition_size, workspace, stream=None) -> None:
    """Second of decode's launches: merge the partition partials into ``out``."""
    _dev(out, context_lens)
    S, Hq, D = out.shape
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _lib.check(_lib.load().pa_decode_reduce(_p(out), _code(out), _p(context_lens), S, Hq, int(num_kv_heads), D,
                                            int(max_context_len), int(partition_size),
                                            _p(workspace) if workspace is not None else None, ws_bytes,
                                            _stream(stream)))


def decode_multi(out, q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len, partition_size=0,
                 workspace=None, stream=None) -> None:
    """Causal attention of the last q_len positions of each context, q [S, q_len, Hq, D], at decode's bandwidth
    (q_len x group <= 16)."""
    _dev(out, q, k_cache, v_cache, block_tables, context_lens)
    NB, Hkv, D, bs = _pools(k_cache, v_cache, q.shape[-1])
    if q.dim() != 4 or q.shape[3] != D:
        raise ValueError("q must be [num_seqs, q_len, num_q_heads, head_dim]")
    S, C, Hq = q.shape[0], q.shape[1], q.shape[2]
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.shape[0] != S:
        raise ValueError("block_tables must be int32 [num_seqs, max_blocks]")
    if context_lens.dtype != torch.int32 or context_lens.shape != (S,):
        raise ValueError("context_lens must be int32 [num_seqs]")
    if not (q.dtype == k_cache.dtype == v_cache.dtype):
        raise TypeError("q and the pools must share one dtype")
    lib = _lib.load()
    need = int(lib.pa_decode_multi_workspace_bytes(S, C, Hq, Hkv, D, int(max_context_len), int(partition_size)))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _lib.check(lib.pa_decode_multi(_p(out), _code(out), _p(q), C, _p(k_cache), _p(v_cache), _p(block_tables),
                                   block_tables.shape[1], _p(context_lens), S, Hq, Hkv, D, bs, NB,
                                   float(scale), int(max_context_len), int(partition_size),
                                   _p(workspace) if workspace is not None else None, ws_bytes, _code(q),
                                   _stream(stream)))


def prefill_chunk(out, q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len, stream=None) -> None:
    """Causal attention of q [S, C, Hq, D] (the last C positions of each context) over the paged cache."""
    _dev(out, q, k_cache, v_cache, block_tables, context_lens)
    NB, Hkv, D, bs = _pools(k_cache, v_cache, q.shape[-1])
    if q.dim() != 4 or q.shape[3] != D:
        raise ValueError("q must be [num_seqs, chunk_len, num_q_heads, head_dim]")
    S, C, Hq = q.shape[0], q.shape[1], q.shape[2]
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.shape[0] != S:
        raise ValueError("block_tables must be int32 [num_seqs, max_blocks]")
    if context_lens.dtype != torch.int32 or context_lens.shape != (S,):
        raise ValueError("context_lens must be int32 [num_seqs]")
    _lib.check(_lib.load().pa_prefill_chunk(_p(out), _code(out), _p(q), C, _p(k_cache), _p(v_cache),
                                            _p(block_tables), block_tables.shape[1], _p(context_lens), S, Hq, Hkv, D,
                                            bs, NB, float(scale), int(max_context_len), _code(q),
                                            _stream(stream)))


def probe_read_bandwidth(buf: torch.Tensor, sink: torch.Tensor, workgroups: int = 4096, stream=None) -> None:
    """Read all of ``buf`` once (HBM read-ceiling probe); ``sink`` is a small int32/uint8 device tensor."""
    _dev(buf, sink)
    _lib.check(_lib.load().pa_probe_read_bandwidth(_p(buf), buf.numel() * buf.element_size(), _p(sink),
                                                   int(workgroups), _stream(stream)))


def probe_gather_bandwidth(buf: torch.Tensor, tiles: torch.Tensor, tile_bytes: int, sink: torch.Tensor,
                           workgroups: int = 1024, stream=None) -> None:
    """Read tiles ``tiles`` (int32 tile indices) of ``tile_bytes`` bytes of ``buf`` once, in the access
    pattern of paged decode (the gather ceiling probe)."""
    _dev(buf, tiles, sink)
    if tiles.dtype != torch.int32 or not tiles.is_contiguous():
        raise ValueError("tiles must be a contiguous int32 tensor")
    _lib.check(_lib.load().pa_probe_gather_bandwidth(_p(buf), buf.numel() * buf.element_size(), _p(tiles),
                                                     tiles.numel(), int(tile_bytes), _p(sink), int(workgroups),
                                                     _stream(stream)))


class StepPlan:
    """One decode step (cache write, decode partitions, merge) on fixed buffers.

    A serving loop launches the same kernels on the same buffers every step;
    only the host bound ``max_context_len`` changes.  The plan checks every
    tensor once, keeps the marshalled C arguments, and each call then costs
    one ctypes call per launch.  The tensors must stay alive and keep their
    storage for the plan's lifetime.  A 4-D ``q`` [S, q_len, Hq, D] plans the
    several-queries-per-sequence decode (pa_decode_multi: both launches in
    one call, ``decode_partitions`` runs it and ``decode_reduce`` is a no-op).

    With ``append=(token_rows, token_positions, new_context_lens)`` the cache
    write is pa_append_step: ``block_tables`` and ``context_lens`` stay on the
    device and the write patches them from the step's slots, so a step ships
    only its tokens' slots / rows / positions and the new lengths (which may
    sit in pinned host memory) instead of whole tables.  With ``host_args``
    those four are CPU tensors whose values each ``cache_write`` copies into
    the kernel arguments (pa_append_step_host): the host may rewrite them as
    soon as the call returns.
    """

    def __init__(self, out, q, k_cache, v_cache, block_tables, context_lens, scale, workspace,
                 key=None, value=None, slot_mapping=None, partition_size=0, stream=None, append=None,
                 host_args=False):
        self._lib = _lib.load()
        self._stream = _stream(stream)
        NB, Hkv, D, bs = _pools(k_cache, v_cache, q.shape[-1])
        self._partition = int(partition_size)
        self._multi = q.dim() == 4
        if self._multi:
            _dev(out, q, k_cache, v_cache, block_tables, context_lens)
            if q.shape[3] != D or out.shape != q.shape:
                raise ValueError("q / out must be [num_seqs, q_len, num_q_heads, head_dim]")
            if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
                raise ValueError("block_tables and context_lens must be int32")
            S, C, Hq = q.shape[0], q.shape[1], q.shape[2]
            ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
            self._multi_head = (_p(out), _code(out), _p(q), C, _p(k_cache), _p(v_cache), _p(block_tables),
                                block_tables.shape[1], _p(context_lens), S, Hq, Hkv, D, bs, NB, float(scale))
            self._multi_tail = (self._partition, _p(workspace) if workspace is not None else None, ws_bytes,
                                _code(q), self._stream)
            self._sizes = (S, Hq, Hkv, D)
            self._q_len = C
        else:
            # the workspace is the caller's, sized for the largest max_context_len the plan will see
            self._args, _ = _decode_args(out, q, k_cache, v_cache, block_tables, context_lens, scale, 0,
                                         partition_size, workspace)
            self._ws_bytes = self._args[18]
            S, Hq = q.shape[0], q.shape[1]
            self._sizes = (S, Hq, Hkv, D)
            self._q_len = 1
            self._reduce_head = (_p(out), _code(out), _p(context_lens), S, Hq, Hkv, D)
        self._write = None
        self._append = None
        if key is not None and append is not None:
            rows, positions, new_ctx = append
            self._append = _append_args(key, value, k_cache, v_cache, slot_mapping, rows, positions, block_tables,
                                        context_lens, new_ctx, stream, host_meta=host_args)
            self._append_fn = self._lib.pa_append_step_host if host_args else self._lib.pa_append_step
        elif key is not None:
            _dev(key, value, slot_mapping)
            if key.shape != value.shape or key.dim() != 3 or key.shape[1:] != (Hkv, D):
                raise ValueError("key / value must be [T, num_kv_heads, head_dim]")
            if slot_mapping.dtype != torch.int64 or slot_mapping.shape != (key.shape[0],):
                raise ValueError("slot_mapping must be int64 [T]")
            if not (key.dtype == value.dtype == k_cache.dtype):
                raise TypeError("key, value and the pools must share one dtype")
            self._write = (_p(key), _p(value), _p(k_cache), _p(v_cache), _p(slot_mapping), key.shape[0], Hkv, D,
                           bs, NB, _code(k_cache), self._stream)

    @staticmethod
    def workspace_bytes_for(num_seqs, q_len, num_q_heads, num_kv_heads, head_dim, max_context_len,
                            partition_size=0) -> int:
        """Workspace a plan of these sizes needs at max_context_len."""
        return int(_lib.load().pa_decode_multi_workspace_bytes(num_seqs, q_len, num_q_heads, num_kv_heads, head_dim,
                                                               int(max_context_len), int(partition_size)))

    def workspace_bytes(self, max_context_len: int) -> int:
        S, Hq, Hkv, D = self._sizes
        return int(self._lib.pa_decode_multi_workspace_bytes(S, self._q_len, Hq, Hkv, D, int(max_context_len),
                                                             self._partition))

    def cache_write(self) -> None:
        if self._append is not None:
            _lib.check(self._append_fn(*self._append))
        else:
            _lib.check(self._lib.pa_reshape_and_cache(*self._write))

    def decode_partitions(self, max_context_len: int) -> None:
        if self._multi:
            _lib.check(self._lib.pa_decode_multi(*self._multi_head, int(max_context_len), *self._multi_tail))
            return
        a = self._args
        _lib.check(self._lib.pa_decode_partitions(*a[:15], int(max_context_len), *a[16:], self._stream))

    def decode_reduce(self, max_context_len: int) -> None:
        if self._multi:
            return
        a = self._args
        _lib.check(self._lib.pa_decode_reduce(*self._reduce_head, int(max_context_len), self._partition, a[17],
                                              self._ws_bytes, self._stream))

    def __call__(self, max_context_len: int) -> None:
        if self._write is not None or self._append is not None:
            self.cache_write()
        self.decode_partitions(max_context_len)
        self.decode_reduce(max_context_len)
