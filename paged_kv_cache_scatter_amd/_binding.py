"""ctypes binding of libpkv.so: argument marshalling only.

Each function checks that the torch tensors it is handed have the shapes,
dtypes, devices and layouts the kernels assume (the C ABI trusts its caller
with buffer sizes), then passes raw device pointers and torch's current HIP
stream to the library. There is no fallback: if the library is missing, or a
call fails, an exception is raised.
"""

from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpkv.so")

F32, BF16 = 0, 1
_DTYPES = {torch.float32: F32, torch.bfloat16: BF16}

_STATUS = {0: "PKV_OK", 1: "PKV_ERR_NULL", 2: "PKV_ERR_DTYPE", 3: "PKV_ERR_SHAPE",
           4: "PKV_ERR_UNSUPPORTED", 5: "PKV_ERR_WORKSPACE", 6: "PKV_ERR_HIP",
           7: "PKV_ERR_ALIGN", 8: "PKV_ERR_CAPACITY"}

# Every symbol include/pkv.h declares.
EXPORTS = ("pkv_slot_mapping", "pkv_write", "pkv_decode_partition",
           "pkv_decode_workspace_bytes", "pkv_decode_schedule", "pkv_decode", "pkv_decode_partials",
           "pkv_decode_reduce", "pkv_decode_step", "pkv_decode_step_partials",
           "pkv_decode_step_noalloc",
           "pkv_decode_shared_workspace_bytes", "pkv_decode_shared", "pkv_prefill",
           "pkv_validate_workspace_bytes", "pkv_validate",
           "pkv_block_bytes", "pkv_plan_pool", "pkv_status_string", "pkv_last_error",
           "pkv_abi_version")


class PkvError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        self.status_name = _STATUS.get(status, f"status {status}")
        super().__init__(f"{self.status_name}: {message}")


class PoolDesc(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int32


def load(path: str | None = None):
    """Load (once) and return the ctypes handle of libpkv.so."""
    global _lib
    if _lib is not None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is not built; run `python -m paged_kv_cache_scatter_amd.build` "
                           "(or __graft_entry__.build())")
    lib = ctypes.CDLL(p)
    lib.pkv_slot_mapping.argtypes = [_P, _I, _I, _P, _P, _I, _I, _I, _P, _P]
    lib.pkv_slot_mapping.restype = ctypes.c_int
    lib.pkv_write.argtypes = [_P, _P, _P, _I, _P, _P, ctypes.POINTER(PoolDesc), _P]
    lib.pkv_write.restype = ctypes.c_int
    lib.pkv_decode_partition.argtypes = [_I, _I, ctypes.POINTER(PoolDesc)]
    lib.pkv_decode_partition.restype = _I
    lib.pkv_decode_workspace_bytes.argtypes = [_I, _I, _I, _I, ctypes.POINTER(PoolDesc)]
    lib.pkv_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.pkv_decode_schedule.argtypes = [_I, _I, _I, _I, ctypes.POINTER(PoolDesc)]
    lib.pkv_decode_schedule.restype = _I
    dec_args = [_P, _I, _I, _P, _P, ctypes.POINTER(PoolDesc), _P, _I, _P, _I, ctypes.c_float,
                _I, _P, _P, ctypes.c_size_t, _P]
    for name in ("pkv_decode", "pkv_decode_partials", "pkv_decode_reduce"):
        f = getattr(lib, name)
        f.argtypes = dec_args
        f.restype = ctypes.c_int
    step_args = [_P, _P, _P, _I, _I, _P, _P, ctypes.POINTER(PoolDesc), _P, _I, _P, _I,
                 ctypes.c_float, _I, _P, _P, ctypes.c_size_t, _P]
    for name in ("pkv_decode_step", "pkv_decode_step_partials"):
        f = getattr(lib, name)
        f.argtypes = step_args
        f.restype = ctypes.c_int
    lib.pkv_decode_step_noalloc.argtypes = [_P, _P, _P, _I, _I, _P, _P, ctypes.POINTER(PoolDesc),
                                            _P, _I, _P, _I, ctypes.c_float, _I, _P, _P]
    lib.pkv_decode_step_noalloc.restype = ctypes.c_int
    lib.pkv_decode_shared_workspace_bytes.argtypes = [_I, _I, _I, _I, _I, _I, _I, _I,
                                                      ctypes.POINTER(PoolDesc)]
    lib.pkv_decode_shared_workspace_bytes.restype = ctypes.c_size_t
    lib.pkv_decode_shared.argtypes = [_P, _I, _I, _P, _P, ctypes.POINTER(PoolDesc), _P, _I, _P, _I,
                                      _P, _P, _I, _I, _I, _I, ctypes.c_float, _I, _P, _P,
                                      ctypes.c_size_t, _P]
    lib.pkv_decode_shared.restype = ctypes.c_int
    lib.pkv_prefill.argtypes = [_P, _P, _I, _I, _I, _I, _P, _P, ctypes.POINTER(PoolDesc), _P,
                                _I, _P, _I, ctypes.c_float, _P, _P]
    lib.pkv_prefill.restype = ctypes.c_int
    lib.pkv_validate_workspace_bytes.argtypes = [_I, _I]
    lib.pkv_validate_workspace_bytes.restype = ctypes.c_size_t
    lib.pkv_validate.argtypes = [_P, _I, _P, _I, _P, _I, _I, _I, _P, ctypes.c_size_t, _P, _P]
    lib.pkv_validate.restype = ctypes.c_int
    lib.pkv_block_bytes.argtypes = [_I, _I, _I, _I, _I]
    lib.pkv_block_bytes.restype = ctypes.c_int64
    lib.pkv_plan_pool.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_double, ctypes.c_int64,
                                  ctypes.c_int64, _I, _I, ctypes.POINTER(ctypes.c_int64),
                                  ctypes.POINTER(ctypes.c_int64)]
    lib.pkv_plan_pool.restype = ctypes.c_int
    lib.pkv_status_string.argtypes = [ctypes.c_int]
    lib.pkv_status_string.restype = ctypes.c_char_p
    lib.pkv_last_error.argtypes = []
    lib.pkv_last_error.restype = ctypes.c_char_p
    lib.pkv_abi_version.argtypes = []
    lib.pkv_abi_version.restype = _I
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        raise PkvError(status, load().pkv_last_error().decode())


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


_raw_stream_fn = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _raw_stream(device_index: int) -> int:
    """Current stream of a device as a raw handle (the cheap path when torch has it)."""
    if _raw_stream_fn is not None:
        return _raw_stream_fn(device_index)
    return torch.cuda.current_stream(device_index).cuda_stream


class PreparedCall:
    """One library call whose arguments were checked and converted once.

    Calling it issues the same call again on the device's current stream (so it
    can be captured into a HIP graph): the tensors it was prepared with are
    used in place, and their contents may change between calls, but they must
    stay alive and keep their shapes. The host cost of a call is one foreign
    function call with pre-built arguments instead of the checks and
    conversions of the plain functions. ``out`` is the output tensor."""

    __slots__ = ("_fn", "_args", "_device", "_keep", "out")

    def __init__(self, name: str, args: tuple, device: torch.device, keep: tuple, out):
        fn = load()[name]            # a handle of its own: no per-call argument conversion
        fn.restype = ctypes.c_int
        self._fn = fn
        self._args = args            # ctypes values, built once
        self._device = device.index if device.index is not None else torch.cuda.current_device()
        self._keep = keep            # the tensors and descriptor the pointers refer to
        self.out = out

    def __call__(self):
        r = self._fn(*self._args, ctypes.c_void_p(_raw_stream(self._device)))
        if r:
            _check(r)
        return self.out


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


_cp = lambda t: ctypes.c_void_p(None if t is None else t.data_ptr())
_ci = ctypes.c_int32


def _need(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _dev(t: torch.Tensor, name: str, dtype=None, shape=None):
    _need(isinstance(t, torch.Tensor), f"{name} must be a torch tensor")
    _need(t.is_cuda, f"{name} must be on the GPU")
    _need(t.is_contiguous(), f"{name} must be contiguous")
    if dtype is not None:
        _need(t.dtype == dtype, f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None:
        _need(tuple(t.shape) == tuple(shape), f"{name} must have shape {tuple(shape)}, "
              f"got {tuple(t.shape)}")


def pool_desc(k_pool: torch.Tensor) -> PoolDesc:
    _need(k_pool.dim() == 4, "pools are [num_blocks, block_size, num_kv_heads, head_dim]")
    _need(k_pool.dtype in _DTYPES, f"pool dtype {k_pool.dtype} is not float32/bfloat16")
    nb, bs, hkv, hd = k_pool.shape
    return PoolDesc(nb, bs, hkv, hd, _DTYPES[k_pool.dtype])


def _check_pools(k_pool, v_pool):
    _dev(k_pool, "k_pool")
    _dev(v_pool, "v_pool", dtype=k_pool.dtype, shape=k_pool.shape)
    _need(k_pool.device == v_pool.device, "pools on different devices")
    return pool_desc(k_pool)


# ---------------------------------------------------------------- slot mapping
def slot_mapping(tables: torch.Tensor, first_pos: torch.Tensor, cu_tokens: torch.Tensor,
                 num_tokens: int, block_size: int, num_blocks: int,
                 out: torch.Tensor | None = None) -> torch.Tensor:
    """Flat slot of every token of a write (segments of consecutive positions)."""
    _dev(tables, "tables", torch.int32)
    _need(tables.dim() == 2, "tables must be [num_segments, max_blocks_per_seq]")
    W, maxb = tables.shape
    _dev(first_pos, "first_pos", torch.int32, (W,))
    _dev(cu_tokens, "cu_tokens", torch.int32, (W + 1,))
    if out is None:
        out = torch.empty(int(num_tokens), dtype=torch.int32, device=tables.device)
    _dev(out, "slot_mapping", torch.int32, (int(num_tokens),))
    _check(load().pkv_slot_mapping(_ptr(tables), maxb, W, _ptr(first_pos), _ptr(cu_tokens),
                                   int(num_tokens), int(block_size), int(num_blocks), _ptr(out),
                                   _stream()))
    return out


# ---------------------------------------------------------------- write
def write(k: torch.Tensor, v: torch.Tensor, slots: torch.Tensor, k_pool: torch.Tensor,
          v_pool: torch.Tensor) -> None:
    """Scatter rows of k, v ([T, Hkv, hd]) into the pools at ``slots`` ([T] int32)."""
    desc = _check_pools(k_pool, v_pool)
    _dev(slots, "slot_mapping", torch.int32)
    _need(slots.dim() == 1, "slot_mapping must be 1-D")
    T = slots.shape[0]
    _dev(k, "k", k_pool.dtype, (T, desc.num_kv_heads, desc.head_dim))
    _dev(v, "v", k_pool.dtype, (T, desc.num_kv_heads, desc.head_dim))
    if debug_enabled():
        _debug_check("write", validate(slots=slots, num_blocks=desc.num_blocks,
                                       block_size=desc.block_size), ("slots_past_pool",
                                                                     "duplicate_slots"))
    _check(load().pkv_write(_ptr(k), _ptr(v), _ptr(slots), T, _ptr(k_pool), _ptr(v_pool),
                            ctypes.byref(desc), _stream()))


# ---------------------------------------------------------------- decode
def decode_partition(num_seqs: int, max_context_len: int, k_pool: torch.Tensor) -> int:
    desc = pool_desc(k_pool)
    return int(load().pkv_decode_partition(int(num_seqs), int(max_context_len),
                                           ctypes.byref(desc)))


# pkv_decode_schedule's values (PKV_SCHED_* of include/pkv.h)
SCHEDULES = {0: "grid", 1: "pieces", 2: "longest_first", 3: "stream_k"}


def decode_schedule(num_seqs: int, num_q_heads: int, max_context_len: int,
                    k_pool: torch.Tensor, partition: int = 0) -> str:
    """The cut pkv_decode / pkv_decode_step use for these sizes (a SCHEDULES name)."""
    desc = pool_desc(k_pool)
    r = int(load().pkv_decode_schedule(int(num_seqs), int(num_q_heads), int(max_context_len),
                                       int(partition), ctypes.byref(desc)))
    if r < 0:
        raise PkvError(3, load().pkv_last_error().decode())   # PKV_ERR_SHAPE
    return SCHEDULES[r]


def decode_workspace_bytes(num_seqs: int, num_q_heads: int, max_context_len: int,
                           k_pool: torch.Tensor, partition: int = 0) -> int:
    desc = pool_desc(k_pool)
    return int(load().pkv_decode_workspace_bytes(int(num_seqs), int(num_q_heads),
                                                 int(max_context_len), int(partition),
                                                 ctypes.byref(desc)))


def decode(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
           block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
           max_context_len: int, out: torch.Tensor | None = None, partition: int = 0,
           workspace: torch.Tensor | None = None, phase: str = "both") -> torch.Tensor:
    """Paged decode attention; q [S, Hq, hd] -> out [S, Hq, hd].

    ``max_context_len`` is a host-side bound on ``context_lens`` (the library
    never reads device memory on the host). ``workspace`` is a uint8 device
    tensor of at least ``decode_workspace_bytes(...)`` bytes (allocated here
    if omitted and needed). A passed workspace must be zero-filled before its
    first use (``torch.zeros``, not ``torch.empty``): its first 256 KiB count
    the pieces merged in the launch, and every call leaves them zero, so one
    buffer serves calls of any size in stream order. ``phase``: "both",
    "partials" or "reduce".
    """
    fn, args, keep = _decode_call(q, k_pool, v_pool, block_tables, context_lens, scale,
                                  max_context_len, out, partition, workspace, phase)
    _debug_tables("decode", k_pool, block_tables, context_lens)
    _check(getattr(load(), fn)(*args, _stream()))
    return keep[-1]


def _decode_call(q, k_pool, v_pool, block_tables, context_lens, scale, max_context_len, out,
                 partition, workspace, phase):
    """Checks of ``decode``; returns (entry point, typed arguments without the
    stream, tensors they point to with ``out`` last)."""
    desc = _check_pools(k_pool, v_pool)
    _dev(q, "q", k_pool.dtype)
    _need(q.dim() == 3 and q.shape[2] == desc.head_dim, "q must be [S, Hq, head_dim]")
    S, Hq, _ = q.shape
    _dev(block_tables, "block_tables", torch.int32)
    _need(block_tables.dim() == 2 and block_tables.shape[0] == S,
          "block_tables must be [S, max_blocks_per_seq]")
    maxb = block_tables.shape[1]
    _dev(context_lens, "context_lens", torch.int32, (S,))
    if out is None:
        out = torch.empty_like(q)
    _dev(out, "out", q.dtype, q.shape)
    if workspace is None:   # a passed workspace is size-checked by the library
        need = decode_workspace_bytes(S, Hq, max_context_len, k_pool, partition)
        if need > 0:
            workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0
    if workspace is not None:
        _dev(workspace, "workspace", torch.uint8)
        ws_bytes = workspace.numel()
    fn = {"both": "pkv_decode", "partials": "pkv_decode_partials",
          "reduce": "pkv_decode_reduce"}[phase]
    args = (_cp(q), _ci(S), _ci(Hq), _cp(k_pool), _cp(v_pool), ctypes.byref(desc),
            _cp(block_tables), _ci(maxb), _cp(context_lens), _ci(int(max_context_len)),
            ctypes.c_float(float(scale)), _ci(int(partition)), _cp(out), _cp(workspace),
            ctypes.c_size_t(ws_bytes))
    return fn, args, (desc, q, k_pool, v_pool, block_tables, context_lens, workspace, out)


def prepare_decode(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                   block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
                   max_context_len: int, out: torch.Tensor | None = None, partition: int = 0,
                   workspace: torch.Tensor | None = None) -> PreparedCall:
    """``decode`` checked and marshalled once: returns a PreparedCall that
    launches the same decode on the current stream each time it is called."""
    fn, args, keep = _decode_call(q, k_pool, v_pool, block_tables, context_lens, scale,
                                  max_context_len, out, partition, workspace, "both")
    _debug_tables("prepare_decode", k_pool, block_tables, context_lens)
    return PreparedCall(fn, args, q.device, keep, keep[-1])


def decode_shared_workspace_bytes(num_seqs: int, num_q_heads: int, max_context_len: int,
                                  num_groups: int, max_group_size: int, max_prefix_len: int,
                                  max_tail_len: int, k_pool: torch.Tensor,
                                  partition: int = 0) -> int:
    desc = pool_desc(k_pool)
    return int(load().pkv_decode_shared_workspace_bytes(
        int(num_seqs), int(num_q_heads), int(max_context_len), int(num_groups),
        int(max_group_size), int(max_prefix_len), int(max_tail_len), int(partition),
        ctypes.byref(desc)))


def decode_shared(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                  block_tables: torch.Tensor, context_lens: torch.Tensor,
                  group_start: torch.Tensor, prefix_lens: torch.Tensor, scale: float,
                  max_context_len: int, max_group_size: int, max_prefix_len: int,
                  max_tail_len: int = -1, out: torch.Tensor | None = None, partition: int = 0,
                  workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Paged decode where groups of consecutive sequences share the leading
    blocks of their tables. ``group_start`` int32 [G+1] (members of group i are
    sequences group_start[i] .. group_start[i+1]-1), ``prefix_lens`` int32 [G]
    (shared tokens of each group). The ``max_*`` arguments are host-side bounds
    (``max_tail_len`` < 0: ``max_context_len``). ``workspace``: at least
    ``decode_shared_workspace_bytes(...)`` bytes, zero-filled before its first
    use as for ``decode``. Same result as ``decode``."""
    desc = _check_pools(k_pool, v_pool)
    _dev(q, "q", k_pool.dtype)
    _need(q.dim() == 3 and q.shape[2] == desc.head_dim, "q must be [S, Hq, head_dim]")
    S, Hq, _ = q.shape
    _dev(block_tables, "block_tables", torch.int32)
    _need(block_tables.dim() == 2 and block_tables.shape[0] == S,
          "block_tables must be [S, max_blocks_per_seq]")
    maxb = block_tables.shape[1]
    _dev(context_lens, "context_lens", torch.int32, (S,))
    _dev(group_start, "group_start", torch.int32)
    _need(group_start.dim() == 1 and group_start.shape[0] >= 1, "group_start must be [G+1]")
    G = group_start.shape[0] - 1
    _dev(prefix_lens, "prefix_lens", torch.int32, (G,))
    if out is None:
        out = torch.empty_like(q)
    _dev(out, "out", q.dtype, q.shape)
    if workspace is None:   # a passed workspace is size-checked by the library
        need = decode_shared_workspace_bytes(S, Hq, max_context_len, G, max_group_size,
                                             max_prefix_len, max_tail_len, k_pool, partition)
        if need > 0:
            workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0
    if workspace is not None:
        _dev(workspace, "workspace", torch.uint8)
        ws_bytes = workspace.numel()
    _debug_tables("decode_shared", k_pool, block_tables, context_lens)
    _check(load().pkv_decode_shared(
        _ptr(q), S, Hq, _ptr(k_pool), _ptr(v_pool), ctypes.byref(desc), _ptr(block_tables), maxb,
        _ptr(context_lens), int(max_context_len), _ptr(group_start), _ptr(prefix_lens), G,
        int(max_group_size), int(max_prefix_len), int(max_tail_len), float(scale),
        int(partition), _ptr(out), _ptr(workspace), ws_bytes, _stream()))
    return out


def decode_step(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                k_pool: torch.Tensor, v_pool: torch.Tensor, block_tables: torch.Tensor,
                context_lens: torch.Tensor, scale: float, max_context_len: int,
                out: torch.Tensor | None = None, partition: int = 0,
                workspace: torch.Tensor | None = None, phase: str = "both") -> torch.Tensor:
    """Decode step with the KV write fused in: k_new / v_new [S, Hkv, hd] are the
    new token of each sequence (position context_lens - 1); they are written into
    their slots and attended. ``workspace`` as for ``decode`` (zero-filled
    before its first use). ``phase``: "both", "partials" (then call
    ``decode(..., phase="reduce")`` with the same arguments) or "reduce"."""
    fn, args, keep = _step_call(q, k_new, v_new, k_pool, v_pool, block_tables, context_lens,
                                scale, max_context_len, out, partition, workspace, phase)
    _debug_tables("decode_step", k_pool, block_tables, context_lens)
    _check(getattr(load(), fn)(*args, _stream()))
    return keep[-1]


def _step_call(q, k_new, v_new, k_pool, v_pool, block_tables, context_lens, scale,
               max_context_len, out, partition, workspace, phase):
    """Checks of ``decode_step``; returns (entry point, typed arguments without
    the stream, tensors they point to with ``out`` last)."""
    desc = _check_pools(k_pool, v_pool)
    _dev(q, "q", k_pool.dtype)
    _need(q.dim() == 3 and q.shape[2] == desc.head_dim, "q must be [S, Hq, head_dim]")
    S, Hq, _ = q.shape
    _dev(k_new, "k_new", k_pool.dtype, (S, desc.num_kv_heads, desc.head_dim))
    _dev(v_new, "v_new", k_pool.dtype, (S, desc.num_kv_heads, desc.head_dim))
    _dev(block_tables, "block_tables", torch.int32)
    _need(block_tables.dim() == 2 and block_tables.shape[0] == S,
          "block_tables must be [S, max_blocks_per_seq]")
    maxb = block_tables.shape[1]
    _dev(context_lens, "context_lens", torch.int32, (S,))
    if out is None:
        out = torch.empty_like(q)
    _dev(out, "out", q.dtype, q.shape)
    if workspace is None:   # a passed workspace is size-checked by the library
        need = decode_workspace_bytes(S, Hq, max_context_len, k_pool, partition)
        if need > 0:
            workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0
    if workspace is not None:
        _dev(workspace, "workspace", torch.uint8)
        ws_bytes = workspace.numel()
    _need(phase in ("both", "partials", "reduce"), f"unknown phase {phase!r}")
    common = (ctypes.byref(desc), _cp(block_tables), _ci(maxb), _cp(context_lens),
              _ci(int(max_context_len)), ctypes.c_float(float(scale)), _ci(int(partition)),
              _cp(out), _cp(workspace), ctypes.c_size_t(ws_bytes))
    keep = (desc, q, k_new, v_new, k_pool, v_pool, block_tables, context_lens, workspace, out)
    if phase == "reduce":
        return "pkv_decode_reduce", (_cp(q), _ci(S), _ci(Hq), _cp(k_pool), _cp(v_pool)) + common, \
            keep
    fn = "pkv_decode_step" if phase == "both" else "pkv_decode_step_partials"
    return fn, (_cp(q), _cp(k_new), _cp(v_new), _ci(S), _ci(Hq), _cp(k_pool), _cp(v_pool)) + \
        common, keep


def prepare_decode_step(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                        k_pool: torch.Tensor, v_pool: torch.Tensor, block_tables: torch.Tensor,
                        context_lens: torch.Tensor, scale: float, max_context_len: int,
                        out: torch.Tensor | None = None, partition: int = 0,
                        workspace: torch.Tensor | None = None) -> PreparedCall:
    """``decode_step`` checked and marshalled once: returns a PreparedCall that
    launches the same fused step on the current stream each time it is called."""
    fn, args, keep = _step_call(q, k_new, v_new, k_pool, v_pool, block_tables, context_lens,
                                scale, max_context_len, out, partition, workspace, "both")
    _debug_tables("prepare_decode_step", k_pool, block_tables, context_lens)
    return PreparedCall(fn, args, q.device, keep, keep[-1])


NOALLOC_SCRATCH_BYTES = 32 << 20   # PKV_NOALLOC_SCRATCH_BYTES of include/pkv.h


def decode_step_noalloc(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                        k_pool: torch.Tensor, v_pool: torch.Tensor, block_tables: torch.Tensor,
                        context_lens: torch.Tensor, scale: float, max_context_len: int,
                        out: torch.Tensor, partition: int = 0) -> torch.Tensor:
    """``decode_step`` without a workspace: the library's fixed scratch array
    holds the split partials, so nothing is allocated (``out`` must be
    passed). Raises PkvError (PKV_ERR_WORKSPACE) when the step needs more
    scratch than the array holds. Calls that may overlap on one GPU race."""
    desc = _check_pools(k_pool, v_pool)
    _dev(q, "q", k_pool.dtype)
    _need(q.dim() == 3 and q.shape[2] == desc.head_dim, "q must be [S, Hq, head_dim]")
    S, Hq, _ = q.shape
    _dev(k_new, "k_new", k_pool.dtype, (S, desc.num_kv_heads, desc.head_dim))
    _dev(v_new, "v_new", k_pool.dtype, (S, desc.num_kv_heads, desc.head_dim))
    _dev(block_tables, "block_tables", torch.int32)
    _need(block_tables.dim() == 2 and block_tables.shape[0] == S,
          "block_tables must be [S, max_blocks_per_seq]")
    _dev(context_lens, "context_lens", torch.int32, (S,))
    _dev(out, "out", q.dtype, q.shape)
    _debug_tables("decode_step_noalloc", k_pool, block_tables, context_lens)
    _check(load().pkv_decode_step_noalloc(
        _ptr(q), _ptr(k_new), _ptr(v_new), S, Hq, _ptr(k_pool), _ptr(v_pool), ctypes.byref(desc),
        _ptr(block_tables), block_tables.shape[1], _ptr(context_lens), int(max_context_len),
        float(scale), int(partition), _ptr(out), _stream()))
    return out


# ---------------------------------------------------------------- prefill
def prefill(q: torch.Tensor, cu_q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
            block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
            max_q_len: int, max_context_len: int,
            out: torch.Tensor | None = None) -> torch.Tensor:
    """Causal attention of packed query chunks q [sum n_s, Hq, hd] over the pool."""
    desc = _check_pools(k_pool, v_pool)
    _dev(q, "q", k_pool.dtype)
    _need(q.dim() == 3 and q.shape[2] == desc.head_dim, "q must be [rows, Hq, head_dim]")
    R, Hq, _ = q.shape
    _dev(block_tables, "block_tables", torch.int32)
    _need(block_tables.dim() == 2, "block_tables must be [S, max_blocks_per_seq]")
    S, maxb = block_tables.shape
    _dev(cu_q, "cu_q", torch.int32, (S + 1,))
    _dev(context_lens, "context_lens", torch.int32, (S,))
    if out is None:
        out = torch.empty_like(q)
    _dev(out, "out", q.dtype, q.shape)
    _debug_tables("prefill", k_pool, block_tables, context_lens)
    _check(load().pkv_prefill(_ptr(q), _ptr(cu_q), S, Hq, int(max_q_len), R, _ptr(k_pool),
                              _ptr(v_pool), ctypes.byref(desc), _ptr(block_tables), maxb,
                              _ptr(context_lens), int(max_context_len), float(scale), _ptr(out),
                              _stream()))
    return out


def abi_version() -> int:
    return int(load().pkv_abi_version())


# ---------------------------------------------------------------- index checks
VALIDATE_FIELDS = ("negative_slots", "slots_past_pool", "duplicate_slots",
                   "invalid_table_entries", "context_past_table")


def validate(slots: torch.Tensor | None = None, block_tables: torch.Tensor | None = None,
             context_lens: torch.Tensor | None = None, *, num_blocks: int, block_size: int,
             workspace: torch.Tensor | None = None) -> dict:
    """Counts of the index errors the kernels would silently skip or mask
    (``pkv_validate``): slots < 0, slots past the pool, duplicate slots of one
    write, table entries outside the pool among the blocks a sequence needs,
    and context lengths outside the table's reach. Synchronises the current
    stream to read the counts. ``workspace``: a zeroed int32 device tensor of
    ``pkv_validate_workspace_bytes`` bytes (allocated here if omitted; left
    zero by the call)."""
    lib = load()
    dev = next((t.device for t in (slots, block_tables) if t is not None), None)
    _need(dev is not None, "validate needs slots or block_tables")
    T, S, maxb = 0, 0, 0
    if slots is not None:
        _dev(slots, "slot_mapping", torch.int32)
        _need(slots.dim() == 1, "slot_mapping must be 1-D")
        T = slots.shape[0]
    if block_tables is not None:
        _dev(block_tables, "block_tables", torch.int32)
        _need(block_tables.dim() == 2, "block_tables must be [S, max_blocks_per_seq]")
        S, maxb = block_tables.shape
        _need(context_lens is not None, "checking tables needs context_lens")
        _dev(context_lens, "context_lens", torch.int32, (S,))
    ws_bytes = 0
    if T > 0:
        need = int(lib.pkv_validate_workspace_bytes(int(num_blocks), int(block_size)))
        if workspace is None:
            workspace = torch.zeros((need + 3) // 4, dtype=torch.int32, device=dev)
        _dev(workspace, "workspace", torch.int32)
        ws_bytes = workspace.numel() * 4
    report = torch.empty(len(VALIDATE_FIELDS), dtype=torch.int32, device=dev)
    _check(lib.pkv_validate(_ptr(slots), T, _ptr(block_tables), maxb, _ptr(context_lens), S,
                            int(num_blocks), int(block_size), _ptr(workspace), ws_bytes,
                            _ptr(report), _stream()))
    return dict(zip(VALIDATE_FIELDS, (int(x) for x in report.cpu())))


def debug_enabled() -> bool:
    """PKV_DEBUG set to anything but "" or "0": the plain binding functions
    validate their index arguments (one extra synchronisation per call) and
    raise PkvError on what the kernels would silently skip or mask. Prepared
    calls are checked once, when prepared."""
    return os.environ.get("PKV_DEBUG", "") not in ("", "0")


def _debug_check(what: str, counts: dict, fatal: tuple):
    bad = {k: counts[k] for k in fatal if counts[k]}
    if bad:
        raise PkvError(3, f"PKV_DEBUG: {what}: " +   # PKV_ERR_SHAPE
                       ", ".join(f"{k} {n}" for k, n in bad.items()))


def _debug_tables(what: str, k_pool: torch.Tensor, block_tables: torch.Tensor,
                  context_lens: torch.Tensor):
    if debug_enabled():
        _debug_check(what, validate(block_tables=block_tables, context_lens=context_lens,
                                    num_blocks=k_pool.shape[0], block_size=k_pool.shape[1]),
                     ("invalid_table_entries", "context_past_table"))


# ---------------------------------------------------------------- pool sizing
def block_bytes(num_layers: int, block_size: int, num_kv_heads: int, head_dim: int,
                itemsize: int) -> int:
    """Bytes of one block of a layered K/V pool (0 if an argument is < 1);
    raises PkvError if the size does not fit in int64."""
    n = int(load().pkv_block_bytes(int(num_layers), int(block_size), int(num_kv_heads),
                                   int(head_dim), int(itemsize)))
    if n < 0:
        raise PkvError(3, load().pkv_last_error().decode())   # PKV_ERR_SHAPE
    return n


def plan_pool(free_bytes: int, total_bytes: int, utilization: float, activation_bytes: int,
              block_bytes: int, block_size: int, max_model_len: int):
    """(num_blocks, requests_at_max_len) for a device; raises PkvError
    (PKV_ERR_CAPACITY) if the pool cannot hold one request of max_model_len."""
    nb, nr = ctypes.c_int64(), ctypes.c_int64()
    _check(load().pkv_plan_pool(int(free_bytes), int(total_bytes), float(utilization),
                                int(activation_bytes), int(block_bytes), int(block_size),
                                int(max_model_len), ctypes.byref(nb), ctypes.byref(nr)))
    return int(nb.value), int(nr.value)
