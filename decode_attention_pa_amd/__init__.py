"""Python binding of libpa_decode.so (paged-attention decode on MI355X).

Argument marshalling only: torch tensors supply device memory and the
current HIP stream; every step of the computation runs in the library's HIP
kernels.  There is no fallback: if the library is not built, or a call
fails, an exception says so.

    import decode_attention_pa_amd as pa
    pa.decode(out, q, k_cache, v_cache, block_tables, seq_lens, query_lens,
              scale, window, num_kv_heads, block_size, max_seq_len=...)

Layouts (see include/pa_decode.h): q/out [T, H_q, D]; k_cache
[num_blocks, H_kv, block_size/16, 2, D/8, 8, 8] (16-slot tiles); v_cache
[num_blocks, H_kv, block_size/8, D, 8] (8-slot tiles);
block_tables int32 [B, max_blocks_per_seq]; seq_lens, query_lens int32 [B].
"""

from __future__ import annotations

import ctypes
import os

__all__ = [
    "PaError", "Dims", "Plan", "Options", "load", "library_path", "plan", "workspace_size",
    "decode", "debug_spans", "check_inputs", "PATH_AUTO", "PATH_VALU", "PATH_MFMA",
    "PATH_VALU_LDS", "F32", "BF16",
    "EXPORTED_SYMBOLS",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
# the in-tree build, or another build of the same library named by
# PA_DECODE_LIBRARY (an absolute path)
_LIB_PATH = os.environ.get("PA_DECODE_LIBRARY") or os.path.join(_HERE, "libpa_decode.so")

PATH_AUTO, PATH_VALU, PATH_MFMA, PATH_VALU_LDS = 0, 1, 2, 3
F32, BF16 = 0, 1
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, 1, 2, 3, 4

EXPORTED_SYMBOLS = (
    "pa_plan_compute", "pa_decode_workspace_size", "pa_decode_workspace_size_ex",
    "pa_decode", "pa_decode_ex", "pa_decode_noalloc", "pa_noalloc_scratch_bytes",
    "pa_pack_kv_cache", "pa_debug_spans", "pa_check_inputs", "pa_stream_read", "pa_status_string",
    "pa_last_error",
)


class PaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("max_query_len", ctypes.c_int32),
                ("max_seq_len", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32),
                ("num_blocks", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("kv_format", ctypes.c_int32), ("q_format", ctypes.c_int32)]


class Plan(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("rows", ctypes.c_int32),
                ("block_rows", ctypes.c_int32), ("span_max", ctypes.c_int32), ("part_size", ctypes.c_int32),
                ("num_parts", ctypes.c_int32), ("waves", ctypes.c_int32),
                ("one_shot", ctypes.c_int32), ("persistent", ctypes.c_int32),
                ("row_tiles", ctypes.c_int32), ("row_blocks", ctypes.c_int32),
                ("streaming", ctypes.c_int32), ("ps_grid", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_uint64)]

    def as_dict(self) -> dict:
        return {f: getattr(self, f) for f, _ in self._fields_}


class Options(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("part_size", ctypes.c_int32),
                ("waves", ctypes.c_int32), ("schedule", ctypes.c_int32),
                ("loads", ctypes.c_int32),
                ("event_begin", ctypes.c_void_p), ("event_end", ctypes.c_void_p),
                ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
                ("q_scale", ctypes.c_void_p)]


_lib = None


def library_path() -> str:
    return _LIB_PATH


def load() -> ctypes.CDLL:
    """Loads the built library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise PaError(ERR_UNSUPPORTED,
                      f"{_LIB_PATH} is not built; run `python -m decode_attention_pa_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I32 = ctypes.c_int32
    pd = ctypes.POINTER(Dims)
    po = ctypes.POINTER(Options)
    lib.pa_plan_compute.argtypes = [pd, I32, I32, I32, I32, po, ctypes.POINTER(Plan)]
    lib.pa_decode_workspace_size_ex.argtypes = [pd, I32, I32, I32, po, ctypes.POINTER(ctypes.c_size_t)]
    lib.pa_decode_workspace_size.argtypes = [pd, I32, I32, I32, ctypes.POINTER(ctypes.c_size_t)]
    lib.pa_decode.argtypes = [P, P, P, P, P, P, P, ctypes.c_float, I32, I32, I32, pd, P,
                              ctypes.c_size_t, P]
    lib.pa_decode_ex.argtypes = lib.pa_decode.argtypes + [po]
    lib.pa_decode_noalloc.argtypes = [P, P, P, P, P, P, P, ctypes.c_float, I32, I32, I32, pd, P, po]
    lib.pa_pack_kv_cache.argtypes = [P, P, P, P, P, I32, I32, I32, I32, I32, I32, I32, P]
    lib.pa_noalloc_scratch_bytes.argtypes = []
    lib.pa_noalloc_scratch_bytes.restype = ctypes.c_size_t
    lib.pa_stream_read.argtypes = [P, ctypes.c_size_t, P, I32, I32, ctypes.POINTER(I32), P]
    lib.pa_debug_spans.argtypes = [P, P, P, I32, I32, I32, pd, po, P, P, P, P, P]
    lib.pa_check_inputs.argtypes = [P, P, P, I32, I32, I32, pd, P, P]
    lib.pa_status_string.argtypes = [I32]
    lib.pa_status_string.restype = ctypes.c_char_p
    lib.pa_last_error.argtypes = []
    lib.pa_last_error.restype = ctypes.c_char_p
    for name in ("pa_plan_compute", "pa_decode_workspace_size", "pa_decode_workspace_size_ex",
                 "pa_decode", "pa_decode_ex", "pa_decode_noalloc", "pa_pack_kv_cache",
                 "pa_debug_spans", "pa_check_inputs", "pa_stream_read"):
        getattr(lib, name).restype = I32
    _lib = lib
    return lib


def _check(status: int):
    if status != OK:
        lib = load()
        raise PaError(status, f"{lib.pa_status_string(status).decode()}: "
                              f"{lib.pa_last_error().decode()}")


KV_NATIVE, KV_FP8_E4M3 = 0, 1
Q_NATIVE, Q_FP8_E4M3 = 0, 1


def make_dims(batch, num_q_heads, head_dim, max_query_len, max_seq_len, max_blocks_per_seq,
              num_blocks, dtype, kv_format=KV_NATIVE, q_format=Q_NATIVE) -> Dims:
    return Dims(int(batch), int(num_q_heads), int(head_dim), int(max_query_len),
                int(max_seq_len), int(max_blocks_per_seq), int(num_blocks), int(dtype),
                int(kv_format), int(q_format))


SCHED_AUTO, SCHED_GRID, SCHED_PERSISTENT = 0, 1, 2
LOADS_AUTO, LOADS_CACHED, LOADS_STREAMING = 0, 1, 2


def make_options(path=0, part_size=0, waves=0, event_begin=None, event_end=None,
                 schedule=0, loads=0, k_scale=None, v_scale=None, q_scale=None) -> Options:
    return Options(int(path), int(part_size), int(waves), int(schedule), int(loads),
                   _event_handle(event_begin), _event_handle(event_end),
                   _scale_ptr(k_scale), _scale_ptr(v_scale), _scale_ptr(q_scale))


def _scale_ptr(t):
    """Device pointer of a float32 scale tensor (one element), or None."""
    if t is None:
        return None
    import torch
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or t.dtype != torch.float32 \
            or t.numel() != 1:
        raise PaError(ERR_INVALID_ARG,
                      "k_scale / v_scale / q_scale must be float32 CUDA tensors of one element")
    return ctypes.c_void_p(t.data_ptr())


def _event_handle(ev):
    if ev is None:
        return None
    return ctypes.c_void_p(int(ev.cuda_event) if hasattr(ev, "cuda_event") else int(ev))


def plan(dims: Dims, window: int, num_kv_heads: int, block_size: int, num_cus: int = 256,
         **opts) -> dict:
    """The launch plan the library would use (no device needed)."""
    p = Plan()
    o = make_options(**opts)
    _check(load().pa_plan_compute(ctypes.byref(dims), int(window), int(num_kv_heads),
                                  int(block_size), int(num_cus), ctypes.byref(o), ctypes.byref(p)))
    return p.as_dict()


def workspace_size(dims: Dims, window: int, num_kv_heads: int, block_size: int, **opts) -> int:
    n = ctypes.c_size_t(0)
    o = make_options(**opts)
    _check(load().pa_decode_workspace_size_ex(ctypes.byref(dims), int(window), int(num_kv_heads),
                                              int(block_size), ctypes.byref(o), ctypes.byref(n)))
    return int(n.value)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise PaError(ERR_INVALID_ARG, f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _stream_handle(stream, device=None):
    """Handle of ``stream``, or of the current stream of ``device`` (default:
    the current device); a given stream must belong to ``device``."""
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    elif device is not None and stream.device != torch.device(device):
        raise PaError(ERR_INVALID_ARG, f"stream is on {stream.device}, the tensors on {device}")
    return ctypes.c_void_p(int(stream.cuda_stream))


def _same_device(dev, **tensors):
    for name, t in tensors.items():
        if t is not None and t.device != dev:
            raise PaError(ERR_INVALID_ARG, f"{name} is on {t.device}, the call's tensors on {dev}")


def _kv_format(k_cache) -> int:
    import torch
    return KV_FP8_E4M3 if k_cache.dtype == torch.float8_e4m3fn else KV_NATIVE


def _q_format(q) -> int:
    import torch
    return Q_FP8_E4M3 if q.dtype == torch.float8_e4m3fn else Q_NATIVE


def dims_for(q, k_cache, block_tables, max_query_len, max_seq_len) -> Dims:
    """Dims of a call; an FP8 query implies a bf16 out (the only one it takes)."""
    T, Hq, D = q.shape
    qf = _q_format(q)
    return make_dims(block_tables.shape[0], Hq, D, max_query_len, max_seq_len,
                     block_tables.shape[1], k_cache.shape[0],
                     BF16 if qf == Q_FP8_E4M3 else _dtype_code(q), _kv_format(k_cache), qf)


def _validate(out, q, k_cache, v_cache, block_tables, seq_lens, query_lens, num_kv_heads, block_size):
    import torch
    for name, t in (("out", out), ("q", q), ("k_cache", k_cache), ("v_cache", v_cache),
                    ("block_tables", block_tables), ("seq_lens", seq_lens),
                    ("query_lens", query_lens)):
        if not isinstance(t, torch.Tensor):
            raise PaError(ERR_INVALID_ARG, f"{name} must be a torch.Tensor")
        if t.device.type != "cuda":
            raise PaError(ERR_INVALID_ARG, f"{name} must be on the GPU")
        if not t.is_contiguous():
            raise PaError(ERR_INVALID_ARG, f"{name} must be contiguous")
    for name, t in (("out", out), ("k_cache", k_cache), ("v_cache", v_cache),
                    ("block_tables", block_tables), ("seq_lens", seq_lens),
                    ("query_lens", query_lens)):
        if t.device != q.device:
            raise PaError(ERR_INVALID_ARG, f"{name} is on {t.device}, q on {q.device}: one GPU per call")
    for name, t in (("block_tables", block_tables), ("seq_lens", seq_lens), ("query_lens", query_lens)):
        if t.dtype != torch.int32:
            raise PaError(ERR_INVALID_ARG, f"{name} must be int32")
    fp8 = k_cache.dtype == torch.float8_e4m3fn
    q8 = q.dtype == torch.float8_e4m3fn
    if q8:
        if not fp8 or v_cache.dtype != torch.float8_e4m3fn or out.dtype != torch.bfloat16:
            raise PaError(ERR_INVALID_ARG, "an FP8 q needs FP8 k_cache / v_cache and a bf16 out")
    elif q.dtype != out.dtype:
        raise PaError(ERR_INVALID_ARG, "q and out must share one dtype")
    elif fp8:
        if v_cache.dtype != torch.float8_e4m3fn or q.dtype != torch.bfloat16:
            raise PaError(ERR_INVALID_ARG, "an FP8 k_cache needs an FP8 v_cache and bf16 q / out")
    elif not (q.dtype == k_cache.dtype == v_cache.dtype):
        raise PaError(ERR_INVALID_ARG, "q, k_cache, v_cache and out must share one dtype")
    if q.dim() != 3 or out.shape != q.shape:
        raise PaError(ERR_INVALID_ARG, "q and out must be [T, H_q, D] of one shape")
    T, Hq, D = q.shape
    nb = k_cache.shape[0]
    E = 16 if fp8 else 8                     # elements per 16-byte column / V group
    if D % E:                                # head dims off the column grid: a row per slot
        if tuple(k_cache.shape) != (nb, num_kv_heads, block_size, D):
            raise PaError(ERR_INVALID_ARG, f"k_cache must be [num_blocks, {num_kv_heads}, "
                                           f"{block_size}, {D}] (head dim not a multiple of {E})")
    elif block_size % 16 or tuple(k_cache.shape) != (nb, num_kv_heads, block_size // 16, 2,
                                                     D // E, 8, E):
        raise PaError(ERR_INVALID_ARG, f"k_cache must be [num_blocks, {num_kv_heads}, "
                                       f"{block_size // 16}, 2, {D // E}, 8, {E}] (16-slot tiles)")
    if block_size % E or tuple(v_cache.shape) != (nb, num_kv_heads, block_size // E, D, E):
        raise PaError(ERR_INVALID_ARG, f"v_cache must be [num_blocks, {num_kv_heads}, "
                                       f"{block_size // E}, {D}, {E}]")
    B = block_tables.shape[0]
    if block_tables.dim() != 2 or seq_lens.shape != (B,) or query_lens.shape != (B,):
        raise PaError(ERR_INVALID_ARG, "block_tables [B, M], seq_lens [B], query_lens [B]")


def _nbytes(t) -> int:
    """Size in bytes of a tensor's storage as the library sees it."""
    return int(t.numel()) * int(t.element_size())


def decode(out, q, k_cache, v_cache, block_tables, seq_lens, query_lens, scale, window,
           num_kv_heads, block_size, max_seq_len, max_query_len, workspace=None,
           stream=None, path=0, part_size=0, waves=0, event_begin=None, event_end=None,
           schedule=0, loads=0, k_scale=None, v_scale=None, q_scale=None):
    """Runs pa_decode_ex on torch tensors; returns ``out``.

    ``max_seq_len`` / ``max_query_len`` are host-known upper bounds of the
    device arrays ``seq_lens`` / ``query_lens`` (the library never reads
    device memory from the host); both are required, since the plan (rows
    per KV head, workspace size, schedule) scales with ``max_query_len``.
    ``workspace`` (CUDA tensor of any dtype, 256-byte aligned) is allocated
    when not given and needed.
    """
    import torch
    _validate(out, q, k_cache, v_cache, block_tables, seq_lens, query_lens, num_kv_heads, block_size)
    if q.shape[0] == 0:
        return out          # no query token in the batch: nothing to compute, nothing to call
    dims = dims_for(q, k_cache, block_tables, max_query_len, max_seq_len)
    opts = make_options(path, part_size, waves, event_begin, event_end, schedule, loads,
                        k_scale, v_scale, q_scale)
    _same_device(q.device, workspace=workspace, k_scale=k_scale, v_scale=v_scale, q_scale=q_scale)
    with torch.cuda.device(q.device):   # the library sizes its plan for the current device
        need = workspace_size(dims, window, num_kv_heads, block_size, path=path,
                              part_size=part_size, waves=waves, schedule=schedule)
        if workspace is None and need:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        ws_ptr = ctypes.c_void_p(workspace.data_ptr()) if workspace is not None else None
        ws_bytes = _nbytes(workspace) if workspace is not None else 0
        _check(load().pa_decode_ex(
            ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(q.data_ptr()),
            ctypes.c_void_p(k_cache.data_ptr()), ctypes.c_void_p(v_cache.data_ptr()),
            ctypes.c_void_p(block_tables.data_ptr()), ctypes.c_void_p(seq_lens.data_ptr()),
            ctypes.c_void_p(query_lens.data_ptr()), ctypes.c_float(scale), int(window),
            int(num_kv_heads), int(block_size), ctypes.byref(dims), ws_ptr, ws_bytes,
            _stream_handle(stream, q.device), ctypes.byref(opts)))
    return out


def decode_noalloc(out, q, k_cache, v_cache, block_tables, seq_lens, query_lens, scale, window,
                   num_kv_heads, block_size, max_seq_len, max_query_len, stream=None, path=0,
                   part_size=0, waves=0, schedule=0, loads=0, k_scale=None, v_scale=None,
                   q_scale=None):
    """Runs pa_decode_noalloc on torch tensors (no workspace: the library's
    static per-GPU scratch holds the partial states); returns ``out``."""
    import torch
    _validate(out, q, k_cache, v_cache, block_tables, seq_lens, query_lens, num_kv_heads, block_size)
    if q.shape[0] == 0:
        return out          # no query token in the batch: nothing to compute, nothing to call
    dims = dims_for(q, k_cache, block_tables, max_query_len, max_seq_len)
    opts = make_options(path, part_size, waves, None, None, schedule, loads, k_scale, v_scale,
                        q_scale)
    _same_device(q.device, k_scale=k_scale, v_scale=v_scale, q_scale=q_scale)
    with torch.cuda.device(q.device):   # the scratch used is the current device's
        _check(load().pa_decode_noalloc(
            ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(q.data_ptr()),
            ctypes.c_void_p(k_cache.data_ptr()), ctypes.c_void_p(v_cache.data_ptr()),
            ctypes.c_void_p(block_tables.data_ptr()), ctypes.c_void_p(seq_lens.data_ptr()),
            ctypes.c_void_p(query_lens.data_ptr()), ctypes.c_float(scale), int(window),
            int(num_kv_heads), int(block_size), ctypes.byref(dims), _stream_handle(stream, q.device),
            ctypes.byref(opts)))
    return out


def pack_kv_cache(k_rows, v_rows, k_cache=None, v_cache=None, block_ids=None, stream=None):
    """Repacks row-layout caches [num_blocks, H_kv, block_size, D] (float32,
    bfloat16 or float8_e4m3fn) into the library's tiled layouts with
    pa_pack_kv_cache; returns (k_cache, v_cache).  Without destination
    tensors they are allocated; with ``block_ids`` (int32 CUDA tensor) only
    those blocks are repacked into the given destinations."""
    import torch
    for name, t in (("k_rows", k_rows), ("v_rows", v_rows)):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or not t.is_contiguous() \
                or t.dim() != 4:
            raise PaError(ERR_INVALID_ARG, f"{name} must be a contiguous 4-d CUDA tensor")
    if k_rows.shape != v_rows.shape or k_rows.dtype != v_rows.dtype:
        raise PaError(ERR_INVALID_ARG, "k_rows and v_rows must share shape and dtype")
    nb, hkv, bs, D = k_rows.shape
    fp8 = k_rows.dtype == torch.float8_e4m3fn
    dtype = BF16 if fp8 else _dtype_code(k_rows)
    E = 16 if fp8 else 8
    if k_cache is None:
        kshape = (nb, hkv, bs // 16, 2, D // E, 8, E) if D % E == 0 else (nb, hkv, bs, D)
        k_cache = torch.empty(kshape, dtype=k_rows.dtype, device=k_rows.device)
    if v_cache is None:
        v_cache = torch.empty((nb, hkv, bs // E, D, E), dtype=k_rows.dtype, device=k_rows.device)
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        if t.numel() != k_rows.numel() or t.dtype != k_rows.dtype or not t.is_contiguous():
            raise PaError(ERR_INVALID_ARG, f"{name} must match k_rows in size and dtype")
    if block_ids is not None and (block_ids.dtype != torch.int32 or block_ids.device.type != "cuda"):
        raise PaError(ERR_INVALID_ARG, "block_ids must be an int32 CUDA tensor")
    dev = k_rows.device
    _same_device(dev, v_rows=v_rows, k_cache=k_cache, v_cache=v_cache, block_ids=block_ids)
    with torch.cuda.device(dev):
        _check(load().pa_pack_kv_cache(
            ctypes.c_void_p(k_rows.data_ptr()), ctypes.c_void_p(v_rows.data_ptr()),
            ctypes.c_void_p(k_cache.data_ptr()), ctypes.c_void_p(v_cache.data_ptr()),
            ctypes.c_void_p(block_ids.data_ptr()) if block_ids is not None else None,
            int(block_ids.numel()) if block_ids is not None else 0, int(nb), int(hkv), int(bs),
            int(D), int(dtype), KV_FP8_E4M3 if fp8 else KV_NATIVE, _stream_handle(stream, dev)))
    return k_cache, v_cache


def noalloc_scratch_bytes() -> int:
    """Size of the static scratch pa_decode_noalloc uses on each GPU."""
    return int(load().pa_noalloc_scratch_bytes())


def stream_read(src, sink, slab=False, stream=None) -> int:
    """pa_stream_read over the bytes of the contiguous CUDA tensor ``src``
    into the int32 CUDA tensor ``sink`` (one workgroup per element at most;
    ``slab``: a contiguous slab per workgroup instead of a grid stride);
    returns the workgroups launched (the XOR of ``sink[:n]`` is the XOR of
    every 32-bit word of ``src``)."""
    import torch
    if not isinstance(src, torch.Tensor) or src.device.type != "cuda" or not src.is_contiguous():
        raise PaError(ERR_INVALID_ARG, "src must be a contiguous CUDA tensor")
    if not isinstance(sink, torch.Tensor) or sink.device.type != "cuda" or sink.dtype != torch.int32:
        raise PaError(ERR_INVALID_ARG, "sink must be an int32 CUDA tensor")
    _same_device(src.device, sink=sink)
    n = ctypes.c_int32(0)
    with torch.cuda.device(src.device):
        _check(load().pa_stream_read(ctypes.c_void_p(src.data_ptr()), _nbytes(src),
                                     ctypes.c_void_p(sink.data_ptr()), int(sink.numel()),
                                     1 if slab else 0, ctypes.byref(n),
                                     _stream_handle(stream, src.device)))
    return int(n.value)


def debug_spans(block_tables, seq_lens, query_lens, window, num_kv_heads, block_size, dims: Dims,
                total_q: int, stream=None, **opts) -> dict:
    """Index facts from the kernels' own helpers (see pa_debug_spans)."""
    import torch
    p = plan(dims, window, num_kv_heads, block_size, **opts)
    dev = block_tables.device
    B = dims.batch
    seq_info = torch.full((B, 4), -7, dtype=torch.int32, device=dev)
    row_info = torch.full((max(total_q, 1), 2), -7, dtype=torch.int32, device=dev)
    blocks = torch.full((B, dims.max_blocks_per_seq), -7, dtype=torch.int32, device=dev)
    parts = torch.full((B, p["num_parts"], 2), -7, dtype=torch.int32, device=dev)
    o = make_options(**opts)
    _same_device(dev, seq_lens=seq_lens, query_lens=query_lens)
    with torch.cuda.device(dev):
        _check(load().pa_debug_spans(
            ctypes.c_void_p(block_tables.data_ptr()), ctypes.c_void_p(seq_lens.data_ptr()),
            ctypes.c_void_p(query_lens.data_ptr()), int(window), int(num_kv_heads),
            int(block_size), ctypes.byref(dims), ctypes.byref(o),
            ctypes.c_void_p(seq_info.data_ptr()), ctypes.c_void_p(row_info.data_ptr()),
            ctypes.c_void_p(blocks.data_ptr()), ctypes.c_void_p(parts.data_ptr()),
            _stream_handle(stream, dev)))
    return dict(seq_info=seq_info, row_info=row_info[:total_q], blocks=blocks, parts=parts, plan=p)


class Prepared:
    """A pa_decode_ex call with its arguments marshalled once.

    For timing loops: ``__call__`` re-issues the same call (same tensors, same
    stream) with only the ctypes call itself on the host path.  Tensors must
    stay alive while the object is used.
    """

    def __init__(self, out, q, k_cache, v_cache, block_tables, seq_lens, query_lens, scale, window,
                 num_kv_heads, block_size, max_seq_len, max_query_len, workspace=None,
                 stream=None, path=0, part_size=0, waves=0, event_begin=None, event_end=None,
                 schedule=0, loads=0, k_scale=None, v_scale=None, q_scale=None):
        import torch
        _validate(out, q, k_cache, v_cache, block_tables, seq_lens, query_lens, num_kv_heads,
                  block_size)
        self.dims = dims_for(q, k_cache, block_tables, max_query_len, max_seq_len)
        self.opts = make_options(path, part_size, waves, event_begin, event_end, schedule, loads,
                                 k_scale, v_scale, q_scale)
        self._events = (event_begin, event_end)
        _same_device(q.device, workspace=workspace, k_scale=k_scale, v_scale=v_scale,
                     q_scale=q_scale)
        self._device = q.device.index if q.device.index is not None else torch.cuda.current_device()
        self.plan = plan(self.dims, window, num_kv_heads, block_size,
                         num_cus=torch.cuda.get_device_properties(q.device).multi_processor_count,
                         path=path, part_size=part_size, waves=waves, schedule=schedule,
                         loads=loads)
        with torch.cuda.device(q.device):
            need = workspace_size(self.dims, window, num_kv_heads, block_size, path=path,
                                  part_size=part_size, waves=waves, schedule=schedule)
        if workspace is None and need:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        self.workspace = workspace
        self._keep = (out, q, k_cache, v_cache, block_tables, seq_lens, query_lens, k_scale, v_scale,
                      q_scale)
        self._empty = q.shape[0] == 0
        vp = ctypes.c_void_p
        self.args = (
            vp(out.data_ptr()), vp(q.data_ptr()), vp(k_cache.data_ptr()), vp(v_cache.data_ptr()),
            vp(block_tables.data_ptr()), vp(seq_lens.data_ptr()), vp(query_lens.data_ptr()),
            ctypes.c_float(scale), int(window), int(num_kv_heads), int(block_size),
            ctypes.byref(self.dims),
            vp(workspace.data_ptr()) if workspace is not None else None,
            _nbytes(workspace) if workspace is not None else 0,
            _stream_handle(stream, q.device), ctypes.byref(self.opts))
        self._fn = load().pa_decode_ex

    def set_events(self, event_begin, event_end):
        """Events the library records around the partition kernel on every
        later call (None to stop).  The objects are kept alive here, since
        the library records into them until they are replaced."""
        self._events = (event_begin, event_end)
        self.opts.event_begin = _event_handle(event_begin)
        self.opts.event_end = _event_handle(event_end)

    def __call__(self):
        if self._empty:
            return          # no query token in the batch
        import torch
        if torch.cuda.current_device() != self._device:
            with torch.cuda.device(self._device):
                st = self._fn(*self.args)
        else:
            st = self._fn(*self.args)
        if st:
            _check(st)


def check_inputs(block_tables, seq_lens, query_lens, window, num_kv_heads, block_size, dims: Dims,
                 stream=None) -> dict:
    """Device-side precondition report of a call's lengths and block tables
    (see pa_check_inputs); waits for the stream."""
    import torch
    dev = block_tables.device
    _same_device(dev, seq_lens=seq_lens, query_lens=query_lens)
    report = torch.empty(4, dtype=torch.int32, device=dev)
    with torch.cuda.device(dev):
        s = _stream_handle(stream, dev)
        _check(load().pa_check_inputs(
            ctypes.c_void_p(block_tables.data_ptr()), ctypes.c_void_p(seq_lens.data_ptr()),
            ctypes.c_void_p(query_lens.data_ptr()), int(window), int(num_kv_heads),
            int(block_size), ctypes.byref(dims), ctypes.c_void_p(report.data_ptr()), s))
    (stream or torch.cuda.current_stream(dev)).synchronize()
    r = report.cpu().tolist()
    none = 0x7fffffff
    return dict(bad_lengths=r[0], bad_entries=r[1],
                first_bad_sequence=None if r[2] == none else r[2],
                first_bad_entry=None if r[3] == none else r[3])
