"""Attention over a paged KV cache on AMD MI355X (gfx950).

Thin Python binding over the C ABI of ``libpagedkv.so`` (declared in
``include/paged_kv.h``).  It only marshals arguments: tensors are passed as
device pointers, the stream is torch's current stream, and every step of the
computation runs in the library's HIP kernels.  There is no fallback: the
library is opened on the first call into it, and that call raises ImportError
if ``lib/libpagedkv.so`` is missing (importing the package alone does not, so
``paged_kv_cache_61_amd.build`` can run on a tree that has not been built).

Functions keep the C names:

* ``paged_kv_write(k, v, slot_mapping, kv_cache_layer)``
* ``paged_attention(q, kv_cache_layer, block_table, seq_lens, query_start_loc,
  num_computed_tokens, scale, ...)``
* ``paged_kv_write_rope(k, v, positions, cos_sin_cache, slot_mapping, kv_cache_layer, ...)``
* ``paged_kv_write_int8(k, v, slot_mapping, kv_cache_i8, kv_scales)`` and
  ``paged_attention_int8(q, kv_cache_i8, kv_scales, block_table, ...)`` (INT8 cache)
* ``paged_kv_write_fp8`` / ``paged_attention_fp8`` (FP8 E4M3 cache: uint8 or
  torch.float8_e4m3fn codes, same arguments)
* ``paged_kv_copy_blocks(kv_cache_layer, copies)``
* ``BlockManager`` — the host block manager / step scheduler (``pkv_bm_*``)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "PagedKVError", "paged_kv_write", "paged_attention", "paged_attention_workspace_size",
    "pkv_read_device_error", "pkv_validate_metadata_host", "lib_path", "load_library",
    "DEVERR_SEQ_LEN", "DEVERR_LIMITS", "DEVERR_QSL", "DEVERR_BLOCK_ID", "DEVERR_SLOT",
    "DEVERR_CAPACITY", "DEVERR_POSITION", "BLOCK_SIZE", "paged_kv_copy_blocks", "paged_kv_write_rope",
    "paged_kv_write_int8", "paged_attention_int8", "paged_kv_write_fp8", "paged_attention_fp8",
    "BlockManager", "Step", "paged_attention_noalloc", "NOALLOC_SCRATCH_BYTES", "paged_attention_staging_bytes",
]

BLOCK_SIZE = 16
PKV_F32, PKV_BF16 = 0, 1
PHASE_PLAN, PHASE_PREFILL, PHASE_ROWS, PHASE_REDUCE = 0, 1, 2, 3
NUM_PHASES = 4
DEVERR_SEQ_LEN, DEVERR_LIMITS, DEVERR_QSL = 0x1, 0x2, 0x4
DEVERR_BLOCK_ID, DEVERR_SLOT, DEVERR_CAPACITY = 0x8, 0x10, 0x20
DEVERR_POSITION = 0x40

_HERE = os.path.dirname(os.path.abspath(__file__))


def lib_path() -> str:
    """``lib/libpagedkv.so``, or the library ``PAGED_KV_LIBRARY`` names (the
    sanitizer build, for CPU-side test runs)."""
    return os.environ.get("PAGED_KV_LIBRARY") or os.path.join(_HERE, "lib", "libpagedkv.so")


class PagedKVError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        detail = _lib.pkv_last_error_detail().decode()
        text = _lib.pkv_status_string(status).decode()
        super().__init__(f"{where}: {text} ({status}){': ' + detail if detail else ''}")


class _PkvStep(ctypes.Structure):
    """Mirror of pkv_step (include/paged_kv.h)."""
    _fields_ = [("max_num_seqs", ctypes.c_int32), ("token_budget", ctypes.c_int32),
                ("max_model_len", ctypes.c_int32),
                ("req_ids", ctypes.c_void_p), ("query_start_loc", ctypes.c_void_p),
                ("seq_lens", ctypes.c_void_p), ("num_computed_tokens", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("slot_mapping", ctypes.c_void_p),
                ("copies", ctypes.c_void_p),
                ("num_reqs", ctypes.c_int32), ("num_tokens", ctypes.c_int32),
                ("num_copies", ctypes.c_int32), ("max_query_len", ctypes.c_int32),
                ("max_seq_len", ctypes.c_int32)]


def load_library() -> ctypes.CDLL:
    path = lib_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m paged_kv_cache_61_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    lib.paged_kv_write.argtypes = [vp, vp, vp, vp, i64, i32, i32, i32, i32, vp, vp]
    lib.paged_kv_write.restype = ctypes.c_int
    lib.paged_attention.argtypes = [vp, vp, vp, vp, vp, vp, vp, f32, i32, i64, i32, i32, i32, i32,
                                    i32, i32, i32, i32, vp, sz, vp]
    lib.paged_attention.restype = ctypes.c_int
    lib.paged_attention_profiled.argtypes = lib.paged_attention.argtypes + [vp]
    lib.paged_attention_profiled.restype = ctypes.c_int
    lib.paged_attention_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, f32, i32, i64, i32, i32, i32, i32,
                                            i32, i32, i32, i32, vp, vp]
    lib.paged_attention_noalloc.restype = ctypes.c_int
    lib.paged_attention_workspace_size.argtypes = [i32, i64, i32, i32, i32, i32]
    lib.paged_attention_workspace_size.restype = sz
    lib.paged_attention_staging_bytes.argtypes = [i32, i32, i32, i32, i64]
    lib.paged_attention_staging_bytes.restype = sz
    lib.pkv_read_device_error.argtypes = [vp, vp]
    lib.pkv_read_device_error.restype = i32
    lib.pkv_validate_metadata_host.argtypes = [vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, i32]
    lib.pkv_validate_metadata_host.restype = ctypes.c_int
    lib.pkv_status_string.argtypes = [ctypes.c_int]
    lib.pkv_status_string.restype = ctypes.c_char_p
    lib.pkv_last_error_detail.argtypes = []
    lib.pkv_last_error_detail.restype = ctypes.c_char_p
    lib.paged_kv_write_rope.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, vp, vp, i64, i32, i32, i32, i32,
                                        i32, vp, vp]
    lib.paged_kv_write_rope.restype = ctypes.c_int
    lib.paged_kv_write_int8.argtypes = [vp, vp, vp, vp, vp, i64, i32, i32, i32, i32, vp, vp]
    lib.paged_kv_write_int8.restype = ctypes.c_int
    lib.paged_attention_int8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, f32, i32, i64, i32, i32, i32, i32,
                                         i32, i32, i32, i32, vp, sz, vp, vp]
    lib.paged_attention_int8.restype = ctypes.c_int
    lib.paged_kv_write_fp8.argtypes = lib.paged_kv_write_int8.argtypes
    lib.paged_kv_write_fp8.restype = ctypes.c_int
    lib.paged_attention_fp8.argtypes = lib.paged_attention_int8.argtypes
    lib.paged_attention_fp8.restype = ctypes.c_int
    lib.paged_kv_copy_blocks.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp, vp]
    lib.paged_kv_copy_blocks.restype = ctypes.c_int
    pbm = ctypes.c_void_p
    lib.pkv_bm_create.argtypes = [i32, i32, ctypes.POINTER(pbm)]
    lib.pkv_bm_create.restype = ctypes.c_int
    lib.pkv_bm_destroy.argtypes = [pbm]
    lib.pkv_bm_destroy.restype = None
    lib.pkv_bm_add_request.argtypes = [pbm, i64, i32]
    lib.pkv_bm_add_request_with_prefix.argtypes = [pbm, i64, i32, i64, i32]
    lib.pkv_bm_fork.argtypes = [pbm, i64, i64]
    lib.pkv_bm_append_tokens.argtypes = [pbm, i64, i32]
    lib.pkv_bm_finish.argtypes = [pbm, i64]
    lib.pkv_bm_num_free_blocks.argtypes = [pbm]
    lib.pkv_bm_num_free_blocks.restype = i32
    lib.pkv_bm_request_state.argtypes = [pbm, i64, vp, vp, vp, i32, vp]
    lib.pkv_bm_schedule.argtypes = [pbm, ctypes.POINTER(_PkvStep)]
    lib.pkv_bm_commit.argtypes = [pbm]
    for f in ("pkv_bm_add_request", "pkv_bm_add_request_with_prefix", "pkv_bm_fork", "pkv_bm_append_tokens",
              "pkv_bm_finish", "pkv_bm_request_state", "pkv_bm_schedule", "pkv_bm_commit"):
        getattr(lib, f).restype = ctypes.c_int
    return lib


class _LazyLibrary:
    """Stands for the ctypes library until first use, then opens it.  Every
    binding reaches the C calls through this object, so a missing library
    raises on the first call instead of at import."""
    _handle: Optional[ctypes.CDLL] = None

    def __getattr__(self, name: str):
        if _LazyLibrary._handle is None:
            _LazyLibrary._handle = load_library()
        return getattr(_LazyLibrary._handle, name)


_lib = _LazyLibrary()

EXPORTED_SYMBOLS = ("paged_kv_write", "paged_attention", "paged_attention_profiled", "paged_attention_noalloc",
                    "paged_attention_workspace_size",
                    "pkv_read_device_error", "pkv_validate_metadata_host", "pkv_status_string",
                    "pkv_last_error_detail", "paged_kv_copy_blocks", "paged_kv_write_rope",
                    "paged_kv_write_int8", "paged_attention_int8", "paged_kv_write_fp8", "paged_attention_fp8",
                    "pkv_bm_create", "pkv_bm_destroy", "pkv_bm_add_request",
                    "pkv_bm_add_request_with_prefix", "pkv_bm_fork", "pkv_bm_append_tokens",
                    "pkv_bm_finish", "pkv_bm_num_free_blocks", "pkv_bm_request_state",
                    "pkv_bm_schedule", "pkv_bm_commit")


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return PKV_BF16
    if t == torch.float32:
        return PKV_F32
    raise TypeError(f"unsupported dtype {t}; use bfloat16 or float32")


def _stream_ptr(stream) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _check_dev(name: str, x: torch.Tensor, dtype: Optional[torch.dtype] = None) -> None:
    if not x.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not x.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and x.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {x.dtype}")


def _check_cache_shape(kv_cache_layer: torch.Tensor):
    """The library reads and writes a layer as ``[2, num_blocks, 16, Hkv, D]``
    (V at row ``num_blocks * 16``); any other shape would send its kernels
    past the tensor, so it is refused before anything is enqueued."""
    if kv_cache_layer.dim() != 5 or kv_cache_layer.shape[0] != 2 or kv_cache_layer.shape[2] != BLOCK_SIZE \
            or kv_cache_layer.shape[1] < 1 or kv_cache_layer.shape[3] < 1:
        raise ValueError(f"kv_cache_layer must be [2, num_blocks, 16, num_kv_heads, head_dim], "
                         f"got {tuple(kv_cache_layer.shape)}")
    return tuple(kv_cache_layer.shape)


def _ptr(x: Optional[torch.Tensor]) -> Optional[int]:
    return None if x is None else (x.data_ptr() or None)


def paged_kv_write(k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor,
                   kv_cache_layer: torch.Tensor, device_error: Optional[torch.Tensor] = None,
                   stream=None) -> None:
    """Store ``k, v [T, Hkv, D]`` at ``slot_mapping [T]`` (int64, -1 = skip) in
    ``kv_cache_layer [2, num_blocks, 16, Hkv, D]``.  Enqueued on ``stream``."""
    _, nb, _, hkv, d = _check_cache_shape(kv_cache_layer)
    for n, x in (("k", k), ("v", v), ("kv_cache_layer", kv_cache_layer)):
        _check_dev(n, x, kv_cache_layer.dtype)
    _check_dev("slot_mapping", slot_mapping, torch.int64)
    if device_error is not None:
        _check_dev("device_error", device_error, torch.int32)
    T = k.shape[0]
    if tuple(k.shape) != (T, hkv, d) or tuple(v.shape) != (T, hkv, d) or slot_mapping.shape != (T,):
        raise ValueError("k, v must be [T, num_kv_heads, head_dim] and slot_mapping [T]")
    st = _lib.paged_kv_write(_ptr(k), _ptr(v), _ptr(slot_mapping), _ptr(kv_cache_layer), T, nb,
                             hkv, d, _dtype_code(kv_cache_layer.dtype), _ptr(device_error),
                             _stream_ptr(stream))
    if st != 0:
        raise PagedKVError(st, "paged_kv_write")


def paged_attention_workspace_size(num_reqs: int, num_tokens: int, num_q_heads: int,
                                   head_dim: int, max_query_len: int, max_seq_len: int) -> int:
    return int(_lib.paged_attention_workspace_size(num_reqs, num_tokens, num_q_heads, head_dim,
                                                   max_query_len, max_seq_len))


def paged_attention_staging_bytes(num_reqs: int, max_blocks_per_req: int, num_kv_heads: int,
                                  head_dim: int, prefill_blocks: int) -> int:
    """Extra workspace with which ``paged_attention_int8`` / ``_fp8`` dequantise
    a step's prefill blocks once (steps whose prefill requests read at most
    ``prefill_blocks`` cache blocks in all)."""
    return int(_lib.paged_attention_staging_bytes(num_reqs, max_blocks_per_req, num_kv_heads, head_dim,
                                                  prefill_blocks))


def paged_attention(q: torch.Tensor, kv_cache_layer: torch.Tensor, block_table: torch.Tensor,
                    seq_lens: torch.Tensor, query_start_loc: torch.Tensor,
                    num_computed_tokens: torch.Tensor, scale: float, *, max_query_len: int,
                    max_seq_len: int, out: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None, stream=None,
                    phase_events=None) -> torch.Tensor:
    """Attention of ``q [T, Hq, D]`` over the paged cache; returns ``out [T, Hq, D]``.

    ``max_query_len`` / ``max_seq_len`` are host-side bounds on the step's
    query lengths and sequence lengths.  ``workspace`` (uint8, on the device)
    is allocated when not given.  ``phase_events``: optional sequence of
    ``2 * NUM_PHASES`` ``torch.cuda.Event`` (or None) recorded around the
    library's internal phases (``paged_attention_profiled``)."""
    _, nb, _, hkv, d = _check_cache_shape(kv_cache_layer)
    _check_dev("q", q, kv_cache_layer.dtype)
    _check_dev("kv_cache_layer", kv_cache_layer)
    for n, x in (("block_table", block_table), ("seq_lens", seq_lens),
                 ("query_start_loc", query_start_loc),
                 ("num_computed_tokens", num_computed_tokens)):
        _check_dev(n, x, torch.int32)
    if q.dim() != 3:
        raise ValueError("q must be [T, num_q_heads, head_dim]")
    T, hq, dq = q.shape
    if dq != d:
        raise ValueError("q head_dim differs from the cache's")
    R = seq_lens.shape[0]
    if query_start_loc.shape != (R + 1,) or num_computed_tokens.shape != (R,):
        raise ValueError("query_start_loc must be [R+1], num_computed_tokens [R]")
    if block_table.dim() != 2 or block_table.shape[0] != R:
        raise ValueError("block_table must be [R, max_blocks_per_req]")
    mb = block_table.shape[1]
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_dev("out", out, q.dtype)
        if out.shape != q.shape:
            raise ValueError("out must have q's shape")
    need = paged_attention_workspace_size(R, T, hq, d, max_query_len, max_seq_len)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    else:
        _check_dev("workspace", workspace, torch.uint8)
    args = (_ptr(out), _ptr(q), _ptr(kv_cache_layer), _ptr(block_table), _ptr(seq_lens),
            _ptr(query_start_loc), _ptr(num_computed_tokens), float(scale), R, T, hq, hkv, d, nb,
            max(mb, 1), max_query_len, max_seq_len, _dtype_code(q.dtype), _ptr(workspace),
            workspace.numel(), _stream_ptr(stream))
    if phase_events is None:
        st = _lib.paged_attention(*args)
    else:
        if len(phase_events) != 2 * NUM_PHASES:
            raise ValueError(f"phase_events needs {2 * NUM_PHASES} entries")
        handles = (ctypes.c_void_p * (2 * NUM_PHASES))(
            *[None if e is None else int(e.cuda_event) for e in phase_events])
        st = _lib.paged_attention_profiled(*args, handles)
    if st != 0:
        raise PagedKVError(st, "paged_attention")
    return out


NOALLOC_SCRATCH_BYTES = 128 << 20


def paged_attention_noalloc(q: torch.Tensor, kv_cache_layer: torch.Tensor, block_table: torch.Tensor,
                            seq_lens: torch.Tensor, query_start_loc: torch.Tensor,
                            num_computed_tokens: torch.Tensor, scale: float, *, max_query_len: int,
                            max_seq_len: int, out: torch.Tensor, device_error: Optional[torch.Tensor] = None,
                            stream=None) -> torch.Tensor:
    """``paged_attention`` with its workspace in the library's static device
    scratch (``NOALLOC_SCRATCH_BYTES`` per GPU): nothing is allocated, so
    ``out`` must be given.  ``device_error`` (int32, one element, on the
    device) gets the step's device error bits OR-ed in.  Calls on one GPU share
    the scratch: calls that may overlap must be ordered by the caller."""
    _, nb, _, hkv, d = _check_cache_shape(kv_cache_layer)
    _check_dev("q", q, kv_cache_layer.dtype)
    _check_dev("kv_cache_layer", kv_cache_layer)
    _check_dev("out", out, q.dtype)
    for n, x in (("block_table", block_table), ("seq_lens", seq_lens),
                 ("query_start_loc", query_start_loc),
                 ("num_computed_tokens", num_computed_tokens)):
        _check_dev(n, x, torch.int32)
    if device_error is not None:
        _check_dev("device_error", device_error, torch.int32)
    if q.dim() != 3 or out.shape != q.shape:
        raise ValueError("q and out must be [T, num_q_heads, head_dim]")
    T, hq, dq = q.shape
    if dq != d:
        raise ValueError("q head_dim differs from the cache's")
    R = seq_lens.shape[0]
    if query_start_loc.shape != (R + 1,) or num_computed_tokens.shape != (R,):
        raise ValueError("query_start_loc must be [R+1], num_computed_tokens [R]")
    if block_table.dim() != 2 or block_table.shape[0] != R:
        raise ValueError("block_table must be [R, max_blocks_per_req]")
    st = _lib.paged_attention_noalloc(_ptr(out), _ptr(q), _ptr(kv_cache_layer), _ptr(block_table),
                                      _ptr(seq_lens), _ptr(query_start_loc), _ptr(num_computed_tokens),
                                      float(scale), R, T, hq, hkv, d, nb, max(block_table.shape[1], 1),
                                      max_query_len, max_seq_len, _dtype_code(q.dtype), _ptr(device_error),
                                      _stream_ptr(stream))
    if st != 0:
        raise PagedKVError(st, "paged_attention_noalloc")
    return out


def pkv_read_device_error(workspace: torch.Tensor, stream=None) -> int:
    """Device error word of the last paged_attention call on ``workspace`` (syncs)."""
    return int(_lib.pkv_read_device_error(_ptr(workspace), _stream_ptr(stream)))


def pkv_validate_metadata_host(block_table, seq_lens, query_start_loc, num_computed_tokens,
                               slot_mapping, num_tokens: int, num_blocks: int,
                               max_query_len: int, max_seq_len: int) -> int:
    """Host-only validation of numpy metadata arrays; returns a pkv_status (0 = ok)."""
    import numpy as np
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    qsl = np.ascontiguousarray(query_start_loc, dtype=np.int32)
    nct = np.ascontiguousarray(num_computed_tokens, dtype=np.int32)
    sm = None if slot_mapping is None else np.ascontiguousarray(slot_mapping, dtype=np.int64)
    p = lambda a: None if a is None else a.ctypes.data_as(ctypes.c_void_p)
    return int(_lib.pkv_validate_metadata_host(p(bt), p(sl), p(qsl), p(nct), p(sm), sl.shape[0],
                                               num_tokens, num_blocks, max(bt.shape[1], 1),
                                               max_query_len, max_seq_len))


def last_error_detail() -> str:
    return _lib.pkv_last_error_detail().decode()


def paged_kv_write_rope(k: torch.Tensor, v: torch.Tensor, positions: torch.Tensor,
                        cos_sin_cache: torch.Tensor, slot_mapping: torch.Tensor,
                        kv_cache_layer: torch.Tensor, *, rotary_dim: Optional[int] = None,
                        is_neox: bool = True, q: Optional[torch.Tensor] = None,
                        device_error: Optional[torch.Tensor] = None, stream=None) -> None:
    """``paged_kv_write`` with RoPE applied to K (and to ``q [T, Hq, D]`` in place
    when given).  ``positions [T]`` int64; ``cos_sin_cache [max_position,
    rotary_dim]`` float32, row p = cos of the rotary_dim/2 angles, then sin."""
    _, nb, _, hkv, d = _check_cache_shape(kv_cache_layer)
    for n, x in (("k", k), ("v", v), ("kv_cache_layer", kv_cache_layer)):
        _check_dev(n, x, kv_cache_layer.dtype)
    _check_dev("slot_mapping", slot_mapping, torch.int64)
    _check_dev("positions", positions, torch.int64)
    _check_dev("cos_sin_cache", cos_sin_cache, torch.float32)
    if q is not None:
        _check_dev("q", q, kv_cache_layer.dtype)
    if device_error is not None:
        _check_dev("device_error", device_error, torch.int32)
    T = k.shape[0]
    if tuple(k.shape) != (T, hkv, d) or tuple(v.shape) != (T, hkv, d) or slot_mapping.shape != (T,) \
            or positions.shape != (T,):
        raise ValueError("k, v must be [T, num_kv_heads, head_dim], slot_mapping and positions [T]")
    if q is not None and (q.dim() != 3 or q.shape[0] != T or q.shape[2] != d):
        raise ValueError("q must be [T, num_q_heads, head_dim]")
    rd = cos_sin_cache.shape[1] if rotary_dim is None else rotary_dim
    st = _lib.paged_kv_write_rope(_ptr(q), _ptr(k), _ptr(v), _ptr(positions), _ptr(cos_sin_cache),
                                  cos_sin_cache.shape[0], rd, int(bool(is_neox)), _ptr(slot_mapping),
                                  _ptr(kv_cache_layer), T, 0 if q is None else q.shape[1], nb, hkv, d,
                                  _dtype_code(kv_cache_layer.dtype), _ptr(device_error), _stream_ptr(stream))
    if st != 0:
        raise PagedKVError(st, "paged_kv_write_rope")


_CODE_DTYPES = {"int8": (torch.int8,), "fp8": (torch.uint8, torch.float8_e4m3fn)}


def _check_i8_cache(kv_cache: torch.Tensor, kv_scales: torch.Tensor, fmt: str = "int8"):
    if kv_cache.dtype not in _CODE_DTYPES[fmt]:
        raise TypeError(f"kv_cache_layer must have dtype {' or '.join(map(str, _CODE_DTYPES[fmt]))}, "
                        f"got {kv_cache.dtype}")
    _check_cache_shape(kv_cache)
    _check_dev("kv_cache_layer", kv_cache)
    _check_dev("kv_scales", kv_scales, torch.float32)
    if tuple(kv_scales.shape) != (2, kv_cache.shape[1], kv_cache.shape[3], BLOCK_SIZE):
        raise ValueError("kv_scales must be float32 [2, num_blocks, num_kv_heads, 16]")


def paged_kv_write_int8(k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor,
                        kv_cache_layer: torch.Tensor, kv_scales: torch.Tensor,
                        device_error: Optional[torch.Tensor] = None, stream=None) -> None:
    """Quantise ``k, v [T, Hkv, D]`` (bf16 / fp32) into the INT8 cache at ``slot_mapping``."""
    _kv_write_8bit("int8", k, v, slot_mapping, kv_cache_layer, kv_scales, device_error, stream)


def paged_kv_write_fp8(k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor,
                       kv_cache_layer: torch.Tensor, kv_scales: torch.Tensor,
                       device_error: Optional[torch.Tensor] = None, stream=None) -> None:
    """Quantise ``k, v [T, Hkv, D]`` (bf16 / fp32) into the FP8 (E4M3) cache at ``slot_mapping``."""
    _kv_write_8bit("fp8", k, v, slot_mapping, kv_cache_layer, kv_scales, device_error, stream)


def _kv_write_8bit(fmt, k, v, slot_mapping, kv_cache_layer, kv_scales, device_error, stream):
    _check_i8_cache(kv_cache_layer, kv_scales, fmt)
    _check_dev("k", k)
    _check_dev("v", v, k.dtype)
    _check_dev("slot_mapping", slot_mapping, torch.int64)
    if device_error is not None:
        _check_dev("device_error", device_error, torch.int32)
    _, nb, _, hkv, d = kv_cache_layer.shape
    T = k.shape[0]
    if tuple(k.shape) != (T, hkv, d) or tuple(v.shape) != (T, hkv, d) or slot_mapping.shape != (T,):
        raise ValueError("k, v must be [T, num_kv_heads, head_dim] and slot_mapping [T]")
    fn = getattr(_lib, f"paged_kv_write_{fmt}")
    st = fn(_ptr(k), _ptr(v), _ptr(slot_mapping), _ptr(kv_cache_layer), _ptr(kv_scales),
            T, nb, hkv, d, _dtype_code(k.dtype), _ptr(device_error), _stream_ptr(stream))
    if st != 0:
        raise PagedKVError(st, f"paged_kv_write_{fmt}")


def paged_attention_int8(q: torch.Tensor, kv_cache_layer: torch.Tensor, kv_scales: torch.Tensor,
                         block_table: torch.Tensor, seq_lens: torch.Tensor, query_start_loc: torch.Tensor,
                         num_computed_tokens: torch.Tensor, scale: float, *, max_query_len: int,
                         max_seq_len: int, out: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None, stream=None,
                         phase_events=None) -> torch.Tensor:
    """``paged_attention`` over an INT8 cache (``kv_cache_layer`` int8 codes,
    ``kv_scales`` float32 per (token, kv head)); ``q`` / ``out`` bf16 or fp32.
    A ``workspace`` larger than ``paged_attention_workspace_size`` (by
    ``paged_attention_staging_bytes``) lets the prefill read blocks
    dequantised once per step."""
    return _attention_8bit("int8", q, kv_cache_layer, kv_scales, block_table, seq_lens, query_start_loc,
                           num_computed_tokens, scale, max_query_len, max_seq_len, out, workspace, stream,
                           phase_events)


def paged_attention_fp8(q: torch.Tensor, kv_cache_layer: torch.Tensor, kv_scales: torch.Tensor,
                        block_table: torch.Tensor, seq_lens: torch.Tensor, query_start_loc: torch.Tensor,
                        num_computed_tokens: torch.Tensor, scale: float, *, max_query_len: int,
                        max_seq_len: int, out: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None, stream=None,
                        phase_events=None) -> torch.Tensor:
    """``paged_attention`` over an FP8 cache (``kv_cache_layer`` E4M3 codes as
    uint8 or float8_e4m3fn, ``kv_scales`` float32 per (token, kv head));
    ``q`` / ``out`` bf16 or fp32.  Workspace and staging as for
    ``paged_attention_int8``."""
    return _attention_8bit("fp8", q, kv_cache_layer, kv_scales, block_table, seq_lens, query_start_loc,
                           num_computed_tokens, scale, max_query_len, max_seq_len, out, workspace, stream,
                           phase_events)


def _attention_8bit(fmt, q, kv_cache_layer, kv_scales, block_table, seq_lens, query_start_loc,
                    num_computed_tokens, scale, max_query_len, max_seq_len, out, workspace, stream,
                    phase_events):
    _check_i8_cache(kv_cache_layer, kv_scales, fmt)
    _check_dev("q", q)
    if q.dim() != 3:
        raise ValueError("q must be [T, num_q_heads, head_dim]")
    for n, x in (("block_table", block_table), ("seq_lens", seq_lens),
                 ("query_start_loc", query_start_loc), ("num_computed_tokens", num_computed_tokens)):
        _check_dev(n, x, torch.int32)
    _, nb, _, hkv, d = kv_cache_layer.shape
    T, hq, dq = q.shape
    if dq != d:
        raise ValueError("q head_dim differs from the cache's")
    R = seq_lens.shape[0]
    if query_start_loc.shape != (R + 1,) or num_computed_tokens.shape != (R,) or block_table.shape[0] != R:
        raise ValueError("query_start_loc must be [R+1], num_computed_tokens [R], block_table [R, *]")
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_dev("out", out, q.dtype)
        if out.shape != q.shape:
            raise ValueError("out must have q's shape")
    need = paged_attention_workspace_size(R, T, hq, d, max_query_len, max_seq_len)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    else:
        _check_dev("workspace", workspace, torch.uint8)
    handles = None
    if phase_events is not None:
        if len(phase_events) != 2 * NUM_PHASES:
            raise ValueError(f"phase_events needs {2 * NUM_PHASES} entries")
        handles = (ctypes.c_void_p * (2 * NUM_PHASES))(
            *[None if e is None else int(e.cuda_event) for e in phase_events])
    fn = getattr(_lib, f"paged_attention_{fmt}")
    st = fn(_ptr(out), _ptr(q), _ptr(kv_cache_layer), _ptr(kv_scales), _ptr(block_table),
            _ptr(seq_lens), _ptr(query_start_loc), _ptr(num_computed_tokens),
            float(scale), R, T, hq, hkv, d, nb, max(block_table.shape[1], 1),
            max_query_len, max_seq_len, _dtype_code(q.dtype), _ptr(workspace),
            workspace.numel(), _stream_ptr(stream), handles)
    if st != 0:
        raise PagedKVError(st, f"paged_attention_{fmt}")
    return out


def paged_kv_copy_blocks(kv_cache_layer: torch.Tensor, copies: torch.Tensor,
                         device_error: Optional[torch.Tensor] = None, stream=None) -> None:
    """Copy whole blocks of ``kv_cache_layer`` (K and V): ``copies [C, 2]`` int32
    on the device holds (source, destination) block ids.  Enqueued on ``stream``."""
    _, nb, _, hkv, d = _check_cache_shape(kv_cache_layer)
    _check_dev("kv_cache_layer", kv_cache_layer)
    _check_dev("copies", copies, torch.int32)
    if device_error is not None:
        _check_dev("device_error", device_error, torch.int32)
    if copies.dim() != 2 or copies.shape[1] != 2:
        raise ValueError("copies must be [C, 2]")
    st = _lib.paged_kv_copy_blocks(_ptr(kv_cache_layer), _ptr(copies), copies.shape[0], nb, hkv, d,
                                   _dtype_code(kv_cache_layer.dtype), _ptr(device_error),
                                   _stream_ptr(stream))
    if st != 0:
        raise PagedKVError(st, "paged_kv_copy_blocks")


class Step:
    """One scheduled step (host numpy arrays, trimmed to the step's sizes)."""

    def __init__(self, **kw):
        self.__dict__.update(kw)

    @property
    def num_reqs(self) -> int:
        return int(self.req_ids.shape[0])

    @property
    def num_tokens(self) -> int:
        return int(self.slot_mapping.shape[0])


class BlockManager:
    """Host block manager and step scheduler of libpagedkv (``pkv_bm_*``).

    Method names follow the C calls: ``add_request``, ``fork``,
    ``append_tokens``, ``finish``, ``schedule`` (returns a :class:`Step` of
    numpy arrays), ``commit``, ``num_free_blocks``, ``request_state``."""

    def __init__(self, num_blocks: int, max_blocks_per_req: int):
        h = ctypes.c_void_p()
        self._check(_lib.pkv_bm_create(num_blocks, max_blocks_per_req, ctypes.byref(h)), "pkv_bm_create")
        self._h = h
        self._destroy = _lib.pkv_bm_destroy  # kept: module globals may be gone at exit
        self.num_blocks = num_blocks
        self.max_blocks_per_req = max_blocks_per_req

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            self._destroy(h)
            self._h = None

    @staticmethod
    def _check(st: int, where: str) -> None:
        if st != 0:
            raise PagedKVError(st, where)

    def add_request(self, req_id: int, num_prompt_tokens: int, prefix_from: Optional[int] = None,
                    prefix_tokens: int = 0) -> None:
        if prefix_from is None:
            self._check(_lib.pkv_bm_add_request(self._h, req_id, num_prompt_tokens), "pkv_bm_add_request")
        else:
            self._check(_lib.pkv_bm_add_request_with_prefix(self._h, req_id, num_prompt_tokens, prefix_from,
                                                            prefix_tokens), "pkv_bm_add_request_with_prefix")

    def fork(self, parent_id: int, child_id: int) -> None:
        self._check(_lib.pkv_bm_fork(self._h, parent_id, child_id), "pkv_bm_fork")

    def append_tokens(self, req_id: int, n: int = 1) -> None:
        self._check(_lib.pkv_bm_append_tokens(self._h, req_id, n), "pkv_bm_append_tokens")

    def finish(self, req_id: int) -> None:
        self._check(_lib.pkv_bm_finish(self._h, req_id), "pkv_bm_finish")

    def num_free_blocks(self) -> int:
        return int(_lib.pkv_bm_num_free_blocks(self._h))

    def request_state(self, req_id: int):
        """(num_tokens, num_computed_tokens, [block ids])"""
        import numpy as np
        nt, nc, nb = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        blocks = np.zeros(self.max_blocks_per_req, np.int32)
        self._check(_lib.pkv_bm_request_state(self._h, req_id, ctypes.byref(nt), ctypes.byref(nc),
                                              blocks.ctypes.data_as(ctypes.c_void_p), blocks.shape[0],
                                              ctypes.byref(nb)), "pkv_bm_request_state")
        return nt.value, nc.value, blocks[:nb.value].tolist()

    def schedule(self, max_num_seqs: int, token_budget: int, max_model_len: int) -> Step:
        import numpy as np
        a = dict(req_ids=np.zeros(max_num_seqs, np.int64),
                 query_start_loc=np.zeros(max_num_seqs + 1, np.int32),
                 seq_lens=np.zeros(max_num_seqs, np.int32),
                 num_computed_tokens=np.zeros(max_num_seqs, np.int32),
                 block_table=np.zeros((max_num_seqs, self.max_blocks_per_req), np.int32),
                 slot_mapping=np.zeros(token_budget, np.int64),
                 copies=np.zeros((max_num_seqs, 2), np.int32))
        p = lambda x: x.ctypes.data_as(ctypes.c_void_p)
        st = _PkvStep(max_num_seqs, token_budget, max_model_len, p(a["req_ids"]), p(a["query_start_loc"]),
                      p(a["seq_lens"]), p(a["num_computed_tokens"]), p(a["block_table"]),
                      p(a["slot_mapping"]), p(a["copies"]), 0, 0, 0, 0, 0)
        self._check(_lib.pkv_bm_schedule(self._h, ctypes.byref(st)), "pkv_bm_schedule")
        R, T, C = st.num_reqs, st.num_tokens, st.num_copies
        return Step(req_ids=a["req_ids"][:R].copy(), query_start_loc=a["query_start_loc"][:R + 1].copy(),
                    seq_lens=a["seq_lens"][:R].copy(), num_computed_tokens=a["num_computed_tokens"][:R].copy(),
                    block_table=a["block_table"][:R].copy(), slot_mapping=a["slot_mapping"][:T].copy(),
                    copies=a["copies"][:C].copy(), max_query_len=st.max_query_len,
                    max_seq_len=st.max_seq_len)

    def commit(self) -> None:
        self._check(_lib.pkv_bm_commit(self._h), "pkv_bm_commit")
