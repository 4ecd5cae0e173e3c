"""ctypes binding of libattnsink.so (argument marshalling only).

Each function here has the name of the C entry point it calls and does nothing but
check tensor placement/dtype/shape, allocate outputs with torch when the caller passes
none, and forward raw device pointers plus the current HIP stream. All arithmetic runs
in the library's HIP kernels. Importing this module raises if the library has not been
built: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

from .build import LIB_PATH

__all__ = [
    "lib", "AttnSinkError", "attn_sink_prefill", "attn_sink_prefill_paged", "attn_sink_decode_paged",
    "attn_sink_decode_paged_partials", "attn_sink_decode_paged_tree", "attn_sink_rope_append",
    "attn_sink_decode_workspace_size",
    "attn_sink_merge_partials", "attn_sink_status_string", "attn_sink_version", "decode_workspace_layout",
    "attn_sink_decode_workspace_layout", "attn_sink_decode_paged_noalloc", "attn_sink_decode_noalloc_capacity",
    "attn_sink_decode_paged_tree_partials", "attn_sink_decode_paged_range_partials", "attn_sink_decode_plan_chunk",
    "EXPORTED_SYMBOLS",
]

EXPORTED_SYMBOLS = (
    "attn_sink_prefill", "attn_sink_prefill_paged", "attn_sink_decode_paged", "attn_sink_decode_paged_partials",
    "attn_sink_decode_paged_tree", "attn_sink_rope_append",
    "attn_sink_decode_workspace_size", "attn_sink_decode_workspace_layout", "attn_sink_merge_partials",
    "attn_sink_status_string", "attn_sink_version", "attn_sink_decode_paged_noalloc",
    "attn_sink_decode_noalloc_capacity", "attn_sink_decode_paged_tree_partials",
    "attn_sink_decode_paged_range_partials", "attn_sink_decode_plan_chunk",
)

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python -m gqa_attention_sinks_sink_amd.build` "
                      "(or __graft_entry__.build()) first")

lib = ctypes.CDLL(LIB_PATH)

_i32, _f32, _vp, _sz = ctypes.c_int32, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
_fp = ctypes.c_void_p  # float* / int32_t* passed as raw addresses

lib.attn_sink_prefill.restype = ctypes.c_int
lib.attn_sink_prefill.argtypes = [_vp, _vp, _vp, _fp, _fp, _fp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                  _f32, _i32, _i32, _vp, _fp, _vp]
lib.attn_sink_prefill_paged.restype = ctypes.c_int
lib.attn_sink_prefill_paged.argtypes = [_vp, _vp, _vp, _fp, _i32, _i32, _fp, _fp, _fp, _i32, _i32, _i32, _i32, _i32,
                                        _i32, _i32, _i32, _f32, _i32, _i32, _vp, _fp, _vp]
lib.attn_sink_decode_paged_tree.restype = ctypes.c_int
lib.attn_sink_decode_paged_tree.argtypes = [_vp, _vp, _vp, _fp, _i32, _i32, _fp, _fp, _fp, _i32, _i32, _i32, _i32, _i32,
                                            _i32, _i32, _f32, _i32, _i32, _vp, _sz, _vp, _fp, _vp]
lib.attn_sink_rope_append.restype = ctypes.c_int
lib.attn_sink_rope_append.argtypes = [_vp, _vp, _vp, _fp, _fp, _fp, _i32, _i32, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                      _i32, _i32, _i32, _f32, _f32, _i32, _f32, _f32, _i32, _vp, _vp]
lib.attn_sink_decode_paged.restype = ctypes.c_int
lib.attn_sink_decode_paged.argtypes = [_vp, _vp, _vp, _fp, _i32, _i32, _fp, _fp, _i32, _i32, _i32, _i32, _i32,
                                       _i32, _i32, _f32, _i32, _i32, _i32, _vp, _sz, _vp, _fp, _vp]
lib.attn_sink_decode_paged_partials.restype = ctypes.c_int
lib.attn_sink_decode_paged_partials.argtypes = [_vp, _vp, _vp, _fp, _i32, _i32, _fp, _fp, _i32, _i32, _i32, _i32,
                                                _i32, _i32, _i32, _f32, _i32, _i32, _i32, _vp, _sz, _vp]
lib.attn_sink_decode_paged_noalloc.restype = ctypes.c_int
lib.attn_sink_decode_paged_noalloc.argtypes = [_vp, _vp, _vp, _fp, _i32, _i32, _fp, _fp, _i32, _i32, _i32, _i32, _i32,
                                               _i32, _i32, _f32, _i32, _i32, _i32, _vp, _fp, _vp]
lib.attn_sink_decode_noalloc_capacity.restype = _sz
lib.attn_sink_decode_noalloc_capacity.argtypes = []
lib.attn_sink_decode_paged_tree_partials.restype = ctypes.c_int
lib.attn_sink_decode_paged_tree_partials.argtypes = [_vp, _vp, _vp, _fp, _i32, _i32, _fp, _fp, _fp, _i32, _i32, _i32,
                                                     _i32, _i32, _i32, _i32, _f32, _i32, _i32, _vp, _sz, _vp]
lib.attn_sink_decode_paged_range_partials.restype = ctypes.c_int
lib.attn_sink_decode_paged_range_partials.argtypes = [_vp, _vp, _vp, _fp, _i32, _i32, _fp, _fp, _fp, _fp, _i32, _i32,
                                                      _i32, _i32, _i32, _i32, _i32, _f32, _i32, _i32, _i32, _vp,
                                                      _sz, _vp]
lib.attn_sink_decode_plan_chunk.restype = ctypes.c_int
lib.attn_sink_decode_plan_chunk.argtypes = [_vp, _i32, _i32, _i32, _i32, _i32, _i32, ctypes.POINTER(ctypes.c_int32)]
lib.attn_sink_decode_workspace_size.restype = _sz
lib.attn_sink_decode_workspace_size.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32]
lib.attn_sink_decode_workspace_layout.restype = ctypes.c_int
lib.attn_sink_decode_workspace_layout.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32, _vp]
lib.attn_sink_merge_partials.restype = ctypes.c_int
lib.attn_sink_merge_partials.argtypes = [_fp, _fp, _i32, _fp, _i32, _i32, _i32, _vp, _fp, _vp]
lib.attn_sink_status_string.restype = ctypes.c_char_p
lib.attn_sink_status_string.argtypes = [ctypes.c_int]
lib.attn_sink_version.restype = ctypes.c_char_p
lib.attn_sink_version.argtypes = []


class AttnSinkError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {attn_sink_status_string(status)} (status {status})")
        self.status = status


def attn_sink_status_string(status: int) -> str:
    return lib.attn_sink_status_string(int(status)).decode()


def attn_sink_version() -> str:
    return lib.attn_sink_version().decode()


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(t: torch.Tensor, name: str, dtype: torch.dtype, device: torch.device):
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _raise(status: int, where: str):
    if status != 0:
        raise AttnSinkError(status, where)


def attn_sink_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, sinks: Optional[torch.Tensor],
                      cu_seqlens_q: torch.Tensor, cu_seqlens_kv: torch.Tensor, max_seqlen_q: int, max_seqlen_kv: int,
                      softmax_scale: Optional[float] = None, causal: bool = True, window: int = 0,
                      out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                      return_lse: bool = True, stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """q [total_q, hq, 64], k/v [total_kv, hkv, 64] bf16; sinks fp32 [hq] or None; cu_seqlens int32 [batch+1]."""
    dev = q.device
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, torch.bfloat16, dev)
    _check(cu_seqlens_q, "cu_seqlens_q", torch.int32, dev)
    _check(cu_seqlens_kv, "cu_seqlens_kv", torch.int32, dev)
    if sinks is not None:
        _check(sinks, "sinks", torch.float32, dev)
    if q.dim() != 3 or k.dim() != 3 or v.shape != k.shape or k.shape[2] != q.shape[2]:
        raise ValueError(f"expected q [T, hq, d] and k, v [T_kv, hkv, d]; got {tuple(q.shape)}, {tuple(k.shape)}, "
                         f"{tuple(v.shape)}")
    total_q, hq, d = q.shape
    total_kv, hkv = k.shape[0], k.shape[1]
    batch = cu_seqlens_q.numel() - 1
    if cu_seqlens_kv.numel() != batch + 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_kv must have the same length")
    if sinks is not None and sinks.numel() != hq:
        raise ValueError(f"sinks must have {hq} entries")
    if out is not None:
        _check(out, "out", torch.bfloat16, dev)
        if out.shape != q.shape:
            raise ValueError("out must have the shape of q")
    if lse is not None:
        _check(lse, "lse", torch.float32, dev)
        if lse.shape != (total_q, hq):
            raise ValueError(f"lse must be [{total_q}, {hq}]")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((total_q, hq), dtype=torch.float32, device=dev)
    st = lib.attn_sink_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(sinks), _ptr(cu_seqlens_q), _ptr(cu_seqlens_kv),
                               batch, total_q, total_kv, int(max_seqlen_q), int(max_seqlen_kv), hq, hkv, d,
                               float(softmax_scale), int(bool(causal)), int(window), _ptr(out), _ptr(lse),
                               _stream(stream))
    _raise(st, "attn_sink_prefill")
    return out, lse


def attn_sink_prefill_paged(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, page_table: torch.Tensor,
                            cu_seqlens_q: torch.Tensor, kv_lens: torch.Tensor, sinks: Optional[torch.Tensor],
                            max_seqlen_q: int, max_kv_len: int, softmax_scale: Optional[float] = None,
                            causal: bool = True, window: int = 0, out: Optional[torch.Tensor] = None,
                            lse: Optional[torch.Tensor] = None, return_lse: bool = True,
                            stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """q [total_q, hq, 64] bf16 (each sequence's newest tokens); caches [num_pages, hkv, page_size, 64] bf16;
    page_table int32 [batch, max_pages]; cu_seqlens_q int32 [batch+1]; kv_lens int32 [batch] (chunk included)."""
    dev = q.device
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _check(t, n, torch.bfloat16, dev)
    for t, n in ((page_table, "page_table"), (cu_seqlens_q, "cu_seqlens_q"), (kv_lens, "kv_lens")):
        _check(t, n, torch.int32, dev)
    if sinks is not None:
        _check(sinks, "sinks", torch.float32, dev)
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape or k_cache.shape[3] != q.shape[2]:
        raise ValueError(f"expected q [T, hq, d] and caches [pages, hkv, page_size, d]; got {tuple(q.shape)}, "
                         f"{tuple(k_cache.shape)}, {tuple(v_cache.shape)}")
    total_q, hq, d = q.shape
    num_pages, hkv, page_size = k_cache.shape[0], k_cache.shape[1], k_cache.shape[2]
    batch = cu_seqlens_q.numel() - 1
    if kv_lens.numel() != batch or page_table.dim() != 2 or page_table.shape[0] != batch:
        raise ValueError("kv_lens must be [batch] and page_table [batch, max_pages] with batch = len(cu_seqlens_q) - 1")
    if sinks is not None and sinks.numel() != hq:
        raise ValueError(f"sinks must have {hq} entries")
    if out is not None:
        _check(out, "out", torch.bfloat16, dev)
        if out.shape != q.shape:
            raise ValueError("out must have the shape of q")
    if lse is not None:
        _check(lse, "lse", torch.float32, dev)
        if lse.shape != (total_q, hq):
            raise ValueError(f"lse must be [{total_q}, {hq}]")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((total_q, hq), dtype=torch.float32, device=dev)
    st = lib.attn_sink_prefill_paged(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(page_table), page_table.shape[1],
                                     num_pages, _ptr(cu_seqlens_q), _ptr(kv_lens), _ptr(sinks), batch, total_q,
                                     int(max_seqlen_q), int(max_kv_len), hq, hkv, d, page_size, float(softmax_scale),
                                     int(bool(causal)), int(window), _ptr(out), _ptr(lse), _stream(stream))
    _raise(st, "attn_sink_prefill_paged")
    return out, lse


_YARN_RAMPS = {"turns": 0, "index": 1}


def attn_sink_rope_append(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens_q: torch.Tensor,
                          kv_lens: torch.Tensor, page_table: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                          max_seqlen_q: int, max_kv_len: int, rope_theta: float, yarn_factor: float = 1.0,
                          yarn_original_len: int = 0, yarn_alpha: float = 1.0, yarn_beta: float = 32.0,
                          yarn_ramp: str = "turns", q_out: Optional[torch.Tensor] = None,
                          stream=None) -> torch.Tensor:
    """q [T, hq, 64], k/v [T, hkv, 64] bf16 (new tokens); caches [pages, hkv, page_size, 64] bf16, updated in
    place; cu_seqlens_q int32 [batch+1]; kv_lens int32 [batch] (new tokens included); yarn_ramp "turns" or
    "index" (ATTN_SINK_YARN_RAMP_TURNS / _INDEX). Returns the rotated q."""
    dev = q.device
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _check(t, n, torch.bfloat16, dev)
    for t, n in ((cu_seqlens_q, "cu_seqlens_q"), (kv_lens, "kv_lens"), (page_table, "page_table")):
        _check(t, n, torch.int32, dev)
    if q.dim() != 3 or k.dim() != 3 or v.shape != k.shape or k.shape[0] != q.shape[0] or k_cache.dim() != 4 or \
            v_cache.shape != k_cache.shape or k_cache.shape[1] != k.shape[1] or k_cache.shape[3] != q.shape[2]:
        raise ValueError(f"expected q [T, hq, d], k/v [T, hkv, d] and caches [pages, hkv, page_size, d]; got "
                         f"{tuple(q.shape)}, {tuple(k.shape)}, {tuple(v.shape)}, {tuple(k_cache.shape)}")
    total_q, hq, d = q.shape
    hkv = k.shape[1]
    batch = cu_seqlens_q.numel() - 1
    if kv_lens.numel() != batch or page_table.dim() != 2 or page_table.shape[0] != batch:
        raise ValueError("kv_lens must be [batch] and page_table [batch, max_pages] with batch = len(cu_seqlens_q) - 1")
    if q_out is None:
        q_out = torch.empty_like(q)
    else:
        _check(q_out, "q_out", torch.bfloat16, dev)
        if q_out.shape != q.shape:
            raise ValueError("q_out must have the shape of q")
    num_pages, page_size = k_cache.shape[0], k_cache.shape[2]
    st = lib.attn_sink_rope_append(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_q), _ptr(kv_lens), _ptr(page_table),
                                   page_table.shape[1], num_pages, _ptr(k_cache), _ptr(v_cache), batch, total_q,
                                   int(max_seqlen_q), int(max_kv_len), hq, hkv, d, page_size, float(rope_theta),
                                   float(yarn_factor), int(yarn_original_len), float(yarn_alpha), float(yarn_beta),
                                   _YARN_RAMPS[yarn_ramp], _ptr(q_out), _stream(stream))
    _raise(st, "attn_sink_rope_append")
    return q_out


def attn_sink_decode_workspace_size(batch: int, q_len: int, max_kv_len: int, num_q_heads: int, head_dim: int,
                                    kv_chunk: int) -> int:
    return int(lib.attn_sink_decode_workspace_size(batch, q_len, max_kv_len, num_q_heads, head_dim, kv_chunk))


class _DecodeLayout(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int64) for name in
                ("rows", "chunks", "partials", "off_indptr", "off_counts", "off_o", "off_lse", "total")]


def attn_sink_decode_workspace_layout(batch: int, q_len: int, max_kv_len: int, num_q_heads: int, head_dim: int,
                                      kv_chunk: int) -> dict:
    """Byte offsets of the plan and partial regions inside the decode workspace, from the library."""
    lay = _DecodeLayout()
    st = lib.attn_sink_decode_workspace_layout(batch, q_len, max_kv_len, num_q_heads, head_dim, kv_chunk,
                                               ctypes.byref(lay))
    _raise(st, "attn_sink_decode_workspace_layout")
    return {name: int(getattr(lay, name)) for name, _ in _DecodeLayout._fields_}


def decode_workspace_layout(batch: int, q_len: int, max_kv_len: int, num_q_heads: int, kv_chunk: int) -> dict:
    """attn_sink_decode_workspace_layout for head_dim 64."""
    return attn_sink_decode_workspace_layout(batch, q_len, max_kv_len, num_q_heads, 64, kv_chunk)


def _decode_args(q, k_cache, v_cache, page_table, kv_lens, sinks, q_len, workspace, kv_chunk, max_kv_len):
    dev = q.device
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _check(t, n, torch.bfloat16, dev)
    _check(page_table, "page_table", torch.int32, dev)
    _check(kv_lens, "kv_lens", torch.int32, dev)
    if sinks is not None:
        _check(sinks, "sinks", torch.float32, dev)
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape or k_cache.shape[3] != q.shape[2]:
        raise ValueError(f"expected q [rows, hq, d] and caches [pages, hkv, page_size, d]; got {tuple(q.shape)}, "
                         f"{tuple(k_cache.shape)}, {tuple(v_cache.shape)}")
    rows, hq, d = q.shape
    batch = kv_lens.numel()
    if rows != batch * q_len:
        raise ValueError(f"q has {rows} rows, expected batch*q_len = {batch * q_len}")
    if page_table.dim() != 2 or page_table.shape[0] != batch:
        raise ValueError(f"page_table must be [{batch}, max_pages_per_seq]")
    if sinks is not None and sinks.numel() != hq:
        raise ValueError(f"sinks must have {hq} entries")
    if workspace is not None:
        _check(workspace, "workspace", workspace.dtype, dev)
    need = attn_sink_decode_workspace_size(batch, q_len, max_kv_len, hq, d, kv_chunk)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    return batch, rows, hq, d, workspace


def attn_sink_decode_paged(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, page_table: torch.Tensor,
                           kv_lens: torch.Tensor, sinks: Optional[torch.Tensor], q_len: int, max_kv_len: int,
                           softmax_scale: Optional[float] = None, causal: bool = True, window: int = 0,
                           kv_chunk: int = 512, workspace: Optional[torch.Tensor] = None,
                           out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                           return_lse: bool = True, stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """q [batch*q_len, hq, 64]; caches [num_pages, hkv, page_size, 64] bf16; page_table int32 [batch, max_pages];
    kv_lens int32 [batch]; workspace uint8 (allocated if None)."""
    batch, rows, hq, d, workspace = _decode_args(q, k_cache, v_cache, page_table, kv_lens, sinks, q_len, workspace,
                                                 kv_chunk, max_kv_len)
    dev = q.device
    if out is not None:
        _check(out, "out", torch.bfloat16, dev)
        if out.shape != q.shape:
            raise ValueError("out must have the shape of q")
    if lse is not None:
        _check(lse, "lse", torch.float32, dev)
        if lse.shape != (rows, hq):
            raise ValueError(f"lse must be [{rows}, {hq}]")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((rows, hq), dtype=torch.float32, device=dev)
    num_pages, hkv, page_size = k_cache.shape[0], k_cache.shape[1], k_cache.shape[2]
    st = lib.attn_sink_decode_paged(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(page_table), page_table.shape[1],
                                    num_pages, _ptr(kv_lens), _ptr(sinks), batch, q_len, int(max_kv_len), hq, hkv, d,
                                    page_size, float(softmax_scale), int(bool(causal)), int(window), int(kv_chunk),
                                    _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(out),
                                    _ptr(lse), _stream(stream))
    _raise(st, "attn_sink_decode_paged")
    return out, lse


def attn_sink_decode_noalloc_capacity() -> int:
    return int(lib.attn_sink_decode_noalloc_capacity())


def attn_sink_decode_paged_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                                   page_table: torch.Tensor, kv_lens: torch.Tensor, sinks: Optional[torch.Tensor],
                                   q_len: int, max_kv_len: int, softmax_scale: Optional[float] = None,
                                   causal: bool = True, window: int = 0, kv_chunk: int = 512,
                                   out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                                   stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """attn_sink_decode_paged with the library's own scratch in place of a workspace. The caller passes out
    (and lse, or None): this function allocates nothing."""
    dev = q.device
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _check(t, n, torch.bfloat16, dev)
    _check(page_table, "page_table", torch.int32, dev)
    _check(kv_lens, "kv_lens", torch.int32, dev)
    if sinks is not None:
        _check(sinks, "sinks", torch.float32, dev)
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape or k_cache.shape[3] != q.shape[2]:
        raise ValueError(f"expected q [rows, hq, d] and caches [pages, hkv, page_size, d]; got {tuple(q.shape)}, "
                         f"{tuple(k_cache.shape)}, {tuple(v_cache.shape)}")
    rows, hq, d = q.shape
    batch = kv_lens.numel()
    if rows != batch * q_len:
        raise ValueError(f"q has {rows} rows, expected batch*q_len = {batch * q_len}")
    if page_table.dim() != 2 or page_table.shape[0] != batch:
        raise ValueError(f"page_table must be [{batch}, max_pages_per_seq]")
    if out is None:
        raise ValueError("out is required (this entry point allocates nothing)")
    _check(out, "out", torch.bfloat16, dev)
    if out.shape != q.shape:
        raise ValueError("out must have the shape of q")
    if lse is not None:
        _check(lse, "lse", torch.float32, dev)
        if lse.shape != (rows, hq):
            raise ValueError(f"lse must be [{rows}, {hq}]")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    num_pages, hkv, page_size = k_cache.shape[0], k_cache.shape[1], k_cache.shape[2]
    st = lib.attn_sink_decode_paged_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(page_table),
                                            page_table.shape[1], num_pages, _ptr(kv_lens), _ptr(sinks), batch, q_len,
                                            int(max_kv_len), hq, hkv, d, page_size, float(softmax_scale),
                                            int(bool(causal)), int(window), int(kv_chunk), _ptr(out), _ptr(lse),
                                            _stream(stream))
    _raise(st, "attn_sink_decode_paged_noalloc")
    return out, lse


def attn_sink_decode_paged_tree(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                                page_table: torch.Tensor, kv_lens: torch.Tensor, tree_mask: torch.Tensor,
                                sinks: Optional[torch.Tensor], q_len: int, max_kv_len: int,
                                softmax_scale: Optional[float] = None, window: int = 0, kv_chunk: int = 512,
                                workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                                lse: Optional[torch.Tensor] = None, return_lse: bool = True,
                                stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """As attn_sink_decode_paged, with tree_mask int32 [batch*q_len] bitmaps (bit i of row t: draft token i
    visible to draft token t) in place of the causal flag."""
    batch, rows, hq, d, workspace = _decode_args(q, k_cache, v_cache, page_table, kv_lens, sinks, q_len, workspace,
                                                 kv_chunk, max_kv_len)
    dev = q.device
    _check(tree_mask, "tree_mask", torch.int32, dev)
    if tree_mask.numel() != rows:
        raise ValueError(f"tree_mask must have batch * q_len = {rows} entries")
    if out is not None:
        _check(out, "out", torch.bfloat16, dev)
        if out.shape != q.shape:
            raise ValueError("out must have the shape of q")
    if lse is not None:
        _check(lse, "lse", torch.float32, dev)
        if lse.shape != (rows, hq):
            raise ValueError(f"lse must be [{rows}, {hq}]")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((rows, hq), dtype=torch.float32, device=dev)
    num_pages, hkv, page_size = k_cache.shape[0], k_cache.shape[1], k_cache.shape[2]
    st = lib.attn_sink_decode_paged_tree(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(page_table), page_table.shape[1],
                                         num_pages, _ptr(kv_lens), _ptr(tree_mask), _ptr(sinks), batch, q_len,
                                         int(max_kv_len), hq, hkv, d, page_size, float(softmax_scale), int(window),
                                         int(kv_chunk), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                         _ptr(out), _ptr(lse), _stream(stream))
    _raise(st, "attn_sink_decode_paged_tree")
    return out, lse


def attn_sink_decode_paged_partials(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                                    page_table: torch.Tensor, kv_lens: torch.Tensor, sinks: Optional[torch.Tensor],
                                    q_len: int, max_kv_len: int, softmax_scale: Optional[float] = None,
                                    causal: bool = True, window: int = 0, kv_chunk: int = 512,
                                    workspace: Optional[torch.Tensor] = None, stream=None) -> dict:
    """The split-KV pass alone. Returns views of the workspace: partial_indptr int32 [rows+1], chunk_counts
    int32 [rows], o_partial fp32 [P, hq, 64], lse_partial fp32 [P, hq] (P = rows x chunk bound), ready for
    attn_sink_merge_partials; plus the workspace itself."""
    batch, rows, hq, d, workspace = _decode_args(q, k_cache, v_cache, page_table, kv_lens, sinks, q_len, workspace,
                                                 kv_chunk, max_kv_len)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    num_pages, hkv, page_size = k_cache.shape[0], k_cache.shape[1], k_cache.shape[2]
    st = lib.attn_sink_decode_paged_partials(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(page_table),
                                             page_table.shape[1], num_pages, _ptr(kv_lens), _ptr(sinks), batch, q_len,
                                             int(max_kv_len), hq, hkv, d, page_size, float(softmax_scale),
                                             int(bool(causal)), int(window), int(kv_chunk), _ptr(workspace),
                                             workspace.numel() * workspace.element_size(), _stream(stream))
    _raise(st, "attn_sink_decode_paged_partials")
    return _partial_views(workspace, batch, q_len, int(max_kv_len), hq, d, kv_chunk)


def _partial_views(workspace, batch, q_len, max_kv_len, hq, d, kv_chunk) -> dict:
    lay = attn_sink_decode_workspace_layout(batch, q_len, max_kv_len, hq, d, kv_chunk)
    ws = workspace.view(torch.uint8).reshape(-1)
    rows, n_p = batch * q_len, lay["partials"]
    return dict(
        workspace=workspace,
        partial_indptr=ws[lay["off_indptr"]:lay["off_indptr"] + 4 * (rows + 1)].view(torch.int32),
        chunk_counts=ws[lay["off_counts"]:lay["off_counts"] + 4 * rows].view(torch.int32),
        o_partial=ws[lay["off_o"]:lay["off_o"] + 4 * n_p * hq * d].view(torch.float32).view(n_p, hq, d),
        lse_partial=ws[lay["off_lse"]:lay["off_lse"] + 4 * n_p * hq].view(torch.float32).view(n_p, hq),
    )


def attn_sink_decode_paged_tree_partials(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                                         page_table: torch.Tensor, kv_lens: torch.Tensor, tree_mask: torch.Tensor,
                                         sinks: Optional[torch.Tensor], q_len: int, max_kv_len: int,
                                         softmax_scale: Optional[float] = None, window: int = 0,
                                         kv_chunk: int = 512, workspace: Optional[torch.Tensor] = None,
                                         stream=None) -> dict:
    """The split-KV pass of attn_sink_decode_paged_tree alone; returns the same views as
    attn_sink_decode_paged_partials."""
    batch, rows, hq, d, workspace = _decode_args(q, k_cache, v_cache, page_table, kv_lens, sinks, q_len, workspace,
                                                 kv_chunk, max_kv_len)
    _check(tree_mask, "tree_mask", torch.int32, q.device)
    if tree_mask.numel() != rows:
        raise ValueError(f"tree_mask must have batch * q_len = {rows} entries")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    num_pages, hkv, page_size = k_cache.shape[0], k_cache.shape[1], k_cache.shape[2]
    st = lib.attn_sink_decode_paged_tree_partials(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(page_table),
                                                  page_table.shape[1], num_pages, _ptr(kv_lens), _ptr(tree_mask),
                                                  _ptr(sinks), batch, q_len, int(max_kv_len), hq, hkv, d, page_size,
                                                  float(softmax_scale), int(window), int(kv_chunk), _ptr(workspace),
                                                  workspace.numel() * workspace.element_size(), _stream(stream))
    _raise(st, "attn_sink_decode_paged_tree_partials")
    return _partial_views(workspace, batch, q_len, int(max_kv_len), hq, d, kv_chunk)


def attn_sink_decode_paged_range_partials(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                                          page_table: torch.Tensor, kv_lens: torch.Tensor, kv_start: torch.Tensor,
                                          kv_total: torch.Tensor, sinks: Optional[torch.Tensor], q_len: int,
                                          max_kv_len: int, softmax_scale: Optional[float] = None,
                                          causal: bool = True, window: int = 0, kv_chunk: int = 512,
                                          workspace: Optional[torch.Tensor] = None, stream=None) -> dict:
    """The split-KV pass over one key range per sequence (kv_lens[b] keys at absolute positions
    kv_start[b].. of a kv_total[b]-key sequence); returns the same views as
    attn_sink_decode_paged_partials."""
    batch, rows, hq, d, workspace = _decode_args(q, k_cache, v_cache, page_table, kv_lens, sinks, q_len, workspace,
                                                 kv_chunk, max_kv_len)
    for t, n in ((kv_start, "kv_start"), (kv_total, "kv_total")):
        _check(t, n, torch.int32, q.device)
        if t.numel() != batch:
            raise ValueError(f"{n} must have batch = {batch} entries")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    num_pages, hkv, page_size = k_cache.shape[0], k_cache.shape[1], k_cache.shape[2]
    st = lib.attn_sink_decode_paged_range_partials(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(page_table),
                                                   page_table.shape[1], num_pages, _ptr(kv_lens), _ptr(kv_start),
                                                   _ptr(kv_total), _ptr(sinks), batch, q_len, int(max_kv_len), hq,
                                                   hkv, d, page_size, float(softmax_scale), int(bool(causal)),
                                                   int(window), int(kv_chunk), _ptr(workspace),
                                                   workspace.numel() * workspace.element_size(), _stream(stream))
    _raise(st, "attn_sink_decode_paged_range_partials")
    return _partial_views(workspace, batch, q_len, int(max_kv_len), hq, d, kv_chunk)


def attn_sink_decode_plan_chunk(kv_lens, q_len: int, num_q_heads: int, num_kv_heads: int, page_size: int,
                                workgroups: int = 0) -> int:
    """kv_chunk for a decode call with these host-side lengths (any int sequence, numpy array or CPU
    tensor); workgroups <= 0 asks the current device for the split kernel's resident grid."""
    import numpy as np
    if isinstance(kv_lens, torch.Tensor):
        if kv_lens.is_cuda:
            raise ValueError("kv_lens must be host data for the planner")
        kv_lens = kv_lens.numpy()
    lens = np.ascontiguousarray(np.asarray(kv_lens, dtype=np.int32).reshape(-1))
    out = ctypes.c_int32(0)
    st = lib.attn_sink_decode_plan_chunk(lens.ctypes.data if lens.size else None, int(lens.size), int(q_len),
                                         int(num_q_heads), int(num_kv_heads), int(page_size), int(workgroups),
                                         ctypes.byref(out))
    _raise(st, "attn_sink_decode_plan_chunk")
    return int(out.value)


def attn_sink_merge_partials(o_partial: torch.Tensor, lse_partial: torch.Tensor, partial_indptr: torch.Tensor,
                             out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                             return_lse: bool = True, stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """o_partial fp32 [P, hq, 64], lse_partial fp32 [P, hq], partial_indptr int32 [rows+1]."""
    dev = o_partial.device
    _check(o_partial, "o_partial", torch.float32, dev)
    _check(lse_partial, "lse_partial", torch.float32, dev)
    _check(partial_indptr, "partial_indptr", torch.int32, dev)
    if o_partial.dim() != 3 or lse_partial.shape != o_partial.shape[:2]:
        raise ValueError("o_partial must be [P, hq, d] and lse_partial [P, hq]")
    n_p, hq, d = o_partial.shape
    rows = partial_indptr.numel() - 1
    if out is not None:
        _check(out, "out", torch.bfloat16, dev)
        if out.shape != (rows, hq, d):
            raise ValueError(f"out must be [{rows}, {hq}, {d}]")
    if lse is not None:
        _check(lse, "lse", torch.float32, dev)
        if lse.shape != (rows, hq):
            raise ValueError(f"lse must be [{rows}, {hq}]")
    if out is None:
        out = torch.empty((rows, hq, d), dtype=torch.bfloat16, device=dev)
    if lse is None and return_lse:
        lse = torch.empty((rows, hq), dtype=torch.float32, device=dev)
    st = lib.attn_sink_merge_partials(_ptr(o_partial), _ptr(lse_partial), n_p, _ptr(partial_indptr), rows, hq, d,
                                      _ptr(out), _ptr(lse), _stream(stream))
    _raise(st, "attn_sink_merge_partials")
    return out, lse
