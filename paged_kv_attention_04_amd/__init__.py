"""Python binding for libpa.so: paged-KV attention for mixed decode / chunked-prefill
batches on MI355X.

Argument marshalling only: every step of the path runs in the library's HIP kernels.
PyTorch supplies device memory and the current HIP stream.  The entry points keep the
C names (``pa_plan``, ``pa_append_kv``, ``pa_attention_batch``); see include/pa.h for
argument meaning, layouts, ownership and errors.  If the library has not been built
the binding raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "_build", "libpa.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "pa.h")

PA_MAX_PREFILL_ROWS = 128
PA_MAX_PREFIX_GROUPS = 16
PA_MAX_PREFIX_GROUP_REQS = 32
PA_NOALLOC_SCRATCH_BYTES = 32 * 1024 * 1024
HEAD_DIM = 128
BLOCK_SIZE = 16

STATUS = {0: "PA_OK", -1: "PA_ERR_NULL", -2: "PA_ERR_SHAPE", -3: "PA_ERR_RANGE", -4: "PA_ERR_WORKSPACE",
          -5: "PA_ERR_UNSUPPORTED", -6: "PA_ERR_HIP", -7: "PA_ERR_NO_BLOCKS"}


class PaError(RuntimeError):
    def __init__(self, fn: str, code: int, extra: str = ""):
        self.code = code
        text = lib().pa_status_string(code).decode() if _lib is not None else ""
        super().__init__(f"{fn} -> {STATUS.get(code, code)} ({text}){extra}")


class Geometry(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("num_blocks", ctypes.c_int32), ("scale", ctypes.c_float)]

    @classmethod
    def make(cls, num_q_heads: int, num_kv_heads: int, num_blocks: int, scale: Optional[float] = None,
             head_dim: int = HEAD_DIM, block_size: int = BLOCK_SIZE) -> "Geometry":
        return cls(num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                   head_dim ** -0.5 if scale is None else scale)


class Plan(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32), ("num_reqs", ctypes.c_int32),
                ("total_q", ctypes.c_int32), ("num_decode_rows", ctypes.c_int32),
                ("num_prefill_rows", ctypes.c_int32), ("split_blocks", ctypes.c_int32),
                ("max_splits", ctypes.c_int32), ("decode_items", ctypes.c_int32), ("prefill_tiles", ctypes.c_int32),
                ("prefill_splits", ctypes.c_int32),
                ("prefill_req", ctypes.c_int32 * PA_MAX_PREFILL_ROWS),
                ("prefill_tile_start", ctypes.c_int32 * (PA_MAX_PREFILL_ROWS + 1)),
                ("num_prefix_groups", ctypes.c_int32), ("prefix_splits", ctypes.c_int32),
                ("prefix_first_req", ctypes.c_int32 * PA_MAX_PREFIX_GROUPS),
                ("prefix_num_reqs", ctypes.c_int32 * PA_MAX_PREFIX_GROUPS),
                ("prefix_blocks", ctypes.c_int32 * PA_MAX_PREFIX_GROUPS),
                ("prefill_tile_tokens", ctypes.c_int32), ("prefix_tile_rows", ctypes.c_int32),
                ("one_launch", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_uint64)]


_lib = None


def lib():
    """Load libpa.so (built in-tree by build.build_library); raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                           "or python -m paged_kv_attention_04_amd.build")
    L = ctypes.CDLL(LIB_PATH)
    P, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    G, PL = ctypes.POINTER(Geometry), ctypes.POINTER(Plan)
    L.pa_plan.argtypes = [G, i32, P, P, i32, i32, i32, PL]
    L.pa_plan_shared_prefix.argtypes = [G, P, P, P, i32, i32, i32, i32, i32, PL]
    L.pa_plan_shared_prefix_q8.argtypes = [G, P, P, P, i32, i32, i32, i32, i32, PL]
    L.pa_append_kv.argtypes = [G, P, P, P, P, P, i32, P]
    L.pa_attention_batch.argtypes = [G, PL, P, P, P, P, i32, P, P, P, P, P, sz, P]
    L.pa_decode_step.argtypes = [G, PL, P, P, P, P, P, P, i32, P, P, P, P, P, sz, P]
    L.pa_attention_step.argtypes = [G, PL, P, P, P, P, P, P, i32, P, P, P, P, P, sz, P]
    L.pa_validate_batch.argtypes = [G, i32, P, P, P, i32, P]
    L.pa_validate_append.argtypes = [G, P, i32, P]
    L.pa_copy_blocks.argtypes = [G, P, P, P, P, i32, P]
    L.pa_append_kv_q8.argtypes = [G, P, P, P, P, i32, P]
    L.pa_attention_batch_q8.argtypes = [G, PL, P, P, P, i32, P, P, P, P, P, sz, P]
    L.pa_attention_batch_noalloc.argtypes = [G, PL, P, P, P, P, i32, P, P, P, P, P]
    L.pa_copy_blocks_q8.argtypes = [G, P, P, P, i32, P]
    L.pa_decode_step_q8.argtypes = [G, PL, P, P, P, P, P, i32, P, P, P, P, P, sz, P]
    L.pa_attention_step_q8.argtypes = [G, PL, P, P, P, P, P, i32, P, P, P, P, P, sz, P]
    f32 = ctypes.c_float
    L.pa_append_kv_fp8.argtypes = [G, P, P, P, P, P, i32, f32, f32, P]
    L.pa_attention_batch_fp8.argtypes = [G, PL, P, P, P, P, i32, P, P, P, P, P, sz, f32, f32, P]
    L.pa_copy_blocks_fp8.argtypes = [G, P, P, P, P, i32, P]
    L.pa_decode_step_fp8.argtypes = [G, PL, P, P, P, P, P, P, i32, P, P, P, P, P, sz, f32, f32, P]
    L.pa_attention_step_fp8.argtypes = [G, PL, P, P, P, P, P, P, i32, P, P, P, P, P, sz, f32, f32, P]
    L.pa_validate_copy.argtypes = [G, P, P, i32, P]
    L.pa_query_num_cus.argtypes = [i32, P]
    L.pa_allocator_create.argtypes = [i32, P]
    L.pa_allocator_destroy.argtypes = [P]
    L.pa_allocator_destroy.restype = None
    L.pa_allocator_alloc.argtypes = [P, i32, P]
    L.pa_allocator_retain.argtypes = [P, P, i32]
    L.pa_allocator_release.argtypes = [P, P, i32, P, i32]
    L.pa_allocator_cow.argtypes = [P, i32, P]
    L.pa_allocator_refcount.argtypes = [P, i32, P]
    L.pa_allocator_num_free.argtypes = [P, P, P]
    L.pa_allocator_sync.argtypes = [P]
    for fn in ("pa_plan", "pa_plan_shared_prefix", "pa_plan_shared_prefix_q8", "pa_append_kv", "pa_attention_batch", "pa_validate_batch",
               "pa_validate_append", "pa_copy_blocks", "pa_validate_copy", "pa_append_kv_q8",
               "pa_attention_batch_q8", "pa_copy_blocks_q8", "pa_append_kv_fp8", "pa_attention_batch_fp8",
               "pa_copy_blocks_fp8", "pa_decode_step_fp8", "pa_attention_step_fp8", "pa_decode_step_q8",
               "pa_attention_step_q8", "pa_attention_batch_noalloc", "pa_query_num_cus", "pa_decode_step", "pa_allocator_create",
               "pa_allocator_alloc", "pa_allocator_retain", "pa_allocator_release", "pa_allocator_cow",
               "pa_allocator_refcount", "pa_allocator_num_free", "pa_allocator_sync"):
        getattr(L, fn).restype = ctypes.c_int
    L.pa_status_string.argtypes = [ctypes.c_int]
    L.pa_status_string.restype = ctypes.c_char_p
    _lib = L
    return L


def header_functions() -> list:
    """Names of the functions include/pa.h declares."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(pa_\w+)\s*\(", text, re.M)))


def _check(fn: str, code: int):
    if code != 0:
        raise PaError(fn, code)


def _np_ptr(a):
    import numpy as np
    assert isinstance(a, np.ndarray) and a.flags.c_contiguous
    return a.ctypes.data_as(ctypes.c_void_p)


def _dev_ptr(t, dtype=None, name="tensor"):
    import torch
    if t is None:
        return None
    if not (isinstance(t, torch.Tensor) and t.is_cuda and t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous device tensor")
    if dtype is not None and t.dtype not in dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _stream_handle(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def num_cus(device: int = 0) -> int:
    v = ctypes.c_int32(0)
    _check("pa_query_num_cus", lib().pa_query_num_cus(device, ctypes.byref(v)))
    return int(v.value)


def pa_plan(geometry: Geometry, qo_len, kv_len, num_cus: int = 256, split_blocks: int = 0,
            prefill_splits: int = 0) -> Plan:
    """Host planner; qo_len / kv_len are host int32 sequences; 0 picks a split automatically."""
    import numpy as np
    qo = np.ascontiguousarray(qo_len, dtype=np.int32)
    kv = np.ascontiguousarray(kv_len, dtype=np.int32)
    if qo.shape != kv.shape:
        raise ValueError("qo_len and kv_len differ in length")
    plan = Plan()
    _check("pa_plan", lib().pa_plan(ctypes.byref(geometry), int(qo.size), _np_ptr(qo), _np_ptr(kv), int(num_cus),
                                    int(split_blocks), int(prefill_splits), ctypes.byref(plan)))
    return plan




def pa_plan_shared_prefix(geometry: Geometry, plan: Plan, qo_len, kv_len, block_tables, num_cus: int = 256,
                          min_shared_blocks: int = 0, prefix_splits: int = 0, split_blocks: int = 0,
                          q8: bool = False) -> Plan:
    """Add shared-prefix groups found in the host block tables to `plan` (in place; also
    returned).  block_tables: host int32 [num_reqs][max_blocks].  prefix_splits /
    split_blocks: 0 lets the planner choose; > 0 forces the value.  q8: the batch runs on a
    q8_0 pool (pa_plan_shared_prefix_q8)."""
    import numpy as np
    qo = np.ascontiguousarray(qo_len, dtype=np.int32)
    kv = np.ascontiguousarray(kv_len, dtype=np.int32)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    if bt.ndim != 2 or bt.shape[0] != qo.size or qo.shape != kv.shape:
        raise ValueError("block_tables must be [num_reqs][max_blocks] and match the lengths")
    name = "pa_plan_shared_prefix_q8" if q8 else "pa_plan_shared_prefix"
    _check(name, getattr(lib(), name)(ctypes.byref(geometry), _np_ptr(qo), _np_ptr(kv), _np_ptr(bt), int(bt.shape[1]),
                                      int(num_cus), int(min_shared_blocks), int(prefix_splits), int(split_blocks),
                                      ctypes.byref(plan)))
    return plan


def _bf16_types():
    import torch
    return (torch.bfloat16, torch.int16, torch.uint16)


def pa_append_kv(geometry: Geometry, k_pool, v_pool, k_new, v_new, slot_mapping, stream=None) -> None:
    import torch
    n = int(slot_mapping.numel())
    if n == 0:
        return
    bf = _bf16_types()
    _check("pa_append_kv", lib().pa_append_kv(
        ctypes.byref(geometry), _dev_ptr(k_pool, bf, "k_pool"), _dev_ptr(v_pool, bf, "v_pool"),
        _dev_ptr(k_new, bf, "k_new"), _dev_ptr(v_new, bf, "v_new"),
        _dev_ptr(slot_mapping, (torch.int32,), "slot_mapping"), n, _stream_handle(stream)))


def pa_decode_step(geometry: Geometry, plan: Plan, q, k_pool, v_pool, k_new, v_new, block_tables, qo_indptr, kv_len,
                   out, lse, workspace=None, stream=None) -> None:
    """A decode-only batch: append each row's new K/V (at position kv_len - 1) and attend,
    in one launch."""
    import torch
    bf, i32 = _bf16_types(), (torch.int32,)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("pa_decode_step", lib().pa_decode_step(
        ctypes.byref(geometry), ctypes.byref(plan), _dev_ptr(q, bf, "q"), _dev_ptr(k_pool, bf, "k_pool"),
        _dev_ptr(v_pool, bf, "v_pool"), _dev_ptr(k_new, bf, "k_new"), _dev_ptr(v_new, bf, "v_new"),
        _dev_ptr(block_tables, i32, "block_tables"), int(block_tables.shape[1]), _dev_ptr(qo_indptr, i32, "qo_indptr"),
        _dev_ptr(kv_len, i32, "kv_len"), _dev_ptr(out, bf, "out"), _dev_ptr(lse, (torch.float32,), "lse"),
        _dev_ptr(workspace, name="workspace"), ws_bytes, _stream_handle(stream)))


def pa_attention_step(geometry: Geometry, plan: Plan, q, k_pool, v_pool, k_new, v_new, block_tables, qo_indptr,
                      kv_len, out, lse, workspace=None, stream=None) -> None:
    """Any batch (decode and chunked-prefill rows): append each row's new K/V (positions
    kv_len - qo_len .. kv_len - 1) and attend, in the attention launches alone."""
    import torch
    bf, i32 = _bf16_types(), (torch.int32,)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("pa_attention_step", lib().pa_attention_step(
        ctypes.byref(geometry), ctypes.byref(plan), _dev_ptr(q, bf, "q"), _dev_ptr(k_pool, bf, "k_pool"),
        _dev_ptr(v_pool, bf, "v_pool"), _dev_ptr(k_new, bf, "k_new"), _dev_ptr(v_new, bf, "v_new"),
        _dev_ptr(block_tables, i32, "block_tables"), int(block_tables.shape[1]), _dev_ptr(qo_indptr, i32, "qo_indptr"),
        _dev_ptr(kv_len, i32, "kv_len"), _dev_ptr(out, bf, "out"), _dev_ptr(lse, (torch.float32,), "lse"),
        _dev_ptr(workspace, name="workspace"), ws_bytes, _stream_handle(stream)))


PA_Q8_TILE_BYTES = 16 * 128 + 16 * (128 // 32) * 2


def q8_pool_shape(num_blocks: int, num_kv_heads: int):
    """Shape of a q8_0 pool (uint8): each (block, KV head) holds its K tile, then its V tile."""
    return (num_blocks, num_kv_heads, 2, PA_Q8_TILE_BYTES)


def pa_append_kv_q8(geometry: Geometry, kv_pool_q8, k_new, v_new, slot_mapping, stream=None) -> None:
    """Quantise new bf16 K/V rows into a q8_0 pool."""
    import torch
    n = int(slot_mapping.numel())
    if n == 0:
        return
    bf, u8 = _bf16_types(), (torch.uint8,)
    _check("pa_append_kv_q8", lib().pa_append_kv_q8(
        ctypes.byref(geometry), _dev_ptr(kv_pool_q8, u8, "kv_pool_q8"), _dev_ptr(k_new, bf, "k_new"),
        _dev_ptr(v_new, bf, "v_new"), _dev_ptr(slot_mapping, (torch.int32,), "slot_mapping"), n,
        _stream_handle(stream)))


def pa_attention_batch_q8(geometry: Geometry, plan: Plan, q, kv_pool_q8, block_tables, qo_indptr, kv_len, out, lse,
                          workspace=None, stream=None) -> None:
    """Decode attention over a q8_0 pool; the rest as pa_attention_batch."""
    import torch
    bf, i32, u8 = _bf16_types(), (torch.int32,), (torch.uint8,)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("pa_attention_batch_q8", lib().pa_attention_batch_q8(
        ctypes.byref(geometry), ctypes.byref(plan), _dev_ptr(q, bf, "q"), _dev_ptr(kv_pool_q8, u8, "kv_pool_q8"),
        _dev_ptr(block_tables, i32, "block_tables"), int(block_tables.shape[1]),
        _dev_ptr(qo_indptr, i32, "qo_indptr"), _dev_ptr(kv_len, i32, "kv_len"), _dev_ptr(out, bf, "out"),
        _dev_ptr(lse, (torch.float32,), "lse"), _dev_ptr(workspace, name="workspace"), ws_bytes,
        _stream_handle(stream)))


def _step_q8(name, geometry, plan, q, kv_pool_q8, k_new, v_new, block_tables, qo_indptr, kv_len, out, lse,
             workspace, stream):
    import torch
    bf, i32, u8 = _bf16_types(), (torch.int32,), (torch.uint8,)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(name, getattr(lib(), name)(
        ctypes.byref(geometry), ctypes.byref(plan), _dev_ptr(q, bf, "q"), _dev_ptr(kv_pool_q8, u8, "kv_pool_q8"),
        _dev_ptr(k_new, bf, "k_new"), _dev_ptr(v_new, bf, "v_new"), _dev_ptr(block_tables, i32, "block_tables"),
        int(block_tables.shape[1]), _dev_ptr(qo_indptr, i32, "qo_indptr"), _dev_ptr(kv_len, i32, "kv_len"),
        _dev_ptr(out, bf, "out"), _dev_ptr(lse, (torch.float32,), "lse"), _dev_ptr(workspace, name="workspace"),
        ws_bytes, _stream_handle(stream)))


def pa_decode_step_q8(geometry: Geometry, plan: Plan, q, kv_pool_q8, k_new, v_new, block_tables, qo_indptr, kv_len,
                      out, lse, workspace=None, stream=None) -> None:
    """pa_decode_step over a q8_0 pool: the new rows quantised and appended inside the launch."""
    _step_q8("pa_decode_step_q8", geometry, plan, q, kv_pool_q8, k_new, v_new, block_tables, qo_indptr, kv_len, out,
             lse, workspace, stream)


def pa_attention_step_q8(geometry: Geometry, plan: Plan, q, kv_pool_q8, k_new, v_new, block_tables, qo_indptr,
                         kv_len, out, lse, workspace=None, stream=None) -> None:
    """pa_attention_step over a q8_0 pool: the new rows quantised and appended inside the launches."""
    _step_q8("pa_attention_step_q8", geometry, plan, q, kv_pool_q8, k_new, v_new, block_tables, qo_indptr, kv_len,
             out, lse, workspace, stream)


def pa_copy_blocks_q8(geometry: Geometry, kv_pool_q8, src_blocks, dst_blocks, stream=None) -> None:
    import torch
    n = int(src_blocks.numel())
    if int(dst_blocks.numel()) != n:
        raise ValueError("src_blocks and dst_blocks differ in length")
    if n == 0:
        return
    u8, i32 = (torch.uint8,), (torch.int32,)
    _check("pa_copy_blocks_q8", lib().pa_copy_blocks_q8(
        ctypes.byref(geometry), _dev_ptr(kv_pool_q8, u8, "kv_pool_q8"), _dev_ptr(src_blocks, i32, "src_blocks"),
        _dev_ptr(dst_blocks, i32, "dst_blocks"), n, _stream_handle(stream)))


def pa_append_kv_fp8(geometry: Geometry, k_pool_fp8, v_pool_fp8, k_new, v_new, slot_mapping, k_scale: float = 1.0,
                     v_scale: float = 1.0, stream=None) -> None:
    """Store new bf16 K/V rows as E4M3 codes of x / scale in FP8 pools (uint8, the bf16 layout)."""
    import torch
    n = int(slot_mapping.numel())
    if n == 0:
        return
    bf, u8 = _bf16_types(), (torch.uint8,)
    _check("pa_append_kv_fp8", lib().pa_append_kv_fp8(
        ctypes.byref(geometry), _dev_ptr(k_pool_fp8, u8, "k_pool_fp8"), _dev_ptr(v_pool_fp8, u8, "v_pool_fp8"),
        _dev_ptr(k_new, bf, "k_new"), _dev_ptr(v_new, bf, "v_new"),
        _dev_ptr(slot_mapping, (torch.int32,), "slot_mapping"), n, float(k_scale), float(v_scale),
        _stream_handle(stream)))


def pa_attention_batch_fp8(geometry: Geometry, plan: Plan, q, k_pool_fp8, v_pool_fp8, block_tables, qo_indptr, kv_len,
                           out, lse, workspace=None, k_scale: float = 1.0, v_scale: float = 1.0, stream=None) -> None:
    """Attention over FP8 pools with per-pool scales; the rest as pa_attention_batch."""
    import torch
    bf, i32, u8 = _bf16_types(), (torch.int32,), (torch.uint8,)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("pa_attention_batch_fp8", lib().pa_attention_batch_fp8(
        ctypes.byref(geometry), ctypes.byref(plan), _dev_ptr(q, bf, "q"), _dev_ptr(k_pool_fp8, u8, "k_pool_fp8"),
        _dev_ptr(v_pool_fp8, u8, "v_pool_fp8"), _dev_ptr(block_tables, i32, "block_tables"),
        int(block_tables.shape[1]), _dev_ptr(qo_indptr, i32, "qo_indptr"), _dev_ptr(kv_len, i32, "kv_len"),
        _dev_ptr(out, bf, "out"), _dev_ptr(lse, (torch.float32,), "lse"), _dev_ptr(workspace, name="workspace"),
        ws_bytes, float(k_scale), float(v_scale), _stream_handle(stream)))


def _step_fp8(name, geometry, plan, q, k_pool_fp8, v_pool_fp8, k_new, v_new, block_tables, qo_indptr, kv_len, out,
              lse, workspace, k_scale, v_scale, stream):
    import torch
    bf, i32, u8 = _bf16_types(), (torch.int32,), (torch.uint8,)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(name, getattr(lib(), name)(
        ctypes.byref(geometry), ctypes.byref(plan), _dev_ptr(q, bf, "q"), _dev_ptr(k_pool_fp8, u8, "k_pool_fp8"),
        _dev_ptr(v_pool_fp8, u8, "v_pool_fp8"), _dev_ptr(k_new, bf, "k_new"), _dev_ptr(v_new, bf, "v_new"),
        _dev_ptr(block_tables, i32, "block_tables"), int(block_tables.shape[1]), _dev_ptr(qo_indptr, i32, "qo_indptr"),
        _dev_ptr(kv_len, i32, "kv_len"), _dev_ptr(out, bf, "out"), _dev_ptr(lse, (torch.float32,), "lse"),
        _dev_ptr(workspace, name="workspace"), ws_bytes, float(k_scale), float(v_scale), _stream_handle(stream)))


def pa_decode_step_fp8(geometry: Geometry, plan: Plan, q, k_pool_fp8, v_pool_fp8, k_new, v_new, block_tables,
                       qo_indptr, kv_len, out, lse, workspace=None, k_scale: float = 1.0, v_scale: float = 1.0,
                       stream=None) -> None:
    """pa_decode_step over FP8 pools: the new rows encoded and appended inside the launch."""
    _step_fp8("pa_decode_step_fp8", geometry, plan, q, k_pool_fp8, v_pool_fp8, k_new, v_new, block_tables, qo_indptr,
              kv_len, out, lse, workspace, k_scale, v_scale, stream)


def pa_attention_step_fp8(geometry: Geometry, plan: Plan, q, k_pool_fp8, v_pool_fp8, k_new, v_new, block_tables,
                          qo_indptr, kv_len, out, lse, workspace=None, k_scale: float = 1.0, v_scale: float = 1.0,
                          stream=None) -> None:
    """pa_attention_step over FP8 pools: the new rows encoded and appended inside the launches."""
    _step_fp8("pa_attention_step_fp8", geometry, plan, q, k_pool_fp8, v_pool_fp8, k_new, v_new, block_tables,
              qo_indptr, kv_len, out, lse, workspace, k_scale, v_scale, stream)


def pa_copy_blocks_fp8(geometry: Geometry, k_pool_fp8, v_pool_fp8, src_blocks, dst_blocks, stream=None) -> None:
    import torch
    n = int(src_blocks.numel())
    if int(dst_blocks.numel()) != n:
        raise ValueError("src_blocks and dst_blocks differ in length")
    if n == 0:
        return
    u8, i32 = (torch.uint8,), (torch.int32,)
    _check("pa_copy_blocks_fp8", lib().pa_copy_blocks_fp8(
        ctypes.byref(geometry), _dev_ptr(k_pool_fp8, u8, "k_pool_fp8"), _dev_ptr(v_pool_fp8, u8, "v_pool_fp8"),
        _dev_ptr(src_blocks, i32, "src_blocks"), _dev_ptr(dst_blocks, i32, "dst_blocks"), n,
        _stream_handle(stream)))


def pa_attention_batch(geometry: Geometry, plan: Plan, q, k_pool, v_pool, block_tables, qo_indptr, kv_len, out, lse,
                       workspace=None, stream=None) -> None:
    import torch
    bf = _bf16_types()
    i32 = (torch.int32,)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("pa_attention_batch", lib().pa_attention_batch(
        ctypes.byref(geometry), ctypes.byref(plan), _dev_ptr(q, bf, "q"), _dev_ptr(k_pool, bf, "k_pool"),
        _dev_ptr(v_pool, bf, "v_pool"), _dev_ptr(block_tables, i32, "block_tables"), int(block_tables.shape[1]),
        _dev_ptr(qo_indptr, i32, "qo_indptr"), _dev_ptr(kv_len, i32, "kv_len"), _dev_ptr(out, bf, "out"),
        _dev_ptr(lse, (torch.float32,), "lse"), _dev_ptr(workspace, None, "workspace"), ws_bytes,
        _stream_handle(stream)))


def pa_attention_batch_noalloc(geometry: Geometry, plan: Plan, q, k_pool, v_pool, block_tables, qo_indptr, kv_len, out,
                               lse, stream=None) -> None:
    """pa_attention_batch without a workspace: split partials and counters live in the
    library's fixed per-device scratch array (PA_NOALLOC_SCRATCH_BYTES); nothing is allocated."""
    import torch
    bf, i32 = _bf16_types(), (torch.int32,)
    _check("pa_attention_batch_noalloc", lib().pa_attention_batch_noalloc(
        ctypes.byref(geometry), ctypes.byref(plan), _dev_ptr(q, bf, "q"), _dev_ptr(k_pool, bf, "k_pool"),
        _dev_ptr(v_pool, bf, "v_pool"), _dev_ptr(block_tables, i32, "block_tables"), int(block_tables.shape[1]),
        _dev_ptr(qo_indptr, i32, "qo_indptr"), _dev_ptr(kv_len, i32, "kv_len"), _dev_ptr(out, bf, "out"),
        _dev_ptr(lse, (torch.float32,), "lse"), _stream_handle(stream)))


def pa_validate_batch(geometry: Geometry, qo_len, kv_len, block_tables):
    """Host check; returns (status_code, bad_request_index)."""
    import numpy as np
    qo = np.ascontiguousarray(qo_len, dtype=np.int32)
    kv = np.ascontiguousarray(kv_len, dtype=np.int32)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    bad = ctypes.c_int32(-1)
    rc = lib().pa_validate_batch(ctypes.byref(geometry), int(qo.size), _np_ptr(qo), _np_ptr(kv), _np_ptr(bt),
                                 int(bt.shape[1]) if bt.ndim == 2 else 0, ctypes.byref(bad))
    return rc, int(bad.value)


def pa_validate_append(geometry: Geometry, slot_mapping):
    """Host check; returns (status_code, bad_token_index)."""
    import numpy as np
    sm = np.ascontiguousarray(slot_mapping, dtype=np.int32)
    bad = ctypes.c_int32(-1)
    rc = lib().pa_validate_append(ctypes.byref(geometry), _np_ptr(sm), int(sm.size), ctypes.byref(bad))
    return rc, int(bad.value)


def pa_copy_blocks(geometry: Geometry, k_pool, v_pool, src_blocks, dst_blocks, stream=None) -> None:
    """Device copy of whole blocks (all KV heads, K and V): block src[i] -> block dst[i]."""
    import torch
    n = int(src_blocks.numel())
    if int(dst_blocks.numel()) != n:
        raise ValueError("src_blocks and dst_blocks differ in length")
    if n == 0:
        return
    bf, i32 = _bf16_types(), (torch.int32,)
    _check("pa_copy_blocks", lib().pa_copy_blocks(
        ctypes.byref(geometry), _dev_ptr(k_pool, bf, "k_pool"), _dev_ptr(v_pool, bf, "v_pool"),
        _dev_ptr(src_blocks, i32, "src_blocks"), _dev_ptr(dst_blocks, i32, "dst_blocks"), n,
        _stream_handle(stream)))


def pa_validate_copy(geometry: Geometry, src_blocks, dst_blocks):
    """(status, bad pair index) for a host block-copy list."""
    import numpy as np
    s = np.ascontiguousarray(src_blocks, dtype=np.int32)
    d = np.ascontiguousarray(dst_blocks, dtype=np.int32)
    if s.shape != d.shape:
        raise ValueError("src_blocks and dst_blocks differ in length")
    bad = ctypes.c_int32(-1)
    rc = lib().pa_validate_copy(ctypes.byref(geometry), _np_ptr(s), _np_ptr(d), int(s.size), ctypes.byref(bad))
    return rc, int(bad.value)


class BlockAllocator:
    """Reference-counted block ids of one pool, with stream-deferred release (the C
    allocator: host bookkeeping, no device memory)."""

    def __init__(self, num_blocks: int):
        h = ctypes.c_void_p()
        _check("pa_allocator_create", lib().pa_allocator_create(int(num_blocks), ctypes.byref(h)))
        self._h = h

    def close(self):
        if self._h:
            lib().pa_allocator_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @staticmethod
    def _ids(blocks):
        import numpy as np
        return np.ascontiguousarray(np.atleast_1d(np.asarray(blocks, dtype=np.int32)))

    def alloc(self, n: int):
        import numpy as np
        out = np.empty(int(n), np.int32)
        _check("pa_allocator_alloc", lib().pa_allocator_alloc(self._h, int(n), _np_ptr(out)))
        return out

    def retain(self, blocks):
        b = self._ids(blocks)
        _check("pa_allocator_retain", lib().pa_allocator_retain(self._h, _np_ptr(b), int(b.size)))

    def release(self, blocks, stream=None, deferred: bool = True):
        """Drop one reference per entry; freed blocks wait for the work queued on `stream`
        (the current stream when None) unless deferred is False."""
        b = self._ids(blocks)
        s = _stream_handle(stream) if deferred else None
        _check("pa_allocator_release", lib().pa_allocator_release(self._h, _np_ptr(b), int(b.size), s,
                                                                  1 if deferred else 0))

    def cow(self, block: int) -> int:
        out = ctypes.c_int32(-1)
        _check("pa_allocator_cow", lib().pa_allocator_cow(self._h, int(block), ctypes.byref(out)))
        return int(out.value)

    def refcount(self, block: int) -> int:
        out = ctypes.c_int32(0)
        _check("pa_allocator_refcount", lib().pa_allocator_refcount(self._h, int(block), ctypes.byref(out)))
        return int(out.value)

    def num_free(self):
        """(free blocks, blocks still waiting for their stream work)."""
        f, w = ctypes.c_int32(0), ctypes.c_int32(0)
        _check("pa_allocator_num_free", lib().pa_allocator_num_free(self._h, ctypes.byref(f), ctypes.byref(w)))
        return int(f.value), int(w.value)

    def sync(self):
        _check("pa_allocator_sync", lib().pa_allocator_sync(self._h))


def workspace_for(plan: Plan, device="cuda"):
    """A zeroed workspace of the size the plan asks for (None if it needs none).  Its
    completion counters must start at zero; the library leaves them zero after each call."""
    import torch
    if plan.workspace_bytes == 0:
        return None
    return torch.zeros(int(plan.workspace_bytes), dtype=torch.uint8, device=device)


def to_device(arr, device="cuda"):
    """numpy array -> device tensor (bf16 bit patterns stay uint16-shaped as int16)."""
    import numpy as np
    import torch
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


def run_workload(wl, split_blocks: int = 0, num_cus: int = 256, device="cuda", validate: bool = True,
                 prefill_splits: int = 0, cascade: bool = False, min_shared_blocks: int = 0, prefix_splits: int = 0,
                 one_launch: Optional[int] = None):
    """Upload a workload (see synthetic.Workload for the fields), append its new tokens,
    plan and run attention; returns host numpy (k_pool, v_pool, out, lse), or
    (kv_pool, None, out, lse) for a q8_0 workload.  one_launch overrides the plan's choice
    of one or two launches for a batch with chunk tiles and decode rows."""
    import numpy as np
    import torch
    g = Geometry.make(wl.num_q_heads, wl.num_kv_heads, wl.num_blocks, wl.scale, wl.head_dim, wl.block_size)
    if validate:
        rc, bad = pa_validate_batch(g, wl.qo_len, wl.kv_len, wl.block_tables)
        if rc:
            raise PaError("pa_validate_batch", rc, f" at request {bad}")
        rc, bad = pa_validate_append(g, wl.slot_mapping)
        if rc:
            raise PaError("pa_validate_append", rc, f" at token {bad}")
    q8 = getattr(wl, "kv_format", "bf16") == "q8_0"
    fp8 = getattr(wl, "kv_format", "bf16") == "fp8"
    plan = pa_plan(g, wl.qo_len, wl.kv_len, num_cus, split_blocks, prefill_splits)
    if cascade:
        pa_plan_shared_prefix(g, plan, wl.qo_len, wl.kv_len, wl.block_tables, num_cus, min_shared_blocks,
                              prefix_splits=prefix_splits, q8=q8)
    if one_launch is not None:
        plan.one_launch = int(one_launch)
    if q8:
        kp, vp = to_device(wl.kv_pool, device), None
    else:
        kp, vp = to_device(wl.k_pool, device), to_device(wl.v_pool, device)
    q = to_device(wl.q, device)
    bt = to_device(wl.block_tables, device)
    qo_indptr = to_device(wl.qo_indptr, device)
    kv = to_device(wl.kv_len, device)
    sm = to_device(wl.slot_mapping, device)
    kn, vn = to_device(wl.k_new, device), to_device(wl.v_new, device)
    out = torch.empty((wl.total_q, wl.num_q_heads, wl.head_dim), dtype=torch.int16, device=device)
    lse = torch.empty((wl.total_q, wl.num_q_heads), dtype=torch.float32, device=device)
    ws = workspace_for(plan, device)
    if q8:
        pa_append_kv_q8(g, kp, kn, vn, sm)
        pa_attention_batch_q8(g, plan, q, kp, bt, qo_indptr, kv, out, lse, ws)
    elif fp8:
        pa_append_kv_fp8(g, kp, vp, kn, vn, sm, wl.k_scale, wl.v_scale)
        pa_attention_batch_fp8(g, plan, q, kp, vp, bt, qo_indptr, kv, out, lse, ws, wl.k_scale, wl.v_scale)
    else:
        pa_append_kv(g, kp, vp, kn, vn, sm)
        pa_attention_batch(g, plan, q, kp, vp, bt, qo_indptr, kv, out, lse, ws)
    torch.cuda.synchronize()
    if q8:
        pools = (kp.cpu().numpy(), None)
    elif fp8:
        pools = (kp.cpu().numpy(), vp.cpu().numpy())
    else:
        pools = (kp.cpu().numpy().view(np.uint16), vp.cpu().numpy().view(np.uint16))
    return pools + (out.cpu().numpy().view(np.uint16), lse.cpu().numpy())
