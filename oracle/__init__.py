"""CPU oracle for paged-KV attention (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  The product library under
``paged_kv_attention_04_amd`` never imports it, and it imports nothing from
there: the two share no code.  The arithmetic lives in ``pa_oracle.c``
(plain double-precision loops, see its header for the definition and the
passages of the pages it follows); this file only compiles it with gcc and
marshals numpy arrays through ctypes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pa_oracle.c")
_BUILD = os.path.join(_HERE, "_build")
_LIB = os.path.join(_BUILD, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP) into oracle/_build/liboracle.so."""
    os.makedirs(_BUILD, exist_ok=True)
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build(force=True)
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    lib.oracle_append.argtypes = [P, P, P, P, P, i32, i32, i32, i32, i32]
    lib.oracle_copy_blocks.argtypes = [P, P, P, P, i32, i32, i32, i32, i32]
    lib.oracle_append.restype = ctypes.c_int
    lib.oracle_attention.argtypes = [P, P, P, P, i32, P, P, i32, i32, i32, i32, i32, i32, f64,
                                     P, P, P, P, P, P]
    lib.oracle_attention.restype = ctypes.c_int
    lib.oracle_double_to_bf16.argtypes = [f64]
    lib.oracle_double_to_bf16.restype = ctypes.c_uint16
    lib.oracle_round_bf16_array.argtypes = [P, P, i64]
    lib.oracle_round_bf16_array.restype = None
    lib.oracle_slot.argtypes = [P, i64, i32]
    lib.oracle_slot.restype = i64
    lib.oracle_attention_q8.argtypes = lib.oracle_attention.argtypes[:1] + lib.oracle_attention.argtypes[2:]
    lib.oracle_attention_q8.restype = ctypes.c_int
    lib.oracle_append_q8.argtypes = [P, P, P, P, i32, i32, i32, i32, i32]
    lib.oracle_append_q8.restype = ctypes.c_int
    lib.oracle_quantize_q8_rows.argtypes = [P, i64, i32, P, P]
    lib.oracle_quantize_q8_rows.restype = ctypes.c_int
    lib.oracle_q8_tile_bytes.argtypes = [i32, i32]
    lib.oracle_q8_tile_bytes.restype = i64
    lib.oracle_float_to_half.argtypes = [ctypes.c_float]
    lib.oracle_float_to_half.restype = ctypes.c_uint16
    lib.oracle_half_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_half_to_double.restype = f64
    lib.oracle_append_fp8.argtypes = [P, P, P, P, P, i32, i32, i32, i32, i32, ctypes.c_float, ctypes.c_float]
    lib.oracle_append_fp8.restype = ctypes.c_int
    lib.oracle_copy_blocks_fp8.argtypes = [P, P, P, P, i32, i32, i32, i32, i32]
    lib.oracle_copy_blocks_fp8.restype = ctypes.c_int
    lib.oracle_attention_fp8.argtypes = [P, P, P, P, i32, P, P, i32, i32, i32, i32, i32, i32, f64, f64, f64,
                                         P, P, P, P, P, P]
    lib.oracle_attention_fp8.restype = ctypes.c_int
    lib.oracle_encode_e4m3_array.argtypes = [P, P, i64]
    lib.oracle_encode_e4m3_array.restype = None
    lib.oracle_decode_e4m3_array.argtypes = [P, P, i64]
    lib.oracle_decode_e4m3_array.restype = None
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
    lib.oracle_set_num_threads.restype = None
    _lib = lib
    return lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads later attention calls may use (timing only; results do not depend on it)."""
    _load().oracle_set_num_threads(int(n))


def round_bf16(x) -> np.ndarray:
    """Double -> bf16 bit patterns, round to nearest even (one rounding step)."""
    x = _c(np.atleast_1d(x), np.float64)
    out = np.empty(x.shape, np.uint16)
    _load().oracle_round_bf16_array(_ptr(x), _ptr(out), x.size)
    return out


def slot(block_table_row, pos: int, block_size: int) -> int:
    bt = _c(block_table_row, np.int32)
    return int(_load().oracle_slot(_ptr(bt), int(pos), int(block_size)))


def append(k_pool, v_pool, k_new, v_new, slot_mapping, num_kv_heads, head_dim, block_size, num_blocks,
           in_place: bool = False):
    """Scatter new K/V rows into (copies of) the pools; returns (k_pool, v_pool)."""
    kp = k_pool if in_place else np.array(k_pool, dtype=np.uint16, copy=True)
    vp = v_pool if in_place else np.array(v_pool, dtype=np.uint16, copy=True)
    assert kp.flags.c_contiguous and vp.flags.c_contiguous
    kn, vn = _c(k_new, np.uint16), _c(v_new, np.uint16)
    sm = _c(slot_mapping, np.int32)
    rc = _load().oracle_append(_ptr(kp), _ptr(vp), _ptr(kn), _ptr(vn), _ptr(sm), int(sm.size),
                               int(num_kv_heads), int(head_dim), int(block_size), int(num_blocks))
    if rc != 0:
        raise ValueError(f"oracle_append failed with code {rc}")
    return kp, vp


def copy_blocks(k_pool, v_pool, src, dst, num_kv_heads, head_dim, block_size, num_blocks):
    """Copies of the pools with block src[i] copied to block dst[i]; returns (k_pool, v_pool)."""
    kp = np.array(k_pool, dtype=np.uint16, copy=True)
    vp = np.array(v_pool, dtype=np.uint16, copy=True)
    s, d = _c(src, np.int32), _c(dst, np.int32)
    if s.shape != d.shape:
        raise ValueError("src and dst differ in length")
    rc = _load().oracle_copy_blocks(_ptr(kp), _ptr(vp), _ptr(s), _ptr(d), int(s.size), int(num_kv_heads),
                                    int(head_dim), int(block_size), int(num_blocks))
    if rc != 0:
        raise ValueError(f"oracle_copy_blocks failed with code {rc}")
    return kp, vp


def float_to_half(x: float) -> int:
    """binary32 value -> binary16 bits, to nearest with ties to even."""
    return int(_load().oracle_float_to_half(float(np.float32(x))))


def half_to_double(h: int) -> float:
    return float(_load().oracle_half_to_double(int(h)))


def q8_tile_bytes(head_dim: int, block_size: int) -> int:
    """Bytes of one q8_0 (block, KV head) tile: [B][D] int8 codes, then [B][D/32] binary16 scales."""
    return int(_load().oracle_q8_tile_bytes(int(head_dim), int(block_size)))


def quantize_q8_rows(x, head_dim: int):
    """bf16 rows [..., D] -> (int8 codes [..., D], binary16 scale bits [..., D/32])."""
    xa = _c(x, np.uint16)
    n = xa.size // head_dim
    codes = np.empty(xa.shape, np.int8)
    scales = np.empty(xa.shape[:-1] + (head_dim // 32,), np.uint16)
    rc = _load().oracle_quantize_q8_rows(_ptr(xa), n, int(head_dim), _ptr(codes), _ptr(scales))
    if rc != 0:
        raise ValueError(f"oracle_quantize_q8_rows failed with code {rc}")
    return codes, scales


def append_q8(kv_pool, k_new, v_new, slot_mapping, num_kv_heads, head_dim, block_size, num_blocks):
    """Quantise new bf16 K/V rows into a copy of a q8_0 pool [num_blocks][Hkv][2][tile bytes]
    (each (block, KV head) holds its K tile, then its V tile)."""
    p = np.array(kv_pool, dtype=np.uint8, copy=True)
    kn, vn = _c(k_new, np.uint16), _c(v_new, np.uint16)
    sm = _c(slot_mapping, np.int32)
    rc = _load().oracle_append_q8(_ptr(p), _ptr(kn), _ptr(vn), _ptr(sm), int(sm.size), int(num_kv_heads),
                                  int(head_dim), int(block_size), int(num_blocks))
    if rc != 0:
        raise ValueError(f"oracle_append_q8 failed with code {rc}")
    return p


def encode_e4m3(x) -> np.ndarray:
    """Doubles -> OCP FP8 E4M3 codes, to nearest with ties to even, saturating at 448."""
    xa = _c(np.atleast_1d(x), np.float64)
    out = np.empty(xa.shape, np.uint8)
    _load().oracle_encode_e4m3_array(_ptr(xa), _ptr(out), xa.size)
    return out


def decode_e4m3(c) -> np.ndarray:
    """OCP FP8 E4M3 codes -> doubles (NaN for S.1111.111)."""
    ca = _c(np.atleast_1d(c), np.uint8)
    out = np.empty(ca.shape, np.float64)
    _load().oracle_decode_e4m3_array(_ptr(ca), _ptr(out), ca.size)
    return out


def append_fp8(k_pool, v_pool, k_new, v_new, slot_mapping, num_kv_heads, head_dim, block_size, num_blocks,
               k_scale: float = 1.0, v_scale: float = 1.0):
    """Store new bf16 K/V rows as E4M3 codes of x / scale into copies of FP8 pools
    [num_blocks][Hkv][B][D] (uint8); returns (k_pool, v_pool)."""
    kp = np.array(k_pool, dtype=np.uint8, copy=True)
    vp = np.array(v_pool, dtype=np.uint8, copy=True)
    kn, vn = _c(k_new, np.uint16), _c(v_new, np.uint16)
    sm = _c(slot_mapping, np.int32)
    rc = _load().oracle_append_fp8(_ptr(kp), _ptr(vp), _ptr(kn), _ptr(vn), _ptr(sm), int(sm.size), int(num_kv_heads),
                                   int(head_dim), int(block_size), int(num_blocks), float(k_scale), float(v_scale))
    if rc != 0:
        raise ValueError(f"oracle_append_fp8 failed with code {rc}")
    return kp, vp


def copy_blocks_fp8(k_pool, v_pool, src, dst, num_kv_heads, head_dim, block_size, num_blocks):
    """copy_blocks for FP8 pools (uint8, one byte per value)."""
    kp = np.array(k_pool, dtype=np.uint8, copy=True)
    vp = np.array(v_pool, dtype=np.uint8, copy=True)
    s, d = _c(src, np.int32), _c(dst, np.int32)
    if s.shape != d.shape:
        raise ValueError("src and dst differ in length")
    rc = _load().oracle_copy_blocks_fp8(_ptr(kp), _ptr(vp), _ptr(s), _ptr(d), int(s.size), int(num_kv_heads),
                                        int(head_dim), int(block_size), int(num_blocks))
    if rc != 0:
        raise ValueError(f"oracle_copy_blocks_fp8 failed with code {rc}")
    return kp, vp


def attention(q, k_pool, v_pool, block_tables, qo_len, kv_len, num_q_heads, num_kv_heads, head_dim,
              block_size, num_blocks, scale, row_select=None, want_f64: bool = False, kv_format: str = "bf16",
              k_scale: float = 1.0, v_scale: float = 1.0):
    """Returns dict(out=bf16 bits [total_q][Hq][D], lse=float32 [total_q][Hq], pairs=int,
    and out_f64 / lse_f64 when ``want_f64``).  Rows not in ``row_select`` are left as zero.
    ``kv_format`` "q8_0" reads the q8_0 pool [num_blocks][Hkv][2][tile bytes] (uint8) passed as
    ``k_pool`` (``v_pool`` is unused); "fp8" reads E4M3 pools (uint8) with ``k_scale`` / ``v_scale``."""
    qa = _c(q, np.uint16)
    extra = ()
    if kv_format == "q8_0":
        kp, fn = _c(k_pool, np.uint8), _load().oracle_attention_q8
        pools = (_ptr(kp),)
    elif kv_format == "fp8":
        kp, vp, fn = _c(k_pool, np.uint8), _c(v_pool, np.uint8), _load().oracle_attention_fp8
        pools = (_ptr(kp), _ptr(vp))
        extra = (float(k_scale), float(v_scale))
    elif kv_format == "bf16":
        kp, vp, fn = _c(k_pool, np.uint16), _c(v_pool, np.uint16), _load().oracle_attention
        pools = (_ptr(kp), _ptr(vp))
    else:
        raise ValueError(f"unknown kv_format {kv_format}")
    bt = _c(block_tables, np.int32)
    qo, kv = _c(qo_len, np.int32), _c(kv_len, np.int32)
    R = int(qo.size)
    total_q = int(qo.sum())
    out = np.zeros((total_q, num_q_heads, head_dim), np.uint16)
    lse = np.zeros((total_q, num_q_heads), np.float32)
    out64 = np.zeros((total_q, num_q_heads, head_dim), np.float64) if want_f64 else None
    lse64 = np.zeros((total_q, num_q_heads), np.float64) if want_f64 else None
    sel = None if row_select is None else _c(row_select, np.uint8)
    pairs = ctypes.c_int64(0)
    rc = fn(_ptr(qa), *pools, _ptr(bt), int(bt.shape[1]), _ptr(qo), _ptr(kv),
                                  R, int(num_q_heads), int(num_kv_heads), int(head_dim), int(block_size),
                                  int(num_blocks), float(scale), *extra, _ptr(sel), _ptr(out), _ptr(lse),
                                  _ptr(out64), _ptr(lse64), ctypes.cast(ctypes.pointer(pairs), ctypes.c_void_p))
    if rc != 0:
        raise ValueError(f"oracle_attention failed with code {rc}")
    res = dict(out=out, lse=lse, pairs=int(pairs.value))
    if want_f64:
        res["out_f64"] = out64
        res["lse_f64"] = lse64
    return res


def run_workload(wl, row_select=None, want_f64: bool = False):
    """Append the workload's new tokens, then attend; returns (k_pool, v_pool, result)."""
    fmt = getattr(wl, "kv_format", "bf16")
    ks, vs = getattr(wl, "k_scale", 1.0), getattr(wl, "v_scale", 1.0)
    if fmt == "q8_0":
        kp = append_q8(wl.kv_pool, wl.k_new, wl.v_new, wl.slot_mapping, wl.num_kv_heads, wl.head_dim,
                       wl.block_size, wl.num_blocks)
        vp = None
    elif fmt == "fp8":
        kp, vp = append_fp8(wl.k_pool, wl.v_pool, wl.k_new, wl.v_new, wl.slot_mapping, wl.num_kv_heads,
                            wl.head_dim, wl.block_size, wl.num_blocks, ks, vs)
    else:
        kp, vp = append(wl.k_pool, wl.v_pool, wl.k_new, wl.v_new, wl.slot_mapping, wl.num_kv_heads,
                        wl.head_dim, wl.block_size, wl.num_blocks)
    res = attention(wl.q, kp, vp, wl.block_tables, wl.qo_len, wl.kv_len, wl.num_q_heads, wl.num_kv_heads,
                    wl.head_dim, wl.block_size, wl.num_blocks, wl.scale, row_select=row_select,
                    want_f64=want_f64, kv_format=fmt, k_scale=ks, v_scale=vs)
    return kp, vp, res
