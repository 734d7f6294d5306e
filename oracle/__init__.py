"""CPU oracle for quantized paged attention -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously-correct host code (``oracle.c``) that the GPU path is
checked against. Only the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package; the library never
does. It shares no code with the HIP library.

Functions take numpy arrays; bf16 tensors travel as ``uint16`` bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

FMT_BF16, FMT_E4M3, FMT_E5M2, FMT_INT8 = 0, 1, 2, 3
MODE_PER_TENSOR, MODE_PER_TOKEN_HEAD, MODE_PER_GROUP = 0, 1, 2
GROUP = 32  # head-dim channels per scale in per-group mode


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` next to it (gcc + OpenMP)."""
    if force or not os.path.exists(_LIB):
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
               "-fno-fast-math", "-Wall", "-Wextra", "-Wno-unused-parameter",
               _SRC, "-o", _LIB + ".tmp", "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


class _Desc(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("fmt", ctypes.c_int32), ("mode", ctypes.c_int32)]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64, f32, f64, u32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_double, ctypes.c_uint32
        D = ctypes.POINTER(_Desc)
        lib.orc_num_threads.argtypes = []; lib.orc_num_threads.restype = ctypes.c_int
        lib.orc_decode.argtypes = [ctypes.c_int, u32]; lib.orc_decode.restype = f64
        lib.orc_encode.argtypes = [ctypes.c_int, f32]; lib.orc_encode.restype = u32
        lib.orc_encode_array.argtypes = [ctypes.c_int, P, i64, P]; lib.orc_encode_array.restype = None
        lib.orc_f64_to_bf16.argtypes = [f64]; lib.orc_f64_to_bf16.restype = ctypes.c_uint16
        lib.orc_qmax.argtypes = [ctypes.c_int]; lib.orc_qmax.restype = f32
        for name in ("orc_page_bytes", "orc_block_bytes", "orc_total_bytes"):
            getattr(lib, name).argtypes = [D]; getattr(lib, name).restype = i64
        lib.orc_page_offset.argtypes = [D, i64, ctypes.c_int, ctypes.c_int]; lib.orc_page_offset.restype = i64
        lib.orc_cache_write.argtypes = [D, P, P, P, i64, i64, P, f32, f32]; lib.orc_cache_write.restype = ctypes.c_int
        lib.orc_read_row.argtypes = [D, P, ctypes.c_int, i64, ctypes.c_int, ctypes.c_int, f32, f32, P]
        lib.orc_read_row.restype = None
        lib.orc_attention.argtypes = [D, P, P, P, i32, P, P, i32, i32, i32, i32, f64, f64, f32, f32, P, P]
        lib.orc_attention.restype = ctypes.c_int
        lib.orc_attention_weights.argtypes = [D, P, P, P, i32, P, P, i32, i32, i32, i32, f64, f64, f32, f32,
                                              i32, i32, i32, P]
        lib.orc_attention_weights.restype = ctypes.c_int
        lib.orc_attention_ext.argtypes = [D, P, P, P, i32, P, P, i32, i32, i32, P, i32, f64, f64, P, P, f32, f32,
                                          P, P]
        lib.orc_attention_ext.restype = ctypes.c_int
        lib.orc_attention_weights_ext.argtypes = [D, P, P, P, i32, P, P, i32, i32, i32, i32, f64, f64, f64, f64,
                                                  f32, f32, i32, i32, i32, P]
        lib.orc_attention_weights_ext.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


class CacheDesc:
    """Cache geometry: pool of ``num_blocks`` blocks of ``block_size`` slots."""

    def __init__(self, num_blocks, block_size, num_kv_heads, head_dim, fmt, mode):
        self.c = _Desc(num_blocks, block_size, num_kv_heads, head_dim, fmt, mode)

    def __getattr__(self, k):
        return getattr(self.__dict__["c"], k)

    @property
    def page_bytes(self):
        return _load().orc_page_bytes(ctypes.byref(self.c))

    @property
    def block_bytes(self):
        return _load().orc_block_bytes(ctypes.byref(self.c))

    @property
    def total_bytes(self):
        return _load().orc_total_bytes(ctypes.byref(self.c))

    def page_offset(self, block, kv, head):
        return _load().orc_page_offset(ctypes.byref(self.c), block, kv, head)


def num_threads() -> int:
    return _load().orc_num_threads()


def decode(fmt: int, code: int) -> float:
    return _load().orc_decode(fmt, code)


def decode_table(fmt: int) -> np.ndarray:
    return np.array([decode(fmt, c) for c in range(256)], dtype=np.float64)


def encode(fmt: int, y: float) -> int:
    return _load().orc_encode(fmt, y)


def encode_array(fmt: int, y: np.ndarray) -> np.ndarray:
    y = np.ascontiguousarray(y, dtype=np.float32)
    out = np.empty(y.shape, dtype=np.uint8)
    _load().orc_encode_array(fmt, _ptr(y), y.size, _ptr(out))
    return out


def qmax(fmt: int) -> float:
    return _load().orc_qmax(fmt)


def f64_to_bf16(x: float) -> int:
    return _load().orc_f64_to_bf16(x)


def cache_write(desc: CacheDesc, cache: np.ndarray, k: np.ndarray, v: np.ndarray, slot_mapping: np.ndarray,
                k_scale: float = 1.0, v_scale: float = 1.0) -> None:
    """Quantise bf16 K/V ``[N, Hkv, D]`` (uint16 bits) into ``cache`` (uint8, in place)."""
    assert cache.dtype == np.uint8 and cache.size >= desc.total_bytes
    assert k.dtype == np.uint16 and v.dtype == np.uint16 and k.shape == v.shape
    slot_mapping = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    n = k.shape[0]
    stride = desc.num_kv_heads * desc.head_dim
    rc = _load().orc_cache_write(ctypes.byref(desc.c), _ptr(cache), _ptr(np.ascontiguousarray(k)),
                                 _ptr(np.ascontiguousarray(v)), n, stride, _ptr(slot_mapping),
                                 float(k_scale), float(v_scale))
    if rc != 0:
        raise ValueError("oracle cache_write: slot outside the pool")


def read_row(desc: CacheDesc, cache: np.ndarray, kv: int, block: int, head: int, off: int,
             k_scale: float = 1.0, v_scale: float = 1.0) -> np.ndarray:
    row = np.empty(desc.head_dim, dtype=np.float64)
    _load().orc_read_row(ctypes.byref(desc.c), _ptr(cache), kv, block, head, off, k_scale, v_scale, _ptr(row))
    return row


def attention(desc: CacheDesc, cache: np.ndarray, q: np.ndarray, block_tables: np.ndarray,
              seq_lens: np.ndarray, query_start_loc: np.ndarray, num_q_heads: int, causal: bool = True,
              window: int = 0, sm_scale: float = 0.0, softcap: float = 0.0, k_scale: float = 1.0,
              v_scale: float = 1.0, want_f64: bool = False, causal_per_seq=None, alibi_slopes=None,
              sinks=None):
    """Plain fp64 attention over the dequantised cache. Returns bf16 bits ``[T_q, Hq, D]`` (uint16)
    and, if ``want_f64``, the fp64 values before rounding. ``causal_per_seq`` (int per sequence),
    ``alibi_slopes`` and ``sinks`` (one float per q head) follow ``orc_attention_ext``."""
    q = np.ascontiguousarray(q, dtype=np.uint16)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    qsl = np.ascontiguousarray(query_start_loc, dtype=np.int32)
    out = np.zeros(q.shape, dtype=np.uint16)
    o64 = np.zeros(q.shape, dtype=np.float64) if want_f64 else None
    cps = None if causal_per_seq is None else np.ascontiguousarray(causal_per_seq, dtype=np.int32)
    al = None if alibi_slopes is None else np.ascontiguousarray(alibi_slopes, dtype=np.float64)
    sk = None if sinks is None else np.ascontiguousarray(sinks, dtype=np.float64)
    rc = _load().orc_attention_ext(ctypes.byref(desc.c), _ptr(cache), _ptr(q), _ptr(bt), bt.shape[1], _ptr(sl),
                                   _ptr(qsl), sl.shape[0], num_q_heads, int(causal), _ptr(cps), int(window),
                                   float(sm_scale), float(softcap), _ptr(al), _ptr(sk), float(k_scale),
                                   float(v_scale), _ptr(out), _ptr(o64))
    if rc != 0:
        raise ValueError("oracle attention: invalid arguments")
    return (out, o64) if want_f64 else out


def attention_weights(desc: CacheDesc, cache: np.ndarray, q: np.ndarray, block_tables: np.ndarray,
                      seq_lens: np.ndarray, query_start_loc: np.ndarray, num_q_heads: int, b: int, i: int,
                      hq: int, causal: bool = True, window: int = 0, sm_scale: float = 0.0,
                      softcap: float = 0.0, k_scale: float = 1.0, v_scale: float = 1.0, alibi_slope: float = 0.0,
                      sink: float = float("-inf")) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.uint16)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    qsl = np.ascontiguousarray(query_start_loc, dtype=np.int32)
    w = np.zeros(max(int(sl[b]), 1), dtype=np.float64)
    rc = _load().orc_attention_weights_ext(ctypes.byref(desc.c), _ptr(cache), _ptr(q), _ptr(bt), bt.shape[1],
                                           _ptr(sl), _ptr(qsl), sl.shape[0], num_q_heads, int(causal), int(window),
                                           float(sm_scale), float(softcap), float(alibi_slope), float(sink),
                                           float(k_scale), float(v_scale), b, i, hq, _ptr(w))
    if rc != 0:
        raise ValueError("oracle attention_weights: invalid arguments")
    return w[: int(sl[b])]
