"""Python binding of libaqp.so: quantized paged attention for MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/aqp.h``; there is no Python or
CPU fallback. Importing this package without the built library raises.

Functions accept torch tensors (device memory for device arguments) or plain
integers (raw pointers); bf16 data travels as ``torch.bfloat16`` or
``torch.int16`` / ``torch.uint16`` bit patterns.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libaqp.so")

KV_AUTO, KV_FP8_E4M3, KV_FP8_E5M2, KV_INT8 = 0, 1, 2, 3
SCALE_PER_TENSOR, SCALE_PER_TOKEN_HEAD, SCALE_PER_GROUP = 0, 1, 2
OK, ERR_INVALID, ERR_UNSUPPORTED, ERR_SCHEDULE_MISMATCH, ERR_SCRATCH_TOO_SMALL, ERR_HIP = 0, -1, -2, -3, -4, -5


class AqpError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"aqp status {status}: {message}")
        self.status = status
        self.message = message


class CacheDesc(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32), ("mode", ctypes.c_int32)]


class AttnParams(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("causal", ctypes.c_int32), ("window", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32),
                ("sm_scale", ctypes.c_float), ("softcap", ctypes.c_float), ("decode_parallelism", ctypes.c_int32),
                ("prefill_rows", ctypes.c_int32), ("causal_per_seq", ctypes.c_void_p), ("alibi_slopes", ctypes.c_void_p),
                ("sinks", ctypes.c_void_p), ("prefill_kv_split", ctypes.c_int32)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python attention_quantized_paged_amd/build.py` "
                          "(there is no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    P, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    lib.aqp_parse_kv_dtype.argtypes = [ctypes.c_char_p, ctypes.POINTER(i32), ctypes.POINTER(i32)]
    lib.aqp_cache_bytes.argtypes = [ctypes.POINTER(CacheDesc), ctypes.POINTER(sz), ctypes.POINTER(sz),
                                    ctypes.POINTER(sz)]
    lib.aqp_cache_write.argtypes = [ctypes.POINTER(CacheDesc), P, P, P, i64, i64, P, f32, f32, P]
    lib.aqp_get_schedule.argtypes = [ctypes.POINTER(AttnParams), ctypes.POINTER(CacheDesc), P, P, i32, P,
                                     ctypes.POINTER(sz), ctypes.POINTER(sz)]
    lib.aqp_paged_attention.argtypes = [ctypes.POINTER(AttnParams), ctypes.POINTER(CacheDesc), P, P, P, P, P, f32,
                                        f32, P, sz, P, P]
    lib.aqp_paged_attention_noalloc.argtypes = [ctypes.POINTER(AttnParams), ctypes.POINTER(CacheDesc), P, P, P, P,
                                                P, f32, f32, P, P]
    lib.aqp_paged_attention_timed.argtypes = [ctypes.POINTER(AttnParams), ctypes.POINTER(CacheDesc), P, P, P, P, P,
                                              f32, f32, P, sz, P, P, ctypes.POINTER(P), i32]
    lib.aqp_last_error.argtypes = []
    lib.aqp_last_error.restype = ctypes.c_char_p
    for fn in ("aqp_parse_kv_dtype", "aqp_cache_bytes", "aqp_cache_write", "aqp_get_schedule", "aqp_paged_attention",
               "aqp_paged_attention_noalloc", "aqp_paged_attention_timed"):
        getattr(lib, fn).restype = ctypes.c_int
    return lib


_lib = _load()
EXPORTED = ("aqp_parse_kv_dtype", "aqp_cache_bytes", "aqp_cache_write", "aqp_get_schedule", "aqp_paged_attention",
            "aqp_last_error")


def _check(rc: int) -> None:
    if rc != OK:
        raise AqpError(rc, _lib.aqp_last_error().decode())


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if isinstance(x, np.ndarray):
        return x.ctypes.data
    return x.data_ptr()  # torch tensor


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _dev_ok(t, name: str, contiguous: bool = True) -> None:
    if hasattr(t, "is_cuda") and not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if contiguous and hasattr(t, "is_contiguous") and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _nbytes(t) -> Optional[int]:
    """Bytes a buffer argument spans (None for raw pointers, which are taken as given)."""
    if t is None or isinstance(t, int):
        return None
    if isinstance(t, np.ndarray):
        return t.nbytes
    if hasattr(t, "untyped_storage"):
        # a view may start inside its storage: the bytes from its first element to the storage end
        st = t.untyped_storage()
        return st.nbytes() - (t.data_ptr() - st.data_ptr())
    return None


def _need(t, nbytes: int, name: str) -> None:
    have = _nbytes(t)
    if have is not None and have < nbytes:
        raise ValueError(f"{name} spans {have} bytes, the call needs {nbytes}")


def parse_kv_dtype(s: str) -> Tuple[int, int]:
    dt, md = ctypes.c_int32(), ctypes.c_int32()
    _check(_lib.aqp_parse_kv_dtype(s.encode(), ctypes.byref(dt), ctypes.byref(md)))
    return dt.value, md.value


def cache_desc(num_blocks: int, block_size: int, num_kv_heads: int, head_dim: int, kv_cache_dtype: str) -> CacheDesc:
    dt, md = parse_kv_dtype(kv_cache_dtype)
    return CacheDesc(num_blocks, block_size, num_kv_heads, head_dim, dt, md)


def attn_params(num_q_heads: int, num_kv_heads: int, head_dim: int, max_blocks_per_seq: int, causal: bool = True,
                window: int = 0, sm_scale: float = 0.0, softcap: float = 0.0,
                decode_parallelism: int = 0, causal_per_seq=None, alibi_slopes=None, sinks=None,
                prefill_rows: int = 0, prefill_kv_split: int = 0) -> AttnParams:
    """causal_per_seq: host int sequence (one flag per sequence) or None; alibi_slopes, sinks:
    device float32 tensors of num_q_heads values (anything with ``data_ptr()``) or None. The
    returned object keeps them alive."""
    p = AttnParams(num_q_heads, num_kv_heads, head_dim, int(causal), window, max_blocks_per_seq, sm_scale,
                   softcap, decode_parallelism, prefill_rows, None, None, None, prefill_kv_split)
    keep = []
    if causal_per_seq is not None:
        cps = np.ascontiguousarray(np.asarray(causal_per_seq), dtype=np.int32)
        keep.append(cps)
        p.causal_per_seq = cps.ctypes.data
    for name, t in (("alibi_slopes", alibi_slopes), ("sinks", sinks)):
        if t is not None:
            if hasattr(t, "dtype") and str(t.dtype) != "torch.float32":
                raise TypeError(f"{name} must be float32")
            if hasattr(t, "numel") and t.numel() != num_q_heads:
                raise ValueError(f"{name} needs num_q_heads values")
            keep.append(t)
            setattr(p, name, t.data_ptr())
    p._keep = keep
    return p


def cache_bytes(desc: CacheDesc) -> Tuple[int, int, int]:
    p, b, t = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(_lib.aqp_cache_bytes(ctypes.byref(desc), ctypes.byref(p), ctypes.byref(b), ctypes.byref(t)))
    return p.value, b.value, t.value


def cache_write(desc: CacheDesc, cache, k, v, slot_mapping, k_scale: float = 1.0, v_scale: float = 1.0,
                token_stride: Optional[int] = None, stream=None) -> None:
    """k, v: bf16 [N, Hkv, D] (token stride may exceed Hkv*D); slot_mapping: int64 [N]."""
    n = int(k.shape[0]) if hasattr(k, "shape") else 0
    if token_stride is None:
        token_stride = int(k.stride(0)) if hasattr(k, "stride") else desc.num_kv_heads * desc.head_dim
    for t, nm in ((cache, "cache"), (slot_mapping, "slot_mapping")):
        _dev_ok(t, nm)
    for t, nm in ((k, "k"), (v, "v")):
        _dev_ok(t, nm, contiguous=False)
    # every buffer spans what the kernel reads or writes, so a mis-sized tensor is refused on the
    # host instead of becoming an out-of-range access on the device
    _need(cache, cache_bytes(desc)[2], "cache")
    if n > 0:
        row = desc.num_kv_heads * desc.head_dim
        if token_stride < row:
            raise ValueError(f"token_stride {token_stride} < num_kv_heads * head_dim = {row}")
        _need(k, 2 * ((n - 1) * token_stride + row), "k")
        _need(v, 2 * ((n - 1) * token_stride + row), "v")
        _need(slot_mapping, 8 * n, "slot_mapping")
        if hasattr(slot_mapping, "element_size") and slot_mapping.element_size() != 8:
            raise ValueError("slot_mapping must be int64")
    _check(_lib.aqp_cache_write(ctypes.byref(desc), _ptr(cache), _ptr(k), _ptr(v), n, token_stride,
                                _ptr(slot_mapping), float(k_scale), float(v_scale), _stream(stream)))


class Schedule:
    """Host bytes of a schedule (``meta``; may be a view of a caller buffer), its scratch size,
    and its header fields (parsed on first use)."""

    def __init__(self, meta: np.ndarray, scratch_bytes: int):
        self.meta = meta
        self.scratch_bytes = scratch_bytes
        self._header = None

    @property
    def header(self) -> dict:
        if self._header is None:
            self._header = parse_header(self.meta)
        return self._header


_HDR_FIELDS = ("magic version dtype mode kv_elem_bytes staged_elem_bytes scale_bytes head_dim block_size num_blocks "
               "num_q_heads num_kv_heads causal window max_blocks_per_seq num_seqs sm_scale softcap total_q_tokens "
               "tile_keys dec_iter_keys dec_waves pf_rows pf_kv_tile heads_per_unit dec_lds_bytes pf_lds_bytes "
               "num_dec_wgs num_dec_segs num_parts num_comb num_pf_items group_heads").split()
_HDR_FIELDS64 = ("off_dec_segs off_dec_wg_start off_comb off_pf_items meta_bytes scratch_bytes page_bytes block_bytes "
                 "dec_kv_keys off_seq_lens num_slots comb_heads num_pf_split num_dec_comb off_dec_first").split()


def parse_header(meta: np.ndarray) -> dict:
    n32 = len(_HDR_FIELDS)
    w = meta[: 4 * n32].view(np.uint32)
    out = {}
    for i, name in enumerate(_HDR_FIELDS):
        if name in ("sm_scale", "softcap"):
            out[name] = float(w[i:i + 1].view(np.float32)[0])
        elif name in ("magic", "version"):
            out[name] = int(w[i])
        else:
            out[name] = int(w[i:i + 1].view(np.int32)[0])
    off = (4 * n32 + 7) // 8 * 8
    w64 = meta[off: off + 8 * len(_HDR_FIELDS64)].view(np.int64)
    for i, name in enumerate(_HDR_FIELDS64):
        out[name] = int(w64[i])
    return out


def get_schedule(params: AttnParams, desc: CacheDesc, seq_lens, query_start_loc,
                 out: Optional[np.ndarray] = None) -> Schedule:
    """seq_lens, query_start_loc: host int32 arrays. With ``out`` (a uint8 host buffer, e.g. the
    numpy view of a pinned tensor) the schedule is written there in one call when it fits."""
    sl = seq_lens if (isinstance(seq_lens, np.ndarray) and seq_lens.dtype == np.int32 and
                      seq_lens.flags["C_CONTIGUOUS"]) else np.ascontiguousarray(np.asarray(seq_lens), dtype=np.int32)
    qsl = query_start_loc if (isinstance(query_start_loc, np.ndarray) and query_start_loc.dtype == np.int32 and
                              query_start_loc.flags["C_CONTIGUOUS"]) else \
        np.ascontiguousarray(np.asarray(query_start_loc), dtype=np.int32)
    if qsl.shape[0] != sl.shape[0] + 1:
        raise ValueError("query_start_loc must have num_seqs + 1 entries")
    scratch = ctypes.c_size_t(0)
    if out is not None:
        nbytes = ctypes.c_size_t(out.size)
        rc = _lib.aqp_get_schedule(ctypes.byref(params), ctypes.byref(desc), sl.ctypes.data, qsl.ctypes.data,
                                   sl.shape[0], out.ctypes.data, ctypes.byref(nbytes), ctypes.byref(scratch))
        if rc == OK:
            return Schedule(out[: nbytes.value], scratch.value)
        if nbytes.value <= out.size:
            _check(rc)
    nbytes = ctypes.c_size_t(0)
    _check(_lib.aqp_get_schedule(ctypes.byref(params), ctypes.byref(desc), sl.ctypes.data, qsl.ctypes.data,
                                 sl.shape[0], None, ctypes.byref(nbytes), ctypes.byref(scratch)))
    meta = np.zeros(nbytes.value, dtype=np.uint8)
    _check(_lib.aqp_get_schedule(ctypes.byref(params), ctypes.byref(desc), sl.ctypes.data, qsl.ctypes.data,
                                 sl.shape[0], meta.ctypes.data, ctypes.byref(nbytes), ctypes.byref(scratch)))
    return Schedule(meta, scratch.value)


def paged_attention(params: AttnParams, desc: CacheDesc, cache, q, block_tables, meta_host, meta_dev,
                    k_scale: float, v_scale: float, scratch, scratch_bytes: int, out, stream=None,
                    events=None) -> None:
    """With ``events`` (up to 6 hipEvent_t handles) the call goes through aqp_paged_attention_timed,
    which records them around each of its kernels on the call's stream."""
    for t, nm in ((cache, "cache"), (q, "q"), (block_tables, "block_tables"), (meta_dev, "meta_dev"), (out, "out")):
        _dev_ok(t, nm)
    if isinstance(meta_host, np.ndarray) and meta_host.nbytes >= 256:
        # sizes the kernels assume, from the schedule they will run (the library itself checks the
        # schedule against desc and params; it cannot see how large the caller's buffers are)
        h = parse_header(meta_host)
        if h["magic"] == 0x53505141:
            rowb = 2 * h["num_q_heads"] * h["head_dim"]
            _need(q, h["total_q_tokens"] * rowb, "q")
            _need(out, h["total_q_tokens"] * rowb, "out")
            _need(block_tables, 4 * h["num_seqs"] * h["max_blocks_per_seq"], "block_tables")
            _need(meta_dev, h["meta_bytes"], "meta_dev")
            _need(cache, cache_bytes(desc)[2], "cache")
            _need(scratch, int(scratch_bytes), "scratch")
    if events is None:
        _check(_lib.aqp_paged_attention(ctypes.byref(params), ctypes.byref(desc), _ptr(cache), _ptr(q),
                                        _ptr(block_tables), _ptr(meta_host), _ptr(meta_dev), float(k_scale),
                                        float(v_scale), _ptr(scratch), int(scratch_bytes), _ptr(out), _stream(stream)))
        return
    # events: up to 6 raw hipEvent_t handles (ints, or None to skip a point)
    ev = (ctypes.c_void_p * len(events))(*[ctypes.c_void_p(int(e)) if e else None for e in events])
    _check(_lib.aqp_paged_attention_timed(ctypes.byref(params), ctypes.byref(desc), _ptr(cache), _ptr(q),
                                          _ptr(block_tables), _ptr(meta_host), _ptr(meta_dev), float(k_scale),
                                          float(v_scale), _ptr(scratch), int(scratch_bytes), _ptr(out),
                                          _stream(stream), ev, len(events)))


# scratch bytes of the library's own buffer behind paged_attention_noalloc
NOALLOC_SCRATCH_BYTES = 64 << 20


def paged_attention_noalloc(params: AttnParams, desc: CacheDesc, cache, q, block_tables, meta_host, meta_dev,
                            k_scale: float, v_scale: float, out, stream=None) -> None:
    """paged_attention with the library's fixed scratch buffer (for callers that cannot allocate)."""
    for t, nm in ((cache, "cache"), (q, "q"), (block_tables, "block_tables"), (meta_dev, "meta_dev"), (out, "out")):
        _dev_ok(t, nm)
    if isinstance(meta_host, np.ndarray) and meta_host.nbytes >= 256:
        h = parse_header(meta_host)
        if h["magic"] == 0x53505141:
            rowb = 2 * h["num_q_heads"] * h["head_dim"]
            _need(q, h["total_q_tokens"] * rowb, "q")
            _need(out, h["total_q_tokens"] * rowb, "out")
            _need(block_tables, 4 * h["num_seqs"] * h["max_blocks_per_seq"], "block_tables")
            _need(meta_dev, h["meta_bytes"], "meta_dev")
            _need(cache, cache_bytes(desc)[2], "cache")
    _check(_lib.aqp_paged_attention_noalloc(ctypes.byref(params), ctypes.byref(desc), _ptr(cache), _ptr(q),
                                            _ptr(block_tables), _ptr(meta_host), _ptr(meta_dev), float(k_scale),
                                            float(v_scale), _ptr(out), _stream(stream)))


def last_error() -> str:
    return _lib.aqp_last_error().decode()
