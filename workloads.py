"""Seeded synthetic workloads for quantized paged attention.

The one module shared by the tests, the benchmark and the oracle runs: it only
draws inputs (query/key/value values, sequence lengths, block tables, slot
mappings, per-tensor calibration scales) and holds none of the method's own
arithmetic. Every array is produced once on the host; the GPU and the oracle
consume identical bytes.

Shapes follow the varlen paged harness of the "Fix CPU FP8 attention scheduler
scratch sizing" page (vllm PR 50194, Code excerpt: (query_len, kv_len) tuples,
num_heads=(q, kv), head_size, block_size, num_blocks, sliding_window,
soft_cap, kv_cache_dtype) and the KV modes of the per-token-head page
(vllm PR 38378). The pages measure on gsm8k and a serving benchmark; those
need datasets and trained weights, so these seeded inputs stand in for them.

Recipe (per workload, seed fixed below):
  * values: fp32 draws from N(0, sigma^2) with numpy's PCG64 generators
    (one child seed per tensor and per fixed 1/16 chunk of its rows, so the
    values do not depend on the thread count), optional outliers (a seeded
    Bernoulli mask multiplies entries by a factor), then rounded to bf16
    (nearest, ties to even);
  * block tables: a seeded permutation of the block pool; sequence b takes the
    next ceil(L_b / block_size) entries; unused entries are -1;
  * slot of token j of sequence b: table[b][j // bs] * bs + j % bs;
  * per-tensor scales (calibration inputs, not computed by the method):
    absmax over the whole K (resp. V) history divided by the format's largest
    code magnitude, in fp32.
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import os
from typing import Tuple

import numpy as np

QMAX = {"fp8_e4m3": 448.0, "fp8_e5m2": 57344.0, "int8": 127.0}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    kv_dtype: str                 # string accepted by the library's dtype parser
    seqs: Tuple[Tuple[int, int], ...]  # (query_len, kv_len) per sequence
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    window: int = 0
    softcap: float = 0.0
    sigma: float = 1.0
    outlier_frac: float = 0.0
    outlier_factor: float = 1.0
    seed: int = 0
    causal: bool = True

    @property
    def seq_lens(self) -> np.ndarray:
        return np.array([l for _, l in self.seqs], dtype=np.int32)

    @property
    def query_lens(self) -> np.ndarray:
        return np.array([q for q, _ in self.seqs], dtype=np.int32)


def _cfg3_seqs(seed: int) -> Tuple[Tuple[int, int], ...]:
    rng = np.random.default_rng(seed)
    lens = rng.integers(512, 8192, size=64, endpoint=True)
    return tuple((1, int(l)) for l in lens)


# The five configurations (the fifth run twice, with two KV modes).
CFG1 = Workload("tiny_decode_fp8e4m3_pt", "fp8_e4m3", ((1, 17), (1, 40)), 4, 2, 64, 16, 8, seed=1001)
CFG2 = Workload("prefill_fp8e4m3_pt_d256_bs2176", "fp8_e4m3", ((1024, 1024),) * 4, 16, 2, 256, 2176, 4,
                seed=1002)
CFG3 = Workload("decode64_fp8e4m3_pt_llama8b", "fp8_e4m3", _cfg3_seqs(1003), 32, 8, 128, 16, 40000,
                outlier_frac=0.01, outlier_factor=20.0, seed=1003)
CFG4 = Workload("mixed_int8_pth", "int8_per_token_head", ((1, 4096),) * 16 + ((512, 2560),) * 2, 32, 8, 128, 16,
                16 * 256 + 2 * 160, seed=1004)
CFG5A = Workload("longctx_fp8e4m3_pth_w4096_cap50", "fp8_per_token_head", ((1, 32768),) * 16, 64, 8, 128, 16,
                 16 * 2048, window=4096, softcap=50.0, sigma=1.5, seed=1005)
CFG5B = Workload("longctx_fp8e5m2_pt_w4096_cap50", "fp8_e5m2", ((1, 32768),) * 16, 64, 8, 128, 16,
                 16 * 2048, window=4096, softcap=50.0, sigma=1.5, seed=1005)

ALL = {w.name: w for w in (CFG1, CFG2, CFG3, CFG4, CFG5A, CFG5B)}


def scaled(w: Workload, **kw) -> Workload:
    """A variant of a workload (used for small parity cases of the big shapes)."""
    return dataclasses.replace(w, **kw)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even (torch's CPU cast)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


_CHUNKS = 16


def _draw_chunk(seed_seq: np.random.SeedSequence, shape, w: Workload) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed_seq))
    x = rng.standard_normal(shape, dtype=np.float32)
    if w.sigma != 1.0:
        x *= np.float32(w.sigma)
    if w.outlier_frac > 0.0:
        mask = rng.random(shape, dtype=np.float32) < np.float32(w.outlier_frac)
        x[mask] *= np.float32(w.outlier_factor)
    return bf16_round(x)


def _draw(seed_seq: np.random.SeedSequence, shape, w: Workload) -> np.ndarray:
    """bf16 bits of the given shape; rows split into _CHUNKS fixed pieces with their own child seeds."""
    n = shape[0]
    out = np.empty(shape, dtype=np.uint16)
    if n == 0:
        return out
    bounds = np.linspace(0, n, _CHUNKS + 1).astype(np.int64)
    kids = seed_seq.spawn(_CHUNKS)

    def fill(i):
        lo, hi = int(bounds[i]), int(bounds[i + 1])
        if hi > lo:
            out[lo:hi] = _draw_chunk(kids[i], (hi - lo,) + tuple(shape[1:]), w)

    with concurrent.futures.ThreadPoolExecutor(max_workers=min(_CHUNKS, os.cpu_count() or 1)) as ex:
        list(ex.map(fill, range(_CHUNKS)))
    return out


@dataclasses.dataclass
class Batch:
    w: Workload
    seq_lens: np.ndarray          # int32 [B]
    query_start_loc: np.ndarray   # int32 [B+1]
    block_tables: np.ndarray      # int32 [B, max_blocks]
    q: np.ndarray                 # bf16 bits [T_q, Hq, D]
    k_hist: np.ndarray            # bf16 bits [sum L, Hkv, D]: every key of every sequence, in sequence order
    v_hist: np.ndarray
    slots_hist: np.ndarray        # int64 [sum L]
    new_mask: np.ndarray          # bool [sum L]: the step's own tokens (last query_len of each sequence)
    k_scale: float
    v_scale: float

    @property
    def kv_start(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.seq_lens, dtype=np.int64)])


def make_batch(w: Workload, with_kv: bool = True) -> Batch:
    ss_tables, ss_q, ss_k, ss_v = np.random.SeedSequence(w.seed).spawn(4)
    rng = np.random.Generator(np.random.PCG64(ss_tables))
    B = len(w.seqs)
    qlens = w.query_lens
    lens = w.seq_lens
    assert np.all(qlens <= lens)
    need = (lens.astype(np.int64) + w.block_size - 1) // w.block_size
    assert need.sum() <= w.num_blocks, "block pool too small for the workload"
    max_blocks = int(max(1, need.max()))
    perm = rng.permutation(w.num_blocks).astype(np.int32)
    bt = np.full((B, max_blocks), -1, dtype=np.int32)
    pos = 0
    for b in range(B):
        bt[b, : need[b]] = perm[pos: pos + need[b]]
        pos += int(need[b])
    qsl = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    Hq, Hkv, D = w.num_q_heads, w.num_kv_heads, w.head_dim
    q = _draw(ss_q, (int(qsl[-1]), Hq, D), w)
    total = int(lens.sum())
    slots = np.empty(total, dtype=np.int64)
    new_mask = np.zeros(total, dtype=bool)
    off = 0
    for b in range(B):
        j = np.arange(int(lens[b]), dtype=np.int64)
        slots[off: off + lens[b]] = bt[b, j // w.block_size].astype(np.int64) * w.block_size + j % w.block_size
        new_mask[off + lens[b] - qlens[b]: off + lens[b]] = True
        off += int(lens[b])
    if with_kv:
        k = _draw(ss_k, (total, Hkv, D), w)
        v = _draw(ss_v, (total, Hkv, D), w)
    else:
        k = v = np.zeros((0, Hkv, D), dtype=np.uint16)
    k_scale = v_scale = 1.0
    fmt = w.kv_dtype
    if fmt in ("fp8_e4m3", "fp8_e5m2", "fp8", "int8") and with_kv:
        qm = np.float32(QMAX[{"fp8_e5m2": "fp8_e5m2", "int8": "int8"}.get(fmt, "fp8_e4m3")])
        k_scale = float(np.float32(np.abs(bf16_to_f32(k)).max()) / qm)
        v_scale = float(np.float32(np.abs(bf16_to_f32(v)).max()) / qm)
    return Batch(w, lens, qsl, bt, q, k, v, slots, new_mask, k_scale, v_scale)


def kv_read_bytes(w: Workload, per_token_head: bool) -> int:
    """Algorithmic KV bytes a decode step must read: every visible key and value code of every
    decode sequence (and its inline scales in per-token-head mode)."""
    total = 0
    per_tok = 2 * w.head_dim + (8 if per_token_head else 0)
    for ql, L in w.seqs:
        if ql != 1:
            continue
        eff = min(L, w.window) if w.window > 0 else L
        total += eff * w.num_kv_heads * per_tok
    return total


def prefill_flops(w: Workload) -> int:
    """Algorithmic flops of the prefill sequences: 4 * D per visible (query, key) pair per q head."""
    total = 0
    for ql, L in w.seqs:
        if ql == 1:
            continue
        pairs = 0
        for i in range(ql):
            p = L - ql + i
            hi = p if w.causal else L - 1
            lo = max(0, p - w.window + 1) if w.window > 0 else 0
            pairs += hi - lo + 1
        total += pairs * 4 * w.head_dim * w.num_q_heads
    return total
