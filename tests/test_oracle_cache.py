"""Pins of the oracle's cache write (quantise + scatter into pages).

Lossless inputs (x = code value * power-of-two scale) must reproduce their codes
exactly; per-token-head scales must equal absmax / qmax; the dequantisation
error of ordinary inputs must stay within half a code step; negative slots are
skipped; every written byte lands in a distinct place.
"""
import numpy as np
import pytest

import oracle
from tests.oracle_helpers import code_values, lossless_kv, random_codes

FMTS = [oracle.FMT_E4M3, oracle.FMT_E5M2, oracle.FMT_INT8]


def _desc(fmt, mode, nb=6, bs=16, hkv=2, d=64):
    return oracle.CacheDesc(nb, bs, hkv, d, fmt, mode)


@pytest.mark.parametrize("fmt", [oracle.FMT_E4M3, oracle.FMT_E5M2])
@pytest.mark.parametrize("scale_exp", [-7, 0, 3])
def test_per_tensor_lossless_roundtrip(fmt, scale_exp):
    rng = np.random.default_rng(11 + fmt + scale_exp)
    d = _desc(fmt, oracle.MODE_PER_TENSOR)
    n = 40
    s = 2.0 ** scale_exp
    kb, kx = lossless_kv(rng, fmt, n, 2, 64, s)
    vb, vx = lossless_kv(rng, fmt, n, 2, 64, s)
    slots = rng.permutation(d.num_blocks * d.block_size)[:n].astype(np.int64)
    cache = np.zeros(d.total_bytes, dtype=np.uint8)
    oracle.cache_write(d, cache, kb, vb, slots, s, s)
    for t in range(n):
        blk, off = divmod(int(slots[t]), d.block_size)
        for h in range(2):
            assert np.array_equal(oracle.read_row(d, cache, 0, blk, h, off, s, s), kx[t, h])
            assert np.array_equal(oracle.read_row(d, cache, 1, blk, h, off, s, s), vx[t, h])


@pytest.mark.parametrize("fmt", [oracle.FMT_E4M3, oracle.FMT_INT8])
def test_per_token_head_scale_is_absmax_over_qmax(fmt):
    rng = np.random.default_rng(21 + fmt)
    d = _desc(fmt, oracle.MODE_PER_TOKEN_HEAD)
    n = 33
    scales = 2.0 ** rng.integers(-10, 4, size=1)[0]
    kb, kx = lossless_kv(rng, fmt, n, 2, 64, scales, per_token_head=True)
    vb, vx = lossless_kv(rng, fmt, n, 2, 64, scales * 2, per_token_head=True)
    slots = np.arange(n, dtype=np.int64) * 2 + 1
    cache = np.zeros(d.total_bytes, dtype=np.uint8)
    oracle.cache_write(d, cache, kb, vb, slots)
    for t in range(n):
        blk, off = divmod(int(slots[t]), d.block_size)
        for h in range(2):
            assert np.array_equal(oracle.read_row(d, cache, 0, blk, h, off), kx[t, h])
            assert np.array_equal(oracle.read_row(d, cache, 1, blk, h, off), vx[t, h])
            # stored scale: the fp32 of absmax/qmax, read from the page tail
            page = d.page_offset(blk, 0, h)
            sc = cache[page + d.block_size * 64 + 4 * off: page + d.block_size * 64 + 4 * off + 4].view(np.float32)[0]
            amax = np.abs(kx[t, h]).max()
            assert sc == np.float32(amax) / np.float32(oracle.qmax(fmt))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("mode", [oracle.MODE_PER_TENSOR, oracle.MODE_PER_TOKEN_HEAD])
def test_dequant_error_within_half_step(fmt, mode):
    rng = np.random.default_rng(31 + fmt + 10 * mode)
    d = _desc(fmt, mode)
    n = 64
    x = (rng.standard_normal((n, 2, 64)) * 3).astype(np.float32)
    from workloads import bf16_round, bf16_to_f32
    kb = bf16_round(x)
    xv = bf16_to_f32(kb).astype(np.float64)
    qm = oracle.qmax(fmt)
    s = float(np.float32(np.abs(xv).max()) / np.float32(qm))
    slots = np.arange(n, dtype=np.int64)
    cache = np.zeros(d.total_bytes, dtype=np.uint8)
    oracle.cache_write(d, cache, kb, kb, slots, s, s)
    vals = code_values(fmt, np.arange(256))
    fin = np.sort(np.unique(np.abs(vals[np.isfinite(vals)])))
    for t in range(n):
        blk, off = divmod(t, d.block_size)
        for h in range(2):
            row = oracle.read_row(d, cache, 0, blk, h, off, s, s)
            if mode == oracle.MODE_PER_TOKEN_HEAD:
                rs = float(np.float32(np.abs(xv[t, h]).max()) / np.float32(qm))
            else:
                rs = s
            y = np.abs(xv[t, h]) / rs
            # half the gap to the neighbouring code around y, plus the fp32 rounding of
            # 1/s and x * (1/s) (a few ulps of y)
            idx = np.clip(np.searchsorted(fin, y), 1, len(fin) - 1)
            gap = fin[idx] - fin[idx - 1]
            assert np.all(np.abs(row - xv[t, h]) <= (0.5 * gap + y * 2.0 ** -21) * rs)


@pytest.mark.parametrize("fmt", FMTS)
def test_zero_row_per_token_head(fmt):
    d = _desc(fmt, oracle.MODE_PER_TOKEN_HEAD)
    z = np.zeros((1, 2, 64), dtype=np.uint16)
    cache = np.full(d.total_bytes, 0xAB, dtype=np.uint8)
    oracle.cache_write(d, cache, z, z, np.array([5], dtype=np.int64))
    for kv in range(2):
        for h in range(2):
            page = d.page_offset(0, kv, h)
            assert np.all(cache[page + 5 * 64: page + 6 * 64] == 0)
            assert cache[page + 16 * 64 + 20: page + 16 * 64 + 24].view(np.float32)[0] == 0.0


def test_negative_slots_skipped_and_writes_disjoint():
    rng = np.random.default_rng(41)
    for mode in (oracle.MODE_PER_TENSOR, oracle.MODE_PER_TOKEN_HEAD):
        d = _desc(oracle.FMT_E4M3, mode, nb=4)
        n = 50
        kb = rng.integers(0x3F00, 0x4000, size=(n, 2, 64)).astype(np.uint16)  # all |x| in [0.5, 2): no zero codes
        slots = rng.permutation(d.num_blocks * d.block_size)[:n].astype(np.int64)
        slots[::7] = -1
        # a byte counts as written if it differs from the fill in a 0x00-filled or a 0xFF-filled run
        changed = np.zeros(d.total_bytes, dtype=bool)
        for fill in (0x00, 0xFF):
            cache = np.full(d.total_bytes, fill, dtype=np.uint8)
            oracle.cache_write(d, cache, kb, kb, slots, 0.01, 0.01)
            changed |= cache != fill
        live = int((slots >= 0).sum())
        per_tok = 2 * 2 * 64 + (2 * 2 * 4 if mode == oracle.MODE_PER_TOKEN_HEAD else 0)
        assert int(changed.sum()) == live * per_tok


def test_slot_outside_pool_is_an_error():
    d = _desc(oracle.FMT_E4M3, oracle.MODE_PER_TENSOR, nb=2)
    kb = np.zeros((1, 2, 64), dtype=np.uint16)
    with pytest.raises(ValueError):
        oracle.cache_write(d, np.zeros(d.total_bytes, np.uint8), kb, kb, np.array([32], dtype=np.int64))


def test_layout_pages_disjoint_and_aligned():
    for mode in (0, 1):
        for bs, d_, h in [(16, 64, 2), (2176, 256, 2), (16, 128, 8), (32, 128, 3)]:
            d = oracle.CacheDesc(3, bs, h, d_, oracle.FMT_E4M3, mode)
            pb = d.page_bytes
            assert pb % 128 == 0 and pb >= bs * d_ + (4 * bs if mode else 0)
            offs = sorted(d.page_offset(b, kv, hh) for b in range(3) for kv in range(2) for hh in range(h))
            assert np.all(np.diff(offs) == pb) and offs[0] == 0 and offs[-1] + pb == d.total_bytes
