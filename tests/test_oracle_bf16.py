"""Pins of the oracle's unquantised ("auto") bf16 cache: stored bytes are the inputs' bits at the
positions the page layout defines (recomputed here from the layout's definition), and attention
over such a cache equals torch's scaled_dot_product_attention in fp64 on the same bf16 values
(decode, causal prefill and a chunk with a window of keys)."""
import numpy as np
import torch

import oracle
from tests.oracle_helpers import contiguous_tables, slots_for
from workloads import bf16_round, bf16_to_f32


def _layout_offset(bs, d, h, block, kv, head):
    page = (bs * d * 2 + 127) // 128 * 128
    return block * 2 * h * page + (kv * h + head) * page


def test_bf16_cache_stores_the_input_bits():
    rng = np.random.default_rng(3)
    nb, bs, h, d, n = 6, 16, 3, 64, 70
    desc = oracle.CacheDesc(nb, bs, h, d, oracle.FMT_BF16, oracle.MODE_PER_TENSOR)
    k = bf16_round((rng.standard_normal((n, h, d)) * 3).astype(np.float32))
    v = bf16_round((rng.standard_normal((n, h, d)) * 3).astype(np.float32))
    slots = rng.permutation(nb * bs)[:n].astype(np.int64)
    slots[::7] = -1
    cache = np.full(desc.total_bytes, 0x5A, np.uint8)
    oracle.cache_write(desc, cache, k, v, slots)
    assert desc.total_bytes == nb * 2 * h * ((bs * d * 2 + 127) // 128 * 128)
    written = np.zeros(desc.total_bytes, bool)
    for t in range(n):
        if slots[t] < 0:
            continue
        blk, off = divmod(int(slots[t]), bs)
        for kv, x in ((0, k), (1, v)):
            for hh in range(h):
                o = _layout_offset(bs, d, h, blk, kv, hh) + off * d * 2
                assert np.array_equal(cache[o:o + 2 * d].view(np.uint16), x[t, hh])
                written[o:o + 2 * d] = True
    assert np.all(cache[~written] == 0x5A)


def _sdpa(q, k, v, g, causal, window=0):
    T, L = q.shape[0], k.shape[0]
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]
    kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(g, dim=0)[None]
    vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(g, dim=0)[None]
    p = L - T + np.arange(T)
    j = np.arange(L)
    ok = np.ones((T, L), bool)
    if causal:
        ok &= j[None, :] <= p[:, None]
    if window:
        ok &= p[:, None] - j[None, :] < window
    mask = torch.from_numpy(np.where(ok, 0.0, -np.inf))
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask[None, None])
    return o[0].permute(1, 0, 2).numpy()


def test_bf16_cache_attention_matches_sdpa():
    rng = np.random.default_rng(4)
    hq, hkv, d, bs = 8, 2, 128, 16
    seqs = ((1, 300), (40, 40), (9, 77))
    for window in (0, 23):
        sl = np.array([L for _, L in seqs], np.int32)
        qsl = np.concatenate([[0], np.cumsum([q for q, _ in seqs])]).astype(np.int32)
        bt, used = contiguous_tables(sl, bs)
        perm = rng.permutation(used + 2).astype(np.int32)
        bt = np.where(bt >= 0, perm[np.maximum(bt, 0)], -1).astype(np.int32)
        desc = oracle.CacheDesc(used + 2, bs, hkv, d, oracle.FMT_BF16, oracle.MODE_PER_TENSOR)
        n = int(sl.sum())
        k = bf16_round(rng.standard_normal((n, hkv, d)).astype(np.float32))
        v = bf16_round(rng.standard_normal((n, hkv, d)).astype(np.float32))
        q = bf16_round(rng.standard_normal((int(qsl[-1]), hq, d)).astype(np.float32))
        cache = np.zeros(desc.total_bytes, np.uint8)
        oracle.cache_write(desc, cache, k, v, slots_for(bt, sl, bs))
        _, o64 = oracle.attention(desc, cache, q, bt, sl, qsl, hq, window=window, want_f64=True)
        off = 0
        for b, (ql, L) in enumerate(seqs):
            kf = bf16_to_f32(k[off:off + L]).astype(np.float64)
            vf = bf16_to_f32(v[off:off + L]).astype(np.float64)
            qf = bf16_to_f32(q[qsl[b]:qsl[b + 1]]).astype(np.float64)
            ref = _sdpa(qf, kf, vf, hq // hkv, True, window)
            np.testing.assert_allclose(o64[qsl[b]:qsl[b + 1]], ref, rtol=1e-10, atol=1e-12)
            off += L
