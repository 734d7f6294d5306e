"""Pins of the oracle's attention against things other than itself.

* lossless caches (K, V = code value * power-of-two scale) against torch's
  scaled_dot_product_attention in fp64 on the CPU (a library routine), with the
  GQA expansion head -> head // (Hq / Hkv), for decode (one query over all keys),
  full causal prefill and non-causal prefill;
* softmax rows sum to one;
* a prefill chunk equals the matching rows of the full prefill (bottom-right
  causal alignment of the (query_len, kv_len) harness tuples);
* window W = 1 keeps only the query's own key, W >= L equals no window, W = 2
  keeps exactly two keys;
* constant V gives that constant, q = 0 gives the mean of the visible values;
* soft-cap: an infinite cap equals no cap, and a two-key closed form;
* paged equals contiguous, and permuting the physical blocks changes nothing.
"""
import numpy as np
import pytest
import torch

import oracle
from tests.oracle_helpers import contiguous_tables, lossless_kv, slots_for, to_bf16_bits
from workloads import bf16_round, bf16_to_f32


class Case:
    def __init__(self, seqs, hq, hkv, d, bs=16, fmt=oracle.FMT_E4M3, mode=oracle.MODE_PER_TENSOR, seed=0,
                 scale_exp=-3, permute=True, kx=None, vx=None, qb=None, extra_blocks=3):
        self.rng = rng = np.random.default_rng(seed)
        self.seqs = seqs
        self.hq, self.hkv, self.d, self.bs = hq, hkv, d, bs
        self.seq_lens = np.array([L for _, L in seqs], dtype=np.int32)
        self.qsl = np.concatenate([[0], np.cumsum([q for q, _ in seqs])]).astype(np.int32)
        bt, used = contiguous_tables(self.seq_lens, bs)
        nb = used + extra_blocks
        if permute:
            perm = rng.permutation(nb).astype(np.int32)
            bt = np.where(bt >= 0, perm[np.maximum(bt, 0)], -1).astype(np.int32)
        self.bt = bt
        self.desc = oracle.CacheDesc(nb, bs, hkv, d, fmt, mode)
        n = int(self.seq_lens.sum())
        s = 2.0 ** scale_exp
        self.s = s
        pth = mode == oracle.MODE_PER_TOKEN_HEAD
        if kx is None:
            self.kb, self.kx = lossless_kv(rng, fmt, n, hkv, d, s, per_token_head=pth)
        else:
            self.kx = kx
            self.kb = to_bf16_bits(kx)
        if vx is None:
            self.vb, self.vx = lossless_kv(rng, fmt, n, hkv, d, s * 2, per_token_head=pth)
        else:
            self.vx = vx
            self.vb = to_bf16_bits(vx)
        self.q = qb if qb is not None else bf16_round(rng.standard_normal((int(self.qsl[-1]), hq, d)).astype(np.float32))
        self.cache = np.zeros(self.desc.total_bytes, dtype=np.uint8)
        oracle.cache_write(self.desc, self.cache, self.kb, self.vb, slots_for(self.bt, self.seq_lens, bs), s, 2 * s)

    def run(self, **kw):
        return oracle.attention(self.desc, self.cache, self.q, self.bt, self.seq_lens, self.qsl, self.hq,
                                k_scale=self.s, v_scale=2 * self.s, **kw)

    def kv_of(self, b):
        o = int(self.seq_lens[:b].sum())
        L = int(self.seq_lens[b])
        return self.kx[o:o + L], self.vx[o:o + L]


def _sdpa(q, k, v, g, causal):
    """q [T, Hq, D], k/v [L, Hkv, D] fp64 -> [T, Hq, D]."""
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]
    kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(g, dim=0)[None]
    vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(g, dim=0)[None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=causal)
    return o[0].permute(1, 0, 2).numpy()


CODECS = [(oracle.FMT_E4M3, oracle.MODE_PER_TENSOR), (oracle.FMT_E5M2, oracle.MODE_PER_TENSOR),
          (oracle.FMT_INT8, oracle.MODE_PER_TOKEN_HEAD), (oracle.FMT_E4M3, oracle.MODE_PER_TOKEN_HEAD)]


@pytest.mark.parametrize("fmt,mode", CODECS)
@pytest.mark.parametrize("hq,hkv,d", [(4, 4, 64), (8, 2, 64), (8, 1, 128)])
def test_decode_and_prefill_match_sdpa_fp64(fmt, mode, hq, hkv, d):
    seqs = [(1, 37), (1, 5), (29, 29), (16, 16)]
    c = Case(seqs, hq, hkv, d, fmt=fmt, mode=mode, seed=hq * 7 + d + fmt)
    out, o64 = c.run(want_f64=True)
    qf = bf16_to_f32(c.q).astype(np.float64)
    for b, (ql, L) in enumerate(seqs):
        k, v = c.kv_of(b)
        qs = qf[c.qsl[b]:c.qsl[b + 1]]
        ref = _sdpa(qs, k, v, hq // hkv, causal=(ql == L))
        np.testing.assert_allclose(o64[c.qsl[b]:c.qsl[b + 1]], ref, rtol=1e-10, atol=1e-12)


def test_non_causal_prefill_matches_sdpa():
    seqs = [(23, 23)]
    c = Case(seqs, 4, 2, 64, seed=3)
    _, o64 = c.run(causal=False, want_f64=True)
    k, v = c.kv_of(0)
    ref = _sdpa(bf16_to_f32(c.q).astype(np.float64), k, v, 2, causal=False)
    np.testing.assert_allclose(o64, ref, rtol=1e-10, atol=1e-12)


def test_softmax_rows_sum_to_one():
    c = Case([(5, 40), (1, 17)], 4, 2, 64, seed=4)
    for b, i, hq, kw in [(0, 0, 0, {}), (0, 4, 3, {}), (1, 0, 1, {}), (0, 2, 2, {"window": 7}),
                         (0, 1, 1, {"softcap": 2.0})]:
        w = oracle.attention_weights(c.desc, c.cache, c.q, c.bt, c.seq_lens, c.qsl, c.hq, b, i, hq,
                                     k_scale=c.s, v_scale=2 * c.s, **kw)
        assert abs(w.sum() - 1.0) < 1e-12
        assert np.all(w >= 0)
        p = int(c.seq_lens[b]) - (int(c.qsl[b + 1]) - int(c.qsl[b])) + i
        assert np.all(w[p + 1:] == 0)  # causal: nothing after the query's own position


@pytest.mark.parametrize("window", [0, 9])
def test_chunk_equals_rows_of_full_prefill(window):
    L, ch = 45, 13
    full = Case([(L, L)], 4, 2, 64, seed=5)
    chunk = Case([(ch, L)], 4, 2, 64, seed=5, kx=full.kx, vx=full.vx, qb=np.ascontiguousarray(full.q[L - ch:]))
    a = full.run(window=window)
    b = chunk.run(window=window)
    assert np.array_equal(a[L - ch:], b)


@pytest.mark.parametrize("window,softcap", [(0, 0.0), (9, 0.0), (0, 3.0)])
def test_row_equals_one_query_sequence_ending_at_its_position(window, softcap):
    """Under the causal mask a query row at position p sees the keys of a one-query sequence of
    p + 1 keys over the same block table: the full-size GPU tests recompute sampled prefill rows
    that way, so the two must agree bit for bit."""
    c = Case([(30, 30), (1, 23), (12, 50)], 8, 2, 64, seed=12)
    full = c.run(window=window, softcap=softcap)
    picks = [(0, 0), (0, 17), (0, 29), (1, 0), (2, 0), (2, 5), (2, 11)]
    seqs = [b for b, _ in picks]
    pos1 = np.array([int(c.seq_lens[b] - (c.qsl[b + 1] - c.qsl[b]) + i + 1) for b, i in picks], np.int32)
    rows = np.array([int(c.qsl[b] + i) for b, i in picks])
    one = oracle.attention(c.desc, c.cache, np.ascontiguousarray(c.q[rows]), c.bt[seqs], pos1,
                           np.arange(len(picks) + 1, dtype=np.int32), c.hq, window=window, softcap=softcap,
                           k_scale=c.s, v_scale=2 * c.s)
    assert np.array_equal(one, full[rows])


def test_window_edges():
    c = Case([(6, 30), (1, 12)], 4, 2, 64, seed=6)
    base = c.run()
    assert np.array_equal(c.run(window=30), base)
    assert np.array_equal(c.run(window=10_000), base)
    # W = 1: only the query's own key is visible -> output = its value row
    out = c.run(window=1)
    for b, (ql, L) in enumerate(c.seqs):
        _, v = c.kv_of(b)
        for i in range(ql):
            p = L - ql + i
            for hq in range(4):
                assert np.array_equal(bf16_to_f32(out[c.qsl[b] + i, hq]).astype(np.float64), v[p, hq // 2])
    # W = 2: exactly keys p-1 and p
    w = oracle.attention_weights(c.desc, c.cache, c.q, c.bt, c.seq_lens, c.qsl, 4, 0, 3, 1, window=2,
                                 k_scale=c.s, v_scale=2 * c.s)
    p = 30 - 6 + 3
    assert set(np.nonzero(w)[0]) == {p - 1, p}


def test_constant_v_and_zero_q():
    seqs = [(1, 33), (7, 20)]
    n = 53
    vx = np.full((n, 2, 64), 0.75)
    c = Case(seqs, 4, 2, 64, seed=7, vx=vx)
    out = c.run()
    assert np.all(bf16_to_f32(out) == np.float32(0.75))
    qz = np.zeros_like(c.q)
    cz = Case(seqs, 4, 2, 64, seed=8, qb=qz)
    _, o64 = cz.run(want_f64=True)
    for b, (ql, L) in enumerate(seqs):
        _, v = cz.kv_of(b)
        for i in range(ql):
            p = L - ql + i
            for hq in range(4):
                np.testing.assert_allclose(o64[cz.qsl[b] + i, hq], v[: p + 1, hq // 2].mean(axis=0), rtol=1e-12,
                                           atol=1e-14)


def test_softcap_limits_and_two_key_closed_form():
    c = Case([(3, 21), (1, 9)], 4, 2, 64, seed=9)
    _, a = c.run(want_f64=True)
    _, b = c.run(softcap=1e30, want_f64=True)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-15)
    # two keys along one axis: z_j = a * b_j / sqrt(D); weights follow softmax(cap * tanh(z / cap))
    d = 64
    kx = np.zeros((2, 1, d)); kx[0, 0, 0] = 4.0; kx[1, 0, 0] = -2.0
    vx = np.zeros((2, 1, d)); vx[0, 0, :] = 1.0; vx[1, 0, :] = -1.0
    qf = np.zeros((1, 1, d), dtype=np.float32); qf[0, 0, 0] = 6.0
    c2 = Case([(1, 2)], 1, 1, d, seed=10, kx=kx, vx=vx, qb=bf16_round(qf), scale_exp=0, permute=False)
    for cap in (0.0, 5.0, 1.5):
        _, o = c2.run(softcap=cap, want_f64=True)
        z = np.array([6.0 * 4.0, 6.0 * -2.0]) / np.sqrt(d)
        if cap > 0:
            z = cap * np.tanh(z / cap)
        w = np.exp(z - z.max()); w /= w.sum()
        np.testing.assert_allclose(o[0, 0], np.full(d, w[0] - w[1]), rtol=1e-12)


def test_paged_equals_contiguous_and_permutation_invariance():
    seqs = [(1, 50), (9, 40), (1, 16)]
    a = Case(seqs, 8, 2, 64, seed=11, permute=False)
    b = Case(seqs, 8, 2, 64, seed=11, permute=True, kx=a.kx, vx=a.vx, qb=a.q)
    c = Case(seqs, 8, 2, 64, seed=12, permute=True, kx=a.kx, vx=a.vx, qb=a.q, extra_blocks=9)
    ra = a.run(window=20, softcap=3.0)
    assert np.array_equal(ra, b.run(window=20, softcap=3.0))
    assert np.array_equal(ra, c.run(window=20, softcap=3.0))


def test_invalid_arguments_rejected():
    c = Case([(1, 10)], 4, 2, 64, seed=13)
    with pytest.raises(ValueError):
        oracle.attention(c.desc, c.cache, c.q, c.bt, c.seq_lens, c.qsl, 3)  # Hq not a multiple of Hkv
    with pytest.raises(ValueError):
        oracle.attention(c.desc, c.cache, c.q, c.bt, c.seq_lens, c.qsl, 4, causal=False, window=4)


def test_absent_blocks_match_sdpa_with_masked_keys():
    """A block-table entry outside the pool (negative, or >= num_blocks) names no block: the keys of
    that logical block take no part in the softmax. Pinned against fp64 SDPA whose additive mask is
    -inf on exactly those keys (on top of the causal mask); a row left with no key at all gives 0."""
    seqs = [(1, 50), (9, 40), (20, 20), (1, 10)]
    c = Case(seqs, 8, 2, 64, seed=21)
    nb = c.desc.num_blocks
    bt = c.bt.copy()
    bt[0, 1] = -1          # keys 16..31 of the first decode
    bt[1, 0] = nb + 7      # keys 0..15 of the chunk (its first queries see nothing else but later keys)
    bt[2, 1] = nb          # the prefill's keys 16..19
    bt[3, 0] = -5          # the last decode has no key left
    _, o64 = oracle.attention(c.desc, c.cache, c.q, bt, c.seq_lens, c.qsl, c.hq, k_scale=c.s, v_scale=2 * c.s,
                              want_f64=True)
    qf = bf16_to_f32(c.q).astype(np.float64)
    g = c.hq // c.hkv
    for b, (ql, L) in enumerate(seqs):
        k, v = c.kv_of(b)
        absent = np.array([not (0 <= bt[b, j // c.bs] < nb) for j in range(L)])
        pos = L - ql + np.arange(ql)
        mask = np.where((np.arange(L)[None, :] <= pos[:, None]) & ~absent[None, :], 0.0, -np.inf)
        qt = torch.from_numpy(qf[c.qsl[b]:c.qsl[b + 1]]).permute(1, 0, 2)[None]
        kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(g, dim=0)[None]
        vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(g, dim=0)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(mask))
        ref = ref[0].permute(1, 0, 2).numpy()
        empty = np.all(np.isinf(mask), axis=1)
        ref[empty] = 0.0  # SDPA leaves NaN where a row has no key; the reading gives 0
        np.testing.assert_allclose(o64[c.qsl[b]:c.qsl[b + 1]], ref, rtol=1e-10, atol=1e-12)
    assert np.all(o64[c.qsl[3]] == 0.0)
    # with the table intact the first decode's row differs: the entry is not ignored
    full = c.run(want_f64=True)[1]
    assert not np.allclose(full[c.qsl[0]], o64[c.qsl[0]])


def test_absent_block_with_sink_gives_zero_and_keeps_weights_finite():
    c = Case([(1, 10)], 4, 2, 64, seed=22)
    bt = c.bt.copy()
    bt[0, 0] = -1
    out = oracle.attention(c.desc, c.cache, c.q, bt, c.seq_lens, c.qsl, c.hq, k_scale=c.s, v_scale=2 * c.s,
                           sinks=np.full(c.hq, 0.5))
    assert np.all(out == 0)
    w = oracle.attention_weights(c.desc, c.cache, c.q, bt, c.seq_lens, c.qsl, c.hq, 0, 0, 1, k_scale=c.s,
                                 v_scale=2 * c.s)
    assert np.all(w == 0)
