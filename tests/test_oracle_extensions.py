"""Pins of the oracle's per-sequence causal flag, ALiBi slopes and attention sinks (the varlen
harness parameters dynamic_causal, use_alibi and use_sink that the "Fix CPU FP8 attention
scheduler scratch sizing" page names in its Code excerpt), against things other than the oracle:

* ALiBi: torch's scaled_dot_product_attention in fp64 with an additive float mask
  slope_h * (j - p) (and -inf above the causal diagonal) on lossless caches;
* sinks: the same routine with one extra key of zeros whose mask entry is the sink logit and
  whose value row is zero (a sink is a logit with no value); a closed form at q = 0;
* zero slopes and -inf sinks change nothing; per-sequence causal flags equal separate runs with
  the matching global flag.
"""
import numpy as np
import torch

import oracle
from tests.test_oracle_attention import Case
from workloads import bf16_to_f32


def _sdpa_masked(q, k, v, g, mask):
    """q [T, Hq, D], k/v [L, Hkv, D], mask [Hq, T, L] additive (fp64) -> [T, Hq, D]."""
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]
    kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(g, dim=0)[None]
    vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(g, dim=0)[None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(mask)[None])
    return o[0].permute(1, 0, 2).numpy()


def _bias(ql, L, slopes, causal=True):
    p = L - ql + np.arange(ql)
    j = np.arange(L)
    rel = (j[None, :] - p[:, None]).astype(np.float64)            # [T, L]
    m = slopes[:, None, None] * rel[None]                          # [Hq, T, L]
    if causal:
        m = np.where(j[None, None, :] > p[None, :, None], -np.inf, m)
    return m


def test_alibi_matches_sdpa_with_additive_bias():
    hq, hkv, d = 8, 2, 64
    slopes = 2.0 ** (-8.0 * np.arange(1, hq + 1) / hq)             # the usual geometric slopes
    c = Case(((1, 70), (23, 23), (9, 40)), hq, hkv, d, seed=11)
    got = c.run(want_f64=True, alibi_slopes=slopes)[1]
    for b, (ql, L) in enumerate(c.seqs):
        k, v = c.kv_of(b)
        qf = bf16_to_f32(c.q[c.qsl[b]:c.qsl[b + 1]]).astype(np.float64)
        ref = _sdpa_masked(qf, k, v, hq // hkv, _bias(ql, L, slopes))
        np.testing.assert_allclose(got[c.qsl[b]:c.qsl[b + 1]], ref, rtol=1e-9, atol=1e-12)


def test_sinks_match_sdpa_with_a_zero_value_key():
    hq, hkv, d = 4, 2, 64
    sinks = np.array([-1.0, 0.5, 3.0, 8.0])
    slopes = np.array([0.0, 0.25, 0.0, 0.0625])
    c = Case(((1, 33), (17, 17), (4, 50)), hq, hkv, d, seed=12)
    got = c.run(want_f64=True, alibi_slopes=slopes, sinks=sinks)[1]
    for b, (ql, L) in enumerate(c.seqs):
        k, v = c.kv_of(b)
        k1 = np.concatenate([k, np.zeros((1,) + k.shape[1:])])
        v1 = np.concatenate([v, np.zeros((1,) + v.shape[1:])])
        mask = np.concatenate([_bias(ql, L, slopes), np.broadcast_to(sinks[:, None, None], (hq, ql, 1))], axis=2)
        qf = bf16_to_f32(c.q[c.qsl[b]:c.qsl[b + 1]]).astype(np.float64)
        ref = _sdpa_masked(qf, k1, v1, hq // hkv, mask)
        np.testing.assert_allclose(got[c.qsl[b]:c.qsl[b + 1]], ref, rtol=1e-9, atol=1e-12)


def test_sink_closed_form_at_zero_query():
    """q = 0: every visible logit is 0, so each of the n keys weighs 1 / (n + e^s)."""
    hq, hkv, d = 2, 1, 64
    c = Case(((5, 12),), hq, hkv, d, seed=13, qb=np.zeros((5, hq, d), dtype=np.uint16))
    for s in (-2.0, 0.0, 1.5):
        for i in range(5):
            w = oracle.attention_weights(c.desc, c.cache, c.q, c.bt, c.seq_lens, c.qsl, hq, 0, i, 1,
                                         k_scale=c.s, v_scale=2 * c.s, sink=s)
            n = 12 - 5 + i + 1
            np.testing.assert_allclose(w[:n], 1.0 / (n + np.exp(s)), rtol=1e-14)
            assert np.all(w[n:] == 0.0)


def test_neutral_values_change_nothing():
    hq, hkv, d = 8, 4, 128
    c = Case(((1, 90), (12, 30)), hq, hkv, d, seed=14, fmt=oracle.FMT_INT8, mode=oracle.MODE_PER_TOKEN_HEAD)
    base = c.run(softcap=9.0, window=17)
    ext = c.run(softcap=9.0, window=17, alibi_slopes=np.zeros(hq), sinks=np.full(hq, -np.inf),
                causal_per_seq=np.ones(2, np.int32))
    assert np.array_equal(base, ext)


def test_per_sequence_causal_equals_separate_runs():
    hq, hkv, d = 4, 2, 64
    c = Case(((9, 9), (6, 20), (1, 7), (5, 5)), hq, hkv, d, seed=15)
    flags = np.array([1, 0, 1, 0], np.int32)
    mixed = c.run(causal_per_seq=flags)
    causal, full = c.run(causal=True), c.run(causal=False)
    for b in range(4):
        rows = slice(c.qsl[b], c.qsl[b + 1])
        assert np.array_equal(mixed[rows], (causal if flags[b] else full)[rows])
    # a non-causal sequence with a window is refused
    try:
        c.run(causal_per_seq=flags, window=3)
    except ValueError:
        pass
    else:
        raise AssertionError("window with a non-causal sequence accepted")
