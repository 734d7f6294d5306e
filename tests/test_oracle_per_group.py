"""Pins of the oracle's per-group scale mode: one dynamic scale per (token, KV head, run of 32
consecutive head-dim channels), absmax / qmax, stored in the page tail as [row][group] fp32.

- A worked example whose scales are exact powers of two and whose scaled values are exactly
  representable codes: the stored bytes follow from the OCP format definition (torch's float8
  types encode the exact values here) and the scales are known in closed form.
- Rows whose groups all reach the row's absmax give byte-identical codes to per-token-head mode
  and replicate its scale.
- The lossless special case (each group built as code x its own power-of-two scale) makes
  quantisation the identity, so attention equals fp64 SDPA on the inputs.
- Dequantisation error stays within half a code step of each group's own scale, a bound the
  coarser per-token-head scale does not meet on rows with small groups."""
import numpy as np
import pytest
import torch

import oracle
from tests.oracle_helpers import code_values, contiguous_tables, random_codes, slots_for, to_bf16_bits
from workloads import bf16_to_f32

QMAX = {oracle.FMT_E4M3: 448.0, oracle.FMT_E5M2: 57344.0, oracle.FMT_INT8: 127.0}
G = oracle.GROUP


def page_of(desc, block, kv, head):
    return block * desc.block_bytes + (kv * desc.num_kv_heads + head) * desc.page_bytes


def encode_exact(fmt, vals):
    """Codes of exactly representable values (torch's float8 / int8 conversion, exact here)."""
    t = torch.from_numpy(np.asarray(vals, dtype=np.float64))
    if fmt == oracle.FMT_INT8:
        assert np.all(np.round(vals) == vals)
        return t.to(torch.int8).numpy().view(np.uint8)
    f8 = {oracle.FMT_E4M3: torch.float8_e4m3fn, oracle.FMT_E5M2: torch.float8_e5m2}[fmt]
    c = t.to(f8)
    assert torch.equal(c.to(torch.float64), t)
    return c.view(torch.uint8).numpy()


@pytest.mark.parametrize("fmt", [oracle.FMT_E4M3, oracle.FMT_E5M2, oracle.FMT_INT8])
def test_worked_example_bytes_and_scales(fmt):
    D, bs = 64, 16
    qm = QMAX[fmt]
    desc = oracle.CacheDesc(2, bs, 1, D, fmt, oracle.MODE_PER_GROUP)
    assert desc.page_bytes == -(-(bs * D + 4 * bs * (D // G)) // 128) * 128
    # group 0 at scale 2^-3, group 1 at scale 2^-7; each group holds +-qmax once
    small = {oracle.FMT_INT8: [0.0, 1.0, -5.0, 64.0], oracle.FMT_E4M3: [0.0, 1.5, -0.25, 96.0],
             oracle.FMT_E5M2: [0.0, 1.5, -0.25, 3072.0]}[fmt]
    vals = np.zeros(D)
    vals[:4] = small
    vals[5] = qm
    vals[G:G + 4] = small[::-1]
    vals[G + 9] = -qm
    scale = np.array([2.0 ** -3] * G + [2.0 ** -7] * G)
    x = vals * scale
    kb = to_bf16_bits(x)[None, None, :]
    cache = np.zeros(desc.total_bytes, dtype=np.uint8)
    oracle.cache_write(desc, cache, kb, kb, np.array([bs + 3], np.int64))  # block 1, row 3
    for kv in (0, 1):
        page = page_of(desc, 1, kv, 0)
        codes = cache[page + 3 * D: page + 4 * D]
        assert np.array_equal(codes, encode_exact(fmt, vals))
        sc = cache[page + bs * D: page + bs * D + 4 * bs * (D // G)].view(np.float32).reshape(bs, D // G)
        assert sc[3, 0] == np.float32(2.0 ** -3) and sc[3, 1] == np.float32(2.0 ** -7)
        assert np.all(np.delete(sc, 3, axis=0) == 0)
        np.testing.assert_array_equal(oracle.read_row(desc, cache, kv, 1, 0, 3), x)


@pytest.mark.parametrize("fmt", [oracle.FMT_E4M3, oracle.FMT_INT8])
def test_groups_sharing_the_row_absmax_match_per_token_head(fmt):
    rng = np.random.default_rng(3)
    D, bs, n, H = 128, 16, 40, 2
    x = rng.standard_normal((n, H, D)).astype(np.float32)
    amax = np.abs(x).max(axis=2, keepdims=True)
    for g in range(D // G):  # every group reaches the row's absmax
        x[:, :, g * G] = amax[..., 0] * np.where(rng.random((n, H)) < 0.5, -1, 1)
    xb = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    slots = rng.permutation(4 * bs)[:n].astype(np.int64)
    dg = oracle.CacheDesc(4, bs, H, D, fmt, oracle.MODE_PER_GROUP)
    dt = oracle.CacheDesc(4, bs, H, D, fmt, oracle.MODE_PER_TOKEN_HEAD)
    cg = np.zeros(dg.total_bytes, np.uint8)
    ct = np.zeros(dt.total_bytes, np.uint8)
    oracle.cache_write(dg, cg, xb, xb, slots)
    oracle.cache_write(dt, ct, xb, xb, slots)
    for t in range(n):
        b, off = int(slots[t] // bs), int(slots[t] % bs)
        for kv in (0, 1):
            for h in range(H):
                pg, pt = page_of(dg, b, kv, h), page_of(dt, b, kv, h)
                assert np.array_equal(cg[pg + off * D: pg + (off + 1) * D], ct[pt + off * D: pt + (off + 1) * D])
                sg = cg[pg + bs * D + 16 * off: pg + bs * D + 16 * (off + 1)].view(np.float32)
                st = ct[pt + bs * D + 4 * off: pt + bs * D + 4 * (off + 1)].view(np.float32)
                assert np.all(sg == st[0])


def _sdpa(q, k, v, g):
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]
    kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(g, dim=0)[None]
    vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(g, dim=0)[None]
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)[0].permute(1, 0, 2).numpy()


def lossless_group_kv(rng, fmt, n, hkv, d):
    """x = value(code) * 2^e with e drawn per (token, head, group) and one +-qmax per group,
    so the dynamic group scale is exactly 2^e and quantisation is the identity."""
    qm = QMAX[fmt]
    vals = code_values(fmt, random_codes(rng, fmt, (n, hkv, d), max_mag=qm)).reshape(n, hkv, d // G, G)
    pos = rng.integers(0, G, size=(n, hkv, d // G))
    sign = np.where(rng.random((n, hkv, d // G)) < 0.5, -1.0, 1.0)
    np.put_along_axis(vals, pos[..., None], (sign * qm)[..., None], axis=3)
    e = rng.integers(-9, -2, size=(n, hkv, d // G, 1)).astype(np.float64)
    x = (vals * 2.0 ** e).reshape(n, hkv, d)
    return to_bf16_bits(x), x


@pytest.mark.parametrize("fmt", [oracle.FMT_E4M3, oracle.FMT_E5M2, oracle.FMT_INT8])
@pytest.mark.parametrize("hq,hkv,d", [(8, 2, 64), (4, 1, 128), (4, 2, 256)])
def test_lossless_attention_matches_sdpa_fp64(fmt, hq, hkv, d):
    rng = np.random.default_rng(11)
    bs, L, ql = 16, 70, 9
    seq_lens = np.array([L], np.int32)
    qsl = np.array([0, ql], np.int32)
    bt, used = contiguous_tables(seq_lens, bs)
    bt = rng.permutation(used + 2).astype(np.int32)[bt]
    desc = oracle.CacheDesc(used + 2, bs, hkv, d, fmt, oracle.MODE_PER_GROUP)
    kb, kx = lossless_group_kv(rng, fmt, L, hkv, d)
    vb, vx = lossless_group_kv(rng, fmt, L, hkv, d)
    cache = np.zeros(desc.total_bytes, np.uint8)
    oracle.cache_write(desc, cache, kb, vb, slots_for(bt, seq_lens, bs), 123.0, 456.0)  # scales ignored
    q = to_bf16_bits(np.round(rng.standard_normal((ql, hq, d)) * 8) / 8)
    _, o64 = oracle.attention(desc, cache, q, bt, seq_lens, qsl, hq, want_f64=True)
    # query i sits at position L - ql + i: causal SDPA over the last ql rows of a full prefill
    qfull = np.zeros((L, hq, d))
    qfull[L - ql:] = bf16_to_f32(q)
    ref = _sdpa(qfull, kx, vx, hq // hkv)[L - ql:]
    np.testing.assert_allclose(o64, ref, rtol=1e-10, atol=1e-12)


def test_error_bound_per_group_beats_per_token_head():
    """int8: |dequant - x| <= s_g / 2 per group (round to nearest, up to the fp32 roundings of
    the scaling); on rows whose first group is 256x larger than the others the per-token-head
    error of the small groups is far above it."""
    rng = np.random.default_rng(5)
    D, bs, n = 128, 16, 32
    x = rng.standard_normal((n, 1, D)).astype(np.float32)
    x[:, :, :G] *= 256.0
    xb = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    xf = bf16_to_f32(xb).astype(np.float64)
    slots = np.arange(n, dtype=np.int64)
    errs = {}
    for mode in (oracle.MODE_PER_GROUP, oracle.MODE_PER_TOKEN_HEAD):
        desc = oracle.CacheDesc(2, bs, 1, D, oracle.FMT_INT8, mode)
        c = np.zeros(desc.total_bytes, np.uint8)
        oracle.cache_write(desc, c, xb, xb, slots)
        deq = np.stack([oracle.read_row(desc, c, 0, int(s // bs), 0, int(s % bs)) for s in slots])
        errs[mode] = np.abs(deq - xf[:, 0])
    sg = np.abs(xf[:, 0].reshape(n, D // G, G)).max(axis=2).astype(np.float32) / np.float32(127.0)
    # half a code step, plus the fp32 roundings of 1/s and x * (1/s) (|x/s| <= 127, two ulps)
    bound = np.repeat(sg.astype(np.float64), G, axis=1) * (0.5 + 127.0 * 2.0 ** -22)
    assert np.all(errs[oracle.MODE_PER_GROUP] <= bound)
    assert errs[oracle.MODE_PER_TOKEN_HEAD][:, G:].max() > 20 * errs[oracle.MODE_PER_GROUP][:, G:].max()


def test_unquantised_cache_has_no_group_scales():
    desc = oracle.CacheDesc(1, 16, 1, 64, oracle.FMT_BF16, oracle.MODE_PER_GROUP)
    kb = np.zeros((1, 1, 64), np.uint16)
    with pytest.raises(ValueError):
        oracle.cache_write(desc, np.zeros(desc.total_bytes, np.uint8), kb, kb, np.array([0], np.int64))
