"""Host-side checks of the C ABI (no GPU): exported symbols, dtype parsing,
layout sizes against the oracle's independent layout, and error paths that
must fail before anything is launched."""
import ctypes
import os
import re

import numpy as np
import pytest

import attention_quantized_paged_amd as aqp
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")


def _declared_symbols():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            src = open(os.path.join(ROOT, "include", fn)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names |= set(re.findall(r"\b(aqp_[a-z_0-9]+)\s*\(", src))
    return names


def test_library_exports_every_declared_symbol():
    declared = _declared_symbols()
    assert declared >= {"aqp_cache_write", "aqp_get_schedule", "aqp_paged_attention", "aqp_parse_kv_dtype",
                        "aqp_cache_bytes", "aqp_last_error"}
    lib = ctypes.CDLL(aqp.LIB_PATH)
    for name in sorted(declared):
        assert hasattr(lib, name), f"{name} declared in include/ but not exported"


def _golden_dtypes():
    rows = []
    for line in open(os.path.join(GOLDEN, "kv_cache_dtypes.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            s, idx, mode = line.split()
            rows.append((s, int(idx), {"per_tensor": 0, "per_token_head": 1}[mode]))
    return rows


@pytest.mark.parametrize("s,idx,mode", _golden_dtypes())
def test_parse_kv_dtype_matches_pages(s, idx, mode):
    # "auto" is the unquantised (bf16) cache
    assert aqp.parse_kv_dtype(s) == (idx, mode)


@pytest.mark.parametrize("s,idx,mode", [("int8", 3, 0), ("fp8_e5m2_per_token_head", 2, 1), ("int8_per_group", 3, 2),
                                        ("fp8_per_group", 1, 2), ("fp8_e5m2_per_group", 2, 2)])
def test_parse_extension_pairs(s, idx, mode):
    """The codec x scale-mode pairs the pages leave for later (the two remaining per-tensor /
    per-token-head pairs and the per-group mode), under this library's names."""
    assert aqp.parse_kv_dtype(s) == (idx, mode)


def test_parse_rejects_unknown():
    with pytest.raises(aqp.AqpError) as e:
        aqp.parse_kv_dtype("fp4")
    assert e.value.status == aqp.ERR_INVALID
    assert aqp.parse_kv_dtype("fp8") == (aqp.KV_FP8_E4M3, aqp.SCALE_PER_TENSOR)


FMT = {aqp.KV_AUTO: oracle.FMT_BF16, aqp.KV_FP8_E4M3: oracle.FMT_E4M3, aqp.KV_FP8_E5M2: oracle.FMT_E5M2,
       aqp.KV_INT8: oracle.FMT_INT8}


@pytest.mark.parametrize("dtype_str", ["fp8_e4m3", "fp8_e5m2", "int8_per_token_head", "fp8_per_token_head", "int8",
                                       "fp8_e5m2_per_token_head", "auto", "int8_per_group", "fp8_per_group",
                                       "fp8_e5m2_per_group"])
@pytest.mark.parametrize("nb,bs,h,d", [(8, 16, 2, 64), (4, 2176, 2, 256), (40000, 16, 8, 128), (3, 32, 3, 128),
                                      (50, 1, 2, 64), (7, 24, 3, 256), (5, 2200, 2, 128)])
def test_cache_bytes_match_oracle_layout(dtype_str, nb, bs, h, d):
    desc = aqp.cache_desc(nb, bs, h, d, dtype_str)
    pb, bb, tb = aqp.cache_bytes(desc)
    od = oracle.CacheDesc(nb, bs, h, d, FMT[desc.dtype], desc.mode)
    assert (pb, bb, tb) == (od.page_bytes, od.block_bytes, od.total_bytes)


@pytest.mark.parametrize("bad", [dict(head_dim=96), dict(block_size=0), dict(block_size=65537), dict(num_kv_heads=0)])
def test_unsupported_geometry(bad):
    kw = dict(num_blocks=4, block_size=16, num_kv_heads=2, head_dim=64)
    kw.update(bad)
    desc = aqp.CacheDesc(kw["num_blocks"], kw["block_size"], kw["num_kv_heads"], kw["head_dim"], aqp.KV_FP8_E4M3, 0)
    with pytest.raises(aqp.AqpError) as e:
        aqp.cache_bytes(desc)
    assert e.value.status in (aqp.ERR_UNSUPPORTED, aqp.ERR_INVALID)


@pytest.mark.parametrize("bs", [1, 3, 8, 24, 40, 2200])
@pytest.mark.parametrize("dtype", ["fp8_e4m3", "int8_per_token_head", "fp8_per_group", "auto"])
def test_any_block_size_geometry(bs, dtype):
    """Block sizes that are not a multiple of 16 are accepted: a page holds block_size rows and
    their scales, rounded up to 128 bytes, as the oracle lays it out; the schedule is built and
    routes prefill work to the 16x16 kernel (the one that gathers tiles spanning blocks)."""
    desc = aqp.cache_desc(64, bs, 2, 128, dtype)
    pb, bb, tb = aqp.cache_bytes(desc)
    od = oracle.CacheDesc(64, bs, 2, 128, FMT[desc.dtype], desc.mode)
    assert (pb, bb, tb) == (od.page_bytes, od.block_bytes, od.total_bytes)
    L = min(64 * bs // 4, 300)
    sl, qsl = np.array([L, 1], np.int32), np.array([0, L, L + 1], np.int32)
    h = aqp.get_schedule(aqp.attn_params(8, 2, 128, -(-L // bs)), desc, sl, qsl).header
    assert h["block_size"] == bs and h["num_pf_items"] > 0
    # the 16x16 kernel's LDS (ring of four steps + four images + two scale slots), not the 32x32 one's
    eb = 2 if dtype == "auto" else 1
    sc = 0 if eb == 2 else 2 * 32 * 4 * (4 if dtype == "fp8_per_group" else 1)
    assert h["pf_lds_bytes"] == 4 * (2 * 32 * 128 * eb + sc) + 4 * 32 * 128 * 2 + (0 if eb == 2 else 2 * 2 * 32 * 4)


def test_row_quotient_is_exact():
    """The kernels split a 16-key tile that spans blocks with the quotient n / block_size taken as
    trunc((n + 1/2) * fl(1 / block_size)) in fp32 (n < block_size + 128): exact for every block
    size up to the library's limit (checked here in the same fp32 arithmetic, all n, all sizes
    up to 4096 and a spread of larger ones)."""
    sizes = np.concatenate([np.arange(1, 4097), np.unique(np.geomspace(4097, 65536, 3000).astype(np.int64)), [65536]])
    for bs in sizes:
        n = np.arange(0, int(bs) + 128, dtype=np.int64)
        rd = np.float32(1.0) / np.float32(bs)
        q = ((n.astype(np.float32) + np.float32(0.5)) * rd).astype(np.int64)
        assert np.array_equal(q, n // bs), bs


@pytest.mark.parametrize("dt,md", [(aqp.KV_AUTO, 1), (aqp.KV_AUTO, 2)])
def test_unbuilt_dtype_mode_pairs_are_errors(dt, md):
    with pytest.raises(aqp.AqpError) as e:
        aqp.cache_bytes(aqp.CacheDesc(4, 16, 2, 64, dt, md))
    assert e.value.status == aqp.ERR_UNSUPPORTED


@pytest.mark.parametrize("dt,md", [(4, 0), (aqp.KV_FP8_E4M3, 3), (-1, 0)])
def test_unknown_dtype_or_mode_is_invalid(dt, md):
    with pytest.raises(aqp.AqpError) as e:
        aqp.cache_bytes(aqp.CacheDesc(4, 16, 2, 64, dt, md))
    assert e.value.status == aqp.ERR_INVALID


def test_cache_write_argument_errors():
    desc = aqp.cache_desc(4, 16, 2, 64, "fp8_e4m3")
    with pytest.raises(aqp.AqpError) as e:  # null pointers
        aqp._check(aqp._lib.aqp_cache_write(ctypes.byref(desc), None, None, None, 5, 128, None, 1.0, 1.0, None))
    assert e.value.status == aqp.ERR_INVALID
    with pytest.raises(aqp.AqpError) as e:  # stride smaller than a token
        aqp._check(aqp._lib.aqp_cache_write(ctypes.byref(desc), 16, 16, 16, 5, 64, 16, 1.0, 1.0, None))
    assert e.value.status == aqp.ERR_INVALID
    with pytest.raises(aqp.AqpError) as e:  # negative per-tensor scale
        aqp._check(aqp._lib.aqp_cache_write(ctypes.byref(desc), 16, 16, 16, 5, 128, 16, -1.0, 1.0, None))
    assert e.value.status == aqp.ERR_INVALID
    # zero tokens: nothing to do, no device touched
    aqp._check(aqp._lib.aqp_cache_write(ctypes.byref(desc), None, None, None, 0, 128, None, 1.0, 1.0, None))


def test_unquantised_cache_geometry_and_limits():
    """The "auto" cache stores two bytes per element: the schedule records that size and sizes
    the decode and prefill LDS from it (no scale bytes). At head_dim 256 the prefill ring holds
    three steps and fills a CU's 160 KB exactly; a decode unit holds 4 q heads."""
    desc = aqp.cache_desc(8, 16, 2, 128, "auto")
    pb, bb, tb = aqp.cache_bytes(desc)
    assert pb == 16 * 128 * 2 and bb == 2 * 2 * pb
    params = aqp.attn_params(8, 2, 128, 4)
    sl, qsl = np.array([40, 17], np.int32), np.array([0, 1, 2], np.int32)
    h = aqp.get_schedule(params, desc, sl, qsl).header
    assert h["kv_elem_bytes"] == 2 and h["staged_elem_bytes"] == 2
    assert h["dec_lds_bytes"] == 4 * (2 * (2 * 16 * 128 * 2) + 4 * 128 * 2) + 4 * 4 * (128 + 4) * 4
    h2 = aqp.get_schedule(params, desc, np.array([40, 17], np.int32), np.array([0, 5, 6], np.int32)).header
    assert h2["num_pf_items"] > 0
    assert h2["pf_lds_bytes"] == 4 * (2 * 32 * 128 * 2) + 4 * 32 * 128 * 2
    assert h2["pf_lds_bytes"] <= 160 * 1024
    d256 = aqp.cache_desc(8, 16, 2, 256, "auto")
    h3 = aqp.get_schedule(aqp.attn_params(8, 2, 256, 4), d256, sl, np.array([0, 5, 6], np.int32)).header
    assert h3["num_pf_items"] > 0 and h3["heads_per_unit"] == 4
    assert h3["pf_lds_bytes"] == 3 * (2 * 32 * 256 * 2) + 4 * 32 * 256 * 2 == 160 * 1024
    # 4 compute waves: a ring of two 16-key tiles (K and V) and 4 q rows each, then the merge area
    assert h3["dec_lds_bytes"] == 4 * (2 * (2 * 16 * 256 * 2) + 4 * 256 * 2) + 4 * 4 * (256 + 4) * 4
    assert h3["dec_lds_bytes"] <= 160 * 1024
    # 8 q heads per KV head: two decode units of 4 heads each
    h4 = aqp.get_schedule(aqp.attn_params(16, 2, 256, 4), aqp.cache_desc(8, 16, 2, 256, "auto"), sl, qsl).header
    assert h4["group_heads"] == 4


def test_timed_call_refuses_a_bad_event_list():
    """The timed entry point checks its event list before anything else."""
    f = aqp._lib.aqp_paged_attention_timed
    args = (None, None, None, None, None, None, None, 1.0, 1.0, None, 0, None, None)
    assert f(*args, None, 2) == aqp.ERR_INVALID
    assert f(*args, None, -1) == aqp.ERR_INVALID
    assert b"event list" in aqp._lib.aqp_last_error()


def test_binding_refuses_mis_sized_buffers():
    """The binding checks every buffer's extent against what the kernels will touch (the C ABI
    takes raw pointers and cannot): too-small q, out, block tables, device schedule, scratch,
    cache, keys, values or slots are refused on the host, before any launch."""
    import numpy as np
    desc = aqp.cache_desc(8, 16, 2, 64, "fp8_e4m3")
    total = aqp.cache_bytes(desc)[2]
    sl, qsl = np.array([40, 9], np.int32), np.array([0, 1, 10], np.int32)
    params = aqp.attn_params(4, 2, 64, 3)
    s = aqp.get_schedule(params, desc, sl, qsl)
    cache = np.zeros(total, np.uint8)
    q = np.zeros((10, 4, 64), np.uint16)
    out = np.zeros((10, 4, 64), np.uint16)
    bt = np.zeros((2, 3), np.int32)
    md = s.meta.copy()
    scr = np.zeros(max(4, s.scratch_bytes), np.uint8)
    good = dict(cache=cache, q=q, block_tables=bt, meta_dev=md, scratch=scr, out=out)
    for name, small in (("q", q[:9]), ("out", out[:9]), ("block_tables", bt[:1]), ("meta_dev", md[:100]),
                        ("cache", cache[:-1]), ("scratch", scr[:1] if s.scratch_bytes > 1 else None)):
        if small is None:
            continue
        a = dict(good, **{name: small})
        with pytest.raises(ValueError, match=name):
            aqp.paged_attention(params, desc, a["cache"], a["q"], a["block_tables"], s.meta, a["meta_dev"], 1.0, 1.0,
                                a["scratch"], s.scratch_bytes, a["out"], stream=0)
    k = np.zeros((5, 2, 64), np.uint16)
    slots = np.arange(5, dtype=np.int64)
    for kk, vv, ss, cc, what in ((k[:, :, :63], k, slots, cache, "k"), (k, k[:, :1], slots, cache, "v"),
                                 (k, k, slots[:4], cache, "slot_mapping"), (k, k, slots, cache[:10], "cache")):
        with pytest.raises(ValueError, match=what):
            aqp.cache_write(desc, cc, kk, vv, ss, 1.0, 1.0, stream=0)


def test_noalloc_refuses_schedules_beyond_its_buffer():
    """The allocation-free call holds a fixed 64 MiB scratch: a schedule needing more (here 4 prefill
    sequences of 1024 tokens split into 8 key runs: 520 MiB of partial results) is refused with
    SCRATCH_TOO_SMALL before any device call (so also on a host without a GPU), nothing launched."""
    sl = np.array([4096] * 4, np.int32)
    qsl = np.array([0, 1024, 2048, 3072, 4096], np.int32)
    desc = aqp.cache_desc(4 * 256, 16, 8, 128, "int8_per_token_head")
    params = aqp.attn_params(32, 8, 128, 256, prefill_kv_split=8)
    s = aqp.get_schedule(params, desc, sl, qsl)
    assert s.scratch_bytes > aqp.NOALLOC_SCRATCH_BYTES
    rc = aqp._lib.aqp_paged_attention_noalloc(ctypes.byref(params), ctypes.byref(desc), 16, 16, 16,
                                              s.meta.ctypes.data, 16, 1.0, 1.0, 16, None)
    assert rc == aqp.ERR_SCRATCH_TOO_SMALL
    assert "64" in aqp.last_error() or str(64 << 20) in aqp.last_error()
