"""Schedule invariants (host only): every visible (query, q head, key) is
covered exactly once; split ranges tile the visible range; the scratch size
matches the partial slots; the header records the element sizes and
geometry; a schedule built for one cache/parameter set is refused for another
(the scheduler/runtime sizing disagreement of the PR 50194 page)."""
import ctypes

import numpy as np
import pytest

import attention_quantized_paged_amd as aqp
import workloads

SEG = np.dtype([(n, "<i4") for n in "seq kvh head0 nheads k_lo k_hi q_tok part".split()])
COMB = np.dtype([(n, "<i4") for n in "kvh head0 nheads q_tok first_slot num_parts part_stride pad0".split()])
PF = np.dtype([(n, "<i4") for n in ("seq kvh q_lo q_hi L ql q_start k_hi_max head0 nheads causal split_lo split_hi slot "
                                   "pad0 pad1").split()])


def h_rows(s):
    return s.header["pf_rows"]


def _arrays(s):
    h, m = s.header, s.meta
    segs = m[h["off_dec_segs"]: h["off_dec_segs"] + 32 * h["num_dec_segs"]].view(SEG)
    wgs = m[h["off_dec_wg_start"]: h["off_dec_wg_start"] + 4 * (h["num_dec_wgs"] + 1)].view(np.int32)
    comb = m[h["off_comb"]: h["off_comb"] + COMB.itemsize * h["num_comb"]].view(COMB)
    pf = m[h["off_pf_items"]: h["off_pf_items"] + PF.itemsize * h["num_pf_items"]].view(PF)
    return segs, wgs, comb, pf


def _sched(seqs, hq, hkv, d, bs, dtype="fp8_e4m3", window=0, causal=True, par=0, nb=None, rows=0, split=0):
    sl = np.array([L for _, L in seqs], np.int32)
    qsl = np.concatenate([[0], np.cumsum([q for q, _ in seqs])]).astype(np.int32)
    mb = int(max(1, max((L + bs - 1) // bs for L in sl)))
    desc = aqp.cache_desc(nb or 4 * mb * len(seqs), bs, hkv, d, dtype)
    params = aqp.attn_params(hq, hkv, d, mb, causal=causal, window=window, decode_parallelism=par, prefill_rows=rows,
                             prefill_kv_split=split)
    return aqp.get_schedule(params, desc, sl, qsl), sl, qsl, params, desc


CASES = [
    (((1, 17), (1, 40)), 4, 2, 64, 16, 0, 0),
    (((1, 1000), (1, 33), (5, 70), (1, 16), (0, 9), (1, 1)), 8, 2, 128, 16, 0, 3),
    (((1, 5000),) * 3 + ((64, 300),), 32, 1, 128, 32, 700, 7),  # G = 32 > 16: two head groups
    (workloads.CFG3.seqs, 32, 8, 128, 16, 0, 0),
    (workloads.CFG4.seqs, 32, 8, 128, 16, 0, 0),
    (workloads.CFG5A.seqs, 64, 8, 128, 16, 4096, 0),
    (workloads.CFG2.seqs, 16, 2, 256, 2176, 0, 0),
    (((3, 40), (70, 70), (1, 90)), 192, 1, 64, 16, 0, 0),  # G = 192 > 128: prefill items split the heads
    # block sizes that are not a multiple of 16 (tiles span blocks; the schedule works in keys)
    (((1, 300), (1, 17), (40, 200), (1, 1)), 8, 2, 128, 1, 0, 0),
    (((1, 1000), (33, 90), (1, 16)), 16, 2, 64, 24, 200, 5),
    (((1, 5000), (30, 30)), 16, 2, 256, 2200, 0, 0),
]


@pytest.mark.parametrize("seqs,hq,hkv,d,bs,window,par", CASES)
def test_decode_coverage_exact(seqs, hq, hkv, d, bs, window, par):
    _check_decode(seqs, hq, hkv, d, bs, window, par)


# the unquantised cache: at head_dim 256 a decode unit holds 4 q heads (8 for one-byte codes)
AUTO_CASES = [
    (((1, 17), (1, 40)), 4, 2, 256, 16, 0, 0),
    (((1, 1000), (1, 33), (5, 70), (1, 16), (0, 9), (1, 1)), 16, 2, 256, 16, 0, 3),
    (((1, 3000),) * 2 + ((40, 300),), 32, 2, 256, 32, 700, 7),
    (((1, 900), (1, 77)), 16, 2, 128, 16, 0, 0),
]


@pytest.mark.parametrize("seqs,hq,hkv,d,bs,window,par", AUTO_CASES)
def test_decode_coverage_exact_unquantised(seqs, hq, hkv, d, bs, window, par):
    _check_decode(seqs, hq, hkv, d, bs, window, par, dtype="auto")


def _check_decode(seqs, hq, hkv, d, bs, window, par, split=0, dtype="fp8_e4m3"):
    s, sl, qsl, params, desc = _sched(seqs, hq, hkv, d, bs, dtype=dtype, window=window, par=par, split=split)
    h = s.header
    segs, wgs, comb, pf = _arrays(s)
    G = hq // hkv
    eb = 2 if dtype == "auto" else 1
    assert h["kv_elem_bytes"] == eb and h["head_dim"] == d and h["block_size"] == bs
    if h["num_dec_wgs"] == 0:
        # no decode work: no segments, no work-group ranges, no parts (nothing is launched)
        assert len(segs) == 0 and h["num_parts"] == 0 and h["num_dec_comb"] == 0
        wgs = np.zeros(1, np.int32)
    assert wgs[0] == 0 and wgs[-1] == len(segs) and np.all(np.diff(wgs) >= 0)
    # each work-group's own copy of its first segment
    first = s.meta[h["off_dec_first"]: h["off_dec_first"] + SEG.itemsize * h["num_dec_wgs"]].view(SEG)
    for w_ in range(h["num_dec_wgs"]):
        assert wgs[w_] < wgs[w_ + 1] and first[w_].tobytes() == segs[wgs[w_]].tobytes()
    # coverage: for each decode (seq, kvh, head) the union of segment ranges is the visible range, disjoint
    cover = {}
    for sg in segs:
        assert sg["k_lo"] < sg["k_hi"]
        for hh in range(sg["head0"], sg["head0"] + sg["nheads"]):
            cover.setdefault((sg["seq"], sg["kvh"], hh), []).append((sg["k_lo"], sg["k_hi"], sg["part"]))
    expect = set()
    for b, (ql, L) in enumerate(seqs):
        if ql != 1:
            continue
        lo = max(0, L - window) if window else 0
        for kvh in range(hkv):
            for hh in range(G):
                key = (b, kvh, hh)
                expect.add(key)
                rs = sorted(cover[key])
                assert rs[0][0] == lo and rs[-1][1] == L
                assert all(rs[i][1] == rs[i + 1][0] for i in range(len(rs) - 1))
                if len(rs) == 1:
                    assert rs[0][2] == -1
                else:
                    assert all(r[2] >= 0 for r in rs)
    assert set(cover) == expect
    # partial slots: each used exactly once and named by exactly one merge item
    parts = sorted(sg["part"] for sg in segs if sg["part"] >= 0)
    assert parts == list(range(h["num_parts"]))
    gh = min(G, 16 if d <= 128 else (4 if eb == 2 else 8))
    assert all(sg["nheads"] <= gh and sg["head0"] % gh == 0 for sg in segs)
    dcomb = comb[: h["num_dec_comb"]]
    assert np.all(dcomb["part_stride"] == gh) and np.all(dcomb["first_slot"] % gh == 0)
    from_comb = sorted(p for c in dcomb for p in range(c["first_slot"] // gh, c["first_slot"] // gh + c["num_parts"]))
    assert from_comb == parts
    # decode parts own the first num_parts x gh slots; split prefill runs the rest
    pf_slots = sum((it["q_hi"] - it["q_lo"]) * it["nheads"] for it in pf if it["slot"] >= 0)
    assert h["num_slots"] == h["num_parts"] * gh + pf_slots
    assert h["scratch_bytes"] == h["num_slots"] * (d + 2) * 4 == s.scratch_bytes
    # balance: work-groups get equal numbers of 16-key tiles (the last may get fewer)
    if len(segs):
        tiles = []
        for w in range(h["num_dec_wgs"]):
            t = 0
            for sg in segs[wgs[w]: wgs[w + 1]]:
                t += (sg["k_hi"] - 1) // 16 - sg["k_lo"] // 16 + 1
            tiles.append(t)
        assert len(tiles) == h["num_dec_wgs"] and min(tiles) > 0
        assert len(set(tiles[:-1])) <= 1 and tiles[-1] <= tiles[0]


def _key_begin(it, window):
    first = it["L"] - it["ql"] + it["q_lo"]
    lo = max(0, first - window + 1) if window else 0
    return lo // 16 * 16


def _steps(it, window):
    kb, ke = max(_key_begin(it, window), it["split_lo"]), min(it["k_hi_max"], it["split_hi"])
    return max(0, -(-(ke - kb) // 32))


@pytest.mark.parametrize("split", [0, 1, 3])
@pytest.mark.parametrize("dtype", ["fp8_e4m3", "int8_per_group", "auto"])
@pytest.mark.parametrize("rows", [0, 64, 128])
@pytest.mark.parametrize("seqs,hq,hkv,d,bs,window,par", CASES)
def test_prefill_coverage_and_order(seqs, hq, hkv, d, bs, window, par, rows, split, dtype):
    """Every (query token, q head) of every prefill sequence is in exactly one item; a split item's
    runs tile its key range in whole 32-key steps, own consecutive blocks of partial-result slots
    and have one merge item per query token; items run heaviest first."""
    _check_prefill(seqs, hq, hkv, d, bs, window, par, rows, split, dtype=dtype)


def _check_prefill(seqs, hq, hkv, d, bs, window, par, rows, split, dtype="fp8_e4m3"):
    # (64-row items at head_dim 256 are not built: that head size runs the 16x16 prefill, whose
    # 8 waves of 16 rows make 128-row items)
    if rows == 64 and d > 128:
        with pytest.raises(aqp.AqpError) as e:
            _sched(seqs, hq, hkv, d, bs, dtype=dtype, window=window, par=par, rows=rows, split=split)
        assert e.value.status == aqp.ERR_UNSUPPORTED
        return
    s, sl, qsl, params, desc = _sched(seqs, hq, hkv, d, bs, dtype=dtype, window=window, par=par, rows=rows, split=split)
    h = s.header
    if rows:
        assert h_rows(s) == rows
    _, _, comb, pf = _arrays(s)
    G = hq // hkv
    gh = min(G, 16 if d <= 128 else (4 if dtype == "auto" else 8))
    _check_launch_order(pf, window)
    families = {}
    for it in pf:
        if it["q_hi"] == it["q_lo"]:
            continue  # launch-order padding
        assert 0 <= it["q_lo"] < it["q_hi"] <= it["ql"]
        assert 0 <= it["head0"] < it["head0"] + it["nheads"] <= G
        assert (it["q_hi"] - it["q_lo"]) * it["nheads"] <= h_rows(s)
        assert it["k_hi_max"] == it["L"] - it["ql"] + it["q_hi"]
        assert it["causal"] == 1
        families.setdefault((it["seq"], it["kvh"], it["q_lo"], it["head0"]), []).append(it)
    seen = {}
    pf_comb = comb[h["num_dec_comb"]:]
    comb_by_first = {int(c["first_slot"]): c for c in pf_comb}
    next_slot = h["num_parts"] * gh
    n_split = 0
    for key, runs in families.items():
        it0 = runs[0]
        for t in range(it0["q_lo"], it0["q_hi"]):
            for hh in range(it0["head0"], it0["head0"] + it0["nheads"]):
                k2 = (it0["seq"], it0["kvh"], t, hh)
                assert k2 not in seen
                seen[k2] = 1
        if len(runs) == 1:
            assert it0["slot"] == -1 and it0["split_lo"] == 0 and it0["split_hi"] == it0["k_hi_max"]
            continue
        assert split != 1
        runs = sorted(runs, key=lambda r: r["split_lo"])
        nrows = (it0["q_hi"] - it0["q_lo"]) * it0["nheads"]
        assert runs[0]["split_lo"] == _key_begin(it0, window) and runs[-1]["split_hi"] == it0["k_hi_max"]
        for a, b in zip(runs, runs[1:]):
            assert a["split_hi"] == b["split_lo"] and (b["split_lo"] - runs[0]["split_lo"]) % 32 == 0
        assert all(_steps(r, window) >= 1 for r in runs)
        slot0 = runs[0]["slot"]
        assert [r["slot"] for r in runs] == [slot0 + i * nrows for i in range(len(runs))]
        assert slot0 >= h["num_parts"] * gh
        for t in range(it0["q_lo"], it0["q_hi"]):
            c = comb_by_first[slot0 + (t - it0["q_lo"]) * it0["nheads"]]
            assert (c["kvh"], c["head0"], c["nheads"], c["q_tok"]) == (it0["kvh"], it0["head0"], it0["nheads"],
                                                                      it0["q_start"] + t)
            assert c["num_parts"] == len(runs) and c["part_stride"] == nrows
        n_split += len(runs)
        next_slot = max(next_slot, slot0 + len(runs) * nrows)
    assert len(pf_comb) == sum(r[0]["q_hi"] - r[0]["q_lo"] for r in families.values() if len(r) > 1)
    assert h["num_pf_split"] == n_split and h["num_slots"] == next_slot
    expect = {(b, k, t, hh) for b, (ql, L) in enumerate(seqs) if ql > 1 for k in range(hkv) for t in range(ql)
              for hh in range(G)}
    assert set(seen) == expect


XCDS = 8


def _check_launch_order(pf, window):
    """Work-group i runs on L2 domain (XCD) i % 8: with 8 or more items, each domain's items run
    longest first, padding (empty items: no rows, no keys, no slot) only after a domain's real
    items, and the domains' work within one item of an equal share; fewer items run longest
    first."""
    real = lambda it: it["q_hi"] > it["q_lo"]
    for it in pf:
        if not real(it):
            assert it["slot"] == -1 and it["k_hi_max"] == 0 and it["split_hi"] == 0
    if len(pf) < XCDS:
        work = [_steps(it, window) for it in pf]
        assert work == sorted(work, reverse=True)
        return
    assert len(pf) % XCDS == 0
    loads = []
    for b in range(XCDS):
        dom = [pf[i] for i in range(b, len(pf), XCDS)]
        flags = [real(it) for it in dom]
        assert flags == sorted(flags, reverse=True), "padding before a real item"
        work = [max(1, _steps(it, window)) for it in dom if real(it)]
        assert work == sorted(work, reverse=True)
        loads.append(sum(work))
    biggest = max(max(1, _steps(it, window)) for it in pf if real(it))
    assert max(loads) <= -(-sum(loads) // XCDS) + biggest


def test_launch_order_keeps_groups_on_few_l2_domains():
    """The large prefill (4 sequences x 2 KV heads, 64 items each of equal total work): each L2
    domain (XCD) gets the items of exactly one (sequence, KV head), so it reads one group's K and V;
    the mixed batch's prefill (2 sequences x 8 KV heads) puts at most 3 groups on a domain."""
    w2 = workloads.CFG2
    s, *_ = _sched(w2.seqs, 16, 2, 256, 2176)
    _, _, _, pf = _arrays(s)
    assert len(pf) == 512
    for b in range(XCDS):
        groups = {(int(it["seq"]), int(it["kvh"])) for it in pf[b::XCDS] if it["q_hi"] > it["q_lo"]}
        assert len(groups) == 1
    w4 = workloads.CFG4
    seqs = [x for x in w4.seqs if x[0] > 1]
    s, *_ = _sched(seqs, 32, 8, 128, 16)
    _, _, _, pf = _arrays(s)
    for b in range(XCDS):
        groups = {(int(it["seq"]), int(it["kvh"])) for it in pf[b::XCDS] if it["q_hi"] > it["q_lo"]}
        assert 1 <= len(groups) <= 3


def test_prefill_split_policy():
    """Automatic key splits only when the batch's prefill items number fewer than the work-groups
    the device holds at once (256 CUs without a device): the mixed batch's 256 items of 128 rows at
    head_dim 128 (two per CU) become 512 runs; the large prefill (512 items, one per CU) and a
    batch with enough items stay whole; 1 turns splitting off; n splits into at most n runs."""
    w4 = workloads.CFG4
    s, *_ = _sched(w4.seqs, 32, 8, 128, 16)
    h = s.header
    assert h["num_pf_items"] == 512 and h["num_pf_split"] == 512
    assert h["comb_heads"] == 4 and h["num_comb"] - h["num_dec_comb"] == 256 * 32  # one per query token
    assert _sched(w4.seqs, 32, 8, 128, 16, split=1)[0].header["num_pf_split"] == 0
    s, *_ = _sched(workloads.CFG2.seqs, 16, 2, 256, 2176)
    assert s.header["num_pf_split"] == 0 and s.header["num_pf_items"] == 512
    many = ((1024, 1024),) * 4  # 1024 items of 128 rows
    assert _sched(many, 32, 8, 128, 16)[0].header["num_pf_split"] == 0
    s, *_ = _sched(((100, 300),), 8, 2, 128, 16, split=4)
    _, _, _, pf = _arrays(s)
    pf = [it for it in pf if it["q_hi"] > it["q_lo"]]  # (without the launch-order padding)
    assert 1 < len(pf) and all(it["slot"] >= 0 for it in pf)
    assert max(sum(1 for x in pf if (x["kvh"], x["q_lo"]) == (it["kvh"], it["q_lo"])) for it in pf) <= 4


def test_schedule_records_element_sizes_and_is_checked():
    s, sl, qsl, params, desc = _sched(((1, 40), (8, 20)), 4, 2, 64, 16)
    h = s.header
    assert (h["magic"], h["kv_elem_bytes"], h["staged_elem_bytes"], h["scale_bytes"]) == (0x53505141, 1, 1, 0)
    assert h["dtype"] == aqp.KV_FP8_E4M3 and h["mode"] == aqp.SCALE_PER_TENSOR

    def call(p, d, meta, scratch_bytes=1 << 20):
        return aqp._lib.aqp_paged_attention(ctypes.byref(p), ctypes.byref(d), 16, 16, 16, meta.ctypes.data, 16,
                                            1.0, 1.0, 16, scratch_bytes, 16, None)

    # built for e4m3 per tensor, used with a per-token-head cache: refused before any launch
    d2 = aqp.cache_desc(desc.num_blocks, 16, 2, 64, "fp8_per_token_head")
    assert call(params, d2, s.meta) == aqp.ERR_SCHEDULE_MISMATCH
    d3 = aqp.cache_desc(desc.num_blocks, 16, 2, 64, "fp8_e5m2")
    assert call(params, d3, s.meta) == aqp.ERR_SCHEDULE_MISMATCH
    d4 = aqp.cache_desc(desc.num_blocks, 32, 2, 64, "fp8_e4m3")
    assert call(params, d4, s.meta) == aqp.ERR_SCHEDULE_MISMATCH
    p2 = aqp.attn_params(4, 2, 64, params.max_blocks_per_seq, window=8)
    assert call(p2, desc, s.meta) == aqp.ERR_SCHEDULE_MISMATCH
    p3 = aqp.attn_params(4, 2, 64, params.max_blocks_per_seq, softcap=30.0)
    assert call(p3, desc, s.meta) == aqp.ERR_SCHEDULE_MISMATCH
    bad = s.meta.copy()
    bad[:4] = 0
    assert call(params, desc, bad) == aqp.ERR_SCHEDULE_MISMATCH
    # a tampered element size in the header is refused
    bad = s.meta.copy()
    bad[16:20] = np.array([2], np.int32).view(np.uint8)  # kv_elem_bytes
    assert call(params, desc, bad) == aqp.ERR_SCHEDULE_MISMATCH
    assert "element size" in aqp.last_error()


def test_scratch_too_small_is_refused():
    s, sl, qsl, params, desc = _sched(((1, 9000), (1, 5000)), 8, 2, 128, 16)
    assert s.scratch_bytes > 0
    rc = aqp._lib.aqp_paged_attention(ctypes.byref(params), ctypes.byref(desc), 16, 16, 16, s.meta.ctypes.data, 16,
                                      1.0, 1.0, 16, s.scratch_bytes - 4, 16, None)
    assert rc == aqp.ERR_SCRATCH_TOO_SMALL


@pytest.mark.parametrize("seqs,err", [(((2, 1),), aqp.ERR_INVALID), (((-1, 5),), aqp.ERR_INVALID)])
def test_bad_lengths(seqs, err):
    sl = np.array([L for _, L in seqs], np.int32)
    qsl = np.concatenate([[0], np.cumsum([q for q, _ in seqs])]).astype(np.int32)
    desc = aqp.cache_desc(8, 16, 2, 64, "fp8_e4m3")
    with pytest.raises(aqp.AqpError) as e:
        aqp.get_schedule(aqp.attn_params(4, 2, 64, 4), desc, sl, qsl)
    assert e.value.status == err


def test_param_errors():
    desc = aqp.cache_desc(8, 16, 2, 64, "fp8_e4m3")
    sl, qsl = np.array([10], np.int32), np.array([0, 1], np.int32)
    for p, err in [(aqp.attn_params(3, 2, 64, 4), aqp.ERR_INVALID),
                   (aqp.attn_params(4, 2, 128, 4), aqp.ERR_INVALID),
                   (aqp.attn_params(4, 2, 64, 4, causal=False, window=4), aqp.ERR_UNSUPPORTED),
                   (aqp.attn_params(4, 2, 64, 0), aqp.ERR_INVALID),
                   (aqp.attn_params(4, 2, 64, 4, softcap=-1.0), aqp.ERR_INVALID)]:
        with pytest.raises(aqp.AqpError) as e:
            aqp.get_schedule(p, desc, sl, qsl)
        assert e.value.status == err
    # too few block-table columns for the sequence
    with pytest.raises(aqp.AqpError):
        aqp.get_schedule(aqp.attn_params(4, 2, 64, 0 + 1), desc, np.array([40], np.int32), qsl)


def test_large_block_size_geometry_is_consistent():
    """Block size 2176 with head_dim 256 (the page's large-prefill regression shape): the LDS the
    schedule sizes equals what the kernels' tiles need, from the 1-byte element size."""
    s, *_ = _sched(((1024, 1024),) * 4, 16, 2, 256, 2176)
    h = s.header
    assert h["pf_kv_tile"] == 32 and h["staged_elem_bytes"] == 1
    # prefill (the 16x16 kernel at head_dim 256): 4 ring stages of codes and scales, two K and two V
    # bf16 images, two scale copies
    assert h["pf_lds_bytes"] == 4 * (2 * 32 * 256 * 1 + 2 * 32 * 4) + 4 * 32 * 256 * 2 + 2 * 2 * 32 * 4
    # decode: per wave 2 ring slots of 16 keys of K and V, one Q slot of 8 heads; merge area of 4 waves
    assert h["dec_lds_bytes"] == 4 * (2 * (2 * 16 * 256) + 8 * 256 * 2) + 4 * 8 * (256 + 4) * 4


def test_prefill32_geometry():
    """Head_dim 128, one-byte codes per token-head (the 32x32 prefill): 4 ring stages of the K and
    V codes of 32 keys and their scales, two bf16 V images and two bf16 K images of a step, and the
    block-table entries of two batches of 64 tiles for up to 4 waves."""
    s, *_ = _sched(((512, 2560),) * 2, 32, 8, 128, 16, dtype="int8_per_token_head")
    h = s.header
    assert h["pf_lds_bytes"] == 4 * (2 * 32 * 128 * 1 + 2 * 32 * 4) + 4 * 32 * 128 * 2 + 2 * 4 * 64 * 4


def test_per_sequence_causal_flags_and_seq_lens_are_recorded():
    """dynamic_causal (one flag per sequence): non-causal prefill items span all L keys, causal
    ones end at the last row's position; the schedule also carries every sequence's key count."""
    seqs = ((12, 40), (9, 9), (1, 77), (20, 20))
    flags = np.array([0, 1, 0, 1], np.int32)
    sl = np.array([L for _, L in seqs], np.int32)
    qsl = np.concatenate([[0], np.cumsum([q for q, _ in seqs])]).astype(np.int32)
    desc = aqp.cache_desc(64, 16, 2, 64, "fp8_e4m3")
    params = aqp.attn_params(8, 2, 64, 8, causal_per_seq=flags)
    s = aqp.get_schedule(params, desc, sl, qsl)
    _, _, _, pf = _arrays(s)
    for it in pf:
        c = flags[it["seq"]]
        assert it["causal"] == c
        assert it["k_hi_max"] == (it["L"] - it["ql"] + it["q_hi"] if c else it["L"])
    h = s.header
    assert np.array_equal(s.meta[h["off_seq_lens"]: h["off_seq_lens"] + 4 * len(seqs)].view(np.int32), sl)
    with pytest.raises(aqp.AqpError) as e:
        aqp.get_schedule(aqp.attn_params(8, 2, 64, 8, causal_per_seq=[1, 2, 0, 1]), desc, sl, qsl)
    assert e.value.status == aqp.ERR_INVALID
    with pytest.raises(aqp.AqpError) as e:
        aqp.get_schedule(aqp.attn_params(8, 2, 64, 8, window=5, causal_per_seq=flags), desc, sl, qsl)
    assert e.value.status == aqp.ERR_UNSUPPORTED


def test_prefill_rows_choice():
    """128 query rows per prefill item by default; 64 at head_dim <= 128 for a prefill-only batch
    whose 128-row items would number fewer than two per CU (256 CUs without a device), and for
    per-group scales at head_dim 128; an explicit choice is kept, recorded and checked."""
    few = ((100, 300), (40, 40))
    assert h_rows(_sched(few, 32, 8, 128, 16)[0]) == 64
    assert h_rows(_sched(few, 8, 2, 64, 16)[0]) == 64
    assert h_rows(_sched(few + ((1, 500),), 32, 8, 128, 16)[0]) == 128  # decode runs beside the prefill
    assert h_rows(_sched(few, 16, 2, 256, 64)[0]) == 128
    # the mixed batch's prefill chunks alone: 256 items of 128 rows split into 512 key runs (two
    # per CU), so the items keep 128 rows
    half = tuple(x for x in workloads.CFG4.seqs if x[0] > 1)
    s_half = _sched(half, 32, 8, 128, 16)[0]
    assert h_rows(s_half) == 128 and s_half.header["num_pf_split"] == 512
    assert h_rows(_sched(half, 32, 8, 128, 16, split=1)[0]) == 64  # without splits: 64-row items
    many = ((1024, 1024),) * 4  # 4 x 32 x 8 = 1024 items of 128 rows
    assert h_rows(_sched(many, 32, 8, 128, 16)[0]) == 128
    assert h_rows(_sched(few, 32, 8, 128, 16, rows=128)[0]) == 128
    assert h_rows(_sched(many, 32, 8, 128, 16, rows=64)[0]) == 64
    # per-group scales at head_dim 128: 64-row items by default (with or without decode work beside
    # them, however many items), 128 when asked; at head_dim 64 and 256 the usual choice
    for dt in ("fp8_per_group", "int8_per_group", "fp8_e5m2_per_group"):
        assert h_rows(_sched(many, 32, 8, 128, 16, dtype=dt)[0]) == 64
        assert h_rows(_sched(few + ((1, 500),), 32, 8, 128, 16, dtype=dt)[0]) == 64
        assert h_rows(_sched(many, 32, 8, 128, 16, dtype=dt, rows=128)[0]) == 128
    assert h_rows(_sched(((1024, 1024),) * 8, 8, 2, 64, 16, dtype="fp8_per_group")[0]) == 128
    assert h_rows(_sched(few, 16, 2, 256, 64, dtype="fp8_per_group")[0]) == 128
    with pytest.raises(aqp.AqpError) as e:
        _sched(few, 32, 8, 128, 16, rows=32)
    assert e.value.status == aqp.ERR_INVALID
    # a schedule of 64-row items used with parameters that ask for 128: refused before any launch
    s, sl, qsl, params, desc = _sched(few, 32, 8, 128, 16, rows=64)
    p128 = aqp.attn_params(32, 8, 128, params.max_blocks_per_seq, prefill_rows=128)
    rc = aqp._lib.aqp_paged_attention(ctypes.byref(p128), ctypes.byref(desc), 16, 16, 16, s.meta.ctypes.data, 16,
                                      1.0, 1.0, 16, 1 << 30, 16, None)
    assert rc == aqp.ERR_SCHEDULE_MISMATCH


@pytest.mark.parametrize("d,bs", [(64, 16), (128, 16), (256, 2176)])
def test_per_group_geometry_and_mismatch(d, bs):
    """Per-group mode: one fp32 scale per 32 channels per row, staged beside the codes (decode: a
    tile's 16 rows x d/32 scales for K and V; prefill: 32 keys' for K and V per ring stage)."""
    ng = d // 32
    hq, hkv = 16, 2
    s, sl, qsl, params, desc = _sched(((1, 300), (40, 40)), hq, hkv, d, bs, dtype="fp8_per_group")
    h = s.header
    assert h["scale_bytes"] == 4 * ng and h["kv_elem_bytes"] == 1
    assert h["pf_lds_bytes"] == 4 * (2 * 32 * d + 2 * 32 * 4 * max(1, ng)) + 4 * 32 * d * 2 + 2 * 2 * 32 * 4
    hpu = 16 if d <= 128 else 8
    gh = min(hq // hkv, hpu)
    stages = 2 if d >= 256 else 3
    assert h["dec_lds_bytes"] == 4 * (stages * (2 * 16 * d + 2 * 16 * 4 * ng) + gh * d * 2) + 4 * gh * (d + 4) * 4
    assert h["dec_lds_bytes"] <= 160 * 1024 and h["pf_lds_bytes"] <= 160 * 1024
    # a schedule built for per-token-head scales is refused for the per-group cache
    s2, *_ = _sched(((1, 300), (40, 40)), hq, hkv, d, bs, dtype="fp8_per_token_head")
    rc = aqp._lib.aqp_paged_attention(ctypes.byref(params), ctypes.byref(desc), 16, 16, 16, s2.meta.ctypes.data, 16,
                                      1.0, 1.0, 16, 1 << 30, 16, None)
    assert rc == aqp.ERR_SCHEDULE_MISMATCH


# ---- randomized batches: the same invariants over shapes no table lists
from hypothesis import given, settings, strategies as st  # noqa: E402


@st.composite
def _batches(draw):
    d = draw(st.sampled_from([64, 128, 256]))
    bs = draw(st.sampled_from([16, 32, 48, 2176, 5, 24, 2200] if d == 256 else [16, 32, 48, 64, 1, 3, 8, 24]))
    hkv = draw(st.integers(1, 4))
    g = draw(st.sampled_from([1, 2, 3, 4, 8, 16, 24, 40]))
    n = draw(st.integers(1, 6))
    seqs = []
    for _ in range(n):
        L = draw(st.integers(1, 3000))
        kind = draw(st.sampled_from(["decode", "prefill", "chunk", "empty"]))
        ql = {"decode": 1, "prefill": L, "chunk": draw(st.integers(1, L)), "empty": 0}[kind]
        seqs.append((ql, L))
    window = draw(st.sampled_from([0, 0, 1, 17, 300]))
    par = draw(st.sampled_from([0, 1, 7, 100]))
    rows = draw(st.sampled_from([0, 64, 128]))
    split = draw(st.sampled_from([0, 1, 2, 5]))
    return tuple(seqs), g * hkv, hkv, d, bs, window, par, rows, split


@settings(max_examples=150, deadline=None, derandomize=True)
@given(_batches())
def test_schedule_invariants_random_batches(batch):
    """Decode coverage, partial slots and balance; prefill coverage, key runs, slots, merge items
    and order: on random mixes of decode, prefill, chunked-prefill and empty sequences."""
    seqs, hq, hkv, d, bs, window, par, rows, split = batch
    _check_decode(seqs, hq, hkv, d, bs, window, par, split=split)
    _check_prefill(seqs, hq, hkv, d, bs, window, par, rows, split)
