"""GPU parity: the HIP path through the C ABI against the oracle.

Cache bytes and scales bit-exact; attention within max-abs 2e-2 and rel-RMS
5e-3 of the oracle's fp64 result (rounded to bf16)."""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_common import Run, compare, say, to_dev, OFMT

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def aqp():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import attention_quantized_paged_amd as m
    return m


W = workloads

# Small versions of every configuration: the oracle finishes them in seconds, they still
# span several tiles, several KV splits and ragged tails.
SMALL = [
    W.CFG1,
    W.scaled(W.CFG2, name="prefill_small_d256_bs2176", seqs=((200, 200), (77, 77), (129, 300)), num_blocks=6),
    W.scaled(W.CFG3, name="decode_small_llama8b", seqs=((1, 700), (1, 33), (1, 1500), (1, 16), (1, 1)),
             num_blocks=300),
    W.scaled(W.CFG4, name="mixed_small_int8_pth", seqs=((1, 600), (1, 257)) + ((70, 310),), num_blocks=120),
    W.scaled(W.CFG5A, name="longctx_small_e4m3_pth", seqs=((1, 2000), (1, 700)), window=500, num_blocks=200),
    W.scaled(W.CFG5B, name="longctx_small_e5m2_pt", seqs=((1, 2000), (1, 700)), window=500, num_blocks=200),
    # extra strength: small cap and window at prefill, short q lengths, G = 32 (two head groups), D = 64
    W.Workload("prefill_cap5_w37_d128", "fp8_e4m3", ((17, 17), (2, 50), (9, 90), (33, 40)), 8, 2, 128, 32, 20,
               window=37, softcap=5.0, seed=77),
    W.Workload("mqa_g32_decode_pth", "fp8_per_token_head", ((1, 300), (1, 45), (5, 60)), 32, 1, 128, 16, 40, seed=78),
    W.Workload("d64_int8_mixed", "int8_per_token_head", ((1, 100), (12, 12), (1, 3)), 8, 4, 64, 16, 20, seed=79),
    W.Workload("d256_e5m2_decode", "fp8_e5m2", ((1, 333), (1, 1024)), 16, 2, 256, 64, 40, softcap=20.0, seed=80),
    W.Workload("noncausal_prefill", "fp8_e4m3", ((40, 40), (7, 7)), 8, 2, 128, 16, 10, causal=False, seed=81),
    # G = 160: a prefill item holds one token and at most 128 of its q heads; D = 256 with softcap at prefill
    W.Workload("g160_mixed_e5m2", "fp8_e5m2", ((3, 40), (1, 70), (20, 33)), 160, 1, 64, 16, 16, seed=82),
    W.Workload("prefill_d256_cap_pth", "fp8_per_token_head", ((37, 37), (5, 80)), 16, 2, 256, 16, 12,
               softcap=8.0, seed=83),
    # head_dim 256 with 16 q heads per KV head: decode units of 8 heads (two per KV head)
    W.Workload("d256_g16_pth_mixed", "fp8_per_token_head", ((1, 300), (1, 77), (3, 40)), 32, 2, 256, 16, 40,
               seed=84),
    # the codec x scale-mode pairs beyond the pages' four: int8 per tensor, e5m2 per token-head
    W.Workload("int8_pt_mixed_d128", "int8", ((1, 900), (1, 31), (48, 200), (1, 257)), 32, 8, 128, 16, 120, seed=85),
    W.Workload("e5m2_pth_mixed_w_cap", "fp8_e5m2_per_token_head", ((1, 1200), (17, 90), (1, 64)), 16, 2, 128, 16, 100,
               window=300, softcap=30.0, seed=86),
    W.Workload("int8_pt_prefill_d256", "int8", ((70, 70), (9, 130)), 16, 2, 256, 32, 12, seed=87),
    W.Workload("e5m2_pth_prefill_d64", "fp8_e5m2_per_token_head", ((45, 45), (3, 99), (1, 20)), 8, 2, 64, 16, 16,
               seed=88),
    # the unquantised ("auto", bf16) cache: decode batches, with splits, window and soft-cap
    W.scaled(W.CFG3, name="auto_decode_llama8b", kv_dtype="auto", seqs=((1, 700), (1, 33), (1, 1500), (1, 16)),
             num_blocks=200),
    W.Workload("auto_decode_d64_w_cap", "auto", ((1, 900), (1, 77), (1, 2000)), 16, 2, 64, 16, 200, window=300,
               softcap=15.0, seed=89),
    W.Workload("auto_mixed_d128", "auto", ((1, 600), (70, 310), (33, 33), (1, 17)), 32, 8, 128, 16, 80, seed=90),
    W.Workload("auto_prefill_d64_w_cap", "auto", ((40, 40), (9, 130)), 8, 2, 64, 32, 12, window=50, softcap=10.0,
               seed=96),
    # the unquantised cache at head_dim 256: decode units of 4 q heads (two or four per KV head),
    # a three-step prefill ring, split decode ranges and split prefill key runs
    W.Workload("auto_d256_decode_g8_split", "auto", ((1, 2500), (1, 77), (1, 1), (1, 640)), 16, 2, 256, 16, 220,
               seed=231),
    W.Workload("auto_d256_prefill_bs2176", "auto", ((300, 300), (37, 37), (5, 80)), 16, 2, 256, 2176, 3, seed=232),
    W.Workload("auto_d256_mixed_g16_w_cap", "auto", ((1, 900), (40, 200), (1, 31), (17, 17)), 32, 2, 256, 32, 60,
               window=150, softcap=20.0, seed=233),
    # block sizes that are not a multiple of 16: a 16-key tile spans up to 16 blocks (block 1) or
    # two (24, 40, 2200); every scale mode, head_dim and the unquantised cache; decode, prefill
    # and mixed batches with window and soft-cap
    W.Workload("bs1_decode_e4m3_pt_d128", "fp8_e4m3", ((1, 300), (1, 17), (1, 1000), (1, 1)), 8, 2, 128, 1, 1400,
               seed=241),
    W.Workload("bs8_mixed_int8_pth_d64", "int8_per_token_head", ((1, 500), (40, 200), (1, 9)), 8, 2, 64, 8, 100,
               seed=242),
    W.Workload("bs24_prefill_e4m3_pt_d128_w_cap", "fp8_e4m3", ((70, 70), (9, 130), (1, 48)), 16, 2, 128, 24, 16,
               window=50, softcap=10.0, seed=243),
    W.Workload("bs40_mixed_pg_e5m2_d256", "fp8_e5m2_per_group", ((1, 700), (1, 41), (5, 90)), 16, 2, 256, 40, 30,
               seed=244),
    W.Workload("bs3_auto_mixed_d128", "auto", ((1, 200), (20, 60), (1, 5)), 8, 2, 128, 3, 100, seed=245),
    W.Workload("bs5_prefill_e4m3_pth_d256", "fp8_per_token_head", ((37, 37), (1, 100)), 16, 2, 256, 5, 40,
               softcap=8.0, seed=246),
    W.Workload("bs1_mixed_pg_int8_d64", "int8_per_group", ((1, 64), (17, 17), (1, 33)), 8, 2, 64, 1, 130, seed=247),
    W.Workload("bs2200_mixed_e4m3_d256", "fp8_e4m3", ((1, 5000), (30, 30)), 16, 2, 256, 2200, 6, seed=248),
    W.Workload("bs7_auto_d256_prefill", "auto", ((50, 50), (3, 70)), 16, 2, 256, 7, 24, seed=249),
    # per-group scales (one per 32 head-dim channels): every codec and head_dim, decode (split and
    # whole), prefill (64- and 128-row items) and mixed batches, window and soft-cap
    W.scaled(W.CFG3, name="pg_e4m3_decode_llama8b", kv_dtype="fp8_per_group",
             seqs=((1, 700), (1, 33), (1, 1500), (1, 16), (1, 1)), num_blocks=300),
    W.Workload("pg_int8_mixed_d128_w_cap", "int8_per_group", ((1, 900), (40, 200), (1, 31), (17, 17)), 32, 8, 128,
               16, 100, window=150, softcap=20.0, seed=97),
    W.Workload("pg_e5m2_mixed_d64", "fp8_e5m2_per_group", ((1, 300), (12, 12), (1, 3), (30, 95)), 8, 2, 64, 16, 40,
               seed=98),
    W.Workload("pg_e4m3_d256_mixed_cap", "fp8_per_group", ((1, 333), (3, 40), (1, 1024), (37, 37)), 32, 2, 256, 64,
               40, softcap=8.0, seed=99),
    W.Workload("pg_int8_prefill_d256_bs2176", "int8_per_group", ((130, 130), (9, 300)), 16, 2, 256, 2176, 3,
               seed=100),
]


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_small_parity(aqp, w):
    r = Run(w, torch, aqp, par=7)
    r.cache_matches()
    out = r.gpu_attention()
    ref, rows = r.oracle_attention()
    compare(out[rows], ref, w.name)


def _alibi_slopes(hq):
    """The usual geometric ALiBi slopes 2^(-8 h / Hq), h = 1 .. Hq."""
    return (2.0 ** (-8.0 * np.arange(1, hq + 1) / hq)).astype(np.float32)


EXT = [
    # (workload, ALiBi, sinks, per-sequence causal flags)
    (W.Workload("ext_decode_alibi_sink_split", "fp8_e4m3", ((1, 900), (1, 40), (1, 2100)), 16, 4, 128, 16, 200,
                seed=101), True, True, None),
    (W.Workload("ext_mixed_pth_alibi_w_cap", "fp8_per_token_head", ((1, 500), (33, 120), (1, 64)), 8, 2, 64, 16, 60,
                window=70, softcap=20.0, seed=102), True, False, None),
    (W.Workload("ext_prefill_sinks_dyncausal", "int8_per_token_head", ((40, 40), (17, 50), (1, 30), (25, 25)), 8, 2,
                128, 16, 40, seed=103), False, True, (1, 0, 1, 0)),
    (W.Workload("ext_d256_all", "fp8_e5m2", ((29, 29), (1, 700), (8, 60)), 16, 2, 256, 32, 40, seed=104),
     True, True, (0, 1, 1)),
]


@pytest.mark.parametrize("case", EXT, ids=[c[0].name for c in EXT])
def test_alibi_sinks_dynamic_causal_parity(aqp, case):
    """The harness parameters the large-prefill page names (use_alibi, use_sink, dynamic_causal):
    ALiBi slopes, per-head sink logits and per-sequence causal flags, decode (split and whole),
    prefill and mixed batches, against the oracle."""
    w, use_alibi, use_sinks, flags = case
    rng = np.random.default_rng(w.seed)
    alibi = _alibi_slopes(w.num_q_heads) if use_alibi else None
    sinks = (rng.standard_normal(w.num_q_heads) * 2.0).astype(np.float32) if use_sinks else None
    r = Run(w, torch, aqp, par=9, alibi=alibi, sinks=sinks, causal_per_seq=flags)
    r.cache_matches()
    out = r.gpu_attention()
    ref, rows = r.oracle_attention()
    compare(out[rows], ref, w.name)


NAN_FILL = [
    W.Workload("nanfill_decode_pth", "fp8_per_token_head", ((1, 37), (1, 100), (1, 16)), 8, 2, 128, 16, 24, seed=91),
    W.Workload("nanfill_mixed_int8", "int8_per_token_head", ((1, 50), (21, 45)), 8, 2, 64, 32, 12, seed=92),
    W.Workload("nanfill_prefill_e4m3", "fp8_e4m3", ((19, 19), (40, 70)), 8, 2, 256, 32, 12, seed=93),
    W.Workload("nanfill_prefill_e4m3_pth_w", "fp8_per_token_head", ((33, 33), (9, 60)), 4, 1, 128, 16, 16, window=20,
               seed=94),
    W.Workload("nanfill_pg_mixed_d128", "fp8_per_group", ((1, 37), (21, 45), (1, 100)), 8, 2, 128, 32, 16, seed=95),
    W.Workload("nanfill_pg_prefill_d256_int8", "int8_per_group", ((19, 19), (40, 70)), 8, 2, 256, 32, 12, seed=101),
]


@pytest.mark.parametrize("w", NAN_FILL, ids=[w.name for w in NAN_FILL])
def test_unwritten_cache_bytes_do_not_leak(aqp, w):
    """Every byte of the cache that the batch does not write holds 0xFF (a NaN pattern for the fp8
    codes and for fp32 scales); rows past each sequence's end share pages with real keys. The
    outputs must not see them."""
    r = Run(w, torch, aqp, fill=0xFF)
    r.cache_matches()
    out = r.gpu_attention()
    ref, rows = r.oracle_attention()
    compare(out[rows], ref, w.name)


ROWS_CASES = [w for w in SMALL if w.name in ("prefill_cap5_w37_d128", "g160_mixed_e5m2", "auto_prefill_d64_w_cap",
                                             "e5m2_pth_mixed_w_cap", "d64_int8_mixed", "noncausal_prefill",
                                             "pg_int8_mixed_d128_w_cap", "pg_e5m2_mixed_d64")]


@pytest.mark.parametrize("rows", [64, 128])
@pytest.mark.parametrize("w", ROWS_CASES, ids=[w.name for w in ROWS_CASES])
def test_prefill_rows_per_item(aqp, w, rows):
    """Both prefill item sizes (64 and 128 query rows per work-group) match the oracle, whichever
    the schedule would pick by itself; G = 160 splits a token's heads into 64-head items."""
    r = Run(w, torch, aqp, prefill_rows=rows)
    out = r.gpu_attention()
    assert r.sched.header["pf_rows"] == rows
    ref, rows_idx = r.oracle_attention()
    compare(out[rows_idx], ref, f"{w.name} rows={rows}")


@pytest.mark.parametrize("split", [1, 2, 5])
@pytest.mark.parametrize("w", ROWS_CASES, ids=[w.name for w in ROWS_CASES])
def test_prefill_kv_split(aqp, w, split):
    """Prefill items cut into key runs (enable_kv_split of the scratch-sizing page's scheduler):
    the runs' partial results merged into the output match the oracle, whole items too."""
    r = Run(w, torch, aqp, prefill_kv_split=split)
    out = r.gpu_attention(calls=2)
    h = r.sched.header
    if split == 1:
        assert h["num_pf_split"] == 0  # (an item of a single 32-key step is never cut)
    assert np.array_equal(r.meta_after, r.sched.meta)
    ref, rows = r.oracle_attention()
    compare(out[rows], ref, f"{w.name} split={split}")


def test_prefill_kv_split_alibi_sinks(aqp):
    """Split prefill runs with ALiBi slopes and sink logits (the merge adds the sink once)."""
    w = W.Workload("split_alibi_sinks_mixed", "fp8_per_token_head", ((1, 90), (70, 300), (1, 33), (24, 24)), 8, 2,
                   128, 16, 40, window=150, softcap=30.0, seed=131)
    rng = np.random.default_rng(w.seed)
    r = Run(w, torch, aqp, alibi=_alibi_slopes(w.num_q_heads),
            sinks=(rng.standard_normal(w.num_q_heads) * 2.0).astype(np.float32), prefill_kv_split=4)
    out = r.gpu_attention()
    assert r.sched.header["num_pf_split"] > 0
    ref, rows = r.oracle_attention()
    compare(out[rows], ref, w.name)


@pytest.mark.parametrize("par", [1, 3, 64, 4096])
def test_decode_split_counts(aqp, par):
    """The same decode batch cut into 1 .. many work-groups gives the same result."""
    w = W.scaled(W.CFG3, name=f"decode_split_{par}", seqs=((1, 3000), (1, 129), (1, 2047)), num_blocks=400)
    r = Run(w, torch, aqp, par=par)
    out = r.gpu_attention()
    ref, rows = r.oracle_attention()
    compare(out[rows], ref, w.name)


def test_reused_schedule_copy_gives_identical_results(aqp):
    """Calls reusing one device copy of the schedule give bit-identical outputs and leave the copy
    unchanged, at several work-group counts."""
    w = W.scaled(W.CFG3, name="reuse_meta", seqs=((1, 3000), (1, 129), (1, 2047), (1, 700)) * 3, num_blocks=1200)
    for par in (0, 3, 40):
        r = Run(w, torch, aqp, par=par)
        last = r.gpu_attention(calls=4)
        first = r.outs[0].cpu().numpy().view(np.uint16)
        assert np.array_equal(first, last), f"par={par}"
        assert np.array_equal(r.meta_after, r.sched.meta), f"par={par}: schedule copy changed"
    ref, rows = r.oracle_attention()
    compare(last[rows], ref, w.name)


def test_timed_call_matches_and_records_its_events_in_order(aqp):
    """aqp_paged_attention_timed gives the output of aqp_paged_attention bit for bit and records its
    six events in order: around the decode kernel, its merge, the prefill kernel and its merge (a
    mixed batch with split decode ranges and split prefill runs)."""
    w = W.scaled(W.CFG4, name="timed_mixed", seqs=((1, 600), (1, 257), (70, 310)), num_blocks=120)
    r = Run(w, torch, aqp, par=7, prefill_kv_split=2)
    plain = r.gpu_attention()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    for e in ev:
        e.record()  # (creates the event)
    torch.cuda.synchronize()
    timed = r.gpu_attention(events=[int(e.cuda_event) for e in ev])
    assert np.array_equal(plain, timed)
    t = [ev[0].elapsed_time(e) for e in ev]
    say(f"  event times (ms): {[round(x, 4) for x in t]}")
    assert all(t[i] <= t[i + 1] + 1e-3 for i in range(5)), t
    assert t[1] > 0 and t[4] > t[3], t
    # a partial list: only the decode kernel's two points
    timed2 = r.gpu_attention(events=[int(ev[0].cuda_event), int(ev[1].cuda_event)])
    assert np.array_equal(plain, timed2) and ev[0].elapsed_time(ev[1]) > 0


GUARDED = [
    # the large-prefill shape the scratch-sizing page's regression test uses (block 2176, head_dim
    # 256), shortened so the oracle stays fast; a split decode; a mixed per-token-head batch
    W.scaled(W.CFG2, name="guard_prefill_bs2176_d256", seqs=((300, 300), (1, 900), (64, 64)), num_blocks=5),
    W.scaled(W.CFG3, name="guard_decode_split", seqs=((1, 3000), (1, 129), (1, 2047)), num_blocks=400),
    W.scaled(W.CFG4, name="guard_mixed_int8_pth", seqs=((1, 600), (70, 310), (1, 17)), num_blocks=80),
    W.Workload("guard_e5m2_pth_d64", "fp8_e5m2_per_token_head", ((1, 70), (9, 40)), 8, 2, 64, 16, 10, seed=95),
]


@pytest.mark.parametrize("w", GUARDED, ids=[w.name for w in GUARDED])
def test_guard_bands_untouched(aqp, w):
    """Cache, scratch and output sit inside larger allocations whose bytes before and after hold a
    pattern: after the cache write and the attention call every guard byte is unchanged (an
    out-of-range write by any kernel, the failure class of a schedule sized for the wrong element
    size, would show here), and the results still match the oracle."""
    G = 1 << 16  # guard bytes on each side
    pat = 0xA5
    say(f"[case] guards {w.name}")
    b = workloads.make_batch(w)
    desc = aqp.cache_desc(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim, w.kv_dtype)
    total = aqp.cache_bytes(desc)[2]
    cbuf = torch.full((total + 2 * G,), pat, dtype=torch.uint8, device="cuda")
    cache = cbuf[G:G + total]
    aqp.cache_write(desc, cache, to_dev(b.k_hist, torch), to_dev(b.v_hist, torch), to_dev(b.slots_hist, torch),
                    b.k_scale, b.v_scale)
    params = aqp.attn_params(w.num_q_heads, w.num_kv_heads, w.head_dim, b.block_tables.shape[1], causal=w.causal,
                             window=w.window, softcap=w.softcap, decode_parallelism=5)
    sch = aqp.get_schedule(params, desc, b.seq_lens, b.query_start_loc)
    nsc = sch.scratch_bytes
    sbuf = torch.full((nsc + 2 * G,), pat, dtype=torch.uint8, device="cuda")
    q = to_dev(b.q, torch)
    nout = q.numel() * 2
    obuf = torch.full((nout + 2 * G,), pat, dtype=torch.uint8, device="cuda")
    out = obuf[G:G + nout].view(torch.int16).view(q.shape)
    aqp.paged_attention(params, desc, cache, q, to_dev(b.block_tables, torch), sch.meta,
                        torch.from_numpy(sch.meta).cuda(), b.k_scale, b.v_scale, sbuf[G:G + nsc] if nsc else None,
                        nsc, out)
    torch.cuda.synchronize()
    for name, buf, n in (("cache", cbuf, total), ("scratch", sbuf, nsc), ("out", obuf, nout)):
        h = buf.cpu().numpy()
        assert np.all(h[:G] == pat) and np.all(h[G + n:] == pat), f"{name}: a guard byte changed"
    od = oracle.CacheDesc(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim, OFMT[desc.dtype], desc.mode)
    ocache = np.full(od.total_bytes, pat, np.uint8)
    oracle.cache_write(od, ocache, b.k_hist, b.v_hist, b.slots_hist, b.k_scale, b.v_scale)
    assert np.array_equal(cache.cpu().numpy(), ocache)
    ref = oracle.attention(od, ocache, b.q, b.block_tables, b.seq_lens, b.query_start_loc, w.num_q_heads,
                           causal=w.causal, window=w.window, softcap=w.softcap, k_scale=b.k_scale, v_scale=b.v_scale)
    compare(out.cpu().numpy().view(np.uint16), ref, w.name)


def test_block_permutation_bit_identical(aqp):
    """Same keys in a contiguous pool or a permuted one: bit-identical GPU output."""
    w = W.scaled(W.CFG4, name="perm_a", seqs=((1, 500), (40, 200)), num_blocks=60)
    r1 = Run(w, torch, aqp)
    o1 = r1.gpu_attention()
    b = r1.b
    # remap every physical block through a permutation and rewrite the cache
    perm = np.random.default_rng(5).permutation(w.num_blocks).astype(np.int32)
    bt2 = np.where(b.block_tables >= 0, perm[np.maximum(b.block_tables, 0)], -1).astype(np.int32)
    slots2 = perm[b.slots_hist // w.block_size].astype(np.int64) * w.block_size + b.slots_hist % w.block_size
    r1.gcache.zero_()
    aqp.cache_write(r1.desc, r1.gcache, to_dev(b.k_hist, torch), to_dev(b.v_hist, torch), to_dev(slots2, torch))
    b.block_tables = bt2
    o2 = r1.gpu_attention()
    assert np.array_equal(o1, o2)


@pytest.mark.parametrize("dtype_str", ["fp8_e4m3", "fp8_e5m2", "int8_per_token_head", "fp8_per_token_head", "int8",
                                       "fp8_e5m2_per_token_head", "auto", "int8_per_group", "fp8_per_group",
                                       "fp8_e5m2_per_group"])
@pytest.mark.parametrize("D", [64, 128, 256])
def test_cache_write_bit_exact(aqp, dtype_str, D):
    """Random slots (some negative), a fused-QKV token stride, specials (zero rows, huge and tiny
    values): GPU cache bytes equal the oracle's, starting from the same fill."""
    rng = np.random.default_rng(D + len(dtype_str))
    say(f"[case] cache_write {dtype_str} D={D}")
    hkv, bs, nb, n = 3, 32, 12, 200
    desc = aqp.cache_desc(nb, bs, hkv, D, dtype_str)
    od = oracle.CacheDesc(nb, bs, hkv, D, OFMT[desc.dtype], desc.mode)
    x = (rng.standard_normal((n, 3 * hkv, D)) * np.exp(rng.uniform(-8, 8, (n, 3 * hkv, 1)))).astype(np.float32)
    x[0] = 0.0
    x[1, :, 5] = -0.0
    x[2, :, 7] = 1e30
    x[3] *= 1e-30
    qkv = workloads.bf16_round(x)  # [n, q|k|v heads, D]: k = heads hkv..2hkv, v = 2hkv..3hkv
    k = np.ascontiguousarray(qkv[:, hkv:2 * hkv])
    v = np.ascontiguousarray(qkv[:, 2 * hkv:])
    slots = rng.permutation(nb * bs)[:n].astype(np.int64)
    slots[::11] = -1
    ks, vs = 0.37, 2.5e-3
    ocache = np.full(od.total_bytes, 0x5A, np.uint8)
    oracle.cache_write(od, ocache, k, v, slots, ks, vs)
    g = torch.full((od.total_bytes,), 0x5A, dtype=torch.uint8, device="cuda")
    dq = to_dev(qkv, torch)
    # k and v as strided views of the fused tensor
    kview = dq[:, hkv:2 * hkv]
    vview = dq[:, 2 * hkv:]
    aqp.cache_write(desc, g, kview, vview, to_dev(slots, torch), ks, vs, token_stride=3 * hkv * D)
    torch.cuda.synchronize()
    gh = g.cpu().numpy()
    bad = np.nonzero(gh != ocache)[0]
    assert bad.size == 0, f"{bad.size} bytes differ at {bad[:10]}"


@pytest.mark.parametrize("dtype_str,scale", [("fp8_e4m3", 1.0), ("fp8_e4m3", 1 / 448.0), ("fp8_e4m3", 3.7),
                                             ("fp8_e5m2", 1.0), ("fp8_e5m2", 1e-3), ("fp8_e5m2", 0.011)])
def test_codec_every_bf16_pattern(aqp, dtype_str, scale):
    """Every finite bf16 bit pattern through the cache write at a per-tensor scale: bit-exact
    against the oracle's encoder (the hardware conversion's rounding, saturation and zero signs)."""
    say(f"[case] codec grid {dtype_str} scale={scale}")
    pats = np.arange(65536, dtype=np.uint32)
    f = (pats << 16).view(np.float32)
    pats = pats[np.isfinite(f)].astype(np.uint16)
    D, hkv = 128, 1
    n = (pats.size + D - 1) // D
    pad = np.zeros(n * D, np.uint16)
    pad[: pats.size] = pats
    k = pad.reshape(n, hkv, D)
    v = np.ascontiguousarray(k[::-1])
    desc = aqp.cache_desc((n + 15) // 16, 16, hkv, D, dtype_str)
    od = oracle.CacheDesc(desc.num_blocks, 16, hkv, D, OFMT[desc.dtype], desc.mode)
    slots = np.arange(n, dtype=np.int64)
    ocache = np.zeros(od.total_bytes, np.uint8)
    oracle.cache_write(od, ocache, k, v, slots, scale, scale)
    g = torch.zeros(od.total_bytes, dtype=torch.uint8, device="cuda")
    aqp.cache_write(desc, g, to_dev(k, torch), to_dev(v, torch), to_dev(slots, torch), scale, scale)
    torch.cuda.synchronize()
    assert np.array_equal(g.cpu().numpy(), ocache)


def test_empty_and_zero_query_batches(aqp):
    desc = aqp.cache_desc(4, 16, 2, 64, "fp8_e4m3")
    params = aqp.attn_params(4, 2, 64, 2)
    s = aqp.get_schedule(params, desc, np.zeros(0, np.int32), np.zeros(1, np.int32))
    assert s.header["num_dec_segs"] == 0 and s.header["num_pf_items"] == 0
    cache = torch.zeros(aqp.cache_bytes(desc)[2], dtype=torch.uint8, device="cuda")
    out = torch.zeros((1, 4, 64), dtype=torch.int16, device="cuda")
    aqp.paged_attention(params, desc, cache, out, torch.zeros((1, 2), dtype=torch.int32, device="cuda"), s.meta,
                        torch.from_numpy(s.meta).cuda(), 1.0, 1.0, None, 0, out)
    # sequences with no queries produce no work
    s2 = aqp.get_schedule(params, desc, np.array([20, 5], np.int32), np.array([0, 0, 0], np.int32))
    assert s2.header["total_q_tokens"] == 0


def _random_workload(seed):
    """A seeded random batch: codec and scale mode, head_dim, block size, GQA ratio, a mix of
    decode, prefill, chunked-prefill and empty sequences, window, soft-cap, outliers."""
    rng = np.random.default_rng(9000 + seed)
    dtypes = ["fp8_e4m3", "fp8_e5m2", "int8", "int8_per_token_head", "fp8_per_token_head",
              "fp8_e5m2_per_token_head", "int8_per_group", "fp8_per_group", "fp8_e5m2_per_group", "auto"]
    dt = dtypes[seed % len(dtypes)]
    d = int(rng.choice([64, 128, 256]))
    bs = int(rng.choice([16, 32, 64, 1, 8, 24]))
    hkv = int(rng.integers(1, 4))
    g = int(rng.choice([1, 2, 4, 6, 8, 16]))
    seqs = []
    for _ in range(int(rng.integers(1, 6))):
        L = int(rng.integers(1, 700))
        kind = rng.choice(["decode", "decode", "prefill", "chunk", "empty"])
        ql = {"decode": 1, "prefill": min(L, 160), "chunk": int(rng.integers(1, min(L, 90) + 1)), "empty": 0}[kind]
        if kind == "prefill":
            L = ql
        seqs.append((ql, L))
    nb = sum(-(-L // bs) for _, L in seqs) + int(rng.integers(0, 8))
    window = int(rng.choice([0, 0, 7, 100]))
    cap = float(rng.choice([0.0, 0.0, 12.0]))
    return W.Workload(f"random_{seed}_{dt}_d{d}", dt, tuple(seqs), g * hkv, hkv, d, bs, nb, window=window, softcap=cap,
                      sigma=float(rng.choice([0.5, 1.0, 2.0])), outlier_frac=float(rng.choice([0.0, 0.01])),
                      outlier_factor=20.0, seed=9000 + seed)


@pytest.mark.parametrize("seed", range(16))
def test_random_batches(aqp, seed):
    """Seeded random batches through the whole path (cache write bit-exact, attention within the
    tolerances), with a random split of the decode work and of the prefill key ranges. Outliers
    over windows of a few keys make outputs that cancel large terms: there the per-element bound
    also admits 2^-8 of sum_j p_j |v_j| (bf16 probabilities); rel-RMS stays 5e-3."""
    w = _random_workload(seed)
    rng = np.random.default_rng(seed)
    r = Run(w, torch, aqp, par=int(rng.choice([0, 1, 5, 50])), prefill_kv_split=int(rng.choice([0, 1, 3])))
    r.cache_matches()
    out = r.gpu_attention()
    ref, rows = r.oracle_attention()
    compare(out[rows], ref, w.name, magnitude=r.oracle_magnitude())
