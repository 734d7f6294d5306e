"""Benchmark of the quantized paged attention hot path on one MI355X.

One step = one pass of the whole path over one decode batch: quantised cache
write of the step's new tokens, the host schedule (built and uploaded), and
paged attention (decode kernel + split-KV merge). Workload: 64 sequences with
one query each, contexts uniform in [512, 8192] (seeded), 32 q heads / 8 KV
heads, head_dim 128, block_size 16, fp8 e4m3 per-tensor cache over a pool of
40000 blocks (randomly permuted block tables), bf16 N(0,1) inputs with 1 % of
the entries scaled by 20. Inputs are synthetic (seeded) and resident in HBM
before timing starts.

value = algorithmic KV bytes read per step (every visible key and value code)
        x steps / elapsed wall time of the timed steps, in GB/s.
A secondary figure runs the large causal prefill (4 x 1024 tokens, 16/2 heads,
head_dim 256, block_size 2176, fp8 e4m3) and reports TFLOP/s over its
algorithmic flops (4 * D per visible (query, key) pair per q head).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2516.6  # 256 CU x 2.4 GHz x 4096 flop/clk/CU, dense


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--quiet", action="store_true")
    ap.add_argument("--preload-ms", type=float, default=200.0,
                    help="wall-clock milliseconds of untimed decode steps run after the warm-up steps and before "
                         "the timed steps (the GPU takes tens of ms of continuous work to reach its working "
                         "clocks); declared in the output line")
    ap.add_argument("--copy-probe", action="store_true",
                    help="time a plain 2 GiB device-to-device copy (calibrates the HBM byte counters and gives "
                         "the achievable read + write rate)")
    ap.add_argument("--mfma-probe", action="store_true",
                    help="time a large bf16 GEMM from the vendor library and hand-written MFMA loops (two shapes), "
                         "with the shader clock they ran at")
    ap.add_argument("--lds-probe", action="store_true",
                    help="LDS read rate (16-byte reads and 8-bit transposed reads) and the result layout of the "
                         "32x32x16 bf16 MFMA, checked on the host")
    ap.add_argument("--stage-probe", action="store_true",
                    help="staging 1 KB pages into LDS three ways (direct global -> LDS copies, register loads, "
                         "register loads plus LDS writes) at the prefill's occupancy")
    ap.add_argument("--gather-probe", action="store_true",
                    help="plain vector loads of the decode batch's K and V pages in the decode's order: the "
                         "achievable rate of that access pattern")
    ap.add_argument("--all-configs", action="store_true",
                    help="one JSON line per configuration (1-5): cache write of its history and one "
                         "attention call, median kernel times with a 1 GiB read between repetitions")
    ap.add_argument("--block-sizes", action="store_true",
                    help="with --all-configs: the decode batch (block 1, 24, 32) and the large prefill (block 8, 24, "
                         "2200) instead of the configurations")
    ap.add_argument("--only", default="",
                    help="with --all-configs: comma-separated workload names to run (default: all)")
    ap.add_argument("--no-oracle", action="store_true",
                    help="with --all-configs: skip the oracle's CPU timing")
    ap.add_argument("--reps", type=int, default=20,
                    help="with --all-configs: timed repetitions of each attention call")
    return ap.parse_args()


def log(args, *a):
    if not args.quiet:
        print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("decode.hip", "device_common.h", "aqp_internal.h"):
        with open(os.path.join(ROOT, "attention_quantized_paged_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profile(bytes_alg_per_launch: float):
    """HBM bytes per launch of the decode kernel from the committed rocprofv3 counter summary,
    or None if it was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", "decode_kernel_decode64_fp8e4m3_pmc.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def setup_decode(torch, aqp, W, args):
    w = W.CFG3
    b = W.make_batch(w)
    desc = aqp.cache_desc(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim, w.kv_dtype)
    total = aqp.cache_bytes(desc)[2]
    cache = torch.zeros(total, dtype=torch.uint8, device="cuda")
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a.view(np.int16) if a.dtype == np.uint16 else a)).cuda()
    old = ~b.new_mask
    aqp.cache_write(desc, cache, dev(b.k_hist[old]), dev(b.v_hist[old]), dev(b.slots_hist[old]), b.k_scale, b.v_scale)
    new_k, new_v, new_s = dev(b.k_hist[b.new_mask]), dev(b.v_hist[b.new_mask]), dev(b.slots_hist[b.new_mask])
    q = dev(b.q)
    out = torch.empty_like(q)
    bt = dev(b.block_tables)
    params = aqp.attn_params(w.num_q_heads, w.num_kv_heads, w.head_dim, b.block_tables.shape[1])
    sch = aqp.get_schedule(params, desc, b.seq_lens, b.query_start_loc)
    # The schedule of each step is built into one of two pinned host buffers and uploaded on a
    # second stream (default priority) into one of two device buffers, so the upload of step
    # i+1 overlaps the kernels of step i. Each buffer is reused only after the work that read it
    # has completed.
    cap = sch.meta.size + (1 << 16)
    meta_pinned = [torch.empty(cap, dtype=torch.uint8).pin_memory() for _ in range(2)]
    meta_np = [t.numpy() for t in meta_pinned]
    meta_dev = [torch.empty(cap, dtype=torch.uint8, device="cuda") for _ in range(2)]
    copied = [torch.cuda.Event(), torch.cuda.Event()]   # upload of buffer slot finished
    consumed = [torch.cuda.Event(), torch.cuda.Event()]  # attention that read slot finished
    used = [False, False]
    copy_stream = torch.cuda.Stream()
    scratch = torch.empty(max(sch.scratch_bytes, 4) * 2, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    return dict(w=w, b=b, desc=desc, cache=cache, new=(new_k, new_v, new_s), q=q, out=out, bt=bt, params=params,
                meta_pinned=meta_pinned, meta_np=meta_np, meta_dev=meta_dev, copied=copied, consumed=consumed,
                used=used, copy_stream=copy_stream, scratch=scratch, sched=sch, step=0,
                main_stream=torch.cuda.current_stream(), stream=torch.cuda.current_stream().cuda_stream)


def decode_step(torch, aqp, s, ev=None):
    b = s["b"]
    st = s["stream"]
    main, cs = s["main_stream"], s["copy_stream"]
    nk, nv, ns = s["new"]
    aqp.cache_write(s["desc"], s["cache"], nk, nv, ns, b.k_scale, b.v_scale, stream=st)
    slot = s["step"] & 1
    s["step"] += 1
    if s["used"][slot]:
        s["copied"][slot].synchronize()  # the pinned buffer's previous upload is done
    sch = aqp.get_schedule(s["params"], s["desc"], b.seq_lens, b.query_start_loc, out=s["meta_np"][slot])
    n = sch.meta.size
    with torch.cuda.stream(cs):
        if s["used"][slot]:
            cs.wait_event(s["consumed"][slot])  # the device buffer's previous reader is done
        s["meta_dev"][slot][:n].copy_(s["meta_pinned"][slot][:n], non_blocking=True)
        s["copied"][slot].record(cs)
    main.wait_event(s["copied"][slot])
    # ev: HIP events the library records on the launch stream before the decode kernel, after it,
    # and after the merge of its split ranges
    aqp.paged_attention(s["params"], s["desc"], s["cache"], s["q"], s["bt"], sch.meta, s["meta_dev"][slot],
                        b.k_scale, b.v_scale, s["scratch"], s["scratch"].numel(), s["out"], stream=st,
                        events=None if ev is None else [int(e.cuda_event) for e in ev])
    s["consumed"][slot].record(main)
    s["used"][slot] = True
    return sch


def run_prefill(torch, aqp, W, args):
    w = W.CFG2
    b = W.make_batch(w)
    desc = aqp.cache_desc(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim, w.kv_dtype)
    cache = torch.zeros(aqp.cache_bytes(desc)[2], dtype=torch.uint8, device="cuda")
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a.view(np.int16) if a.dtype == np.uint16 else a)).cuda()
    aqp.cache_write(desc, cache, dev(b.k_hist), dev(b.v_hist), dev(b.slots_hist), b.k_scale, b.v_scale)
    q = dev(b.q)
    out = torch.empty_like(q)
    bt = dev(b.block_tables)
    params = aqp.attn_params(w.num_q_heads, w.num_kv_heads, w.head_dim, b.block_tables.shape[1])
    sch = aqp.get_schedule(params, desc, b.seq_lens, b.query_start_loc)
    meta_dev = torch.from_numpy(sch.meta).cuda()
    scratch = torch.empty(max(sch.scratch_bytes, 4), dtype=torch.uint8, device="cuda")
    call = lambda: aqp.paged_attention(params, desc, cache, q, bt, sch.meta, meta_dev, b.k_scale, b.v_scale, scratch,
                                       scratch.numel(), out)
    for _ in range(3):
        call()
    torch.cuda.synchronize()
    ms, p10, p90 = timed_flushed(torch, call, 20)
    flops = W.prefill_flops(w)
    tf = flops / (ms * 1e-3) / 1e12
    return {"workload": w.name, "tflops": round(tf, 2), "frac_of_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4),
            "ms_per_call": round(ms, 4), "ms_p10_p90": [round(p10, 4), round(p90, 4)], "flops": flops,
            "timing": "median of 20 HIP-event pairs, each after a 1 GiB read (cold L2 and Infinity Cache)"}


_FLUSH = None


def timed_flushed(torch, fn, reps):
    """Median, p10 and p90 of HIP-event times of fn(), each repetition after a 1 GiB read that
    evicts L2 and the Infinity Cache (a read, so no dirty lines are written back meanwhile)."""
    global _FLUSH
    if _FLUSH is None:
        _FLUSH = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    ts = []
    for _ in range(reps):
        _FLUSH.sum()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    return float(np.median(ts)), float(np.percentile(ts, 10)), float(np.percentile(ts, 90))


def run_cache_write(torch, aqp, W, s):
    """Quantise-and-scatter of the decode batch's whole history (every token of every sequence)
    into its cache: algorithmic bytes = bf16 K and V read + one code byte each written + the slot
    index, per (token, KV head)."""
    w, b, desc = s["w"], s["b"], s["desc"]
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a.view(np.int16) if a.dtype == np.uint16 else a)).cuda()
    k, v, slots = dev(b.k_hist), dev(b.v_hist), dev(b.slots_hist)
    call = lambda: aqp.cache_write(desc, s["cache"], k, v, slots, b.k_scale, b.v_scale)
    for _ in range(2):
        call()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(10)]
    for e0, e1 in evs:
        e0.record()
        call()
        e1.record()
    torch.cuda.synchronize()
    ms = float(np.median([e0.elapsed_time(e1) for e0, e1 in evs]))
    n = int(slots.numel())
    byts = n * w.num_kv_heads * w.head_dim * 2 * (2 + 1) + n * 8
    del k, v, slots
    return {"workload": f"history of {w.name}", "tokens": n, "gbs": round(byts / (ms * 1e-3) / 1e9, 1),
            "frac_of_hbm_peak": round(byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "ms_per_call": round(ms, 4),
            "bytes": byts, "timing": "median of 10 HIP-event pairs"}


def cpu_baseline(W, s, target_seconds=10.0):
    """The oracle (plain C, OpenMP) running the same step on the host: quantised cache write of
    the step's new tokens into its own cache, then attention for every sequence of the batch.
    Repeated until about target_seconds of work; KV bytes read per second."""
    import oracle
    w, b = s["w"], s["b"]
    fmt = {1: oracle.FMT_E4M3, 2: oracle.FMT_E5M2, 3: oracle.FMT_INT8}[s["desc"].dtype]
    od = oracle.CacheDesc(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim, fmt, s["desc"].mode)
    ocache = np.zeros(od.total_bytes, dtype=np.uint8)
    old, new = ~b.new_mask, b.new_mask
    oracle.cache_write(od, ocache, b.k_hist[old], b.v_hist[old], b.slots_hist[old], b.k_scale, b.v_scale)
    nk, nv, ns = (np.ascontiguousarray(x[new]) for x in (b.k_hist, b.v_hist, b.slots_hist))
    kv_bytes = W.kv_read_bytes(w, per_token_head=False)
    steps, elapsed = 0, 0.0
    while elapsed < target_seconds:
        t0 = time.perf_counter()
        oracle.cache_write(od, ocache, nk, nv, ns, b.k_scale, b.v_scale)
        oracle.attention(od, ocache, b.q, b.block_tables, b.seq_lens, b.query_start_loc, w.num_q_heads,
                         k_scale=b.k_scale, v_scale=b.v_scale)
        elapsed += time.perf_counter() - t0
        steps += 1
    return {"value": round(kv_bytes * steps / elapsed / 1e9, 3), "unit": "GB/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{steps} full steps of the same decode batch (cache write of its 64 new tokens + attention "
                      f"over {kv_bytes / 1e6:.1f} MB of KV per step) in {elapsed:.1f} s; fp64 attention over the "
                      f"dequantised, gathered cache"}


def run_all_configs(torch, aqp, W, args):
    """Every configuration through the whole path once: the cache write of its full history
    (bf16 K/V drawn on the device, per-tensor scales absmax/qmax of that history), then one
    paged-attention call; medians of HIP-event times over repetitions separated by a 1 GiB read
    (cold L2 and Infinity Cache). Decode KV GB/s counts every visible key and value code (and
    per-token-head scales); prefill TFLOP/s counts 4 * D flops per visible (query, key) pair and
    q head. Mixed batches report the one call's time against both units."""
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")

    spread = {}

    def timed(fn, reps, key=None):
        ts = []
        for _ in range(reps):
            flush.sum()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        if key:
            spread[key] = [round(float(np.percentile(ts, 10)), 4), round(float(np.percentile(ts, 90)), 4)]
        return float(np.median(ts))

    import oracle
    ofmt = {0: oracle.FMT_BF16, 1: oracle.FMT_E4M3, 2: oracle.FMT_E5M2, 3: oracle.FMT_INT8}

    # the decode batch and the large prefill once more over an unquantised (bf16, "auto") cache:
    # the same kernels with two-byte elements, for the quantisation's saving side by side
    auto3 = W.scaled(W.CFG3, name="decode64_bf16_auto_llama8b", kv_dtype="auto")
    auto2 = W.scaled(W.CFG2, name="prefill_bf16_auto_d256_bs2176", kv_dtype="auto")
    only = set(x for x in args.only.split(",") if x)
    configs = (W.CFG1, W.CFG2, W.CFG3, W.CFG4, W.CFG5A, W.CFG5B, auto3, auto2)
    if args.block_sizes:
        # the decode batch and the large prefill with only the block size changed (block sizes that
        # are not a multiple of 16 take the kernels that gather a tile row by row)
        configs = tuple(W.scaled(W.CFG3, name=f"decode64_fp8e4m3_pt_llama8b_bs{bs}", block_size=bs,
                                 num_blocks=-(-40000 * 16 // bs) + 64) for bs in (1, 24, 32)) + \
                  tuple(W.scaled(W.CFG2, name=f"prefill_fp8e4m3_pt_d256_bs{bs}", block_size=bs,
                                 num_blocks=4 * -(-1024 // bs) + 8) for bs in (8, 24, 2200))
    for w in configs:
        if only and w.name not in only:
            continue
        log(args, f"[bench] {w.name}")
        b = W.make_batch(w, with_kv=False)
        desc = aqp.cache_desc(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim, w.kv_dtype)
        cache = torch.zeros(aqp.cache_bytes(desc)[2], dtype=torch.uint8, device="cuda")
        n = int(b.seq_lens.sum())
        g = torch.Generator(device="cuda").manual_seed(w.seed)
        k = (torch.randn((n, w.num_kv_heads, w.head_dim), device="cuda", generator=g) * w.sigma).to(torch.bfloat16)
        v = (torch.randn((n, w.num_kv_heads, w.head_dim), device="cuda", generator=g) * w.sigma).to(torch.bfloat16)
        pth = desc.mode == 1
        qm = {0: 1.0, 1: 448.0, 2: 57344.0, 3: 127.0}[desc.dtype]
        eb = 2 if desc.dtype == 0 else 1
        ks = float(k.float().abs().max()) / qm
        vs = float(v.float().abs().max()) / qm
        slots = torch.from_numpy(b.slots_hist).cuda()
        cw = lambda: aqp.cache_write(desc, cache, k, v, slots, ks, vs)
        cw()
        cw_ms = timed(cw, 5)
        cw_bytes = n * w.num_kv_heads * w.head_dim * 2 * (2 + eb) + n * 8 + (n * w.num_kv_heads * 8 if pth else 0)
        host16 = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)
        kh, vh = host16(k), host16(v)
        del k, v
        q = (torch.randn((int(b.query_start_loc[-1]), w.num_q_heads, w.head_dim), device="cuda", generator=g)
             * w.sigma).to(torch.bfloat16)
        out = torch.empty_like(q)
        bt = torch.from_numpy(b.block_tables).cuda()
        params = aqp.attn_params(w.num_q_heads, w.num_kv_heads, w.head_dim, b.block_tables.shape[1], causal=w.causal,
                                 window=w.window, softcap=w.softcap)
        sch = aqp.get_schedule(params, desc, b.seq_lens, b.query_start_loc)
        md = torch.from_numpy(sch.meta.copy()).cuda()
        scr = torch.empty(max(4, sch.scratch_bytes), dtype=torch.uint8, device="cuda")
        att = lambda: aqp.paged_attention(params, desc, cache, q, bt, sch.meta, md, ks, vs, scr, scr.numel(), out)
        for _ in range(3):
            att()
        att_ms = timed(att, args.reps, key="attention")
        parts = {}
        qlens = b.query_start_loc[1:] - b.query_start_loc[:-1]
        if (qlens == 1).any() and (qlens > 1).any():
            # a mixed batch: its decode and its prefill sequences each alone, same inputs and cache
            for kind, sel in (("decode_only", qlens == 1), ("prefill_only", qlens > 1)):
                idx = np.nonzero(sel)[0]
                ql = qlens[idx]
                qsl = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
                rows = torch.from_numpy(np.concatenate([np.arange(b.query_start_loc[i], b.query_start_loc[i + 1])
                                                        for i in idx])).cuda()
                qp = q[rows].contiguous()
                op = torch.empty_like(qp)
                btp = torch.from_numpy(np.ascontiguousarray(b.block_tables[idx])).cuda()
                schp = aqp.get_schedule(params, desc, np.ascontiguousarray(b.seq_lens[idx]), qsl)
                mdp = torch.from_numpy(schp.meta.copy()).cuda()
                scrp = torch.empty(max(4, schp.scratch_bytes), dtype=torch.uint8, device="cuda")
                fn = lambda: aqp.paged_attention(params, desc, cache, qp, btp, schp.meta, mdp, ks, vs, scrp,
                                                 scrp.numel(), op)
                for _ in range(3):
                    fn()
                parts[kind] = timed(fn, args.reps, key=kind)
        kvb = W.kv_read_bytes(w, per_token_head=pth) * eb
        fl = W.prefill_flops(w)
        # the oracle on the host's cores: its own cache write of the same history, then one
        # attention call over the whole batch (three when the first takes under three seconds)
        ots = []
        if not args.no_oracle:
            od = oracle.CacheDesc(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim, ofmt[desc.dtype], desc.mode)
            ocache = np.zeros(od.total_bytes, dtype=np.uint8)
            oracle.cache_write(od, ocache, kh, vh, b.slots_hist, ks, vs)
            qh = host16(q)
            while len(ots) < 3 and (not ots or ots[0] < 3.0):
                t0 = time.perf_counter()
                oracle.attention(od, ocache, qh, b.block_tables, b.seq_lens, b.query_start_loc, w.num_q_heads,
                                 causal=w.causal, window=w.window, softcap=w.softcap, k_scale=ks, v_scale=vs)
                ots.append(time.perf_counter() - t0)
            del ocache
        del kh, vh
        o_s = float(np.median(ots)) if ots else float("nan")
        row = {"workload": w.name, "kv_cache_dtype": w.kv_dtype, "attention_ms": round(att_ms, 4),
               "attention_ms_p10_p90": spread["attention"],
               "cache_write": {"tokens": n, "ms": round(cw_ms, 4), "gbs": round(cw_bytes / cw_ms / 1e6, 1),
                               "frac_of_hbm_peak": round(cw_bytes / cw_ms / 1e6 / HBM_PEAK_GBS, 4)},
               "oracle_cpu": {"attention_s": round(o_s, 3), "calls": len(ots), "cores": oracle.num_threads(),
                              "kind": "oracle"} if ots else None}
        if kvb and ots:
            row["oracle_cpu"]["decode_gbs"] = round(kvb / o_s / 1e9, 3)
        if fl and ots:
            row["oracle_cpu"]["prefill_gflops"] = round(fl / o_s / 1e9, 2)
        if kvb:
            row["decode_kv_bytes"] = kvb
            row["decode_gbs"] = round(kvb / att_ms / 1e6, 1)
            row["decode_frac_of_hbm_peak"] = round(kvb / att_ms / 1e6 / HBM_PEAK_GBS, 4)
        if fl:
            row["prefill_flops"] = fl
            row["prefill_tflops"] = round(fl / att_ms / 1e9, 1)
            row["prefill_frac_of_bf16_peak"] = round(fl / att_ms / 1e9 / BF16_PEAK_TFLOPS, 4)
        if parts:
            d_ms, p_ms = parts["decode_only"], parts["prefill_only"]
            row["alone"] = {
                "decode_only_ms": round(d_ms, 4), "decode_only_ms_p10_p90": spread["decode_only"],
                "decode_only_gbs": round(kvb / d_ms / 1e6, 1),
                "decode_only_frac_of_hbm_peak": round(kvb / d_ms / 1e6 / HBM_PEAK_GBS, 4),
                "prefill_only_ms": round(p_ms, 4), "prefill_only_ms_p10_p90": spread["prefill_only"],
                "prefill_only_tflops": round(fl / p_ms / 1e9, 1),
                "prefill_only_frac_of_bf16_peak": round(fl / p_ms / 1e9 / BF16_PEAK_TFLOPS, 4),
                "sum_of_parts_ms": round(d_ms + p_ms, 4)}
        print(json.dumps(row), flush=True)
        del cache, q, out, scr


def copy_probe(torch):
    """A plain 2 GiB device-to-device copy: the achievable read + write rate, and the calibration
    of the HBM byte counters (a copy of n bytes reads n and writes n)."""
    n = 1 << 31
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    ts = []
    for _ in range(10):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    ms = float(np.median(ts))
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "ms": round(ms, 4),
                      "GBps_read_plus_write": round(2 * n / ms / 1e6, 1)}), flush=True)


def probe_lib():
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "attention_quantized_paged_amd", "libaqp_probe.so"))
    i32, i64, P = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    lib.aqp_probe_mfma_loop.argtypes = [i32, i32, i32, i32, P, P]
    lib.aqp_probe_gather.argtypes = [P, P, i64, i32, i32, i32, P, P]
    lib.aqp_probe_mfma_chain.argtypes = [i32, i32, i32, P, P]
    lib.aqp_probe_mfma32_layout.argtypes = [P, P, P, P]
    lib.aqp_probe_lds_read.argtypes = [i32, i32, i32, P, P]
    lib.aqp_probe_stage.argtypes = [P, P, i64, i32, i32, i32, i32, P, P]
    lib.aqp_probe_xcc.argtypes = [i32, P, P]
    lib.aqp_probe_mfma_valu.argtypes = [i32, i32, i32, i32, i32, P, P]
    return lib


def mfma_valu_probe(torch):
    """Cycles per 32x32x16 MFMA when each is followed by nv independent fp32 multiply-adds, at one
    wave per SIMD (96 KB of LDS per work-group of 4 waves) and at two: whether a wave's vector ALU
    instructions run under its own MFMAs."""
    lib = probe_lib()
    cus = lib.aqp_probe_cu_count()
    st = torch.cuda.current_stream().cuda_stream
    for wps, lds in ((1, 96 * 1024), (2, 64 * 1024)):
        blocks = cus * wps
        out = torch.zeros(blocks * 4 * 5, dtype=torch.int64, device="cuda")
        for nacc in (1, 2):
            for nv in (0, 4, 8, 12, 16, 24):
                iters = 200
                launch = lambda: lib.aqp_probe_mfma_valu(nv, nacc, blocks, iters, lds, out.data_ptr(), st)
                ms, clk, cyc = _clock_and_time(torch, launch, 3, out)
                per = float(np.median(cyc)) / (iters * 8 * nacc)
                print(json.dumps({"mfma_valu": "32x32x16 bf16 + fp32 fma", "waves_per_simd": wps, "chains": nacc,
                                  "fma_per_mfma": nv, "cycles_per_mfma": round(per, 2), "clock_mhz": round(clk, 1)}),
                      flush=True)


def xcc_probe(torch):
    """The die (XCD) each work-group of a launch runs on, as the launch order maps them."""
    lib = probe_lib()
    st = torch.cuda.current_stream().cuda_stream
    for blocks in (64, 4096):
        out = torch.full((blocks,), -1, dtype=torch.int32, device="cuda")
        assert lib.aqp_probe_xcc(blocks, out.data_ptr(), st) == 0
        torch.cuda.synchronize()
        x = out.cpu().numpy()
        rr = bool(np.all(x == np.arange(blocks) % 8))
        print(json.dumps({"xcc_probe_blocks": blocks, "first_32": x[:32].tolist(), "round_robin_mod_8": rr,
                          "counts": np.bincount(x[x >= 0], minlength=8).tolist()}), flush=True)


def stage_probe(torch):
    """Rates of the ways of staging 1 KB pages into LDS (direct global -> LDS copies one at a time
    and in batches, plain register loads, register loads plus LDS writes) at the prefill's occupancy (one or two
    work-groups of 4 waves per CU), from an L2-sized buffer (4 MB, the prefill's shared K and V)
    and from a 2 GiB one (HBM)."""
    lib = probe_lib()
    cus = lib.aqp_probe_cu_count()
    st = torch.cuda.current_stream().cuda_stream
    for label, nbytes in (("4MB", 4 << 20), ("2GiB", 2 << 30)):
        buf = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
        rng = np.random.default_rng(7)
        npg = nbytes // 1024
        # every wave reads 256 pages: sequential runs (as the prefill's 1 KB copies of consecutive
        # rows), the runs in random order
        runs = rng.permutation(npg // 16)
        for wgs in (1, 2):
            blocks = wgs * cus
            total = blocks * 4 * 256
            pg = (runs[np.arange(total // 16) % runs.size][:, None] * 16 + np.arange(16)[None, :]).reshape(-1)[:total]
            pages = (pg.astype(np.int64) * 1024)
            assert pages.min() >= 0 and pages.max() + 1024 <= nbytes
            pd = torch.from_numpy(pages).cuda()
            out = torch.empty(blocks * 256, dtype=torch.int32, device="cuda")
            for mode, mname in ((0, "global_load_lds"), (1, "register"), (2, "register+ds_write"),
                                (3, "global_load_lds_batched"), (4, "global_load_lds_window+lds_read"),
                                (5, "global_load_lds_window")):
                if mode >= 4 and pages.size * 1024 > nbytes:
                    continue  # (these modes read the wave's pages consecutively from the buffer's start)
                for inflight in (4, 8, 12):
                    lds = (96 if wgs == 1 else 80) * 1024
                    call = lambda: lib.aqp_probe_stage(buf.data_ptr(), pd.data_ptr(), pages.size, mode, inflight, blocks,
                                                       lds, out.data_ptr(), st)
                    assert call() == 0
                    torch.cuda.synchronize()
                    ms = timed_flushed(torch, call, 10)[0] if label == "2GiB" else _timed_plain(torch, call, 20)
                    print(json.dumps({"stage": mname, "source": label, "wgs_per_cu": wgs, "pages_in_flight_per_wave": inflight,
                                      "bytes": int(pages.size) * 1024, "ms": round(ms, 4),
                                      "GBps": round(pages.size * 1024 / ms / 1e6, 1)}), flush=True)
        del buf


def _timed_plain(torch, fn, reps):
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fn()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def _clock_and_time(torch, launch, reps, out):
    """Mean milliseconds per launch over reps launches, and the median shader clock (MHz) the waves
    of the last launch ran at (s_memtime cycles over s_memrealtime's 100 MHz ticks)."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(2):
        assert launch() == 0
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        launch()
    e1.record()
    torch.cuda.synchronize()
    o = out.view(-1, 5).cpu().numpy().astype(np.int64)
    clk = float(np.median((o[:, 2] - o[:, 1]) / np.maximum(o[:, 4] - o[:, 3], 1) * 100.0))
    cyc = o[:, 2] - o[:, 1]
    return e0.elapsed_time(e1) / reps, clk, cyc


def lds_probe(torch):
    """The result layout of v_mfma_f32_32x32x16_bf16 (checked against a host product), then the LDS
    read rate in bytes per clock per CU for 16-byte reads and 8-bit transposed reads, at one and
    two waves per SIMD."""
    lib = probe_lib()
    st = torch.cuda.current_stream().cuda_stream
    rng = np.random.default_rng(7)
    A = rng.integers(-4, 5, size=(32, 16)).astype(np.float32)
    B = rng.integers(-4, 5, size=(16, 32)).astype(np.float32)
    av = np.zeros((64, 8), np.float32)
    bv = np.zeros((64, 8), np.float32)
    for l in range(64):
        for j in range(8):
            av[l, j] = A[l % 32, 8 * (l // 32) + j]
            bv[l, j] = B[8 * (l // 32) + j, l % 32]
    C = A @ B
    want = np.zeros((64, 16), np.float32)
    for l in range(64):
        for i in range(16):
            want[l, i] = C[8 * (i // 4) + 4 * (l // 32) + (i % 4), l % 32]
    a_d, b_d = torch.from_numpy(av).cuda(), torch.from_numpy(bv).cuda()
    o_d = torch.zeros(64 * 16, dtype=torch.float32, device="cuda")
    assert lib.aqp_probe_mfma32_layout(a_d.data_ptr(), b_d.data_ptr(), o_d.data_ptr(), st) == 0
    got = o_d.view(64, 16).cpu().numpy()
    print(json.dumps({"mfma32x32x16_layout": "A: lane l row l%32, k 8(l/32)..+7; B: lane l col l%32, same k; "
                                             "C reg i of lane l: row 8(i/4) + 4(l/32) + i%4, col l%32",
                      "matches": bool(np.array_equal(got, want))}), flush=True)
    cus = lib.aqp_probe_cu_count()
    for kind, name, bytes_per_read in ((0, "ds_read_b128", 1024), (1, "ds_read_b64_tr_b8", 512)):
        for wpc in (4, 8):
            blocks = wpc // 4 * cus
            iters = 20000
            out = torch.zeros(blocks * 4 * 5, dtype=torch.int64, device="cuda")
            ms, clk, cyc = _clock_and_time(torch, lambda: lib.aqp_probe_lds_read(kind, blocks, iters, out.data_ptr(), st),
                                           3, out)
            # bytes per CU per clock over the waves' own loop cycles (median wave)
            per_cu = wpc * iters * 8 * bytes_per_read / float(np.median(cyc))
            print(json.dumps({"lds_read": name, "waves_per_cu": wpc, "bytes_per_clk_per_cu": round(per_cu, 1),
                              "shader_clock_mhz": round(clk, 1), "ms": round(ms, 4)}), flush=True)


def mfma_probe(torch):
    """The vendor library's large bf16 GEMM, then hand-written loops of independent bf16 MFMAs on
    every SIMD in two shapes: TFLOP/s, and the shader clock the waves ran at (their s_memtime
    cycles over s_memrealtime's 100 MHz ticks), so the rate can be set against the peak at that
    clock as well as against the nominal 2.4 GHz."""
    n = 8192
    a = torch.randn((n, n), device="cuda").to(torch.bfloat16)
    b = torch.randn((n, n), device="cuda").to(torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        torch.matmul(a, b)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 10
    tf = 2 * n ** 3 / ms / 1e9
    print(json.dumps({"gemm": f"bf16 {n}x{n}x{n} torch.matmul", "ms": round(ms, 4), "tflops": round(tf, 1),
                      "frac_of_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4)}), flush=True)
    del a, b
    lib = probe_lib()
    cus = lib.aqp_probe_cu_count()
    st = torch.cuda.current_stream().cuda_stream
    for nacc in (1, 2):
        for wpc in (4, 8):
            blocks = wpc // 4 * cus
            iters = 2000
            out = torch.zeros(blocks * 4 * 5, dtype=torch.int64, device="cuda")
            ms, clk, cyc = _clock_and_time(torch, lambda: lib.aqp_probe_mfma_chain(nacc, blocks, iters, out.data_ptr(), st),
                                           3, out)
            n_mfma = iters * 8 * nacc
            print(json.dumps({"mfma_chain": f"v_mfma_f32_32x32x16_bf16, {nacc} dependent chain(s) per wave, "
                                            f"{wpc} waves per CU", "shader_clock_mhz": round(clk, 1),
                              "simd_cycles_per_mfma": round(float(np.median(cyc)) / (wpc // 4) / n_mfma, 2),
                              "ms": round(ms, 4)}), flush=True)
    for shape, nacc, flops_per in ((16, 8, 16384), (16, 16, 16384), (32, 4, 32768), (32, 8, 32768)):
        for wpc in (4, 8, 16):  # waves per CU: 1, 2 and 4 per SIMD
            iters = 40000 // nacc * (16 if shape == 16 else 8)
            blocks = wpc // 4 * cus
            out = torch.zeros(blocks * 4 * 5, dtype=torch.int64, device="cuda")
            for _ in range(3):
                assert lib.aqp_probe_mfma_loop(shape, nacc, blocks, iters, out.data_ptr(), st) == 0
            torch.cuda.synchronize()
            e0.record()
            for _ in range(5):
                lib.aqp_probe_mfma_loop(shape, nacc, blocks, iters, out.data_ptr(), st)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / 5
            tf = blocks * 4 * iters * nacc * flops_per / ms / 1e9
            o = out.view(-1, 5).cpu().numpy().astype(np.int64)
            clk_mhz = float(np.median((o[:, 2] - o[:, 1]) / np.maximum(o[:, 4] - o[:, 3], 1) * 100.0))
            # cycles one MFMA occupies its SIMD at this rate and clock
            cyc = (4 * cus * clk_mhz * 1e6) / (tf * 1e12 / flops_per)
            print(json.dumps({"mfma_loop": f"independent {'v_mfma_f32_16x16x32_bf16' if shape == 16 else 'v_mfma_f32_32x32x16_bf16'}"
                                           f", {nacc} accumulators, {wpc} waves per CU", "cus": cus,
                              "ms": round(ms, 4), "tflops": round(tf, 1),
                              "frac_of_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4),
                              "shader_clock_mhz": round(clk_mhz, 1),
                              "frac_of_peak_at_that_clock": round(tf / (BF16_PEAK_TFLOPS * clk_mhz / 2400.0), 4),
                              "simd_cycles_per_mfma": round(cyc, 2)}), flush=True)


def gather_probe(torch, aqp, W):
    """Plain 16-byte vector loads of the decode batch's K and V pages (2 KB each at head_dim 128,
    block 16, one-byte codes), in the decode's order: per (sequence, KV head), block by block, the
    K page then the V page; each wave a contiguous run of that list. Medians with a 1 GiB read
    before each repetition. The bytes are exactly the decode's algorithmic KV bytes."""
    w = W.CFG3
    b = W.make_batch(w, with_kv=False)
    desc = aqp.cache_desc(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim, w.kv_dtype)
    page, blk, total = aqp.cache_bytes(desc)
    cache = torch.ones(total // 4, dtype=torch.float32, device="cuda")
    pages = []
    for s, L in enumerate(b.seq_lens):
        nblk = (int(L) + w.block_size - 1) // w.block_size
        for h in range(w.num_kv_heads):
            for j in range(nblk):
                base = int(b.block_tables[s, j]) * blk
                pages += [base + h * page, base + (w.num_kv_heads + h) * page]
    pages = np.array(pages, dtype=np.int64)
    assert page == 2048, "the probe is written for 2 KB pages"
    assert pages.min() >= 0 and pages.max() + page <= total
    # whole pages, as the decode reads whole 16-key tiles (the algorithmic figure counts the
    # visible keys only, about 0.4 % less)
    nbytes = int(pages.size) * page
    pd = torch.from_numpy(pages).cuda()
    lib = probe_lib()
    cus = lib.aqp_probe_cu_count()
    st = torch.cuda.current_stream().cuda_stream
    alg = W.kv_read_bytes(w, per_token_head=False)
    rows = []
    for wgs_per_cu in (2, 4, 8):
        blocks = wgs_per_cu * cus
        out = torch.empty(blocks * 256, dtype=torch.int32, device="cuda")
        for inflight in (2, 4, 8):
            call = lambda: lib.aqp_probe_gather(cache.data_ptr(), pd.data_ptr(), pages.size, page, inflight, blocks,
                                                out.data_ptr(), st)
            assert call() == 0
            torch.cuda.synchronize()
            ms, p10, p90 = timed_flushed(torch, call, 20)
            rows.append({"gather": "decode64 K/V pages, 2 KB each, plain 16-byte loads",
                         "waves_per_cu": 4 * wgs_per_cu, "pages_in_flight_per_wave": inflight,
                         "pages": int(pages.size), "bytes": int(nbytes), "ms": round(ms, 4),
                         "GBps": round(nbytes / ms / 1e6, 1), "frac_of_hbm_peak": round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4),
                         "decode_algorithmic_bytes": alg})
            print(json.dumps(rows[-1]), flush=True)
    best = max(rows, key=lambda r: r["GBps"])
    print(json.dumps({"gather_best_GBps": best["GBps"], "frac_of_hbm_peak": best["frac_of_hbm_peak"],
                      "at": {k: best[k] for k in ("waves_per_cu", "pages_in_flight_per_wave")}}), flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU: the path has no multi-GPU "
                                   "component (sharding by sequence or KV head needs no exchange)",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    torch.cuda.set_device(0)
    if args.stage_probe:
        stage_probe(torch)
        xcc_probe(torch)
        mfma_valu_probe(torch)
        return
    if args.copy_probe:
        copy_probe(torch)
        return
    if args.mfma_probe:
        mfma_probe(torch)
        return
    if args.lds_probe:
        lds_probe(torch)
        return
    import attention_quantized_paged_amd as aqp
    import workloads as W

    if args.gather_probe:
        gather_probe(torch, aqp, W)
        return
    if args.all_configs:
        run_all_configs(torch, aqp, W, args)
        return

    log(args, "[bench] setting up decode batch")
    s = setup_decode(torch, aqp, W, args)
    w = s["w"]
    kv_bytes = W.kv_read_bytes(w, per_token_head=False)
    extra = {}
    # the secondary figures first: they are not part of the timed steps, and their kernels already
    # bring the GPU toward its working clocks
    if not args.no_prefill:
        log(args, "[bench] prefill figure")
        extra["prefill"] = run_prefill(torch, aqp, W, args)
        log(args, "[bench] cache-write figure")
        extra["cache_write"] = run_cache_write(torch, aqp, W, s)
    for _ in range(args.warmup):
        decode_step(torch, aqp, s)
    torch.cuda.synchronize()
    # declared pre-load: untimed decode steps for a fixed wall time, so the timed steps run at the
    # clocks the GPU holds under this load whatever the warm-up count
    pre_steps, t0 = 0, time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < args.preload_ms:
        decode_step(torch, aqp, s)
        pre_steps += 1
    torch.cuda.synchronize()
    pre_ms = (time.perf_counter() - t0) * 1e3
    log(args, f"[bench] timing {args.steps} steps (after {args.warmup} warm-up steps and a pre-load of "
              f"{pre_steps} steps in {pre_ms:.0f} ms)")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        sch = decode_step(torch, aqp, s)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # kernel time: the same steps again, the library recording HIP events on the launch stream
    # right before the decode kernel, right after it and after the split-KV merge (timing events
    # serialise the stream, so they stay out of the step timing)
    log(args, f"[bench] timing {args.steps} attention launches")
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for ev in evs:
        for e in ev:
            e.record()  # (creates the event, so that its handle exists)
    torch.cuda.synchronize()
    for i in range(args.steps):
        decode_step(torch, aqp, s, evs[i])
    torch.cuda.synchronize()
    dec_ms = float(np.mean([e0.elapsed_time(e1) for e0, e1, _ in evs]))
    merge_ms = float(np.mean([e1.elapsed_time(e2) for _, e1, e2 in evs]))
    attn_ms = float(np.mean([e0.elapsed_time(e2) for e0, _, e2 in evs]))
    ms_per_step = elapsed / args.steps * 1e3
    value = kv_bytes * args.steps / elapsed / 1e9
    h = sch.header
    achieved = kv_bytes / (dec_ms * 1e-3) / 1e9
    result = {
        "metric": "decode KV-read HBM GB/s (% of peak) + prefill TFLOP/s, paged attn over fp8/int8 KV",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "preload": {"steps": pre_steps, "ms": round(pre_ms, 1),
                    "what": "untimed decode steps after the warm-up, for a fixed wall time, before the timed steps"},
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": len(w.seqs), "q_heads": w.num_q_heads, "kv_heads": w.num_kv_heads,
                   "head_dim": w.head_dim, "block_size": w.block_size, "kv_cache_dtype": w.kv_dtype,
                   "context": "uniform[512,8192] seeded", "kv_bytes_per_step": kv_bytes,
                   "new_tokens_per_step": int(s["b"].new_mask.sum()), "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic_from_profile(kv_bytes),
                     "kernel": "decode_kernel",
                     "kernel_ms": round(dec_ms, 4), "merge_ms": round(merge_ms, 4),
                     "launch_ms": round(attn_ms, 4),
                     "launch_frac": round(kv_bytes / (attn_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "decode_workgroups": h["num_dec_wgs"],
                     "partials": h["num_parts"]},
    }
    result.update(extra)
    if not args.no_cpu_baseline:
        log(args, "[bench] oracle CPU baseline")
        result["cpu_baseline"] = cpu_baseline(W, s)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
