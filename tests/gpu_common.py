"""Helpers for the GPU parity tests: run the HIP path through the C ABI and the
oracle on identical host inputs, and compare."""
import sys

import numpy as np

import oracle
import workloads

# Attention tolerances against the oracle (bf16 outputs): rel-RMS 5e-3 over all
# compared elements; max-abs 2e-2 per element wherever the reference value is below 4 in
# magnitude, where one bf16 ulp (2^-6 in [2, 4)) is finer than 2e-2. From |o| >= 4 one ulp
# is 2^-5 = 0.031 or more: there two correct roundings of nearly equal results (the kernel's
# own fp32 error, probabilities rounded to bf16 before the PV product, is a few parts in 1e3 of
# the output magnitude) can differ by one ulp, so the bound is one ulp of the reference.
MAX_ABS = 2e-2
REL_RMS = 5e-3


def bf16_ulp(x):
    a = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def element_bound(ref):
    """Per-element bound: 2e-2 where |ref| < 4, one bf16 ulp of ref (>= 2^-5) from 4 on."""
    ref = np.asarray(ref, dtype=np.float64)
    return np.where(np.abs(ref) < 4.0, MAX_ABS, np.maximum(MAX_ABS, bf16_ulp(ref)))

OFMT = {0: oracle.FMT_BF16, 1: oracle.FMT_E4M3, 2: oracle.FMT_E5M2, 3: oracle.FMT_INT8}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(a, torch):
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def bits_to_f32(u16):
    return workloads.bf16_to_f32(u16)


def compare(out_u16, ref_u16, where="", magnitude=None):
    """max-abs and relative RMS of two bf16 arrays; asserts the tolerances. `magnitude` (bf16, the
    oracle's sum_j p_j |v_j| per element) widens the per-element bound to 2^-8 of it: the
    probabilities (and, per group, the scaled values) enter the PV product as bf16, each term
    with a relative error up to 2^-9, so an output formed by cancellation of large terms carries
    an error that scales with the terms, not with the output."""
    a = bits_to_f32(out_u16).astype(np.float64)
    b = bits_to_f32(ref_u16).astype(np.float64)
    assert np.all(np.isfinite(a)), f"{where}: non-finite GPU output"
    diff = a - b
    max_abs = float(np.abs(diff).max()) if diff.size else 0.0
    rel = float(np.sqrt((diff ** 2).sum() / max((b ** 2).sum(), 1e-300))) if diff.size else 0.0
    bound = element_bound(b)
    if magnitude is not None:
        bound = np.maximum(bound, 2.0 ** -8 * bits_to_f32(magnitude).astype(np.float64))
    worst = int(np.argmax(np.abs(diff) / bound)) if diff.size else 0
    n_over_2e2 = int((np.abs(diff) > MAX_ABS).sum())
    say(f"  {where}: max_abs={max_abs:.3e} rel_rms={rel:.3e} n={diff.size} above_2e-2={n_over_2e2} "
        f"worst: gpu={a.flat[worst]:.6g} ref={b.flat[worst]:.6g}" if diff.size else f"  {where}: empty")
    assert np.all(np.abs(diff) <= bound), f"{where}: element error above 2e-2 (|o| < 4) or 1 ulp (|o| >= 4): {max_abs}"
    assert rel <= REL_RMS, f"{where}: rel_rms {rel}"
    return max_abs, rel


class Run:
    """One workload through both paths."""

    def __init__(self, w, torch, aqp, two_call_write=True, fill=0, par=0, alibi=None, sinks=None,
                 causal_per_seq=None, prefill_rows=0, prefill_kv_split=0):
        """alibi, sinks: float32 numpy arrays of one value per q head (or None); causal_per_seq:
        one flag per sequence (or None)."""
        self.w, self.torch, self.aqp = w, torch, aqp
        self.alibi, self.sinks, self.causal_per_seq = alibi, sinks, causal_per_seq
        say(f"[case] {w.name} seqs={len(w.seqs)} Hq={w.num_q_heads} Hkv={w.num_kv_heads} D={w.head_dim} "
            f"bs={w.block_size} dtype={w.kv_dtype} window={w.window} cap={w.softcap}")
        self.b = b = workloads.make_batch(w)
        self.desc = aqp.cache_desc(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim, w.kv_dtype)
        self.odesc = oracle.CacheDesc(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim,
                                      OFMT[self.desc.dtype], self.desc.mode)
        _, _, total = aqp.cache_bytes(self.desc)
        assert total == self.odesc.total_bytes
        self.ocache = np.full(total, fill, dtype=np.uint8)
        oracle.cache_write(self.odesc, self.ocache, b.k_hist, b.v_hist, b.slots_hist, b.k_scale, b.v_scale)
        self.gcache = torch.full((total,), fill, dtype=torch.uint8, device="cuda")
        k, v, s = to_dev(b.k_hist, torch), to_dev(b.v_hist, torch), to_dev(b.slots_hist, torch)
        if two_call_write:
            old = torch.from_numpy(~b.new_mask).cuda()
            new = torch.from_numpy(b.new_mask).cuda()
            for m in (old, new):
                aqp.cache_write(self.desc, self.gcache, k[m].contiguous(), v[m].contiguous(), s[m].contiguous(),
                                b.k_scale, b.v_scale)
        else:
            aqp.cache_write(self.desc, self.gcache, k, v, s, b.k_scale, b.v_scale)
        torch.cuda.synchronize()
        del k, v, s
        mb = b.block_tables.shape[1]
        dev32 = lambda a: None if a is None else torch.from_numpy(np.asarray(a, np.float32)).cuda()
        self.params = aqp.attn_params(w.num_q_heads, w.num_kv_heads, w.head_dim, mb, causal=w.causal,
                                      window=w.window, softcap=w.softcap, decode_parallelism=par,
                                      causal_per_seq=causal_per_seq, alibi_slopes=dev32(alibi), sinks=dev32(sinks),
                                      prefill_rows=prefill_rows, prefill_kv_split=prefill_kv_split)

    def cache_matches(self):
        g = self.gcache.cpu().numpy()
        bad = np.nonzero(g != self.ocache)[0]
        assert bad.size == 0, f"{bad.size} cache bytes differ, first at {bad[:8]}"

    def gpu_attention(self, calls=1, events=None):
        """Output of the last of `calls` attention calls that reuse one device copy of the schedule
        (with `events`, hipEvent_t handles, through the timed entry point)."""
        torch, aqp, b = self.torch, self.aqp, self.b
        sch = aqp.get_schedule(self.params, self.desc, b.seq_lens, b.query_start_loc)
        meta_dev = torch.from_numpy(sch.meta).cuda()
        scratch = torch.empty(max(sch.scratch_bytes, 4), dtype=torch.uint8, device="cuda")
        q = to_dev(b.q, torch)
        bt = to_dev(b.block_tables, torch)
        self.outs = []
        for _ in range(calls):
            out = torch.full(q.shape, -1, dtype=torch.int16, device="cuda")  # NaN pattern: every row must be written
            aqp.paged_attention(self.params, self.desc, self.gcache, q, bt, sch.meta, meta_dev, b.k_scale, b.v_scale,
                                scratch, sch.scratch_bytes, out, events=events)
            self.outs.append(out)
        torch.cuda.synchronize()
        self.sched = sch
        self.meta_after = meta_dev.cpu().numpy()
        return self.outs[-1].cpu().numpy().view(np.uint16)

    def oracle_magnitude(self):
        """sum_j p_j |v_j| of every output element (bf16): the oracle on a copy of its cache whose
        V codes have their sign bits cleared (int8: the absolute code, which never overflows
        under absmax / 127 scaling; fp8 and bf16: the top bit)."""
        w, od = self.w, self.odesc
        absc = self.ocache.copy()
        n = w.block_size * w.head_dim
        for blk in range(w.num_blocks):
            for h in range(w.num_kv_heads):
                o = od.page_offset(blk, 1, h)
                if self.desc.dtype == 3:
                    absc[o:o + n] = np.abs(absc[o:o + n].view(np.int8).astype(np.int16)).astype(np.uint8)
                elif self.desc.dtype == 0:
                    absc[o:o + 2 * n] = (absc[o:o + 2 * n].view(np.uint16) & 0x7FFF).view(np.uint8)
                else:
                    absc[o:o + n] &= 0x7F
        saved, self.ocache = self.ocache, absc
        try:
            return self.oracle_attention()[0]
        finally:
            self.ocache = saved

    def oracle_attention(self, seqs=None):
        """Oracle output rows of the chosen sequences (default all), on the oracle's own cache."""
        b = self.b
        idx = list(range(len(b.seq_lens))) if seqs is None else list(seqs)
        sl = b.seq_lens[idx]
        ql = (b.query_start_loc[1:] - b.query_start_loc[:-1])[idx]
        qsl = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
        rows = np.concatenate([np.arange(b.query_start_loc[i], b.query_start_loc[i + 1]) for i in idx])
        q = np.ascontiguousarray(b.q[rows])
        f64 = lambda a: None if a is None else np.asarray(a, np.float32).astype(np.float64)
        cps = None if self.causal_per_seq is None else np.asarray(self.causal_per_seq, np.int32)[idx]
        out = oracle.attention(self.odesc, self.ocache, q, b.block_tables[idx], sl, qsl, self.w.num_q_heads,
                               causal=self.w.causal, window=self.w.window, softcap=self.w.softcap,
                               k_scale=b.k_scale, v_scale=b.v_scale, causal_per_seq=cps,
                               alibi_slopes=f64(self.alibi), sinks=f64(self.sinks))
        return out, rows
