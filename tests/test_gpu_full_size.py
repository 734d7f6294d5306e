"""Parity at every configuration's full size, in the launch configuration the benchmark times
(default decode parallelism and prefill item size):
- the whole cache pool written on the GPU (the history, then the step's own tokens) equals the
  oracle's byte for byte;
- attention output rows are compared with the oracle for every decode sequence and for sampled
  prefill rows (first, middle, last and random query tokens of each prefill sequence). The oracle
  computes a sampled row as a one-query sequence that ends at the row's position over the same
  block table: under the causal mask (and window) it sees exactly the keys the row sees."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_common import Run, compare, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def aqp():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import attention_quantized_paged_amd as m
    return m


FULL = [W.CFG1, W.CFG2, W.CFG3, W.CFG4, W.CFG5A, W.CFG5B]
ROWS_PER_PREFILL_SEQ = 24


def sampled_rows(b, rng):
    """(sequence, query index) pairs: the query of every decode sequence, and up to
    ROWS_PER_PREFILL_SEQ query tokens of each prefill sequence."""
    qsl = b.query_start_loc
    picks = []
    for s in range(len(b.seq_lens)):
        ql = int(qsl[s + 1] - qsl[s])
        if ql == 1:
            picks.append((s, 0))
        elif ql > 1:
            idx = {0, ql // 2, ql - 1}
            idx |= set(int(i) for i in rng.choice(ql, size=min(ql, ROWS_PER_PREFILL_SEQ - 3), replace=False))
            picks += [(s, i) for i in sorted(idx)]
    return picks


@pytest.mark.parametrize("w", FULL, ids=[w.name for w in FULL])
def test_full_size_parity(aqp, w):
    assert w.causal, "the one-query recomputation of sampled rows relies on the causal mask"
    r = Run(w, torch, aqp)
    say(f"  {w.name}: cache pool {r.ocache.size / 1e6:.0f} MB, {len(r.b.slots_hist)} tokens written")
    r.cache_matches()
    out = r.gpu_attention()
    # every row of every query token was written (the output starts as a NaN pattern), whichever
    # work-group ran its item
    assert np.all(np.isfinite(W.bf16_to_f32(out))), f"{w.name}: output rows left unwritten"
    h = r.sched.header
    say(f"  {w.name}: decode work-groups {h['num_dec_wgs']}, partials {h['num_parts']}, "
        f"prefill items {h['num_pf_items']} of {h['pf_rows']} rows")
    b = r.b
    qsl = b.query_start_loc
    picks = sampled_rows(b, np.random.default_rng(w.seed))
    seqs = np.array([s for s, _ in picks], dtype=np.int64)
    pos1 = np.array([int(b.seq_lens[s] - (qsl[s + 1] - qsl[s]) + i + 1) for s, i in picks], dtype=np.int32)
    rows = np.array([int(qsl[s] + i) for s, i in picks], dtype=np.int64)
    ref = oracle.attention(r.odesc, r.ocache, np.ascontiguousarray(b.q[rows]), b.block_tables[seqs], pos1,
                           np.arange(len(picks) + 1, dtype=np.int32), w.num_q_heads, causal=True,
                           window=w.window, softcap=w.softcap, k_scale=b.k_scale, v_scale=b.v_scale)
    compare(out[rows], ref, f"{w.name} full size, {len(picks)} query tokens x {w.num_q_heads} heads")
