"""Parity at every configuration's full size, in the launch configuration the benchmark times
(default decode parallelism and prefill item size):
- the whole cache pool written on the GPU (the history, then the step's own tokens) equals the
  oracle's byte for byte;
- every attention output row (every query token of every sequence, every q head) is compared
  with the oracle's."""
import numpy as np
import pytest
import torch

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


@pytest.mark.parametrize("w", FULL, ids=[w.name for w in FULL])
def test_full_size_parity(aqp, w):
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
    ref, rows = r.oracle_attention()
    compare(out[rows], ref, f"{w.name} full size, every row: {len(rows)} query tokens x {w.num_q_heads} heads")
