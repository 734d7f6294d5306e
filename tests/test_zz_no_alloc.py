"""The allocation-free attention call (aqp_paged_attention_noalloc), through the C ABI: its output
equals that of aqp_paged_attention with a caller scratch buffer, bit for bit (the same kernels and
schedule; only the scratch address and the stream arrangement differ), on two calls in a row, the
first on the mixed batch (decode splits and prefill key splits: 33.5 MiB of partial results) and the
second on a smaller mixed batch, which finds the first call's partial results still in the buffer."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_common import Run, compare, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def aqp():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import attention_quantized_paged_amd as m
    return m


def _both(r, aqp):
    b = r.b
    sch = aqp.get_schedule(r.params, r.desc, b.seq_lens, b.query_start_loc)
    assert 0 < sch.scratch_bytes <= aqp.NOALLOC_SCRATCH_BYTES
    meta_dev = torch.from_numpy(sch.meta).cuda()
    q = to_dev(b.q, torch)
    bt = to_dev(b.block_tables, torch)
    scratch = torch.empty(sch.scratch_bytes, dtype=torch.uint8, device="cuda")
    ref = torch.full(q.shape, -1, dtype=torch.int16, device="cuda")
    aqp.paged_attention(r.params, r.desc, r.gcache, q, bt, sch.meta, meta_dev, b.k_scale, b.v_scale, scratch,
                        sch.scratch_bytes, ref)
    out = torch.full(q.shape, -1, dtype=torch.int16, device="cuda")  # NaN pattern: every row must be written
    aqp.paged_attention_noalloc(r.params, r.desc, r.gcache, q, bt, sch.meta, meta_dev, b.k_scale, b.v_scale, out)
    torch.cuda.synchronize()
    h = sch.header
    say(f"  scratch {sch.scratch_bytes / 2**20:.3f} MiB, decode partials {h['num_parts']}, "
        f"prefill split runs {h['num_pf_split']}")
    return out.cpu().numpy().view(np.uint16), ref.cpu().numpy().view(np.uint16)


def test_noalloc_equals_caller_scratch_two_calls(aqp):
    small = W.scaled(W.CFG4, name="mixed_int8_pth_small", seqs=((1, 1024),) * 4 + ((128, 640),))
    for w in (W.CFG4, small):
        r = Run(w, torch, aqp)
        out, ref = _both(r, aqp)
        assert np.all(np.isfinite(W.bf16_to_f32(out))), f"{w.name}: rows left unwritten"
        compare(out, ref, f"{w.name}: allocation-free call against the caller-scratch call")
        assert np.array_equal(out, ref), f"{w.name}: outputs differ"
