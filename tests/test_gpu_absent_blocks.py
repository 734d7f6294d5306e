"""Block-table entries outside the pool (negative, or >= num_blocks) name no block: the keys of
that logical block are absent and take no part in the softmax, the same reading the oracle takes;
a row left with no key and no sink writes zeros. Every address the kernels form stays inside the
pool (an absent tile is read from block 0 and masked), so these cases cannot fault.

Covered: decode, with an absent entry past a decode wave's 64th tile (one work-group per
sequence, so each of its four waves walks more than 64 tiles) and split ranges whose every key
is absent; prefill at head_dim 128 and 256, per-tensor and per-token-head codes, with key splits;
block sizes that are not a multiple of 16 (absent rows inside a tile); a cache whose unwritten
bytes are NaN codes."""
import numpy as np
import pytest

import workloads as W
from tests.gpu_common import Run, compare, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def aqp():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import attention_quantized_paged_amd as m
    return m


def _absent(r, holes):
    """Replace block-table entries (sequence, logical block) of an already written cache by entries
    outside the pool (alternately -1 and num_blocks + 3)."""
    bt = r.b.block_tables
    nb = r.w.num_blocks
    for i, (s, j) in enumerate(holes):
        assert bt[s, j] >= 0
        bt[s, j] = -1 if i % 2 == 0 else nb + 3


def test_decode_absent_blocks_past_64_tiles(aqp):
    # 6400 keys = 400 tiles; with one decode work-group each wave takes 100 of them: tile t goes to
    # wave t % 4 as its (t // 4)-th, so blocks 270 and 301 are the 68th and 76th tiles of waves 2, 1
    w = W.Workload("absent_decode_long", "fp8_e4m3", ((1, 6400), (1, 40), (1, 500)), 16, 4, 128, 16, 480,
                   seed=201)
    r = Run(w, torch, aqp, par=1, fill=0xFF)
    _absent(r, [(0, 5), (0, 270), (0, 301), (0, 399), (1, 0), (1, 1), (1, 2), (2, 7)])
    out = r.gpu_attention()
    ref, rows = r.oracle_attention()
    assert np.all(ref[1] == 0), "a sequence with no key left outputs zeros"
    compare(out[rows], ref, w.name)


@pytest.mark.parametrize("par", [0, 9, 200])
def test_decode_absent_blocks_split(aqp, par):
    w = W.Workload("absent_decode_pth_split", "fp8_per_token_head", ((1, 3000), (1, 300), (1, 1000)), 16, 4, 128,
                   16, 300, window=700, softcap=30.0, seed=202)
    r = Run(w, torch, aqp, par=par, fill=0xFF)
    # the second sequence loses every block (its split parts are all empty), the others a few
    _absent(r, [(0, 150), (0, 187), (1, 0), (1, 5), (1, 10), (1, 15), (2, 62), (2, 30)]
            + [(1, j) for j in range(1, 19) if j not in (5, 10, 15)])
    out = r.gpu_attention()
    ref, rows = r.oracle_attention()
    compare(out[rows], ref, f"{w.name} par={par}")


PREFILL = [
    W.Workload("absent_prefill_d128_pt", "fp8_e4m3", ((300, 300), (40, 200), (1, 90)), 16, 4, 128, 16, 50,
               seed=203),
    W.Workload("absent_prefill_d128_int8_pth", "int8_per_token_head", ((300, 300), (40, 200), (1, 90)), 16, 4, 128,
               16, 50, seed=204),
    W.Workload("absent_prefill_d256_e4m3", "fp8_e4m3", ((200, 200), (33, 150)), 16, 2, 256, 32, 16, seed=205),
    W.Workload("absent_prefill_d64_pg", "fp8_per_group", ((120, 120), (20, 64)), 8, 2, 64, 16, 16, seed=206),
    # block sizes that are not a multiple of 16: an absent block masks some rows of a tile only
    W.Workload("absent_prefill_bs8_d128_pth", "fp8_per_token_head", ((300, 300), (40, 200), (1, 90)), 16, 4, 128, 8,
               100, seed=207),
    W.Workload("absent_prefill_bs3_d64_pg", "int8_per_group", ((120, 120), (20, 64)), 8, 2, 64, 3, 70, seed=208),
]


@pytest.mark.parametrize("par", [0, 9])
def test_decode_absent_blocks_odd_block_size(aqp, par):
    w = W.Workload("absent_decode_bs5_pth", "int8_per_token_head", ((1, 900), (1, 50), (1, 333)), 16, 4, 128, 5, 300,
                   window=400, seed=209)
    r = Run(w, torch, aqp, par=par, fill=0xFF)
    # single 5-key blocks inside tiles, the second sequence's every block
    _absent(r, [(0, 3), (0, 100), (0, 179), (2, 0), (2, 66)] + [(1, j) for j in range(10)])
    out = r.gpu_attention()
    ref, rows = r.oracle_attention()
    assert np.all(ref[1] == 0), "a sequence with no key left outputs zeros"
    compare(out[rows], ref, f"{w.name} par={par}")


@pytest.mark.parametrize("split", [1, 3])
@pytest.mark.parametrize("w", PREFILL, ids=[w.name for w in PREFILL])
def test_prefill_absent_blocks(aqp, w, split):
    r = Run(w, torch, aqp, fill=0xFF, prefill_kv_split=split)
    bs = w.block_size
    holes = [(0, 0), (0, 3), (0, (w.seqs[0][1] - 1) // bs), (1, 1)]
    if len(w.seqs) > 2:
        holes.append((2, 2))
    _absent(r, holes)
    out = r.gpu_attention()
    ref, rows = r.oracle_attention()
    say(f"  rows with no key left: {int(np.sum(np.all(ref.reshape(len(ref), -1) == 0, axis=1)))}")
    compare(out[rows], ref, f"{w.name} split={split}")
