"""Pins of the oracle's fp8 / int8 codec against things other than itself.

* decode: the OCP anchor values (tests/golden/ocp_fp8_anchors.txt) and torch's
  own float8_e4m3fn / float8_e5m2 types (an independent library decoder);
* encode: brute-force nearest-code search over the decode table (ties to the
  even code), torch's fp32 -> float8 casts inside the finite range, and
  numpy's rint for int8;
* saturation at 448 / 57344, sign of zero, subnormals, int8 clamp.
"""
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
FMTS = {"e4m3": oracle.FMT_E4M3, "e5m2": oracle.FMT_E5M2}
TORCH = {oracle.FMT_E4M3: torch.float8_e4m3fn, oracle.FMT_E5M2: torch.float8_e5m2}
MAXF = {oracle.FMT_E4M3: 448.0, oracle.FMT_E5M2: 57344.0}


def _anchors():
    rows = []
    with open(os.path.join(GOLDEN, "ocp_fp8_anchors.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                fmt, code, val = line.split()
                rows.append((FMTS[fmt], int(code, 16), val))
    return rows


@pytest.mark.parametrize("fmt,code,val", _anchors())
def test_decode_anchors(fmt, code, val):
    got = oracle.decode(fmt, code)
    if val == "nan":
        assert np.isnan(got)
    elif val == "-0":
        assert got == 0.0 and np.signbit(got)
    else:
        assert got == float(val)
        if float(val) == 0.0:
            assert not np.signbit(got)


@pytest.mark.parametrize("fmt", [oracle.FMT_E4M3, oracle.FMT_E5M2])
def test_decode_table_matches_torch_float8(fmt):
    tab = oracle.decode_table(fmt)
    ref = torch.arange(256, dtype=torch.uint8).view(TORCH[fmt]).to(torch.float64).numpy()
    same_nan = np.isnan(tab) == np.isnan(ref)
    assert same_nan.all()
    m = ~np.isnan(ref)
    assert np.array_equal(tab[m], ref[m])
    assert np.array_equal(np.signbit(tab[m]), np.signbit(ref[m]))


@pytest.mark.parametrize("fmt", [oracle.FMT_E4M3, oracle.FMT_E5M2])
def test_decode_table_structure(fmt):
    """Positive codes are strictly increasing and negative codes mirror them."""
    tab = oracle.decode_table(fmt)
    pos = tab[:128]
    fin = pos[np.isfinite(pos)]
    assert np.all(np.diff(fin) > 0)
    assert fin.max() == MAXF[fmt]
    for c in range(128):
        if np.isfinite(tab[c]):
            assert tab[c + 128] == -tab[c]


def test_int8_decode_is_twos_complement():
    tab = oracle.decode_table(oracle.FMT_INT8)
    assert np.array_equal(tab, np.arange(256).astype(np.uint8).view(np.int8).astype(np.float64))


def _all_bf16_times(scales):
    pats = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    pats = pats[np.isfinite(pats)]
    with np.errstate(over="ignore"):
        return np.concatenate([(pats * np.float32(s)).astype(np.float32) for s in scales])


SCALES = [1.0, 0.5, 3.7, 1.0 / 448.0, 448.0 / 3.0, 1e-3, 37.1, 2.0 ** -20, 1.0 / 57344.0 * 3.0]


def _brute_force_fp8(fmt, y):
    """Nearest finite code by search over the decode table; ties go to the code whose
    last mantissa bit is 0; beyond the largest finite value -> the largest finite value."""
    tab = oracle.decode_table(fmt)
    codes = np.array([c for c in range(128) if np.isfinite(tab[c])])
    vals = tab[codes]
    order = np.argsort(vals)
    codes, vals = codes[order], vals[order]
    a = np.abs(y.astype(np.float64))
    a_clamped = np.minimum(a, vals[-1])
    idx = np.searchsorted(vals, a_clamped)
    idx = np.clip(idx, 1, len(vals) - 1)
    lo, hi = vals[idx - 1], vals[idx]
    dlo, dhi = a_clamped - lo, hi - a_clamped
    pick_hi = (dhi < dlo) | ((dhi == dlo) & ((codes[idx] & 1) == 0))
    best = np.where(pick_hi, codes[idx], codes[idx - 1])
    best = np.where(a_clamped <= vals[0], codes[0], best)
    sign = np.signbit(y).astype(np.int64) << 7
    return (best | sign).astype(np.uint8)


@pytest.mark.parametrize("fmt", [oracle.FMT_E4M3, oracle.FMT_E5M2])
def test_encode_matches_brute_force_every_bf16_times_scale_grid(fmt):
    y = _all_bf16_times(SCALES)
    y = y[np.isfinite(y)]
    got = oracle.encode_array(fmt, y)
    ref = _brute_force_fp8(fmt, y)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(y[i]), hex(got[i]), hex(ref[i])) for i in bad[:8]]


@pytest.mark.parametrize("fmt", [oracle.FMT_E4M3, oracle.FMT_E5M2])
def test_encode_matches_torch_cast_inside_range(fmt):
    y = _all_bf16_times([1.0, 0.37, 5.1])
    y = y[np.isfinite(y) & (np.abs(y) <= MAXF[fmt])]
    got = oracle.encode_array(fmt, y)
    ref = torch.from_numpy(y).to(TORCH[fmt]).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("fmt", [oracle.FMT_E4M3, oracle.FMT_E5M2])
def test_encode_saturates_and_keeps_zero_sign(fmt):
    m = MAXF[fmt]
    maxcode = 0x7E if fmt == oracle.FMT_E4M3 else 0x7B
    for y in [m, m * 1.01, m * 4, 3.0e38, float("inf")]:
        assert oracle.encode(fmt, y) == maxcode
        assert oracle.encode(fmt, -y) == maxcode | 0x80
    assert oracle.encode(fmt, 0.0) == 0x00
    assert oracle.encode(fmt, -0.0) == 0x80
    assert oracle.encode(fmt, -1e-30) == 0x80
    assert oracle.encode(fmt, 1e-30) == 0x00


def test_encode_subnormal_ties_to_even():
    # e4m3 subnormal quantum 2^-9: 0.5 quantum ties to 0, 1.5 quanta to 2 quanta, 2.5 to 2.
    q = 2.0 ** -9
    assert oracle.encode(oracle.FMT_E4M3, 0.5 * q) == 0x00
    assert oracle.encode(oracle.FMT_E4M3, 1.5 * q) == 0x02
    assert oracle.encode(oracle.FMT_E4M3, 2.5 * q) == 0x02
    # 1.0625 lies halfway between 1.0 (0x38) and 1.125 (0x39): tie goes to 0x38
    assert oracle.encode(oracle.FMT_E4M3, 1.0625) == 0x38
    assert oracle.encode(oracle.FMT_E4M3, 1.1875) == 0x3A


def test_int8_encode_matches_rint_and_clamp():
    y = _all_bf16_times([1.0, 0.5, 1.0 / 3.0, 100.0])
    y = y[np.isfinite(y)]
    got = oracle.encode_array(oracle.FMT_INT8, y).view(np.int8)
    ref = np.clip(np.rint(y.astype(np.float64)), -128, 127).astype(np.int8)
    assert np.array_equal(got, ref)
    assert oracle.encode(oracle.FMT_INT8, 2.5) == 2
    assert oracle.encode(oracle.FMT_INT8, -2.5) == (-2) & 0xFF
    assert oracle.encode(oracle.FMT_INT8, 1000.0) == 127
    assert oracle.encode(oracle.FMT_INT8, -1000.0) == 0x80


def test_bf16_rounding_of_fp64():
    # ties to even at bf16 precision (8 significant bits)
    assert oracle.f64_to_bf16(1.0 + 2.0 ** -8) == 0x3F80
    assert oracle.f64_to_bf16(1.0 + 3 * 2.0 ** -8) == 0x3F82
    assert oracle.f64_to_bf16(1.0 + 2.0 ** -8 + 2.0 ** -30) == 0x3F81
    assert oracle.f64_to_bf16(-2.0) == 0xC000
    rng = np.random.default_rng(5)
    x = rng.standard_normal(2000) * 10.0 ** rng.integers(-30, 30, 2000)
    got = np.array([oracle.f64_to_bf16(float(v)) for v in x], dtype=np.uint16)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)
