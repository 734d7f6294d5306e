"""Small builders shared by the oracle pin tests (test-side only)."""
import numpy as np
import torch

import oracle

TORCH_F8 = {oracle.FMT_E4M3: torch.float8_e4m3fn, oracle.FMT_E5M2: torch.float8_e5m2}


def code_values(fmt, codes):
    """Values of codes via torch's float8 types / int8 (not via the oracle)."""
    c = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    if fmt == oracle.FMT_INT8:
        return c.view(torch.int8).to(torch.float64).numpy()
    return c.view(TORCH_F8[fmt]).to(torch.float64).numpy()


def to_bf16_bits(x64):
    """Exact fp64 -> bf16 bits (asserts exactness)."""
    t = torch.from_numpy(np.asarray(x64, dtype=np.float64))
    b = t.to(torch.bfloat16)
    assert torch.equal(b.to(torch.float64), t), "value not exactly representable in bf16"
    return b.view(torch.int16).numpy().view(np.uint16)


def random_codes(rng, fmt, shape, max_mag=None):
    """Random finite codes, optionally with |value| <= max_mag."""
    if fmt == oracle.FMT_INT8:
        lim = 127 if max_mag is None else int(max_mag)
        return rng.integers(-lim, lim + 1, size=shape).astype(np.int8).view(np.uint8)
    vals = code_values(fmt, np.arange(256))
    ok = np.isfinite(vals)
    if max_mag is not None:
        ok &= np.abs(vals) <= max_mag
    pool = np.nonzero(ok)[0].astype(np.uint8)
    return rng.choice(pool, size=shape)


def lossless_kv(rng, fmt, n_tok, hkv, d, scale, per_token_head=False):
    """K or V whose quantisation is exact: x = value(code) * scale with scale a power of two.
    With per_token_head, each row holds one element of magnitude qmax, so that the dynamic
    scale absmax / qmax equals `scale` exactly."""
    qmax = {oracle.FMT_E4M3: 448.0, oracle.FMT_E5M2: 57344.0, oracle.FMT_INT8: 127.0}[fmt]
    codes = random_codes(rng, fmt, (n_tok, hkv, d), max_mag=qmax)
    vals = code_values(fmt, codes)
    if per_token_head:
        pos = rng.integers(0, d, size=(n_tok, hkv))
        sign = np.where(rng.random((n_tok, hkv)) < 0.5, -1.0, 1.0)
        np.put_along_axis(vals, pos[..., None], (sign * qmax)[..., None], axis=2)
    x = vals * scale
    return to_bf16_bits(x), x


def contiguous_tables(seq_lens, bs):
    need = [(int(L) + bs - 1) // bs for L in seq_lens]
    mb = max(1, max(need))
    bt = np.full((len(seq_lens), mb), -1, dtype=np.int32)
    nxt = 0
    for b, n in enumerate(need):
        bt[b, :n] = np.arange(nxt, nxt + n)
        nxt += n
    return bt, nxt


def slots_for(bt, seq_lens, bs):
    out = []
    for b, L in enumerate(seq_lens):
        j = np.arange(int(L))
        out.append(bt[b, j // bs].astype(np.int64) * bs + j % bs)
    return np.concatenate(out)
