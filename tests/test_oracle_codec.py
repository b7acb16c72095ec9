"""Pins of the oracle's scalar codecs (CPU only).

The oracle's E4M3 / E8M0 / BF16 conversions are checked against things other
than themselves: the OCP MX v1.0 anchor values (tests/golden), torch's own
float8_e4m3fn / float8_e8m0fnu / bfloat16 decoders and casts (library
routines), and an exhaustive nearest-value search over the finite E4M3 grid.
"""
import math
import os

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_anchors():
    rows = []
    with open(os.path.join(GOLDEN, "e4m3_e8m0_anchors.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            kind, code, val = line.split()
            rows.append((kind, int(code, 16), val))
    return rows


def test_anchor_values(oracle_mod):
    for kind, code, val in _read_anchors():
        got = oracle_mod.e4m3_decode(code) if kind == "e4m3" else oracle_mod.e8m0_decode(code)
        if val == "nan":
            assert math.isnan(got), (kind, hex(code))
        elif val == "-0":
            assert got == 0.0 and math.copysign(1.0, got) < 0
        else:
            assert got == float(val), (kind, hex(code), got, val)


def test_e4m3_decode_matches_torch_all_codes(oracle_mod):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle_mod.e4m3_decode_table()
    nan_ref = np.isnan(ref)
    assert np.array_equal(nan_ref, np.isnan(got))
    assert set(np.nonzero(nan_ref)[0].tolist()) == {0x7F, 0xFF}
    assert np.array_equal(ref[~nan_ref], got[~nan_ref])
    # sign of zero
    assert math.copysign(1.0, got[0x80]) < 0 and math.copysign(1.0, got[0x00]) > 0


def test_e8m0_decode_matches_torch_all_codes(oracle_mod):
    if not hasattr(torch, "float8_e8m0fnu"):
        pytest.skip("torch lacks float8_e8m0fnu")
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = np.array([oracle_mod.e8m0_decode(c) for c in range(256)])
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert np.array_equal(ref[:255], got[:255])


def test_e4m3_encode_inverts_decode(oracle_mod):
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        assert oracle_mod.e4m3_encode(oracle_mod.e4m3_decode(c)) == c, hex(c)


def _nearest_even_search(v: np.ndarray) -> np.ndarray:
    """Independent statement of saturating round-to-nearest-even onto the E4M3
    grid: search the 127 finite non-negative E4M3 values (codes 0x00..0x7E,
    increasing), pick the nearest, break ties toward the even code, and clamp
    at 448.  Sign handled separately (kept, including on zero)."""
    grid_codes = np.arange(0x7F, dtype=np.int64)
    grid = torch.tensor(grid_codes, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.all(np.diff(grid) > 0)
    a = np.abs(v)
    hi = np.searchsorted(grid, a, side="left")          # grid[hi-1] < a <= grid[hi]
    hi = np.clip(hi, 1, grid.size - 1)
    lo = hi - 1
    d_lo = a - grid[lo]
    d_hi = grid[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (grid_codes[hi] % 2 == 0))
    code = np.where(pick_hi, grid_codes[hi], grid_codes[lo])
    code = np.where(a >= grid[-1], 0x7E, code)            # saturate
    code = np.where(a == 0, 0, code)
    sign = np.signbit(v).astype(np.int64) << 7
    return (code | sign).astype(np.uint8)


def test_e4m3_encode_exhaustive_bf16_times_powers_of_two(oracle_mod):
    """Every finite BF16 value times every power of two 2^t, t in [-119, 127]
    (the range of 2^-s for scales of BF16 blocks), against the search."""
    bits = np.arange(65536, dtype=np.uint32)
    x = (bits << 16).view(np.float32).astype(np.float64)
    x = x[np.isfinite(x)]
    for t0 in range(-119, 128, 16):
        ts = np.arange(t0, min(t0 + 16, 128))
        v = (x[None, :] * np.ldexp(1.0, ts)[:, None]).reshape(-1)
        got = oracle_mod.e4m3_encode_array(v)
        ref = _nearest_even_search(v)
        bad = np.nonzero(got != ref)[0]
        assert bad.size == 0, (t0, v[bad[:5]], got[bad[:5]], ref[bad[:5]])


def test_e4m3_encode_matches_torch_cast_in_range(oracle_mod):
    rng = np.random.default_rng(1)
    v = np.concatenate([
        rng.uniform(-448, 448, 200000),
        rng.standard_normal(200000) * 2.0 ** rng.integers(-14, 8, 200000),
        np.array([0.0, -0.0, 448.0, -448.0, 2.0 ** -10, 2.0 ** -9, 3 * 2.0 ** -11]),
    ])
    v = v[np.abs(v) <= 448.0]      # torch does not saturate above 448; compare in range
    got = oracle_mod.e4m3_encode_array(v)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)


def test_e4m3_encode_special(oracle_mod):
    assert oracle_mod.e4m3_encode(float("nan")) == 0x7F
    assert oracle_mod.e4m3_encode(float("inf")) == 0x7E
    assert oracle_mod.e4m3_encode(float("-inf")) == 0xFE
    assert oracle_mod.e4m3_encode(464.0) == 0x7E          # would round to 480
    assert oracle_mod.e4m3_encode(-1000.0) == 0xFE
    assert oracle_mod.e4m3_encode(-0.0) == 0x80
    assert oracle_mod.e4m3_encode(2.0 ** -10) == 0x00      # tie between 0 and 2^-9 -> even
    assert oracle_mod.e4m3_encode(3 * 2.0 ** -10) == 0x02  # tie between 1 and 2 (x2^-9) -> even
    assert oracle_mod.e4m3_encode(7.5 * 2.0 ** -9) == 0x08  # tie 7 vs 8 (x2^-9) -> 0x08


def test_bf16_codec_matches_torch(oracle_mod):
    bits = np.arange(65536, dtype=np.uint32)
    ref = (bits << 16).view(np.float32).astype(np.float64)
    got = np.array([oracle_mod.bf16_decode(int(b)) for b in bits[::97]])
    r = ref[::97]
    fin = np.isfinite(r)
    assert np.array_equal(got[fin], r[fin])
    rng = np.random.default_rng(2)
    v = np.concatenate([rng.standard_normal(20000) * 2.0 ** rng.integers(-140, 127, 20000),
                        np.ldexp(1.0 + np.arange(0, 256) / 512.0, -130)])
    # torch rounds double -> bfloat16 through float, so compare on inputs
    # that are already floats (the only inputs the dequantizer produces).
    v32 = v.astype(np.float32).astype(np.float64)
    got32 = np.array([oracle_mod.bf16_encode(float(a)) for a in v32], dtype=np.uint16)
    ref32 = torch.from_numpy(v32.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got32, ref32)
