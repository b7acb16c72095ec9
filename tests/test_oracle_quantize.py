"""Pins of the oracle's quantizer and dequantizer (CPU only).

Checked against: hand-worked blocks (tests/golden/quantize_blocks.txt), a
brute-force statement of the scale rule and of the element rounding, the
page's 8.25 bits per element, power-of-two equivariance, the max-code
invariant, axis equivalence, idempotence on quantizer outputs, and torch's
E4M3 decoder for the dequantizer.
"""
import math
import os

import numpy as np
import pytest
import torch

from workloads import bf16_bits_to_f32, f32_to_bf16_bits, normal_bf16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_blocks():
    out = []
    with open(os.path.join(GOLDEN, "quantize_blocks.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, vals, scale, codes = [t.strip() for t in line.split("|")]
            out.append((name, [int(v, 16) for v in vals.split()], int(scale, 16),
                        [int(c, 16) for c in codes.split()]))
    return out


@pytest.mark.parametrize("case", _golden_blocks(), ids=lambda c: c[0])
def test_hand_worked_blocks(oracle_mod, case):
    name, vals, scale, codes = case
    for axis in (1, 0):
        x = np.zeros(32, np.uint16)
        x[:len(vals)] = vals
        xm = x[None, :] if axis == 1 else x[:, None]
        q, s = oracle_mod.quantize(xm, axis)
        assert s.size == 1 and int(s.reshape(-1)[0]) == scale, (name, axis, hex(int(s.reshape(-1)[0])))
        fill = 0x7F if scale == 0xFF else 0x00
        expect = codes + [fill] * (32 - len(codes))
        assert q.reshape(-1).tolist() == expect, (name, axis, q.reshape(-1).tolist())


def _torch_e4m3_values():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _brute_force_block(xbits):
    """Brute-force statement of the block quantizer:
    scale code c = the unique code with 256 <= amax * 2^(127-c) < 512, or 0 if
    no code in 0..254 reaches 256 (tiny or zero blocks), 0xFF for NaN/Inf;
    element = the finite E4M3 code nearest to x * 2^(127-c) (ties to the even
    code), clamped at +-448, sign kept."""
    x = bf16_bits_to_f32(np.array(xbits, np.uint16)).astype(np.float64)
    if not np.all(np.isfinite(x)):
        return 0xFF, [0x7F] * 32
    amax = np.max(np.abs(x))
    c = 0
    for cand in range(255):
        if 256.0 <= amax * 2.0 ** (127 - cand) < 512.0:
            c = cand
            break
    vals = _torch_e4m3_values()
    finite_codes = [k for k in range(0x7F)]
    out = []
    for xv in x:
        v = xv * 2.0 ** (127 - c)
        a = abs(v)
        best = None
        for k in finite_codes:
            d = abs(vals[k] - a)
            if best is None or d < best[0] or (d == best[0] and k % 2 == 0):
                best = (d, k)
        k = 0x7E if a >= 448 else best[1]
        if math.copysign(1.0, v) < 0:
            k |= 0x80
        out.append(k)
    return c, out


def test_brute_force_tiny_blocks(oracle_mod):
    rng = np.random.default_rng(3)
    blocks = []
    for i in range(60):
        kind = i % 6
        if kind == 0:
            b = normal_bf16(rng, (32,))
        elif kind == 1:
            b = normal_bf16(rng, (32,), std=2.0 ** -130)      # BF16 subnormals
        elif kind == 2:
            b = normal_bf16(rng, (32,), std=2.0 ** 100)
        elif kind == 3:
            b = rng.integers(0, 65536, 32).astype(np.uint16)   # any bit pattern
        elif kind == 4:
            b = normal_bf16(rng, (32,))
            b[rng.integers(0, 32, 5)] = 0x8000                   # -0 entries
        else:
            b = normal_bf16(rng, (32,), std=1e-3)
            b[0] = 0x4370                                        # 240: significand 1.875
        blocks.append(b)
    for b in blocks:
        q, s = oracle_mod.quantize(b[None, :], 1)
        c, codes = _brute_force_block(b)
        assert int(s[0, 0]) == c
        assert q[0].tolist() == codes


def test_bits_per_element_is_8_25(oracle_mod):
    # The format paragraph of the page's pipeline section: 8.25 bits per element.
    x = normal_bf16(np.random.default_rng(0), (64, 256))
    for axis in (0, 1):
        q, s = oracle_mod.quantize(x, axis)
        assert (q.nbytes + s.nbytes) * 8 / x.size == 8.25


def test_max_code_invariant_and_power_of_two(oracle_mod):
    rng = np.random.default_rng(4)
    x = normal_bf16(rng, (256, 512), outlier_frac=0.01)
    x[7] = normal_bf16(rng, (512,), std=2.0 ** -128)
    q, s = oracle_mod.quantize(x, 1)
    qb = q.reshape(256, 16, 32)
    mag = (qb & 0x7F).max(axis=2)
    normal = s > 0
    assert np.all((mag[normal] >= 0x78) & (mag[normal] <= 0x7E))
    assert np.all(mag[~normal] <= 0x7E)
    assert np.all(s < 0xFF)


def test_power_of_two_equivariance(oracle_mod):
    rng = np.random.default_rng(5)
    x = normal_bf16(rng, (64, 256))
    q0, s0 = oracle_mod.quantize(x, 1)
    for k in (-20, -3, 1, 7, 40):
        xk = f32_to_bf16_bits(bf16_bits_to_f32(x) * np.float32(2.0 ** k))
        qk, sk = oracle_mod.quantize(xk, 1)
        assert np.array_equal(qk, q0)
        assert np.array_equal(sk.astype(int), s0.astype(int) + k)


def test_axis_equivalence(oracle_mod):
    rng = np.random.default_rng(6)
    x = normal_bf16(rng, (96, 160), outlier_frac=0.05)
    q0, s0 = oracle_mod.quantize(x, 0)
    q1, s1 = oracle_mod.quantize(np.ascontiguousarray(x.T), 1)
    assert np.array_equal(q0, q1) and np.array_equal(s0, s1)


@pytest.mark.parametrize("std", [1.0, 0.02, 2.0 ** -128, 2.0 ** 60])
def test_idempotence_on_quantizer_outputs(oracle_mod, std):
    rng = np.random.default_rng(7)
    x = normal_bf16(rng, (64, 512), std=std, outlier_frac=0.01)
    for axis in (0, 1):
        q, s = oracle_mod.quantize(x, axis)
        for dt in ("bf16", "f32"):
            d = oracle_mod.dequantize(q, s, 64, 512, axis, dt)
            if dt == "f32":
                d32 = d.astype(np.float32)
                back = f32_to_bf16_bits(d32)
                assert np.array_equal(bf16_bits_to_f32(back), d32)   # on the BF16 grid
                d = back
            q2, s2 = oracle_mod.quantize(d, axis)
            assert np.array_equal(q2, q) and np.array_equal(s2, s), (axis, dt)


def test_dequantize_exhaustive_against_torch_decoder(oracle_mod):
    """All 256 element codes x all 256 scale codes, fp64/fp32/bf16 outputs."""
    vals = _torch_e4m3_values()
    q = np.tile(np.arange(256, dtype=np.uint8), (256, 1))           # [scale code][elem]
    s = np.repeat(np.arange(256, dtype=np.uint8)[:, None], 256 // 32, axis=1)
    d64 = oracle_mod.dequantize(q, s, 256, 256, 1, "f64")
    ref = vals[None, :] * np.where(np.arange(256) == 255, np.nan,
                                   np.ldexp(1.0, np.arange(256) - 127))[:, None]
    assert np.array_equal(np.isnan(d64), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(d64[ok], ref[ok])
    d32 = oracle_mod.dequantize(q, s, 256, 256, 1, "f32")
    ref32 = ref.astype(np.float32)
    assert np.array_equal(d32.view(np.uint32)[ok], ref32.view(np.uint32)[ok])
    d16 = oracle_mod.dequantize(q, s, 256, 256, 1, "bf16")
    ref16 = torch.from_numpy(ref32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(d16[ok], ref16[ok])
    assert np.all((d16[~ok] & 0x7FFF) > 0x7F80)   # NaN stays NaN


def test_dequantize_axis0_orientation(oracle_mod):
    rng = np.random.default_rng(8)
    x = normal_bf16(rng, (64, 96))
    q, s = oracle_mod.quantize(x, 0)
    d0 = oracle_mod.dequantize(q, s, 64, 96, 0, "f64")
    d1 = oracle_mod.dequantize(q, s, 96, 64, 1, "f64")
    assert np.array_equal(d0, d1.T)
    rel = np.abs(d0 - bf16_bits_to_f32(x)) / (np.abs(bf16_bits_to_f32(x)) + 1e-30)
    assert np.median(rel) < 0.05
