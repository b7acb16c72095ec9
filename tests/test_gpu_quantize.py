"""GPU parity of mxfp8_quantize / mxfp8_dequantize against the oracle.

Quantize must match bit for bit: every element byte and every scale byte.
Inputs: the seeded workloads (tiny, Qwen3-8B qkv at full size, MLP shapes),
an exhaustive sweep of every BF16 value under every scale it can meet, the
special values (zeros, -0, subnormals, ties, saturation, NaN/Inf), and ragged
shapes.  Dequantize: every (element code, scale code) pair, both dtypes.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from conftest import to_dev, to_host

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _check_quantize(mx, oracle_mod, x_bits, axis, name):
    _say("quantize", name, x_bits.shape, "axis", axis)
    q_ref, s_ref = oracle_mod.quantize(x_bits, axis)
    q, s = mx.quantize(to_dev(x_bits), axis)
    torch.cuda.synchronize()
    q, s = to_host(q), to_host(s)
    bad_s = np.argwhere(s != s_ref)
    assert bad_s.size == 0, (name, "scale mismatch at", bad_s[:5], s[tuple(bad_s[0])], s_ref[tuple(bad_s[0])])
    bad_q = np.argwhere(q != q_ref)
    assert bad_q.size == 0, (name, "element mismatch at", bad_q[:5], q[tuple(bad_q[0])], q_ref[tuple(bad_q[0])])


def _sweep_matrix():
    """Blocks that pin each scale code c in [0, 246] with a block max of BF16
    exponent field c + 8 (mantissa all ones), filled with every BF16 pattern
    whose magnitude does not exceed that max, both signs."""
    blocks = []
    for c in range(0, 247):
        E = c + 8
        amax = (E << 7) | 0x7F
        mags = np.arange(0, amax + 1, dtype=np.uint32)
        vals = np.concatenate([mags, mags | 0x8000]).astype(np.uint16)
        n = (vals.size + 30) // 31
        pad = np.zeros(n * 31, np.uint16)
        pad[:vals.size] = vals
        b = np.empty((n, 32), np.uint16)
        b[:, 0] = amax
        b[:, 1:] = pad.reshape(n, 31)
        blocks.append(b)
    return np.concatenate(blocks)


def test_quantize_exhaustive_conversion(mx, oracle_mod):
    m = _sweep_matrix()                         # [n_blocks, 32]
    rows = m.shape[0] - m.shape[0] % 64
    x = np.ascontiguousarray(m[:rows].reshape(rows // 64, 64 * 32))
    _check_quantize(mx, oracle_mod, x, 1, "exhaustive-sweep-axis1")
    # the same blocks down the columns for axis 0: column j of [32, n] is block j
    n = (m.shape[0] // 128) * 128
    x0 = np.ascontiguousarray(m[:n].T)
    _check_quantize(mx, oracle_mod, x0, 0, "exhaustive-sweep-axis0")


def _special_blocks():
    rng = np.random.default_rng(20)
    out = []
    base = wl.normal_bf16(rng, (64, 32))
    out.append(base)
    z = np.zeros((4, 32), np.uint16)
    z[1, :] = 0x8000                                        # -0 block
    z[2, 5] = 0x8000
    z[3, ::2] = 0x0001                                      # smallest subnormals
    out.append(z)
    sub = wl.normal_bf16(rng, (16, 32), std=2.0 ** -130)   # subnormal blocks
    out.append(sub)
    big = wl.normal_bf16(rng, (16, 32), std=2.0 ** 120)     # near the BF16 top
    out.append(big)
    sp = wl.normal_bf16(rng, (8, 32))
    sp[0, 3] = 0x7FC0                                       # NaN
    sp[1, 7] = 0xFF80                                       # -Inf
    sp[2, 0] = 0x7F80                                       # +Inf
    sp[3, 31] = 0x7F81                                      # signalling-NaN pattern
    sp[4, :] = 0x7F7F                                       # BF16 max everywhere
    sp[5, 0] = 0x4370; sp[5, 1:] = 0x3F80                   # 240 (significand 1.875) saturates
    sp[6, 0] = 0x4380; sp[6, 1] = 0x3F88; sp[6, 2] = 0x3F98  # ties at the E4M3 grid
    out.append(sp)
    # blocks whose max is a BF16 normal with exponent field 1..7 (below
    # 2^-119): floor(log2 amax) - 8 < -127, so the scale clamps to code 0
    # and the elements are not all below 448 * 2^-127 -- eight blocks per
    # field, the rest of each block drawn from every smaller magnitude
    lo = np.zeros((56, 32), np.uint16)
    for i, E in enumerate(range(1, 8)):
        for r in range(8):
            row = i * 8 + r
            mx_bits = (E << 7) | int(rng.integers(0, 128))
            lo[row, :] = rng.integers(0, mx_bits + 1, 32)
            lo[row, int(rng.integers(0, 32))] = mx_bits
            lo[row] |= (rng.integers(0, 2, 32) << 15).astype(np.uint16)
    out.append(lo)
    return np.concatenate(out)


def test_quantize_special_values(mx, oracle_mod):
    x = _special_blocks()                                   # [rows, 32]
    rows = x.shape[0]
    _check_quantize(mx, oracle_mod, x, 1, "special-axis1")
    xr = np.ascontiguousarray(x[: rows - rows % 32])
    _check_quantize(mx, oracle_mod, np.ascontiguousarray(xr.T), 0, "special-axis0")


def test_quantize_tiny_config(mx, oracle_mod):
    d = wl.tiny(0)
    for name in ("W", "X"):
        for axis in (1, 0):
            _check_quantize(mx, oracle_mod, d[name], axis, "tiny-" + name)


@pytest.mark.parametrize("rows,cols", [(1, 32), (3, 96), (32, 32), (33, 64), (96, 4128),
                                       (160, 200), (64, 129), (32, 1), (224, 77)])
def test_quantize_ragged(mx, oracle_mod, rows, cols):
    rng = np.random.default_rng(rows * 7919 + cols)
    x = wl.normal_bf16(rng, (rows, cols), outlier_frac=0.02)
    if cols % 32 == 0:
        _check_quantize(mx, oracle_mod, x, 1, "ragged")
    if rows % 32 == 0:
        _check_quantize(mx, oracle_mod, x, 0, "ragged")


def test_quantize_qkv_full_size(mx, oracle_mod):
    d = wl.qkv(0)
    _check_quantize(mx, oracle_mod, d["W"], 1, "qkv-W")
    _check_quantize(mx, oracle_mod, d["X"], 1, "qkv-X")


def test_quantize_mlp_shapes_both_axes(mx, oracle_mod):
    rng = np.random.default_rng(21)
    x = wl.normal_bf16(rng, (1024, 4096), outlier_frac=0.01)
    _check_quantize(mx, oracle_mod, x, 1, "mlp-X-axis1")
    _check_quantize(mx, oracle_mod, x, 0, "mlp-X-axis0")
    dy = wl.normal_bf16(rng, (512, 12288), std=2.0 ** -10)
    _check_quantize(mx, oracle_mod, dy, 0, "mlp-dY-axis0")
    w = wl.normal_bf16(rng, (4096, 1536), std=0.02)
    _check_quantize(mx, oracle_mod, w, 0, "mlp-W-axis0")


def test_quantize_deterministic_and_idempotent(mx, oracle_mod):
    rng = np.random.default_rng(22)
    x = wl.normal_bf16(rng, (256, 1024), outlier_frac=0.01)
    xd = to_dev(x)
    q0, s0 = mx.quantize(xd, 1)
    for _ in range(5):
        q1, s1 = mx.quantize(xd, 1)
        assert torch.equal(q0, q1) and torch.equal(s0, s1)
    d = mx.dequantize(q0, s0, 256, 1024, 1, torch.bfloat16)
    q2, s2 = mx.quantize(d, 1)
    assert torch.equal(q0, q2) and torch.equal(s0, s2)       # byte-for-byte re-quantization


def test_dequantize_exhaustive(mx, oracle_mod):
    q = np.tile(np.arange(256, dtype=np.uint8), (256, 1))
    s = np.repeat(np.arange(256, dtype=np.uint8)[:, None], 8, axis=1)
    for dt, tdt in (("f32", torch.float32), ("bf16", torch.bfloat16)):
        _say("dequantize exhaustive", dt)
        ref = oracle_mod.dequantize(q, s, 256, 256, 1, dt)
        got = to_host(mx.dequantize(to_dev(q), to_dev(s), 256, 256, 1, tdt))
        if dt == "f32":
            ref_b, got_b = ref.view(np.uint32), got.view(np.uint32)
            nan_r, nan_g = np.isnan(ref), np.isnan(got)
        else:
            ref_b, got_b = ref, got
            nan_r, nan_g = (ref & 0x7FFF) > 0x7F80, (got & 0x7FFF) > 0x7F80
        assert np.array_equal(nan_r, nan_g)
        bad = np.argwhere((ref_b != got_b) & ~nan_r)
        assert bad.size == 0, (dt, bad[:5])


@pytest.mark.parametrize("rows,cols", [(64, 256), (96, 100), (32, 33), (4096, 4096)])
def test_dequantize_axis0_and_axis1(mx, oracle_mod, rows, cols):
    rng = np.random.default_rng(rows + cols)
    x = wl.normal_bf16(rng, (rows, cols), outlier_frac=0.01)
    for axis in (0, 1):
        if axis == 1 and cols % 32:
            continue
        q, s = oracle_mod.quantize(x, axis)
        for dt, tdt in (("f32", torch.float32), ("bf16", torch.bfloat16)):
            _say("dequantize", rows, cols, axis, dt)
            ref = oracle_mod.dequantize(q, s, rows, cols, axis, dt)
            got = to_host(mx.dequantize(to_dev(q), to_dev(s), rows, cols, axis, tdt))
            assert np.array_equal(got.view(np.uint8), ref.view(np.uint8)), (axis, dt)


def test_quantize_many_matches_oracle(mx, oracle_mod):
    """mxfp8_quantize_many over 11 tensors (two launches: 8 + 3), ragged block
    counts (steps of 64 blocks that end inside a tensor), the special blocks
    and the exhaustive sweep among them: every output equals the oracle's
    axis-1 quantize, bit for bit."""
    rng = np.random.default_rng(91)
    xs = [wl.normal_bf16(rng, (r, c), outlier_frac=0.02) for r, c in
          [(1, 32), (3, 96), (33, 64), (96, 4128), (160, 224), (7, 2048), (2, 32)]]
    xs.insert(2, _special_blocks())
    xs.insert(5, np.ascontiguousarray(_sweep_matrix()[:50000]))
    xs += [wl.normal_bf16(rng, (513, 1056)), wl.normal_bf16(rng, (64, 64), std=1e-30)]
    _say("quantize many", len(xs))
    items = []
    for x in xs:
        r, c = x.shape
        items.append((to_dev(x), torch.full((r, c), 0xEE, dtype=torch.uint8, device="cuda"),
                      torch.full((r, c // 32), 0xEE, dtype=torch.uint8, device="cuda")))
    mx.quantize_many_(items)
    torch.cuda.synchronize()
    for i, (x, (_, q, s)) in enumerate(zip(xs, items)):
        q_ref, s_ref = oracle_mod.quantize(x, 1)
        assert np.array_equal(to_host(s), s_ref), i
        assert np.array_equal(to_host(q), q_ref), i


def _layout_target(mx, r, c, packed):
    if packed:
        return mx.PackedWeight(torch.full((mx.packed_bytes(1, r, c, 0),), 0xEE, dtype=torch.uint8, device="cuda"),
                               torch.full((mx.packed_bytes(1, r, c, 1),), 0xEE, dtype=torch.uint8, device="cuda"),
                               1, r, c)
    return (torch.full((r, c), 0xEE, dtype=torch.uint8, device="cuda"),
            torch.full((r, c // 32), 0xEE, dtype=torch.uint8, device="cuda"))


def _check_layout_target(mx, oracle_mod, x, target, what):
    r, c = x.shape
    q_ref, s_ref = oracle_mod.quantize(x, 1)
    if isinstance(target, mx.PackedWeight):
        qp_ref, sp_ref = oracle_mod.pack(q_ref.reshape(1, r, c), s_ref.reshape(1, r, c // 32), 1, r, c)
        assert np.array_equal(to_host(target.q), qp_ref), what
        assert np.array_equal(to_host(target.s), sp_ref), what
    else:
        assert np.array_equal(to_host(target[1]), s_ref), what
        assert np.array_equal(to_host(target[0]), q_ref), what


def test_quantize_many_layouts_matches_oracle(mx, oracle_mod):
    """mxfp8_quantize_many_layouts over 8 tensors, canonical and packed
    targets alternating, rows that are not multiples of 16 or 256, columns
    that are not multiples of 128, the special blocks and the exhaustive sweep
    among them: canonical entries equal the oracle's axis-1 quantize, packed
    entries the oracle's packing of it (padding rows and blocks included), bit
    for bit; buffers start as 0xEE so every byte must be written."""
    rng = np.random.default_rng(92)
    xs = [wl.normal_bf16(rng, (1, 32)), _special_blocks(), wl.normal_bf16(rng, (33, 64), outlier_frac=0.02),
          np.ascontiguousarray(_sweep_matrix()[:20000]), wl.normal_bf16(rng, (300, 320)),
          wl.normal_bf16(rng, (513, 1056)), wl.normal_bf16(rng, (17, 4128)), wl.normal_bf16(rng, (256, 128))]
    for first_packed in (True, False):
        _say("quantize many layouts, first packed", first_packed)
        items = []
        for i, x in enumerate(xs):
            r, c = x.shape
            items.append((to_dev(x), _layout_target(mx, r, c, (i % 2 == 0) == first_packed)))
        mx.quantize_many_layouts_(items)
        torch.cuda.synchronize()
        for i, (x, (_, target)) in enumerate(zip(xs, items)):
            _check_layout_target(mx, oracle_mod, x, target, (i, first_packed))


def test_quantize_many_layouts_qkv(mx, oracle_mod):
    """The qkv layer's weight into its canonical grid and its activations into
    the packed layout in one launch (the default bench step)."""
    d = wl.qkv(0)
    _say("quantize many layouts qkv")
    items = [(to_dev(d["W"]), _layout_target(mx, *d["W"].shape, False)),
             (to_dev(d["X"]), _layout_target(mx, *d["X"].shape, True))]
    mx.quantize_many_layouts_(items)
    torch.cuda.synchronize()
    for name, (_, target) in zip(("W", "X"), items):
        _check_layout_target(mx, oracle_mod, d[name], target, name)


def test_quantize_many_qkv_pair(mx, oracle_mod):
    """The qkv layer's weight and activations in one launch equal the oracle."""
    d = wl.qkv(0)
    _say("quantize many qkv")
    items = []
    for name in ("W", "X"):
        r, c = d[name].shape
        items.append((to_dev(d[name]), torch.empty((r, c), dtype=torch.uint8, device="cuda"),
                      torch.empty((r, c // 32), dtype=torch.uint8, device="cuda")))
    mx.quantize_many_(items)
    torch.cuda.synchronize()
    for name, (_, q, s) in zip(("W", "X"), items):
        q_ref, s_ref = oracle_mod.quantize(d[name], 1)
        assert np.array_equal(to_host(s), s_ref), name
        assert np.array_equal(to_host(q), q_ref), name
