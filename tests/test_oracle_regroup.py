"""CPU pins of the oracle's regrouped token-blocked grid (oracle.regroup_rows,
oracle.quantize_grouped_axis0), written from the learner paragraph of "The
pipeline" (token-axis 32-blocks for the weight-gradient GEMM, experts' token
groups padded to 32).

What fixes them, independently of the functions' own code:
  - identity layout: the regrouped grid is exactly quantize(x, axis=0);
  - pad rows are zero rows, whose blocks the (separately pinned) quantizer
    maps to zero codes and scale code 0;
  - with group boundaries on 32-row block boundaries no block straddles two
    groups, so regrouping commutes with quantization: every column block of
    the regrouped grid equals the matching block of quantize(x, axis=0);
  - a hand-worked 2-group layout with known destination positions.
"""
import numpy as np
import pytest

import workloads as wl


def _case(seed, sizes, pad_to, cols=64):
    rng = np.random.default_rng(seed)
    src = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    dst = np.concatenate([[0], np.cumsum([-(-n // pad_to) * pad_to for n in sizes])]).astype(np.int32)
    x = wl.normal_bf16(rng, (int(src[-1]), cols), outlier_frac=0.02)
    return x, src, dst


def test_identity_layout_is_plain_axis0(oracle_mod):
    x, src, _ = _case(1, [64, 32, 0, 96], 32)
    q, s = oracle_mod.quantize_grouped_axis0(x, src, src, x.shape[0])
    rq, rs = oracle_mod.quantize(x, 0)
    assert np.array_equal(q, rq) and np.array_equal(s, rs)


def test_zero_rows_quantize_to_zero_codes_and_scale_zero(oracle_mod):
    q, s = oracle_mod.quantize(np.zeros((64, 96), np.uint16), 0)
    assert not q.any() and not s.any()


@pytest.mark.parametrize("sizes", [[32, 96, 0, 160, 64], [224], [0, 0, 32], [128, 128, 32]])
def test_regrouping_commutes_with_quantization(oracle_mod, sizes):
    x, src, dst = _case(sum(sizes) + len(sizes), sizes, 128)
    rows_out = int(dst[-1]) + 64                      # trailing rows in no group
    q, s = oracle_mod.quantize_grouped_axis0(x, src, dst, rows_out)
    rq, rs = oracle_mod.quantize(x, 0)
    assert q.shape == (x.shape[1], rows_out) and s.shape == (x.shape[1], rows_out // 32)
    covered = np.zeros(rows_out, bool)
    for g in range(len(sizes)):
        n = int(src[g + 1] - src[g])
        covered[dst[g]:dst[g] + n] = True
        assert np.array_equal(q[:, dst[g]:dst[g] + n], rq[:, src[g]:src[g + 1]])
        assert np.array_equal(s[:, dst[g] // 32:(dst[g] + n) // 32], rs[:, src[g] // 32:src[g + 1] // 32])
    assert not q[:, ~covered].any()
    assert not s[:, ~covered[::32]].any()


def test_hand_worked_two_groups(oracle_mod):
    # group 0: rows 0..31 -> 0..31; group 1: rows 32..95 -> 128..191; rows_out 256
    x = np.zeros((96, 32), np.uint16)
    x[5, 7] = 0x3F80                     # 1.0 in group 0, block 0
    x[40, 3] = 0x4000                    # 2.0 in group 1, first block -> dest row 136
    x[70, 31] = 0xC040                   # -3.0 in group 1, second block -> dest row 166
    q, s = oracle_mod.quantize_grouped_axis0(x, [0, 32, 96], [0, 128, 256], 256)
    nz = sorted(zip(*np.nonzero(q)))
    assert nz == [(3, 136), (7, 5), (31, 166)]
    # each of these blocks holds a single power-of-two multiple, which the
    # quantizer represents exactly: decode (pinned decoders) gives it back
    for (c, r), v in (((7, 5), 1.0), ((3, 136), 2.0), ((31, 166), -3.0)):
        got = oracle_mod.e4m3_decode(int(q[c, r])) * oracle_mod.e8m0_decode(int(s[c, r // 32]))
        assert got == v
    assert sorted(zip(*np.nonzero(s))) == [(3, 4), (7, 0), (31, 5)]


def test_malformed_tables_are_refused(oracle_mod):
    x = np.zeros((64, 32), np.uint16)
    with pytest.raises(AssertionError):
        oracle_mod.regroup_rows(x, [0, 64], [0, 32], 64)      # destination shorter than source
