"""GPU parity of the MoE learner calls against the oracle.

mxfp8_quantize_batched and mxfp8_quantize_gather must equal the oracle's
quantize (per matrix / of the gathered, zero-padded rows) bit for bit;
mxfp8_grouped_gemm_wgrad must equal, per group, the oracle's GEMM over the
group's token columns within 1e-4 * sum|ab| (+ bf16 rounding); an empty group
must give exact zeros.  The expert data-gradient path (weights quantized
along N per expert, repacked, grouped GEMM) is checked end to end.
"""
import numpy as np
import pytest

import workloads as wl
from conftest import sample_rows, to_dev, to_host

pytestmark = pytest.mark.gpu


def _say(*a):
    print("moe-train case:", *a, flush=True)


@pytest.mark.parametrize("batch,rows,cols", [(3, 64, 96), (2, 96, 160), (4, 1536, 2048), (8, 2048, 768)])
@pytest.mark.parametrize("axis", [0, 1])
def test_quantize_batched_matches_per_matrix(mx, oracle_mod, batch, rows, cols, axis):
    _say("batched", batch, rows, cols, axis)
    rng = np.random.default_rng(batch + rows + cols + axis)
    x = wl.normal_bf16(rng, (batch, rows, cols), std=0.02)
    q, s = mx.quantize_batched(to_dev(x), axis)
    qh, sh = to_host(q), to_host(s)
    for b in range(batch):
        rq, rs = oracle_mod.quantize(x[b], axis)
        assert np.array_equal(qh[b], rq) and np.array_equal(sh[b], rs), b


def _routing(seed, tokens, experts, topk):
    rng = np.random.default_rng(seed)
    route = wl.zipf_topk_routing(rng, tokens, experts, topk)
    offsets, row_token, counts = wl.group_layout(route, experts)
    return rng, offsets, row_token, counts


@pytest.mark.parametrize("tokens,experts,topk,hidden", [(64, 8, 2, 64), (512, 16, 4, 256), (8192, 128, 8, 2048)])
def test_quantize_gather_matches_gathered_quantize(mx, oracle_mod, tokens, experts, topk, hidden):
    _say("gather", tokens, experts, topk, hidden)
    rng, offsets, row_token, _ = _routing(tokens + experts, tokens, experts, topk)
    x = wl.normal_bf16(rng, (tokens, hidden))
    idx = row_token.copy()
    if idx.size > 8:
        idx[3] = tokens + 5          # out of range -> zero row, never read
        idx[5] = -7
    q, s = mx.quantize_gather(to_dev(x), to_dev(idx))
    gathered = np.zeros((idx.size, hidden), np.uint16)
    ok = (idx >= 0) & (idx < tokens)
    gathered[ok] = x[idx[ok]]
    rq, rs = oracle_mod.quantize(gathered, 1)
    assert np.array_equal(to_host(q), rq) and np.array_equal(to_host(s), rs)


def _check_wgrad(oracle_mod, c_dev, aq, as_, bq, bs, offsets, out_dtype, rows=None):
    G = len(offsets) - 1
    for g in range(G):
        lo, hi = int(offsets[g]), int(offsets[g + 1])
        cg = c_dev[g]
        if hi == lo:
            assert np.all(cg == 0), g
            continue
        A, As = np.ascontiguousarray(aq[:, lo:hi]), np.ascontiguousarray(as_[:, lo // 32:hi // 32])
        B, Bs = np.ascontiguousarray(bq[:, lo:hi]), np.ascontiguousarray(bs[:, lo // 32:hi // 32])
        c_ref, c_abs = oracle_mod.gemm(A, As, B, Bs, rows=rows)
        got = cg if rows is None else cg[rows]
        ok, worst = oracle_mod.gemm_bound_ok(got, c_ref, c_abs, out_dtype)
        assert ok, (g, worst)


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_wgrad_small_ragged_with_empty_group(mx, oracle_mod, out):
    import torch
    _say("wgrad small", out)
    rng = np.random.default_rng(17)
    T, M, N = 384, 200, 300
    offsets = np.array([0, 32, 32, 224, 384], np.int32)      # group 1 empty
    dy = wl.normal_bf16(rng, (T, M), std=2.0 ** -10)
    x = wl.normal_bf16(rng, (T, N))
    aq, as_ = mx.quantize(to_dev(dy), 0)                      # [M][T]
    bq, bs = mx.quantize(to_dev(x), 0)                        # [N][T]
    dt = torch.float32 if out == "f32" else torch.bfloat16
    c = mx.grouped_gemm_wgrad(aq, as_, bq, bs, to_dev(offsets), dt)
    torch.cuda.synchronize()
    ch = to_host(c) if out == "f32" else wl.bf16_bits_to_f32(to_host(c))
    _check_wgrad(oracle_mod, ch, to_host(aq), to_host(as_), to_host(bq), to_host(bs), offsets, out)


@pytest.mark.parametrize("proj,M,N", [("down", 2048, 768), ("gate_up", 1536, 2048)])
def test_wgrad_moe_full_config_sampled(mx, oracle_mod, proj, M, N):
    """The Qwen3-30B-A3B experts' weight gradients at the MoE config's size:
    8192 tokens, Zipf(1.1) top-8 routing over 128 experts, groups padded to
    32 (T = 67,616 token rows).  down: dW_g[2048 x 768] = dY_g^T h_g;
    gate_up: dW_g[1536 x 2048] = dY_g^T X_g.  Every expert's gradient is
    checked on 256 of its M rows (one in every 256-row tile)."""
    import torch
    _say("wgrad moe", proj)
    rng, offsets, row_token, counts = _routing(3, 8192, 128, 8)
    T = int(offsets[-1])
    real = row_token >= 0
    dy = np.zeros((T, M), np.uint16)
    dy[real] = wl.normal_bf16(rng, (int(real.sum()), M), std=2.0 ** -10)
    h = np.zeros((T, N), np.uint16)
    h[real] = wl.normal_bf16(rng, (int(real.sum()), N))
    aq, as_ = mx.quantize(to_dev(dy), 0)
    bq, bs = mx.quantize(to_dev(h), 0)
    c = mx.grouped_gemm_wgrad(aq, as_, bq, bs, to_dev(offsets), torch.float32)
    torch.cuda.synchronize()
    ch = to_host(c)
    del c
    rows = sample_rows(M, 256, 256, 38)
    _check_wgrad(oracle_mod, ch, to_host(aq), to_host(as_), to_host(bq), to_host(bs), offsets, "f32", rows=rows)


def test_dgrad_through_transposed_expert_weights(mx, oracle_mod):
    """dX = dH W_g per expert: W_g quantized along N (batched axis 0), repacked,
    grouped GEMM -- against the oracle's grouped GEMM on the same grids."""
    import torch
    _say("dgrad")
    G, N, K = 8, 256, 512
    rng, offsets, row_token, _ = _routing(5, 256, G, 2)
    Mt = int(offsets[-1])
    w = wl.normal_bf16(rng, (G, N, K), std=0.02)             # forward weights [N][K]
    wtq, wts = mx.quantize_batched(to_dev(w), 0)             # [G][K][N]
    packed = mx.repack(wtq, wts)
    dh = np.zeros((Mt, N), np.uint16)
    real = row_token >= 0
    dh[real] = wl.normal_bf16(rng, (int(real.sum()), N), std=2.0 ** -10)
    aq, as_ = mx.quantize(to_dev(dh), 1)
    c = mx.grouped_gemm(aq, as_, packed, to_dev(offsets), torch.float32)
    torch.cuda.synchronize()
    c_ref, c_abs, grp = oracle_mod.grouped_gemm(to_host(aq), to_host(as_), to_host(wtq), to_host(wts), offsets)
    inside = grp >= 0
    ok, worst = oracle_mod.gemm_bound_ok(to_host(c)[inside], c_ref[inside], c_abs[inside], "f32")
    assert ok, worst


def _pad128(offsets):
    sizes = np.diff(np.asarray(offsets, np.int64))
    return np.concatenate([[0], np.cumsum(-(-sizes // 128) * 128)]).astype(np.int32)


# (8192, 128, 8, 2048): the MoE learner's dY, an input above the nontemporal-load threshold
@pytest.mark.parametrize("tokens,experts,topk,cols", [(64, 8, 2, 64), (512, 16, 4, 256), (8192, 128, 8, 768),
                                                      (8192, 128, 8, 2048)])
@pytest.mark.parametrize("row_grid", [True, False])
def test_quantize_dual_grouped_matches_oracle(mx, oracle_mod, tokens, experts, topk, cols, row_grid):
    """mxfp8_quantize_dual_grouped: the row grid equals quantize(x, 1) and the
    regrouped token-blocked grid equals the oracle's quantize of the regrouped
    matrix, pads included (the outputs are filled with 0xFF first, so pads must
    be written), bit for bit."""
    import torch
    _say("dual grouped", tokens, experts, topk, cols, row_grid)
    rng, offsets, row_token, _ = _routing(tokens + cols, tokens, experts, topk)
    T = int(offsets[-1])
    x = np.zeros((T, cols), np.uint16)
    real = row_token >= 0
    x[real] = wl.normal_bf16(rng, (int(real.sum()), cols), outlier_frac=0.01)
    dst = _pad128(offsets)
    rows_out = int(dst[-1]) + 64                       # trailing rows in no group
    xd = to_dev(x)
    q_col = torch.full((cols, rows_out), 0xFF, dtype=torch.uint8, device=xd.device)
    s_col = torch.full((cols, rows_out // 32), 0xFF, dtype=torch.uint8, device=xd.device)
    q_row = s_row = None
    if row_grid:
        q_row = torch.full((T, cols), 0xFF, dtype=torch.uint8, device=xd.device)
        s_row = torch.full((T, cols // 32), 0xFF, dtype=torch.uint8, device=xd.device)
    mx.quantize_dual_grouped_into(xd, to_dev(offsets), to_dev(dst), q_col, s_col, q_row, s_row)
    torch.cuda.synchronize()
    rq, rs = oracle_mod.quantize_grouped_axis0(x, offsets, dst, rows_out)
    assert np.array_equal(to_host(q_col), rq) and np.array_equal(to_host(s_col), rs)
    if row_grid:
        rq1, rs1 = oracle_mod.quantize(x, 1)
        assert np.array_equal(to_host(q_row), rq1) and np.array_equal(to_host(s_row), rs1)


def test_quantize_dual_grouped_malformed_tables_stay_in_bounds(mx, oracle_mod):
    """Misaligned, overlapping and out-of-range offsets are clamped on the
    device: the call completes, the row grid is unaffected, and the blocks of
    the well-formed groups land where the oracle puts them."""
    import torch
    _say("dual grouped malformed")
    rng = np.random.default_rng(9)
    x = wl.normal_bf16(rng, (256, 64))
    # group 1 runs backwards (empty after clamping), group 2 starts off a block
    # boundary, group 3's destination is misaligned, group 4 lies past the end;
    # no destination range overlaps group 0's, whose result is therefore fixed
    src = np.array([0, 64, 48, 160, 256, 10 ** 6], np.int32)
    dst = np.array([0, 128, 100, 300, 2 ** 30, 7], np.int32)
    rows_out = 512
    q_row, s_row, q_col, s_col = mx.quantize_dual_grouped(to_dev(x), to_dev(src), to_dev(dst), rows_out)
    torch.cuda.synchronize()
    rq1, rs1 = oracle_mod.quantize(x, 1)
    assert np.array_equal(to_host(q_row), rq1) and np.array_equal(to_host(s_row), rs1)
    # group 0 (rows 0..63 -> 0..63) is well formed
    rq0, rs0 = oracle_mod.quantize(x, 0)
    assert np.array_equal(to_host(q_col)[:, 0:64], rq0[:, 0:64])
    assert np.array_equal(to_host(s_col)[:, 0:2], rs0[:, 0:2])


@pytest.mark.parametrize("tokens,experts,topk,M,N,out", [(512, 16, 4, 256, 320, "f32"),
                                                        (2048, 128, 8, 2048, 768, "f32"),
                                                        (512, 16, 4, 192, 256, "bf16")])
def test_wgrad_aligned_groups_match_oracle(mx, oracle_mod, tokens, experts, topk, M, N, out):
    """Weight gradients over the regrouped token-blocked grids (every group
    starting and ending on a multiple of 128 tokens, T % 128 == 0): the GEMM's
    aligned path against the oracle per group, and against the same gradients
    computed over the 32-padded grids (same exact values: pads add zeros)."""
    import torch
    _say("wgrad aligned", tokens, experts, topk, M, N, out)
    rng, offsets, row_token, _ = _routing(tokens + M, tokens, experts, topk)
    T = int(offsets[-1])
    real = row_token >= 0
    dy = np.zeros((T, M), np.uint16)
    dy[real] = wl.normal_bf16(rng, (int(real.sum()), M), std=2.0 ** -10)
    h = np.zeros((T, N), np.uint16)
    h[real] = wl.normal_bf16(rng, (int(real.sum()), N))
    dst = _pad128(offsets)
    T128 = int(dst[-1])
    od, dd = to_dev(offsets), to_dev(dst)
    _, _, aq, as_ = mx.quantize_dual_grouped(to_dev(dy), od, dd, T128, row_grid=False)
    _, _, bq, bs = mx.quantize_dual_grouped(to_dev(h), od, dd, T128, row_grid=False)
    dt = torch.float32 if out == "f32" else torch.bfloat16
    c = mx.grouped_gemm_wgrad(aq, as_, bq, bs, dd, dt)
    torch.cuda.synchronize()
    ch = to_host(c.float()) if out == "bf16" else to_host(c)
    rows = None if M * N <= 256 * 320 else np.sort(rng.choice(M, 24, replace=False))
    _check_wgrad(oracle_mod, ch, to_host(aq), to_host(as_), to_host(bq), to_host(bs), dst, out, rows=rows)
    # the same gradients over the 32-padded grids, against one reference
    a32, s32 = oracle_mod.quantize(dy, 0)
    b32, t32 = oracle_mod.quantize(h, 0)
    _check_wgrad(oracle_mod, ch, a32, s32, b32, t32, offsets, out, rows=rows)


@pytest.mark.parametrize("tokens,experts,topk,hidden", [(64, 8, 2, 64), (512, 16, 4, 288), (8192, 128, 8, 2048)])
def test_quantize_gather_packed_matches_oracle_pack(mx, oracle_mod, tokens, experts, topk, hidden):
    """mxfp8_quantize_gather_packed: the packed layout of the gathered,
    zero-padded rows (out-of-range indices included) is exactly the oracle's
    pack of its quantize along K (the small cases; padding rows and blocks
    included, the buffers filled with 0xEE first) and, at the MoE layer's
    size, exactly mxfp8_repack of mxfp8_quantize_gather's grid."""
    import torch
    _say("gather packed", tokens, experts, topk, hidden)
    rng, offsets, row_token, _ = _routing(tokens + experts + 1, tokens, experts, topk)
    x = wl.normal_bf16(rng, (tokens, hidden), outlier_frac=0.01)
    idx = row_token.copy()
    if idx.size > 8:
        idx[3] = tokens + 5
        idx[5] = -7
    R = idx.size
    xd, idd = to_dev(x), to_dev(idx)
    out = mx.PackedWeight(torch.full((mx.packed_bytes(1, R, hidden, 0),), 0xEE, dtype=torch.uint8, device=xd.device),
                          torch.full((mx.packed_bytes(1, R, hidden, 1),), 0xEE, dtype=torch.uint8, device=xd.device),
                          1, R, hidden)
    mx.quantize_gather_packed_(xd, idd, out)
    torch.cuda.synchronize()
    if R * hidden <= 1 << 22:
        gathered = np.zeros((R, hidden), np.uint16)
        ok = (idx >= 0) & (idx < tokens)
        gathered[ok] = x[idx[ok]]
        rq, rs = oracle_mod.quantize(gathered, 1)
        qp, sp = oracle_mod.pack(rq.reshape(1, R, hidden), rs.reshape(1, R, hidden // 32), 1, R, hidden)
        assert np.array_equal(to_host(out.q), qp) and np.array_equal(to_host(out.s), sp)
    else:
        q, s = mx.quantize_gather(xd, idd)
        ref = mx.repack(q, s)
        torch.cuda.synchronize()
        assert torch.equal(out.q, ref.q) and torch.equal(out.s, ref.s)


@pytest.mark.parametrize("tokens,experts,topk,cols", [(64, 8, 2, 64), (512, 16, 4, 288), (8192, 128, 8, 768),
                                                      (8192, 128, 8, 2048)])
@pytest.mark.parametrize("row_grid,col_packed", [(True, True), (False, True), (True, False)])
def test_quantize_dual_grouped_packed_matches(mx, oracle_mod, tokens, experts, topk, cols, row_grid, col_packed):
    """mxfp8_quantize_dual_grouped_packed: the regrouped token-blocked grid is
    byte for byte mxfp8_quantize_dual_grouped's canonical grid, or in the
    packed layout mxfp8_repack of it (pad blocks, trailing blocks in no group
    and the layout's padding included; outputs filled first),
    and the packed row grid (if asked for) the oracle's pack of quantize(x, 1)
    on the small cases, mxfp8_repack of the canonical row grid at the MoE
    learner's sizes."""
    import torch
    _say("dual grouped packed", tokens, experts, topk, cols, row_grid, col_packed)
    rng, offsets, row_token, _ = _routing(tokens + cols + 3, tokens, experts, topk)
    T = int(offsets[-1])
    x = np.zeros((T, cols), np.uint16)
    real = row_token >= 0
    x[real] = wl.normal_bf16(rng, (int(real.sum()), cols), outlier_frac=0.01)
    dst = _pad128(offsets)
    rows_out = int(dst[-1]) + 64
    xd, so, do = to_dev(x), to_dev(offsets), to_dev(dst)
    dev = xd.device

    def pw(n, k):
        return mx.PackedWeight(torch.full((mx.packed_bytes(1, n, k, 0),), 0xEE, dtype=torch.uint8, device=dev),
                               torch.full((mx.packed_bytes(1, n, k, 1),), 0xEE, dtype=torch.uint8, device=dev),
                               1, n, k)
    if col_packed:
        pc = pw(cols, rows_out)
    else:
        pc = (torch.full((cols, rows_out), 0xEE, dtype=torch.uint8, device=dev),
              torch.full((cols, rows_out // 32), 0xEE, dtype=torch.uint8, device=dev))
    pr = pw(T, cols) if row_grid else None
    mx.quantize_dual_grouped_packed_(xd, so, do, pc, pr)
    q_row, s_row, q_col, s_col = mx.quantize_dual_grouped(xd, so, do, rows_out)
    if col_packed:
        ref_c = mx.repack(q_col, s_col)
        torch.cuda.synchronize()
        assert torch.equal(pc.q, ref_c.q) and torch.equal(pc.s, ref_c.s)
    else:
        torch.cuda.synchronize()
        assert torch.equal(pc[0], q_col) and torch.equal(pc[1], s_col)
    if not row_grid:
        return
    if T * cols <= 1 << 22:
        rq, rs = oracle_mod.quantize(x, 1)
        qp, sp = oracle_mod.pack(rq.reshape(1, T, cols), rs.reshape(1, T, cols // 32), 1, T, cols)
        assert np.array_equal(to_host(pr.q), qp) and np.array_equal(to_host(pr.s), sp)
    else:
        ref = mx.repack(q_row, s_row)
        torch.cuda.synchronize()
        assert torch.equal(pr.q, ref.q) and torch.equal(pr.s, ref.s)


@pytest.mark.parametrize("tokens,experts,topk,M,N,out", [(512, 16, 4, 256, 320, "f32"), (512, 16, 4, 192, 256, "bf16"),
                                                        (8192, 128, 8, 1536, 2048, "f32"),
                                                        (8192, 128, 8, 2048, 768, "f32")])
def test_wgrad_packed_matches_canonical(mx, oracle_mod, tokens, experts, topk, M, N, out):
    """mxfp8_grouped_gemm_wgrad_packed over the regrouped token-blocked grids
    in the packed layout equals mxfp8_grouped_gemm_wgrad over the canonical
    grids bit for bit (every expert, an empty one included: zeros), and on the
    small cases the oracle per expert within the GEMM bound."""
    import torch
    _say("wgrad packed", tokens, experts, topk, M, N, out)
    rng, offsets, row_token, _ = _routing(tokens + M + N, tokens, experts, topk)
    offsets = offsets.copy()
    offsets[2] = offsets[1]                        # expert 1 without tokens (expert 2 takes its rows)
    Tg = int(offsets[-1])
    real = row_token >= 0
    dy = np.zeros((Tg, M), np.uint16)
    xx = np.zeros((Tg, N), np.uint16)
    dy[real] = wl.normal_bf16(rng, (int(real.sum()), M), std=2.0 ** -10)
    xx[real] = wl.normal_bf16(rng, (int(real.sum()), N))     # as the other wgrad oracle checks
    dst = _pad128(offsets)
    assert dst[2] == dst[1]
    T = int(dst[-1])
    so, do = to_dev(offsets), to_dev(dst)
    dev = so.device
    tdt = torch.float32 if out == "f32" else torch.bfloat16

    def pw(n, k):
        return mx.PackedWeight(torch.empty(mx.packed_bytes(1, n, k, 0), dtype=torch.uint8, device=dev),
                               torch.empty(mx.packed_bytes(1, n, k, 1), dtype=torch.uint8, device=dev), 1, n, k)
    pa, pb = pw(M, T), pw(N, T)
    dyd, xxd = to_dev(dy), to_dev(xx)
    mx.quantize_dual_grouped_packed_(dyd, so, do, pa)
    mx.quantize_dual_grouped_packed_(xxd, so, do, pb)
    _, _, aq, as_ = mx.quantize_dual_grouped(dyd, so, do, T, row_grid=False)
    _, _, bq, bs = mx.quantize_dual_grouped(xxd, so, do, T, row_grid=False)
    c_ref = mx.grouped_gemm_wgrad(aq, as_, bq, bs, do, tdt)
    c = torch.full((experts, M, N), 7.0, dtype=tdt, device=dev)
    mx.grouped_gemm_wgrad_packed(pa, pb, do, tdt, out=c)
    torch.cuda.synchronize()
    iv = torch.int32 if out == "f32" else torch.int16
    assert torch.equal(c.view(iv), c_ref.view(iv))
    assert bool(torch.all(c[1] == 0))
    if tokens <= 512:
        _check_wgrad(oracle_mod, to_host(c.float()) if out == "bf16" else to_host(c), to_host(aq), to_host(as_),
                     to_host(bq), to_host(bs), dst, out)
