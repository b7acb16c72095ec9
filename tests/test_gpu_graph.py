"""Library calls recorded into a HIP graph and replayed.

The sampler of "End-to-End MXFP8 RL on Blackwell" (verl blog), section "The
pipeline", sampler paragraph, rewrites its weights in place and replays
captured graphs.  The library's calls allocate nothing and never synchronize,
so a caller can record them once and replay them after every update.

Bars: every replay equals an eager run of the same calls on the same inputs
bit for bit (quantize and repack are exact; the GEMMs are deterministic), with
eager work and synchronizations between the replays; the first replay is also
checked against the oracle (quantize bit-exact, GEMM within 1e-4 * sum|ab| plus
the bf16 rounding of the output).
"""
import numpy as np
import pytest

import workloads as wl
from conftest import to_dev, to_host

pytestmark = pytest.mark.gpu


def _say(*a):
    print("graph case:", *a, flush=True)


def test_graph_replay_dense_step_matches_eager(mx, oracle_mod):
    import torch
    M, N, K = 96, 300, 320
    _say("dense", M, N, K)
    dev = torch.device("cuda:0")
    X = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    W = torch.empty((N, K), dtype=torch.bfloat16, device=dev)

    def buffers():
        return dict(xq=torch.empty((M, K), dtype=torch.uint8, device=dev),
                    xs=torch.empty((M, K // 32), dtype=torch.uint8, device=dev),
                    wq=torch.empty((N, K), dtype=torch.uint8, device=dev),
                    ws=torch.empty((N, K // 32), dtype=torch.uint8, device=dev),
                    w=mx.PackedWeight(torch.empty(mx.packed_bytes(1, N, K, 0), dtype=torch.uint8, device=dev),
                                      torch.empty(mx.packed_bytes(1, N, K, 1), dtype=torch.uint8, device=dev),
                                      1, N, K),
                    y=torch.empty((M, N), dtype=torch.bfloat16, device=dev),
                    y32=torch.empty((M, N), dtype=torch.float32, device=dev))

    def step(b):
        mx.quantize_into(W, 1, b["wq"], b["ws"])
        mx.quantize_into(X, 1, b["xq"], b["xs"])
        mx.repack_(b["wq"], b["ws"], b["w"])
        mx.gemm(b["xq"], b["xs"], b["w"], torch.bfloat16, out=b["y"])
        mx.gemm(b["xq"], b["xs"], (b["wq"], b["ws"]), torch.float32, out=b["y32"])

    g_buf, e_buf = buffers(), buffers()
    X.zero_()
    W.zero_()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(g_buf)
    torch.cuda.synchronize()

    for rep in range(3):
        rng = np.random.default_rng(100 + rep)
        x = wl.normal_bf16(rng, (M, K), outlier_frac=0.01)
        w = wl.normal_bf16(rng, (N, K), std=0.02)
        X.copy_(to_dev(x))          # new inputs written into the captured storage
        W.copy_(to_dev(w))
        graph.replay()
        torch.cuda.synchronize()
        step(e_buf)                 # eager reference on the same inputs
        torch.cuda.synchronize()
        for key in ("xq", "xs", "wq", "ws", "y", "y32"):
            assert np.array_equal(to_host(g_buf[key]), to_host(e_buf[key])), (rep, key)
        assert np.array_equal(to_host(g_buf["w"].q), to_host(e_buf["w"].q)), rep
        assert np.array_equal(to_host(g_buf["w"].s), to_host(e_buf["w"].s)), rep
        if rep == 0:
            xq, xs = oracle_mod.quantize(x, 1)
            wq, ws = oracle_mod.quantize(w, 1)
            assert np.array_equal(to_host(g_buf["xq"]), xq) and np.array_equal(to_host(g_buf["xs"]), xs)
            assert np.array_equal(to_host(g_buf["wq"]), wq) and np.array_equal(to_host(g_buf["ws"]), ws)
            c_ref, c_abs = oracle_mod.gemm(xq, xs, wq, ws)
            y = wl.bf16_bits_to_f32(to_host(g_buf["y"]))
            ok, worst = oracle_mod.gemm_bound_ok(y, c_ref, c_abs, "bf16")
            assert ok, worst
            ok, worst = oracle_mod.gemm_bound_ok(to_host(g_buf["y32"]), c_ref, c_abs, "f32")
            assert ok, worst


def test_graph_replay_grouped_new_offsets_each_replay(mx, oracle_mod):
    """The grouped GEMM reads its group offsets on the device, so one captured
    graph serves every routing: new offsets are copied in before each replay."""
    import torch
    G, N, K, M_total = 5, 192, 256, 384
    _say("grouped", G, N, K, M_total)
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(7)
    wb = wl.normal_bf16(rng, (G * N, K), std=0.02)
    bq, bs = oracle_mod.quantize(wb, 1)
    w = mx.repack(to_dev(bq.reshape(G, N, K)), to_dev(bs.reshape(G, N, K // 32)))
    A = torch.empty((M_total, K), dtype=torch.bfloat16, device=dev)
    offs = torch.zeros(G + 1, dtype=torch.int32, device=dev)

    def buffers():
        return dict(aq=torch.empty((M_total, K), dtype=torch.uint8, device=dev),
                    as_=torch.empty((M_total, K // 32), dtype=torch.uint8, device=dev),
                    y=torch.zeros((M_total, N), dtype=torch.float32, device=dev))

    def step(b):
        mx.quantize_into(A, 1, b["aq"], b["as_"])
        mx.grouped_gemm(b["aq"], b["as_"], w, offs, torch.float32, out=b["y"])

    g_buf, e_buf = buffers(), buffers()
    A.zero_()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(g_buf)
    torch.cuda.synchronize()

    layouts = [[0, 32, 96, 96, 224, 384], [0, 0, 160, 192, 352, 384], [0, 64, 64, 64, 64, 320]]
    for rep, lay in enumerate(layouts):
        a = wl.normal_bf16(np.random.default_rng(200 + rep), (M_total, K))
        A.copy_(to_dev(a))
        offs.copy_(torch.tensor(lay, dtype=torch.int32))
        g_buf["y"].zero_()
        e_buf["y"].zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        step(e_buf)
        torch.cuda.synchronize()
        yg = to_host(g_buf["y"])
        assert np.array_equal(yg, to_host(e_buf["y"])), rep
        aq, as_ = oracle_mod.quantize(a, 1)
        assert np.array_equal(to_host(g_buf["aq"]), aq)
        c_ref, c_abs, grp = oracle_mod.grouped_gemm(aq, as_, bq.reshape(G, N, K),
                                                    bs.reshape(G, N, K // 32), np.array(lay, np.int32))
        inside = grp >= 0
        ok, worst = oracle_mod.gemm_bound_ok(yg[inside], c_ref[inside], c_abs[inside], "f32")
        assert ok, (rep, worst)
        # rows outside [o_0, o_G) are not written (zero from the fill above)
        assert np.all(yg[~inside] == 0), rep


def test_graph_replay_splitk_and_regrouped_wgrad(mx, oracle_mod):
    """Split-K GEMM (workspace reused across replays) and the MoE weight-
    gradient path (regrouped quantize with its pad pass, aligned grouped-K
    GEMM) recorded once and replayed with new inputs and new group offsets;
    every replay equals an eager run bit for bit, and the first is checked
    against the oracle."""
    import torch
    _say("splitk + regrouped wgrad")
    dev = torch.device("cuda:0")
    M, N, K = 64, 512, 4096                           # few tiles: split-K applies
    X = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    W = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
    wsb = mx.gemm_splitk_workspace_bytes(M, N, K)
    assert wsb > 0
    G, T, C1, C2 = 4, 512, 256, 192
    T128 = T + 128 * G
    dy = torch.empty((T, C1), dtype=torch.bfloat16, device=dev)
    h = torch.empty((T, C2), dtype=torch.bfloat16, device=dev)
    src = torch.zeros(G + 1, dtype=torch.int32, device=dev)
    dst = torch.zeros(G + 1, dtype=torch.int32, device=dev)

    def buffers():
        u8 = dict(dtype=torch.uint8, device=dev)
        return dict(xq=torch.empty((M, K), **u8), xs=torch.empty((M, K // 32), **u8),
                    wq=torch.empty((N, K), **u8), ws=torch.empty((N, K // 32), **u8),
                    wk=torch.empty(wsb, **u8), y=torch.empty((M, N), dtype=torch.bfloat16, device=dev),
                    aq=torch.empty((C1, T128), **u8), as_=torch.empty((C1, T128 // 32), **u8),
                    bq=torch.empty((C2, T128), **u8), bs=torch.empty((C2, T128 // 32), **u8),
                    dw=torch.empty((G, C1, C2), dtype=torch.float32, device=dev))

    def step(b):
        mx.quantize_into(X, 1, b["xq"], b["xs"])
        mx.quantize_into(W, 1, b["wq"], b["ws"])
        mx.gemm(b["xq"], b["xs"], (b["wq"], b["ws"]), torch.bfloat16, out=b["y"], workspace=b["wk"])
        mx.quantize_dual_grouped_into(dy, src, dst, b["aq"], b["as_"])
        mx.quantize_dual_grouped_into(h, src, dst, b["bq"], b["bs"])
        mx.grouped_gemm_wgrad(b["aq"], b["as_"], b["bq"], b["bs"], dst, torch.float32, out=b["dw"])

    g_buf, e_buf = buffers(), buffers()
    for t in (X, W, dy, h):
        t.zero_()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(g_buf)
    torch.cuda.synchronize()
    layouts = [[0, 96, 96, 352, 512], [0, 256, 288, 288, 512], [0, 32, 64, 96, 512]]
    for rep, lay in enumerate(layouts):
        rng = np.random.default_rng(300 + rep)
        x, w = wl.normal_bf16(rng, (M, K)), wl.normal_bf16(rng, (N, K), std=0.02)
        dyh, hh = wl.normal_bf16(rng, (T, C1), std=2.0 ** -10), wl.normal_bf16(rng, (T, C2))
        sizes = np.diff(lay)
        dlay = np.concatenate([[0], np.cumsum(-(-sizes // 128) * 128)]).astype(np.int32)
        for t, v in ((X, x), (W, w), (dy, dyh), (h, hh)):
            t.copy_(to_dev(v))
        src.copy_(torch.tensor(lay, dtype=torch.int32))
        dst.copy_(torch.from_numpy(dlay))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        step(e_buf)
        torch.cuda.synchronize()
        for key in ("xq", "xs", "y", "aq", "as_", "bq", "bs", "dw"):
            assert np.array_equal(to_host(g_buf[key]), to_host(e_buf[key])), (rep, key)
        if rep == 0:
            xq, xs = oracle_mod.quantize(x, 1)
            wq, ws = oracle_mod.quantize(w, 1)
            c_ref, c_abs = oracle_mod.gemm(xq, xs, wq, ws)
            ok, worst = oracle_mod.gemm_bound_ok(wl.bf16_bits_to_f32(to_host(g_buf["y"])), c_ref, c_abs, "bf16")
            assert ok, worst
            rq, rs = oracle_mod.quantize_grouped_axis0(dyh, lay, dlay, T128)
            assert np.array_equal(to_host(g_buf["aq"]), rq) and np.array_equal(to_host(g_buf["as_"]), rs)


def test_graph_replay_packed_many_weight_sync(mx, oracle_mod):
    """A weight sync recorded once (mxfp8_quantize_packed_many, 34 weights: two
    launches) and replayed after new weights are written in place: every
    replay equals the eager call, and the first equals the oracle.  The job
    table is passed by value, so the recorded launches keep it after the host
    array is gone."""
    import torch
    shapes = [(1, 300, 320), (2, 256, 128), (1, 40, 4160), (3, 17, 96)] * 8 + [(1, 513, 96), (1, 1, 32)]
    _say("packed many", len(shapes))
    dev = torch.device("cuda:0")
    Ws = [torch.zeros((b, N, K), dtype=torch.bfloat16, device=dev) for b, N, K in shapes]

    def buffers():
        out = []
        for i, (b, N, K) in enumerate(shapes):
            pw = mx.PackedWeight(torch.empty(mx.packed_bytes(b, N, K, 0), dtype=torch.uint8, device=dev),
                                 torch.empty(mx.packed_bytes(b, N, K, 1), dtype=torch.uint8, device=dev), b, N, K)
            q = s = None
            if i % 3 != 1:
                q = torch.empty((b, N, K), dtype=torch.uint8, device=dev)
                s = torch.empty((b, N, K // 32), dtype=torch.uint8, device=dev)
            out.append((pw, q, s))
        return out

    g_buf, e_buf = buffers(), buffers()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        mx.quantize_packed_many_([(W,) + o for W, o in zip(Ws, g_buf)])
    torch.cuda.synchronize()
    for rep in range(3):
        rng = np.random.default_rng(400 + rep)
        hosts = [wl.normal_bf16(rng, (b * N, K), std=0.02 * (rep + 1)) for b, N, K in shapes]
        for W, w in zip(Ws, hosts):
            W.copy_(to_dev(w).view(W.shape))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        mx.quantize_packed_many_([(W,) + o for W, o in zip(Ws, e_buf)])
        torch.cuda.synchronize()
        for i, ((pg, qg, sg), (pe, qe, se)) in enumerate(zip(g_buf, e_buf)):
            assert torch.equal(pg.q, pe.q) and torch.equal(pg.s, pe.s), (rep, i)
            if qg is not None:
                assert torch.equal(qg, qe) and torch.equal(sg, se), (rep, i)
        if rep == 0:
            for (b, N, K), w, (pg, qg, sg) in zip(shapes, hosts, g_buf):
                rq, rs = oracle_mod.quantize(w, 1)
                qp_ref, sp_ref = oracle_mod.pack(rq.reshape(b, N, K), rs.reshape(b, N, K // 32), b, N, K)
                assert np.array_equal(to_host(pg.q), qp_ref) and np.array_equal(to_host(pg.s), sp_ref)
                if qg is not None:
                    assert np.array_equal(to_host(qg).reshape(b * N, K), rq)


def test_graph_replay_quantize_many_and_packed_axis0(mx, oracle_mod):
    """The list quantizer (weight and activations along K in one launch) and
    the transposed-weight packed quantizer, recorded once and replayed after
    in-place input updates: every replay equals the eager calls; the first
    also equals the oracle."""
    import torch
    _say("quantize many + packed axis0")
    dev = torch.device("cuda:0")
    N, K, M = 320, 288, 96
    W = torch.zeros((N, K), dtype=torch.bfloat16, device=dev)
    X = torch.zeros((M, K), dtype=torch.bfloat16, device=dev)

    def buffers():
        return dict(wq=torch.empty((N, K), dtype=torch.uint8, device=dev),
                    ws=torch.empty((N, K // 32), dtype=torch.uint8, device=dev),
                    xq=torch.empty((M, K), dtype=torch.uint8, device=dev),
                    xs=torch.empty((M, K // 32), dtype=torch.uint8, device=dev),
                    wt=mx.PackedWeight(torch.empty(mx.packed_bytes(1, K, N, 0), dtype=torch.uint8, device=dev),
                                       torch.empty(mx.packed_bytes(1, K, N, 1), dtype=torch.uint8, device=dev),
                                       1, K, N))

    def step(b):
        mx.quantize_many_([(W, b["wq"], b["ws"]), (X, b["xq"], b["xs"])])
        mx.quantize_packed_axis0_(W, b["wt"])

    g_buf, e_buf = buffers(), buffers()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(g_buf)
    torch.cuda.synchronize()
    for rep in range(3):
        rng = np.random.default_rng(500 + rep)
        w = wl.normal_bf16(rng, (N, K), std=0.02)
        x = wl.normal_bf16(rng, (M, K), outlier_frac=0.01)
        W.copy_(to_dev(w))
        X.copy_(to_dev(x))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        step(e_buf)
        torch.cuda.synchronize()
        for key in ("wq", "ws", "xq", "xs"):
            assert torch.equal(g_buf[key], e_buf[key]), (rep, key)
        assert torch.equal(g_buf["wt"].q, e_buf["wt"].q) and torch.equal(g_buf["wt"].s, e_buf["wt"].s), rep
        if rep == 0:
            rq, rs = oracle_mod.quantize(w, 1)
            assert np.array_equal(to_host(g_buf["wq"]), rq) and np.array_equal(to_host(g_buf["ws"]), rs)
            rq, rs = oracle_mod.quantize(x, 1)
            assert np.array_equal(to_host(g_buf["xq"]), rq) and np.array_equal(to_host(g_buf["xs"]), rs)
            q0, s0 = oracle_mod.quantize(w, 0)
            qp, sp = oracle_mod.pack(q0.reshape(1, K, N), s0.reshape(1, K, N // 32), 1, K, N)
            assert np.array_equal(to_host(g_buf["wt"].q), qp) and np.array_equal(to_host(g_buf["wt"].s), sp)


def test_graph_replay_packed_step_and_packed_split(mx, oracle_mod):
    """The default bench step's calls (W along K into its canonical grid and X
    straight into the packed operand layout in one mxfp8_quantize_many_layouts
    launch, repack of W, mxfp8_gemm_packed) and the packed split-K call
    (mxfp8_gemm_packed_splitk with its workspace), recorded once and replayed
    on new inputs: every replay equals the eager calls bit for bit."""
    import torch
    M, N, K = 300, 264, 1024
    Ms = 512                                        # the split case: 2 x 8 tiles, two K slices
    _say("packed step + packed split", M, N, K, Ms)
    dev = torch.device("cuda:0")
    X = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    Xs = torch.empty((Ms, K), dtype=torch.bfloat16, device=dev)
    W = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
    need = mx.gemm_splitk_workspace_bytes(Ms, N, K)
    assert need > 0

    def pw(rows):
        return mx.PackedWeight(torch.empty(mx.packed_bytes(1, rows, K, 0), dtype=torch.uint8, device=dev),
                               torch.empty(mx.packed_bytes(1, rows, K, 1), dtype=torch.uint8, device=dev), 1, rows, K)

    def buffers():
        return dict(wq=torch.empty((N, K), dtype=torch.uint8, device=dev),
                    ws=torch.empty((N, K // 32), dtype=torch.uint8, device=dev),
                    w=pw(N), a=pw(M), a2=pw(Ms),
                    y=torch.empty((M, N), dtype=torch.bfloat16, device=dev),
                    y2=torch.empty((Ms, N), dtype=torch.float32, device=dev),
                    wk=torch.empty(need, dtype=torch.uint8, device=dev))

    def step(b):
        mx.quantize_many_layouts_([(W, (b["wq"], b["ws"])), (X, b["a"]), (Xs, b["a2"])])
        mx.repack_(b["wq"], b["ws"], b["w"])
        mx.gemm_packed(b["a"], b["w"], torch.bfloat16, out=b["y"])
        mx.gemm_packed(b["a2"], b["w"], torch.float32, out=b["y2"], workspace=b["wk"])

    g_buf, e_buf = buffers(), buffers()
    for t in (X, Xs, W):
        t.zero_()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(g_buf)
    torch.cuda.synchronize()
    for rep in range(3):
        rng = np.random.default_rng(300 + rep)
        x = wl.normal_bf16(rng, (M, K), outlier_frac=0.01)
        xs = wl.normal_bf16(rng, (Ms, K))
        w = wl.normal_bf16(rng, (N, K), std=0.02)
        X.copy_(to_dev(x))
        Xs.copy_(to_dev(xs))
        W.copy_(to_dev(w))
        graph.replay()
        torch.cuda.synchronize()
        step(e_buf)
        torch.cuda.synchronize()
        for key in ("wq", "ws", "y", "y2"):
            assert np.array_equal(to_host(g_buf[key]), to_host(e_buf[key])), (rep, key)
        for key in ("w", "a", "a2"):
            assert np.array_equal(to_host(g_buf[key].q), to_host(e_buf[key].q)), (rep, key)
            assert np.array_equal(to_host(g_buf[key].s), to_host(e_buf[key].s)), (rep, key)
        if rep == 0:
            xq, xsc = oracle_mod.quantize(x, 1)
            wq, wsc = oracle_mod.quantize(w, 1)
            qp, sp = oracle_mod.pack(xq.reshape(1, M, K), xsc.reshape(1, M, K // 32), 1, M, K)
            assert np.array_equal(to_host(g_buf["a"].q), qp) and np.array_equal(to_host(g_buf["a"].s), sp)
            c_ref, c_abs = oracle_mod.gemm(xq, xsc, wq, wsc)
            ok, worst = oracle_mod.gemm_bound_ok(wl.bf16_bits_to_f32(to_host(g_buf["y"])), c_ref, c_abs, "bf16")
            assert ok, worst
            x2q, x2s = oracle_mod.quantize(xs, 1)
            c2, a2 = oracle_mod.gemm(x2q, x2s, wq, wsc)
            ok, worst = oracle_mod.gemm_bound_ok(to_host(g_buf["y2"]), c2, a2, "f32")
            assert ok, worst
