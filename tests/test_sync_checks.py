"""Host logic of the post-sync checks, with faults injected into a CPU stub.

The stub backend stands in for the GPU: it quantizes and packs with the oracle
and computes the self-check's relative error from the oracle's GEMM of the
quantized probe against whatever the packed storage holds (so a stale packed
layout shows up exactly as it would through the serving kernel).  Faults:
a stale layout (C3), replaced storage (C4) and a weight left out of a sync
(C5), plus the off / warn / error modes.
"""
import math
import warnings

import numpy as np
import pytest

import workloads as wl
from mxfp8_block_scaled_05_amd.sync import SyncCheckError, WeightSync, selfcheck_passed


class OracleBackend:
    def __init__(self, oracle):
        self.o = oracle
        self.skip_pack = False

    def alloc(self, batch, N, K):
        packed = {"q": np.zeros(self.o.packed_bytes(batch, N, K, 0), np.uint8),
                  "s": np.zeros(self.o.packed_bytes(batch, N, K, 1), np.uint8)}
        return packed, np.zeros((batch, N, K), np.uint8), np.zeros((batch, N, K // 32), np.uint8)

    def addresses(self, e):
        return (e.packed["q"].ctypes.data, e.packed["s"].ctypes.data)

    def write(self, e, w_bits):
        q, s = self.o.quantize(w_bits.reshape(e.batch * e.N, e.K), 1)
        e.q[...] = q.reshape(e.q.shape)
        e.s[...] = s.reshape(e.s.shape)
        if not self.skip_pack:
            qp, sp = self.o.pack(e.q, e.s, e.batch, e.N, e.K)
            e.packed["q"][...] = qp
            e.packed["s"][...] = sp

    def rel_err(self, e, index, seed):
        rng = np.random.default_rng(seed)
        x = wl.normal_bf16(rng, (32, e.K))
        xq, xs = self.o.quantize(x, 1)
        # what the serving GEMM reads: the packed storage, unpacked
        pq, ps = self.o.unpack(e.packed["q"], e.packed["s"], e.batch, e.N, e.K)
        y, _ = self.o.gemm(xq, xs, pq[index], ps[index])
        w = self.o.dequantize(e.q[index], e.s[index], e.N, e.K, 1, "f64")
        yref = wl.bf16_bits_to_f32(x).astype(np.float64) @ w.T
        return float(np.linalg.norm(y - yref) / np.linalg.norm(yref))


def _make(oracle_mod, mode="error"):
    b = OracleBackend(oracle_mod)
    ws = WeightSync(mode=mode, backend=b, seed=3)
    ws.register("qkv", 64, 128)
    ws.register("o", 32, 64)
    ws.register("experts", 32, 64, batch=2, kind="expert")
    return ws, b


def _sync(ws, seed, skip=()):
    rng = np.random.default_rng(seed)
    ws.begin()
    for name, e in ws.entries.items():
        if name in skip:
            continue
        ws.update(name, wl.normal_bf16(rng, (e.batch, e.N, e.K), std=0.02))
    return ws.finish()


def test_verdict_rule():
    assert selfcheck_passed(0.027, 0.25) and selfcheck_passed(0.25, 0.25)
    assert not selfcheck_passed(0.2501, 0.25)
    assert not selfcheck_passed(float("nan"), 0.25) and not selfcheck_passed(math.inf, 0.25)


def test_healthy_syncs_pass(oracle_mod):
    ws, _ = _make(oracle_mod)
    for seed in (1, 2):
        rep = _sync(ws, seed)
        assert rep.verdicts == {"C5": "pass", "C4": "pass", "C3": "pass"}
        # the activation-quantization cost only: a few percent, as on the page
        assert set(rep.selfcheck) == {"qkv", "experts"}
        for err in rep.selfcheck.values():
            assert 0.005 < err < 0.1, err


def test_stale_layout_is_caught(oracle_mod):
    ws, b = _make(oracle_mod)
    _sync(ws, 1)
    b.skip_pack = True                    # canonical tensors updated, derived layout not rebuilt
    with pytest.raises(SyncCheckError, match="C3"):
        _sync(ws, 2)
    rep = ws.reports[-1]
    assert rep.verdicts["C4"] == "pass" and rep.verdicts["C5"] == "pass"
    assert all(err > 0.5 for err in rep.selfcheck.values())   # order 1


def test_replaced_storage_is_caught(oracle_mod):
    ws, _ = _make(oracle_mod)
    _sync(ws, 1)
    e = ws.entries["o"]
    e.packed = {"q": e.packed["q"].copy(), "s": e.packed["s"].copy()}   # new buffers, same bytes
    with pytest.raises(SyncCheckError, match="C4.*o"):
        _sync(ws, 2)
    assert ws.reports[-1].verdicts["C3"] == "pass"


def test_incomplete_sync_is_caught(oracle_mod):
    ws, _ = _make(oracle_mod)
    _sync(ws, 1)
    with pytest.raises(SyncCheckError, match="C5.*experts"):
        _sync(ws, 2, skip=("experts",))
    rep = ws.reports[-1]
    assert rep.verdicts["C4"] == "pass"
    assert set(rep.selfcheck) == {"qkv"}      # only written layers are probed


def test_modes(oracle_mod, monkeypatch):
    ws, b = _make(oracle_mod, mode="warn")
    _sync(ws, 1)
    b.skip_pack = True
    with warnings.catch_warnings(record=True) as got:
        warnings.simplefilter("always")
        rep = _sync(ws, 2)
    assert rep.failed == ["C3"] and any("C3" in str(w.message) for w in got)
    ws_off, b_off = _make(oracle_mod, mode="off")
    b_off.skip_pack = True
    rep = _sync(ws_off, 1)
    assert rep.failed == [] and all(v.startswith("not run") for v in rep.verdicts.values())
    monkeypatch.setenv("MXFP8_SYNC_CHECK", "error")
    assert WeightSync(backend=b).mode == "error"
    with pytest.raises(ValueError):
        WeightSync(mode="loud", backend=b)
