"""Shared-grid weight synchronization with the page's post-sync checks.

"End-to-End MXFP8 RL on Blackwell" (verl blog), section "The pipeline": the
sampler receives the learner's forward weight grid, rebuilds every derived
kernel layout from it after each synchronization and writes it into the
storage its captured graphs read.  Section "Correctness: how it fails" lists
what a synchronization must preserve; the ones a single device can check are
enforced here after every sync:

  C3 derived state    -- one dense layer and one expert are run through the
                         serving GEMM on a random probe and compared with a
                         GEMM on the dequantized synchronized weights
                         (relative Frobenius error, tolerance 0.25);
  C4 storage identity -- every weight's packed buffers are still the ones
                         registered (the addresses a graph captured);
  C5 completeness     -- every registered weight was written in this sync;
  C7 observability    -- each check reports a verdict, or why it could not run.

Mode (constructor argument, else the MXFP8_SYNC_CHECK environment variable):
"off" runs no check, "warn" (default) warns on a failed check, "error" raises
SyncCheckError.  The GPU work goes through a backend object so the host logic
can be exercised without a GPU.
"""
from __future__ import annotations

import math
import os
import warnings
from dataclasses import dataclass, field

MODES = ("off", "warn", "error")


class SyncCheckError(RuntimeError):
    pass


def selfcheck_passed(rel_err: float, tolerance: float) -> bool:
    """A layer passes when its relative error is finite and within tolerance."""
    return rel_err is not None and math.isfinite(rel_err) and rel_err <= tolerance


@dataclass
class Entry:
    name: str
    kind: str                 # "dense" or "expert"
    batch: int
    N: int
    K: int
    packed: object            # backend's packed weight (q/s storage)
    q: object                 # canonical grid (what the learner sends)
    s: object
    addr: tuple = ()          # storage addresses at registration
    generation: int = -1      # last sync that wrote this weight


@dataclass
class CheckReport:
    generation: int
    mode: str
    verdicts: dict = field(default_factory=dict)   # check -> "pass" / "fail: ..." / "not run: ..."
    selfcheck: dict = field(default_factory=dict)  # layer -> relative error

    @property
    def failed(self):
        return [k for k, v in self.verdicts.items() if v.startswith("fail")]


class GpuBackend:
    """The library on the current device."""

    def __init__(self):
        import mxfp8_block_scaled_05_amd as mx
        self.mx = mx

    def alloc(self, batch, N, K):
        import torch
        mx = self.mx
        packed = mx.PackedWeight(torch.empty(mx.packed_bytes(batch, N, K, 0), dtype=torch.uint8, device="cuda"),
                                 torch.empty(mx.packed_bytes(batch, N, K, 1), dtype=torch.uint8, device="cuda"),
                                 batch, N, K)
        q = torch.empty((batch, N, K), dtype=torch.uint8, device="cuda")
        s = torch.empty((batch, N, K // 32), dtype=torch.uint8, device="cuda")
        return packed, q, s

    def addresses(self, e: Entry):
        return (e.packed.q.data_ptr(), e.packed.s.data_ptr())

    def write(self, e: Entry, w):
        self.mx.quantize_packed_(w, e.packed, e.q, e.s)

    def rel_err(self, e: Entry, index: int, seed: int):
        return self.mx.selfcheck_rel_err(e.q[index], e.s[index], e.packed, index=index, seed=seed)[0]


class WeightSync:
    def __init__(self, mode: str | None = None, tolerance: float = 0.25, backend=None, seed: int = 0):
        mode = mode or os.environ.get("MXFP8_SYNC_CHECK", "warn")
        if mode not in MODES:
            raise ValueError("mode must be one of %s" % (MODES,))
        self.mode = mode
        self.tolerance = tolerance
        self.backend = backend if backend is not None else GpuBackend()
        self.seed = seed
        self.entries: dict[str, Entry] = {}
        self.generation = 0
        self.reports: list[CheckReport] = []

    def register(self, name: str, N: int, K: int, batch: int = 1, kind: str = "dense") -> Entry:
        """Allocate a weight's canonical grid and packed storage once; graphs
        capture the packed storage, every later sync rewrites it in place."""
        if name in self.entries:
            raise ValueError("weight %r already registered" % name)
        if kind not in ("dense", "expert"):
            raise ValueError("kind must be 'dense' or 'expert'")
        packed, q, s = self.backend.alloc(batch, N, K)
        e = Entry(name, kind, batch, N, K, packed, q, s)
        e.addr = self.backend.addresses(e)
        self.entries[name] = e
        return e

    def begin(self) -> int:
        self.generation += 1
        return self.generation

    def update(self, name: str, w_bf16) -> None:
        """Quantize one weight along K into its canonical grid and packed storage."""
        e = self.entries[name]
        self.backend.write(e, w_bf16)
        e.generation = self.generation

    def finish(self) -> CheckReport:
        rep = CheckReport(self.generation, self.mode)
        if self.mode == "off":
            rep.verdicts = {c: "not run: checks off" for c in ("C3", "C4", "C5")}
            self.reports.append(rep)
            return rep
        stale = sorted(n for n, e in self.entries.items() if e.generation != self.generation)
        rep.verdicts["C5"] = "pass" if not stale else "fail: not written in this sync: %s" % ", ".join(stale)
        moved = sorted(n for n, e in self.entries.items() if self.backend.addresses(e) != e.addr)
        rep.verdicts["C4"] = "pass" if not moved else "fail: storage replaced since capture: %s" % ", ".join(moved)
        # C3 on the first dense layer and the first expert (matrix 0) that were written
        probes = []
        for kind in ("dense", "expert"):
            cands = [e for e in self.entries.values() if e.kind == kind and e.generation == self.generation]
            if cands:
                probes.append(cands[0])
        if not probes:
            rep.verdicts["C3"] = "not run: no written layer to probe"
        else:
            bad = []
            for e in probes:
                err = self.backend.rel_err(e, 0, self.seed + self.generation)
                rep.selfcheck[e.name] = err
                if not selfcheck_passed(err, self.tolerance):
                    bad.append("%s %.4g" % (e.name, err))
            rep.verdicts["C3"] = "pass" if not bad else "fail: relative error above %.2f: %s" % (
                self.tolerance, ", ".join(bad))
        self.reports.append(rep)
        if rep.failed:
            msg = "weight sync %d: %s" % (self.generation, "; ".join("%s %s" % (k, rep.verdicts[k]) for k in rep.failed))
            if self.mode == "error":
                raise SyncCheckError(msg)
            warnings.warn(msg, RuntimeWarning, stacklevel=2)
        return rep
