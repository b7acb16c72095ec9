import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU test")


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle
    oracle._load()
    return oracle


@pytest.fixture(scope="session")
def mx():
    """The HIP library's Python binding on cuda:0 (GPU tests only)."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mxfp8_block_scaled_05_amd as m
    m.lib()
    torch.cuda.set_device(0)
    return m


def to_dev(a):
    """numpy array -> device tensor with the same bytes (uint16 -> bfloat16)."""
    import numpy as np
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def to_host(t):
    import numpy as np
    import torch
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def sample_rows(n_rows, tile, count, seed, groups=None):
    """Sorted, distinct row indices of an [n_rows x N] output for sampled
    parity: one random row from every `tile`-row tile (or, with `groups` =
    offsets of row groups, one from every non-empty group), the first and last
    row, then random rows until `count` are drawn (all rows if count >=
    n_rows)."""
    import numpy as np
    rng = np.random.default_rng(seed)
    if count >= n_rows:
        return np.arange(n_rows, dtype=np.int64)
    pick = {0, n_rows - 1}
    if groups is not None:
        off = np.asarray(groups, np.int64)
        for lo, hi in zip(off[:-1], off[1:]):
            if hi > lo:
                pick.add(int(rng.integers(lo, hi)))
    else:
        for t0 in range(0, n_rows, tile):
            pick.add(int(rng.integers(t0, min(n_rows, t0 + tile))))
    while len(pick) < count:
        pick.add(int(rng.integers(0, n_rows)))
    return np.array(sorted(pick), dtype=np.int64)
