"""Shared plumbing for the GPU parity tests (torch for memory only)."""
from __future__ import annotations

import os
import sys

import numpy as np

import oracle

LOG = os.environ.get("EXQ_TEST_LOG")   # optional progress file, e.g. one that outlives a crashed run


def note(msg: str) -> None:
    """Name the case before a GPU step, on stderr and, if EXQ_TEST_LOG is set, in that file."""
    sys.stderr.write("[exq-test] %s\n" % msg)
    sys.stderr.flush()
    if not LOG:
        return
    try:
        os.makedirs(os.path.dirname(os.path.abspath(LOG)), exist_ok=True)
        with open(LOG, "a") as f:
            f.write(msg + "\n")
    except OSError:
        pass


def to_dev(a: np.ndarray):
    import torch
    if a.dtype == np.float16:
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def y_to_np(y) -> np.ndarray:
    import torch
    torch.cuda.synchronize()
    return y.cpu().numpy()


def assert_within(y: np.ndarray, y_ref: np.ndarray, bound: np.ndarray, what: str):
    ok, worst = oracle.within_tolerance(y.astype(np.float64), y_ref, bound)
    assert ok, "%s: max |err| / (2e-3*B + 1e-5) = %.3f" % (what, worst)
    return worst


def sample_cols(N: int, count: int, seed: int) -> np.ndarray:
    """Edges of the first and last 64-column tiles plus a seeded sample."""
    rng = np.random.default_rng(seed)
    edge = [0, 1, 63, 64, N - 65, N - 64, N - 2, N - 1]
    pick = rng.choice(N, size=min(count, N), replace=False)
    return np.unique(np.concatenate([np.array([c for c in edge if 0 <= c < N]), pick])).astype(np.int64)
