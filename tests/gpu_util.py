"""Helpers for the GPU tests: move seeded bf16 bit arrays to and from the
device, run the HIP path through the C ABI, and compare with the oracle."""
from __future__ import annotations

import numpy as np

import oracle


def torch_mod():
    import torch
    return torch


def to_dev(bits: np.ndarray):
    torch = torch_mod()
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def to_bits(t) -> np.ndarray:
    torch = torch_mod()
    torch.cuda.synchronize()
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def assert_parity(y_bits: np.ndarray, y_ref: np.ndarray, what: str):
    p = oracle.parity(y_bits, y_ref)
    assert p["finite"], "%s: non-finite output" % what
    assert p["rel_fro"] <= oracle.REL_FRO_TOL, "%s: rel_fro %.3e" % (what, p["rel_fro"])
    assert p["max_abs"] <= oracle.MAX_ABS_TOL, "%s: max_abs %.3e" % (what, p["max_abs"])
    return p


def banner(msg: str):
    print("[gpu-test] " + msg, flush=True)


def tile_cover(n: int, block: int, seed: int, extra=()) -> np.ndarray:
    """Sorted distinct indices of range(n): one at a seeded offset inside
    every `block`-sized block (so every output tile of width >= block holds
    at least one), the first and the last index, and `extra`."""
    rng = np.random.default_rng(seed)
    starts = np.arange(0, n, block)
    picks = starts + rng.integers(0, np.minimum(block, n - starts))
    ex = np.array([e for e in extra if 0 <= e < n], dtype=np.int64)
    return np.unique(np.concatenate([picks, [0, n - 1], ex]).astype(np.int64))
