"""Helpers shared by the GPU parity tests (tolerances, transfers, flushing prints)."""

from __future__ import annotations

import sys

import numpy as np

# Output tolerance (rel L2 <= 1e-3, max|dy| <= 1e-3 * max|y|), from the arithmetic: the float16
# output rounding alone contributes up to 2^-11 relative per element (~2e-4 relative
# L2 on random data); float32 accumulation adds ~sqrt(K)*2^-24.
REL_L2_TOL = 1e-3
MAX_ABS_REL_TOL = 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_gpu(a: np.ndarray):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_np(t) -> np.ndarray:
    return t.detach().cpu().numpy()


def assert_close(y_gpu, y_ref: np.ndarray, what: str = ""):
    """relative L2 <= 1e-3 and max |dy| <= 1e-3 * max |y_ref| (float64 reference)."""
    y = np.asarray(y_gpu, dtype=np.float64)
    ref = np.asarray(y_ref, dtype=np.float64)
    assert y.shape == ref.shape, (what, y.shape, ref.shape)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    nref = np.linalg.norm(ref)
    if nref == 0:
        assert np.all(y == 0), what
        return 0.0, 0.0
    rel = np.linalg.norm(y - ref) / nref
    mx = np.max(np.abs(y - ref)) / np.max(np.abs(ref))
    assert rel <= REL_L2_TOL and mx <= MAX_ABS_REL_TOL, f"{what}: rel L2 {rel:.3e}, max-abs ratio {mx:.3e}"
    return rel, mx
