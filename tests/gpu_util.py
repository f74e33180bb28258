"""Shared helpers for the GPU parity tests (imported by tests only)."""
import math

import numpy as np
import torch

import workloads

DEV = "cuda:0"

# Tolerances (stated by the workload spec): fp32 outputs within relative
# error 1e-3; bf16-operand gradients within 2e-2, read elementwise against
# |r| + RMS(r), the RMS taken over all the reference entries compared (an
# entry of a sum that cancels to ~0 gets the scale of the whole output), and
# as a relative Frobenius error.
Y_RTOL = 1e-3
GRAD_TOL = 2e-2


def to_dev(t: torch.Tensor) -> torch.Tensor:
    return t.contiguous().to(DEV)


def host(t: torch.Tensor):
    """Device or host tensor -> numpy array for the oracle (bf16 as uint16 bits)."""
    t = t.detach().cpu().contiguous()
    return workloads.host_array(t)


def f32_bits_equal(a: np.ndarray, b: np.ndarray) -> bool:
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = np.ascontiguousarray(b, dtype=np.float32)
    return a.shape == b.shape and bool((a.view(np.uint32) == b.view(np.uint32)).all())


def assert_y_close(y: np.ndarray, ref: np.ndarray, what: str = "Y"):
    y = y.astype(np.float64)
    err = np.abs(y - ref)
    bad = err > Y_RTOL * np.abs(ref)
    assert not bad.any(), (
        f"{what}: {int(bad.sum())} of {bad.size} entries beyond rel {Y_RTOL}; "
        f"worst {float((err / np.maximum(np.abs(ref), 1e-30)).max()):.3e}")


def assert_grad_close(g: np.ndarray, ref: np.ndarray, what: str, tol: float = GRAD_TOL):
    g = g.astype(np.float64)
    err = np.abs(g - ref)
    rms = math.sqrt(float(np.mean(ref * ref))) if ref.size else 0.0
    bad = err > tol * (np.abs(ref) + rms)
    assert not bad.any(), f"{what}: {int(bad.sum())} of {bad.size} entries beyond {tol} (|r| + rms)"
    nr = float(np.linalg.norm(ref))
    assert float(np.linalg.norm(g - ref)) <= tol * nr + 1e-30, f"{what}: relative Frobenius error too large"


def sample_pairs(rows: int, cols: int, count: int, seed: int):
    rng = np.random.default_rng(seed)
    r = rng.integers(0, rows, size=count)
    c = rng.integers(0, cols, size=count)
    # always include the four corners (ragged tile edges)
    r = np.concatenate([r, [0, 0, rows - 1, rows - 1]])
    c = np.concatenate([c, [0, cols - 1, 0, cols - 1]])
    return r.astype(np.int64), c.astype(np.int64)
