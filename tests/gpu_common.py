"""Shared helpers of the GPU parity tests: device buffers, tolerances and comparisons.

The tolerance is the one the parity bar fixes for floating point: per output,
|y_gpu - y_ref| <= 1e-3 * sum_k |w_k x_k| (A, from the f64 oracle), plus 2^-23 |y_ref| for the
f32 rounding of a residual add.  A NaN anywhere fails.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import dequant_gemv_q4_amd as q  # noqa: E402
from dequant_gemv_q4_amd import device as D  # noqa: E402

REL = 1e-3


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q.lib()   # the HIP library must be built and loadable; no fallback exists


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def dev(a):
    return D.to_device(a)


def host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def tol_gemv(A, yref):
    return REL * A + 2.0 ** -23 * np.abs(yref)


def assert_within(got, ref, tol, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert not np.isnan(got).any(), f"{what}: NaN in GPU output"
    err = np.abs(got - ref)
    bad = err > tol
    if bad.any():
        i = np.unravel_index(np.argmax(err - tol), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {err.size} outputs outside tolerance; "
                             f"worst at {i}: gpu={got[i]!r} ref={ref[i]!r} err={err[i]:.3e} "
                             f"tol={np.asarray(tol)[i] if np.ndim(tol) else tol:.3e}")


def gus_tol(g, u, Ag, Au):
    """Tolerance of h = silu(g) u propagated from the per-output bounds of g and u,
    |dg| <= 1e-3 Ag and |du| <= 1e-3 Au: |dh| <= |silu'| |dg| |u| + |silu(g)| |du| + |silu'| |dg| |du|
    with sup |silu'| < 1.1."""
    sg = g / (1.0 + np.exp(-g))
    return REL * (1.1 * Ag * np.abs(u) + np.abs(sg) * Au) + REL * REL * 1.1 * Ag * Au


def gpu_matrix(fmt, W_gguf, N, K):
    return D.pack(fmt, W_gguf, N, K)
