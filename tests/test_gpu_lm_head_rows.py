"""The matrix-core GEMV (nb 5-16; from nb 3 or 4 for most formats on matrices of at least 2^24
weights) on lm_head-sized matrices: 65521..65536 rows (and 8192, the smallest that takes nb 3-4;
Q8_0, Q6_K and the affine format at nb 4 and Q5_K at nb 3 as vector-path contrasts), K <= 2048, where
each workgroup owns one group of 16 whole-row tiles (one wave per tile, every K step of its rows).
Every format, every epilogue, K that is not a multiple of a scale round, a ragged last tile;
sampled rows against the f64 oracle ("Crate inferencelayer" docs: the lm_head GEMV of the decode
step), repeated launches bit for bit."""
import numpy as np
import pytest

from gpu_common import (assert_within, dev, gpu_matrix, gus_tol, host, require_gpu, say,
                        tol_gemv, torch)

import dequant_gemv_q4_amd as q
from dequant_gemv_q4_amd import device as D
import oracle
import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    oracle.build(force=False)


def _sample(g, N):
    """Rows to check: the first and last two tiles whole, 384 more at random."""
    rows = set(range(32)) | set(range(N - 32, N)) | set(g.choice(N, 384, replace=False).tolist())
    return np.array(sorted(rows), dtype=np.int64)


CB = wl.iq4_codebook()


def _matrix(fmt, g, N, K):
    if fmt in (q.IQ4_NL, q.IQ4_XS):
        oracle.set_codebook(CB)
    return wl.matrix(fmt, g, N, K)


def _packed(fmt, W, N, K):
    return D.pack(fmt, W, N, K, codebook=CB if fmt in (q.IQ4_NL, q.IQ4_XS) else None)


@pytest.mark.parametrize("fmt,N,K,nb", [
    (q.Q4_0, 65536, 2048, 16), (q.Q4_0, 65536, 2048, 5), (q.Q4_0, 65530, 1536, 9),
    (q.Q8_0, 65536, 2048, 16), (q.Q8_0, 65536, 1600, 7), (q.Q4_K, 65536, 2048, 16),
    (q.Q5_0, 65536, 2048, 8), (q.Q5_K, 65536, 1536, 16), (q.Q6_K, 65536, 2048, 6),
    (q.IQ4_NL, 65536, 2048, 16), (q.IQ4_XS, 65536, 2048, 12), (q.Q1_0, 65536, 2048, 16),
    (q.AQ4, 65533, 2048, 10), (q.Q4_0, 65536, 2048, 4), (q.Q4_K, 65536, 2048, 4),
    (q.Q4_0, 8192, 2048, 4), (q.Q8_0, 65536, 2048, 4), (q.Q4_0, 65536, 2048, 3),
    (q.Q4_K, 8192, 2048, 3), (q.Q4_0, 8191, 2048, 3), (q.IQ4_NL, 8192, 2048, 4),
    (q.IQ4_XS, 8192, 2048, 3), (q.Q1_0, 65536, 2048, 3), (q.Q5_0, 8192, 2048, 3),
    (q.Q5_K, 65536, 2048, 4), (q.Q5_K, 65536, 2048, 3), (q.Q6_K, 65536, 2048, 4),
    (q.AQ4, 8192, 2048, 4)])
def test_lm_head_rows_parity(fmt, N, K, nb):
    say(f"lm_head rows fmt={fmt} N={N} K={K} nb={nb}")
    g = wl.rng(7000 + fmt, N + K + nb)
    W = _matrix(fmt, g, N, K)
    x = wl.normal_f32(g, (nb, K))
    Wd = _packed(fmt, W, N, K)
    y = torch.empty((nb, N), dtype=torch.float32, device="cuda")
    q.qgemv(fmt, Wd, N, K, dev(x), nb, y)
    y1 = host(y)
    q.qgemv(fmt, Wd, N, K, dev(x), nb, y)
    assert np.array_equal(host(y), y1), "repeated launches differ"
    rows = _sample(g, N)
    yr, A = oracle.gemv(fmt, W, N, K, x, rows=rows)
    assert_within(y1[:, rows], yr, tol_gemv(A, yr), f"lm_head rows fmt={fmt} N={N} K={K} nb={nb}")


@pytest.mark.parametrize("fmt,nb", [(q.Q4_0, 8), (q.Q6_K, 8), (q.Q4_0, 4), (q.Q4_K, 3)])
def test_lm_head_rows_epilogues(fmt, nb):
    """Norm prologue, residual add (in place), gated product and argmax at 65536 rows (at nb 3-4
    every one but the gated product on the matrix cores)."""
    N, K = 65536, 2048
    say(f"lm_head rows epilogues fmt={fmt} nb={nb}")
    g = wl.rng(7100 + fmt, 1)
    W = _matrix(fmt, g, N, K)
    Wu = _matrix(fmt, g, N, K)
    x = wl.normal_f32(g, (nb, K))
    gamma = (1.0 + 0.1 * g.standard_normal(K)).astype(np.float32)
    res = wl.normal_f32(g, (nb, N))
    eps = 1e-6
    Wd, Wud = gpu_matrix(fmt, W, N, K), gpu_matrix(fmt, Wu, N, K)
    rows = _sample(g, N)

    y = torch.empty((nb, N), dtype=torch.float32, device="cuda")
    q.qgemv_nrm(fmt, Wd, N, K, dev(x), dev(gamma), eps, nb, y)
    yr, A = oracle.qgemv_nrm(fmt, W, N, K, x, gamma, eps, rows=rows)
    assert_within(host(y)[:, rows], yr, tol_gemv(A, yr), "nrm")

    yres = dev(res.copy())
    q.qgemv_res(fmt, Wd, N, K, dev(x), yres, nb, yres)          # in place
    yr, A = oracle.qgemv_res(fmt, W, N, K, x, res, rows=rows)
    assert_within(host(yres)[:, rows], yr, tol_gemv(A, yr), "res")

    yg = torch.empty((nb, N), dtype=torch.float32, device="cuda")
    q.qgemv_gus_nrm(fmt, Wd, Wud, N, K, dev(x), dev(gamma), eps, nb, yg)
    xn = oracle.rmsnorm(x, gamma, eps)
    gr, Ag = oracle.gemv(fmt, W, N, K, xn, rows=rows)
    ur, Au = oracle.gemv(fmt, Wu, N, K, xn, rows=rows)
    ref = oracle.swiglu(gr, ur)
    assert_within(host(yg)[:, rows], ref, gus_tol(gr, ur, Ag, Au), "gus")

    logits = torch.empty((nb, N), dtype=torch.float32, device="cuda")
    idx = torch.empty((nb,), dtype=torch.int32, device="cuda")
    ws = D.workspace(q.OP_ARGMAX, fmt, N, K, nb)
    q.qgemv_argmax(fmt, Wd, N, K, dev(x), nb, logits, idx, ws)
    lg, ig = host(logits), host(idx)
    for r in range(nb):
        i = int(ig[r])
        assert lg[r, i] == lg[r].max() and int(np.argmax(lg[r])) == i, r
    yr, A = oracle.gemv(fmt, W, N, K, x, rows=rows)
    assert_within(lg[:, rows], yr, tol_gemv(A, yr), "argmax logits")
