"""Q4_K row batches (5 <= nb <= 16) on the matrix cores against the f64 oracle ("Crate
inferencelayer" docs, gemv_q4_k_lcpp_src: w = d sc q - dmin m per 32-weight sub-block): every GEMV
entry point, K of one and two classes, integer inputs bit for bit, all-zero weights exactly zero,
and sub-blocks whose weights mostly cancel (the centred arithmetic)."""
import numpy as np
import pytest

from gpu_common import assert_within, dev, gpu_matrix, gus_tol, host, require_gpu, say, tol_gemv, torch

import dequant_gemv_q4_amd as q
from dequant_gemv_q4_amd import device as D
import oracle
import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    oracle.build(force=False)


def _gemv(W, N, K, x):
    nb = x.shape[0]
    y = torch.empty((nb, N), dtype=torch.float32, device="cuda")
    q.qgemv(q.Q4_K, gpu_matrix(q.Q4_K, W, N, K), N, K, dev(x), nb, y)
    return host(y)


@pytest.mark.parametrize("N,K,nb", [(16, 256, 5), (300, 2048, 5), (301, 2048, 8), (77, 4096, 16),
                                    (4100, 2048, 16), (33, 3072, 11), (1000, 1024, 7)])
def test_q4_k_row_batch(N, K, nb):
    say(f"q4_k mfma N={N} K={K} nb={nb}")
    g = wl.rng(4000, N + K + nb)
    W = wl.q4_k_matrix(g, N, K)
    x = wl.normal_f32(g, (nb, K))
    y = _gemv(W, N, K, x)
    yr, A = oracle.gemv(q.Q4_K, W, N, K, x)
    assert_within(y, yr, tol_gemv(A, yr), f"q4_k N={N} K={K} nb={nb}")


@pytest.mark.parametrize("nb", [5, 16])
def test_q4_k_row_batch_fused(nb):
    say(f"q4_k mfma fused nb={nb}")
    N, K = 520, 2048
    g = wl.rng(4100, nb)
    W, Wu = wl.q4_k_matrix(g, N, K), wl.q4_k_matrix(g, N, K)
    x = wl.normal_f32(g, (nb, K))
    gamma = wl.gamma_f32(g, K)
    r = wl.normal_f32(g, (nb, N))
    Wp, Wup = gpu_matrix(q.Q4_K, W, N, K), gpu_matrix(q.Q4_K, Wu, N, K)
    y = torch.empty((nb, N), dtype=torch.float32, device="cuda")
    q.qgemv_nrm(q.Q4_K, Wp, N, K, dev(x), dev(gamma), 1e-5, nb, y)
    yr, A = oracle.qgemv_nrm(q.Q4_K, W, N, K, x, gamma, 1e-5)
    assert_within(host(y), yr, tol_gemv(A, yr), "nrm")
    q.qgemv_res(q.Q4_K, Wp, N, K, dev(x), dev(r), nb, y)
    yr, A = oracle.qgemv_res(q.Q4_K, W, N, K, x, r)
    assert_within(host(y), yr, tol_gemv(A, yr), "res")
    q.qgemv_gus_nrm(q.Q4_K, Wp, Wup, N, K, dev(x), dev(gamma), 1e-5, nb, y)
    hr, gr, ur, Ag, Au = oracle.qgemv_gus_nrm(q.Q4_K, W, Wu, N, K, x, gamma, 1e-5)
    assert_within(host(y), hr, gus_tol(gr, ur, Ag, Au), "gus")
    logits = torch.empty((nb, N), dtype=torch.float32, device="cuda")
    idx = torch.empty((nb,), dtype=torch.int32, device="cuda")
    q.qgemv_argmax(q.Q4_K, Wp, N, K, dev(x), nb, logits, idx,
                   D.workspace(q.OP_ARGMAX, q.Q4_K, N, K, nb))
    yr, A = oracle.gemv(q.Q4_K, W, N, K, x)
    lg, ig = host(logits), host(idx)
    tol = tol_gemv(A, yr)
    assert_within(lg, yr, tol, "argmax logits")
    for b in range(nb):
        i, m = int(ig[b]), int(np.argmax(yr[b]))
        assert int(np.argmax(lg[b])) == i
        assert i == m or yr[b, m] - yr[b, i] <= tol[b, m] + tol[b, i]


def _pow2_q4_k(g, N, K):
    W = wl.q4_k_matrix(g, N, K).reshape(N, -1, 144).copy()
    for o in (0, 2):
        W[..., o:o + 2] = (2.0 ** -g.integers(4, 9, size=W.shape[:2])).astype("<f2")[..., None].view(np.uint8)
    return W.reshape(N, -1)


@pytest.mark.parametrize("nb", [5, 9, 16])
def test_q4_k_row_batch_integer_bitwise(nb):
    say(f"q4_k mfma integer nb={nb}")
    N, K = 48, 512
    g = wl.rng(4200, nb)
    W = _pow2_q4_k(g, N, K)
    x = g.integers(-3, 4, size=(nb, K)).astype(np.float32)
    y = _gemv(W, N, K, x)
    yr, _ = oracle.gemv(q.Q4_K, W, N, K, x)
    assert np.array_equal(y.astype(np.float64), yr)


def test_q4_k_row_batch_zero_weights():
    """Scales and mins 0: every output exactly 0."""
    N, K, nb = 40, 2048, 16
    g = wl.rng(4300, 1)
    W = wl.q4_k_matrix(g, N, K).reshape(N, -1, 144).copy()
    W[..., 4:16] = 0
    y = _gemv(W.reshape(N, -1), N, K, wl.normal_f32(g, (nb, K)))
    assert np.array_equal(y, np.zeros_like(y))


@pytest.mark.parametrize("nb", [6, 16])
def test_q4_k_row_batch_cancellation(nb):
    """Sub-blocks whose weights mostly sit at 0 (d sc q = dmin m for the common q) with same-sign
    x: the error stays relative to sum |w x|."""
    say(f"q4_k mfma cancellation nb={nb}")
    N, K = 64, 1024
    g = wl.rng(4400, nb)
    W = wl.q4_k_matrix(g, N, K).reshape(N, -1, 144).copy()
    W[..., 2:4] = W[..., 0:2]                                    # dmin = d
    # every (sc, m) = (1, 9): w = d (q - 9); most nibbles 9
    W[..., 4:16] = np.array([1, 1, 1, 1, 9, 9, 9, 9, 0x91, 0x91, 0x91, 0x91], np.uint8)
    W[..., 16:144] = 0x99
    for n in range(N):
        for b in range(W.shape[1]):
            pos = g.choice(128, size=3, replace=False)
            W[n, b, 16 + pos] = g.integers(0, 256, size=3, dtype=np.uint8)
    W = W.reshape(N, -1)
    for j in range(8):
        assert oracle.q4k_scale_min(W[0, 4:16].tobytes(), j) == (1, 9)
    x = g.uniform(0.9, 1.0, size=(nb, K)).astype(np.float32)
    y = _gemv(W, N, K, x)
    yr, A = oracle.gemv(q.Q4_K, W, N, K, x)
    assert_within(y, yr, tol_gemv(A, yr), "q4_k cancellation")
